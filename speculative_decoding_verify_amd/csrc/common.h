// Device helpers shared by the libsdv kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16;  // raw bf16 bit pattern
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

#define SDV_DEV __device__ __forceinline__

SDV_DEV float bf2f(bf16 u) { return __uint_as_float(((uint32_t)u) << 16); }

// fp32 -> bf16, round to nearest even (inputs are finite)
SDV_DEV bf16 f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16)(u >> 16);
}

template <typename T> SDV_DEV float to_f(T v);
template <> SDV_DEV float to_f<float>(float v) { return v; }
template <> SDV_DEV float to_f<bf16>(bf16 v) { return bf2f(v); }

template <typename T> SDV_DEV T from_f(float v);
template <> SDV_DEV float from_f<float>(float v) { return v; }
template <> SDV_DEV bf16 from_f<bf16>(float v) { return f2bf(v); }

SDV_DEV u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// streamed once: do not keep in the caches
SDV_DEV u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
SDV_DEV void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// One 16-byte-per-lane MFMA step of C[16x16] += A[16 x k] * B[k x 16].
// Lane l supplies A row (l % 16) and B column (l % 16) for the k values of lane
// group l / 16; the same element position in A and B must hold the same k.
//   bf16: one v_mfma_f32_16x16x32_bf16 (8 k values per lane, k = 32)
//   fp32: four v_mfma_f32_16x16x4_f32 (element e of each lane per instruction, k = 16)
// Output: lane l holds C[4 * (l / 16) + i][l % 16] in element i.
template <typename T> SDV_DEV f32x4 mma16(u32x4 a, u32x4 b, f32x4 c);
template <> SDV_DEV f32x4 mma16<bf16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
template <> SDV_DEV f32x4 mma16<float>(u32x4 a, u32x4 b, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  return c;
}

// Split pairs: a bf16 model carries each activation value as x = hi + lo + O(2^-16 |x|),
// two bf16 numbers that enter a bf16 MFMA as two operands.
SDV_DEV void split1(float x, bf16& hi, bf16& lo) {
  hi = f2bf(x);
  lo = f2bf(x - bf2f(hi));
}
SDV_DEV uint32_t pack2(bf16 a, bf16 b) { return (uint32_t)a | ((uint32_t)b << 16); }

// Query rows (read by the attention kernels): one row per chunk row; bf16 models
// store k group g (8 values) at bytes g * 32 as 8 hi parts then 8 lo parts, fp32
// models store fp32.
template <typename T> SDV_DEV void row_store1(void* row, int k, float x);
template <> SDV_DEV void row_store1<float>(void* row, int k, float x) { ((float*)row)[k] = x; }
template <> SDV_DEV void row_store1<bf16>(void* row, int k, float x) {
  bf16 hi, lo;
  split1(x, hi, lo);
  bf16* g = (bf16*)row + (k >> 3) * 16 + (k & 7);
  g[0] = hi;
  g[8] = lo;
}

// GEMM activation operands ("A": M rows x K values, 4 bytes per value) are stored
// in the lane order of the MFMA A operand, so that every wave load of a GEMM reads
// one contiguous kilobyte.  Rows go 16 to a row tile; row tile rt holds the K / KS
// k steps (KS = 32 bf16, 16 fp32) one after another, 64 * KS bytes each:
//   bf16: 1 KB of hi parts, then 1 KB of lo parts; lane l's 16 bytes in each hold
//         row 16 rt + l % 16, k = 32 s + 8 (l / 16) + 0..7;
//   fp32: 1 KB; lane l's 16 bytes hold row 16 rt + l % 16, k = 16 s + 4 (l / 16) + 0..3.
// A buffer of M rows takes 16 * ceil(M / 16) * K * 4 bytes.  Rows past M in the last
// tile are never written, and the GEMMs never read them.
template <typename T> SDV_DEV size_t act_pos(int K, int m, int k);
template <> SDV_DEV size_t act_pos<bf16>(int K, int m, int k) {
  return ((size_t)(m >> 4) * (K >> 5) + (k >> 5)) * 2048 + (size_t)((((k >> 3) & 3) << 4) | (m & 15)) * 16 +
         (k & 7) * 2;
}
template <> SDV_DEV size_t act_pos<float>(int K, int m, int k) {
  return ((size_t)(m >> 4) * (K >> 4) + (k >> 4)) * 1024 + (size_t)((((k >> 2) & 3) << 4) | (m & 15)) * 16 +
         (k & 3) * 4;
}

// act_store1: value k of row m; act_store4: values k0..k0+3 (k0 % 4 == 0);
// act_store8: values k0..k0+7 (k0 % 8 == 0)
template <typename T> SDV_DEV void act_store1(void* a, int K, int m, int k, float x);
template <> SDV_DEV void act_store1<float>(void* a, int K, int m, int k, float x) {
  *(float*)((char*)a + act_pos<float>(K, m, k)) = x;
}
template <> SDV_DEV void act_store1<bf16>(void* a, int K, int m, int k, float x) {
  bf16 hi, lo;
  split1(x, hi, lo);
  char* p = (char*)a + act_pos<bf16>(K, m, k);
  *(bf16*)p = hi;
  *(bf16*)(p + 1024) = lo;
}
template <typename T> SDV_DEV void act_store4(void* a, int K, int m, int k0, const float (&x)[4]);
template <> SDV_DEV void act_store4<float>(void* a, int K, int m, int k0, const float (&x)[4]) {
  *(float4*)((char*)a + act_pos<float>(K, m, k0)) = make_float4(x[0], x[1], x[2], x[3]);
}
template <> SDV_DEV void act_store4<bf16>(void* a, int K, int m, int k0, const float (&x)[4]) {
  bf16 h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) split1(x[e], h[e], l[e]);
  char* p = (char*)a + act_pos<bf16>(K, m, k0);
  *(uint2*)p = make_uint2(pack2(h[0], h[1]), pack2(h[2], h[3]));
  *(uint2*)(p + 1024) = make_uint2(pack2(l[0], l[1]), pack2(l[2], l[3]));
}
template <typename T> SDV_DEV void act_store8(void* a, int K, int m, int k0, const float (&x)[8]);
template <> SDV_DEV void act_store8<float>(void* a, int K, int m, int k0, const float (&x)[8]) {
  *(float4*)((char*)a + act_pos<float>(K, m, k0)) = make_float4(x[0], x[1], x[2], x[3]);
  *(float4*)((char*)a + act_pos<float>(K, m, k0 + 4)) = make_float4(x[4], x[5], x[6], x[7]);
}
template <> SDV_DEV void act_store8<bf16>(void* a, int K, int m, int k0, const float (&x)[8]) {
  bf16 h[8], l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) split1(x[e], h[e], l[e]);
  char* p = (char*)a + act_pos<bf16>(K, m, k0);
  st16(p, u32x4{pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7])});
  st16(p + 1024, u32x4{pack2(l[0], l[1]), pack2(l[2], l[3]), pack2(l[4], l[5]), pack2(l[6], l[7])});
}

// ---------------------------------------------------------------------------
// Hand-off between the workgroups of one kernel (split reductions finished by the
// workgroup that arrives last).  The producers' parts go through device-scope buffer
// stores (cache policy sc1: written through the compute unit's and the XCD's caches),
// and the last workgroup reads them with device-scope loads (sc1: not served from a
// possibly stale cache of another XCD).  Each producer waits until its stores have
// completed before it counts itself in, so a workgroup that sees the count complete
// finds every part in place.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int CPOL_DEVICE = 16;   // sc1
SDV_DEV rsrc_t dev_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
SDV_DEV void st_dev16(rsrc_t r, uint32_t off, u32x4 v) { __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, CPOL_DEVICE); }
SDV_DEV void st_dev8(rsrc_t r, uint32_t off, u32x2 v) { __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, CPOL_DEVICE); }
SDV_DEV u32x4 ld_dev16(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CPOL_DEVICE); }
SDV_DEV u32x2 ld_dev8(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, CPOL_DEVICE); }

// Wait until every vector memory load and store of the wave has completed (the
// vector-memory counter at zero; export and LDS counters left alone).
SDV_DEV void vmem_wait_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// LDS DMA: 16 bytes from global address g (per lane) land in LDS at lds + 16 * lane
// (lds uniform across the wave), without passing through registers; completion is
// counted by the vector-memory counter.
SDV_DEV void lds_dma16(const void* g, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
#endif
}
// wait until at most N vector memory operations of the wave are outstanding
template <int N> SDV_DEV void vmem_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// the same, and every LDS access of the wave complete
template <int N> SDV_DEV void vmem_lds_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}
// a bare workgroup barrier (no counter waits); the fences keep the compiler from moving
// memory accesses across it
SDV_DEV void bare_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// a workgroup barrier after the wave's own LDS accesses have completed (so its LDS
// writes are visible to the workgroup behind it); vector memory loads stay in flight
SDV_DEV void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((3 << 14) | (7 << 4) | 15);   // lgkmcnt(0); vmcnt 63 and expcnt 7: no wait
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Every thread's stores are complete, then thread 0 counts the workgroup in on
// `counter` (zero before the launch).  True in all threads of the workgroup that
// arrives n-th (last).  `flag` is an int in LDS.
SDV_DEV bool arrive_last(uint32_t* counter, uint32_t n, int* flag) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0)
    *flag = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n - 1;
  __syncthreads();
  return *flag != 0;
}

// elements of T held in 16 bytes
template <typename T> struct Vec16 { static constexpr int N = 16 / sizeof(T); };

SDV_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Sum over a 256-thread block in a fixed order (deterministic).  `red` holds 8 floats.
// Sum over a block of NW waves in a fixed order (deterministic).  `red` holds NW floats.
template <int NW>
SDV_DEV float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float t = red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) t += red[i];
  __syncthreads();
  return t;
}

SDV_DEV float block_sum_256(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float t = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return t;
}

// per-sequence error word (device)
SDV_DEV void set_err(int32_t* err, int b, int bits) {
  if (err) atomicOr(err + b, bits);
}
