// Chunked causal / tree-masked GQA attention over a paged KV cache, split over keys.
// Queries and the output are fp32; keys and values are the cache type.
//
// A verify pass attends from T chunk rows (audio chunk + drafts + branch rows) to
// the C cached slots and to the chunk rows that are ancestors-or-self of each row
// ("Decode Before You Hear", page 1, method step 4 with the runner-up branch of
// step 2).  The T*G query rows of one kv head (G = H / Hkv) share every K/V tile,
// so a workgroup owns (sequence, kv head, key split) and all of that head's query
// tiles; K/V tiles are staged once in LDS and reused by every query tile.
//
// Per tile of KT keys (32 for bf16, 16 for fp32) and query tile of 16 rows:
//   S^T = K Q^T      on MFMA: keys are the A rows, queries the B columns, so each
//                    lane ends up holding scores of one query for 8 (bf16) or 4
//                    (fp32) keys;
//   online softmax   in fp32 (exp2 domain), per lane, with the row max exchanged
//                    across the 4 lane groups;
//   O^T += V^T P^T   on MFMA: the scores a lane already holds are exactly its B
//                    operand, because V is stored transposed inside each page and,
//                    for bf16, the 32 keys of a tile are assigned to MFMA rows so
//                    that lane group g holds keys 8g..8g+7 (rows 4g..4g+3 of the two
//                    S^T tiles map to keys 8g..8g+3 and 8g+4..8g+7).
// Partials (unnormalised O, running max, running sum) of the key splits are merged
// per query row with log-sum-exp weights by the workgroup that finishes last (the
// hand-off of common.h), or, where a group's merge would not fit its LDS scratch, by
// the separate combine kernel.
#include <hip/hip_ext.h>

#include "common.h"
#include "kernels.h"

#include <algorithm>
#include <type_traits>

namespace sdv {

// Query operand of one lane.  The q buffer holds the queries pre-scaled by
// log2(e)/sqrt(dh) in the query-row format (4 bytes per value), so for bf16 the 8
// values of lane group lg in k step ks are one 16-byte hi load and one 16-byte lo
// load; for fp32 the 4 values are one load.  `off` is the value index of the head's
// first value (row * H * dh + head * dh).
template <bool BF, int DH, int KS, int VE>
SDV_DEV void load_q(const void* q, size_t off, bool ok, int lg, u32x4 (&out)[DH / KS][BF ? 2 : 1]) {
  const u32x4 zero = {0u, 0u, 0u, 0u};
  const char* base = (const char*)q + off * 4;
#pragma unroll
  for (int ks = 0; ks < DH / KS; ++ks) {
    const char* g = base + (size_t)(ks * KS + lg * VE) * 4;
    if constexpr (BF) {
      out[ks][0] = ok ? ld16(g) : zero;
      out[ks][1] = ok ? ld16(g + 16) : zero;
    } else {
      out[ks][0] = ok ? ld16(g) : zero;
    }
  }
}

// Physical pages of every logical page the split can reach, [k_begin/16, (k_begin +
// split_keys)/16), staged in LDS once per workgroup (-1 where the table entry is out of
// range), so key and value loads never wait on a block-table load.  The range does
// not depend on the sequence length, so the table loads need not wait for it.  The
// host keeps split_keys a multiple of 16 and at most 16 * (512 - 1).
constexpr int ATTN_MAX_PAGES = 512;
SDV_DEV int stage_pages(const AttnArgs& a, const int32_t* bt, int k_begin, int* sPage) {
  const int pg0 = k_begin >> 4;
  const int npg = min(a.split_keys >> 4, ATTN_MAX_PAGES);
  for (int i = threadIdx.x; i < npg; i += blockDim.x) {
    const int pg = pg0 + i;
    int phys = pg < a.max_blocks ? bt[pg] : -1;
    if (phys < 0 || phys >= a.n_blocks) phys = -1;
    sPage[i] = phys;
  }
  __syncthreads();
  return pg0;
}

// Word w (0..3) of a row's ancestor mask held in registers, by selects (a per-lane
// index into a register array would become a loop over the distinct indices).
SDV_DEV uint32_t anc_word(const uint32_t (&m)[4], int w) {
  return w == 0 ? m[0] : w == 1 ? m[1] : w == 2 ? m[2] : m[3];
}

// Reductions over the lane pairs (l, l ^ 16) and (l, l ^ 32) with gfx950's lane-swap
// instructions: after v_permlane16_swap / v_permlane32_swap of a value with itself,
// the two results at every lane are the values of the lower and the upper lane of its
// pair, so both lanes of a pair compute the same result from the same two operands.
// Plain VALU, where a shuffle would take a round trip through the LDS crossbar.
SDV_DEV float pair16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
SDV_DEV float pair32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
SDV_DEV float pair16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
SDV_DEV float pair32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Probabilities as a bf16 hi/lo operand pair, cheaply: hi = p rounded half-up to 8
// significant bits, lo = the exact remainder p - hi truncated to bf16, so
// |p - hi - lo| < 2^-15 |p|.  v_perm gathers the upper halves of two words.
SDV_DEV void split_probs_fast(const float (&p)[8], u32x4& hi, u32x4& lo) {
  uint32_t h[8], l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = (__float_as_uint(p[e]) + 0x8000u) & 0xFFFF0000u;
    l[e] = __float_as_uint(p[e] - __uint_as_float(h[e]));
  }
  hi.x = __builtin_amdgcn_perm(h[1], h[0], 0x07060302u); hi.y = __builtin_amdgcn_perm(h[3], h[2], 0x07060302u);
  hi.z = __builtin_amdgcn_perm(h[5], h[4], 0x07060302u); hi.w = __builtin_amdgcn_perm(h[7], h[6], 0x07060302u);
  lo.x = __builtin_amdgcn_perm(l[1], l[0], 0x07060302u); lo.y = __builtin_amdgcn_perm(l[3], l[2], 0x07060302u);
  lo.z = __builtin_amdgcn_perm(l[5], l[4], 0x07060302u); lo.w = __builtin_amdgcn_perm(l[7], l[6], 0x07060302u);
}

// The same hi/lo pair with gfx950's packed conversion: hi = p rounded to nearest even
// bf16, lo = (p - hi) rounded likewise (p - hi is exact in fp32), so |p - hi - lo| <=
// 2^-18 |p|; one conversion covers two values and yields the operand word directly.
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));
SDV_DEV uint32_t cvt_pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_v){a, b}, bf16x2_v));
}
SDV_DEV void split_probs_pk(const float (&p)[8], u32x4& hi, u32x4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = cvt_pk_bf16(p[2 * e], p[2 * e + 1]);
    const float r0 = p[2 * e] - __uint_as_float(h[e] << 16);
    const float r1 = p[2 * e + 1] - __uint_as_float(h[e] & 0xFFFF0000u);
    l[e] = cvt_pk_bf16(r0, r1);
  }
  hi = u32x4{h[0], h[1], h[2], h[3]};
  lo = u32x4{l[0], l[1], l[2], l[3]};
}

// Merge of the split partial states of query rows [qi0, qi1) of (sequence b, kv head
// g), run by the last workgroup of the group to finish; splits are taken in order:
//   M = max_s m_s,  w_s = 2^(m_s - M) / sum_s' 2^(m_s' - M) l_s',  o = sum_s w_s o_s.
// wgt is LDS scratch of n_splits * (qi1 - qi0) floats.
template <typename T, int DH>
SDV_DEV void attn_merge(const AttnArgs& a, int b, int g, int qi0, int qi1, float* wgt) {
  const int nr = qi1 - qi0, ns = a.n_splits, G = a.H / a.Hkv;
  const size_t grp = ((size_t)b * a.Hkv + g) * ns * a.nq_pad;   // (split 0, row 0) of the group
  const rsrc_t rml = dev_rsrc(a.pml + grp * 2, (uint32_t)ns * a.nq_pad * 8);
  const rsrc_t rpo = dev_rsrc(a.po + grp * DH, (uint32_t)ns * a.nq_pad * DH * 4);
  for (int i = threadIdx.x; i < nr; i += blockDim.x) {
    float m[ATTN_MAX_SPLITS], l[ATTN_MAX_SPLITS];
#pragma unroll
    for (int s = 0; s < ATTN_MAX_SPLITS; ++s) {
      const u32x2 v = ld_dev8(rml, (uint32_t)((min(s, ns - 1) * a.nq_pad + qi0 + i) * 8));
      m[s] = __uint_as_float(v.x);
      l[s] = __uint_as_float(v.y);
    }
    float M = m[0];
#pragma unroll
    for (int s = 1; s < ATTN_MAX_SPLITS; ++s) M = fmaxf(M, m[s]);
    float L = 0.f;
#pragma unroll
    for (int s = 0; s < ATTN_MAX_SPLITS; ++s) {
      m[s] = s < ns ? __builtin_amdgcn_exp2f(m[s] - M) : 0.f;
      L += m[s] * l[s];
    }
    const float inv = 1.f / L;
#pragma unroll
    for (int s = 0; s < ATTN_MAX_SPLITS; ++s)
      if (s < ns) wgt[s * nr + i] = m[s] * inv;
  }
  __syncthreads();
  constexpr int NC = DH / 4;   // 16-byte chunks of an output row
  constexpr int SU = 16;       // splits loaded per round
  for (int it = threadIdx.x; it < nr * NC; it += blockDim.x) {
    const int i = it / NC, c = it % NC;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < ns; s0 += SU) {
      u32x4 v[SU];
#pragma unroll
      for (int u = 0; u < SU; ++u)
        v[u] = ld_dev16(rpo, (uint32_t)(((min(s0 + u, ns - 1) * a.nq_pad + qi0 + i) * DH + 4 * c) * 4));
#pragma unroll
      for (int u = 0; u < SU; ++u) {
        const float wv = s0 + u < ns ? wgt[(s0 + u) * nr + i] : 0.f;
        acc[0] += wv * __uint_as_float(v[u].x);
        acc[1] += wv * __uint_as_float(v[u].y);
        acc[2] += wv * __uint_as_float(v[u].z);
        acc[3] += wv * __uint_as_float(v[u].w);
      }
    }
    const int qi = qi0 + i, t = qi / G, h = g * G + qi % G;
    act_store4<T>(a.o, a.H * DH, b * a.T + t, h * DH + 4 * c, acc);
  }
}

// The same merge for at most 8 splits in one memory round trip per item: a thread's
// item (row, 16-byte chunk) needs every split's (m, l) and output chunk, all loaded
// at once, and the next item's loads are issued before the current one is finished.
template <typename T, int DH>
SDV_DEV void attn_merge8(const AttnArgs& a, int b, int g, int qi0, int qi1) {
  constexpr int MS = 8, NC = DH / 4;
  const int nr = qi1 - qi0, ns = a.n_splits, G = a.H / a.Hkv;
  const int n_items = nr * NC;
  const size_t grp = ((size_t)b * a.Hkv + g) * ns * a.nq_pad;
  const rsrc_t rml = dev_rsrc(a.pml + grp * 2, (uint32_t)ns * a.nq_pad * 8);
  const rsrc_t rpo = dev_rsrc(a.po + grp * DH, (uint32_t)ns * a.nq_pad * DH * 4);
  struct Buf {
    u32x2 ml[MS];
    u32x4 po[MS];
  };
  auto load = [&](int it, Buf& bf) {
    it = min(it, n_items - 1);
    const int i = it / NC, c = it % NC;
#pragma unroll
    for (int s = 0; s < MS; ++s) {
      const uint32_t row = (uint32_t)(min(s, ns - 1) * a.nq_pad + qi0 + i);
      bf.ml[s] = ld_dev8(rml, row * 8);
      bf.po[s] = ld_dev16(rpo, (row * DH + 4 * c) * 4);
    }
  };
  auto finish = [&](int it, const Buf& bf) {
    if (it >= n_items) return;
    const int i = it / NC, c = it % NC;
    float M = __uint_as_float(bf.ml[0].x);
#pragma unroll
    for (int s = 1; s < MS; ++s) M = fmaxf(M, __uint_as_float(bf.ml[s].x));
    float L = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < MS; ++s) {
      const float wv = s < ns ? __builtin_amdgcn_exp2f(__uint_as_float(bf.ml[s].x) - M) : 0.f;
      L += wv * __uint_as_float(bf.ml[s].y);
      acc[0] += wv * __uint_as_float(bf.po[s].x);
      acc[1] += wv * __uint_as_float(bf.po[s].y);
      acc[2] += wv * __uint_as_float(bf.po[s].z);
      acc[3] += wv * __uint_as_float(bf.po[s].w);
    }
    const float inv = 1.f / L;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] *= inv;
    const int qi = qi0 + i, t = qi / G, h = g * G + qi % G;
    act_store4<T>(a.o, a.H * DH, b * a.T + t, h * DH + 4 * c, acc);
  };
  Buf A, B;
  const int step = blockDim.x;
  int it = threadIdx.x;
  load(it, A);
  for (; it < n_items; it += 2 * step) {
    load(it + step, B);
    finish(it, A);
    if (it + 2 * step < n_items) load(it + 2 * step, A);
    finish(it + step, B);
  }
}

template <typename T, int DH, int NQW>
__global__ __launch_bounds__(512) void attn_chunk(AttnArgs a) {
  constexpr bool BF = sizeof(T) == 2;
  constexpr int VE = Vec16<T>::N;          // elements per 16 B
  constexpr int KS = 4 * VE;               // contraction length of one mma16 step
  constexpr int KT = BF ? 32 : 16;         // keys per tile
  constexpr int KROW = DH + VE;            // padded LDS row of K (elements)
  constexpr int VROW = 16 + VE;            // padded LDS row of V^T (elements)
  constexpr int NPG = KT / 16;             // pages per tile
  constexpr int PE = BF ? 8 : 4;           // scores per lane per tile

  // K and V^T tiles; after the key loop the same LDS is the merge scratch
  constexpr int KBYTES = KT * KROW * (int)sizeof(T), VBYTES = NPG * DH * VROW * (int)sizeof(T);
  __shared__ __attribute__((aligned(16))) char lds_raw[std::max(KBYTES + VBYTES, ATTN_MERGE_FLOATS * 4)];
  T* const ldsK = (T*)lds_raw;
  T* const ldsV = (T*)(lds_raw + KBYTES);

  const int split = blockIdx.z, g = blockIdx.x, b = blockIdx.y / a.n_qg;
  const int lane = threadIdx.x & 63, NW = blockDim.x >> 6;
  // this wave's query tiles: q_base + w + j*NW, q_base = (query group) * NW * NQW
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int q_base = (blockIdx.y % a.n_qg) * NW * NQW;
  const int r = lane & 15, lg = lane >> 4;
  const int G = a.H / a.Hkv;
  const int C = min(max(a.seq_len[b], 0), a.max_ctx);
  const int nkeys = C + a.T;
  const int nq = a.T * G;
  const int NQT = (nq + 15) >> 4;
  const int k_begin = split * a.split_keys;
  const int k_end = min(nkeys, k_begin + a.split_keys);
  const int32_t* bt = a.block_table + (size_t)b * a.max_blocks;
  const T* kp = (const T*)a.k_pages;
  const T* vp = (const T*)a.v_pages;
  // queries of this wave: tiles w, w + NW, ... (loaded before the page table is
  // staged, so both round trips overlap)
  constexpr int QP = BF ? 2 : 1;   // q enters bf16 MFMAs as a hi + lo pair
  u32x4 qreg[NQW][DH / KS][QP];
  uint32_t anc[NQW][4];
  float mrun[NQW], lrun[NQW];
  f32x4 acc[NQW][DH / 16];
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < NQW; ++j) {
    const int qi = (q_base + w + j * NW) * 16 + r;
    const bool ok = qi < nq;
    const int t = ok ? qi / G : 0;
    const int h = g * G + (ok ? qi % G : 0);
    load_q<BF, DH, KS, VE>(a.q, ((size_t)(b * a.T + t) * a.H + h) * DH, ok, lg, qreg[j]);
#pragma unroll
    for (int c = 0; c < 4; ++c) anc[j][c] = a.anc[t * 4 + c];
    mrun[j] = -1e30f;
    lrun[j] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) acc[j][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __shared__ int sPage[ATTN_MAX_PAGES];
  const int pg0 = stage_pages(a, bt, k_begin, sPage);

  // K (token-major) and V^T (dh-major) of a tile go through LDS; each thread holds
  // its 16-byte chunks of the next tile in registers while the current one is used.
  // Slots at or beyond the split end read as zero (values past the sequence end too,
  // so no stale value is ever read).  The block has at least 4 waves.
  constexpr int KCH = KT * DH / VE, VCH = NPG * DH * (16 / VE);
  constexpr int MAXC = (std::max(KCH, VCH) + 255) / 256;
  u32x4 kst[MAXC], vst[MAXC];
  auto fetch = [&](int kt0) {
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int c = threadIdx.x + i * blockDim.x;
      u32x4 v = zero;
      if (c < KCH) {
        const int key = c / (DH / VE), d0 = (c % (DH / VE)) * VE;
        const int slot = kt0 + key;
        const int phys = slot < k_end ? sPage[(slot >> 4) - pg0] : -1;
        if (phys >= 0) v = ld16(kp + (((size_t)phys * a.Hkv + g) * 16 + (slot & 15)) * DH + d0);
      }
      kst[i] = v;
      v = zero;
      if (c < VCH) {
        const int p = c / (DH * (16 / VE)), rem = c % (DH * (16 / VE));
        const int dd = rem / (16 / VE), o0 = (rem % (16 / VE)) * VE;
        const int slot0 = kt0 + p * 16 + o0;
        const int phys = slot0 < k_end ? sPage[(slot0 >> 4) - pg0] : -1;
        if (phys >= 0) {
          v = ld16(vp + (((size_t)phys * a.Hkv + g) * DH + dd) * 16 + o0);
          if (slot0 + VE > nkeys) {
            T e[VE];
            __builtin_memcpy(e, &v, 16);
#pragma unroll
            for (int ii = 0; ii < VE; ++ii)
              if (slot0 + ii >= nkeys) e[ii] = T(0);
            __builtin_memcpy(&v, e, 16);
          }
        }
      }
      vst[i] = v;
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int c = threadIdx.x + i * blockDim.x;
      if (c < KCH) {
        const int key = c / (DH / VE), d0 = (c % (DH / VE)) * VE;
        st16(&ldsK[key * KROW + d0], kst[i]);
      }
      if (c < VCH) {
        const int p = c / (DH * (16 / VE)), rem = c % (DH * (16 / VE));
        const int dd = rem / (16 / VE), o0 = (rem % (16 / VE)) * VE;
        st16(&ldsV[(p * DH + dd) * VROW + o0], vst[i]);
      }
    }
  };

  constexpr int NH = BF ? 2 : 1;                     // 16-key halves of a tile
  const int krow0 = BF ? 8 * (r >> 2) + (r & 3) : r;  // K row of this lane (half 0)
  // query tiles of this wave that exist (wave-uniform)
  const int nj = min(NQW, max(0, (NQT - (q_base + w) + NW - 1) / NW));
  // The query loads are complete before the key loop: the loop's waits then cover
  // only the tile prefetch (otherwise the first score MFMAs of every tile would wait
  // on the in-order load counter until the next tile's loads had landed).
  vmem_wait_all();
  if (k_begin < k_end) fetch(k_begin);
  for (int kt0 = k_begin; kt0 < k_end; kt0 += KT) {
    __syncthreads();   // every wave is done with the previous tile
    store();
    __syncthreads();
    if (kt0 + KT < k_end) fetch(kt0 + KT);

    // ---- scores S^T of all this wave's query tiles; each K operand is read from LDS
    //      once and used by every query tile
    f32x4 sc[NQW][NH];
#pragma unroll
    for (int j = 0; j < NQW; ++j)
#pragma unroll
      for (int hv = 0; hv < NH; ++hv) sc[j][hv] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < DH / KS; ++ks) {
      u32x4 kk[NH];
#pragma unroll
      for (int hv = 0; hv < NH; ++hv) kk[hv] = ld16(&ldsK[(krow0 + 4 * hv) * KROW + ks * KS + lg * VE]);
#pragma unroll
      for (int qp = 0; qp < QP; ++qp)
#pragma unroll
        for (int j = 0; j < NQW; ++j)
          if (j < nj)
#pragma unroll
            for (int hv = 0; hv < NH; ++hv) sc[j][hv] = mma16<T>(kk[hv], qreg[j][ks][qp], sc[j][hv]);
    }
    float sv[NQW][PE];
#pragma unroll
    for (int j = 0; j < NQW; ++j)
#pragma unroll
      for (int hv = 0; hv < NH; ++hv)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[j][4 * hv + i] = sc[j][hv][i];
    // ---- mask only tiles that reach the chunk rows or the split end (wave-uniform)
    if (kt0 + KT > C || kt0 + KT > k_end) {
#pragma unroll
      for (int e = 0; e < PE; ++e) {
        // straight-line visibility: inside the split, and a cached slot or an
        // ancestor-or-self chunk row
        const int sl = kt0 + PE * lg + e;
        const bool live = sl < k_end;
        const int jr = max(sl - C, 0);
#pragma unroll
        for (int j = 0; j < NQW; ++j) {
          const bool vis = live & ((sl < C) | (((anc_word(anc[j], jr >> 5) >> (jr & 31)) & 1u) != 0u));
          sv[j][e] = vis ? sv[j][e] : -INFINITY;
        }
      }
    }
    // ---- online softmax; rescale only when some row's maximum rises
    float mnew[NQW];
    bool rise = false;
#pragma unroll
    for (int j = 0; j < NQW; ++j) {
      float mx = sv[j][0];
#pragma unroll
      for (int e = 1; e < PE; ++e) mx = fmaxf(mx, sv[j][e]);
      mx = pair32_max(pair16_max(mx));
      mnew[j] = fmaxf(mrun[j], mx);
      rise |= mnew[j] > mrun[j];
    }
    if (__any(rise)) {
#pragma unroll
      for (int j = 0; j < NQW; ++j) {
        const float alpha = __builtin_amdgcn_exp2f(mrun[j] - mnew[j]);
        mrun[j] = mnew[j];
        lrun[j] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DH / 16; ++dt) acc[j][dt] *= alpha;
      }
    }
    u32x4 pop[NQW][QP];   // P operand(s) of each query tile
#pragma unroll
    for (int j = 0; j < NQW; ++j) {
      float pj[PE], ps = 0.f;
#pragma unroll
      for (int e = 0; e < PE; ++e) {
        pj[e] = __builtin_amdgcn_exp2f(sv[j][e] - mrun[j]);
        ps += pj[e];
      }
      lrun[j] += ps;
      if constexpr (BF) {
        split_probs_fast(pj, pop[j][0], pop[j][QP - 1]);
      } else {
        pop[j][0].x = __float_as_uint(pj[0]); pop[j][0].y = __float_as_uint(pj[1]);
        pop[j][0].z = __float_as_uint(pj[2]); pop[j][0].w = __float_as_uint(pj[3]);
      }
    }
    // ---- O^T += V^T P^T; each V operand is read from LDS once
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) {
      const u32x4 va = BF ? ld16(&ldsV[((lg >> 1) * DH + dt * 16 + r) * VROW + (lg & 1) * 8])
                          : ld16(&ldsV[(dt * 16 + r) * VROW + lg * 4]);
#pragma unroll
      for (int j = 0; j < NQW; ++j)
        if (j < nj)
#pragma unroll
          for (int qp = 0; qp < QP; ++qp) acc[j][dt] = mma16<T>(va, pop[j][qp], acc[j][dt]);
    }
  }

  // ---- the split's partial state (or, with a single split, the output rows)
  const bool fused = a.sem != nullptr;
  const bool direct = fused && a.n_splits == 1;
  const size_t grp = ((size_t)b * a.Hkv + g) * a.n_splits * a.nq_pad;
  const rsrc_t rpo = dev_rsrc(a.po + grp * DH, (uint32_t)a.n_splits * a.nq_pad * DH * 4);
  const rsrc_t rml = dev_rsrc(a.pml + grp * 2, (uint32_t)a.n_splits * a.nq_pad * 8);
#pragma unroll
  for (int j = 0; j < NQW; ++j) {
    const int qt = q_base + w + j * NW;
    if (qt >= NQT) continue;
    float l = lrun[j];
    l = pair32_sum(pair16_sum(l));
    const int qi = qt * 16 + r;
    const uint32_t pr = (uint32_t)(split * a.nq_pad + qi);
    if (direct) {
      if (qi < nq) {
        const float inv = 1.f / l;
        const int orow = b * a.T + qi / G;
        const int h = g * G + qi % G;
#pragma unroll
        for (int dt = 0; dt < DH / 16; ++dt) {
          const float v[4] = {acc[j][dt][0] * inv, acc[j][dt][1] * inv, acc[j][dt][2] * inv, acc[j][dt][3] * inv};
          act_store4<T>(a.o, a.H * DH, orow, h * DH + dt * 16 + 4 * lg, v);
        }
      }
    } else {
#pragma unroll
      for (int dt = 0; dt < DH / 16; ++dt)
        st_dev16(rpo, (pr * DH + dt * 16 + 4 * lg) * 4, __builtin_bit_cast(u32x4, acc[j][dt]));
      if (lg == 0) st_dev8(rml, pr * 8, u32x2{__float_as_uint(mrun[j]), __float_as_uint(l)});
    }
  }
  if (!fused || direct) return;
  __shared__ int is_last;
  const int qg = blockIdx.y % a.n_qg;
  if (!arrive_last(a.sem + ((size_t)b * a.Hkv + g) * a.n_qg + qg, a.n_splits, &is_last)) return;
  if (a.n_splits <= 8) attn_merge8<T, DH>(a, b, g, q_base * 16, min(nq, (q_base + NW * NQW) * 16));
  else attn_merge<T, DH>(a, b, g, q_base * 16, min(nq, (q_base + NW * NQW) * 16), (float*)lds_raw);
}

// bf16 attention with K/V staged by LDS DMA.  Same work decomposition, online softmax,
// P V and split hand-off as attn_chunk; what changes is the staging.  A 32-key tile is
// two pages of K and two of V of one kv head, each page a contiguous block of 16 * dh
// bf16 in the cache, so the tile is copied as 1 KB wave-loads (global_load_lds: no
// registers, no LDS stores, the page address uniform per load) into a ring of R
// tiles; one barrier per tile.  A 16-byte LDS read of a wave is served in four sets of
// 16 lanes, {0-7, 24-31}, {8-15, 16-23}, {32-39, 56-63} and {40-47, 48-55} (measured
// on the device), each without bank conflicts when its lanes hit distinct 16-byte
// slots modulo 256 bytes.  The value operand reads meet that in the cache's own page
// layout; the key rows are 256 (dh 128) or 128 (dh 64) bytes, so inside LDS the
// 16-byte chunks of a key are permuted (chunk index XOR bits of the key), which a
// wave-load can do where padding would not fit.
// how far (log2 units) a row's running maximum may rise above the reference point of
// its probabilities before O and l are rescaled to it
constexpr float ATTN_RESCALE_LAG = 8.f;
template <int DH> struct DmaTile {
  static constexpr int PAGE_B = 16 * DH * 2;   // one page of one kv head, K or V
  static constexpr int TILE_B = 4 * PAGE_B;    // K pages 0, 1, then V pages 0, 1
  static constexpr int NLD = TILE_B / 1024;    // 1 KB wave-loads per tile
  static constexpr int LPP = PAGE_B / 1024;    // wave-loads per page
  static constexpr int KROWB = 2 * DH;         // bytes of one key (token) row
};
// chunk c of key k (0..31 in the tile) sits at chunk c ^ kswz(k) of its row
template <int DH> SDV_DEV int kswz(int k) {
  if constexpr (DH == 128) return (k & 3) | (((k >> 3) & 3) << 2);
  else return ((k >> 1) & 1) | (((k >> 3) & 3) << 1);
}

// waves per SIMD the register budget of attn_dma aims at (one query tile per wave):
// three at dh 128, four at dh 64
template <int DH> constexpr int dma_waves() { return DH == 128 ? 3 : 4; }

template <int DH, int NQW, int NW, int R>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(dma_waves<DH>())))
void attn_dma(AttnArgs a) {
  static_assert(NQW == 1, "one query tile per wave");
  using T = bf16;
  using G = DmaTile<DH>;
  constexpr int KT = 32, VE = 8, KS = 32, PE = 8, NH = 2, QP = 2;
  constexpr int LPW = G::NLD / NW;             // wave-loads per wave per tile
  static_assert(G::NLD % NW == 0, "tile loads split evenly over the waves");
  constexpr int RING_B = R * G::TILE_B;
  __shared__ __attribute__((aligned(1024))) char ring[RING_B > ATTN_MERGE_FLOATS * 4 ? RING_B : ATTN_MERGE_FLOATS * 4];
  __shared__ __attribute__((aligned(8))) int sPage[ATTN_MAX_PAGES];

  const int split = blockIdx.z, g = blockIdx.x, b = blockIdx.y / a.n_qg;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q_base = (blockIdx.y % a.n_qg) * NW * NQW;
  const int r = lane & 15, lg = lane >> 4;
  const int Gq = a.H / a.Hkv;
  const int C = min(max(a.seq_len[b], 0), a.max_ctx);
  const int nkeys = C + a.T;
  const int nq = a.T * Gq;
  const int NQT = (nq + 15) >> 4;
  const int k_begin = split * a.split_keys;
  const int k_end = min(nkeys, k_begin + a.split_keys);
  const int32_t* bt = a.block_table + (size_t)b * a.max_blocks;
  const char* kp = (const char*)a.k_pages + (size_t)g * G::PAGE_B;
  const char* vp = (const char*)a.v_pages + (size_t)g * G::PAGE_B;
  const size_t page_stride = (size_t)a.Hkv * G::PAGE_B;

  u32x4 qreg[NQW][DH / KS][QP];
  uint32_t anc[NQW][4];
  float mrun[NQW], lrun[NQW];
  f32x4 acc[NQW][DH / 16];
#pragma unroll
  for (int j = 0; j < NQW; ++j) {
    const int qi = (q_base + w + j * NW) * 16 + r;
    const bool ok = qi < nq;
    const int t = ok ? qi / Gq : 0;
    const int h = g * Gq + (ok ? qi % Gq : 0);
    load_q<true, DH, KS, VE>(a.q, ((size_t)(b * a.T + t) * a.H + h) * DH, ok, lg, qreg[j]);
#pragma unroll
    for (int c = 0; c < 4; ++c) anc[j][c] = a.anc[t * 4 + c];
    mrun[j] = -1e30f;
    lrun[j] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) acc[j][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  stage_pages(a, bt, k_begin, sPage);   // sPage[i]: page k_begin / 16 + i

  // this wave's wave-loads of a tile: u = w + NW * i; the LDS offset inside the tile and
  // this lane's offset inside the source page (the inverse of the chunk permutation)
  int ld_lds[LPW], ld_src[LPW], ld_part[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int u = w + NW * i;
    const int part = u / G::LPP, sub = u % G::LPP;
    const int o = sub * 1024 + lane * 16;       // byte offset of this lane's 16 bytes in the page
    ld_part[i] = part;
    ld_lds[i] = part * G::PAGE_B + sub * 1024;
    if (part < 2) {
      const int row = o / G::KROWB, cl = (o % G::KROWB) >> 4;
      ld_src[i] = row * G::KROWB + ((cl ^ kswz<DH>(part * 16 + row)) << 4);
    } else {
      ld_src[i] = o;   // values keep the page's layout
    }
  }
  // the two physical pages of tile t of the split in one LDS read (k_begin is a
  // multiple of 32, so the pair is 8-byte aligned)
  auto pages_of = [&](int t) { return *(const int2*)&sPage[2 * t]; };
  // bit k set: the k-th newest issued tile had a page outside the table, so the wave
  // issued fewer loads for it than LPW and the counter waits must not count on them
  uint32_t short_tiles = 0;
  auto issue = [&](int2 ph, int slot) {
    char* dst = ring + slot * G::TILE_B;
    const int ph0 = __builtin_amdgcn_readfirstlane(ph.x), ph1 = __builtin_amdgcn_readfirstlane(ph.y);
    short_tiles = (short_tiles << 1) | ((ph0 < 0 || ph1 < 0) ? 1u : 0u);
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int part = ld_part[i];
      const int phys = (part & 1) ? ph1 : ph0;
      if (phys >= 0) {
        const char* src = (part < 2 ? kp : vp) + (size_t)phys * page_stride + ld_src[i];
        lds_dma16(src, dst + ld_lds[i]);
      } else {
        *(u32x4*)(dst + ld_lds[i] + lane * 16) = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  // per-lane LDS offsets of the MFMA operands inside a tile
  int koff[NH][DH / KS], voff[DH / 16];
  {
    const int krow0 = 8 * (r >> 2) + (r & 3);
#pragma unroll
    for (int hv = 0; hv < NH; ++hv) {
      const int key = krow0 + 4 * hv;
#pragma unroll
      for (int ks = 0; ks < DH / KS; ++ks)
        koff[hv][ks] = (key >> 4) * G::PAGE_B + (key & 15) * G::KROWB + (((ks * 4 + lg) ^ kswz<DH>(key)) << 4);
    }
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) {
      const int row = dt * 16 + r;
      voff[dt] = (2 + (lg >> 1)) * G::PAGE_B + row * 32 + ((lg & 1) << 4);
    }
  }

  const int nj = min(NQW, max(0, (NQT - (q_base + w) + NW - 1) / NW));
  const int n_tiles = k_begin < k_end ? (k_end - k_begin + KT - 1) / KT : 0;

  // tile `t` has landed in its slot and every wave sees it, and every wave is done with
  // tile t - 1 (with the dead values of the tile holding the sequence end zeroed).
  // `later` tiles issued after t may stay in flight: their loads are the wave's newest,
  // so waiting until at most later * LPW loads are outstanding leaves exactly those
  // (later = R - 2, else 0: wait for all; also 0 when one of those tiles had a page
  // outside the table, whose loads were not issued)
  auto land = [&](int t, int later) {
    if (later == R - 2 && (short_tiles & ((1u << (R - 2)) - 1u)) == 0u) vmem_lds_wait<(R - 2) * LPW>();
    else vmem_lds_wait<0>();
    bare_barrier();
    const int kt0 = k_begin + t * KT;
    if (kt0 + KT > nkeys) {
      const int j0 = nkeys - kt0;
      char* vs = ring + (t % R) * G::TILE_B + 2 * G::PAGE_B;
      for (int e = threadIdx.x; e < (KT - j0) * DH; e += 64 * NW) {
        const int j = j0 + e / DH, row = e % DH;
        const int tok = j & 15;
        *(uint16_t*)(vs + (j >> 4) * G::PAGE_B + row * 32 + tok * 2) = 0;
      }
      vmem_lds_wait<0>();
      bare_barrier();
    }
  };

  vmem_wait_all();   // the query loads are complete before the ring starts
#pragma unroll
  for (int u = 0; u < R - 1; ++u)
    if (u < n_tiles) issue(pages_of(u), u);
  // pages of the tile the loop issues next, read a whole tile ahead so the read's
  // latency is never waited on
  int2 ph_next = pages_of(min(R - 1, max(n_tiles - 1, 0)));
  for (int it = 0; it < n_tiles; ++it) {
    const int kt0 = k_begin + it * KT;
    // issued so far: tiles up to min(it + R - 2, n_tiles - 1)
    land(it, it + R - 2 <= n_tiles - 1 ? R - 2 : 0);
    // the slot of tile it - 1 is free: refill it with tile it + R - 1
    if (it + R - 1 < n_tiles) issue(ph_next, (it + R - 1) % R);
    ph_next = pages_of(min(it + R, n_tiles - 1));
    if (nj == 0) continue;   // a wave without query tiles only stages K/V
    const char* sl = ring + (it % R) * G::TILE_B;
    const bool edge = kt0 + KT > C || kt0 + KT > k_end;   // the tile reaches the chunk rows or the split end

    u32x4 kk[DH / KS][NH];
    f32x4 sc[NQW][NH];
    float sv[NQW][PE];
    float mnew[NQW];
    u32x4 pop[NQW][QP];
    u32x4 va[DH / 16];
    auto read_k = [&]() {
#pragma unroll
      for (int ks = 0; ks < DH / KS; ++ks)
#pragma unroll
        for (int hv = 0; hv < NH; ++hv) kk[ks][hv] = *(const u32x4*)(sl + koff[hv][ks]);
    };
    auto read_v = [&]() {
#pragma unroll
      for (int dt = 0; dt < DH / 16; ++dt) va[dt] = *(const u32x4*)(sl + voff[dt]);
    };
    // S^T of query tile j
    auto scores = [&](int j) {
#pragma unroll
      for (int hv = 0; hv < NH; ++hv) sc[j][hv] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DH / KS; ++ks)
#pragma unroll
        for (int qp = 0; qp < QP; ++qp)
#pragma unroll
          for (int hv = 0; hv < NH; ++hv) sc[j][hv] = mma16<T>(kk[ks][hv], qreg[j][ks][qp], sc[j][hv]);
    };
    // the lane's 8 scores of tile j, masked where the tile needs it (wave-uniform test);
    // the row maxima; true where a row's maximum leaves the reference point behind.
    // The reference point mrun of a row moves up to the row's maximum only when that
    // maximum exceeds it by more than ATTN_RESCALE_LAG (log2 units); until then the
    // probabilities are taken against the old reference and stay below
    // 2^ATTN_RESCALE_LAG, so most tiles skip the rescale of O and l.  O / l and the
    // split merge are the same for any reference point.
    auto row_max = [&](int j) {
#pragma unroll
      for (int hv = 0; hv < NH; ++hv)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[j][4 * hv + i] = sc[j][hv][i];
      if (edge) {
#pragma unroll
        for (int e = 0; e < PE; ++e) {
          const int sl_ = kt0 + PE * lg + e;
          const bool live = sl_ < k_end;
          const int jr = max(sl_ - C, 0);
          const bool vis = live & ((sl_ < C) | (((anc_word(anc[j], jr >> 5) >> (jr & 31)) & 1u) != 0u));
          sv[j][e] = vis ? sv[j][e] : -INFINITY;
        }
      }
      float mx = sv[j][0];
#pragma unroll
      for (int e = 1; e < PE; ++e) mx = fmaxf(mx, sv[j][e]);
      mx = pair32_max(pair16_max(mx));
      mnew[j] = fmaxf(mrun[j], mx);
      return mnew[j] > mrun[j] + ATTN_RESCALE_LAG;
    };
    auto rescale = [&](int j) {
      const float alpha = __builtin_amdgcn_exp2f(mrun[j] - mnew[j]);
      mrun[j] = mnew[j];
      lrun[j] *= alpha;
#pragma unroll
      for (int dt = 0; dt < DH / 16; ++dt) acc[j][dt] *= alpha;
    };
    // probabilities of tile j as the hi/lo operand pair; the row sums
    auto probs = [&](int j) {
      float pj[PE];
#pragma unroll
      for (int e = 0; e < PE; ++e) pj[e] = __builtin_amdgcn_exp2f(sv[j][e] - mrun[j]);
      lrun[j] += ((pj[0] + pj[1]) + (pj[2] + pj[3])) + ((pj[4] + pj[5]) + (pj[6] + pj[7]));
      split_probs_pk(pj, pop[j][0], pop[j][1]);
    };
    // O^T += V^T P^T of tile j
    auto pv = [&](int j) {
#pragma unroll
      for (int dt = 0; dt < DH / 16; ++dt)
#pragma unroll
        for (int qp = 0; qp < QP; ++qp) acc[j][dt] = mma16<T>(va[dt], pop[j][qp], acc[j][dt]);
    };

    // scores of every query tile of the wave with all K operands read first, the V
    // operands read while the softmax runs, then P V
    read_k();
#pragma unroll
    for (int j = 0; j < NQW; ++j) {
      if (j == 0 || j < nj) {
        scores(j);
        if (j == 0) {
          __builtin_amdgcn_sched_group_barrier(0x100, DH / KS * NH, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, DH / KS * QP * NH, 0);
        }
      } else {
#pragma unroll
        for (int hv = 0; hv < NH; ++hv) sc[j][hv] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    read_v();
    bool rise = false;
#pragma unroll
    for (int j = 0; j < NQW; ++j) rise |= row_max(j);
    if (__any(rise)) {
#pragma unroll
      for (int j = 0; j < NQW; ++j) rescale(j);
    }
#pragma unroll
    for (int j = 0; j < NQW; ++j) probs(j);
#pragma unroll
    for (int j = 0; j < NQW; ++j)
      if (j == 0 || j < nj) pv(j);
  }
  __syncthreads();   // every wave is done with the ring (its memory is the merge scratch)

  // ---- the split's partial state (or, with a single split, the output rows)
  const bool fused = a.sem != nullptr;
  const bool direct = fused && a.n_splits == 1;
  const size_t grp = ((size_t)b * a.Hkv + g) * a.n_splits * a.nq_pad;
  const rsrc_t rpo = dev_rsrc(a.po + grp * DH, (uint32_t)a.n_splits * a.nq_pad * DH * 4);
  const rsrc_t rml = dev_rsrc(a.pml + grp * 2, (uint32_t)a.n_splits * a.nq_pad * 8);
#pragma unroll
  for (int j = 0; j < NQW; ++j) {
    const int qt = q_base + w + j * NW;
    if (qt >= NQT) continue;
    float l = lrun[j];
    l = pair32_sum(pair16_sum(l));
    const int qi = qt * 16 + r;
    const uint32_t pr = (uint32_t)(split * a.nq_pad + qi);
    if (direct) {
      if (qi < nq) {
        const float inv = 1.f / l;
        const int orow = b * a.T + qi / Gq;
        const int h = g * Gq + qi % Gq;
#pragma unroll
        for (int dt = 0; dt < DH / 16; ++dt) {
          const float v[4] = {acc[j][dt][0] * inv, acc[j][dt][1] * inv, acc[j][dt][2] * inv, acc[j][dt][3] * inv};
          act_store4<T>(a.o, a.H * DH, orow, h * DH + dt * 16 + 4 * lg, v);
        }
      }
    } else {
#pragma unroll
      for (int dt = 0; dt < DH / 16; ++dt)
        st_dev16(rpo, (pr * DH + dt * 16 + 4 * lg) * 4, __builtin_bit_cast(u32x4, acc[j][dt]));
      if (lg == 0) st_dev8(rml, pr * 8, u32x2{__float_as_uint(mrun[j]), __float_as_uint(l)});
    }
  }
  if (!fused || direct) return;
  __shared__ int is_last;
  const int qg = blockIdx.y % a.n_qg;
  if (!arrive_last(a.sem + ((size_t)b * a.Hkv + g) * a.n_qg + qg, a.n_splits, &is_last)) return;
  if (a.n_splits <= 8) attn_merge8<T, DH>(a, b, g, q_base * 16, min(nq, (q_base + NW * NQW) * 16));
  else attn_merge<T, DH>(a, b, g, q_base * 16, min(nq, (q_base + NW * NQW) * 16), (float*)ring);
}

// Register path for few query tiles per kv head (at most 3): every wave holds all
// query tiles of the head (pre-scaled by log2(e)/sqrt(dh)) and streams its own
// interleaved key tiles straight from the pages into MFMA operands (two waves per
// SIMD; the next tile's operands are loaded as soon as the current ones are read).
// Per tile the score MFMAs of all query tiles are interleaved; the visibility mask is
// evaluated only on tiles that reach the chunk rows or the end of the split; the
// accumulators are rescaled only when some row's running maximum rises.  The 4 waves
// of the workgroup merge their states through LDS and write one partial per split.
template <typename T, int DH, int NQT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attn_reg(AttnArgs a) {
  constexpr bool BF = sizeof(T) == 2;
  constexpr int VE = Vec16<T>::N;
  constexpr int KS = 4 * VE;
  constexpr int KT = BF ? 32 : 16;
  constexpr int PE = BF ? 8 : 4;
  constexpr int NH = BF ? 2 : 1;                  // 16-key halves of a tile
  constexpr int NKA = NH * (DH / KS);             // K operand loads per tile
  constexpr int NVA = DH / 16;                    // V operand loads per tile
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, r = lane & 15, lg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = a.H / a.Hkv;
  const int C = min(max(a.seq_len[b], 0), a.max_ctx);
  const int nkeys = C + a.T;
  const int nq = a.T * G;
  const int k_begin = split * a.split_keys;
  const int k_end = min(nkeys, k_begin + a.split_keys);
  const int ntiles = k_end > k_begin ? (k_end - k_begin + KT - 1) / KT : 0;
  const int32_t* bt = a.block_table + (size_t)b * a.max_blocks;
  const T* kp = (const T*)a.k_pages;
  const T* vp = (const T*)a.v_pages;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  // the queries are loaded before the page table is staged, so both round trips overlap
  constexpr int QP = BF ? 2 : 1;
  u32x4 qreg[NQT][DH / KS][QP];
  uint32_t anc[NQT][4];
  float mrun[NQT], lrun[NQT];
  f32x4 acc[NQT][DH / 16];
#pragma unroll
  for (int j = 0; j < NQT; ++j) {
    const int qi = j * 16 + r;
    const bool ok = qi < nq;
    const int t = ok ? qi / G : 0;
    const int h = g * G + (ok ? qi % G : 0);
    load_q<BF, DH, KS, VE>(a.q, ((size_t)(b * a.T + t) * a.H + h) * DH, ok, lg, qreg[j]);
#pragma unroll
    for (int c = 0; c < 4; ++c) anc[j][c] = a.anc[t * 4 + c];
    mrun[j] = -1e30f;
    lrun[j] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) acc[j][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __shared__ int sPage[ATTN_MAX_PAGES];
  const int pg0 = stage_pages(a, bt, k_begin, sPage);

  // K and V^T operands of key tile `it` (relative to k_begin).  Loads are branch-free:
  // a slot past the split end reads the split's last valid slot instead (its scores
  // are masked and, past the sequence end, its values zeroed in compute_tile); a
  // page whose table entry is out of range reads page 0 and is treated the same way.
  const int last = max(k_end - 1, k_begin);
  auto page_of = [&](int slot) {
    const int ph = sPage[(min(slot, last) >> 4) - pg0];
    return ph < 0 ? 0 : ph;
  };
  auto load_k = [&](int it, u32x4 (&ko)[NKA]) {
    const int kt0 = k_begin + min(it, max(ntiles - 1, 0)) * KT;
    // K rows: a bf16 tile has two 16-key halves whose rows map to keys 8*(r/4) + r%4 (+4)
#pragma unroll
    for (int hv = 0; hv < NH; ++hv) {
      const int key = BF ? 8 * (r >> 2) + (r & 3) + 4 * hv : r;
      const int slot = min(kt0 + key, last);
      const T* src = kp + (((size_t)page_of(slot) * a.Hkv + g) * 16 + (slot & 15)) * DH + lg * VE;
#pragma unroll
      for (int ks = 0; ks < DH / KS; ++ks) ko[hv * (DH / KS) + ks] = ld16(src + ks * KS);
    }
  };
  auto load_v = [&](int it, u32x4 (&vo)[NVA]) {
    const int kt0 = k_begin + min(it, max(ntiles - 1, 0)) * KT;
    // V^T: lane holds dh row dt*16 + r for keys PE*lg .. PE*lg + PE - 1 (one page)
    const int slot0 = min(kt0 + PE * lg, last & ~(PE - 1));
    const T* vsrc = vp + (((size_t)page_of(slot0) * a.Hkv + g) * DH + r) * 16 + (slot0 & 15);
#pragma unroll
    for (int dt = 0; dt < NVA; ++dt) vo[dt] = ld16(vsrc + (size_t)dt * 16 * 16);
  };

  // One register set per wave: the next tile's K is loaded as soon as the score
  // MFMAs have read the current one, its V after P V (two waves per SIMD cover the
  // latency).
  auto compute_tile = [&](int it, u32x4 (&ko)[NKA], u32x4 (&vo)[NVA]) {
    const int kt0 = k_begin + it * KT;
    f32x4 sc[NQT][NH];
#pragma unroll
    for (int j = 0; j < NQT; ++j)
#pragma unroll
      for (int hv = 0; hv < NH; ++hv) sc[j][hv] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < DH / KS; ++ks)
#pragma unroll
      for (int qp = 0; qp < QP; ++qp)
#pragma unroll
        for (int j = 0; j < NQT; ++j)
#pragma unroll
          for (int hv = 0; hv < NH; ++hv) sc[j][hv] = mma16<T>(ko[hv * (DH / KS) + ks], qreg[j][ks][qp], sc[j][hv]);
    load_k(it + 4, ko);
    float sv[NQT][PE];
#pragma unroll
    for (int j = 0; j < NQT; ++j)
#pragma unroll
      for (int hv = 0; hv < NH; ++hv)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[j][4 * hv + i] = sc[j][hv][i];
    // only tiles that reach the chunk rows (tree / causal mask), the split end or a
    // page with an out-of-range table entry need a mask (wave-uniform test)
    bool bad_page = false;
#pragma unroll
    for (int pp = 0; pp < KT / 16; ++pp) {
      const int sl = kt0 + pp * 16;
      bad_page |= sl <= last && sPage[(sl >> 4) - pg0] < 0;
    }
    if (kt0 + KT > C || kt0 + KT > k_end || bad_page) {
#pragma unroll
      for (int e = 0; e < PE; ++e) {
        // straight-line visibility (no short-circuit branches): inside the split, on
        // a valid page, and a cached slot or an ancestor-or-self chunk row
        const int sl = kt0 + PE * lg + e;
        const bool live = (sl < k_end) & (sPage[(min(sl, last) >> 4) - pg0] >= 0);
        const int jr = max(sl - C, 0);
#pragma unroll
        for (int j = 0; j < NQT; ++j) {
          const bool vis = live & ((sl < C) | (((anc_word(anc[j], jr >> 5) >> (jr & 31)) & 1u) != 0u));
          sv[j][e] = vis ? sv[j][e] : -INFINITY;
        }
      }
      // values of keys that are not real cache rows (past the sequence end or on an
      // invalid page) may hold anything; zero them so 0 * value stays 0
      const int sl0 = kt0 + PE * lg;
      const bool pg_ok = sl0 <= last && sPage[(sl0 >> 4) - pg0] >= 0;
#pragma unroll
      for (int dt = 0; dt < NVA; ++dt) {
        T e8[VE];
        __builtin_memcpy(e8, &vo[dt], 16);
#pragma unroll
        for (int i = 0; i < VE; ++i) e8[i] = (pg_ok & (sl0 + i < k_end)) ? e8[i] : T(0);
        __builtin_memcpy((void*)&vo[dt], e8, 16);
      }
    }
    float mnew[NQT];
    bool rise = false;
#pragma unroll
    for (int j = 0; j < NQT; ++j) {
      float mx = sv[j][0];
#pragma unroll
      for (int e = 1; e < PE; ++e) mx = fmaxf(mx, sv[j][e]);
      mx = pair32_max(pair16_max(mx));
      mnew[j] = fmaxf(mrun[j], mx);
      rise |= mnew[j] > mrun[j] + ATTN_RESCALE_LAG;   // the lazy reference point of attn_dma
    }
    if (__any(rise)) {
#pragma unroll
      for (int j = 0; j < NQT; ++j) {
        const float alpha = __builtin_amdgcn_exp2f(mrun[j] - mnew[j]);
        mrun[j] = mnew[j];
        lrun[j] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DH / 16; ++dt) acc[j][dt] *= alpha;
      }
    }
#pragma unroll
    for (int j = 0; j < NQT; ++j) {
      float p[PE];
#pragma unroll
      for (int e = 0; e < PE; ++e) p[e] = __builtin_amdgcn_exp2f(sv[j][e] - mrun[j]);
      if constexpr (PE == 8) lrun[j] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      else {
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < PE; ++e) ps += p[e];
        lrun[j] += ps;
      }
      if constexpr (BF) {
        u32x4 phi, plo;
        split_probs_pk(p, phi, plo);
#pragma unroll
        for (int dt = 0; dt < DH / 16; ++dt) {
          acc[j][dt] = mma16<T>(vo[dt], phi, acc[j][dt]);
          acc[j][dt] = mma16<T>(vo[dt], plo, acc[j][dt]);
        }
      } else {
        u32x4 pb;
        pb.x = __float_as_uint(p[0]); pb.y = __float_as_uint(p[1]);
        pb.z = __float_as_uint(p[2]); pb.w = __float_as_uint(p[3]);
#pragma unroll
        for (int dt = 0; dt < DH / 16; ++dt) acc[j][dt] = mma16<T>(vo[dt], pb, acc[j][dt]);
      }
    }
    load_v(it + 4, vo);
  };

  // tiles w, w+4, w+8, ... of the split
  u32x4 kA[NKA], vA[NVA];
  load_k(w, kA);
  load_v(w, vA);
  for (int it = w; it < ntiles; it += 4) compute_tile(it, kA, vA);

  // ---- merge the 4 waves: LDS holds each wave's (m, l) and O^T accumulators
  __shared__ float sm[4][NQT][64], sl[4][NQT][64];
  __shared__ float so[4][NQT][DH / 16][4][64];
#pragma unroll
  for (int j = 0; j < NQT; ++j) {
    float l = lrun[j];
    l = pair32_sum(pair16_sum(l));
    sm[w][j][lane] = mrun[j];
    sl[w][j][lane] = l;
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) so[w][j][dt][i][lane] = acc[j][dt][i];
  }
  __syncthreads();
  // the split's partial state (or, with a single split, the output rows)
  const bool fused = a.sem != nullptr;
  const bool direct = fused && a.n_splits == 1;
  const size_t grp = ((size_t)b * a.Hkv + g) * a.n_splits * a.nq_pad;
  const rsrc_t rpo = dev_rsrc(a.po + grp * DH, (uint32_t)a.n_splits * a.nq_pad * DH * 4);
  const rsrc_t rml = dev_rsrc(a.pml + grp * 2, (uint32_t)a.n_splits * a.nq_pad * 8);
  for (int idx = threadIdx.x; idx < NQT * 64; idx += 256) {
    const int j = idx / 64, ln = idx % 64;
    const int qi = j * 16 + (ln & 15);
    float M = sm[0][j][ln];
#pragma unroll
    for (int k = 1; k < 4; ++k) M = fmaxf(M, sm[k][j][ln]);
    float wk[4], L = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) { wk[k] = exp2f(sm[k][j][ln] - M); L += wk[k] * sl[k][j][ln]; }
    const uint32_t pr = (uint32_t)(split * a.nq_pad + qi);
    const float inv = 1.f / L;
    const int orow = b * a.T + min(qi, nq - 1) / G;
    const int h = g * G + qi % G;
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[i] = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) v[i] += wk[k] * so[k][j][dt][i][ln];
      }
      const int d0 = dt * 16 + 4 * (ln >> 4);
      if (direct) {
        if (qi < nq) {
          const float vo[4] = {v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv};
          act_store4<T>(a.o, a.H * DH, orow, h * DH + d0, vo);
        }
      } else {
        st_dev16(rpo, (pr * DH + d0) * 4,
                 u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])});
      }
    }
    if (!direct && (ln >> 4) == 0) st_dev8(rml, pr * 8, u32x2{__float_as_uint(M), __float_as_uint(L)});
  }
  if (!fused || direct) return;
  __shared__ int is_last;
  if (!arrive_last(a.sem + (size_t)b * a.Hkv + g, a.n_splits, &is_last)) return;
  if (a.n_splits <= 8) attn_merge8<T, DH>(a, b, g, 0, nq);
  else attn_merge<T, DH>(a, b, g, 0, nq, &so[0][0][0][0][0]);
}

// Split merge as its own kernel (many splits or large merges): item (row, head) of
// the chunk takes DH / 4 threads, each owning 4 consecutive output values; a thread
// loads every split's (m, l) pair and 16-byte output chunk in one round, then sums
// the splits in order.
// MAXS: registers for that many splits (the launch takes the smallest of 8, 16, 32
// that holds n_splits; room for 32 would cost two waves per SIMD)
template <typename T, int DH, int MAXS>
__global__ __launch_bounds__(256) void attn_combine(CombineArgs a) {
  constexpr int TPI = DH / 4;   // threads per item
  const int item = blockIdx.x * (256 / TPI) + threadIdx.x / TPI;
  const int c4 = threadIdx.x % TPI;
  if (item >= a.B * a.T * a.H) return;
  const int row = item / a.H, h = item % a.H;
  const int b = row / a.T, t = row % a.T;
  const int G = a.H / a.Hkv, g = h / G, qi = t * G + h % G;
  const size_t base0 = (((size_t)b * a.Hkv + g) * a.n_splits) * a.nq_pad + qi;
  float2 ml[MAXS];
  float4 v[MAXS];
#pragma unroll
  for (int s = 0; s < MAXS; ++s) {
    if (s < a.n_splits) {
      const size_t bs = base0 + (size_t)s * a.nq_pad;
      ml[s] = *(const float2*)(a.pml + bs * 2);
      v[s] = *(const float4*)(a.po + bs * DH + 4 * c4);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < MAXS; ++s)
    if (s < a.n_splits) M = fmaxf(M, ml[s].x);
  float den = 0.f, num[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < MAXS; ++s) {
    if (s < a.n_splits) {
      const float wgt = exp2f(ml[s].x - M);
      den += wgt * ml[s].y;
      num[0] += wgt * v[s].x;
      num[1] += wgt * v[s].y;
      num[2] += wgt * v[s].z;
      num[3] += wgt * v[s].w;
    }
  }
  const float out[4] = {num[0] / den, num[1] / den, num[2] / den, num[3] / den};
  act_store4<T>(a.o, a.H * DH, row, h * DH + 4 * c4, out);
}

// the register path serves heads with few query tiles (its merge buffers and
// operands grow with NQT and dh)
bool attn_uses_reg_path(bool bf, int dh, int NQT) {
  if (dh == 64) return NQT <= (bf ? 3 : 2);
  return NQT <= 1;
}

// query tiles per wave that fit without register spills
template <typename T, int DH> constexpr int attn_cap() {
  return DH == 128 ? 2 : 3;
}

// query tiles per group when the (sequence, kv head) pairs alone fill the GPU
#ifndef SDV_ATTN_WIDE_GROUP_TILES
#define SDV_ATTN_WIDE_GROUP_TILES 4
#endif
// (sequence, kv head) pairs from which groups are limited to SDV_ATTN_WIDE_GROUP_TILES
#ifndef SDV_ATTN_WIDE_HEADS
#define SDV_ATTN_WIDE_HEADS 256
#endif
// query tiles per group of the bf16 (LDS DMA) path below that: small groups and more
// key splits keep three workgroups resident per CU (8B tree pass: 51 -> 42 us)
#ifndef SDV_ATTN_FEW_GROUP_TILES
#define SDV_ATTN_FEW_GROUP_TILES 3
#endif
// tiles in the LDS ring of attn_dma
#ifndef SDV_ATTN_RING
#define SDV_ATTN_RING 3
#endif

template <typename T, int DH>
int attn_shape(int NQT, int heads, int* nqw_out, int* nw_out) {
  // bf16 stages K/V by LDS DMA, whose wave-loads split evenly over 4 or 8 waves, one
  // query tile per wave (its registers leave room for three waves per SIMD)
  constexpr bool DMA = sizeof(T) == 2;
  constexpr int CAP = DMA ? 1 : attn_cap<T, DH>();
  // query groups of at most 8 waves x CAP tiles -- of at most 4 tiles (one per SIMD)
  // when the (sequence, kv head) pairs alone fill the GPU (heads >= 256: no key splits
  // are needed, and a shorter busiest SIMD beats reading the keys and values once per
  // group; measured on the batched 64-row pass); inside a group, the shape whose
  // busiest SIMD (wave w runs on SIMD w % 4, and takes tiles w, w + nw, ...) carries
  // the fewest query tiles per key tile, then the fewest tiles per wave (registers),
  // then the fewest waves; at least 4 waves (waves without query tiles still stage K/V)
  constexpr int WG = SDV_ATTN_WIDE_GROUP_TILES;
  constexpr int FG = SDV_ATTN_FEW_GROUP_TILES;
  const int n_qg = std::max((NQT + 8 * CAP - 1) / (8 * CAP), heads >= SDV_ATTN_WIDE_HEADS ? (NQT + WG - 1) / WG
                                                             : DMA ? (NQT + FG - 1) / FG : 1);
  const int Q = (NQT + n_qg - 1) / n_qg;
  int best_nw = 8, best_nqw = CAP, best_load = 1 << 30;
  for (int nqw = 1; nqw <= CAP; ++nqw)
    for (int nw = 4; nw <= 8; ++nw) {
      if (nw * nqw < Q || (DMA && nw != 4 && nw != 8)) continue;
      int load[4] = {0, 0, 0, 0};
      for (int w = 0; w < nw; ++w)
        for (int j = 0; j < nqw; ++j)
          if (w + j * nw < Q) ++load[w % 4];
      const int mx = std::max(std::max(load[0], load[1]), std::max(load[2], load[3]));
      if (mx < best_load || (mx == best_load && (nqw < best_nqw || (nqw == best_nqw && nw < best_nw)))) {
        best_load = mx;
        best_nw = nw;
        best_nqw = nqw;
      }
    }
  *nqw_out = best_nqw;
  *nw_out = best_nw;
  return n_qg;
}

int attn_query_groups(bool is_bf16, int dh, int T, int G, int heads, int* rows_per_group) {
  const int NQT = (T * G + 15) / 16;
  if (attn_uses_reg_path(is_bf16, dh, NQT)) {
    *rows_per_group = T * G;
    return 1;
  }
  int nqw, nw, n_qg;
  if (is_bf16)
    n_qg = dh == 64 ? attn_shape<bf16, 64>(NQT, heads, &nqw, &nw) : attn_shape<bf16, 128>(NQT, heads, &nqw, &nw);
  else
    n_qg = dh == 64 ? attn_shape<float, 64>(NQT, heads, &nqw, &nw) : attn_shape<float, 128>(NQT, heads, &nqw, &nw);
  *rows_per_group = std::min(T * G, nw * nqw * 16);
  return n_qg;
}

// A launch that records ev0 when the kernel starts and ev1 when it ends (both
// nullable: a plain launch).
template <typename K, typename Arg>
static void launch_ev(K kernel, dim3 grid, dim3 block, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1, const Arg& a) {
  if (ev0 || ev1) hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev0, ev1, 0, a);
  else kernel<<<grid, block, 0, s>>>(a);
}

template <typename T, int DH>
static hipError_t launch_attn_t(AttnArgs a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  const int G = a.H / a.Hkv;
  const int NQT = (a.T * G + 15) / 16;
  if (attn_uses_reg_path(sizeof(T) == 2, DH, NQT)) {
    dim3 grid(a.n_splits, a.Hkv, a.B);
    a.n_qg = 1;
    if constexpr (DH == 128) {
      launch_ev(attn_reg<T, DH, 1>, grid, 256, s, ev0, ev1, a);   // the register path takes one query tile at dh 128
    } else {
      switch (NQT) {
        case 1: launch_ev(attn_reg<T, DH, 1>, grid, 256, s, ev0, ev1, a); break;
        case 2: launch_ev(attn_reg<T, DH, 2>, grid, 256, s, ev0, ev1, a); break;
        default: launch_ev(attn_reg<T, DH, 3>, grid, 256, s, ev0, ev1, a); break;
      }
    }
    return hipGetLastError();
  }
  int nqw, nw;
  a.n_qg = attn_shape<T, DH>(NQT, a.B * a.Hkv, &nqw, &nw);
  // workgroups go out in order of their linear index, x fastest: kv heads, then
  // (sequence, query group), then key splits, so every sequence's first split (the
  // longest) starts before any later split and the short ones fill the tail; the
  // workgroups of one kv head land on one XCD (index mod 8) and share its L2
  dim3 grid(a.Hkv, a.B * a.n_qg, a.n_splits);
  if constexpr (sizeof(T) == 2) {
    constexpr int R = SDV_ATTN_RING;
    if (nqw != 1) return hipErrorInvalidValue;
    if (nw == 4) launch_ev(attn_dma<DH, 1, 4, R>, grid, 256, s, ev0, ev1, a);
    else if (nw == 8) launch_ev(attn_dma<DH, 1, 8, R>, grid, 512, s, ev0, ev1, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
  dim3 block(64 * nw);
  switch (nqw) {
    case 1: launch_ev(attn_chunk<T, DH, 1>, grid, block, s, ev0, ev1, a); break;
    case 2: launch_ev(attn_chunk<T, DH, 2>, grid, block, s, ev0, ev1, a); break;
    case 3:
      if constexpr (attn_cap<T, DH>() >= 3) { launch_ev(attn_chunk<T, DH, 3>, grid, block, s, ev0, ev1, a); break; }
      return hipErrorInvalidValue;
    case 4:
      if constexpr (attn_cap<T, DH>() >= 4) { launch_ev(attn_chunk<T, DH, 4>, grid, block, s, ev0, ev1, a); break; }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attention(bool is_bf16, int dh, const AttnArgs& a, hipStream_t s, hipEvent_t ev0,
                            hipEvent_t ev1) {
  if (is_bf16) return dh == 64 ? launch_attn_t<bf16, 64>(a, s, ev0, ev1) : launch_attn_t<bf16, 128>(a, s, ev0, ev1);
  return dh == 64 ? launch_attn_t<float, 64>(a, s, ev0, ev1) : launch_attn_t<float, 128>(a, s, ev0, ev1);
}

hipError_t launch_combine(bool is_bf16, const CombineArgs& a, hipStream_t s, hipEvent_t ev1) {
  if (a.n_splits > 32) return hipErrorInvalidValue;
  const int items = a.B * a.T * a.H;
  const int grid = (items + 256 / (a.dh / 4) - 1) / (256 / (a.dh / 4));
  auto go = [&](auto t_tag, auto dh_tag) {
    using T = decltype(t_tag);
    constexpr int DH = decltype(dh_tag)::value;
    if (a.n_splits <= 8) launch_ev(attn_combine<T, DH, 8>, grid, 256, s, nullptr, ev1, a);
    else if (a.n_splits <= 16) launch_ev(attn_combine<T, DH, 16>, grid, 256, s, nullptr, ev1, a);
    else launch_ev(attn_combine<T, DH, 32>, grid, 256, s, nullptr, ev1, a);
  };
  using D64 = std::integral_constant<int, 64>;
  using D128 = std::integral_constant<int, 128>;
  if (is_bf16) {
    if (a.dh == 64) go(bf16{}, D64{});
    else go(bf16{}, D128{});
  } else {
    if (a.dh == 64) go(float{}, D64{});
    else go(float{}, D128{});
  }
  return hipGetLastError();
}

}  // namespace sdv
