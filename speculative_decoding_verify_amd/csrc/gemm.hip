// Weight-streaming GEMM for few rows: out[m, n] = sum_k A[m, k] * W[n, k].
//
// The decoder projections of a verify pass multiply M = B*T (tens of) activation rows
// by weight matrices of tens to hundreds of MB, so every launch is bound by reading W
// from HBM once.  The design serves that stream:
//   * W is packed once at load time into 1 KB tiles (16 rows x one k step) laid out
//     in lane order, so each wave load instruction reads one contiguous kilobyte that
//     is already the B operand of a 16x16 MFMA;
//   * the activations arrive in the operand format too (the tile format of
//     common.h, one contiguous kilobyte per wave load): bf16 models store each value
//     as a bf16 hi/lo pair (two MFMAs; the product carries ~16 significant bits of the
//     activation, only the weights are bf16), fp32 models use the fp32 MFMA;
//   * the four waves of a workgroup take every fourth k step of the workgroup's range;
//     each wave keeps D k steps of loads (W tiles and activation pairs) in flight in
//     registers and consumes the oldest, so HBM sees a steady stream with no
//     workgroup barrier inside the k loop;
//   * the waves' partial tiles are summed through LDS in a fixed order, then one of
//     the epilogues below runs on the finished tile.
// Grid: x = groups of NT weight tiles (16 * NT packed rows), y = splits of K (fp32
// partials summed in split order by the consumer), z = blocks of 16 * MT rows.
//
// Epilogues (all but PARTIAL need the whole K range in one workgroup, S = 1):
//   PARTIAL  fp32 partial sums of each split;
//   QKV      rotary embedding on q and k: packed rows 0-7 of a tile are the first
//            members (element i) and rows 8-15 the second members (element i + dh/2)
//            of 8 rotation pairs; q scaled by log2(e)/sqrt(dh) and written in the
//            query-row format, k and v rounded to the cache type and appended to
//            the paged cache (k token-major, v transposed inside the page) at the
//            page and slot the prologue resolved for the row;
//   SWIGLU   rows 0-7 of a tile are gate rows f, rows 8-15 the up rows of the same f:
//            h = silu(gate) * up, stored in the activation tile format;
//   LOGITS   fp32 logits plus per-(row, column group) statistics: largest value, its
//            index (lowest on ties), second-largest value and sum of exp(v - largest).
#include <hip/hip_ext.h>

#include <algorithm>
#include <type_traits>
#include <utility>

#include "common.h"
#include "kernels.h"

namespace sdv {

// Epilogues on a finished tile (LDS, 16 * MT rows x 16 * NT columns; row m_base + ml,
// packed column group cg).  The q/k/v epilogue takes each item's rotary pair and K/V
// destination from qkv_in(item slot u, row m, element i).
struct QkvItem {
  float2 rope;
  int2 dst;
};

template <typename T, int MT, int NT, int EPI, typename QkvIn>
SDV_DEV void gemm_epilogue(const GemmArgs& a, float (*tile)[16 * NT + 1], int cg, int split, int m_base,
                           QkvIn qkv_in) {
  constexpr int TC = 16 * NT;
  if constexpr (EPI == EPI_PARTIAL) {
    float* out = a.out + (size_t)split * a.out_split_stride;
    for (int idx = threadIdx.x; idx < 16 * MT * TC; idx += 256) {
      const int ml = idx / TC, c = idx % TC;
      const int m = m_base + ml, n = cg * TC + c;
      if (m < a.M && n < a.N) out[(size_t)m * a.ldo + n] = tile[ml][c];
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    for (int idx = threadIdx.x; idx < 16 * MT * NT * 8; idx += 256) {
      const int ml = idx / (NT * 8), pc = idx % (NT * 8);
      const int t = pc >> 3, i = pc & 7;
      const int m = m_base + ml;
      const int f = (cg * NT + t) * 8 + i;
      if (m >= a.M || f >= a.pair_n) continue;
      const float gt = tile[ml][t * 16 + i];
      const float up = tile[ml][t * 16 + 8 + i];
      const float sl = gt / (1.f + expf(-gt));
      act_store1<T>(a.out_act, a.pair_n, m, f, sl * up);
    }
  } else if constexpr (EPI == EPI_QKV) {
    const QkvEpi& e = a.qkv;
    const int half = a.pair_n;  // dh / 2
    const int dh = 2 * half;
    constexpr int QI = (16 * MT * NT * 8 + 255) / 256;
    constexpr int QU = QI <= 8 ? QI : 1;   // unrolled when the items come from registers
#pragma unroll QU
    for (int u = 0; u < QI; ++u) {
      const int idx = threadIdx.x + 256 * u;
      const int ml = idx / (NT * 8), pc = idx % (NT * 8);
      const int t = pc >> 3, ii = pc & 7;
      const int m = m_base + ml;
      const int p = (cg * NT + t) * 8 + ii;  // rotation pair
      const int hh = p / half, i = p % half;  // head (q, k, then v heads) and element
      if (idx >= 16 * MT * NT * 8 || m >= a.M || hh >= e.H + 2 * e.Hkv) continue;
      const float x1 = tile[ml][t * 16 + ii];
      const float x2 = tile[ml][t * 16 + 8 + ii];
      float y1 = x1, y2 = x2;
      const QkvItem in = qkv_in(u, m, i);
      if (hh < e.H + e.Hkv) {
        const float2 cs = in.rope;  // (cos, sin)
        y1 = x1 * cs.x - x2 * cs.y;
        y2 = x2 * cs.x + x1 * cs.y;
      }
      if (hh < e.H) {
        char* qrow = (char*)e.q + (size_t)m * e.H * dh * 4;
        row_store1<T>(qrow, hh * dh + i, y1 * e.q_scale);
        row_store1<T>(qrow, hh * dh + i + half, y2 * e.q_scale);
      } else {
        const int phys = in.dst.x;   // -1: the prologue reported the row
        if (phys < 0) continue;
        const bool is_k = hh < e.H + e.Hkv;
        const int g = is_k ? hh - e.H : hh - e.H - e.Hkv;
        const size_t page = (size_t)phys * e.Hkv + g;
        const int off = in.dst.y;
        if (is_k) {
          T* kp = (T*)e.k_pages + (page * 16 + off) * dh;
          kp[i] = from_f<T>(y1);
          kp[i + half] = from_f<T>(y2);
        } else {
          T* vp = (T*)e.v_pages + page * dh * 16;
          vp[(size_t)i * 16 + off] = from_f<T>(y1);
          vp[(size_t)(i + half) * 16 + off] = from_f<T>(y2);
        }
      }
    }
  } else {  // EPI_LOGITS
    // 8 threads per row, thread j over columns j, j + 8, ...; the 8 partial states
    // meet in a fixed xor butterfly, so every thread of the row ends with the same
    // values: largest (lowest index on ties), second largest (equal to the largest on
    // a tie), then the sum of exp(v - largest).
    const int nc = min(TC, a.N - cg * TC);
    const int sub = threadIdx.x & 7;
    for (int ml0 = 0; ml0 < 16 * MT; ml0 += 32) {
      const int ml = ml0 + (threadIdx.x >> 3);
      const bool row_ok = ml < 16 * MT;
      float m1 = -INFINITY, m2 = -INFINITY;
      int i1 = 0x7fffffff;
      if (row_ok)
        for (int c = sub; c < nc; c += 8) {
          const float v = tile[ml][c];
          if (v > m1) { m2 = m1; m1 = v; i1 = cg * TC + c; }
          else if (v > m2) m2 = v;
        }
#pragma unroll
      for (int o = 1; o < 8; o <<= 1) {
        const float om1 = __shfl_xor(m1, o), om2 = __shfl_xor(m2, o);
        const int oi1 = __shfl_xor(i1, o);
        const bool other_wins = om1 > m1 || (om1 == m1 && oi1 < i1);
        const float lose = other_wins ? m1 : om1;   // the losing group's largest
        m2 = fmaxf(fmaxf(m2, om2), lose);
        if (other_wins) { m1 = om1; i1 = oi1; }
      }
      float se = 0.f;
      if (row_ok)
        for (int c = sub; c < nc; c += 8) se += __expf(tile[ml][c] - m1);
#pragma unroll
      for (int o = 1; o < 8; o <<= 1) se += __shfl_xor(se, o);
      const int m = m_base + ml;
      if (row_ok && sub == 0 && m < a.M) a.stats[(size_t)m * a.n_groups + cg] = make_float4(m1, __int_as_float(i1), m2, se);
    }
    if (a.logits) {
      for (int idx = threadIdx.x; idx < 16 * MT * TC; idx += 256) {
        const int ml = idx / TC, c = idx % TC;
        const int m = m_base + ml, n = cg * TC + c;
        if (m < a.M && n < a.N) a.logits[(size_t)m * a.ldl + n] = tile[ml][c];
      }
    }
  }
}

template <typename T, int MT, int NT, int D, int EPI>
__global__ __launch_bounds__(256) void gemm_stream(GemmArgs a) {
  constexpr bool BF = sizeof(T) == 2;
  constexpr int KS = BF ? 32 : 16;   // k values per step (one 1 KB weight tile)
  constexpr int TC = 16 * NT;        // packed columns of the workgroup
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, lg = lane >> 4;
  const int cg = blockIdx.x, split = blockIdx.y;
  const int m_base = blockIdx.z * (16 * MT);

  const int ksteps = a.K / KS;
  const int s0 = split * a.steps_per_split;
  const int s1 = min(ksteps, s0 + a.steps_per_split);
  const int nk = max(0, (s1 - s0 - wave + 3) >> 2);  // this wave: steps s0 + wave + 4j
  const int ntiles = (a.N + 15) >> 4;

  const char* wp[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int tile = min(cg * NT + t, ntiles - 1);
    wp[t] = (const char*)a.W + ((size_t)tile * ksteps + s0 + wave) * 1024 + lane * 16;
  }
  // activation k steps are 64 * KS bytes apart in a row tile (tile format); lanes of
  // rows past M read the last row's chunk (same address, no extra traffic)
  const int row_tiles = (a.M + 15) >> 4;
  const char* ap[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int rt = min(blockIdx.z * MT + mt, row_tiles - 1);
    const int rr = min(r, a.M - 1 - rt * 16);
    ap[mt] = (const char*)a.A + ((size_t)rt * ksteps + s0 + wave) * (64 * KS) + (lg * 16 + rr) * 16;
  }

  constexpr int AL = BF ? 2 : 1;
  u32x4 wb[D][NT], ab[D][MT][AL];
  // SwiGLU launches start each workgroup's walk over its k steps at a different step
  // (by its place among the workgroups of its XCD), so that the workgroups resident on
  // an XCD read different activation steps at a time instead of all the same ones
  // (1.7B gate/up 19.5 -> 18.2 us; on the other epilogues it measured no better)
  const int rot = (EPI == EPI_SWIGLU && nk > 0) ? (int)(((blockIdx.x >> 3) + blockIdx.y * 5) % (unsigned)nk) : 0;
  auto issue = [&](int j_, u32x4 (&w)[NT], u32x4 (&av)[MT][AL]) {
    const int j = j_ + rot < nk ? j_ + rot : j_ + rot - nk;
#pragma unroll
    for (int t = 0; t < NT; ++t) w[t] = ld16_stream(wp[t] + (size_t)j * 4096);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int h = 0; h < AL; ++h) av[mt][h] = ld16(ap[mt] + (size_t)j * (4 * 64 * KS) + 1024 * h);
  };
  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const u32x4 (&w)[NT], const u32x4 (&av)[MT][AL]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int h = 0; h < AL; ++h) acc[mt][t] = mma16<T>(av[mt][h], w[t], acc[mt][t]);
  };

  // q/k/v epilogue inputs of this thread's items (rotary pair and K/V destination),
  // loaded before the k loop so their latency hides under the weight stream
  constexpr int QI = EPI == EPI_QKV ? (16 * MT * NT * 8 + 255) / 256 : 1;
  float2 ep_rope[QI];
  int2 ep_dst[QI];
  if constexpr (EPI == EPI_QKV) {
    const int half = a.pair_n;
#pragma unroll
    for (int u = 0; u < QI; ++u) {
      const int idx = threadIdx.x + 256 * u;
      const int ml = idx / (NT * 8), pc = idx % (NT * 8);
      const int m = min(m_base + ml, a.M - 1);
      const int i = ((cg * NT + (pc >> 3)) * 8 + (pc & 7)) % half;
      ep_rope[u] = a.qkv.rope[(size_t)m * half + i];   // chunk row m = b * T + t
      ep_dst[u] = a.qkv.kv_dst[m];
    }
  }

#pragma unroll
  for (int u = 0; u < D - 1; ++u)
    if (u < nk) issue(u, wb[u], ab[u]);
  // steady state: every prefetch of the group is in range (no branches, so the
  // compiler keeps D - 1 steps of loads outstanding)
  int j0 = 0;
  for (; j0 + 2 * D - 2 < nk; j0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      issue(j0 + u + D - 1, wb[(u + D - 1) % D], ab[(u + D - 1) % D]);
      compute(wb[u], ab[u]);
    }
  }
  // tail: at most 2D - 2 steps remain
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int j = j0 + g * D + u;
      if (j < nk) {
        if (j + D - 1 < nk) issue(j + D - 1, wb[(u + D - 1) % D], ab[(u + D - 1) % D]);
        compute(wb[u], ab[u]);
      }
    }

  // ---- sum the four waves in a fixed order, (w0 + w2) + (w1 + w3), into tile[row][col]
  constexpr int NE = MT * NT * 4;
  __shared__ float red[2][NE][64];
  __shared__ float tile[16 * MT][TC + 1];
  if (wave >= 2) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[wave - 2][(mt * NT + t) * 4 + v][lane] = acc[mt][t][v];
  }
  __syncthreads();
  if (wave < 2) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[mt][t][v] += red[wave][(mt * NT + t) * 4 + v][lane];
  }
  __syncthreads();
  if (wave == 1) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[0][(mt * NT + t) * 4 + v][lane] = acc[mt][t][v];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          tile[mt * 16 + 4 * lg + v][t * 16 + r] = acc[mt][t][v] + red[0][(mt * NT + t) * 4 + v][lane];
  }
  __syncthreads();

  gemm_epilogue<T, MT, NT, EPI>(a, tile, cg, split, m_base, [&](int u, int, int) {
    if constexpr (EPI == EPI_QKV) return QkvItem{ep_rope[u], ep_dst[u]};
    else return QkvItem{};
  });
}

// ---------------------------------------------------------------------------
// Tiled GEMM for many rows (M > 80, e.g. a batch of sessions): the weights are no
// longer the only stream, every packed tile is reused by up to 128 rows.  A
// workgroup computes a 128 x (32 * WN) output tile; wave (wm, wn) of its 2 x 2 waves
// owns 64 x (16 * WN) (4 x WN MFMA tiles).  Each k step's operands, 2 * WN weight
// tiles and 8 row tiles of activations (all of them 1 KB blocks in MFMA lane order),
// are copied once per workgroup from global memory into an LDS ring of R steps by
// LDS DMA (global_load_lds, no registers held while in flight), and every wave
// reads the blocks it multiplies from LDS, so each byte crosses the L2 -> CU path
// once per workgroup instead of once per wave that uses it.  Grid: x = row blocks
// (fastest, so the workgroups that share a column group's weights run together and
// the weights come from HBM once), y = splits of K (split-partials epilogue only), z =
// column groups.  The finished tile goes through LDS (the ring's memory) to the shared
// epilogues.

template <typename T, int WN, int R>
constexpr int tiled_lds_bytes() {
  constexpr int AL = sizeof(T) == 2 ? 2 : 1;
  constexpr int ring = R * (2 * WN + 8 * AL) * 1024;
  // with a two-step ring the epilogue runs on 64-row halves of the output block, so
  // that two workgroups fit in a CU's LDS
  constexpr int tile = (R == 2 ? 64 : 128) * (32 * WN + 1) * 4;
  return ring > tile ? ring : tile;
}

// columns per group in the tiled GEMM's workgroup order (measured on the 2624-row
// batched pass: 2, 4, 8, 12, 16, 32 columns gave 142.5, 141.2, 140.6-141.1, 141.4,
// 142.1, 144.1 ms against 143.4-143.8 with row blocks alone first)
constexpr int TILED_GROUP_COLS = 8;

template <typename T, int WN, int R, int EPI>
__global__ __launch_bounds__(256) void gemm_tiled(GemmArgs a) {
  constexpr bool BF = sizeof(T) == 2;
  constexpr int KS = BF ? 32 : 16;
  constexpr int AL = BF ? 2 : 1;
  constexpr int WM = 4;              // MFMA row tiles per wave
  constexpr int MT = 2 * WM, NT = 2 * WN;
  constexpr int TC = 16 * NT;
  constexpr int NL = NT + MT * AL;   // 1 KB blocks per k step: weight tiles, then row tiles
  constexpr int SB = NL * 1024;      // bytes of one ring slot
  static_assert(NL % 4 == 0, "blocks per step split evenly over the 4 waves");
  constexpr int NPW = NL / 4;        // blocks each wave copies per step
  __shared__ __attribute__((aligned(1024))) char smem[tiled_lds_bytes<T, WN, R>()];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 15, lg = lane >> 4;
  // workgroup -> (row block rb, K split sp, column group cg).  Workgroups are dealt to
  // the 8 XCDs round-robin by linear id; when the grid divides by 8, XCD x takes the
  // x-th eighth of the items.  Items run in groups of TILED_GROUP_COLS columns (a
  // column is a (split, column group) pair), row blocks in sequence inside a group, so
  // the workgroups resident on an XCD at a time share both the weight slices of a few
  // columns and the activation slices of a few row blocks in its L2.
  int rb = blockIdx.x, sp = blockIdx.y, cg = blockIdx.z;
  {
    const int RB = gridDim.x, SP = gridDim.y, n = RB * SP * gridDim.z;
    const int L = blockIdx.x + RB * (blockIdx.y + SP * blockIdx.z);
    if ((n & 7) == 0) {
      constexpr int GC = TILED_GROUP_COLS;
      const int I = (L & 7) * (n >> 3) + (L >> 3);
      const int ncol = SP * gridDim.z;
      const int grp = I / (GC * RB), within = I % (GC * RB);
      const int cols = min(GC, ncol - grp * GC);   // the last group may be narrower
      rb = within / cols;
      const int col = grp * GC + within % cols;
      sp = col % SP;
      cg = col / SP;
    }
  }
  const int m_base = rb * (16 * MT);
  const int ksteps = a.K / KS;
  // this workgroup's k steps [s0, s0 + nk): split sp of the K range (fp32 partials
  // summed by the consumer; the other epilogues take the whole range)
  const int s0 = sp * a.steps_per_split;
  const int nk = max(0, min(ksteps, s0 + a.steps_per_split) - s0);
  const int ntiles = (a.N + 15) >> 4;
  const int row_tiles = (a.M + 15) >> 4;

  // this wave's blocks of every step: block c = wave + 4 i; global address of this
  // lane's 16 bytes at step 0 and the step stride
  const char* gp[NPW];
  int gstride[NPW];
#pragma unroll
  for (int i = 0; i < NPW; ++i) {
    const int c = wave + 4 * i;
    if (c < NT) {
      const int tile = min(cg * NT + c, ntiles - 1);
      gp[i] = (const char*)a.W + ((size_t)tile * ksteps + s0) * 1024 + lane * 16;
      gstride[i] = 1024;
    } else {
      const int q = c - NT, mt8 = q / AL, h = q % AL;
      const int rt = min(rb * MT + mt8, row_tiles - 1);
      const int rr = min(r, a.M - 1 - rt * 16);   // rows past M: the last row's chunk
      gp[i] = (const char*)a.A + ((size_t)rt * ksteps + s0) * (64 * KS) + h * 1024 + (lg * 16 + rr) * 16;
      gstride[i] = 64 * KS;
    }
  }
  auto copy_step = [&](int s, int slot) {
    char* dst = smem + slot * SB;
#pragma unroll
    for (int i = 0; i < NPW; ++i) lds_dma16(gp[i] + (size_t)s * gstride[i], dst + (wave + 4 * i) * 1024);
  };

  f32x4 acc[WM][WN];
#pragma unroll
  for (int mt = 0; mt < WM; ++mt)
#pragma unroll
    for (int t = 0; t < WN; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int u = 0; u < R - 1; ++u)
    if (u < nk) copy_step(u, u);
  for (int j = 0; j < nk; ++j) {
    // this wave's copies of step j have landed (later steps may still be in flight);
    // after the barrier every wave's have, and every wave is done with step j - 1
    if (j + R - 2 < nk) vmem_wait<(R - 2) * NPW>();
    else vmem_wait<0>();
    // a bare barrier: __syncthreads() would also wait for the copies still in flight.
    // The compiler fences keep every LDS access on its side of it.
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (j + R - 1 < nk) copy_step(j + R - 1, (j + R - 1) % R);
    const char* slot = smem + (j % R) * SB + lane * 16;
    u32x4 av[WM][AL];
#pragma unroll
    for (int mt = 0; mt < WM; ++mt)
#pragma unroll
      for (int h = 0; h < AL; ++h) av[mt][h] = *(const u32x4*)(slot + (NT + (wm * WM + mt) * AL + h) * 1024);
#pragma unroll
    for (int t = 0; t < WN; ++t) {
      const u32x4 w = *(const u32x4*)(slot + (wn * WN + t) * 1024);
#pragma unroll
      for (int mt = 0; mt < WM; ++mt)
#pragma unroll
        for (int h = 0; h < AL; ++h) acc[mt][t] = mma16<T>(av[mt][h], w, acc[mt][t]);
    }
  }

  __syncthreads();   // the ring's memory becomes the output tile
  float (*tile)[TC + 1] = reinterpret_cast<float (*)[TC + 1]>(smem);
  if constexpr (R == 2) {
    // half h: the two waves of rows 64h .. 64h + 63 store them, then all threads run the
    // epilogue on them
    for (int hf = 0; hf < 2; ++hf) {
      if (wm == hf) {
#pragma unroll
        for (int mt = 0; mt < WM; ++mt)
#pragma unroll
          for (int t = 0; t < WN; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) tile[mt * 16 + 4 * lg + v][wn * 16 * WN + t * 16 + r] = acc[mt][t][v];
      }
      __syncthreads();
      gemm_epilogue<T, MT / 2, NT, EPI>(a, tile, cg, sp, m_base + hf * 16 * WM, [&](int, int m, int i) {
        if constexpr (EPI == EPI_QKV) return QkvItem{a.qkv.rope[(size_t)m * a.pair_n + i], a.qkv.kv_dst[m]};
        else return QkvItem{};
      });
      __syncthreads();
    }
    return;
  }
#pragma unroll
  for (int mt = 0; mt < WM; ++mt)
#pragma unroll
    for (int t = 0; t < WN; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) tile[wm * 16 * WM + mt * 16 + 4 * lg + v][wn * 16 * WN + t * 16 + r] = acc[mt][t][v];
  __syncthreads();
  gemm_epilogue<T, MT, NT, EPI>(a, tile, cg, sp, m_base, [&](int, int m, int i) {
    if constexpr (EPI == EPI_QKV) return QkvItem{a.qkv.rope[(size_t)m * a.pair_n + i], a.qkv.kv_dst[m]};
    else return QkvItem{};
  });
}

// ---------------------------------------------------------------------------
// Column-split weight-streaming GEMM for few rows (M <= 80).  In gemm_stream the four
// waves of a workgroup split the k range of one weight slice, so every workgroup
// fetches the activation operand of its whole k range for only NT weight tiles; with
// bf16 pairs at 65 rows that is 10 KB of activations per 1 KB weight tile step, more
// bytes through each CU than the weights.  Here the waves split the columns: wave w
// owns NT packed tiles of the workgroup's NW NT (NW = 4 waves, or 8 for split
// partials), over the workgroup's k range, so one copy of a k step's activation blocks
// serves every wave.  The threads fetch the step's blocks (16 bytes each, P steps ahead
// into registers) and store them to an LDS double buffer; each wave reads them back in
// operand order and streams its own weight tiles through a register ring D steps deep.
// One LDS barrier per k step.
// Grid: x = column groups of NW NT tiles, y = splits of K.  Epilogues: PARTIAL (the
// split's fp32 partial sums, stored from the accumulators); the others take the whole
// K in one workgroup (one split) and go through an LDS tile to the shared epilogue.
// A q/k/v or SwiGLU launch with K splits writes partials with PARTIAL and gemm_finish
// sums them.  (Handing the partials to the last workgroup of each column group
// instead, through device-coherent stores and an arrival counter, measured slower on
// the 8B gate/up projection: 61 against 51 us with the finish launch.)

template <int... I, typename F>
SDV_DEV void static_for_impl(std::integer_sequence<int, I...>, F&& f) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
SDV_DEV void static_for(F&& f) {
  static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

constexpr int cgcd(int x, int y) { return y == 0 ? x : cgcd(y, x % y); }

#ifndef SDV_WIDE_P
#define SDV_WIDE_P 2
#endif
constexpr int WIDE_P = SDV_WIDE_P;

template <typename T, int MT, int NT, int D, int EPI, int NW = 4>
__global__ __launch_bounds__(64 * NW) void gemm_wide(GemmArgs a) {
  static_assert(NW == 4 || EPI == EPI_PARTIAL, "the shared epilogues take 256 threads");
  constexpr int NTHR = 64 * NW;
  constexpr bool BF = sizeof(T) == 2;
  constexpr int KS = BF ? 32 : 16;
  constexpr int AL = BF ? 2 : 1;
  constexpr int NB = MT * AL;                 // 1 KB activation blocks per k step
  constexpr int NCH = (NB * 64 + NTHR - 1) / NTHR;  // 16-byte chunks of a step per thread
  constexpr int P = WIDE_P;                   // k steps of activation loads ahead
  constexpr int TW = NW * NT;                 // packed tiles of the workgroup
  // register ring slots, staging slots and LDS buffers are indexed by compile-time
  // step residues
  constexpr int U2 = D * 2 / cgcd(D, 2);
  constexpr int U = U2 * P / cgcd(U2, P);
  static_assert(U % P == 0, "unroll covers the staging ring");
  constexpr int E = (D - 1 > P + 1) ? D - 1 : P + 1;   // look-ahead of a step's issues
  // a buffer holds every thread's NCH chunks: chunks past the NB blocks land in a pad
  // that is never read, so no load or store of the staging path takes a branch
  __shared__ __attribute__((aligned(16))) char abuf[2][NCH * NTHR * 16];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, lg = lane >> 4;
  const int cg = blockIdx.x, sp = blockIdx.y;
  const int ksteps = a.K / KS;
  const int s0 = sp * a.steps_per_split;
  const int nk = max(0, min(ksteps, s0 + a.steps_per_split) - s0);
  const int ntiles = (a.N + 15) >> 4;
  const int row_tiles = (a.M + 15) >> 4;

  // this wave's weight tiles (past the last tile: the last one again; its columns are
  // not stored): lane's 16 bytes at step s0, steps 1 KB apart
  const char* wp[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int tile = min(cg * TW + wave * NT + t, ntiles - 1);
    wp[t] = (const char*)a.W + ((size_t)tile * ksteps + s0) * 1024 + lane * 16;
  }
  // this thread's activation chunks c = threadIdx.x + NTHR i of a step's NB blocks
  // (block b = row tile * AL + half; steps 64 * KS bytes apart in a row tile); lanes of
  // rows past M read the last row's chunk, chunks past the blocks the last chunk
  const char* cp[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = threadIdx.x + NTHR * i;
    const int cc = min(c, NB * 64 - 1);
    const int b = cc >> 6, l = cc & 63;
    const int rt = min(b / AL, row_tiles - 1), h = b % AL;
    const int rr = min(l & 15, a.M - 1 - rt * 16);
    cp[i] = (const char*)a.A + ((size_t)rt * ksteps + s0) * (64 * KS) + h * 1024 + ((l >> 4) * 16 + rr) * 16;
  }

  u32x4 wb[D][NT];
  u32x4 st[P][NCH];
  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto load_w = [&](int j, u32x4 (&dst)[NT]) {
#pragma unroll
    for (int t = 0; t < NT; ++t) dst[t] = ld16_stream(wp[t] + (size_t)j * 1024);
  };
  auto load_a = [&](int j, u32x4 (&dst)[NCH]) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) dst[i] = ld16(cp[i] + (size_t)j * (64 * KS));
  };
  auto store_a = [&](const u32x4 (&src)[NCH], int buf) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) *(u32x4*)(&abuf[buf][(threadIdx.x + NTHR * i) * 16]) = src[i];
  };
  // k step j (j % U == u): issue the loads that run ahead, stage step j + 1 into the
  // other LDS buffer, multiply step j, then the barrier that publishes step j + 1 and
  // frees step j's buffer
  auto step = [&](int j, auto uc, bool guard) {
    constexpr int u = decltype(uc)::value;
    if (!guard || j + D - 1 < nk) load_w(j + D - 1, wb[(u + D - 1) % D]);
    if (!guard || j + 1 < nk) {
      store_a(st[(u + 1) % P], (u + 1) & 1);
      if (!guard || j + 1 + P < nk) load_a(j + 1 + P, st[(u + 1) % P]);
    }
    // keep the loads ahead of the step's multiplies (the scheduler would sink them
    // towards their uses, a step later, and shorten the look-ahead)
    __builtin_amdgcn_sched_barrier(0);
    // every block of the step read from LDS first, so their latencies overlap
    const char* blk = &abuf[u & 1][lane * 16];
    u32x4 av[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) av[b] = *(const u32x4*)(blk + b * 1024);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[b / AL][t] = mma16<T>(av[b], wb[u % D][t], acc[b / AL][t]);
    lds_barrier();
  };

#pragma unroll
  for (int u = 0; u < P; ++u)
    if (u < nk) load_a(u, st[u]);
#pragma unroll
  for (int u = 0; u < D - 1; ++u)
    if (u < nk) load_w(u, wb[u]);
  if (nk > 0) {
    store_a(st[0], 0);
    if (P < nk) load_a(P, st[0]);
  }
  lds_barrier();
  int j0 = 0;
  // steady state: every look-ahead of the group is in range, no branches
  for (; j0 + U - 1 + E < nk; j0 += U) static_for<U>([&](auto uc) { step(j0 + decltype(uc)::value, uc, false); });
  for (; j0 < nk; j0 += U)
    static_for<U>([&](auto uc) {
      if (j0 + decltype(uc)::value < nk) step(j0 + decltype(uc)::value, uc, true);
    });

  if constexpr (EPI == EPI_PARTIAL) {
    float* out = a.out + (size_t)sp * a.out_split_stride;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int n = (cg * TW + wave * NT + t) * 16 + r;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = mt * 16 + 4 * lg + v;
          if (m < a.M && n < a.N) out[(size_t)m * a.ldo + n] = acc[mt][t][v];
        }
      }
  } else {
    __shared__ float tile[16 * MT][16 * TW + 1];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) tile[mt * 16 + 4 * lg + v][(wave * NT + t) * 16 + r] = acc[mt][t][v];
    __syncthreads();
    gemm_epilogue<T, MT, TW, EPI>(a, tile, cg, sp, 0, [&](int, int m, int i) {
      if constexpr (EPI == EPI_QKV) return QkvItem{a.qkv.rope[(size_t)m * a.pair_n + i], a.qkv.kv_dst[m]};
      else return QkvItem{};
    });
  }
}

// Split-K finish of a wide q/k/v or SwiGLU launch: rows [0, M) of column group cg (16 NT
// columns) summed over the a.n_split partials in split order (at most MAXS), then the
// shared epilogue on the finished tile.  Each thread loads all of its partials before
// it adds any.  Grid: x = column groups of NT tiles.
template <typename T, int MT, int NT, int EPI, int MAXS>
__global__ __launch_bounds__(256) void gemm_finish(GemmArgs a) {
  constexpr int TC = 16 * NT;
  constexpr int RC = TC / 4;                  // 16-byte chunks per tile row
  constexpr int CPT = (16 * MT * RC + 255) / 256;   // chunks per thread
  __shared__ float tile[16 * MT][TC + 1];
  const int cg = blockIdx.x;
  const int S = a.n_split;
  // q/k/v epilogue inputs of this thread's items (the epilogue's item order), loaded
  // first so that their latency overlaps the partials'
  constexpr int QI = EPI == EPI_QKV ? (16 * MT * NT * 8 + 255) / 256 : 1;
  QkvItem items[QI];
  if constexpr (EPI == EPI_QKV) {
    const int half = a.pair_n;
#pragma unroll
    for (int u = 0; u < QI; ++u) {
      const int idx = threadIdx.x + 256 * u;
      const int m = min(idx / (NT * 8), a.M - 1), pc = idx % (NT * 8);
      const int i = ((cg * NT + (pc >> 3)) * 8 + (pc & 7)) % half;
      items[u] = QkvItem{a.qkv.rope[(size_t)m * half + i], a.qkv.kv_dst[m]};
    }
  }
  // 16-byte chunks (row ml, columns n .. n + 3; N and the row pitch are multiples of
  // 16): every partial of every chunk of the thread is loaded before any is added
  f32x4 v[CPT][MAXS];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int idx = threadIdx.x + 256 * c;
    const int ml = idx / RC, n = cg * TC + (idx % RC) * 4;
    const bool ok = idx < 16 * MT * RC && ml < a.M && n < a.N;
    const float* p = a.out + (size_t)min(ml, a.M - 1) * a.ldo + min(n, a.N - 4);
#pragma unroll
    for (int s = 0; s < MAXS; ++s)
      v[c][s] = (ok && s < S) ? *(const f32x4*)(p + (size_t)s * a.out_split_stride) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int idx = threadIdx.x + 256 * c;
    if (idx < 16 * MT * RC) {
      f32x4 x = v[c][0];
#pragma unroll
      for (int s = 1; s < MAXS; ++s) x += v[c][s];
#pragma unroll
      for (int e = 0; e < 4; ++e) tile[idx / RC][(idx % RC) * 4 + e] = x[e];
    }
  }
  __syncthreads();
  gemm_epilogue<T, MT, NT, EPI>(a, tile, cg, 0, 0, [&](int u, int, int) { return items[u]; });
}

// ---------------------------------------------------------------------------
// Weight packing: packed row n (of n_packed, a multiple of 16) takes source row
// src_row(n); rows past the sources are zero.  One thread per 16-byte chunk.
template <typename T>
__global__ __launch_bounds__(256) void pack_kernel(PackArgs a) {
  constexpr int VE = 16 / sizeof(T);   // values per 16-byte chunk
  constexpr int KS = 4 * VE;           // k values per tile
  const int ksteps = a.K / KS;
  const size_t nchunks = (size_t)a.n_packed * ksteps * 4;
  for (size_t c = (size_t)blockIdx.x * 256 + threadIdx.x; c < nchunks; c += (size_t)gridDim.x * 256) {
    // chunk c: tile c / 64, lane c % 64 = (k group, row) inside the tile
    const size_t tidx = c >> 6;
    const int ln = (int)(c & 63);
    const int kg = ln >> 4, rr = ln & 15;
    const int n = (int)(tidx / ksteps) * 16 + rr;
    const int ks = (int)(tidx % ksteps);
    int which = -1, row = 0;
    if (a.kind == 0) {
      if (n < a.rows[0]) { which = 0; row = n; }
    } else {
      const int t = n >> 4, i = n & 15;
      const int p = t * 8 + (i & 7);  // pair index
      const bool second = i >= 8;
      int vrow;                        // row of the sources viewed as one matrix
      if (a.kind == 1) {
        const int half = a.head_dim / 2;
        vrow = (p / half) * a.head_dim + p % half + (second ? half : 0);
      } else {
        vrow = p + (second ? a.rows[0] : 0);
      }
      int base = 0;
      for (int s = 0; s < 3; ++s) {
        if (vrow >= base && vrow < base + a.rows[s]) { which = s; row = vrow - base; break; }
        base += a.rows[s];
      }
    }
    u32x4 v = {0u, 0u, 0u, 0u};
    if (which >= 0) v = ld16((const T*)a.src[which] + (size_t)row * a.K + ks * KS + kg * VE);
    st16((char*)a.dst + c * 16, v);
  }
}

hipError_t launch_pack(bool is_bf16, const PackArgs& a, hipStream_t s) {
  const int eb = is_bf16 ? 2 : 4;
  const size_t nchunks = (size_t)a.n_packed * a.K * eb / 16;
  const int blocks = (int)std::min<size_t>(8192, (nchunks + 255) / 256);
  if (blocks < 1) return hipSuccess;
  if (is_bf16) pack_kernel<bf16><<<blocks, 256, 0, s>>>(a);
  else pack_kernel<float><<<blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// host-side dispatch over the instantiated (MT, NT, D) configurations

// LDS bytes of a configuration: two wave-partial buffers + the output tile
constexpr int gemm_lds_bytes(int MT, int NT) { return 2 * MT * NT * 4 * 64 * 4 + 16 * MT * (16 * NT + 1) * 4; }
constexpr int LDS_LIMIT = 160 * 1024;
int gemm_lds_ok(int MT, int NT) { return gemm_lds_bytes(MT, NT) <= LDS_LIMIT; }

struct Launch {
  dim3 grid;
  hipStream_t s;
  hipEvent_t ev0, ev1;
};

template <typename T, int MT, int NT, int D, int EPI>
static hipError_t launch_one(const Launch& L, const GemmArgs& a) {
  // the q/k/v epilogue is planned with two tiles per workgroup only
  if constexpr (gemm_lds_bytes(MT, NT) <= LDS_LIMIT && (EPI != EPI_QKV || NT == 2)) {
    if (L.ev0) hipExtLaunchKernelGGL(gemm_stream<T, MT, NT, D, EPI>, L.grid, dim3(256), 0, L.s, L.ev0, L.ev1, 0, a);
    else gemm_stream<T, MT, NT, D, EPI><<<L.grid, 256, 0, L.s>>>(a);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

template <typename T, int NT, int D, int EPI>
static hipError_t launch_mt(int MT, const Launch& L, const GemmArgs& a) {
  switch (MT) {
    case 1: return launch_one<T, 1, NT, D, EPI>(L, a);
    case 2: return launch_one<T, 2, NT, D, EPI>(L, a);
    case 3: return launch_one<T, 3, NT, D, EPI>(L, a);
    case 4: return launch_one<T, 4, NT, D, EPI>(L, a);
    case 5: return launch_one<T, 5, NT, D, EPI>(L, a);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int WN, int R, int EPI>
static hipError_t launch_tiled(const Launch& L, const GemmArgs& a) {
  static_assert(tiled_lds_bytes<T, WN, R>() <= LDS_LIMIT, "tiled GEMM LDS");
  if (L.ev0) hipExtLaunchKernelGGL(gemm_tiled<T, WN, R, EPI>, L.grid, dim3(256), 0, L.s, L.ev0, L.ev1, 0, a);
  else gemm_tiled<T, WN, R, EPI><<<L.grid, 256, 0, L.s>>>(a);
  return hipGetLastError();
}

// the column-split kernel: 3 weight steps in flight per wave; NT 1-4 tiles per wave for
// split partials, 3-4 for the head
#ifndef SDV_WIDE_D
#define SDV_WIDE_D 3
#endif
constexpr int WIDE_D = SDV_WIDE_D;

template <typename T, int MT, int NT, int EPI, int NW = 4>
static hipError_t launch_wide_one(const Launch& L, const GemmArgs& a) {
  if (L.ev0 || L.ev1)
    hipExtLaunchKernelGGL(gemm_wide<T, MT, NT, WIDE_D, EPI, NW>, L.grid, dim3(64 * NW), 0, L.s, L.ev0, L.ev1, 0, a);
  else gemm_wide<T, MT, NT, WIDE_D, EPI, NW><<<L.grid, 64 * NW, 0, L.s>>>(a);
  return hipGetLastError();
}

template <typename T, int MT, int EPI>
static hipError_t launch_wide_nt(int NT, int NW, const Launch& L, const GemmArgs& a) {
  if constexpr (EPI == EPI_PARTIAL && MT >= 3) {   // eight waves: split partials from 33 rows
    if (NW == 8) {
      if (NT == 1) return launch_wide_one<T, MT, 1, EPI, 8>(L, a);
      if (NT == 2) return launch_wide_one<T, MT, 2, EPI, 8>(L, a);
      if (NT == 3) return launch_wide_one<T, MT, 3, EPI, 8>(L, a);
      return hipErrorInvalidValue;
    }
  }
  if (NW != 4) return hipErrorInvalidValue;
  if constexpr (EPI == EPI_PARTIAL)
    if (NT == 1) return launch_wide_one<T, MT, 1, EPI>(L, a);
  if constexpr (EPI != EPI_LOGITS)
    if (NT == 2) return launch_wide_one<T, MT, 2, EPI>(L, a);
  if (NT == 3) return launch_wide_one<T, MT, 3, EPI>(L, a);
  if (NT == 4) return launch_wide_one<T, MT, 4, EPI>(L, a);
  return hipErrorInvalidValue;
}

template <typename T, int EPI>
static hipError_t launch_wide(int NT, int NW, int MT, const Launch& L, const GemmArgs& a) {
  switch (MT) {
    case 1: return launch_wide_nt<T, 1, EPI>(NT, NW, L, a);
    case 2: return launch_wide_nt<T, 2, EPI>(NT, NW, L, a);
    case 3: return launch_wide_nt<T, 3, EPI>(NT, NW, L, a);
    case 4: return launch_wide_nt<T, 4, EPI>(NT, NW, L, a);
    case 5: return launch_wide_nt<T, 5, EPI>(NT, NW, L, a);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int EPI>
static hipError_t launch_cfg(const GemmCfg& c, int MT, const Launch& L, const GemmArgs& a) {
  if (c.wide) return launch_wide<T, EPI>(c.NT, c.NW, MT, L, a);
  if (c.tiled) {
    if (c.NT == 4 && c.D == 3) return launch_tiled<T, 4, 3, EPI>(L, a);
    if (c.NT == 8 && c.D == 2) return launch_tiled<T, 8, 2, EPI>(L, a);
    return hipErrorInvalidValue;
  }
  if (c.NT == 2 && c.D == 4) return launch_mt<T, 2, 4, EPI>(MT, L, a);
  if (c.NT == 4 && c.D == 2) return launch_mt<T, 4, 2, EPI>(MT, L, a);
  if constexpr (EPI == EPI_LOGITS) {   // LM head on one or two row tiles: deeper ring
    if (c.NT == 4 && c.D == 4 && MT == 1) return launch_one<T, 1, 4, 4, EPI>(L, a);
    if (c.NT == 4 && c.D == 4 && MT == 2) return launch_one<T, 2, 4, 4, EPI>(L, a);
  }
  if (c.NT == 8 && c.D == 2) return launch_mt<T, 8, 2, EPI>(MT, L, a);
  if constexpr (EPI == EPI_SWIGLU || EPI == EPI_LOGITS)   // six tiles: gate/up and LM head only
    if (c.NT == 6 && c.D == 2) return launch_mt<T, 6, 2, EPI>(MT, L, a);
  return hipErrorInvalidValue;
}

template <typename T, int MT, int NT, int EPI, int MAXS>
static hipError_t launch_finish_one(const Launch& L, const GemmArgs& a) {
  if (L.ev1) hipExtLaunchKernelGGL(gemm_finish<T, MT, NT, EPI, MAXS>, L.grid, dim3(256), 0, L.s, nullptr, L.ev1, 0, a);
  else gemm_finish<T, MT, NT, EPI, MAXS><<<L.grid, 256, 0, L.s>>>(a);
  return hipGetLastError();
}

// two tiles per workgroup up to 8 splits, one beyond (the partials of a thread's
// chunks are all in registers at once)
template <typename T, int MT, int EPI>
static hipError_t launch_finish_s(int NTF, const Launch& L, const GemmArgs& a) {
  if (NTF == 2 && a.n_split <= 4) return launch_finish_one<T, MT, 2, EPI, 4>(L, a);
  if (NTF == 2 && a.n_split <= 8) return launch_finish_one<T, MT, 2, EPI, 8>(L, a);
  if (NTF == 1 && a.n_split <= 16) return launch_finish_one<T, MT, 1, EPI, 16>(L, a);
  return hipErrorInvalidValue;
}

template <typename T, int EPI>
static hipError_t launch_finish_t(int NTF, int MT, const Launch& L, const GemmArgs& a) {
  switch (MT) {
    case 1: return launch_finish_s<T, 1, EPI>(NTF, L, a);
    case 2: return launch_finish_s<T, 2, EPI>(NTF, L, a);
    case 3: return launch_finish_s<T, 3, EPI>(NTF, L, a);
    case 4: return launch_finish_s<T, 4, EPI>(NTF, L, a);
    case 5: return launch_finish_s<T, 5, EPI>(NTF, L, a);
    default: return hipErrorInvalidValue;
  }
}

int gemm_finish_tiles(int n_split) { return n_split <= 8 ? 2 : 1; }

hipError_t launch_gemm_finish(bool is_bf16, const GemmCfg& c, int MT, int epi, dim3 grid, const GemmArgs& a,
                              hipStream_t s, hipEvent_t ev_stop) {
  if (c.NTF != gemm_finish_tiles(a.n_split) || a.n_split < 1) return hipErrorInvalidValue;
  const Launch L{grid, s, nullptr, ev_stop};
  if (epi == EPI_QKV)
    return is_bf16 ? launch_finish_t<bf16, EPI_QKV>(c.NTF, MT, L, a) : launch_finish_t<float, EPI_QKV>(c.NTF, MT, L, a);
  if (epi == EPI_SWIGLU)
    return is_bf16 ? launch_finish_t<bf16, EPI_SWIGLU>(c.NTF, MT, L, a) : launch_finish_t<float, EPI_SWIGLU>(c.NTF, MT, L, a);
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(bool is_bf16, const GemmCfg& c, int MT, int epi, dim3 grid, const GemmArgs& a,
                       hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  const Launch L{grid, s, ev_start, (ev_start || c.wide) ? ev_stop : nullptr};
#define SDV_EPI(E)                                                                          \
  if (epi == E) return is_bf16 ? launch_cfg<bf16, E>(c, MT, L, a) : launch_cfg<float, E>(c, MT, L, a);
  SDV_EPI(EPI_PARTIAL)
  SDV_EPI(EPI_QKV)
  SDV_EPI(EPI_SWIGLU)
  SDV_EPI(EPI_LOGITS)
#undef SDV_EPI
  return hipErrorInvalidValue;
}

}  // namespace sdv
