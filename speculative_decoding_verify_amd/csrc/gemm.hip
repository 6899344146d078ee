// Weight-streaming GEMM for few rows: out[m, n] = sum_k A[m, k] * W[n, k].
//
// A (activations) is fp32.  With bf16 weights each group of 8 activations enters
// the bf16 MFMA as a hi + lo pair (two MFMAs), so products carry ~16 significant
// bits of the activation; only the weights are bf16.  With fp32 weights the fp32
// MFMA is used directly.
//
// The decoder projections of a verify pass multiply M = B*T (tens of) activation
// rows by weight matrices of tens to hundreds of MB, so the kernel is bound by
// streaming W from HBM once.  Work layout:
//   * a workgroup has WN x WK waves: the WN waves take different column tiles, the
//     WK waves split the workgroup's K range (reduced through LDS in a fixed order);
//   * blockIdx.x: a column group of WN * NT * 16 weight rows; blockIdx.y: a split of
//     K across workgroups (fp32 partials, summed in split order by the consumer);
//     blockIdx.z: a block of 16 * MT activation rows;
//   * each lane streams 16 contiguous bytes of a weight row per k step (four lanes
//     cover 64 B of one row); the next U steps are in flight while the current U are
//     multiplied (software pipeline); the activation tile is read through the caches.
//
// Epilogues (all but PARTIAL need the whole K range in one workgroup, S = 1):
//   PARTIAL  fp32 partial sums of each split;
//   QKV      rotary embedding on q and k (both halves of every rotation pair sit in
//            the same workgroup); q written row-major in fp32, k and v rounded to the
//            cache type and appended to the paged cache (k token-major, v transposed
//            inside the page);
//   SWIGLU   h = silu(gate) * up in fp32 (gate and up rows of the same index in one workgroup);
//   LOGITS   fp32 logits plus per-(row, column group) statistics: largest value, its
//            index (lowest on ties), second-largest value and sum of exp(v - largest).
#include "common.h"
#include "kernels.h"

namespace sdv {

// weight row of local pair/plain column (wave-group q, tile ct, lane row r)
template <int NT>
SDV_DEV int map_col(const GemmArgs& a, int q, int ct, int r) {
  if (a.pair_mode == PAIR_NONE) return (q * NT + ct) * 16 + r;
  constexpr int H = NT / 2;
  const int j = ct % H, second = ct >= H;
  const int p = (q * H + j) * 16 + r;  // pair index
  if (a.pair_mode == PAIR_SWIGLU) return p + (second ? a.pair_off : 0);
  // rotation pairs of a head: element i with i + dh/2
  const int half = a.pair_off;
  return (p / half) * 2 * half + p % half + (second ? half : 0);
}

template <typename T, int MT, int NT, int WN, int WK, int U, int EPI>
__global__ __launch_bounds__(64 * WN * WK) void gemm_rows(GemmArgs a) {
  constexpr int VE = Vec16<T>::N;   // elements per lane per step (8 bf16 / 4 fp32)
  constexpr int KS = VE * 4;        // k per step across the 4 lane groups
  constexpr int NTH = 64 * WN * WK;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wn = wave % WN, wk = wave / WN;
  const int r = lane & 15, lg = lane >> 4;
  const int cg = blockIdx.x, split = blockIdx.y;
  const int m_base = blockIdx.z * (16 * MT);

  const int total_steps = a.K / KS;
  const int s0 = split * a.steps_per_split;
  const int s1 = min(total_steps, s0 + a.steps_per_split);
  const int nst = max(0, s1 - s0);
  const int ws0 = s0 + (nst * wk) / WK, ws1 = s0 + (nst * (wk + 1)) / WK;

  const T* wrow[NT];
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    const int n = min(map_col<NT>(a, cg * WN + wn, ct, r), a.N - 1);
    const T* base = n < a.N0   ? (const T*)a.W0 + (size_t)n * a.K
                    : n < a.N1 ? (const T*)a.W1 + (size_t)(n - a.N0) * a.K
                               : (const T*)a.W2 + (size_t)(n - a.N1) * a.K;
    wrow[ct] = base + lg * VE;
  }
  const float* arow[MT];
  bool avalid[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = m_base + mt * 16 + r;
    avalid[mt] = m < a.M;
    const int row = avalid[mt] ? (a.a_rows ? a.a_rows[m] : m) : 0;
    arow[mt] = (const float*)a.A + (size_t)row * a.lda + lg * VE;
  }
  constexpr bool BF = sizeof(T) == 2;
  constexpr int AL = BF ? 2 : 1;   // 16-byte activation loads per k step (8 or 4 fp32)

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) acc[mt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 wb[U][NT];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int ct = 0; ct < NT; ++ct)
      wb[u][ct] = (ws0 + u < ws1) ? ld16_stream(wrow[ct] + (size_t)(ws0 + u) * KS) : zero;
  for (int st = ws0; st < ws1; st += U) {
    u32x4 ab[U][MT][AL];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int h = 0; h < AL; ++h)
          ab[u][mt][h] = (avalid[mt] && st + u < ws1) ? ld16(arow[mt] + (size_t)(st + u) * KS + 4 * h) : zero;
    u32x4 wn_[U][NT];
    const int nx = st + U;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int ct = 0; ct < NT; ++ct)
        wn_[u][ct] = (nx + u < ws1) ? ld16_stream(wrow[ct] + (size_t)(nx + u) * KS) : zero;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if constexpr (BF) {
          u32x4 hi, lo;
          split_hi_lo(ab[u][mt][0], ab[u][mt][AL - 1], hi, lo);
#pragma unroll
          for (int ct = 0; ct < NT; ++ct) {
            acc[mt][ct] = mma16<T>(hi, wb[u][ct], acc[mt][ct]);
            acc[mt][ct] = mma16<T>(lo, wb[u][ct], acc[mt][ct]);
          }
        } else {
#pragma unroll
          for (int ct = 0; ct < NT; ++ct) acc[mt][ct] = mma16<T>(ab[u][mt][0], wb[u][ct], acc[mt][ct]);
        }
      }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) wb[u][ct] = wn_[u][ct];
  }

  // ---- reduce the WK waves of each column tile through LDS (fixed order) into
  //      tile[row][local column], local column = (wn * NT + ct) * 16 + r
  constexpr int NE = MT * NT * 4;
  constexpr int TC = WN * NT * 16;          // columns of the workgroup
  __shared__ float tile[16 * MT][TC + 1];
  if constexpr (WK > 1) {
    __shared__ float red[WK][WN][NE][64];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int ct = 0; ct < NT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wk][wn][(mt * NT + ct) * 4 + i][lane] = acc[mt][ct][i];
    __syncthreads();
    for (int idx = threadIdx.x; idx < WN * NE * 64; idx += NTH) {
      const int ln = idx & 63, e = (idx >> 6) % NE, q = (idx >> 6) / NE;
      float v = 0.f;
#pragma unroll
      for (int k = 0; k < WK; ++k) v += red[k][q][e][ln];
      const int i = e & 3, t = e >> 2, ct = t % NT, mt = t / NT;
      tile[mt * 16 + 4 * (ln >> 4) + i][(q * NT + ct) * 16 + (ln & 15)] = v;
    }
  } else {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int ct = 0; ct < NT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) tile[mt * 16 + 4 * lg + i][(wn * NT + ct) * 16 + r] = acc[mt][ct][i];
  }
  __syncthreads();

  if constexpr (EPI == EPI_PARTIAL) {
    float* out = a.out + (size_t)split * a.out_split_stride;
    for (int idx = threadIdx.x; idx < 16 * MT * TC; idx += NTH) {
      const int ml = idx / TC, c = idx % TC;
      const int m = m_base + ml, n = cg * TC + c;
      if (m < a.M && n < a.N) out[(size_t)m * a.ldo + n] = tile[ml][c];
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    // local column (q*NT + ct)*16 + r: ct < NT/2 gate, ct >= NT/2 up of the same row
    constexpr int H = NT / 2;
    for (int idx = threadIdx.x; idx < 16 * MT * WN * H * 16; idx += NTH) {
      const int ml = idx / (WN * H * 16), pc = idx % (WN * H * 16);
      const int q = pc / (H * 16), j = (pc / 16) % H, rr = pc % 16;
      const int m = m_base + ml;
      const int f = ((cg * WN + q) * H + j) * 16 + rr;
      if (m >= a.M || f >= a.pair_off) continue;
      const float gt = tile[ml][(q * NT + j) * 16 + rr];
      const float up = tile[ml][(q * NT + H + j) * 16 + rr];
      const float sl = gt / (1.f + expf(-gt));
      ((float*)a.out_act)[(size_t)m * a.pair_off + f] = sl * up;
    }
  } else if constexpr (EPI == EPI_QKV) {
    constexpr int H = NT / 2;
    const QkvEpi& e = a.qkv;
    const int half = a.pair_off;          // dh / 2
    const int dh = 2 * half;
    for (int idx = threadIdx.x; idx < 16 * MT * WN * H * 16; idx += NTH) {
      const int ml = idx / (WN * H * 16), pc = idx % (WN * H * 16);
      const int q = pc / (H * 16), j = (pc / 16) % H, rr = pc % 16;
      const int m = m_base + ml;
      const int p = ((cg * WN + q) * H + j) * 16 + rr;   // pair index
      const int hh = p / half, i = p % half;              // head (q, k, then v heads) and pair
      if (m >= a.M || hh >= e.H + 2 * e.Hkv) continue;
      const float x1 = tile[ml][(q * NT + j) * 16 + rr];
      const float x2 = tile[ml][(q * NT + H + j) * 16 + rr];
      const int b = m / e.T, t = m % e.T;
      float y1 = x1, y2 = x2;
      if (hh < e.H + e.Hkv) {
        const float2 cs = e.rope[(size_t)(b * e.T + t) * half + i];  // (cos, sin)
        y1 = x1 * cs.x - x2 * cs.y;
        y2 = x2 * cs.x + x1 * cs.y;
      }
      if (hh < e.H) {
        float* qo = (float*)e.q + (size_t)m * e.H * dh + hh * dh;
        qo[i] = y1;
        qo[i + half] = y2;
      } else {
        const int C = e.seq_len[b];
        const int slot = C + t;
        if (C < 0 || C > e.max_ctx || slot >= e.max_blocks * 16) {
          if (i == 0) set_err(e.err, b, 0x4);
          continue;
        }
        const int phys = e.block_table[(size_t)b * e.max_blocks + (slot >> 4)];
        if (phys < 0 || phys >= e.n_blocks) {
          if (i == 0) set_err(e.err, b, 0x4);
          continue;
        }
        const bool is_k = hh < e.H + e.Hkv;
        const int g = is_k ? hh - e.H : hh - e.H - e.Hkv;
        const size_t page = (size_t)phys * e.Hkv + g;
        const int off = slot & 15;
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
    for (int ml = threadIdx.x; ml < 16 * MT; ml += NTH) {
      const int m = m_base + ml;
      if (m >= a.M) continue;
      float m1 = -INFINITY, m2 = -INFINITY;
      int i1 = 0x7fffffff;
      const int nc = min(TC, a.N - cg * TC);
      for (int c = 0; c < nc; ++c) {
        const float v = tile[ml][c];
        if (v > m1) { m2 = m1; m1 = v; i1 = cg * TC + c; }
        else if (v > m2) m2 = v;
      }
      float se = 0.f;
      for (int c = 0; c < nc; ++c) se += __expf(tile[ml][c] - m1);
      a.stats[(size_t)m * a.n_groups + cg] = make_float4(m1, __int_as_float(i1), m2, se);
    }
    if (a.logits) {
      for (int idx = threadIdx.x; idx < 16 * MT * TC; idx += NTH) {
        const int ml = idx / TC, c = idx % TC;
        const int m = m_base + ml, n = cg * TC + c;
        if (m < a.M && n < a.N) a.logits[(size_t)m * a.ldl + n] = tile[ml][c];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host-side dispatch: the instantiated (WN, WK, NT, U) configurations

// LDS bytes of a configuration (wave-reduction buffer + output tile)
constexpr int gemm_lds_bytes(int MT, int NT, int WN, int WK) {
  return (WK > 1 ? WK * WN * MT * NT * 4 * 64 * 4 : 0) + 16 * MT * (WN * NT * 16 + 1) * 4;
}
constexpr int LDS_LIMIT = 160 * 1024;

template <typename T, int MT, int NT, int WN, int WK, int EPI>
static hipError_t launch_one(dim3 grid, const GemmArgs& a, hipStream_t s) {
  if constexpr (gemm_lds_bytes(MT, NT, WN, WK) <= LDS_LIMIT) {
    gemm_rows<T, MT, NT, WN, WK, 4, EPI><<<grid, 64 * WN * WK, 0, s>>>(a);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

template <typename T, int NT, int WN, int WK, int EPI>
static hipError_t launch_mt(int MT, dim3 grid, const GemmArgs& a, hipStream_t s) {
  switch (MT) {
    case 1: return launch_one<T, 1, NT, WN, WK, EPI>(grid, a, s);
    case 2: return launch_one<T, 2, NT, WN, WK, EPI>(grid, a, s);
    case 3: return launch_one<T, 3, NT, WN, WK, EPI>(grid, a, s);
    case 4: return launch_one<T, 4, NT, WN, WK, EPI>(grid, a, s);
    case 5: return launch_one<T, 5, NT, WN, WK, EPI>(grid, a, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int EPI>
static hipError_t launch_cfg(const GemmCfg& c, int MT, dim3 grid, const GemmArgs& a, hipStream_t s) {
  // (NT, WN, WK) combinations; pair epilogues need an even NT
  if (c.NT == 2 && c.WN == 1 && c.WK == 4) return launch_mt<T, 2, 1, 4, EPI>(MT, grid, a, s);
  if (c.NT == 4 && c.WN == 1 && c.WK == 4) return launch_mt<T, 4, 1, 4, EPI>(MT, grid, a, s);
  if (c.NT == 2 && c.WN == 2 && c.WK == 2) return launch_mt<T, 2, 2, 2, EPI>(MT, grid, a, s);
  if (c.NT == 4 && c.WN == 2 && c.WK == 2) return launch_mt<T, 4, 2, 2, EPI>(MT, grid, a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(bool is_bf16, const GemmCfg& c, int MT, int epi, dim3 grid, const GemmArgs& a,
                       hipStream_t s) {
#define SDV_EPI(E)                                                                          \
  if (epi == E) return is_bf16 ? launch_cfg<bf16, E>(c, MT, grid, a, s) : launch_cfg<float, E>(c, MT, grid, a, s);
  SDV_EPI(EPI_PARTIAL)
  SDV_EPI(EPI_QKV)
  SDV_EPI(EPI_SWIGLU)
  SDV_EPI(EPI_LOGITS)
#undef SDV_EPI
  return hipErrorInvalidValue;
}

}  // namespace sdv
