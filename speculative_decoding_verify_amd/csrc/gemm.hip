// Weight-streaming GEMM for few rows: out[m, n] = sum_k A[m, k] * W[n, k].
//
// The decoder projections of a verify pass multiply M = B*T (tens of) activation
// rows by weight matrices of tens to hundreds of MB, so the kernel is bound by
// streaming W from HBM once.  Layout of the work:
//   * blockIdx.x: a group of 16*NT output columns (NT MFMA column tiles);
//   * blockIdx.y: a split of K across workgroups (fp32 partial sums per split);
//   * blockIdx.z: a block of 16*MT rows (MT MFMA row tiles, all held by each wave);
//   * the 4 waves of a workgroup take consecutive quarters of its K range and are
//     reduced through LDS in a fixed order, so results are deterministic.
// Each lane streams 16 contiguous bytes of a weight row per k step (4 lanes cover
// 64 B of one row), U steps are issued back to back to keep bytes in flight, and
// the activation tile is read through the caches (it is small and L2-resident).
//
// Epilogues: EPI_PARTIAL writes the fp32 partial of each split; EPI_LOGITS (one
// split) writes logits and per-(row, column group) statistics: largest value, its
// index (lowest on ties), second-largest value and sum of exp(v - largest).
#include "common.h"
#include "kernels.h"

namespace sdv {

template <typename T, int MT, int NT, int EPI, int U>
__global__ __launch_bounds__(256) void gemm_small_m(GemmArgs a) {
  constexpr int VE = Vec16<T>::N;   // elements per lane per step (8 bf16 / 4 fp32)
  constexpr int KS = VE * 4;        // k per step across the 4 lane groups
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane & 15, lg = lane >> 4;
  const int cg = blockIdx.x, split = blockIdx.y;
  const int m_base = blockIdx.z * (16 * MT);
  const int n_base = cg * (16 * NT);

  const int total_steps = a.K / KS;
  const int s0 = split * a.steps_per_split;
  const int s1 = min(total_steps, s0 + a.steps_per_split);
  const int nst = max(0, s1 - s0);
  const int ws0 = s0 + (nst * w) / 4, ws1 = s0 + (nst * (w + 1)) / 4;

  const T* wrow[NT];
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    int n = min(n_base + ct * 16 + r, a.N - 1);
    const T* base = n < a.N0   ? (const T*)a.W0 + (size_t)n * a.K
                    : n < a.N1 ? (const T*)a.W1 + (size_t)(n - a.N0) * a.K
                               : (const T*)a.W2 + (size_t)(n - a.N1) * a.K;
    wrow[ct] = base + lg * VE;
  }
  const T* arow[MT];
  bool avalid[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int m = m_base + mt * 16 + r;
    avalid[mt] = m < a.M;
    int row = avalid[mt] ? (a.a_rows ? a.a_rows[m] : m) : 0;
    arow[mt] = (const T*)a.A + (size_t)row * a.lda + lg * VE;
  }

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) acc[mt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int st = ws0; st < ws1; st += U) {
    u32x4 wv[U][NT], av[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (st + u < ws1) {
        const size_t k = (size_t)(st + u) * KS;
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) wv[u][ct] = ld16_stream(wrow[ct] + k);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (st + u < ws1) {
        const size_t k = (size_t)(st + u) * KS;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) av[u][mt] = avalid[mt] ? ld16(arow[mt] + k) : zero;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (st + u < ws1) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int ct = 0; ct < NT; ++ct) acc[mt][ct] = mma16<T>(av[u][mt], wv[u][ct], acc[mt][ct]);
      }
    }
  }

  // reduce the 4 waves through LDS: red[w][e][lane], e = (mt*NT + ct)*4 + i
  constexpr int NE = MT * NT * 4;
  __shared__ float red[4][NE][64];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ct = 0; ct < NT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[w][(mt * NT + ct) * 4 + i][lane] = acc[mt][ct][i];
  __syncthreads();

  if constexpr (EPI == EPI_PARTIAL) {
    float* out = a.out + (size_t)split * a.out_split_stride;
    for (int idx = threadIdx.x; idx < NE * 64; idx += 256) {
      const int e = idx >> 6, ln = idx & 63;
      const float v = red[0][e][ln] + red[1][e][ln] + red[2][e][ln] + red[3][e][ln];
      const int i = e & 3, t = e >> 2, ct = t % NT, mt = t / NT;
      const int m = m_base + mt * 16 + 4 * (ln >> 4) + i;
      const int n = n_base + ct * 16 + (ln & 15);
      if (m < a.M && n < a.N) out[(size_t)m * a.ldo + n] = v;
    }
  } else {
    // tile[m][c] for the statistics pass (reuses no LDS of `red`: separate buffer)
    __shared__ float tile[16 * MT][16 * NT + 1];
    for (int idx = threadIdx.x; idx < NE * 64; idx += 256) {
      const int e = idx >> 6, ln = idx & 63;
      const float v = red[0][e][ln] + red[1][e][ln] + red[2][e][ln] + red[3][e][ln];
      const int i = e & 3, t = e >> 2, ct = t % NT, mt = t / NT;
      const int ml = mt * 16 + 4 * (ln >> 4) + i;
      const int c = ct * 16 + (ln & 15);
      tile[ml][c] = v;
      const int m = m_base + ml, n = n_base + c;
      if (a.logits && m < a.M && n < a.N) a.logits[(size_t)m * a.ldl + n] = v;
    }
    __syncthreads();
    for (int ml = threadIdx.x; ml < 16 * MT; ml += 256) {
      const int m = m_base + ml;
      if (m >= a.M) continue;
      float m1 = -INFINITY, m2 = -INFINITY;
      int i1 = 0x7fffffff;
      const int nc = min(16 * NT, a.N - n_base);
      for (int c = 0; c < nc; ++c) {
        const float v = tile[ml][c];
        if (v > m1) { m2 = m1; m1 = v; i1 = n_base + c; }
        else if (v > m2) m2 = v;
      }
      float se = 0.f;
      for (int c = 0; c < nc; ++c) se += __expf(tile[ml][c] - m1);
      a.stats[(size_t)m * a.n_groups + cg] = make_float4(m1, __int_as_float(i1), m2, se);
    }
  }
}

// ---------------------------------------------------------------------------
// host-side dispatch over (dtype, MT, NT, epilogue)

template <typename T, int NT, int EPI>
static hipError_t launch_mt(int MT, dim3 grid, GemmArgs a, hipStream_t s) {
  constexpr int U = 4;
  switch (MT) {
    case 1: gemm_small_m<T, 1, NT, EPI, U><<<grid, 256, 0, s>>>(a); break;
    case 2: gemm_small_m<T, 2, NT, EPI, U><<<grid, 256, 0, s>>>(a); break;
    case 3: gemm_small_m<T, 3, NT, EPI, U><<<grid, 256, 0, s>>>(a); break;
    case 4: gemm_small_m<T, 4, NT, EPI, U><<<grid, 256, 0, s>>>(a); break;
    case 5: gemm_small_m<T, 5, NT, EPI, U><<<grid, 256, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm(bool is_bf16, int MT, int NT, int epi, dim3 grid, const GemmArgs& a, hipStream_t s) {
  if (NT != 2 && NT != 1) return hipErrorInvalidValue;
  if (is_bf16) {
    if (epi == EPI_PARTIAL)
      return NT == 2 ? launch_mt<bf16, 2, EPI_PARTIAL>(MT, grid, a, s) : launch_mt<bf16, 1, EPI_PARTIAL>(MT, grid, a, s);
    return NT == 2 ? launch_mt<bf16, 2, EPI_LOGITS>(MT, grid, a, s) : launch_mt<bf16, 1, EPI_LOGITS>(MT, grid, a, s);
  }
  if (epi == EPI_PARTIAL)
    return NT == 2 ? launch_mt<float, 2, EPI_PARTIAL>(MT, grid, a, s) : launch_mt<float, 1, EPI_PARTIAL>(MT, grid, a, s);
  return NT == 2 ? launch_mt<float, 2, EPI_LOGITS>(MT, grid, a, s) : launch_mt<float, 1, EPI_LOGITS>(MT, grid, a, s);
}

}  // namespace sdv
