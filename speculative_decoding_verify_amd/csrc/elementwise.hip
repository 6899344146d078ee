// Row-wise kernels of the verify forward: prologue (tree bookkeeping and the
// rotary table), embedding + first norm, residual add + RMSNorm, and the LM-head
// statistics reduction.  The residual stream is fp32; normalised rows are written
// in the activation tile format of the GEMMs (bf16 hi/lo pairs for bf16 models, fp32
// otherwise; common.h).
//
// Every split-K reduction sums the partials in split order 0..S-1 so results are
// deterministic.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace sdv {

// ---------------------------------------------------------------------------
// Prologue: tree bookkeeping (depth(j) = depth(parent(j)) + 1 and the
// ancestor-or-self bits of every chunk row), the LM-head row gather list, the
// rotary table of the pass (for chunk row t of sequence b at position
// p = seq_len[b] + depth(t), entry i holds (cos, sin) of p * theta^(-2i/dh),
// evaluated in fp64 and rounded to fp32) and the cache page and slot every chunk
// row's K/V goes to (slot seq_len[b] + t).
__global__ __launch_bounds__(256) void prologue_kernel(PrologueArgs a) {
  __shared__ int32_t par[128], dep[128];
  __shared__ uint32_t anc[128][4];
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  // parents (an invalid one is reported and replaced by the previous row)
  for (int j = threadIdx.x; j < a.T; j += blockDim.x) {
    int p = a.parent ? a.parent[j] : j - 1;
    const bool ok = j == 0 ? p == -1 : (p >= 0 && p < j);
    if (!ok) { bad = 1; p = j - 1; }
    par[j] = p;
  }
  __syncthreads();
  // every row walks up to the root (parents strictly decrease, so the walk ends)
  for (int j = threadIdx.x; j < a.T; j += blockDim.x) {
    uint32_t m[4] = {0u, 0u, 0u, 0u};
    int d = -1;
    for (int k = j; k >= 0; k = par[k]) {
#pragma unroll
      for (int c = 0; c < 4; ++c) m[c] |= (k >> 5) == c ? 1u << (k & 31) : 0u;
      ++d;
    }
    dep[j] = d;
    for (int c = 0; c < 4; ++c) anc[j][c] = m[c];
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int j = threadIdx.x; j < a.T; j += blockDim.x) {
      a.depth[j] = dep[j];
      for (int c = 0; c < 4; ++c) a.anc[j * 4 + c] = anc[j][c];
    }
    for (int i = threadIdx.x; i < a.B * a.R; i += blockDim.x) {
      const int b = i / a.R, r = i % a.R;
      int row = a.logit_rows[r];
      if (row < 0 || row >= a.T) { set_err(a.err, b, 0x2); row = 0; }
      a.lm_rows[i] = b * a.T + row;
    }
    if (bad)
      for (int b = threadIdx.x; b < a.B; b += blockDim.x) set_err(a.err, b, 0x2);
  }
  const int half = a.dh / 2;
  const double l2t = log2((double)a.rope_theta);
  const int n = a.B * a.T * half;
  for (int idx = blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += gridDim.x * blockDim.x) {
    const int i = idx % half, bt = idx / half, t = bt % a.T, b = bt / a.T;
    const double pos = (double)(max(a.seq_len[b], 0) + dep[t]);
    const double ang = pos * exp2(-(2.0 * i / a.dh) * l2t);
    double sn, cs;
    sincos(ang, &sn, &cs);
    a.rope[idx] = make_float2((float)cs, (float)sn);
  }
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < a.n_zero; i += gridDim.x * blockDim.x) a.zero[i] = 0u;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < a.B * a.T; i += gridDim.x * blockDim.x) {
    const int b = i / a.T, t = i % a.T;
    const int C = a.seq_len[b];
    const int slot = C + t;
    int phys = -1;
    if (C >= 0 && C <= a.max_ctx && slot < a.max_blocks * 16) phys = a.block_table[(size_t)b * a.max_blocks + (slot >> 4)];
    if (phys < 0 || phys >= a.n_blocks) {
      phys = -1;
      set_err(a.err, b, 0x4);
    }
    a.kv_dst[i] = make_int2(phys, slot & 15);
  }
}

hipError_t launch_prologue(const PrologueArgs& a, hipStream_t s) {
  const int n = a.B * a.T * (a.dh / 2);
  const int blocks = max(1, min(64, (n + 255) / 256));
  prologue_kernel<<<blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// RMSNorm of one fp32 row held in registers (NTHR threads, PER elements each,
// element c = threadIdx.x * PER + i), stored as row m of an activation operand.
// The thread's PER gain values, loaded up front (before the block reduction's
// barrier, which loads cannot cross).
template <int PER>
SDV_DEV void load_gain(const float* gain, int d, float (&g)[PER]) {
  const int c0 = threadIdx.x * PER;
#pragma unroll
  for (int q = 0; q < PER / 4; ++q) {
    const float4 v = c0 < d ? ((const float4*)(gain + c0))[q] : make_float4(0.f, 0.f, 0.f, 0.f);
    g[4 * q] = v.x; g[4 * q + 1] = v.y; g[4 * q + 2] = v.z; g[4 * q + 3] = v.w;
  }
}

template <typename T, int PER, int NTHR = 256>
SDV_DEV void norm_store(const float (&v)[PER], int d, const float (&gain)[PER], void* out, int m, float eps,
                        float* red) {
  static_assert(PER % 8 == 0, "whole k groups per thread");
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) ss += v[i] * v[i];
  ss = NTHR == 256 ? block_sum_256(ss, red) : block_sum<NTHR / 64>(ss, red);
  const float rs = rsqrtf(ss / (float)d + eps);
  const int c0 = threadIdx.x * PER;
  if (c0 < d) {
#pragma unroll
    for (int g = 0; g < PER / 8; ++g) {
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = v[g * 8 + e] * rs * gain[g * 8 + e];
      act_store8<T>(out, d, m, c0 + g * 8, y);
    }
  }
}

template <typename T, int PER>
__global__ __launch_bounds__(256) void embed_norm_kernel(EmbedArgs a) {
  __shared__ float red[8];
  const int m = blockIdx.x;
  int tok = a.tokens[m];
  if (tok < 0 || tok >= a.V) {
    if (threadIdx.x == 0) set_err(a.err, m / a.T, 0x1);
    tok = 0;
  }
  const T* e = (const T*)a.embed + (size_t)tok * a.d;
  const int c0 = threadIdx.x * PER;
  float gn[PER];
  load_gain<PER>(a.gain, a.d, gn);
  float v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    v[i] = c0 < a.d ? to_f<T>(e[c0 + i]) : 0.f;
    if (c0 < a.d) a.x[(size_t)m * a.d + c0 + i] = v[i];
  }
  norm_store<T, PER>(v, a.d, gn, a.a, m, a.eps, red);
}

// x + sum of the S split partials (in split order), then RMSNorm -> a.  Each thread
// owns PER consecutive columns; all partial loads are issued before use, into
// registers for at most MAXS partials (the launch picks the smallest of 4, 8, 16 that
// holds S: with room for 16, PER = 16 takes every register and one wave per SIMD; the
// batched pass, S = 3: 75 -> 60 us per launch).  Block j:
// without a.rows, row j (x updated in place); with a.rows, output row j < n_rows
// normalises source row rows[j], and the blocks after those write hidden rows.
template <typename T, int PER, int MAXS, int NTHR = 256>
__global__ __launch_bounds__(NTHR) void resid_norm_kernel(ResidNormArgs a) {
  __shared__ float red[NTHR / 64 > 8 ? NTHR / 64 : 8];
  const bool gather = a.rows != nullptr;
  const bool hidden_only = gather && (int)blockIdx.x >= a.n_rows;
  const int m = !gather ? blockIdx.x : hidden_only ? blockIdx.x - a.n_rows : a.rows[blockIdx.x];
  const int c0 = threadIdx.x * PER;
  const bool on = c0 < a.d;
  float v[PER], gn[PER];
  load_gain<PER>(a.gain, a.d, gn);
  float4 x0[PER / 4];
#pragma unroll
  for (int q = 0; q < PER / 4; ++q) x0[q] = on ? ((const float4*)(a.x + (size_t)m * a.d + c0))[q] : make_float4(0.f, 0.f, 0.f, 0.f);
  float4 acc4[PER / 4];
#pragma unroll
  for (int q = 0; q < PER / 4; ++q) acc4[q] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (on) {
    float4 pv[MAXS][PER / 4];
#pragma unroll
    for (int s = 0; s < MAXS; ++s)
      if (s < a.S) {
        const float4* p = (const float4*)(a.part + (size_t)s * a.part_stride + (size_t)m * a.d + c0);
#pragma unroll
        for (int q = 0; q < PER / 4; ++q) pv[s][q] = p[q];
      }
#pragma unroll
    for (int s = 0; s < MAXS; ++s)
      if (s < a.S) {
#pragma unroll
        for (int q = 0; q < PER / 4; ++q) {
          acc4[q].x += pv[s][q].x; acc4[q].y += pv[s][q].y; acc4[q].z += pv[s][q].z; acc4[q].w += pv[s][q].w;
        }
      }
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
      float4 x = x0[q];
      x.x += acc4[q].x; x.y += acc4[q].y; x.z += acc4[q].z; x.w += acc4[q].w;
      if (!gather) ((float4*)(a.x + (size_t)m * a.d + c0))[q] = x;
      if (hidden_only) ((float4*)(a.hidden + (size_t)m * a.d + c0))[q] = x;
      v[4 * q] = x.x; v[4 * q + 1] = x.y; v[4 * q + 2] = x.z; v[4 * q + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i) v[i] = 0.f;
  }
  if (hidden_only) return;   // uniform over the block
  norm_store<T, PER, NTHR>(v, a.d, gn, a.a, blockIdx.x, a.eps, red);
}

// PER columns per thread: the smallest of 8, 16, 24, 32 with 256 * PER >= d and
// d % PER == 0 (d is a multiple of 64, so PER = 8 always divides it)
template <typename T>
static hipError_t launch_rows(bool resid, int d, int blocks, const void* args, hipStream_t s) {
#define SDV_ROWS(P)                                                                          \
  if (256 * P >= d && d % P == 0) {                                                          \
    if (resid && ((const ResidNormArgs*)args)->S <= 4)                                       \
      resid_norm_kernel<T, P, 4><<<blocks, 256, 0, s>>>(*(const ResidNormArgs*)args);        \
    else if (resid && ((const ResidNormArgs*)args)->S <= 8)                                  \
      resid_norm_kernel<T, P, 8><<<blocks, 256, 0, s>>>(*(const ResidNormArgs*)args);        \
    else if (resid) resid_norm_kernel<T, P, 16><<<blocks, 256, 0, s>>>(*(const ResidNormArgs*)args); \
    else embed_norm_kernel<T, P><<<blocks, 256, 0, s>>>(*(const EmbedArgs*)args);           \
    return hipGetLastError();                                                           \
  }
  SDV_ROWS(8) SDV_ROWS(16) SDV_ROWS(24) SDV_ROWS(32)
#undef SDV_ROWS
  return hipErrorInvalidValue;
}

hipError_t launch_embed_norm(bool is_bf16, const EmbedArgs& a, hipStream_t s) {
  return is_bf16 ? launch_rows<bf16>(false, a.d, a.M, &a, s) : launch_rows<float>(false, a.d, a.M, &a, s);
}
// Few rows of a wide model (fewer rows than compute units, d above 2048): 8 columns per
// thread and d / 8 threads per row, so the partial loads spread over more waves
template <typename T, int NTHR>
static hipError_t launch_resid_wide(const ResidNormArgs& a, int blocks, hipStream_t s) {
  if (a.S <= 4) resid_norm_kernel<T, 8, 4, NTHR><<<blocks, NTHR, 0, s>>>(a);
  else if (a.S <= 8) resid_norm_kernel<T, 8, 8, NTHR><<<blocks, NTHR, 0, s>>>(a);
  else resid_norm_kernel<T, 8, 16, NTHR><<<blocks, NTHR, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_resid_norm(bool is_bf16, const ResidNormArgs& a, hipStream_t s) {
  if (a.S > 16 || (a.rows && a.n_rows < 1)) return hipErrorInvalidValue;
  const int blocks = a.rows ? a.n_rows + (a.hidden ? a.M : 0) : a.M;
  if (blocks <= 256 && a.d > 2048 && a.d % 8 == 0) {
    if (a.d <= 4096) return is_bf16 ? launch_resid_wide<bf16, 512>(a, blocks, s) : launch_resid_wide<float, 512>(a, blocks, s);
    if (a.d <= 8192) return is_bf16 ? launch_resid_wide<bf16, 1024>(a, blocks, s) : launch_resid_wide<float, 1024>(a, blocks, s);
  }
  return is_bf16 ? launch_rows<bf16>(true, a.d, blocks, &a, s) : launch_rows<float>(true, a.d, blocks, &a, s);
}

// ---------------------------------------------------------------------------
// Merge the LM-head column-group statistics of each row (one wave per row):
// argmax (lowest index among equal maxima), top-2 margin and log-sum-exp.
struct Top2 {
  float m1, m2, se;
  int i1;
};
SDV_DEV Top2 top2_merge(Top2 x, Top2 y) {
  const bool ywins = y.m1 > x.m1 || (y.m1 == x.m1 && y.i1 < x.i1);
  const Top2 win = ywins ? y : x, lose = ywins ? x : y;
  Top2 o;
  o.m1 = win.m1;
  o.i1 = win.i1;
  o.m2 = fmaxf(win.m2, lose.m1);
  o.se = win.se + (lose.se > 0.f ? lose.se * __expf(lose.m1 - win.m1) : 0.f);
  return o;
}

__global__ __launch_bounds__(256) void row_reduce_kernel(RowReduceArgs a) {
  const int row = blockIdx.x;
  Top2 acc = {-INFINITY, -INFINITY, 0.f, 0x7fffffff};
  for (int c = threadIdx.x; c < a.n_groups; c += 256) {
    const float4 s = a.stats[(size_t)row * a.n_groups + c];
    acc = top2_merge(acc, Top2{s.x, s.z, s.w, __float_as_int(s.y)});
  }
  __shared__ float sm1[256], sm2[256], sse[256];
  __shared__ int si1[256];
  sm1[threadIdx.x] = acc.m1; sm2[threadIdx.x] = acc.m2; sse[threadIdx.x] = acc.se; si1[threadIdx.x] = acc.i1;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) {
      const int u = threadIdx.x + o;
      Top2 x{sm1[threadIdx.x], sm2[threadIdx.x], sse[threadIdx.x], si1[threadIdx.x]};
      Top2 y{sm1[u], sm2[u], sse[u], si1[u]};
      x = top2_merge(x, y);
      sm1[threadIdx.x] = x.m1; sm2[threadIdx.x] = x.m2; sse[threadIdx.x] = x.se; si1[threadIdx.x] = x.i1;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    a.argmax[row] = si1[0];
    a.margin[row] = sm1[0] - sm2[0];
    a.lse[row] = sm1[0] + logf(sse[0]);
  }
}

hipError_t launch_row_reduce(const RowReduceArgs& a, hipStream_t s) {
  row_reduce_kernel<<<a.rows, 256, 0, s>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Codebook heads ("An Efficient vLLM-Based Inference Pipeline for Unified Audio
// Understanding and Generation", page 2, Figure 1 and the paired-guidance section).
// Stream s scores codes with W_cb (h_n + e_s), h_n the final-normed hidden row; by
// linearity that is W_cb h_n + W_cb e_s, so the head GEMM runs on the B*R logit rows
// plus the S embedding rows, and the merge kernel adds the two.

template <typename T>
__global__ __launch_bounds__(256) void stream_rows_kernel(StreamRowsArgs a) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < a.S * a.d; i += gridDim.x * blockDim.x) {
    const int s = i / a.d, k = i % a.d;
    act_store1<T>(a.act, a.d, a.first_row + s, k, a.e[i]);
  }
}

hipError_t launch_stream_rows(bool is_bf16, const StreamRowsArgs& a, hipStream_t s) {
  const int blocks = std::max(1, std::min(64, (a.S * a.d + 255) / 256));
  if (is_bf16) stream_rows_kernel<bf16><<<blocks, 256, 0, s>>>(a);
  else stream_rows_kernel<float><<<blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

// One workgroup per (b, r, s): logits of codebook s for logit row r of sequence b.
// Rows of a guidance pair (partners c < u) both get u + w (c - u), evaluated in fp32
// as written.  Statistics: argmax (lowest index on ties), top-2 margin, log-sum-exp,
// reduced in a fixed order.
__global__ __launch_bounds__(256) void cb_merge_kernel(CbMergeArgs a) {
  const int s = blockIdx.x % a.S;
  const int br = blockIdx.x / a.S;
  const int b = br / a.R, r = br % a.R;
  int p = a.partner ? a.partner[b] : -1;
  if (p >= 0 && !(p < a.B && p != b && a.partner[p] == b)) {
    if (threadIdx.x == 0) set_err(a.err, b, 0x20);
    p = -1;
  }
  const int c = p >= 0 ? min(b, p) : b, u = p >= 0 ? max(b, p) : -1;
  const size_t rc = (size_t)(c * a.R + r) * a.Vc, ru = (size_t)((u < 0 ? 0 : u) * a.R + r) * a.Vc;
  const size_t re = (size_t)(a.B * a.R + s) * a.Vc;
  float* lout = a.logits ? a.logits + ((size_t)(b * a.R + r) * a.S + s) * a.Vc : nullptr;
  Top2 acc = {-INFINITY, -INFINITY, 0.f, 0x7fffffff};
  for (int v = threadIdx.x; v < a.Vc; v += 256) {
    float lc = 0.f, lu = 0.f, le = 0.f;
    for (int k = 0; k < a.n_split; ++k) {
      const float* pb = a.base + (size_t)k * a.split_stride;
      lc += pb[rc + v];
      le += pb[re + v];
      if (u >= 0) lu += pb[ru + v];
    }
    const float cv = lc + le;
    float x = cv;
    if (u >= 0) {
      const float uv = lu + le;
      x = uv + a.w * (cv - uv);
    }
    if (lout) lout[v] = x;
    acc = top2_merge(acc, Top2{x, -INFINITY, 1.f, v});
  }
  __shared__ float sm1[256], sm2[256], sse[256];
  __shared__ int si1[256];
  sm1[threadIdx.x] = acc.m1; sm2[threadIdx.x] = acc.m2; sse[threadIdx.x] = acc.se; si1[threadIdx.x] = acc.i1;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) {
      const int q = threadIdx.x + o;
      Top2 x{sm1[threadIdx.x], sm2[threadIdx.x], sse[threadIdx.x], si1[threadIdx.x]};
      Top2 y{sm1[q], sm2[q], sse[q], si1[q]};
      x = top2_merge(x, y);
      sm1[threadIdx.x] = x.m1; sm2[threadIdx.x] = x.m2; sse[threadIdx.x] = x.se; si1[threadIdx.x] = x.i1;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    if (a.cb_argmax) a.cb_argmax[(size_t)br * a.S + s] = si1[0];
    if (s == 0) {
      a.argmax[br] = a.token_base + si1[0];
      a.margin[br] = sm1[0] - sm2[0];
      a.lse[br] = sm1[0] + logf(sse[0]);
    }
  }
}

hipError_t launch_cb_merge(const CbMergeArgs& a, hipStream_t s) {
  cb_merge_kernel<<<a.B * a.R * a.S, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace sdv
