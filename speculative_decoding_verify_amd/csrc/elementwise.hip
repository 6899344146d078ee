// Row-wise kernels of the verify forward: tree prologue, embedding + first norm,
// residual add + RMSNorm, QKV epilogue (split-K reduction, rotary embedding, paged
// KV append), SwiGLU, and the LM-head statistics reduction.
//
// Every split-K reduction sums the partials in split order 0..S-1 so results are
// deterministic.  Rounding to the storage type happens exactly where a bf16 model
// stores values: normalised activations, q/k/v after RoPE, attention output and
// SwiGLU output; the residual stream stays fp32.
#include "common.h"
#include "kernels.h"

namespace sdv {

// ---------------------------------------------------------------------------
// Tree bookkeeping (one block): depth(j) = depth(parent(j)) + 1, and the
// ancestor-or-self bit set of every chunk row; LM-head row gather list.
__global__ void prologue_kernel(PrologueArgs a) {
  __shared__ int32_t dep[128];
  __shared__ uint32_t anc[128][4];
  __shared__ int bad;
  if (threadIdx.x == 0) {
    bad = 0;
    for (int j = 0; j < a.T; ++j) {
      int p = a.parent ? a.parent[j] : j - 1;
      bool ok = j == 0 ? p == -1 : (p >= 0 && p < j);
      if (!ok) { bad = 1; p = j - 1; }
      uint32_t m[4] = {0u, 0u, 0u, 0u};
      if (p >= 0) {
        for (int c = 0; c < 4; ++c) m[c] = anc[p][c];
        dep[j] = dep[p] + 1;
      } else {
        dep[j] = 0;
      }
      m[j >> 5] |= 1u << (j & 31);
      for (int c = 0; c < 4; ++c) anc[j][c] = m[c];
    }
  }
  __syncthreads();
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

hipError_t launch_prologue(const PrologueArgs& a, hipStream_t s) {
  prologue_kernel<<<1, 128, 0, s>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// RMSNorm of one fp32 row held in registers (256 threads, PER elements each).
template <typename T, int PER>
SDV_DEV void norm_store(const float (&v)[PER], int d, const float* gain, T* out, float eps, float* red) {
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = threadIdx.x + i * 256;
    if (c < d) ss += v[i] * v[i];
  }
  ss = block_sum_256(ss, red);
  const float rs = rsqrtf(ss / (float)d + eps);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = threadIdx.x + i * 256;
    if (c < d) out[c] = from_f<T>(v[i] * rs * gain[c]);
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
  float v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = threadIdx.x + i * 256;
    v[i] = c < a.d ? to_f<T>(e[c]) : 0.f;
    if (c < a.d) a.x[(size_t)m * a.d + c] = v[i];
  }
  norm_store<T, PER>(v, a.d, a.gain, (T*)a.a + (size_t)m * a.d, a.eps, red);
}

template <typename T, int PER>
__global__ __launch_bounds__(256) void resid_norm_kernel(ResidNormArgs a) {
  __shared__ float red[8];
  const int m = blockIdx.x;
  float v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = threadIdx.x + i * 256;
    if (c < a.d) {
      float acc = 0.f;
      for (int s = 0; s < a.S; ++s) acc += a.part[(size_t)s * a.part_stride + (size_t)m * a.d + c];
      v[i] = a.x[(size_t)m * a.d + c] + acc;
      a.x[(size_t)m * a.d + c] = v[i];
      if (a.hidden) a.hidden[(size_t)m * a.d + c] = v[i];
    } else {
      v[i] = 0.f;
    }
  }
  norm_store<T, PER>(v, a.d, a.gain, (T*)a.a + (size_t)m * a.d, a.eps, red);
}

template <typename T>
static hipError_t launch_rows(bool resid, int d, int M, const void* args, hipStream_t s) {
  const int per = (d + 255) / 256;
#define SDV_ROWS(P)                                                                     \
  if (per <= P) {                                                                       \
    if (resid) resid_norm_kernel<T, P><<<M, 256, 0, s>>>(*(const ResidNormArgs*)args); \
    else embed_norm_kernel<T, P><<<M, 256, 0, s>>>(*(const EmbedArgs*)args);           \
    return hipGetLastError();                                                           \
  }
  SDV_ROWS(1) SDV_ROWS(2) SDV_ROWS(4) SDV_ROWS(8) SDV_ROWS(16) SDV_ROWS(32)
#undef SDV_ROWS
  return hipErrorInvalidValue;
}

hipError_t launch_embed_norm(bool is_bf16, const EmbedArgs& a, hipStream_t s) {
  return is_bf16 ? launch_rows<bf16>(false, a.d, a.M, &a, s) : launch_rows<float>(false, a.d, a.M, &a, s);
}
hipError_t launch_resid_norm(bool is_bf16, const ResidNormArgs& a, hipStream_t s) {
  return is_bf16 ? launch_rows<bf16>(true, a.d, a.M, &a, s) : launch_rows<float>(true, a.d, a.M, &a, s);
}

// ---------------------------------------------------------------------------
// QKV epilogue: one block per chunk row m = b*T + t.  Sums the split partials,
// applies the rotary embedding (rotate-half pairs (i, i + dh/2), angle
// pos * theta^(-2i/dh) with pos = seq_len[b] + depth[t], computed in fp64),
// rounds to the storage type, writes q, and appends k and v to the paged cache at
// slot seq_len[b] + t (k token-major, v transposed inside the page).
template <typename T>
__global__ __launch_bounds__(256) void qkv_epilogue_kernel(QkvArgs a) {
  const int m = blockIdx.x, b = m / a.T, t = m % a.T;
  const int C = a.seq_len[b];
  const int slot = C + t;
  const int half = a.dh / 2;
  const int nh = a.H + 2 * a.Hkv;
  const int N = nh * a.dh;
  const int cap = a.max_blocks * 16;
  bool ok = (C >= 0) && (C <= a.max_ctx) && (slot < cap);
  int phys = -1;
  if (ok) {
    phys = a.block_table[(size_t)b * a.max_blocks + (slot >> 4)];
    ok = phys >= 0 && phys < a.n_blocks;
  }
  if (!ok && threadIdx.x == 0) set_err(a.err, b, 0x4);
  const double pos = (double)(max(C, 0) + a.depth[t]);
  const double l2t = log2((double)a.rope_theta);
  for (int idx = threadIdx.x; idx < nh * half; idx += blockDim.x) {
    const int hh = idx / half, i = idx % half;
    const int c1 = hh * a.dh + i, c2 = c1 + half;
    float x1 = 0.f, x2 = 0.f;
    for (int s = 0; s < a.S; ++s) {
      const float* p = a.part + (size_t)s * a.part_stride + (size_t)m * N;
      x1 += p[c1];
      x2 += p[c2];
    }
    float y1 = x1, y2 = x2;
    if (hh < a.H + a.Hkv) {
      const double ang = pos * exp2(-(2.0 * i / a.dh) * l2t);
      double sn, cs;
      sincos(ang, &sn, &cs);
      const float c = (float)cs, sf = (float)sn;
      y1 = x1 * c - x2 * sf;
      y2 = x2 * c + x1 * sf;
    }
    if (hh < a.H) {
      T* q = (T*)a.q + (size_t)m * a.H * a.dh;
      q[c1] = from_f<T>(y1);
      q[c2] = from_f<T>(y2);
    } else if (ok) {
      const int g = (hh < a.H + a.Hkv) ? hh - a.H : hh - a.H - a.Hkv;
      const size_t page = (size_t)phys * a.Hkv + g;
      const int off = slot & 15;
      if (hh < a.H + a.Hkv) {
        T* kp = (T*)a.k_pages + (page * 16 + off) * a.dh;
        kp[i] = from_f<T>(y1);
        kp[i + half] = from_f<T>(y2);
      } else {
        T* vp = (T*)a.v_pages + page * a.dh * 16;
        vp[(size_t)i * 16 + off] = from_f<T>(y1);
        vp[(size_t)(i + half) * 16 + off] = from_f<T>(y2);
      }
    }
  }
}

hipError_t launch_qkv_epilogue(bool is_bf16, const QkvArgs& a, hipStream_t s) {
  const int M = a.B * a.T;
  if (is_bf16) qkv_epilogue_kernel<bf16><<<M, 256, 0, s>>>(a);
  else qkv_epilogue_kernel<float><<<M, 256, 0, s>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// SwiGLU: h = silu(gate) * up, with silu(z) = z / (1 + exp(-z)).
template <typename T>
__global__ __launch_bounds__(256) void swiglu_kernel(SwigluArgs a) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)a.M * a.F) return;
  const int m = (int)(idx / a.F), f = (int)(idx % a.F);
  float gt = 0.f, up = 0.f;
  for (int s = 0; s < a.S; ++s) {
    const float* p = a.part + (size_t)s * a.part_stride + (size_t)m * 2 * a.F;
    gt += p[f];
    up += p[a.F + f];
  }
  const float sl = gt / (1.f + expf(-gt));
  ((T*)a.h)[idx] = from_f<T>(sl * up);
}

hipError_t launch_swiglu(bool is_bf16, const SwigluArgs& a, hipStream_t s) {
  const size_t n = (size_t)a.M * a.F;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (is_bf16) swiglu_kernel<bf16><<<blocks, 256, 0, s>>>(a);
  else swiglu_kernel<float><<<blocks, 256, 0, s>>>(a);
  return hipGetLastError();
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
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= a.rows) return;
  Top2 acc = {-INFINITY, -INFINITY, 0.f, 0x7fffffff};
  for (int c = lane; c < a.n_groups; c += 64) {
    const float4 s = a.stats[(size_t)row * a.n_groups + c];
    acc = top2_merge(acc, Top2{s.x, s.z, s.w, __float_as_int(s.y)});
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    Top2 oth;
    oth.m1 = __shfl_xor(acc.m1, o);
    oth.m2 = __shfl_xor(acc.m2, o);
    oth.se = __shfl_xor(acc.se, o);
    oth.i1 = __shfl_xor(acc.i1, o);
    // merge in a lane-order-independent way: the lower lane's state first
    acc = (lane & o) ? top2_merge(oth, acc) : top2_merge(acc, oth);
  }
  if (lane == 0) {
    a.argmax[row] = acc.i1;
    a.margin[row] = acc.m1 - acc.m2;
    a.lse[row] = acc.m1 + logf(acc.se);
  }
}

hipError_t launch_row_reduce(const RowReduceArgs& a, hipStream_t s) {
  row_reduce_kernel<<<(a.rows + 3) / 4, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace sdv
