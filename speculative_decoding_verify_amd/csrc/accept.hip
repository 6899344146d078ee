// Acceptance and cache-commit kernels.
//
// Greedy acceptance follows "Decode Before You Hear" (page 1), method step 4:
// n = min({i-1 : y~_i != argmax p_i} U {gamma}) plus the correction argmax
// p_{n+1}; with a runner-up branch (step 2) it becomes a walk down the draft tree.
// Speculative sampling follows "speculative-decoding-omni" (page 3), section 2:
// accept x with probability min(1, p(x)/q(x)), on the first rejection draw from
// norm(max(0, p - q)), otherwise a bonus draw from p.
#include "common.h"
#include "kernels.h"

namespace sdv {

// ---------------------------------------------------------------------------
// Greedy tree walk: one block per sequence stages its tokens, the tree and the
// argmax of every logit row in LDS; every row checks in parallel whether it is the
// accepted child of its parent (its token equals the parent's argmax), then one
// thread walks from the last audio row along the accepted children, and all threads
// write the path and the commit moves.
__global__ __launch_bounds__(128) void accept_greedy_kernel(GreedyArgs a) {
  __shared__ int32_t tok[128], par[128], am_of_row[128], path[128], child_of[128], n_match[128];
  __shared__ int32_t s_n, s_base;
  const int b = blockIdx.x;
  for (int j = threadIdx.x; j < a.T; j += blockDim.x) {
    tok[j] = a.tokens[(size_t)b * a.T + j];
    par[j] = a.parent ? a.parent[j] : j - 1;
    am_of_row[j] = -1;
    child_of[j] = 0x7fffffff;
    n_match[j] = 0;
  }
  if (threadIdx.x == 0) s_base = a.base_len ? a.base_len[b] : 0;
  __syncthreads();
  for (int i = threadIdx.x; i < a.R; i += blockDim.x) {
    const int row = a.logit_rows[i];
    if (row >= 0 && row < a.T) am_of_row[row] = a.argmax[(size_t)b * a.R + i];
  }
  __syncthreads();
  for (int j = threadIdx.x; j < a.T; j += blockDim.x) {
    const int p = par[j];
    if (p >= 0 && p < j && am_of_row[p] >= 0 && tok[j] == am_of_row[p]) {
      atomicMin(&child_of[p], j);   // siblings with equal tokens: the lowest row, reported below
      atomicAdd(&n_match[p], 1);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int node = a.L_a - 1, n = 0, next = -1;
    for (;;) {
      const int am = am_of_row[node];
      next = am;
      if (am < 0) break;
      if (n_match[node] > 1) set_err(a.err, b, 0x10);
      const int child = child_of[node];
      if (child == 0x7fffffff) break;
      path[n++] = child;
      node = child;
    }
    s_n = n;
    a.n_out[b] = n;
    a.next_out[b] = next;
    if (a.base_len && a.keep_out) a.keep_out[b] = s_base + a.L_a + n;
  }
  __syncthreads();
  const int n = s_n, base = s_base;
  for (int i = threadIdx.x; i < a.T; i += blockDim.x) {
    if (a.path_out) a.path_out[(size_t)b * a.T + i] = i < n ? path[i] : -1;
    if (a.base_len && a.move_src && a.move_dst) {
      // accepted row path[i] must end at slot base + L_a + i
      const bool mv = i < n && path[i] != a.L_a + i;
      a.move_src[(size_t)b * a.T + i] = mv ? base + path[i] : -1;
      a.move_dst[(size_t)b * a.T + i] = mv ? base + a.L_a + i : -1;
    }
  }
}

hipError_t launch_accept_greedy(const GreedyArgs& a, hipStream_t s) {
  accept_greedy_kernel<<<a.B, 128, 0, s>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// KV commit: block (b, layer) validates the sequence's plan, performs its moves in
// ascending order (each thread owns fixed element positions, so a slot written by
// one move and read by a later one is handled in order) and sets seq_len.  The move
// lists are staged in LDS, 256 entries at a time, and validated in parallel.
__global__ __launch_bounds__(256) void kv_rollback_kernel(RollbackArgs a) {
  constexpr int CH = 256;
  __shared__ int32_t msrc[CH], mdst[CH];
  __shared__ int ok;
  const int b = blockIdx.x, l = blockIdx.y;
  const int cap = a.max_blocks * 16;
  const int32_t* bt = a.block_table + (size_t)b * a.max_blocks;
  const int keep = a.keep_len[b];
  if (threadIdx.x == 0) ok = keep >= 0 && keep <= cap;
  __syncthreads();
  for (int c0 = 0; c0 < a.max_move; c0 += CH) {
    const int i = c0 + threadIdx.x;
    if (i < a.max_move) {
      const int s = a.move_src[(size_t)b * a.max_move + i];
      if (s >= 0) {
        const int d = a.move_dst[(size_t)b * a.max_move + i];
        bool good = s < cap && d >= 0 && d < cap;
        if (good) {
          const int ps = bt[s >> 4], pd = bt[d >> 4];
          good = ps >= 0 && ps < a.n_blocks && pd >= 0 && pd < a.n_blocks;
        }
        if (!good) ok = 0;
      }
    }
  }
  __syncthreads();
  if (!ok) {
    if (l == 0 && threadIdx.x == 0) set_err(a.err, b, 0x8);
    return;
  }
  const int per = a.Hkv * a.dh;
  for (int c0 = 0; c0 < a.max_move; c0 += CH) {
    const int n = min(CH, a.max_move - c0);
    if (threadIdx.x < n) {
      msrc[threadIdx.x] = a.move_src[(size_t)b * a.max_move + c0 + threadIdx.x];
      mdst[threadIdx.x] = a.move_dst[(size_t)b * a.max_move + c0 + threadIdx.x];
    }
    __syncthreads();
    for (int i = 0; i < n; ++i) {
      const int s = msrc[i], d = mdst[i];
      if (s < 0 || s == d) continue;
      const size_t ps = (size_t)l * a.n_blocks + bt[s >> 4], pd = (size_t)l * a.n_blocks + bt[d >> 4];
      const int os = s & 15, od = d & 15;
      for (int e = threadIdx.x; e < per; e += blockDim.x) {
        const int g = e / a.dh, dd = e % a.dh;
        const size_t ks = ((ps * a.Hkv + g) * 16 + os) * a.dh + dd, kd = ((pd * a.Hkv + g) * 16 + od) * a.dh + dd;
        const size_t vs = ((ps * a.Hkv + g) * a.dh + dd) * 16 + os, vd = ((pd * a.Hkv + g) * a.dh + dd) * 16 + od;
        if (a.elem_bytes == 2) {
          ((bf16*)a.k_pages)[kd] = ((const bf16*)a.k_pages)[ks];
          ((bf16*)a.v_pages)[vd] = ((const bf16*)a.v_pages)[vs];
        } else {
          ((float*)a.k_pages)[kd] = ((const float*)a.k_pages)[ks];
          ((float*)a.v_pages)[vd] = ((const float*)a.v_pages)[vs];
        }
      }
    }
    __syncthreads();
  }
  if (l == 0 && threadIdx.x == 0) a.seq_len[b] = keep;
}

hipError_t launch_kv_rollback(const RollbackArgs& a, hipStream_t s) {
  dim3 grid(a.B, a.L);
  kv_rollback_kernel<<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Speculative sampling.
//
// Rows: target rows r < B*(k+1) (row b*(k+1)+i), then draft rows (b*k+i).
// All exponentials are taken of (z - rowmax) * c with c = log2(e) / temperature,
// which keeps the argument exact-ish for the terms that matter.

static constexpr float LOG2E = 1.4426950408889634f;

SDV_DEV void ms_merge(float& m, double& s, float m2, double s2, float c) {
  if (s2 == 0.0) return;
  if (s == 0.0) { m = m2; s = s2; return; }
  if (m2 > m) { s = s * (double)exp2f((m - m2) * c) + s2; m = m2; }
  else s += s2 * (double)exp2f((m2 - m) * c);
}

__global__ __launch_bounds__(256) void spec_row_stats_kernel(SampleArgs a) {
  const int row = blockIdx.x;
  const int nt = a.B * (a.k + 1);
  const float* z = row < nt ? a.tgt + (size_t)row * a.V : a.drf + (size_t)(row - nt) * a.V;
  const float c = LOG2E * a.inv_temp;
  float m = -INFINITY;
  double s = 0.0;
  // online max / sum; 16-byte loads when the row is aligned
  const bool vec = ((reinterpret_cast<uintptr_t>(z) & 15) == 0);
  const int nv = vec ? a.V / 4 : 0;
  for (int i = threadIdx.x; i < nv; i += 256) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(z) + i);
    const float vm = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
    if (vm > m) { s = s * (double)exp2f((m - vm) * c); m = vm; }
    s += (double)(exp2f((v.x - m) * c) + exp2f((v.y - m) * c) + exp2f((v.z - m) * c) + exp2f((v.w - m) * c));
  }
  for (int i = nv * 4 + threadIdx.x; i < a.V; i += 256) {
    const float v = z[i];
    if (v > m) { s = s * (double)exp2f((m - v) * c); m = v; }
    s += (double)exp2f((v - m) * c);
  }
  // block merge in a fixed pattern
  __shared__ float sm[256];
  __shared__ double ss[256];
  sm[threadIdx.x] = m;
  ss[threadIdx.x] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) {
      float m1 = sm[threadIdx.x];
      double s1 = ss[threadIdx.x];
      ms_merge(m1, s1, sm[threadIdx.x + o], ss[threadIdx.x + o], c);
      sm[threadIdx.x] = m1;
      ss[threadIdx.x] = s1;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    a.row_m[row] = sm[0];
    a.row_s[row] = ss[0];
  }
}

// p(x) in fp64 from the row statistics
SDV_DEV double prob_at(float zx, float m, double s, float inv_temp) {
  return exp2((double)(zx - m) * (1.4426950408889634 * (double)inv_temp)) / s;
}

__global__ void spec_decide_kernel(SampleArgs a) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= a.B) return;
  const int nt = a.B * (a.k + 1);
  int pos = a.k;
  for (int i = 0; i < a.k; ++i) {
    int x = a.drafts[(size_t)b * a.k + i];
    x = min(max(x, 0), a.V - 1);
    const int rt = b * (a.k + 1) + i, rd = nt + b * a.k + i;
    const double px = prob_at(a.tgt[(size_t)rt * a.V + x], a.row_m[rt], a.row_s[rt], a.inv_temp);
    const double qx = prob_at(a.drf[(size_t)(rd - nt) * a.V + x], a.row_m[rd], a.row_s[rd], a.inv_temp);
    const bool acc = qx > 0.0 ? a.u_acc[(size_t)b * a.k + i] < px / qx : px > 0.0;
    if (!acc) { pos = i; break; }
  }
  a.first_rej[b] = pos;
  a.n_out[b] = pos;
}

// quantised weight of index v for the draw of sequence b: max(0, p - q) at a
// rejection (which = 0) or p (which = 1, also the bonus row)
SDV_DEV long long qweight(const SampleArgs& a, int b, int pos, int v, int which) {
  const int nt = a.B * (a.k + 1);
  const float c = LOG2E * a.inv_temp;
  const int rt = b * (a.k + 1) + pos;
  const float p = exp2f((a.tgt[(size_t)rt * a.V + v] - a.row_m[rt]) * c) * (float)(1.0 / a.row_s[rt]);
  float w = p;
  if (which == 0 && pos < a.k) {
    const int rd = nt + b * a.k + pos;
    const float q = exp2f((a.drf[(size_t)(rd - nt) * a.V + v] - a.row_m[rd]) * c) * (float)(1.0 / a.row_s[rd]);
    w = fmaxf(0.f, p - q);
  }
  return (long long)((double)w * 1099511627776.0);  // floor(w * 2^40), w >= 0
}

__global__ __launch_bounds__(256) void spec_chunk_sum_kernel(SampleArgs a) {
  const int b = blockIdx.y, ch = blockIdx.x;
  const int pos = a.first_rej[b];
  const int v0 = ch * a.chunk, v1 = min(a.V, v0 + a.chunk);
  long long s0 = 0, s1 = 0;
  for (int v = v0 + threadIdx.x; v < v1; v += 256) {
    s0 += qweight(a, b, pos, v, 0);
    s1 += qweight(a, b, pos, v, 1);
  }
  __shared__ long long r0[256], r1[256];
  r0[threadIdx.x] = s0;
  r1[threadIdx.x] = s1;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) { r0[threadIdx.x] += r0[threadIdx.x + o]; r1[threadIdx.x] += r1[threadIdx.x + o]; }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    a.chunk_sum[((size_t)b * a.n_chunks + ch) * 2] = r0[0];
    a.chunk_sum[((size_t)b * a.n_chunks + ch) * 2 + 1] = r1[0];
  }
}

// inverse CDF: smallest v with (running sum of weights up to v) > floor(u * total)
__global__ __launch_bounds__(256) void spec_find_kernel(SampleArgs a) {
  const int b = blockIdx.x;
  const int pos = a.first_rej[b];
  __shared__ long long pre[257];
  __shared__ int sel_chunk, which_s;
  __shared__ long long target_s;
  if (threadIdx.x == 0) {
    int which = 0;
    long long S = 0;
    for (int c = 0; c < a.n_chunks; ++c) S += a.chunk_sum[((size_t)b * a.n_chunks + c) * 2];
    if (S <= 0) {  // empty residual (p == q): draw from p
      which = 1;
      S = 0;
      for (int c = 0; c < a.n_chunks; ++c) S += a.chunk_sum[((size_t)b * a.n_chunks + c) * 2 + 1];
    }
    const double u = a.u_smp[(size_t)b * (a.k + 1) + pos];
    long long target = (long long)(u * (double)S);
    if (target >= S) target = S - 1;
    if (target < 0) target = 0;
    long long run = 0;
    int c = 0;
    for (; c < a.n_chunks; ++c) {
      const long long cs = a.chunk_sum[((size_t)b * a.n_chunks + c) * 2 + which];
      if (run + cs > target) break;
      run += cs;
    }
    if (c >= a.n_chunks) c = a.n_chunks - 1;
    sel_chunk = c;
    which_s = which;
    target_s = target - run;
  }
  __syncthreads();
  const int c = sel_chunk, which = which_s;
  const long long target = target_s;
  const int v0 = c * a.chunk, v1 = min(a.V, v0 + a.chunk);
  // each thread owns a contiguous run of the chunk
  const int per = (a.chunk + 255) / 256;
  const int my0 = v0 + threadIdx.x * per, my1 = min(v1, my0 + per);
  long long mine = 0;
  for (int v = my0; v < my1; ++v) mine += qweight(a, b, pos, v, which);
  pre[threadIdx.x + 1] = mine;
  if (threadIdx.x == 0) pre[0] = 0;
  __syncthreads();
  if (threadIdx.x == 0)
    for (int i = 1; i <= 256; ++i) pre[i] += pre[i - 1];
  __syncthreads();
  // the thread whose run contains the crossing finds the index
  if (pre[threadIdx.x] <= target && pre[threadIdx.x + 1] > target) {
    long long run = pre[threadIdx.x];
    int tok = my1 - 1;
    for (int v = my0; v < my1; ++v) {
      run += qweight(a, b, pos, v, which);
      if (run > target) { tok = v; break; }
    }
    a.tok_out[b] = tok;
  }
  // no crossing inside the chunk can only come from an empty chunk selection
  if (threadIdx.x == 0 && pre[256] <= target) a.tok_out[b] = v1 - 1;
}

hipError_t launch_accept_sample(const SampleArgs& a, hipStream_t s) {
  const int rows = a.B * (2 * a.k + 1);
  spec_row_stats_kernel<<<rows, 256, 0, s>>>(a);
  spec_decide_kernel<<<(a.B + 63) / 64, 64, 0, s>>>(a);
  spec_chunk_sum_kernel<<<dim3(a.n_chunks, a.B), 256, 0, s>>>(a);
  spec_find_kernel<<<a.B, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace sdv
