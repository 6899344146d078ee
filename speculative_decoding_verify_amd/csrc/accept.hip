// Acceptance and cache-commit kernels.
//
// Greedy acceptance follows "Decode Before You Hear" (page 1), method step 4:
// n = min({i-1 : y~_i != argmax p_i} U {gamma}) plus the correction argmax
// p_{n+1}; with a runner-up branch (step 2) it becomes a walk down the draft tree.
// Speculative sampling follows "speculative-decoding-omni" (page 3), section 2:
// accept x with probability min(1, p(x)/q(x)), on the first rejection draw from
// norm(max(0, p - q)), otherwise a bonus draw from p.
#include <hip/hip_ext.h>

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

// Masked vocabulary entries (logit -inf) have probability 0.  While a thread has
// seen nothing but -inf its maximum is -inf and its sum 0; the exponent then takes
// 0 in place of the maximum so that the -inf terms add 0 instead of NaN.
SDV_DEV float safe_max(float m) { return m == -INFINITY ? 0.f : m; }

// one workgroup per logit row; each thread issues SR 16-byte loads before any
// arithmetic, so a wave keeps SR KB of the row in flight
static constexpr int SR = 8;

__global__ __launch_bounds__(256) void spec_row_stats_kernel(SampleArgs a) {
  const int row = blockIdx.x;
  const int nt = a.B * (a.k + 1);
  const float* z = row < nt ? a.tgt + (size_t)row * a.V : a.drf + (size_t)(row - nt) * a.V;
  const float c = LOG2E * a.inv_temp;
  float m = -INFINITY;
  double s = 0.0;
  // online max / sum over 16-byte loads when the row is aligned
  const bool vec = ((reinterpret_cast<uintptr_t>(z) & 15) == 0);
  const int nv = vec ? a.V / 4 : 0;
  const f32x4* zv = reinterpret_cast<const f32x4*>(z);
  int i = threadIdx.x;
  for (; i + (SR - 1) * 256 < nv; i += SR * 256) {
    f32x4 v[SR];
#pragma unroll
    for (int u = 0; u < SR; ++u) v[u] = __builtin_nontemporal_load(zv + i + u * 256);
    float vm = m;
#pragma unroll
    for (int u = 0; u < SR; ++u) vm = fmaxf(vm, fmaxf(fmaxf(v[u].x, v[u].y), fmaxf(v[u].z, v[u].w)));
    if (vm > m) { s = s * (double)exp2f((m - vm) * c); m = vm; }
    const float me = safe_max(m);
#pragma unroll
    for (int u = 0; u < SR; ++u)
      s += (double)(exp2f((v[u].x - me) * c) + exp2f((v[u].y - me) * c) + exp2f((v[u].z - me) * c) +
                    exp2f((v[u].w - me) * c));
  }
  for (; i < nv; i += 256) {
    const f32x4 v = __builtin_nontemporal_load(zv + i);
    const float vm = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
    if (vm > m) { s = s * (double)exp2f((m - vm) * c); m = vm; }
    const float me = safe_max(m);
    s += (double)(exp2f((v.x - me) * c) + exp2f((v.y - me) * c) + exp2f((v.z - me) * c) + exp2f((v.w - me) * c));
  }
  for (int j = nv * 4 + threadIdx.x; j < a.V; j += 256) {
    const float v = z[j];
    if (v > m) { s = s * (double)exp2f((m - v) * c); m = v; }
    s += (double)exp2f((v - safe_max(m)) * c);
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

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
// 1, 2, 3", SC'11): ten rounds of two 32x32 -> 64-bit products on the even counter
// words, the high halves xor-ed into the odd words together with the round key, and
// a Weyl increment of the key between rounds.
SDV_DEV uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t hi0 = __umulhi(0xD2511F53u, c.x), lo0 = 0xD2511F53u * c.x;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c.z), lo1 = 0xCD9E8D57u * c.z;
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// The two uniforms of (seq, pos) under key `seed`: counter (seq, pos, 0, stream).
// U0 = r0 * 2^-32 from stream 0 decides acceptance; U1 = (r1 * 2^21 + (r2 >> 11)) *
// 2^-53 from stream 1 drives the draw.
SDV_DEV double philox_u0(unsigned long long seed, uint32_t seq, uint32_t pos) {
  const uint4 r = philox4x32_10(make_uint4(seq, pos, 0u, 0u), (uint32_t)seed, (uint32_t)(seed >> 32));
  return (double)r.x * 0x1p-32;
}
SDV_DEV double philox_u1(unsigned long long seed, uint32_t seq, uint32_t pos) {
  const uint4 r = philox4x32_10(make_uint4(seq, pos, 0u, 1u), (uint32_t)seed, (uint32_t)(seed >> 32));
  return (double)(((unsigned long long)r.y << 21) + (r.z >> 11)) * 0x1p-53;
}

SDV_DEV uint32_t seq_of(const SampleArgs& a, int b) { return a.seq_ids ? (uint32_t)a.seq_ids[b] : (uint32_t)b; }

// Decision of sequence b: the position of its draw (the first draft position whose
// test fails, or k when every draft passes), whether a decision up to that position
// lies within FLAG_TOL of its threshold, and whether a draft id is outside [0, V).
// Called by the 64 lanes of one wave: lane i of each group of 64 positions evaluates
// position base + i, and the ballot keeps the lowest failing position.  A draft
// outside q's support (q(x) = 0) passes iff p(x) > 0.
struct Decision {
  int pos;
  bool near, bad;
};

static constexpr double FLAG_TOL = 1e-6;

SDV_DEV Decision decide(const SampleArgs& a, int b) {
  const int nt = a.B * (a.k + 1);
  const int lane = threadIdx.x & 63;
  const uint32_t seq = seq_of(a, b);
  bool bad = false;
  for (int base = 0; base < a.k; base += 64) {
    const int i = base + lane;
    const int x = i < a.k ? a.drafts[(size_t)b * a.k + i] : 0;
    bad |= __ballot(x < 0 || x >= a.V) != 0;
  }
  Decision d{a.k, false, bad};
  if (bad) return d;
  for (int base = 0; base < a.k; base += 64) {
    const int i = base + lane;
    bool rej = false, near = false;
    if (i < a.k) {
      const int x = a.drafts[(size_t)b * a.k + i];
      const int rt = b * (a.k + 1) + i, rd = nt + b * a.k + i;
      const double px = prob_at(a.tgt[(size_t)rt * a.V + x], a.row_m[rt], a.row_s[rt], a.inv_temp);
      const double qx = prob_at(a.drf[(size_t)(rd - nt) * a.V + x], a.row_m[rd], a.row_s[rd], a.inv_temp);
      const double u = philox_u0(a.seed, seq, (uint32_t)i);
      bool acc;
      if (qx > 0.0) {
        const double ratio = px / qx;
        acc = u < ratio;
        near = fabs(u - ratio) < FLAG_TOL;
      } else {
        acc = px > 0.0;
      }
      rej = !acc;
    }
    const unsigned long long mask = __ballot(rej), nmask = __ballot(near);
    if (mask) {
      const int first = __ffsll(mask) - 1;
      const unsigned long long upto = first == 63 ? ~0ull : ((2ull << first) - 1);
      d.pos = base + first;
      d.near |= (nmask & upto) != 0;
      return d;
    }
    d.near |= nmask != 0;
  }
  return d;
}

// The two rows a draw at position `pos` reads: p_pos, and q_pos at a rejection
// (pos < k); each with its maximum and 1/sum.
struct DrawRows {
  const float* zp;
  const float* zq;  // nullptr for the bonus draw (pos == k)
  float pm, qm, pinv, qinv, c;
};

SDV_DEV DrawRows draw_rows(const SampleArgs& a, int b, int pos) {
  const int nt = a.B * (a.k + 1);
  const int rt = b * (a.k + 1) + pos;
  DrawRows r;
  r.c = LOG2E * a.inv_temp;
  r.zp = a.tgt + (size_t)rt * a.V;
  r.pm = a.row_m[rt];
  r.pinv = (float)(1.0 / a.row_s[rt]);
  r.zq = nullptr;
  r.qm = 0.f;
  r.qinv = 0.f;
  if (pos < a.k) {
    const int rd = nt + b * a.k + pos;
    r.zq = a.drf + (size_t)(rd - nt) * a.V;
    r.qm = a.row_m[rd];
    r.qinv = (float)(1.0 / a.row_s[rd]);
  }
  return r;
}

// floor(w * 2^40) for w in [0, 1]: the quantised weight
SDV_DEV long long quantise(float w) { return (long long)((double)w * 1099511627776.0); }

// Quantised weights of one vocabulary entry from its two logits: w0 = max(0, p - q)
// at a rejection (p at the bonus position), w1 = p.  Contraction is off so that the
// sum pass and the search pass compute bit-identical weights.
SDV_DEV void pair_weights(const DrawRows& r, bool has_q, float zp, float zq, long long& w0, long long& w1) {
#pragma clang fp contract(off)
  const float p = exp2f((zp - r.pm) * r.c) * r.pinv;
  float w = p;
  if (has_q) {
    const float q = exp2f((zq - r.qm) * r.c) * r.qinv;
    w = fmaxf(0.f, p - q);
  }
  w0 = quantise(w);
  w1 = quantise(p);
}

// One workgroup per (chunk of the vocabulary, sequence): wave 0 takes the accept /
// reject decision of the sequence (the chunk-0 workgroup writes it out), then every
// thread sums the quantised weights of its share of the chunk for both draws.  A
// sequence with an invalid draft id sums nothing.
__global__ __launch_bounds__(256) void spec_chunk_sum_kernel(SampleArgs a) {
  const int b = blockIdx.y, ch = blockIdx.x;
  __shared__ int pos_s, bad_s;
  if (threadIdx.x < 64) {
    const Decision d = decide(a, b);
    if (threadIdx.x == 0) {
      pos_s = d.pos;
      bad_s = d.bad;
      if (ch == 0) {
        a.first_rej[b] = d.bad ? -1 : d.pos;
        a.seq_flags[b] = (d.near ? SAMPLE_FLAG_NEAR_ACCEPT : 0u) | (d.bad ? SAMPLE_FLAG_BAD_DRAFT : 0u);
        a.n_out[b] = d.bad ? -1 : d.pos;
      }
    }
  }
  __syncthreads();
  if (bad_s) {
    if (threadIdx.x == 0) {
      a.chunk_sum[((size_t)b * a.n_chunks + ch) * 2] = 0;
      a.chunk_sum[((size_t)b * a.n_chunks + ch) * 2 + 1] = 0;
    }
    return;
  }
  const int pos = pos_s;
  const DrawRows r = draw_rows(a, b, pos);
  const bool has_q = r.zq != nullptr;
  const float* zq = has_q ? r.zq : r.zp;
  const int v0 = ch * a.chunk, v1 = min(a.V, v0 + a.chunk);
  long long s0 = 0, s1 = 0;
  const bool vec = ((reinterpret_cast<uintptr_t>(r.zp + v0) | reinterpret_cast<uintptr_t>(zq + v0)) & 15) == 0;
  const int n4 = vec ? (v1 - v0) >> 2 : 0;
  const f32x4* p4 = reinterpret_cast<const f32x4*>(r.zp + v0);
  const f32x4* q4 = reinterpret_cast<const f32x4*>(zq + v0);
  for (int j0 = threadIdx.x; j0 < n4; j0 += 4 * 256) {
    f32x4 x[4], y[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = min(j0 + u * 256, n4 - 1);
      x[u] = p4[j];
      y[u] = q4[j];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (j0 + u * 256 < n4) {
        long long w0, w1;
        pair_weights(r, has_q, x[u].x, y[u].x, w0, w1); s0 += w0; s1 += w1;
        pair_weights(r, has_q, x[u].y, y[u].y, w0, w1); s0 += w0; s1 += w1;
        pair_weights(r, has_q, x[u].z, y[u].z, w0, w1); s0 += w0; s1 += w1;
        pair_weights(r, has_q, x[u].w, y[u].w, w0, w1); s0 += w0; s1 += w1;
      }
    }
  }
  for (int v = v0 + n4 * 4 + threadIdx.x; v < v1; v += 256) {
    long long w0, w1;
    pair_weights(r, has_q, r.zp[v], zq[v], w0, w1);
    s0 += w0;
    s1 += w1;
  }
  // integer sums: exact in any order
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    s0 += __shfl_xor(s0, o, 64);
    s1 += __shfl_xor(s1, o, 64);
  }
  __shared__ long long r0[4], r1[4];
  if ((threadIdx.x & 63) == 0) {
    r0[threadIdx.x >> 6] = s0;
    r1[threadIdx.x >> 6] = s1;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    a.chunk_sum[((size_t)b * a.n_chunks + ch) * 2] = r0[0] + r0[1] + r0[2] + r0[3];
    a.chunk_sum[((size_t)b * a.n_chunks + ch) * 2 + 1] = r1[0] + r1[1] + r1[2] + r1[3];
  }
}

// Inclusive prefix sum of one value per thread over the 256 threads: a shuffle scan
// inside each wave, then the totals of the lower waves (through `wtot`, 4 entries
// that no other call uses).  Also returns the block total.
SDV_DEV long long block_scan(long long v, long long* wtot, long long& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const long long t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  if (lane == 63) wtot[w] = v;
  __syncthreads();
  long long below = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const long long t = wtot[i];
    below += i < w ? t : 0;
    total += t;
  }
  return v + below;
}

// Inverse CDF of sequence b's draw: the smallest index v whose running sum of
// quantised weights exceeds floor(u * total).  The draw takes the residual weights;
// when they are all zero (p == q on this position) it takes p.  Threads own
// contiguous runs, first of chunks (their sums from the previous kernel), then of
// the selected chunk's entries (weights staged in LDS by coalesced loads); a prefix
// scan finds the run that holds the crossing and its thread walks it.
__global__ __launch_bounds__(256) void spec_find_kernel(SampleArgs a) {
  constexpr int PER = SAMPLE_CHUNK / 256;
  static_assert((PER & (PER - 1)) == 0, "entries per thread must be a power of two");
  const int b = blockIdx.x;
  __shared__ long long wts[SAMPLE_CHUNK];
  __shared__ long long wtot[3][4];
  __shared__ int sel_s;
  __shared__ long long rem_s;
  const int pos = a.first_rej[b];
  if (pos < 0) {  // invalid draft id: no draw
    if (threadIdx.x == 0) {
      a.tok_out[b] = -1;
      if (a.flags_out) a.flags_out[b] = a.seq_flags[b];
    }
    return;
  }
  const long long* cs = a.chunk_sum + (size_t)b * a.n_chunks * 2;
  const int cper = (a.n_chunks + 255) / 256;
  const int c0 = min(a.n_chunks, (int)threadIdx.x * cper), c1 = min(a.n_chunks, c0 + cper);
  long long t0 = 0, t1 = 0;
  for (int c = c0; c < c1; ++c) {
    t0 += cs[2 * c];
    t1 += cs[2 * c + 1];
  }
  long long S0, S1;
  const long long inc0 = block_scan(t0, wtot[0], S0);
  const long long inc1 = block_scan(t1, wtot[1], S1);
  const int which = S0 > 0 ? 0 : 1;
  const long long S = which == 0 ? S0 : S1;
  const double u = philox_u1(a.seed, seq_of(a, b), (uint32_t)pos);
  long long target = (long long)(u * (double)S);
  if (target >= S) target = S - 1;
  if (target < 0) target = 0;
  // the chunk holding the crossing (the last chunk when the total is zero)
  if (threadIdx.x == 0) {
    sel_s = a.n_chunks - 1;
    rem_s = 0;
  }
  __syncthreads();
  {
    const long long inc = which == 0 ? inc0 : inc1;
    long long run = inc - (which == 0 ? t0 : t1);
    if (run <= target && inc > target) {
      for (int c = c0; c < c1; ++c) {
        const long long w = cs[2 * c + which];
        if (run + w > target) {
          sel_s = c;
          rem_s = target - run;
          break;
        }
        run += w;
      }
    }
  }
  __syncthreads();
  const int c = sel_s;
  const long long rem = rem_s;
  const int v0 = c * SAMPLE_CHUNK, n = min(a.V - v0, SAMPLE_CHUNK);
  const DrawRows r = draw_rows(a, b, pos);
  const bool has_q = r.zq != nullptr;
  const float* zp = r.zp + v0;
  const float* zq = (has_q ? r.zq : r.zp) + v0;
  // stage the chosen weights of the chunk: entry j = threadIdx.x + 256 u
  {
    float xp[PER], xq[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int j = min((int)threadIdx.x + 256 * u, n - 1);
      xp[u] = zp[j];
      xq[u] = zq[j];
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int j = threadIdx.x + 256 * u;
      long long w0, w1;
      pair_weights(r, has_q, xp[u], xq[u], w0, w1);
      wts[j] = j < n ? (which == 0 ? w0 : w1) : 0;
    }
  }
  __syncthreads();
  // thread t owns entries t*PER .. t*PER + PER - 1
  const long long* mw = wts + threadIdx.x * PER;
  long long mine = 0;  // summed in a lane-rotated order (fewer LDS bank conflicts; exact)
#pragma unroll
  for (int i = 0; i < PER; ++i) mine += mw[(i + threadIdx.x) & (PER - 1)];
  long long total;
  const long long inc = block_scan(mine, wtot[2], total);
  long long run = inc - mine;
  // a draw whose target lies within FLAG_TOL (in probability units, 2^40 per unit) of a
  // partial sum is flagged: the partial sums are monotone, so the nearest ones are the
  // two around the crossing entry
  constexpr long long TOL_Q = (long long)(FLAG_TOL * 1099511627776.0);
  if (run <= rem && inc > rem) {
    int j = PER - 1;
    long long before = run, after = inc;
    for (int i = 0; i < PER; ++i) {
      if (run + mw[i] > rem) {
        j = i;
        before = run;
        after = run + mw[i];
        break;
      }
      run += mw[i];
    }
    a.tok_out[b] = v0 + threadIdx.x * PER + j;
    const bool near = rem - before < TOL_Q || after - rem < TOL_Q;
    if (a.flags_out) a.flags_out[b] = a.seq_flags[b] | (near ? SAMPLE_FLAG_NEAR_DRAW : 0u);
  }
  // no crossing inside the chunk: only when the total weight is zero (invalid rows)
  if (threadIdx.x == 0 && total <= rem) {
    a.tok_out[b] = v0 + n - 1;
    if (a.flags_out) a.flags_out[b] = a.seq_flags[b] | SAMPLE_FLAG_NEAR_DRAW;
  }
}

// The uniforms themselves, for callers that draw elsewhere and for tests.
__global__ __launch_bounds__(256) void philox_uniforms_kernel(PhiloxArgs a) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)a.B * a.n_pos) return;
  const int b = (int)(i / a.n_pos), pos = (int)(i % a.n_pos);
  const uint32_t seq = a.seq_ids ? (uint32_t)a.seq_ids[b] : (uint32_t)b;
  if (a.u0) a.u0[i] = philox_u0(a.seed, seq, (uint32_t)pos);
  if (a.u1) a.u1[i] = philox_u1(a.seed, seq, (uint32_t)pos);
}

hipError_t launch_philox_uniforms(const PhiloxArgs& a, hipStream_t s) {
  const long long n = (long long)a.B * a.n_pos;
  philox_uniforms_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_accept_sample(const SampleArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  const int rows = a.B * (2 * a.k + 1);
  if (ev0) hipExtLaunchKernelGGL(spec_row_stats_kernel, dim3(rows), dim3(256), 0, s, ev0, ev1, 0, a);
  else spec_row_stats_kernel<<<rows, 256, 0, s>>>(a);
  spec_chunk_sum_kernel<<<dim3(a.n_chunks, a.B), 256, 0, s>>>(a);
  spec_find_kernel<<<a.B, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace sdv
