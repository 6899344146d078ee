// Drafting in the idle window ("Decode Before You Hear", page 1, method steps 1 and 2;
// the top-k first-token tree of its weaknesses and future-directions sections).
//
// With the cache at x_{<t} and a hypothesised chunk (silence), branch k of a draft tree
// starts from the (k+1)-th ranked token of p_1 = p(. | x_{<t}, a_sil) (branch 0 is the
// greedy draft, branch 1 the runner-up argmax over V \ {y~_1}) and continues greedily.
// The host enqueues one verify forward per draft position; these kernels rank the
// first tokens and move each step's argmax into the draft buffer and the next step's
// chunk, so the drafted tokens never leave the device.
#include "common.h"
#include "kernels.h"

namespace sdv {

// (value, index) pairs in the order of a draft ranking: larger value first, lower
// index first among equal values.
SDV_DEV bool ranks_before(float v, int i, float w, int j) { return v > w || (v == w && i < j); }

// Top-K of every logit row: round k takes the best entry that ranks after the pick of
// round k - 1, so each round is one pass over the row and a block reduction.  One
// workgroup per row; the picks go to drafts[b][k][0] (k < K).
__global__ __launch_bounds__(256) void draft_topk_kernel(DraftTopkArgs a) {
  const int b = blockIdx.x;
  const float* z = a.logits + (size_t)b * a.V;
  __shared__ float sv[256];
  __shared__ int si[256];
  __shared__ float prev_v;
  __shared__ int prev_i;
  if (threadIdx.x == 0) {
    prev_v = INFINITY;
    prev_i = -1;
  }
  __syncthreads();
  for (int k = 0; k < a.K; ++k) {
    const float pv = prev_v;
    const int pi = prev_i;
    float bv = -INFINITY;
    int bi = -1;
    for (int i = threadIdx.x; i < a.V; i += 256) {
      const float v = z[i];
      if (ranks_before(pv, pi, v, i) && (bi < 0 || ranks_before(v, i, bv, bi))) {
        bv = v;
        bi = i;
      }
    }
    sv[threadIdx.x] = bv;
    si[threadIdx.x] = bi;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if (threadIdx.x < o) {
        const float v = sv[threadIdx.x + o];
        const int i = si[threadIdx.x + o];
        if (i >= 0 && (si[threadIdx.x] < 0 || ranks_before(v, i, sv[threadIdx.x], si[threadIdx.x]))) {
          sv[threadIdx.x] = v;
          si[threadIdx.x] = i;
        }
      }
      __syncthreads();
    }
    if (threadIdx.x == 0) {
      a.drafts[((size_t)b * a.K + k) * a.max_len] = si[0];
      prev_v = sv[0];
      prev_i = si[0];
    }
    __syncthreads();
  }
}

hipError_t launch_draft_topk(const DraftTopkArgs& a, hipStream_t s) {
  draft_topk_kernel<<<a.B, 256, 0, s>>>(a);
  return hipGetLastError();
}

// One drafting step's bookkeeping, one workgroup per sequence:
//   save   (first call) remember the committed length, clear the draft buffer and set
//          the first pass's logit row;
//   keep   keep_out[b] = saved[b] + keep_delta (the rollback target of the next call);
//   scatter drafts[b][prev_branch[r]][prev_pos] = argmax[b][r] for the n_prev branches
//          of the step that just ran;
//   build  the next chunk: row 0 is the root token, then for each of the n_act active
//          branches its first s tokens (drafted positions 0..s-1) as a chain under the
//          root; its last row is a logit row.
__global__ __launch_bounds__(128) void draft_step_kernel(DraftStepArgs a) {
  const int b = blockIdx.x;
  int32_t* dr = a.drafts + (size_t)b * a.K * a.max_len;
  if (a.save) {
    if (threadIdx.x == 0) a.saved[b] = a.seq_len[b];
    if (b == 0 && threadIdx.x == 0) a.logit_rows[0] = a.first_row;
    for (int i = threadIdx.x; i < a.K * a.max_len; i += blockDim.x) dr[i] = -1;
  }
  if (a.keep_out && threadIdx.x == 0) a.keep_out[b] = (a.save ? a.seq_len[b] : a.saved[b]) + a.keep_delta;
  if (threadIdx.x < a.n_prev) dr[a.prev_branch[threadIdx.x] * a.max_len + a.prev_pos] =
      a.argmax[(size_t)b * a.n_prev + threadIdx.x];
  __syncthreads();
  if (a.n_act == 0) return;
  const int T = 1 + a.n_act * a.s;
  for (int j = threadIdx.x; j < T; j += blockDim.x) {
    int tok, par;
    if (j == 0) {
      tok = a.root[(size_t)b * a.root_stride];
      par = -1;
    } else {
      const int r = (j - 1) / a.s, i = (j - 1) % a.s;
      tok = dr[a.act_branch[r] * a.max_len + i];
      par = i == 0 ? 0 : j - 1;
    }
    a.tokens[(size_t)b * T + j] = tok;
    if (b == 0) a.parent[j] = par;
  }
  if (b == 0 && threadIdx.x < a.n_act) a.logit_rows[threadIdx.x] = a.s * (threadIdx.x + 1);
}

hipError_t launch_draft_step(const DraftStepArgs& a, hipStream_t s) {
  draft_step_kernel<<<a.B, 128, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace sdv
