/*
 * sdv.h -- C ABI of the single-forward speculative verification library (libsdv.so).
 *
 * The operations follow the problem statement of "Decode Before You Hear:
 * Speculative Listening for Chunk-Interleaved Full-Duplex Speech Language
 * Models" (page 1, section "Method steps", steps 4 and 6) and the acceptance
 * rule of "speculative-decoding-omni" (page 3, section 2):
 *
 *   sdv_verify_forward  one decoder forward over [audio chunk ; draft (; runner-up
 *                       branch)] on top of a paged KV cache, yielding every draft
 *                       position's target distribution as logits plus fused
 *                       argmax / top-2 margin / log-sum-exp (step 4);
 *   sdv_accept_greedy   n = min({i-1 : y~_i != argmax p_i} U {gamma}) and the
 *                       correction argmax p_{n+1}, generalised to a tree walk (step 4);
 *   sdv_accept_sample   speculative-sampling acceptance: accept x_i with probability
 *                       min(1, p/q), resample the first rejection from
 *                       norm(max(0, p - q)), bonus token from p when all pass
 *                       (step 6; page 3 section 2);
 *   sdv_kv_rollback     set committed lengths and compact an accepted branch
 *                       ("roll the KV cache back", step 4);
 *   sdv_pack_weights    one-time rearrangement of row-major weight matrices into
 *                       the packed tile layout the verify forward streams.
 *
 * Conventions shared by every call
 *   - All data pointers are DEVICE pointers unless a comment says "host".
 *   - The caller owns every buffer (weights, cache pages, inputs, outputs and the
 *     workspace).  The library never allocates or frees device memory, never
 *     synchronises the stream and keeps no state between calls.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and is
 *     asynchronous: outputs are valid once the stream reaches that point.
 *   - Host-checkable problems (NULL pointer, unsupported shape, workspace too small)
 *     return a negative sdv_status before anything is enqueued; sdv_last_error()
 *     then returns a message (thread-local, valid until the next call on the thread).
 *   - Data-dependent problems found on the device (token id outside [0, V), a tree
 *     parent that is not an earlier row, a cache that would overflow its capacity)
 *     set bits in the caller's int32 error word for that sequence; that sequence's
 *     results are then unspecified, other sequences are unaffected, and the kernels
 *     never read or write outside their buffers.
 *   - Storage type of weights, embedding and KV pages: fp32 (SDV_F32) or bf16
 *     (SDV_BF16, raw 16-bit patterns); norm gains are always fp32.  The embedding is
 *     row-major [V, d]; the projection matrices and the LM head are PACKED (below).
 *
 * Packed weights
 *   A matrix with rows n (output features) and columns k (input features, K of
 *   them) is stored as 1 KB tiles of 16 rows x KS columns, KS = 32 (bf16) or 16
 *   (fp32).  Tile (n / 16, k / KS) starts at byte ((n / 16) * (K / KS) + k / KS) * 1024;
 *   inside it, the 16 bytes holding row n % 16 and columns of k group
 *   g = (k % KS) / (KS / 4) start at byte (g * 16 + n % 16) * 16.  Rows past the
 *   sources are zero (the row count is rounded up to a multiple of 16).  Which source
 *   row becomes packed row n depends on the kind:
 *     SDV_PACK_PLAIN    row n of the one source;
 *     SDV_PACK_QKV      sources Wq [H*dh, d], Wk [Hkv*dh, d], Wv [Hkv*dh, d] viewed
 *                       as one matrix of whole heads; rotation pair p (head p / (dh/2),
 *                       element i = p % (dh/2), paired with i + dh/2) gives packed row
 *                       16 * (p / 8) + p % 8 to element i and 16 * (p / 8) + 8 + p % 8
 *                       to element i + dh/2 (v heads are paired the same way);
 *     SDV_PACK_GATE_UP  sources Wg [F, d], Wu [F, d]: packed row 16 * (f / 8) + f % 8
 *                       is gate row f, 16 * (f / 8) + 8 + f % 8 is up row f.
 *   sdv_pack_weights writes this layout on the device; sdv_packed_bytes gives its size.
 */
#ifndef SDV_H
#define SDV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SDV_ABI_VERSION 9   /* 9: multi-codebook streams (sdv_phase_mask, sdv_stream_commit) */
#define SDV_PAGE 16          /* tokens per KV-cache page */
#define SDV_MAX_T 128        /* rows per verify pass (chunk + drafts + branches) */
#define SDV_SAMPLE_MAX_K 1024  /* draft positions per sequence of sdv_accept_sample */

typedef enum {
  SDV_OK = 0,
  SDV_ERR_NULL = -1,        /* a required pointer is NULL */
  SDV_ERR_SHAPE = -2,       /* inconsistent or out-of-range sizes */
  SDV_ERR_UNSUPPORTED = -3, /* valid but not implemented (e.g. head_dim not 64/128) */
  SDV_ERR_WORKSPACE = -4,   /* workspace smaller than sdv_*_workspace_size() */
  SDV_ERR_LAUNCH = -5       /* the HIP runtime rejected a launch */
} sdv_status;

typedef enum { SDV_F32 = 0, SDV_BF16 = 1 } sdv_dtype;

typedef enum { SDV_PACK_PLAIN = 0, SDV_PACK_QKV = 1, SDV_PACK_GATE_UP = 2 } sdv_pack_kind;

/* Which head produces the next-token distributions of a verify pass. */
typedef enum { SDV_HEAD_LM = 0, SDV_HEAD_CODEBOOK = 1 } sdv_head;

/* device-side error bits written to the per-sequence error word */
#define SDV_EBAD_TOKEN    0x1   /* a token id outside [0, vocab) (treated as 0) */
#define SDV_EBAD_PARENT   0x2   /* parent[j] not in [0, j) for j > 0, or parent[0] != -1 */
#define SDV_EOVERFLOW     0x4   /* seq_len + T exceeds the cache capacity or max_ctx + T */
#define SDV_EBAD_MOVE     0x8   /* a rollback move or keep_len outside the capacity */
#define SDV_EDUP_SIBLING  0x10  /* two children of one tree row carry the same token */
#define SDV_EBAD_PAIR     0x20  /* cfg_partner[b] out of range or not mutual (row uses its own logits) */

/* One decoder layer: pre-norm attention block and SwiGLU FFN block.  Matrices are
 * packed (see above); the shapes given are those of the row-major sources. */
typedef struct {
  const float* attn_norm;  /* [d] RMSNorm gain before attention */
  const void* wqkv;        /* SDV_PACK_QKV of Wq [H*dh, d], Wk, Wv [Hkv*dh, d] */
  const void* wo;          /* SDV_PACK_PLAIN of Wo [d, H*dh] */
  const float* ffn_norm;   /* [d] RMSNorm gain before the FFN */
  const void* wgu;         /* SDV_PACK_GATE_UP of Wg, Wu [F, d] */
  const void* wd;          /* SDV_PACK_PLAIN of Wd [d, F] */
} sdv_layer;

/* Decoder: token embedding, n_layers pre-norm blocks, final RMSNorm, untied LM head.
 * Attention: query head h reads kv head h / (H / Hkv); scale 1/sqrt(dh); rotary
 * embedding of rotate-half form (element i pairs with i + dh/2, angle
 * pos * rope_theta^(-2i/dh)) on queries and keys. */
typedef struct {
  int32_t n_layers, d, n_heads, n_kv_heads, head_dim, ffn, vocab;
  int32_t dtype;             /* sdv_dtype of every matrix, the embedding and the KV pages */
  float eps;                 /* RMSNorm epsilon: x / sqrt(mean(x^2) + eps) * g */
  float rope_theta;
  const void* embed;         /* [V, d] row-major */
  const float* final_norm;   /* [d] */
  const void* lm_head;       /* SDV_PACK_PLAIN of W_lm [V, d] */
  const sdv_layer* layers;   /* HOST array of n_layers entries (device pointers inside) */
  /* Codebook heads ("An Efficient vLLM-Based Inference Pipeline for Unified Audio
   * Understanding and Generation", page 2, Figure 1): S audio streams of Vc codes;
   * stream s scores codes with W_cb (RMSNorm(h; final_norm) + e_s), W_cb shared by all
   * streams.  Code c of codebook 0 is backbone token codebook_base + c.  Zero / NULL
   * when the model has no codebook heads. */
  int32_t n_codebooks;       /* S */
  int32_t codebook_size;     /* Vc */
  int32_t codebook_base;     /* backbone id of code 0 of codebook 0 */
  const void* codebook;      /* SDV_PACK_PLAIN of W_cb [Vc, d] */
  const float* stream_emb;   /* [S, d] fp32 stream embeddings e_s */
} sdv_model;

/* Paged KV cache.  Logical slot s of sequence b lives in physical page
 * block_table[b * max_blocks + s / 16] at offset s % 16.
 *   k_pages: [n_layers][n_blocks][Hkv][16][dh]   (token-major within a page)
 *   v_pages: [n_layers][n_blocks][Hkv][dh][16]   (transposed within a page)
 * seq_len[b] is the committed length C_b; capacity is max_blocks * 16 slots. */
typedef struct {
  void* k_pages;
  void* v_pages;
  const int32_t* block_table;  /* [B, max_blocks] */
  int32_t* seq_len;            /* [B] */
  int32_t n_blocks;            /* physical pages per layer */
  int32_t max_blocks;          /* table entries per sequence */
  int32_t batch;               /* B */
} sdv_kv;

/* One verify pass over T chunk rows per sequence.
 *   tokens   [B, T]: rows 0..L_a-1 are the audio chunk, later rows are drafts.
 *   parent   [T] tree parents shared by all sequences (parent[0] = -1, parent[j] in
 *            [0, j)), or NULL for a chain (parent[j] = j - 1).  Row j is written to
 *            slot seq_len[b] + j and takes rotary position seq_len[b] + depth(j); it
 *            attends to all seq_len[b] cached slots and to the chunk rows that are j
 *            or its ancestors.
 *   logit_rows [R] chunk rows whose next-token distributions are produced (for
 *            greedy acceptance: L_a-1 and every draft row).
 *   max_ctx  host-side upper bound on every seq_len[b]; sizes the attention grid.
 *   head     SDV_HEAD_LM: logits over the full vocabulary from the LM head;
 *            SDV_HEAD_CODEBOOK: per-codebook logits from the codebook heads, and the
 *            statistics and argmax of codebook 0 (as backbone ids) for acceptance.
 *   cfg_partner [B] device, nullable (codebook head only): classifier-free guidance
 *            pairs ("paired scheduling", page 2).  For rows b and p = cfg_partner[b]
 *            with cfg_partner[p] == b, the lower index is the conditional row c, the
 *            other the unconditional row u, and BOTH rows get the guided logits
 *            u + cfg_w (c - u) of every codebook, so they accept the same tokens (the
 *            caller feeds both rows the same tokens).  -1 = no guidance for row b. */
typedef struct {
  int32_t batch, T, L_a, R, max_ctx;
  const int32_t* tokens;
  const int32_t* parent;       /* nullable */
  const int32_t* logit_rows;
  int32_t head;                /* sdv_head */
  const int32_t* cfg_partner;  /* nullable */
  float cfg_w;
} sdv_verify_in;

/* Outputs of sdv_verify_forward (all device, [B, R] unless noted):
 *   logits  fp32 [B, R, V] or NULL (the statistics below are produced either way);
 *           codebook head: fp32 [B, R, S, Vc] (guided for rows of a pair)
 *   argmax  int32: index of the largest logit, lowest index on ties; codebook head:
 *           codebook_base + the argmax code of codebook 0 (margin and lse likewise
 *           describe codebook 0)
 *   margin  fp32: largest minus second-largest logit (0 on a tie)
 *   lse     fp32: log(sum_v exp(logit_v))
 *   hidden  fp32 [B, T, d] or NULL: residual stream after the last layer
 *   err     int32 [B]: device error bits (OR-ed in; the caller clears it)
 *   cb_argmax  see the field
 *   prof_events  nullable host array of n_prof_events caller-created hipEvent_t
 *           handles: when given, the i-th projection of the pass (decoder
 *           projections in order q/k/v, o, gate/up, down per layer, then the LM head)
 *           records event 2i when its GEMM kernel starts and event 2i+1 when its last
 *           kernel ends (the GEMM, or the kernel that sums its K-split partials and
 *           applies the epilogue when it has one), both recorded by the dispatches
 *           themselves (hipExtLaunchKernel), for as many projections as there are
 *           event pairs.
 *   attn_prof_events  nullable host array of n_attn_prof_events caller-created events:
 *           layer l's attention records event 2l when its kernel starts and event
 *           2l + 1 when the last kernel of that layer's attention (the split merge, when
 *           it runs as a kernel of its own) ends, for the layers that have a pair. */
typedef struct {
  float* logits;
  int32_t* argmax;
  float* margin;
  float* lse;
  float* hidden;
  int32_t* err;
  void* const* prof_events;
  int32_t n_prof_events;
  int32_t* cb_argmax;          /* codebook head: int32 [B, R, S] argmax code per codebook, nullable */
  void* const* attn_prof_events;
  int32_t n_attn_prof_events;
} sdv_verify_out;

/* Bytes of workspace sdv_verify_forward needs for this model and pass shape. */
size_t sdv_verify_workspace_size(const sdv_model* m, int32_t batch, int32_t T, int32_t R,
                                 int32_t max_ctx);

/* The verify forward ("Method steps", step 4).  Writes K/V of the T rows into the
 * cache pages at slots seq_len[b] + j; does NOT change seq_len (commit with
 * sdv_kv_rollback).  Requires head_dim 64 or 128, H % Hkv == 0, d and F multiples
 * of 64, d <= 8192, 1 <= T <= SDV_MAX_T, 1 <= R <= T. */
sdv_status sdv_verify_forward(const sdv_model* m, const sdv_kv* kv, const sdv_verify_in* in,
                              sdv_verify_out* out, void* workspace, size_t workspace_bytes,
                              void* stream);

/* The verify forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, results and effects as sdv_verify_forward; the
 * workspace is a static device array of SDV_NOALLOC_MAX_WORKSPACE bytes inside the
 * library (one per GPU, held until the process ends).  A pass whose
 * sdv_verify_workspace_size exceeds that returns SDV_ERR_WORKSPACE before anything is
 * enqueued.  Calls on one GPU share the array: calls that overlap on one GPU (other
 * streams, other threads) race and must be serialised by the caller.  Allocates and
 * frees nothing. */
#define SDV_NOALLOC_MAX_WORKSPACE (64u << 20)
sdv_status sdv_verify_forward_noalloc(const sdv_model* m, const sdv_kv* kv, const sdv_verify_in* in,
                                      sdv_verify_out* out, void* stream);

/* Greedy acceptance ("Method steps", step 4) for every sequence b.
 *   Walk from row L_a-1; at each row, the child row whose token equals that row's
 *   argmax is accepted and the walk continues from it; stop when no child matches.
 *   On a chain this is n = min({i-1 : y~_i != argmax p_i} U {gamma}).
 *   argmax   [B, R] from sdv_verify_forward, aligned with logit_rows (every row on a
 *            walk must be in logit_rows, otherwise the walk stops there).
 *   n_out    [B] accepted draft rows (0 <= n <= depth of the tree)
 *   next_out [B] the correction (or bonus) token argmax at the last accepted row
 *   path_out [B, T] accepted rows in order, -1 padded (nullable)
 *   base_len [B] nullable; when given (normally kv->seq_len) the commit plan is
 *            also written: keep_out[b] = base_len[b] + L_a + n, and for i < T
 *            move_src/move_dst [B, T] = slots to copy so that accepted row i ends at
 *            slot base + L_a + i (-1 where no copy is needed).
 *   err      [B] device error bits (duplicate sibling tokens), nullable. */
sdv_status sdv_accept_greedy(int32_t batch, int32_t T, int32_t L_a, const int32_t* tokens,
                             const int32_t* parent, int32_t R, const int32_t* logit_rows,
                             const int32_t* argmax, const int32_t* base_len,
                             int32_t* n_out, int32_t* next_out, int32_t* path_out,
                             int32_t* keep_out, int32_t* move_src, int32_t* move_dst,
                             int32_t* err, void* stream);

/* Speculative-sampling acceptance ("Method steps", step 6; page 3, section 2).
 *   tgt_logits [B, k+1, V] fp32 target logits (row i scores draft position i, row k
 *              the bonus position); drf_logits [B, k, V] fp32 draft logits;
 *   drafts [B, k]; p = softmax(tgt / temperature), q = softmax(drf / temperature).
 *   Random numbers: Philox4x32-10 (Salmon et al., SC'11) under the 64-bit key `seed`
 *   (low word first), counter (s, i, 0, stream) with s = seq_ids[b] (seq_ids NULL:
 *   s = b) and i the 0-based position; U0(s, i) = r0 * 2^-32 from stream 0,
 *   U1(s, i) = (r1 * 2^21 + (r2 >> 11)) * 2^-53 from stream 1 (sdv_philox_uniforms
 *   writes the same numbers).
 *   For i = 0..k-1 in order: accept drafts[b,i] iff U0(s, i) < p(x)/q(x) (if q(x) = 0:
 *   iff p(x) > 0).  At the first rejection i: token = inverse CDF of w = max(0, p_i - q_i)
 *   (of p_i if w is empty) at U1(s, i), n = i.  If all pass: n = k, token = inverse CDF
 *   of p_k at U1(s, k).  The inverse CDF returns the smallest index whose running sum
 *   exceeds u * total, with weights quantised to 2^-40 so the draw does not depend on
 *   summation order.
 *   Logits of -inf (masked vocabulary entries) have probability 0; every row needs at
 *   least one finite logit.
 *   Outputs n_out [B], tok_out [B] (int32); flags_out [B] (nullable) per sequence:
 *     SDV_SAMPLE_NEAR_ACCEPT  an acceptance test up to the draw position had
 *                             |U0 - p(x)/q(x)| < 1e-6 (another rounding could decide
 *                             it the other way);
 *     SDV_SAMPLE_NEAR_DRAW    the draw's target u * total lies within 1e-6 (probability
 *                             units) of a partial sum;
 *     SDV_SAMPLE_BAD_DRAFT    a draft id outside [0, V): n_out and tok_out are -1.
 *   k <= SDV_SAMPLE_MAX_K; temperature finite and > 0.
 *   prof_events: nullable host array of 2 caller-created hipEvent_t handles; when
 *   given, the launch that reads every logit row (maximum and exponential sum per
 *   row) records event 0 when it starts and event 1 when it ends. */
#define SDV_SAMPLE_NEAR_ACCEPT 0x1
#define SDV_SAMPLE_NEAR_DRAW   0x2
#define SDV_SAMPLE_BAD_DRAFT   0x100
size_t sdv_sample_workspace_size(int32_t batch, int32_t k, int32_t vocab);
sdv_status sdv_accept_sample(int32_t batch, int32_t k, int32_t vocab, const float* tgt_logits,
                             const float* drf_logits, const int32_t* drafts, float temperature,
                             uint64_t seed, const int32_t* seq_ids, int32_t* n_out, int32_t* tok_out,
                             uint32_t* flags_out, void* workspace, size_t workspace_bytes,
                             void* const* prof_events, void* stream);

/* The Philox4x32-10 uniforms sdv_accept_sample uses, written out: for b < B and
 * pos < n_pos, u0_out[b, pos] = U0(s, pos) and u1_out[b, pos] = U1(s, pos) (both
 * [B, n_pos] fp64, either nullable), s = seq_ids[b] or b. */
sdv_status sdv_philox_uniforms(uint64_t seed, const int32_t* seq_ids, int32_t batch, int32_t n_pos,
                               double* u0_out, double* u1_out, void* stream);

/* Drafting in the idle window ("Method steps", steps 1 and 2; the top-k first-token
 * tree of page 1's weaknesses and future directions).  With the cache of every
 * sequence at its committed length C_b (seq_len), the hypothesised chunk
 * chunk [B, L_a] (e.g. L_a silence tokens) is run once; from its last row's
 * distribution p_1, branch k (k < n_branches) starts with the (k+1)-th ranked token
 * (larger logit first, lower index on ties: branch 0 is the greedy draft, branch 1 the
 * runner-up argmax over V minus the greedy token) and is continued greedily to
 * branch_len[k] tokens: token i+1 = argmax p(. | x_{<t}, chunk, branch tokens 0..i),
 * lowest index on ties.  Every draft position of all branches is one verify forward
 * (the branches as a tree under the chunk's last row), enqueued on `stream` without
 * a host round trip.
 *   branch_len  HOST [n_branches], each in [1, SDV_MAX_T]; 1 <= n_branches <= 16;
 *               1 + s * (branches longer than s) <= SDV_MAX_T for every s.
 *   drafts      [B, n_branches, max_k branch_len] int32 out, -1 past a branch's end.
 *   err         [B] device error bits (as sdv_verify_forward; OR-ed in).
 * The drafting rows' K/V are written to slots C_b.. and discarded: seq_len is back at
 * C_b when the call's work completes.  max_ctx bounds every C_b;
 * max_ctx + L_a - 1 + (rows of the widest pass) must fit the cache. */
typedef struct {
  int32_t batch, L_a, n_branches, max_ctx;
  const int32_t* chunk;        /* [B, L_a] device */
  const int32_t* branch_len;   /* HOST [n_branches] */
} sdv_draft_in;
size_t sdv_draft_workspace_size(const sdv_model* m, int32_t batch, int32_t L_a, int32_t n_branches,
                                const int32_t* branch_len, int32_t max_ctx);
sdv_status sdv_draft_tree(const sdv_model* m, const sdv_kv* kv, const sdv_draft_in* in, int32_t* drafts,
                          int32_t* err, void* workspace, size_t workspace_bytes, void* stream);

/* Hypothesis pool ("Method steps", steps 3 and 5): every draft of a session is stored
 * and indexed by its n-grams (n = 1..max_n); after a verify pass, the longest n-gram at
 * the end of the output found in the pool gives the continuation the next pass
 * verifies.  The caller owns the arrays (device):
 *   tokens, seg_end  [capacity] int32: stored draft tokens in insertion order, and for
 *                    each the end position (exclusive) of its draft;
 *   keys [n_slots] uint64, vals [n_slots] int32: the hash index (n_slots a power of two,
 *                    at least about twice the n-grams stored; sdv_pool_clear empties it);
 *   count [1] int32: tokens stored.
 * An indexed n-gram is one followed by at least one token of its own draft; its entry
 * holds the position after its most recent occurrence (later drafts, and later
 * positions inside a draft, win).  Keys are 64-bit hashes of (n, tokens); a lookup
 * also compares the stored tokens, so a hash collision can only lose a match
 * (probability about (n-grams)^2 / 2^64), never return a wrong one. */
#define SDV_POOL_MAX_N 16
#define SDV_POOL_EFULL_STORE 0x1   /* err bit: storage full, the draft was not stored */
#define SDV_POOL_EFULL_INDEX 0x2   /* err bit: hash table full, some n-gram not indexed */
typedef struct {
  int32_t* tokens;
  int32_t* seg_end;
  uint64_t* keys;
  int32_t* vals;
  int32_t* count;
  int32_t capacity, n_slots, max_n;
} sdv_pool;

/* Empty the pool (count = 0, every slot free). */
sdv_status sdv_pool_clear(const sdv_pool* pool, void* stream);

/* Append one draft (device [len] int32) and index its n-grams.  err: [1] device error
 * bits (SDV_POOL_EFULL_*), nullable. */
sdv_status sdv_pool_insert(const sdv_pool* pool, const int32_t* draft, int32_t len, int32_t* err,
                           void* stream);

/* For each query q < batch: the output suffix suffix[q, 0..suffix_len[q]-1] (device
 * [batch, suffix_cap], lengths [batch]; lengths beyond suffix_cap count as suffix_cap).
 * The longest n <= min(max_n, length) whose last-n-token n-gram is indexed is matched;
 * cont[q] (device [batch, max_out]) gets the tokens after its most recent occurrence up
 * to the end of that draft or max_out tokens (-1 padded), cont_len[q] their number and
 * match_n[q] (nullable) the n matched (0 and an empty continuation when nothing
 * matches). */
sdv_status sdv_pool_lookup(const sdv_pool* pool, int32_t batch, const int32_t* suffix, const int32_t* suffix_len,
                           int32_t suffix_cap, int32_t max_out, int32_t* cont, int32_t* cont_len,
                           int32_t* match_n, void* stream);

/* Multi-codebook streams ("An Efficient vLLM-Based Inference Pipeline for Unified Audio
 * Understanding and Generation", page 2): the delay pattern (stream s of S codebooks is
 * shifted by s steps, so frame f of stream s is produced at audio step f + s) and its
 * de-interleave into an S x frames code matrix; the primary stream (codebook 0, the
 * backbone token) and the S - 1 auxiliary streams buffered per session; and the phase
 * state machine with its dynamic vocabulary mask: text (text ids only) -> transition
 * (the fixed bridge tokens) -> audio (codebook-0 ids; ends with the end-of-audio code)
 * -> drain (S - 1 pad codes, which flush the delay buffer) -> text.  The modality of a
 * row is the partition of its UNMASKED argmax: ids below text_end are text, ids
 * [codebook_base, codebook_base + Vc) are codebook 0.  A verify pass keeps the phase it
 * starts in; a row that leaves it stops acceptance (argmax -1): a text row whose
 * unmasked argmax is a codebook-0 id (the model switches to audio), a transition row
 * past the bridge, a drain row past its S - 1 steps. */
#define SDV_PHASE_TEXT 0
#define SDV_PHASE_TRANSITION 1
#define SDV_PHASE_AUDIO 2
#define SDV_PHASE_DRAIN 3
#define SDV_MOD_TEXT 0
#define SDV_MOD_AUDIO 1
#define SDV_MOD_OTHER 2
typedef struct {
  int32_t n_codebooks, codebook_size, codebook_base, text_end;
  int32_t eoa_code;            /* codebook-0 code that ends the audio phase */
  int32_t pad_code;            /* codebook-0 code the drain steps carry */
  int32_t n_bridge;
  int32_t max_frames;          /* frames the code matrix holds */
  const int32_t* bridge;       /* [n_bridge] device backbone ids of the transition */
} sdv_stream_cfg;
/* Per-session state, device arrays the caller owns (phase SDV_PHASE_TEXT, the others 0
 * and frames -1 at the start; matrix entries the caller pre-fills, e.g. -1):
 *   phase, phase_pos [B]  the phase and the tokens taken in it (transition / drain);
 *   step [B]              audio steps of the current segment;
 *   frames [B]            frames of the segment once its end-of-audio code arrived, -1 before;
 *   matrix [B, S, max_frames]  codes: matrix[b, s, f] = code of frame f of stream s. */
typedef struct {
  int32_t* phase;
  int32_t* phase_pos;
  int32_t* step;
  int32_t* frames;
  int32_t* matrix;
} sdv_stream_state;

/* The phase mask of a pass: for logit row r of session b (row at logits + (b R + r)
 * row_stride, holding ids id_offset .. id_offset + n_ids - 1; the LM head's rows, or
 * codebook 0's with id_offset = codebook_base) and its prediction depth k = depth[r]
 * within the pass: modality_out = partition of the unmasked argmax (nullable output);
 * argmax_out = argmax under the phase's mask (lowest index on ties), -1 where the row
 * leaves the phase (text: modality audio; transition: bridge[pos + k], -1 past it;
 * audio: codebook-0 ids; drain: the pad code while pos + k < S - 1, then -1).  Feed
 * argmax_out to sdv_accept_greedy. */
sdv_status sdv_phase_mask(const sdv_stream_cfg* cfg, int32_t batch, int32_t R, const float* logits,
                          int64_t row_stride, int32_t id_offset, int32_t n_ids, const int32_t* depth,
                          const sdv_stream_state* state, int32_t* argmax_out, int32_t* modality_out,
                          void* stream);

/* Commit of a pass: the accepted path (tokens of path rows 0..n-1, then next unless it
 * is -1) of every session, in order, through the phase machine; in the audio and drain
 * phases step i's codes (cb_argmax of the logit row that predicted it: row L_a - 1 for
 * i = 0, path[i - 1] after; [B, R, S], nullable outside audio passes) are written with
 * the delay pattern: at audio step t, stream s's code is frame t - s (frames >= 0, below
 * max_frames and, once the end-of-audio code has arrived at step F, below F).  A text
 * pass whose walk stopped at a row of modality audio (modality [B, R] from
 * sdv_phase_mask) switches to the transition phase (the audio phase when there are no
 * bridge tokens). */
sdv_status sdv_stream_commit(const sdv_stream_cfg* cfg, int32_t batch, int32_t T, int32_t L_a, int32_t R,
                             const int32_t* tokens, const int32_t* logit_rows, const int32_t* n_acc,
                             const int32_t* next, const int32_t* path, const int32_t* cb_argmax,
                             const int32_t* modality, const sdv_stream_state* state, void* stream);

/* KV commit / rollback (step 4: roll the cache back to x_{<t}; commit n + 1 tokens).
 *   keep_len [B]: new committed length per sequence (seq_len[b] := keep_len[b]).
 *   move_src, move_dst [B, max_move] (both NULL or both given): for i = 0..max_move-1
 *   in order, when move_src[b,i] >= 0, slot move_src[b,i] of every layer is copied to
 *   slot move_dst[b,i].  Moves run in ascending i per sequence, so a destination may
 *   be a later move's source.  Idempotent for in-place (src == dst) entries.
 *   err [B] nullable: SDV_EBAD_MOVE when a slot or keep_len exceeds the capacity
 *   (that sequence is then left unchanged). */
sdv_status sdv_kv_rollback(const sdv_model* m, const sdv_kv* kv, const int32_t* keep_len,
                           const int32_t* move_src, const int32_t* move_dst, int32_t max_move,
                           int32_t* err, void* stream);

/* Packed weights (layout in the header comment).
 *   sdv_packed_bytes: bytes of the packed form of a matrix with `rows` rows in total
 *   (all sources together) and K columns; 0 for invalid arguments.
 *   sdv_pack_weights: reads the row-major device sources (src0 [rows0, K], src1
 *   [rows1, K], src2 [rows2, K]; unused sources NULL with 0 rows) and writes the packed
 *   matrix to dst (device, dst_bytes >= sdv_packed_bytes).  K must be a multiple of
 *   32 (bf16) or 16 (fp32).  SDV_PACK_PLAIN takes src0 only; SDV_PACK_QKV takes q, k,
 *   v with whole heads of head_dim (64 or 128) rows and equal k and v rows;
 *   SDV_PACK_GATE_UP takes gate and up with equal rows, a multiple of 8.  Sources and
 *   destination must not overlap.  Asynchronous on `stream`. */
size_t sdv_packed_bytes(int32_t dtype, int32_t rows, int32_t K);
sdv_status sdv_pack_weights(int32_t kind, int32_t dtype, int32_t K, int32_t head_dim, const void* src0,
                            int32_t rows0, const void* src1, int32_t rows1, const void* src2,
                            int32_t rows2, void* dst, size_t dst_bytes, void* stream);

const char* sdv_last_error(void);
int32_t sdv_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SDV_H */
