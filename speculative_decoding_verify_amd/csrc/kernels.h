// Kernel argument blocks and launchers of libsdv (internal; not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdv {

enum { EPI_PARTIAL = 0, EPI_LOGITS = 1, EPI_QKV = 2, EPI_SWIGLU = 3 };

// QKV epilogue: rotary embedding + q write + paged K/V append
struct QkvEpi {
  void* q;                  // [M, H*dh] queries times q_scale, query-row format (common.h)
  void* k_pages;            // this layer: [n_blocks][Hkv][16][dh]
  void* v_pages;            //             [n_blocks][Hkv][dh][16]
  const int2* kv_dst;       // [B*T] (physical page, slot in page) of each chunk row, page -1: none
  const float2* rope;       // [B*T][dh/2] (cos, sin) of each chunk row's position
  int B, T, H, Hkv;
  float q_scale;            // log2(e) / sqrt(dh): attention works in the exp2 domain
};

// Activation operands of the GEMMs ("A", M rows x K values) use the tile format of
// common.h: bf16 models carry split pairs (x = hi + lo + O(2^-16 |x|)), fp32 models
// fp32, 16-row tiles in MFMA lane order.
//
// Weights are packed in 1 KB tiles of 16 rows x KS k values (KS = 32 bf16 / 16 fp32):
// tile (n / 16, k / KS) sits at ((n / 16) * (K / KS) + k / KS) * 1024 bytes; inside,
// the 16-byte chunk of row n % 16 and k group ((k % KS) / (KS / 4)) sits at
// (k group * 16 + n % 16) * 16, so lane l of a wave reads chunk l.  Pair packings put
// the two members of 8 pairs into one tile: rows 0-7 the first members, rows 8-15
// the second members of the same pairs.
struct GemmArgs {
  const void* A;            // activation operand, M rows x K (tile format)
  int M;
  const void* W;            // packed weight tiles
  int N;                    // output columns (packed rows) that are written
  int K;
  int steps_per_split;      // k steps (KS values) per workgroup split
  int pair_n;               // SWIGLU: F (pairs = h columns); QKV: dh / 2
  float* out;               // PARTIAL: out[split * out_split_stride + m * ldo + n]
  long long out_split_stride;
  int ldo;
  void* out_act;            // SWIGLU: h [M, F] in the activation tile format
  QkvEpi qkv;               // QKV epilogue arguments
  float* logits;            // LOGITS: logits[m * ldl + n] (nullable)
  int ldl;
  float4* stats;            // LOGITS: stats[m * n_groups + column group]
  int n_groups;
  int n_split;              // gemm_finish: split partials in `out` to sum
};

// launch configuration: NT weight tiles per workgroup, D k steps in flight per wave;
// tiled: the many-row kernel (128-row blocks; NT = MFMA column tiles per wave, D = k
// steps in its LDS ring); wide: the column-split few-row kernel (NT tiles per wave,
// 4 NT per workgroup; q/k/v and SwiGLU launches write split partials that gemm_finish
// sums over column groups of NTF tiles)
struct GemmCfg {
  int NT, D;
  bool tiled = false;
  bool wide = false;
  int NTF = 0;
  int NW = 4;               // wide: waves per workgroup (8 only for split partials)
};
int gemm_lds_ok(int MT, int NT);
// With ev_start / ev_stop set, the events are recorded by the dispatch itself at the
// kernel's start and end (hipExtLaunchKernel), so their interval is the kernel's own
// execution time.
hipError_t launch_gemm(bool is_bf16, const GemmCfg& c, int MT, int epi, dim3 grid, const GemmArgs& a,
                       hipStream_t s, hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
// the split-K finish of a wide q/k/v or SwiGLU launch (grid: column groups of c.NTF
// tiles, c.NTF = gemm_finish_tiles(splits))
int gemm_finish_tiles(int n_split);
hipError_t launch_gemm_finish(bool is_bf16, const GemmCfg& c, int MT, int epi, dim3 grid, const GemmArgs& a,
                              hipStream_t s, hipEvent_t ev_stop = nullptr);

// weight packing (one-time, at model load): rows of up to three row-major [rows, K]
// sources, viewed as one matrix, rearranged into tiles; kind 0 plain, 1 q/k/v rotation
// pairs (head_dim), 2 gate/up pairs
struct PackArgs {
  int kind, K, head_dim;
  const void* src[3];
  int rows[3];
  int n_packed;             // packed rows (multiple of 16)
  void* dst;
};
hipError_t launch_pack(bool is_bf16, const PackArgs& a, hipStream_t s);

struct AttnArgs {
  const void* q;            // [B*T, H*dh] queries pre-scaled by log2(e)/sqrt(dh), query-row format
  const void* k_pages;      // this layer's pages: [n_blocks][Hkv][16][dh]
  const void* v_pages;      //                      [n_blocks][Hkv][dh][16]
  const int32_t* block_table;
  int max_blocks, n_blocks;
  const int32_t* seq_len;
  const uint32_t* anc;      // [T][4] ancestor-or-self bits of each chunk row
  int B, T, H, Hkv;
  int split_keys, n_splits;
  float* po;                // [B][Hkv][n_splits][nq_pad][dh] unnormalised output
  float* pml;               // [B][Hkv][n_splits][nq_pad][2] (running max in log2 units, sum)
  int nq_pad;
  int n_qg;                 // query-tile groups per (sequence, kv head); grid.z = B * n_qg
  int max_ctx;              // cached lengths are clamped to [0, max_ctx] (max_ctx + T fits the table)
  // In-kernel merge: when sem is set, the last workgroup of each (sequence, kv head,
  // query group) to finish merges the split partials and writes o; sem holds one
  // arrival counter per (sequence, kv head, query group), zero before the launch.
  // With sem NULL the partials are left for launch_combine.
  uint32_t* sem;
  void* o;                  // [B*T, H*dh] output rows, activation tile format
};

// Query groups per (sequence, kv head) of the attention launch and the query rows a
// group spans (the merge of one group needs n_splits * rows floats of LDS scratch).
int attn_query_groups(bool is_bf16, int dh, int T, int G, int heads, int* rows_per_group);
constexpr int ATTN_MERGE_FLOATS = 4096;
constexpr int ATTN_MAX_SPLITS = 32;

// ev0 / ev1 (nullable): recorded when the attention kernel starts and ends
hipError_t launch_attention(bool is_bf16, int dh, const AttnArgs& a, hipStream_t s, hipEvent_t ev0 = nullptr,
                            hipEvent_t ev1 = nullptr);
bool attn_uses_reg_path(bool bf, int dh, int NQT);  // keys per tile: 32 bf16 / 16 fp32 either way

struct CombineArgs {
  const float* po;
  const float* pml;
  void* o;                  // [B*T, H*dh] activation tile format
  int B, T, H, Hkv, dh, n_splits, nq_pad;
};
// ev1 (nullable): recorded when the combine kernel ends
hipError_t launch_combine(bool is_bf16, const CombineArgs& a, hipStream_t s, hipEvent_t ev1 = nullptr);

struct PrologueArgs {
  const int32_t* parent;    // nullable
  const int32_t* logit_rows;
  const int32_t* seq_len;   // [B] cached length: rotary positions are seq_len + depth
  int B, T, R;
  int32_t* depth;           // [T]
  uint32_t* anc;            // [T][4]
  int32_t* lm_rows;         // [B*R] = b*T + logit_rows[r]
  float2* rope;             // [B*T][dh/2] (cos, sin)
  int dh;
  float rope_theta;
  int32_t* err;             // [B]
  uint32_t* zero;           // n_zero words cleared (the attention arrival counters)
  int n_zero;
  // destination of each chunk row's K/V: slot seq_len[b] + t through the block table;
  // a slot outside [0, max_ctx + T) or the table, or an invalid page, sets error 0x4
  const int32_t* block_table;
  int max_blocks, n_blocks, max_ctx;
  int2* kv_dst;             // [B*T] (physical page, slot in page), page -1 when invalid
};
hipError_t launch_prologue(const PrologueArgs& a, hipStream_t s);

struct EmbedArgs {
  const int32_t* tokens;    // [B*T]
  const void* embed;        // [V, d]
  const float* gain;        // first layer attention-norm gain
  float* x;                 // [M, d] fp32 residual
  void* a;                  // [M, d] normalised rows, activation tile format
  int M, T, d, V;
  float eps;
  int32_t* err;
};
hipError_t launch_embed_norm(bool is_bf16, const EmbedArgs& a, hipStream_t s);

// Residual add + RMSNorm.  Without `rows`: x[m] += sum of the partials, and row m of
// `a` gets the normalised row, for m < M.  With `rows` (after the last layer): x is
// left as it is; output row j < n_rows of `a` gets the normalised row rows[j] (the
// LM-head operand), and with `hidden` set, hidden[m] = x[m] + partials for m < M.
struct ResidNormArgs {
  float* x;                 // [M, d] fp32 residual
  const float* part;        // [S][M][d] partial sums to add
  long long part_stride;
  int S;
  const float* gain;
  void* a;                  // normalised rows, activation tile format
  float* hidden;            // nullable [M, d] updated residual (with `rows` only)
  int M, d;
  float eps;
  const int32_t* rows;      // nullable [n_rows] source rows of the output rows
  int n_rows;
};
hipError_t launch_resid_norm(bool is_bf16, const ResidNormArgs& a, hipStream_t s);

struct RowReduceArgs {
  const float4* stats;      // [rows][n_groups]
  int rows, n_groups;
  int32_t* argmax;
  float* margin;
  float* lse;
};
hipError_t launch_row_reduce(const RowReduceArgs& a, hipStream_t s);

// Stream embedding rows e_s written as activation rows first_row + s (codebook head).
struct StreamRowsArgs {
  const float* e;           // [S, d]
  int S, d;
  void* act;                // activation operand (tile format of the model type)
  int first_row;
};
hipError_t launch_stream_rows(bool is_bf16, const StreamRowsArgs& a, hipStream_t s);

// Codebook logits of the logit rows plus guidance merge and statistics.  `base` holds
// the head GEMM's split partials: base[split][row][Vc] with rows b*R + r for the logit
// rows and B*R + s for W_cb e_s.
struct CbMergeArgs {
  const float* base;
  long long split_stride;
  int n_split;
  int B, R, S, Vc;
  const int32_t* partner;   // [B] nullable
  float w;
  int token_base;           // backbone id of code 0 of codebook 0
  float* logits;            // [B, R, S, Vc] nullable
  int32_t* cb_argmax;       // [B, R, S] nullable
  int32_t* argmax;          // [B, R] (codebook 0, backbone ids)
  float* margin;            // [B, R]
  float* lse;               // [B, R]
  int32_t* err;             // [B]
};
hipError_t launch_cb_merge(const CbMergeArgs& a, hipStream_t s);

struct GreedyArgs {
  int B, T, L_a, R;
  const int32_t* tokens;
  const int32_t* parent;
  const int32_t* logit_rows;
  const int32_t* argmax;
  const int32_t* base_len;
  int32_t *n_out, *next_out, *path_out, *keep_out, *move_src, *move_dst, *err;
};
hipError_t launch_accept_greedy(const GreedyArgs& a, hipStream_t s);

struct RollbackArgs {
  void* k_pages;
  void* v_pages;
  const int32_t* block_table;
  int32_t* seq_len;
  int max_blocks, n_blocks, B, L, Hkv, dh, elem_bytes;
  const int32_t* keep_len;
  const int32_t* move_src;
  const int32_t* move_dst;
  int max_move;
  int32_t* err;
};
hipError_t launch_kv_rollback(const RollbackArgs& a, hipStream_t s);

// vocabulary entries per chunk of the sampling draw (one workgroup sums a chunk)
constexpr int SAMPLE_CHUNK = 4096;

struct SampleArgs {
  int B, k, V;
  const float* tgt;         // [B, k+1, V]
  const float* drf;         // [B, k, V]
  const int32_t* drafts;    // [B, k]
  unsigned long long seed;  // Philox key
  const int32_t* seq_ids;   // [B] nullable: Philox counter word 0 of sequence b (NULL: b)
  float inv_temp;
  float* row_m;             // [B*(k+1) + B*k] row maximum of the raw logits
  double* row_s;            // [..] sum_v 2^((z_v - max) * log2(e) / temperature)
  int32_t* first_rej;       // [B] position of the draw (first rejection, or k); -1: invalid draft
  uint32_t* seq_flags;      // [B] decision flags (SAMPLE_FLAG_*) handed to the draw
  long long* chunk_sum;     // [B][n_chunks][2] quantised weights: draw row, p row
  int n_chunks, chunk;      // chunk == SAMPLE_CHUNK
  int32_t* n_out;
  int32_t* tok_out;
  uint32_t* flags_out;      // [B] nullable
};
// values of the per-sequence flag word (the ABI's SDV_SAMPLE_* bits)
constexpr uint32_t SAMPLE_FLAG_NEAR_ACCEPT = 0x1, SAMPLE_FLAG_NEAR_DRAW = 0x2, SAMPLE_FLAG_BAD_DRAFT = 0x100;
// ev0 / ev1 (nullable): recorded at the start and end of the row-statistics launch
hipError_t launch_accept_sample(const SampleArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1);

// Philox4x32-10 uniforms of counters (seq, pos, 0, stream): u0 from stream 0, u1 from
// stream 1, [B, n_pos] each (nullable)
struct PhiloxArgs {
  unsigned long long seed;
  const int32_t* seq_ids;   // [B] nullable (NULL: b)
  int B, n_pos;
  double* u0;
  double* u1;
};
hipError_t launch_philox_uniforms(const PhiloxArgs& a, hipStream_t s);

// drafting: the K best first tokens of each row (larger logit first, lower index on ties)
constexpr int DRAFT_MAX_BRANCHES = 16;
struct DraftTopkArgs {
  const float* logits;      // [B, V]
  int B, V, K;
  int32_t* drafts;          // [B, K, max_len]: writes position 0 of each branch
  int max_len;
};
hipError_t launch_draft_topk(const DraftTopkArgs& a, hipStream_t s);

// one drafting step's bookkeeping (draft.hip)
struct DraftStepArgs {
  int B, K, max_len;
  int32_t* drafts;          // [B, K, max_len]
  int save;                 // first call: saved = seq_len, drafts = -1, logit_rows[0] = first_row
  int first_row;
  const int32_t* seq_len;   // [B]
  int32_t* saved;           // [B]
  int32_t* keep_out;        // [B] nullable: saved + keep_delta
  int keep_delta;
  // scatter of the previous step's argmax (one per active branch of that step)
  const int32_t* argmax;    // [B, n_prev]
  int n_prev, prev_pos;
  int prev_branch[DRAFT_MAX_BRANCHES];
  // the next chunk: root row + the first s tokens of each active branch
  const int32_t* root;      // root token of sequence b at root[b * root_stride]
  int root_stride;
  int n_act, s;
  int act_branch[DRAFT_MAX_BRANCHES];
  int32_t* tokens;          // [B, 1 + n_act * s]
  int32_t* parent;          // [1 + n_act * s]
  int32_t* logit_rows;      // [n_act]
};
hipError_t launch_draft_step(const DraftStepArgs& a, hipStream_t s);

// hypothesis pool (pool.hip)
constexpr int POOL_EFULL_STORE = 0x1;       // storage capacity exceeded: draft not stored
constexpr int POOL_EFULL_INDEX = 0x2;       // hash table full: an n-gram not indexed
struct PoolArgs {
  int32_t* tokens;          // [capacity]
  int32_t* seg_end;         // [capacity]
  unsigned long long* keys; // [n_slots]
  int32_t* vals;            // [n_slots]
  int32_t* count;           // [1]
  int capacity, n_slots, max_n;
  const int32_t* draft;     // [len]
  int len;
  int32_t* err;             // [1] nullable
};
hipError_t launch_pool_insert(const PoolArgs& a, hipStream_t s);
hipError_t launch_pool_clear(const PoolArgs& a, hipStream_t s);
struct PoolLookupArgs {
  const int32_t* tokens;
  const int32_t* seg_end;
  const unsigned long long* keys;
  const int32_t* vals;
  const int32_t* count;
  int n_slots, max_n;
  int B;
  const int32_t* suffix;    // [B, suffix_cap]
  const int32_t* suffix_len;// [B]
  int suffix_cap, max_out;
  int32_t* cont;            // [B, max_out]
  int32_t* cont_len;        // [B]
  int32_t* match_n;         // [B] nullable
};
hipError_t launch_pool_lookup(const PoolLookupArgs& a, hipStream_t s);

// multi-codebook stream bookkeeping (streams.hip); phase and modality values follow the
// ABI's SDV_PHASE_* / SDV_MOD_*
constexpr int STREAM_TEXT = 0, STREAM_TRANSITION = 1, STREAM_AUDIO = 2, STREAM_DRAIN = 3;
constexpr int STREAM_MOD_TEXT = 0, STREAM_MOD_AUDIO = 1, STREAM_MOD_OTHER = 2;
struct StreamCfgDev {
  int S, Vc, base, text_end, eoa_code, pad_code, n_bridge, max_frames;
  const int32_t* bridge;    // [n_bridge] device
};
struct PhaseMaskArgs {
  StreamCfgDev cfg;
  int B, R;
  const float* logits;      // row (b, r) at logits + (b * R + r) * row_stride
  long long row_stride;
  int id_offset, n_ids;     // the row holds ids id_offset .. id_offset + n_ids - 1
  const int32_t* depth;     // [R] prediction depth of each logit row in the pass
  const int32_t* phase;     // [B]
  const int32_t* phase_pos; // [B]
  int32_t* argmax_out;      // [B, R]
  int32_t* modality_out;    // [B, R] nullable
};
hipError_t launch_phase_mask(const PhaseMaskArgs& a, hipStream_t s);
struct StreamCommitArgs {
  StreamCfgDev cfg;
  int B, T, L_a, R;
  const int32_t* tokens;    // [B, T]
  const int32_t* logit_rows;// [R]
  const int32_t* n;         // [B]
  const int32_t* next;      // [B]
  const int32_t* path;      // [B, T]
  const int32_t* cb_argmax; // [B, R, S] nullable
  const int32_t* modality;  // [B, R] nullable
  int32_t *phase, *phase_pos, *step, *frames;   // [B] state
  int32_t* matrix;          // [B, S, max_frames]
};
hipError_t launch_stream_commit(const StreamCommitArgs& a, hipStream_t s);

}  // namespace sdv
