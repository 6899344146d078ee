// libsdv host side: argument checks, launch plan, workspace layout and the C ABI.
//
// The plan depends only on host-known sizes (model shape, B, T, R, max_ctx), so a
// sequence of calls with the same sizes issues identical launches; the caller may
// capture them in a graph.  Nothing here allocates device memory or synchronises.
#include <stdarg.h>
#include <stdio.h>
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/sdv.h"
#include "kernels.h"

using namespace sdv;

// Scratch memory of sdv_verify_forward_noalloc: one array per GPU, allocated when the
// code object loads and held until the process ends.  Host code never uses the
// array's name as an address (on the host it is only a stand-in for the symbol): it
// takes each GPU's device address from hipGetSymbolAddress (current_scratch below).
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)SDV_NOALLOC_MAX_WORKSPACE;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_err;

sdv_status fail(sdv_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
sdv_status fail(sdv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }

// target workgroups per launch (256 compute units)
constexpr int TARGET_WG_GEMM = 256;
// workgroups of the column-split GEMM resident at once
#ifndef SDV_WIDE_SLOTS
#define SDV_WIDE_SLOTS 256
#endif
constexpr int WIDE_SLOTS = SDV_WIDE_SLOTS;
// row tiles from which the column-split kernel replaces gemm_stream (at 3 row tiles,
// 41 rows of the 1.7B shape, gemm_stream measured faster on every projection; at 5,
// 65 rows of the 8B shape, the column-split kernel on o, down and q/k/v)
#ifndef SDV_WIDE_MIN_MT
#define SDV_WIDE_MIN_MT 4
#endif
constexpr int WIDE_MIN_MT = SDV_WIDE_MIN_MT;
#ifndef SDV_ATTN_TARGET_WG
#define SDV_ATTN_TARGET_WG 256
#endif
constexpr int TARGET_WG_ATTN = SDV_ATTN_TARGET_WG;  // register path, measured: one workgroup per CU beats two rounds
// the bf16 LDS-DMA path keeps three workgroups per CU
#ifndef SDV_ATTN_DMA_TARGET_WG
#define SDV_ATTN_DMA_TARGET_WG 768
#endif
constexpr int TARGET_WG_ATTN_DMA = SDV_ATTN_DMA_TARGET_WG;
// ... and when the (sequence, kv head, query group) triples alone fill those slots: the
// grid goes out split by split, longest first, so more (shorter) splits make the tail
// finer (batched 64-row pass: 987 -> 960 us per layer at four splits instead of three)
#ifndef SDV_ATTN_DMA_WIDE_TARGET_WG
#define SDV_ATTN_DMA_WIDE_TARGET_WG 6144
#endif
constexpr int TARGET_WG_ATTN_DMA_WIDE = SDV_ATTN_DMA_WIDE_TARGET_WG;
constexpr long long ATTN_MERGE_MAX_READ = 32768;  // floats of partial output one merging workgroup reads

struct GemmPlan {
  GemmCfg cfg;
  int epi;
  int S, spp, ncg, MT, row_blocks;
};

// N: packed weight rows of the launch (pair epilogues: both members of every pair)
GemmPlan plan_gemm(int M, int N, int K, bool bf, int epi) {
  GemmPlan p;
  const int KS = bf ? 32 : 16;
  p.epi = epi;
  const int ntiles = cdiv(N, 16);
  const int steps = K / KS;
  if (M > 80) {
    // many rows (batched sessions): the tiled kernel, 128-row blocks, 2 x WN column
    // tiles per workgroup (WN = 8 when that still gives a full grid)
    p.MT = 8;
    p.row_blocks = cdiv(M, 128);
    const int wn = (long long)cdiv(ntiles, 16) * p.row_blocks >= TARGET_WG_GEMM ? 8 : 4;
    // LDS ring of 3 k steps at WN = 4; at WN = 8 a ring of 2 steps and an epilogue on
    // 64-row halves keep the workgroup at 64 KB, two per CU (the batched 2624-row pass:
    // gate/up 997 -> 809 us, o 214 -> 160, down 507 -> 415, q/k/v 300 -> 248)
    p.cfg = GemmCfg{wn, wn == 8 ? 2 : 3, true};
    p.ncg = cdiv(ntiles, 2 * wn);
    // split-partials launches split K so that the grid's last round of workgroups is
    // as full as possible (at least 16 k steps per split, at most 4 splits)
    int S = 1;
    if (epi == EPI_PARTIAL) {
      const long long wg1 = (long long)p.ncg * p.row_blocks;
      double best = 0.0;
      for (int sp = 1; sp <= 4 && steps / sp >= 16; ++sp) {
        const long long n = wg1 * sp;
        const double eff = (double)n / (double)(cdiv(n, TARGET_WG_GEMM) * TARGET_WG_GEMM);
        if (eff > best + 1e-9) { best = eff; S = sp; }
      }
    }
    p.spp = cdiv(steps, S);
    p.S = cdiv(steps, p.spp);
    return p;
  }
  p.MT = std::max(1, cdiv(M, 16));
  p.row_blocks = 1;
#ifndef SDV_GEMM_STREAM_ONLY
  // (also the split-partial launches over a long K at 33-48 rows: the 1.7B down
  // projection, K = 8192 at 41 rows, 12.9 -> 10.8 us with the residual norm of its
  // 16 partials; its o projection, K = 2048, measured slower)
  if ((p.MT >= WIDE_MIN_MT || (p.MT == 3 && epi == EPI_PARTIAL && K >= 4096)) && epi != EPI_LOGITS) {
    // the column-split kernel (4 NT tiles per workgroup, the activation steps fetched
    // once per workgroup): take the tiles per wave, the K splits and the way the splits
    // meet that minimise an estimate of the launch time.  A compute unit moves its
    // workgroups' weight tiles, activation steps and partial tiles at about 50 GB/s
    // (the measured rate of the weight-streaming kernels through one CU's vector memory
    // path), the whole launch at most at the weights' HBM rate.  Split partials are
    // read back once: by the residual-norm kernel after o and down, by gemm_finish
    // (one dependent launch more) after q/k/v and SwiGLU, whose epilogues otherwise
    // run in the workgroup (one split).
    const int NB = p.MT * (bf ? 2 : 1);   // KB of activations per k step
    const bool fin = epi == EPI_QKV || epi == EPI_SWIGLU;
    const double cu_bw = 50e3, hbm_bw = 7.2e6, l2_bw = 5e6, finish_us = 5.0;   // bytes per us
    double best = 1e300;
    for (int nt = fin ? 2 : 1; nt <= 4; ++nt) {
      const int ncg = cdiv(ntiles, 4 * nt);
      const double tile_b = 16.0 * p.MT * 64 * nt * 4;
      for (int S = 1; S <= 16; ++S) {
        const int spp = cdiv(steps, S), Se = cdiv(steps, spp);
        if (Se != S || (S > 1 && spp < 4)) continue;
        const long long wgs = (long long)ncg * S;
        const double per_wg = (4.0 * nt * spp + (double)spp * NB) * 1024 + (S > 1 || !fin ? tile_b : 0.0);
        const double t0 = std::max((double)cdiv(wgs, WIDE_SLOTS) * per_wg / cu_bw, (double)ntiles * 16 * K * (bf ? 2 : 4) / hbm_bw);
        const double t = t0 + (fin && S == 1 ? 0.0 : (double)S * M * N * 4 / l2_bw + (fin ? finish_us : 0.0));
        if (t < best - 1e-9) {
          best = t;
          p.cfg = GemmCfg{nt, 3, false, true, fin && S > 1 ? gemm_finish_tiles(S) : 0};
          p.ncg = ncg;
          p.spp = spp;
          p.S = S;
        }
      }
    }
    // split partials from eight waves of half the tiles each (the same columns per
    // workgroup, so the same grid and partials): two waves per SIMD overlap one's
    // multiplies with the other's loads (8B shape: down 27.6 -> 26.1 us, o 14.7 ->
    // 13.9; the q/k/v and gate/up launches measured no better)
    if (epi == EPI_PARTIAL && p.cfg.NT % 2 == 0) {
      p.cfg.NT /= 2;
      p.cfg.NW = 8;
    }
    return p;
  }
#endif
  // configurations measured on the decoder shapes: few tiles per workgroup and a
  // deeper register ring where the grid would otherwise be small (q/k/v and o
  // projections), more tiles per workgroup as the row tiles grow
  if (epi == EPI_QKV || (epi == EPI_PARTIAL && p.MT < 4 && ntiles <= 128 && K <= 4096)) p.cfg = GemmCfg{2, 4};
  else if (epi == EPI_PARTIAL && K <= 4096) p.cfg = GemmCfg{4, 2};
  else if (epi == EPI_LOGITS && p.MT <= 2) p.cfg = GemmCfg{4, 4};
  else if (epi == EPI_LOGITS && p.MT == 3) p.cfg = GemmCfg{6, 2};  // 2 waves per SIMD fit (8 tiles: 1)
  else if (epi == EPI_SWIGLU && p.MT >= 4) {
    // at 4-5 row tiles the activation re-reads (one copy per workgroup) cost as much as
    // the weights, so wide workgroups pay; take the width whose grid fills its last
    // round of workgroups best, the widest on ties (8B shape: 6 tiles = 256 workgroups)
    p.cfg = GemmCfg{4, 2};
    double best = -1.0;
    for (int nt : {8, 6, 4}) {
      const long long n = cdiv(ntiles, nt);
      const double eff = (double)n / (double)(cdiv(n, TARGET_WG_GEMM) * TARGET_WG_GEMM);
      if (eff > best + 1e-9 && gemm_lds_ok(p.MT, nt)) { best = eff; p.cfg = GemmCfg{nt, 2}; }
    }
  }
  else if (p.MT >= (epi == EPI_LOGITS ? 3 : 4) && gemm_lds_ok(p.MT, 8)) p.cfg = GemmCfg{8, 2};
  else p.cfg = GemmCfg{4, 2};
  p.ncg = cdiv(ntiles, p.cfg.NT);
  int S = 1;
  if (epi == EPI_PARTIAL) {
    const int target = p.cfg.NT == 2 ? 512 : 256;
    S = cdiv(target, (long long)p.ncg * p.row_blocks);
    S = std::max(1, std::min({S, 16, std::max(1, steps / 8)}));
  }
  p.spp = cdiv(steps, S);
  p.S = cdiv(steps, p.spp);
  return p;
}

struct Plan {
  bool bf;
  int eb;  // element bytes
  int M, Mr, G, nq_pad;
  GemmPlan qkv, o, gu, dn, lm, cb;
  int S;  // codebook streams (0: the model has no codebook heads)
  int split_keys, n_splits;
  int n_qg;         // attention query groups per (sequence, kv head)
  bool attn_fused;  // split partials merged inside the attention kernel
  size_t part_floats;
  size_t off_x, off_a, off_alm, off_q, off_o, off_h, off_part, off_po, off_pml, off_stats, off_depth, off_anc,
      off_lmrows, off_rope, off_cb, off_sem, off_kvdst, total;
  size_t n_sem;     // attention arrival counters: [layer][B][Hkv][n_qg]
};

sdv_status check_model(const sdv_model* m) {
  if (!m) return fail(SDV_ERR_NULL, "model is NULL");
  if (m->dtype != SDV_F32 && m->dtype != SDV_BF16) return fail(SDV_ERR_SHAPE, "dtype %d", m->dtype);
  if (m->n_layers < 1 || m->d < 32 || m->n_heads < 1 || m->n_kv_heads < 1 || m->ffn < 32 || m->vocab < 2)
    return fail(SDV_ERR_SHAPE, "model sizes out of range");
  if (m->head_dim != 64 && m->head_dim != 128) return fail(SDV_ERR_UNSUPPORTED, "head_dim %d (64 or 128)", m->head_dim);
  if (m->n_heads % m->n_kv_heads) return fail(SDV_ERR_SHAPE, "n_heads %% n_kv_heads != 0");
  if (m->d % 64 || m->ffn % 64) return fail(SDV_ERR_UNSUPPORTED, "d and ffn must be multiples of 64");
  if (m->d > 8192) return fail(SDV_ERR_UNSUPPORTED, "d > 8192");
  if (!m->embed || !m->final_norm || !m->lm_head || !m->layers) return fail(SDV_ERR_NULL, "model pointer NULL");
  if (m->n_codebooks < 0) return fail(SDV_ERR_SHAPE, "n_codebooks < 0");
  if (m->n_codebooks > 0) {
    if (!m->codebook || !m->stream_emb) return fail(SDV_ERR_NULL, "codebook pointers NULL");
    if (m->codebook_size < 2 || m->codebook_base < 0 || (long long)m->codebook_base + m->codebook_size > m->vocab)
      return fail(SDV_ERR_SHAPE, "codebook size/base outside the vocabulary");
  }
  for (int l = 0; l < m->n_layers; ++l) {
    const sdv_layer& L = m->layers[l];
    if (!L.attn_norm || !L.wqkv || !L.wo || !L.ffn_norm || !L.wgu || !L.wd)
      return fail(SDV_ERR_NULL, "layer %d has a NULL pointer", l);
  }
  return SDV_OK;
}

Plan make_plan(const sdv_model* m, int B, int T, int R, int max_ctx) {
  Plan p;
  p.bf = m->dtype == SDV_BF16;
  p.eb = p.bf ? 2 : 4;
  p.M = B * T;
  p.Mr = B * R;
  p.G = m->n_heads / m->n_kv_heads;
  const int d = m->d, dh = m->head_dim, H = m->n_heads, Hkv = m->n_kv_heads, F = m->ffn;
  const int qd = H * dh, kd = Hkv * dh;
  p.qkv = plan_gemm(p.M, qd + 2 * kd, d, p.bf, EPI_QKV);
  p.o = plan_gemm(p.M, d, qd, p.bf, EPI_PARTIAL);
  p.gu = plan_gemm(p.M, 2 * F, d, p.bf, EPI_SWIGLU);
  p.dn = plan_gemm(p.M, d, F, p.bf, EPI_PARTIAL);
  p.lm = plan_gemm(p.Mr, m->vocab, d, p.bf, EPI_LOGITS);
  p.S = m->n_codebooks > 0 ? m->n_codebooks : 0;
  if (p.S) p.cb = plan_gemm(p.Mr + p.S, m->codebook_size, d, p.bf, EPI_PARTIAL);
  p.part_floats = std::max((size_t)p.o.S * p.M * d, (size_t)p.dn.S * p.M * d);
  // column-split q/k/v and SwiGLU launches sum their split partials in the finish
  if (p.qkv.cfg.wide && p.qkv.S > 1) p.part_floats = std::max(p.part_floats, (size_t)p.qkv.S * p.M * (qd + 2 * kd));
  if (p.gu.cfg.wide && p.gu.S > 1) p.part_floats = std::max(p.part_floats, (size_t)p.gu.S * p.M * 2 * F);
  // attention: split the keys so that the grid fills the GPU (the register path
  // has four waves per workgroup, each streaming its own key tiles)
  const int KT = p.bf ? 32 : 16;
  const int nkeys = max_ctx + T;
  const int NQT = cdiv(T * p.G, 16);
  int rows_per_group = 0;
  p.n_qg = attn_query_groups(p.bf, dh, T, p.G, B * Hkv, &rows_per_group);
  const bool dma = p.bf && !attn_uses_reg_path(true, dh, NQT);
  const long long groups = (long long)B * Hkv * p.n_qg;
  const int target = !dma ? TARGET_WG_ATTN : groups >= TARGET_WG_ATTN_DMA ? TARGET_WG_ATTN_DMA_WIDE : TARGET_WG_ATTN_DMA;
  int ns = cdiv(target, (long long)B * Hkv * p.n_qg);
  ns = std::max(1, std::min({ns, ATTN_MAX_SPLITS, cdiv(nkeys, KT)}));
  ns = std::max(ns, cdiv(nkeys, 255 * KT));  // a split spans at most 511 pages (staged in LDS)
  p.split_keys = cdiv(cdiv(nkeys, ns), KT) * KT;
  p.n_splits = cdiv(nkeys, p.split_keys);
  p.nq_pad = NQT * 16;
  // the last workgroup of a group merges in-kernel while the partials it reads stay
  // small; larger merges go to the combine kernel, which spreads them over the GPU
  const long long merge_floats = (long long)p.n_splits * rows_per_group;
  p.attn_fused = p.n_splits <= ATTN_MAX_SPLITS && merge_floats <= ATTN_MERGE_FLOATS &&
                 merge_floats * dh <= ATTN_MERGE_MAX_READ;
  p.n_sem = p.attn_fused ? (size_t)m->n_layers * B * Hkv * p.n_qg : 0;

  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes, 256); return at; };
  p.off_x = take((size_t)p.M * d * 4);
  // activation operands take 4 bytes per value (bf16 hi/lo pairs or fp32) in whole
  // 16-row tiles; the head operand holds the B * R logit rows and the codebook
  // head's S stream-embedding rows
  const size_t mpad = (size_t)cdiv(p.M, 16) * 16;
  p.off_a = take(mpad * d * 4);
  p.off_alm = take((size_t)cdiv(p.Mr + p.S, 16) * 16 * d * 4);
  p.off_q = take((size_t)p.M * qd * 4);
  p.off_o = take(mpad * qd * 4);
  p.off_h = take(mpad * F * 4);
  p.off_part = take(p.part_floats * 4);
  const size_t nqs = (size_t)B * Hkv * p.n_splits * p.nq_pad;
  p.off_po = take(nqs * dh * 4);
  p.off_pml = take(nqs * 2 * 4);
  p.off_stats = take((size_t)p.Mr * p.lm.ncg * 16);
  p.off_depth = take((size_t)T * 4);
  p.off_anc = take((size_t)T * 16);
  p.off_lmrows = take((size_t)p.Mr * 4);
  p.off_rope = take((size_t)p.M * (dh / 2) * 8);
  p.off_cb = p.S ? take((size_t)p.cb.S * (p.Mr + p.S) * m->codebook_size * 4) : o;
  p.off_sem = take(p.n_sem * 4);
  p.off_kvdst = take((size_t)p.M * 8);
  p.total = o;
  return p;
}

#define SDV_LAUNCH(expr)                                                                   \
  do {                                                                                     \
    hipError_t e_ = (expr);                                                                \
    if (e_ != hipSuccess) return fail(SDV_ERR_LAUNCH, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

struct ProfEvents {
  void* const* ev = nullptr;
  int n_pairs = 0;
  int next = 0;
};

// one weight-streaming GEMM launch; `a` carries the operands and epilogue targets (the
// split-partials buffer in a.out, also for the q/k/v and SwiGLU launches of the
// column-split kernel, whose finish applies their epilogue)
sdv_status run_gemm(ProfEvents& pe, const Plan& P, const GemmPlan& g, GemmArgs a, hipStream_t s) {
  a.steps_per_split = g.spp;
  a.out_split_stride = (long long)a.M * a.N;
  a.ldo = a.N;
  a.ldl = a.N;
  a.n_groups = g.ncg;
  a.n_split = g.S;
  const dim3 grid = g.cfg.tiled ? dim3(g.row_blocks, g.S, g.ncg) : dim3(g.ncg, g.S, g.row_blocks);
  const bool prof = pe.ev && pe.next < pe.n_pairs;
  hipEvent_t e0 = prof ? (hipEvent_t)pe.ev[2 * pe.next] : nullptr;
  hipEvent_t e1 = prof ? (hipEvent_t)pe.ev[2 * pe.next + 1] : nullptr;
  if (g.cfg.wide && g.epi != EPI_PARTIAL && g.cfg.NTF == 0 && g.S > 1)
    return fail(SDV_ERR_LAUNCH, "column-split epilogue %d planned with %d K splits", g.epi, g.S);
  if (g.cfg.wide && g.cfg.NTF > 0) {
    if (!a.out) return fail(SDV_ERR_LAUNCH, "split partials buffer missing");
    SDV_LAUNCH(launch_gemm(P.bf, g.cfg, g.MT, EPI_PARTIAL, grid, a, s, e0, nullptr));
    const int ntiles = cdiv(a.N, 16);
    SDV_LAUNCH(launch_gemm_finish(P.bf, g.cfg, g.MT, g.epi, dim3(cdiv(ntiles, g.cfg.NTF)), a, s, e1));
  } else {
    SDV_LAUNCH(launch_gemm(P.bf, g.cfg, g.MT, g.epi, grid, a, s, e0, e1));
  }
  if (pe.ev) ++pe.next;
  return SDV_OK;
}

GemmArgs gemm_args(const void* A, int M, const void* W, int N, int K) {
  GemmArgs a;
  memset(&a, 0, sizeof a);
  a.A = A;
  a.M = M;
  a.W = W;
  a.N = N;
  a.K = K;
  return a;
}

// The device address of each GPU's copy of `scratch`, looked up once per device.
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// device address of the current device's scratch array (looked up on the first call
// on that device, with that device current)
sdv_status current_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SDV_ERR_LAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= MAX_DEVICES) return fail(SDV_ERR_UNSUPPORTED, "device ordinal %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(SDV_ERR_LAUNCH, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SDV_OK;
}

sdv_status verify_forward_impl(const sdv_model* m, const sdv_kv* kv, const sdv_verify_in* in, sdv_verify_out* out,
                               void* ws, size_t ws_bytes, void* stream, bool use_scratch);

}  // namespace

extern "C" {

int32_t sdv_abi_version(void) { return SDV_ABI_VERSION; }
const char* sdv_last_error(void) { return g_err.c_str(); }

size_t sdv_verify_workspace_size(const sdv_model* m, int32_t batch, int32_t T, int32_t R, int32_t max_ctx) {
  if (check_model(m) != SDV_OK || batch < 1 || T < 1 || T > SDV_MAX_T || R < 1 || R > T || max_ctx < 0) return 0;
  return make_plan(m, batch, T, R, max_ctx).total;
}

sdv_status sdv_verify_forward(const sdv_model* m, const sdv_kv* kv, const sdv_verify_in* in, sdv_verify_out* out,
                              void* ws, size_t ws_bytes, void* stream) {
  return verify_forward_impl(m, kv, in, out, ws, ws_bytes, stream, false);
}

sdv_status sdv_verify_forward_noalloc(const sdv_model* m, const sdv_kv* kv, const sdv_verify_in* in,
                                      sdv_verify_out* out, void* stream) {
  return verify_forward_impl(m, kv, in, out, nullptr, 0, stream, true);
}

}  // extern "C"

namespace {

// The passes of a draft tree: pass 0 runs the chunk (T = L_a, one logit row); pass
// s >= 1 runs the root row plus the first s tokens of every branch longer than s.
struct DraftPass {
  int T, R, max_ctx, n_act;
  int act[DRAFT_MAX_BRANCHES];
};

struct DraftPlan {
  int K, max_len, T_max;
  std::vector<DraftPass> passes;
  size_t verify_ws;
  size_t off_tokens, off_parent, off_rows, off_argmax, off_margin, off_lse, off_logits, off_saved, off_keep, total;
};

sdv_status make_draft_plan(const sdv_model* m, int B, int L_a, int K, const int32_t* len, int max_ctx,
                           DraftPlan* out) {
  sdv_status st = check_model(m);
  if (st != SDV_OK) return st;
  if (B < 1) return fail(SDV_ERR_SHAPE, "batch %d", B);
  if (L_a < 1 || L_a > SDV_MAX_T) return fail(SDV_ERR_SHAPE, "L_a = %d outside [1, %d]", L_a, SDV_MAX_T);
  if (K < 1 || K > DRAFT_MAX_BRANCHES) return fail(SDV_ERR_SHAPE, "%d branches outside [1, %d]", K, DRAFT_MAX_BRANCHES);
  if (K > m->vocab) return fail(SDV_ERR_SHAPE, "more branches than vocabulary entries");
  if (!len) return fail(SDV_ERR_NULL, "branch_len is NULL");
  if (max_ctx < 0) return fail(SDV_ERR_SHAPE, "max_ctx < 0");
  DraftPlan& P = *out;
  P.K = K;
  P.max_len = 0;
  for (int k = 0; k < K; ++k) {
    if (len[k] < 1 || len[k] > SDV_MAX_T) return fail(SDV_ERR_SHAPE, "branch_len[%d] = %d", k, len[k]);
    P.max_len = std::max(P.max_len, (int)len[k]);
  }
  P.passes.clear();
  DraftPass p0{};
  p0.T = L_a;
  p0.R = 1;
  p0.max_ctx = max_ctx;
  P.passes.push_back(p0);
  P.T_max = L_a;
  for (int s = 1; s < P.max_len; ++s) {
    DraftPass p{};
    for (int k = 0; k < K; ++k)
      if (len[k] > s) p.act[p.n_act++] = k;
    p.T = 1 + s * p.n_act;
    p.R = p.n_act;
    p.max_ctx = max_ctx + L_a - 1;
    if (p.T > SDV_MAX_T)
      return fail(SDV_ERR_SHAPE, "drafting pass %d would take %d rows (at most %d)", s, p.T, SDV_MAX_T);
    P.T_max = std::max(P.T_max, p.T);
    P.passes.push_back(p);
  }
  P.verify_ws = 0;
  for (const DraftPass& p : P.passes) P.verify_ws = std::max(P.verify_ws, make_plan(m, B, p.T, p.R, p.max_ctx).total);
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes, 256); return at; };
  take(P.verify_ws);
  P.off_tokens = take((size_t)B * P.T_max * 4);
  P.off_parent = take((size_t)P.T_max * 4);
  P.off_rows = take((size_t)K * 4);
  P.off_argmax = take((size_t)B * K * 4);
  P.off_margin = take((size_t)B * K * 4);
  P.off_lse = take((size_t)B * K * 4);
  P.off_logits = take((size_t)B * m->vocab * 4);
  P.off_saved = take((size_t)B * 4);
  P.off_keep = take((size_t)B * 4);
  P.total = o;
  return SDV_OK;
}

sdv_status verify_forward_impl(const sdv_model* m, const sdv_kv* kv, const sdv_verify_in* in, sdv_verify_out* out,
                               void* ws, size_t ws_bytes, void* stream, bool use_scratch) {
  sdv_status st = check_model(m);
  if (st != SDV_OK) return st;
  if (!kv || !in || !out) return fail(SDV_ERR_NULL, "kv/in/out is NULL");
  if (!kv->k_pages || !kv->v_pages || !kv->block_table || !kv->seq_len) return fail(SDV_ERR_NULL, "kv pointer NULL");
  if (!in->tokens || !in->logit_rows) return fail(SDV_ERR_NULL, "tokens/logit_rows NULL");
  if (!out->argmax || !out->margin || !out->lse || !out->err) return fail(SDV_ERR_NULL, "output pointer NULL");
  const int B = in->batch, T = in->T, R = in->R;
  if (B < 1 || B != kv->batch) return fail(SDV_ERR_SHAPE, "batch %d (kv batch %d)", B, kv->batch);
  if (T < 1 || T > SDV_MAX_T) return fail(SDV_ERR_SHAPE, "T = %d outside [1, %d]", T, SDV_MAX_T);
  if (R < 1 || R > T) return fail(SDV_ERR_SHAPE, "R = %d outside [1, T]", R);
  if (in->L_a < 0 || in->L_a > T) return fail(SDV_ERR_SHAPE, "L_a = %d outside [0, T]", in->L_a);
  if (in->max_ctx < 0) return fail(SDV_ERR_SHAPE, "max_ctx < 0");
  if (kv->max_blocks < 1 || kv->n_blocks < 1) return fail(SDV_ERR_SHAPE, "empty cache");
  if ((long long)in->max_ctx + T > (long long)kv->max_blocks * SDV_PAGE)
    return fail(SDV_ERR_SHAPE, "max_ctx + T exceeds the cache capacity");
  if (in->head != SDV_HEAD_LM && in->head != SDV_HEAD_CODEBOOK) return fail(SDV_ERR_SHAPE, "head %d", in->head);
  if (in->head == SDV_HEAD_CODEBOOK && m->n_codebooks < 1) return fail(SDV_ERR_UNSUPPORTED, "model has no codebook heads");
  if (in->head == SDV_HEAD_LM && in->cfg_partner) return fail(SDV_ERR_UNSUPPORTED, "guidance pairs need the codebook head");
  const Plan P = make_plan(m, B, T, R, in->max_ctx);
  if ((long long)B * P.n_qg > 65535)
    return fail(SDV_ERR_UNSUPPORTED, "batch %d x %d query groups exceeds the attention grid", B, P.n_qg);
  if (use_scratch) {
    if (P.total > NOALLOC_SCRATCH_BYTES)
      return fail(SDV_ERR_WORKSPACE, "pass needs %zu bytes of scratch, more than the %zu-byte static scratch of "
                  "sdv_verify_forward_noalloc (use sdv_verify_forward with a workspace)", P.total,
                  NOALLOC_SCRATCH_BYTES);
    if ((st = current_scratch(&ws)) != SDV_OK) return st;
    ws_bytes = NOALLOC_SCRATCH_BYTES;
  }
  if (!ws || ws_bytes < P.total) return fail(SDV_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, P.total);

  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  float* x = (float*)(w + P.off_x);
  void* act = w + P.off_a;
  void* alm = w + P.off_alm;
  void* q = w + P.off_q;
  void* o = w + P.off_o;
  void* h = w + P.off_h;
  float* part = (float*)(w + P.off_part);
  float* po = (float*)(w + P.off_po);
  float* pml = (float*)(w + P.off_pml);
  float4* stats = (float4*)(w + P.off_stats);
  int32_t* depth = (int32_t*)(w + P.off_depth);
  uint32_t* anc = (uint32_t*)(w + P.off_anc);
  int32_t* lm_rows = (int32_t*)(w + P.off_lmrows);
  uint32_t* sem = (uint32_t*)(w + P.off_sem);
  int2* kv_dst = (int2*)(w + P.off_kvdst);

  const int d = m->d, H = m->n_heads, Hkv = m->n_kv_heads, dh = m->head_dim, F = m->ffn, V = m->vocab;
  const int qd = H * dh, kd = Hkv * dh, M = P.M;
  const size_t layer_elems = (size_t)kv->n_blocks * Hkv * SDV_PAGE * dh;

  ProfEvents pe;
  if (out->prof_events && out->n_prof_events >= 2) {
    pe.ev = out->prof_events;
    pe.n_pairs = out->n_prof_events / 2;
  }
  float2* rope = (float2*)(w + P.off_rope);
  {
    PrologueArgs a{in->parent, in->logit_rows, kv->seq_len, B, T, R, depth, anc, lm_rows, rope, dh,
                   m->rope_theta, out->err, sem, (int)P.n_sem,
                   kv->block_table, kv->max_blocks, kv->n_blocks, in->max_ctx, kv_dst};
    SDV_LAUNCH(launch_prologue(a, s));
  }
  {
    EmbedArgs a{in->tokens, m->embed, m->layers[0].attn_norm, x, act, M, T, d, V, m->eps, out->err};
    SDV_LAUNCH(launch_embed_norm(P.bf, a, s));
  }
  for (int l = 0; l < m->n_layers; ++l) {
    const sdv_layer& L = m->layers[l];
    void* kp = (char*)kv->k_pages + l * layer_elems * P.eb;
    void* vp = (char*)kv->v_pages + l * layer_elems * P.eb;
    // q, k, v projections with rotary embedding and paged K/V append
    {
      GemmArgs a = gemm_args(act, M, L.wqkv, qd + 2 * kd, d);
      a.pair_n = dh / 2;
      a.qkv = QkvEpi{q, kp, vp, kv_dst, rope, B, T, H, Hkv, (float)(1.4426950408889634 / sqrt((double)dh))};
      a.out = part;
      if ((st = run_gemm(pe, P, P.qkv, a, s)) != SDV_OK) return st;
    }
    {
      AttnArgs a{q, kp, vp, kv->block_table, kv->max_blocks, kv->n_blocks, kv->seq_len, anc, B, T, H, Hkv,
                 P.split_keys, P.n_splits, po, pml, P.nq_pad, P.n_qg, in->max_ctx,
                 P.attn_fused ? sem + (size_t)l * B * Hkv * P.n_qg : nullptr, o};
      // with attention events: event 2l at the attention kernel's start, 2l + 1 at the
      // end of the kernel that finishes the layer's attention (the combine, if any)
      const bool aprof = out->attn_prof_events && 2 * l + 1 < out->n_attn_prof_events;
      hipEvent_t ae0 = aprof ? (hipEvent_t)out->attn_prof_events[2 * l] : nullptr;
      hipEvent_t ae1 = aprof ? (hipEvent_t)out->attn_prof_events[2 * l + 1] : nullptr;
      SDV_LAUNCH(launch_attention(P.bf, dh, a, s, ae0, P.attn_fused ? ae1 : nullptr));
      if (!P.attn_fused) {
        CombineArgs c{po, pml, o, B, T, H, Hkv, dh, P.n_splits, P.nq_pad};
        SDV_LAUNCH(launch_combine(P.bf, c, s, ae1));
      }
    }
    {
      GemmArgs a = gemm_args(o, M, L.wo, d, qd);
      a.out = part;
      if ((st = run_gemm(pe, P, P.o, a, s)) != SDV_OK) return st;
    }
    {
      ResidNormArgs a{x, part, (long long)M * d, P.o.S, L.ffn_norm, act, nullptr, M, d, m->eps, nullptr, 0};
      SDV_LAUNCH(launch_resid_norm(P.bf, a, s));
    }
    // gate/up projections with the SwiGLU epilogue
    {
      GemmArgs a = gemm_args(act, M, L.wgu, 2 * F, d);
      a.pair_n = F;
      a.out_act = h;
      a.out = part;
      if ((st = run_gemm(pe, P, P.gu, a, s)) != SDV_OK) return st;
    }
    {
      GemmArgs a = gemm_args(h, M, L.wd, d, F);
      a.out = part;
      if ((st = run_gemm(pe, P, P.dn, a, s)) != SDV_OK) return st;
    }
    if (l + 1 < m->n_layers) {
      ResidNormArgs a{x, part, (long long)M * d, P.dn.S, m->layers[l + 1].attn_norm, act, nullptr, M, d, m->eps,
                      nullptr, 0};
      SDV_LAUNCH(launch_resid_norm(P.bf, a, s));
    } else {
      // final norm of the logit rows only, gathered into the head operand (rows
      // b * R + r), plus the hidden rows when asked for
      ResidNormArgs a{x, part, (long long)M * d, P.dn.S, m->final_norm, alm, out->hidden, M, d, m->eps,
                      lm_rows, P.Mr};
      SDV_LAUNCH(launch_resid_norm(P.bf, a, s));
    }
  }
  if (in->head == SDV_HEAD_CODEBOOK) {
    // codebook heads: W_cb on the final-normed logit rows and on the stream
    // embeddings (rows Mr..Mr+S-1 of the head operand), then merge + statistics
    const int S = P.S, Vc = m->codebook_size;
    float* cbl = (float*)(w + P.off_cb);
    StreamRowsArgs sr{m->stream_emb, S, d, alm, P.Mr};
    SDV_LAUNCH(launch_stream_rows(P.bf, sr, s));
    GemmArgs a = gemm_args(alm, P.Mr + S, m->codebook, Vc, d);
    a.out = cbl;
    if ((st = run_gemm(pe, P, P.cb, a, s)) != SDV_OK) return st;
    CbMergeArgs c{cbl, (long long)(P.Mr + S) * Vc, P.cb.S, B, R, S, Vc, in->cfg_partner, in->cfg_w,
                  m->codebook_base, out->logits, out->cb_argmax, out->argmax, out->margin, out->lse, out->err};
    SDV_LAUNCH(launch_cb_merge(c, s));
  } else {
    {
      GemmArgs a = gemm_args(alm, P.Mr, m->lm_head, V, d);
      a.logits = out->logits;
      a.stats = stats;
      if ((st = run_gemm(pe, P, P.lm, a, s)) != SDV_OK) return st;
    }
    {
      RowReduceArgs a{stats, P.Mr, P.lm.ncg, out->argmax, out->margin, out->lse};
      SDV_LAUNCH(launch_row_reduce(a, s));
    }
  }
  return SDV_OK;
}

}  // namespace

extern "C" {

sdv_status sdv_accept_greedy(int32_t B, int32_t T, int32_t L_a, const int32_t* tokens, const int32_t* parent,
                             int32_t R, const int32_t* logit_rows, const int32_t* argmax, const int32_t* base_len,
                             int32_t* n_out, int32_t* next_out, int32_t* path_out, int32_t* keep_out,
                             int32_t* move_src, int32_t* move_dst, int32_t* err, void* stream) {
  if (!tokens || !logit_rows || !argmax || !n_out || !next_out) return fail(SDV_ERR_NULL, "NULL argument");
  if (B < 1 || T < 1 || T > SDV_MAX_T || R < 1 || R > T) return fail(SDV_ERR_SHAPE, "B/T/R out of range");
  if (L_a < 1 || L_a > T) return fail(SDV_ERR_SHAPE, "L_a = %d outside [1, T]", L_a);
  if ((move_src == nullptr) != (move_dst == nullptr)) return fail(SDV_ERR_NULL, "move_src/move_dst: give both or neither");
  GreedyArgs a{B, T, L_a, R, tokens, parent, logit_rows, argmax, base_len, n_out, next_out, path_out, keep_out,
               move_src, move_dst, err};
  SDV_LAUNCH(launch_accept_greedy(a, (hipStream_t)stream));
  return SDV_OK;
}

size_t sdv_packed_bytes(int32_t dtype, int32_t rows, int32_t K) {
  if ((dtype != SDV_F32 && dtype != SDV_BF16) || rows < 1 || K < 1) return 0;
  return (size_t)cdiv(rows, 16) * 16 * K * (dtype == SDV_BF16 ? 2 : 4);
}

sdv_status sdv_pack_weights(int32_t kind, int32_t dtype, int32_t K, int32_t head_dim, const void* src0,
                            int32_t rows0, const void* src1, int32_t rows1, const void* src2, int32_t rows2,
                            void* dst, size_t dst_bytes, void* stream) {
  if (dtype != SDV_F32 && dtype != SDV_BF16) return fail(SDV_ERR_SHAPE, "dtype %d", dtype);
  const int KS = dtype == SDV_BF16 ? 32 : 16;
  if (K < KS || K % KS) return fail(SDV_ERR_SHAPE, "K = %d must be a positive multiple of %d", K, KS);
  if (!dst || !src0) return fail(SDV_ERR_NULL, "dst or src0 is NULL");
  if (rows0 < 1 || rows1 < 0 || rows2 < 0) return fail(SDV_ERR_SHAPE, "row counts out of range");
  if ((rows1 > 0 && !src1) || (rows2 > 0 && !src2)) return fail(SDV_ERR_NULL, "a source with rows is NULL");
  const long long total = (long long)rows0 + rows1 + rows2;
  PackArgs a;
  a.kind = kind;
  a.K = K;
  a.head_dim = head_dim;
  a.src[0] = src0;
  a.src[1] = rows1 ? src1 : nullptr;
  a.src[2] = rows2 ? src2 : nullptr;
  a.rows[0] = rows0;
  a.rows[1] = rows1;
  a.rows[2] = rows2;
  if (kind == SDV_PACK_PLAIN) {
    if (rows1 || rows2) return fail(SDV_ERR_SHAPE, "plain packing takes one source");
  } else if (kind == SDV_PACK_QKV) {
    if (head_dim != 64 && head_dim != 128) return fail(SDV_ERR_UNSUPPORTED, "head_dim %d (64 or 128)", head_dim);
    if (rows0 % head_dim || rows1 % head_dim || rows2 % head_dim || rows1 != rows2 || rows1 < head_dim)
      return fail(SDV_ERR_SHAPE, "q/k/v rows must be whole heads, k and v alike");
  } else if (kind == SDV_PACK_GATE_UP) {
    if (rows0 != rows1 || rows2 || rows0 % 8) return fail(SDV_ERR_SHAPE, "gate and up need equal rows, a multiple of 8");
  } else {
    return fail(SDV_ERR_SHAPE, "pack kind %d", kind);
  }
  a.n_packed = cdiv(total, 16) * 16;
  const size_t need = sdv_packed_bytes(dtype, (int32_t)total, K);
  if (dst_bytes < need) return fail(SDV_ERR_WORKSPACE, "destination %zu < %zu bytes", dst_bytes, need);
  a.dst = dst;
  SDV_LAUNCH(launch_pack(dtype == SDV_BF16, a, (hipStream_t)stream));
  return SDV_OK;
}

sdv_status sdv_kv_rollback(const sdv_model* m, const sdv_kv* kv, const int32_t* keep_len, const int32_t* move_src,
                           const int32_t* move_dst, int32_t max_move, int32_t* err, void* stream) {
  if (!m || !kv || !keep_len) return fail(SDV_ERR_NULL, "NULL argument");
  if (!kv->k_pages || !kv->v_pages || !kv->block_table || !kv->seq_len) return fail(SDV_ERR_NULL, "kv pointer NULL");
  if ((move_src == nullptr) != (move_dst == nullptr)) return fail(SDV_ERR_NULL, "move_src/move_dst: give both or neither");
  if (move_src && max_move < 1) return fail(SDV_ERR_SHAPE, "max_move < 1");
  if (kv->batch < 1) return fail(SDV_ERR_SHAPE, "batch < 1");
  RollbackArgs a{kv->k_pages, kv->v_pages, kv->block_table, kv->seq_len, kv->max_blocks, kv->n_blocks, kv->batch,
                 m->n_layers, m->n_kv_heads, m->head_dim, m->dtype == SDV_BF16 ? 2 : 4, keep_len, move_src,
                 move_dst, move_src ? max_move : 0, err};
  SDV_LAUNCH(launch_kv_rollback(a, (hipStream_t)stream));
  return SDV_OK;
}


size_t sdv_sample_workspace_size(int32_t B, int32_t k, int32_t V) {
  if (B < 1 || k < 1 || k > SDV_SAMPLE_MAX_K || V < 2) return 0;
  const size_t rows = (size_t)B * (2 * k + 1);
  const int nch = cdiv(V, SAMPLE_CHUNK);
  return align_up(rows * 4, 256) + align_up(rows * 8, 256) + 2 * align_up((size_t)B * 4, 256) +
         align_up((size_t)B * nch * 2 * 8, 256);
}

sdv_status sdv_accept_sample(int32_t B, int32_t k, int32_t V, const float* tgt, const float* drf,
                             const int32_t* drafts, float temperature, uint64_t seed, const int32_t* seq_ids,
                             int32_t* n_out, int32_t* tok_out, uint32_t* flags_out, void* ws, size_t ws_bytes,
                             void* const* prof_events, void* stream) {
  if (!tgt || !drf || !drafts || !n_out || !tok_out) return fail(SDV_ERR_NULL, "NULL argument");
  if (B < 1 || k < 1 || V < 2) return fail(SDV_ERR_SHAPE, "B/k/V out of range");
  if (k > SDV_SAMPLE_MAX_K) return fail(SDV_ERR_SHAPE, "k = %d > %d", k, SDV_SAMPLE_MAX_K);
  if (!(temperature > 0.f) || !isfinite(temperature)) return fail(SDV_ERR_SHAPE, "temperature must be finite and > 0");
  const size_t need = sdv_sample_workspace_size(B, k, V);
  if (!ws || ws_bytes < need) return fail(SDV_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  const size_t rows = (size_t)B * (2 * k + 1);
  char* w = (char*)ws;
  SampleArgs a;
  a.B = B;
  a.k = k;
  a.V = V;
  a.tgt = tgt;
  a.drf = drf;
  a.drafts = drafts;
  a.seed = seed;
  a.seq_ids = seq_ids;
  a.inv_temp = 1.f / temperature;
  a.row_m = (float*)w;
  w += align_up(rows * 4, 256);
  a.row_s = (double*)w;
  w += align_up(rows * 8, 256);
  a.first_rej = (int32_t*)w;
  w += align_up((size_t)B * 4, 256);
  a.seq_flags = (uint32_t*)w;
  w += align_up((size_t)B * 4, 256);
  a.chunk_sum = (long long*)w;
  a.chunk = SAMPLE_CHUNK;
  a.n_chunks = cdiv(V, SAMPLE_CHUNK);
  a.n_out = n_out;
  a.tok_out = tok_out;
  a.flags_out = flags_out;
  SDV_LAUNCH(launch_accept_sample(a, (hipStream_t)stream, prof_events ? (hipEvent_t)prof_events[0] : nullptr,
                                  prof_events ? (hipEvent_t)prof_events[1] : nullptr));
  return SDV_OK;
}

size_t sdv_draft_workspace_size(const sdv_model* m, int32_t batch, int32_t L_a, int32_t n_branches,
                                const int32_t* branch_len, int32_t max_ctx) {
  DraftPlan P;
  if (make_draft_plan(m, batch, L_a, n_branches, branch_len, max_ctx, &P) != SDV_OK) return 0;
  return P.total;
}

sdv_status sdv_draft_tree(const sdv_model* m, const sdv_kv* kv, const sdv_draft_in* in, int32_t* drafts,
                          int32_t* err, void* ws, size_t ws_bytes, void* stream) {
  if (!kv || !in || !drafts || !err) return fail(SDV_ERR_NULL, "kv/in/drafts/err is NULL");
  if (!in->chunk) return fail(SDV_ERR_NULL, "chunk is NULL");
  if (!kv->k_pages || !kv->v_pages || !kv->block_table || !kv->seq_len) return fail(SDV_ERR_NULL, "kv pointer NULL");
  DraftPlan P;
  sdv_status st = make_draft_plan(m, in->batch, in->L_a, in->n_branches, in->branch_len, in->max_ctx, &P);
  if (st != SDV_OK) return st;
  const int B = in->batch, K = P.K, L_a = in->L_a;
  if (B != kv->batch) return fail(SDV_ERR_SHAPE, "batch %d (kv batch %d)", B, kv->batch);
  const long long cap = (long long)kv->max_blocks * SDV_PAGE;
  for (const DraftPass& p : P.passes)
    if ((long long)p.max_ctx + p.T > cap) return fail(SDV_ERR_SHAPE, "max_ctx + drafting rows exceed the cache capacity");
  if (!ws || ws_bytes < P.total) return fail(SDV_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, P.total);
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  int32_t* tokens = (int32_t*)(w + P.off_tokens);
  int32_t* parent = (int32_t*)(w + P.off_parent);
  int32_t* rows = (int32_t*)(w + P.off_rows);
  int32_t* argmax = (int32_t*)(w + P.off_argmax);
  int32_t* saved = (int32_t*)(w + P.off_saved);
  int32_t* keep = (int32_t*)(w + P.off_keep);
  float* logits = (float*)(w + P.off_logits);

  DraftStepArgs d;
  memset(&d, 0, sizeof d);
  d.B = B;
  d.K = K;
  d.max_len = P.max_len;
  d.drafts = drafts;
  d.seq_len = kv->seq_len;
  d.saved = saved;
  d.argmax = argmax;
  d.root = in->chunk + (L_a - 1);
  d.root_stride = L_a;
  d.tokens = tokens;
  d.parent = parent;
  d.logit_rows = rows;
  // remember C, clear the drafts, set the first pass's logit row; keep = C + L_a - 1
  d.save = 1;
  d.first_row = L_a - 1;
  d.keep_out = keep;
  d.keep_delta = L_a - 1;
  SDV_LAUNCH(launch_draft_step(d, s));
  d.save = 0;
  d.keep_out = nullptr;

  sdv_verify_out vo;
  memset(&vo, 0, sizeof vo);
  vo.argmax = argmax;
  vo.margin = (float*)(w + P.off_margin);
  vo.lse = (float*)(w + P.off_lse);
  vo.err = err;
  // pass 0: the hypothesised chunk; the first tokens of all branches from its last row
  {
    sdv_verify_in vi{B, L_a, L_a, 1, in->max_ctx, in->chunk, nullptr, rows, SDV_HEAD_LM, nullptr, 1.f};
    vo.logits = logits;
    if ((st = verify_forward_impl(m, kv, &vi, &vo, ws, P.verify_ws, stream, false)) != SDV_OK) return st;
    vo.logits = nullptr;
    DraftTopkArgs t{logits, B, m->vocab, K, drafts, P.max_len};
    SDV_LAUNCH(launch_draft_topk(t, s));
  }
  // commit the chunk rows but the last, which is the root of the following passes
  if ((st = sdv_kv_rollback(m, kv, keep, nullptr, nullptr, 0, err, stream)) != SDV_OK) return st;
  for (size_t pi = 1; pi < P.passes.size(); ++pi) {
    const DraftPass& p = P.passes[pi];
    const int sx = (int)pi;
    if (pi >= 2) {
      const DraftPass& q = P.passes[pi - 1];
      d.n_prev = q.n_act;
      d.prev_pos = sx - 1;
      for (int r = 0; r < q.n_act; ++r) d.prev_branch[r] = q.act[r];
    }
    d.n_act = p.n_act;
    d.s = sx;
    for (int r = 0; r < p.n_act; ++r) d.act_branch[r] = p.act[r];
    SDV_LAUNCH(launch_draft_step(d, s));
    sdv_verify_in vi{B, p.T, 1, p.R, p.max_ctx, tokens, parent, rows, SDV_HEAD_LM, nullptr, 1.f};
    if ((st = verify_forward_impl(m, kv, &vi, &vo, ws, P.verify_ws, stream, false)) != SDV_OK) return st;
  }
  // the last pass's tokens, and the cache back at C
  d.n_prev = 0;
  if (P.passes.size() >= 2) {
    const DraftPass& q = P.passes.back();
    d.n_prev = q.n_act;
    d.prev_pos = (int)P.passes.size() - 1;
    for (int r = 0; r < q.n_act; ++r) d.prev_branch[r] = q.act[r];
  }
  d.n_act = 0;
  d.keep_out = keep;
  d.keep_delta = 0;
  SDV_LAUNCH(launch_draft_step(d, s));
  return sdv_kv_rollback(m, kv, keep, nullptr, nullptr, 0, err, stream);
}

namespace {

sdv_status pool_args(const sdv_pool* p, PoolArgs* a) {
  if (!p) return fail(SDV_ERR_NULL, "pool is NULL");
  if (!p->tokens || !p->seg_end || !p->keys || !p->vals || !p->count) return fail(SDV_ERR_NULL, "pool pointer NULL");
  if (p->capacity < 1) return fail(SDV_ERR_SHAPE, "pool capacity %d", p->capacity);
  if (p->n_slots < 1 || (p->n_slots & (p->n_slots - 1))) return fail(SDV_ERR_SHAPE, "n_slots %d is not a power of two", p->n_slots);
  if (p->max_n < 1 || p->max_n > SDV_POOL_MAX_N) return fail(SDV_ERR_SHAPE, "max_n %d outside [1, %d]", p->max_n, SDV_POOL_MAX_N);
  memset(a, 0, sizeof *a);
  a->tokens = p->tokens;
  a->seg_end = p->seg_end;
  a->keys = (unsigned long long*)p->keys;
  a->vals = p->vals;
  a->count = p->count;
  a->capacity = p->capacity;
  a->n_slots = p->n_slots;
  a->max_n = p->max_n;
  return SDV_OK;
}

}  // namespace

sdv_status sdv_pool_clear(const sdv_pool* pool, void* stream) {
  PoolArgs a;
  sdv_status st = pool_args(pool, &a);
  if (st != SDV_OK) return st;
  SDV_LAUNCH(launch_pool_clear(a, (hipStream_t)stream));
  return SDV_OK;
}

sdv_status sdv_pool_insert(const sdv_pool* pool, const int32_t* draft, int32_t len, int32_t* err, void* stream) {
  PoolArgs a;
  sdv_status st = pool_args(pool, &a);
  if (st != SDV_OK) return st;
  if (!draft) return fail(SDV_ERR_NULL, "draft is NULL");
  if (len < 1 || len > pool->capacity) return fail(SDV_ERR_SHAPE, "draft length %d", len);
  a.draft = draft;
  a.len = len;
  a.err = err;
  SDV_LAUNCH(launch_pool_insert(a, (hipStream_t)stream));
  return SDV_OK;
}

sdv_status sdv_pool_lookup(const sdv_pool* pool, int32_t batch, const int32_t* suffix, const int32_t* suffix_len,
                           int32_t suffix_cap, int32_t max_out, int32_t* cont, int32_t* cont_len, int32_t* match_n,
                           void* stream) {
  PoolArgs pa;
  sdv_status st = pool_args(pool, &pa);
  if (st != SDV_OK) return st;
  if (!suffix || !suffix_len || !cont || !cont_len) return fail(SDV_ERR_NULL, "NULL argument");
  if (batch < 1 || suffix_cap < 1 || max_out < 1) return fail(SDV_ERR_SHAPE, "batch/suffix_cap/max_out out of range");
  PoolLookupArgs a{pa.tokens, pa.seg_end, pa.keys, pa.vals, pa.count, pa.n_slots, pa.max_n, batch, suffix, suffix_len,
                   suffix_cap, max_out, cont, cont_len, match_n};
  SDV_LAUNCH(launch_pool_lookup(a, (hipStream_t)stream));
  return SDV_OK;
}

namespace {

sdv_status stream_cfg(const sdv_stream_cfg* c, StreamCfgDev* d) {
  if (!c) return fail(SDV_ERR_NULL, "stream cfg is NULL");
  if (c->n_codebooks < 1 || c->codebook_size < 2 || c->codebook_base < 0 || c->text_end < 0 ||
      c->text_end > c->codebook_base || c->max_frames < 1)
    return fail(SDV_ERR_SHAPE, "stream cfg sizes out of range");
  if (c->eoa_code < 0 || c->eoa_code >= c->codebook_size || c->pad_code < 0 || c->pad_code >= c->codebook_size)
    return fail(SDV_ERR_SHAPE, "end-of-audio / pad code outside the codebook");
  if (c->n_bridge < 0 || (c->n_bridge > 0 && !c->bridge)) return fail(SDV_ERR_NULL, "bridge tokens NULL");
  *d = StreamCfgDev{c->n_codebooks, c->codebook_size, c->codebook_base, c->text_end, c->eoa_code, c->pad_code,
                    c->n_bridge, c->max_frames, c->bridge};
  return SDV_OK;
}

}  // namespace

sdv_status sdv_phase_mask(const sdv_stream_cfg* cfg, int32_t batch, int32_t R, const float* logits,
                          int64_t row_stride, int32_t id_offset, int32_t n_ids, const int32_t* depth,
                          const sdv_stream_state* state, int32_t* argmax_out, int32_t* modality_out, void* stream) {
  PhaseMaskArgs a;
  sdv_status st = stream_cfg(cfg, &a.cfg);
  if (st != SDV_OK) return st;
  if (!logits || !depth || !state || !state->phase || !state->phase_pos || !argmax_out)
    return fail(SDV_ERR_NULL, "NULL argument");
  if (batch < 1 || R < 1 || n_ids < 1 || id_offset < 0 || row_stride < n_ids) return fail(SDV_ERR_SHAPE, "sizes out of range");
  a.B = batch;
  a.R = R;
  a.logits = logits;
  a.row_stride = row_stride;
  a.id_offset = id_offset;
  a.n_ids = n_ids;
  a.depth = depth;
  a.phase = state->phase;
  a.phase_pos = state->phase_pos;
  a.argmax_out = argmax_out;
  a.modality_out = modality_out;
  SDV_LAUNCH(launch_phase_mask(a, (hipStream_t)stream));
  return SDV_OK;
}

sdv_status sdv_stream_commit(const sdv_stream_cfg* cfg, int32_t batch, int32_t T, int32_t L_a, int32_t R,
                             const int32_t* tokens, const int32_t* logit_rows, const int32_t* n_acc,
                             const int32_t* next, const int32_t* path, const int32_t* cb_argmax,
                             const int32_t* modality, const sdv_stream_state* state, void* stream) {
  StreamCommitArgs a;
  sdv_status st = stream_cfg(cfg, &a.cfg);
  if (st != SDV_OK) return st;
  if (!tokens || !logit_rows || !n_acc || !next || !path || !state) return fail(SDV_ERR_NULL, "NULL argument");
  if (!state->phase || !state->phase_pos || !state->step || !state->frames || !state->matrix)
    return fail(SDV_ERR_NULL, "stream state pointer NULL");
  if (batch < 1 || T < 1 || T > SDV_MAX_T || R < 1 || R > T || L_a < 1 || L_a > T)
    return fail(SDV_ERR_SHAPE, "B/T/R/L_a out of range");
  a.B = batch;
  a.T = T;
  a.L_a = L_a;
  a.R = R;
  a.tokens = tokens;
  a.logit_rows = logit_rows;
  a.n = n_acc;
  a.next = next;
  a.path = path;
  a.cb_argmax = cb_argmax;
  a.modality = modality;
  a.phase = state->phase;
  a.phase_pos = state->phase_pos;
  a.step = state->step;
  a.frames = state->frames;
  a.matrix = state->matrix;
  SDV_LAUNCH(launch_stream_commit(a, (hipStream_t)stream));
  return SDV_OK;
}

sdv_status sdv_philox_uniforms(uint64_t seed, const int32_t* seq_ids, int32_t B, int32_t n_pos, double* u0_out,
                               double* u1_out, void* stream) {
  if (!u0_out && !u1_out) return fail(SDV_ERR_NULL, "both outputs are NULL");
  if (B < 1 || n_pos < 1) return fail(SDV_ERR_SHAPE, "B/n_pos out of range");
  PhiloxArgs a{seed, seq_ids, B, n_pos, u0_out, u1_out};
  SDV_LAUNCH(launch_philox_uniforms(a, (hipStream_t)stream));
  return SDV_OK;
}

}  // extern "C"
