"""Benchmark of the single-forward verify step on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  kv_rollback(C)  ->  verify_forward([audio chunk ; drafts])  ->  accept_greedy  ->
  kv_rollback(C + L_a + n)
(the speculative-sampling workload times accept_sample alone).  Inputs are resident
in HBM before timing.  Prints ONE JSON line.

By default every workload runs, largest first: the batched multi-codebook pass (32
sessions x guidance pairs on the 8B backbone) carries the headline value, and the
8B tree pass, the 1.7B pass, the sampling acceptance and the toy fp32 pass follow as
sub-objects of the same line (`configs`), each with the roofline of its dominant
kernel (timed live with HIP events the library records on its launch stream), the
roofline of the whole pass and the CPU oracle timed on a bounded sample.

  python bench.py [--gpus 1] [--steps K] [--warmup W]
                  [--workload all|c5-codebook|8b-bf16-tree|1.7b-bf16|toy-f32|sample]
                  [--scenario silence|random] [--graph] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
MFMA_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, TFLOP/s
MFMA_F32_TFLOPS = 157.3    # MI355X fp32 (the fp32 model's matrix work runs at this rate at best)
METRIC = "verified tokens/s per verify pass (chunk+draft) at 1 GPU; % of HBM roofline"

# -- stored HBM traffic of dominant kernels -------------------------------------------
# From two rocprofv3 counter runs of the same bench command (FETCH_SIZE, then WRITE_SIZE,
# KiB per dispatch averaged over the kernel's dispatches), each scaled by what the same
# counter reads for a plain 256 MiB device copy (`bench.py --copy-calibration`: FETCH_SIZE
# reads 131,084 KiB for 262,144 KiB copied, factor 2.000; WRITE_SIZE reads 262,144 KiB,
# factor 1.000).  An entry counts only for its workload and kernel and while the sha256
# of the kernel's sources is the one it was taken on; otherwise traffic is null.
FETCH_FACTOR = 262144.0 / 131084.0
WRITE_FACTOR = 1.0
GEMM_SOURCES = ("speculative_decoding_verify_amd/csrc/gemm.hip", "speculative_decoding_verify_amd/csrc/common.h",
                "speculative_decoding_verify_amd/csrc/kernels.h")
ATTN_SOURCES = ("speculative_decoding_verify_amd/csrc/attention.hip", "speculative_decoding_verify_amd/csrc/common.h",
                "speculative_decoding_verify_amd/csrc/kernels.h")
SAMPLE_SOURCES = ("speculative_decoding_verify_amd/csrc/accept.hip", "speculative_decoding_verify_amd/csrc/common.h",
                  "speculative_decoding_verify_amd/csrc/kernels.h")
KERNEL_SOURCES = {"qkv": GEMM_SOURCES, "o": GEMM_SOURCES, "gate_up": GEMM_SOURCES, "down": GEMM_SOURCES,
                  "lm_head": GEMM_SOURCES, "codebook_head": GEMM_SOURCES, "attention": ATTN_SOURCES,
                  "row_stats": SAMPLE_SOURCES}
TRAFFIC = [
    # rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE, on `bench.py --workload <w> --steps 2
    # --warmup 1 --no-cpu-baseline` (--no-drafting for the single-sequence passes);
    # means over every dispatch of the kernel; a kind of two kernels sums both
    {"workload": "c5-codebook", "kernel": "attention",   # sdv::attn_dma<128, 1, 4, 3>, 216 dispatches
     "sha256": "202be0ec9a006cc92dd0a041f3778f24e3f5d77b238d18c2da8ad17aac80500f",
     "fetch_kib": 1824697.22, "write_kib": 250554.12},
    # gate/up on the 8B shape is two kernels: sdv::gemm_wide<bf16, 5, 3, 3, PARTIAL> (the
    # gate/up half of that instance's 360 dispatches; the other half is q/k/v) and
    # sdv::gemm_finish<bf16, 5, 2, SWIGLU, 4> (180 dispatches)
    {"workload": "8b-bf16", "kernel": "gate_up",
     "sha256": "68255c2adf92e34f0c9cb1ba0a4d306a4b147dd9fffa684b27a8fc585321d7a5",
     "fetch_kib": 103018.57 + 6255.50, "write_kib": 12480.0 + 3168.0},
    {"workload": "1.7b-bf16", "kernel": "gate_up",       # sdv::gemm_stream<bf16, 3, 4, 2, SWIGLU>, 120 dispatches
     "sha256": "68255c2adf92e34f0c9cb1ba0a4d306a4b147dd9fffa684b27a8fc585321d7a5",
     "fetch_kib": 34376.60, "write_kib": 1344.0},
    {"workload": "toy-f32", "kernel": "attention",       # sdv::attn_reg<float, 64, 2>, 10 dispatches
     "sha256": "202be0ec9a006cc92dd0a041f3778f24e3f5d77b238d18c2da8ad17aac80500f",
     "fetch_kib": 890.11, "write_kib": 583.13},
    {"workload": "sample", "kernel": "row_stats",        # sdv::spec_row_stats_kernel, 5 dispatches
     "sha256": "4bee3d41264a24db90d895fc36caa70c5105b66d46e8d082e43ae4b4f01e1f82",
     "fetch_kib": 284938.81, "write_kib": 60.00},
]


def source_sha(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counter_traffic(entry, workload, kernel):
    """HBM bytes per launch from a stored counter reading, or None when the entry is for
    another workload or kernel or the kernel's sources have changed since."""
    if not entry or entry["workload"] != workload or entry["kernel"] != kernel:
        return None
    if entry["sha256"] != source_sha(KERNEL_SOURCES[kernel]):
        return None
    return (entry["fetch_kib"] * FETCH_FACTOR + entry["write_kib"] * WRITE_FACTOR) * 1024.0


def stored_traffic(workload, kernel):
    for e in TRAFFIC:
        t = counter_traffic(e, workload, kernel)
        if t is not None:
            return t
    return None


# -- host description for the CPU baselines --------------------------------------------

def host_info():
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        pass
    return {"cores": cores, "cpu_model": model, "blas_threads": blas}


def cpu_record(value, unit, sample):
    h = host_info()
    return {"value": value, "unit": unit, "cores": h["cores"], "kind": "oracle", "sample": sample,
            "cpu_model": h["cpu_model"], "blas_threads": h["blas_threads"]}


# -- algorithmic work of a verify pass ---------------------------------------------------

def pass_bytes(sh, T, R, ctx, head_rows=None, head_cols=None):
    """Algorithmic HBM bytes of one verify pass: every weight read once (embedding: the
    gathered rows), KV read (the cached rows), KV written (the chunk rows), fp32 logits of
    the rows acceptance needs.  ctx: cached length per sequence.  head_rows / head_cols:
    the logit matrix (default R rows per sequence over the full vocabulary)."""
    eb = sh.elem_bytes
    B = len(ctx)
    head_cols = sh.vocab if head_cols is None else head_cols
    head_rows = B * R if head_rows is None else head_rows
    w = sh.n_layers * (sh.layer_params() - 2 * sh.d) * eb + head_cols * sh.d * eb
    w += sh.n_layers * 2 * sh.d * 4 + sh.d * 4          # fp32 norm gains
    w += B * T * sh.d * eb                               # gathered embedding rows
    kv_row = sh.n_layers * 2 * sh.kv_dim * eb
    return w + sum(ctx) * kv_row + B * T * kv_row + head_rows * head_cols * 4


def attn_visible_keys(T, C, parent):
    """sum over chunk rows j of the keys row j attends to: C cached + its ancestors-or-self."""
    depth = np.zeros(T, dtype=np.int64)
    for j in range(1, T):
        depth[j] = depth[parent[j] if parent is not None else j - 1] + 1
    return int(T * C + (depth + 1).sum())


def launch_work(sh, B, T, R, ctx, parent, head="lm"):
    """Algorithmic bytes and FLOPs of one launch of each kernel kind (per layer for the
    decoder kinds): weights read once, activation rows in and out at 4 bytes per value
    (the bf16 hi/lo pair or fp32), K/V read once per (sequence, kv head)."""
    eb = sh.elem_bytes
    d, F, H, Hkv, dh = sh.d, sh.ffn, sh.n_heads, sh.n_kv_heads, sh.head_dim
    M, Mr = B * T, B * R
    qd, kd = H * dh, Hkv * dh
    work = {
        "qkv": (( qd + 2 * kd) * d * eb + M * d * 4 + M * qd * 4 + M * 2 * kd * eb, 2.0 * M * (qd + 2 * kd) * d),
        "attention": (sum(C + T for C in ctx) * 2 * kd * eb + 2 * M * qd * 4,
                      4.0 * H * dh * sum(attn_visible_keys(T, C, parent) for C in ctx)),
        "o": (d * qd * eb + M * qd * 4 + M * d * 4, 2.0 * M * d * qd),
        "gate_up": (2 * F * d * eb + M * d * 4 + M * F * 4, 2.0 * M * 2 * F * d),
        "down": (d * F * eb + M * F * 4 + M * d * 4, 2.0 * M * d * F),
    }
    if head == "lm":
        work["lm_head"] = (sh.vocab * d * eb + Mr * d * 4 + Mr * sh.vocab * 4, 2.0 * Mr * sh.vocab * d)
    else:
        S, Vc = sh.n_codebooks, sh.codebook_size
        work["codebook_head"] = (Vc * d * eb + (Mr + S) * d * 4 + (Mr + S) * Vc * 4, 2.0 * (Mr + S) * Vc * d)
    return work


def mfma_peak(sh):
    return MFMA_BF16_TFLOPS if sh.dtype == "bf16" else MFMA_F32_TFLOPS


def roofline_of(kind, nbytes, flops, us, sh, workload, launches):
    """Roofline of one kernel kind from its algorithmic bytes and FLOPs per launch and
    its average launch duration: bound by HBM when its arithmetic intensity is below
    the ridge (peak FLOP/s over peak bytes/s), by the matrix cores otherwise."""
    peak_tf = mfma_peak(sh)
    ridge = peak_tf * 1e12 / (HBM_PEAK_GBS * 1e9)
    if flops / nbytes > ridge:
        achieved = flops / (us * 1e-6) / 1e12
        r = {"bound": "mfma", "achieved": achieved, "peak": peak_tf, "unit": "TFLOP/s", "frac": achieved / peak_tf}
    else:
        achieved = nbytes / (us * 1e-6) / 1e9
        r = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": achieved / HBM_PEAK_GBS}
    r.update({"traffic": stored_traffic(workload, kind), "kernel": kind, "bytes_per_launch": int(nbytes),
              "flops_per_launch": flops, "avg_launch_us": us, "launches_per_pass": launches})
    return r


GEMM_KINDS = ("qkv", "o", "gate_up", "down")


def live_kernel_times(sdv, ver, sh, step, steps, head_kind):
    """Average launch duration (us) of each kernel kind over `steps` passes, from HIP
    events the library records on the launch stream around each GEMM launch and each
    layer's attention."""
    import torch
    L = sh.n_layers
    n_gemm = 4 * L + 1
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_gemm)]
    aev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * L)]
    ver.set_profile_events(ev, aev)
    g, a = [], []
    for _ in range(steps):
        step()
        torch.cuda.synchronize()
        g.append([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(n_gemm)])
        a.append([aev[2 * i].elapsed_time(aev[2 * i + 1]) for i in range(L)])
    ver.set_profile_events(None)
    g = np.asarray(g) * 1e3
    a = np.asarray(a) * 1e3
    per_layer = g[:, :4 * L].reshape(steps, L, 4)
    us = {k: float(per_layer[:, :, i].mean()) for i, k in enumerate(GEMM_KINDS)}
    us["attention"] = float(a.mean())
    us[head_kind] = float(g[:, -1].mean())
    return us


def kernel_table(sh, us, work, workload, head_kind):
    """Roofline of every kernel kind plus the dominant one (largest time per pass)."""
    L = sh.n_layers
    table = {}
    for kind, t in us.items():
        nb, fl = work[kind]
        table[kind] = roofline_of(kind, nb, fl, t, sh, workload, 1 if kind == head_kind else L)
    dom = max(table, key=lambda k: table[k]["avg_launch_us"] * table[k]["launches_per_pass"])
    return table, dom


def timed_steps(step, steps, warmup):
    """Mean ms per step over `steps` steps between two host synchronisations, and the
    distribution of single steps (median, p10, p90 in ms) over as many more steps, each
    between two HIP events on the launch stream (torch's current stream).  The events
    stay out of the timed region: a marker between steps adds a few us to a small one."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    return ms, step_distribution([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])


def step_distribution(per_step_ms):
    t = np.asarray(per_step_ms, dtype=np.float64)
    return {"median": float(np.median(t)), "p10": float(np.percentile(t, 10)), "p90": float(np.percentile(t, 90)),
            "n": int(t.size)}


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# -- drafting (untimed set-up) ----------------------------------------------------------

def draft_under_silence(sdv, model, kv, C, L_a, gamma, silence_id=0, n_branch=0, reps=0):
    """Greedy drafting on the GPU path: sdv_draft_tree with the chunk under silence gives
    the main draft (gamma tokens) and, with n_branch > 0, the runner-up branch (the
    second-best first token continued greedily).  The cache is left at C.  With reps > 0
    the call is also timed (median of reps calls)."""
    import torch
    lens = [gamma] + ([n_branch] if n_branch else [])
    drafter = sdv.Drafter(model, kv, L_a, lens, max_ctx=C)
    drafter.set_chunk(np.full((kv.batch, L_a), silence_id, dtype=np.int32))
    out = drafter.run()
    torch.cuda.synchronize()
    d = out["drafts"].cpu().numpy()[0]
    main = [int(x) for x in d[0, :gamma]]
    branch = [int(x) for x in d[1, :n_branch]] if n_branch else []
    timing = None
    if reps:
        times = []
        for _ in range(reps):
            t0 = time.perf_counter()
            drafter.run()
            torch.cuda.synchronize()
            times.append(time.perf_counter() - t0)
        ms = float(np.median(times)) * 1e3
        # every pass streams all weights and reads the cache: pass 0 the L_a chunk rows,
        # pass s the root plus s rows of each branch longer than s
        sh = model.shape
        passes = [(L_a, 1, C)] + [(1 + s * sum(1 for n in lens if n > s), sum(1 for n in lens if n > s), C + L_a - 1)
                                  for s in range(1, max(lens))]
        nbytes = sum(pass_bytes(sh, T, R, [c]) for T, R, c in passes)
        timing = {"ms": ms, "passes": len(passes), "draft_tokens": sum(lens), "tokens_per_s": sum(lens) / ms * 1e3,
                  "chunk_budget_frac": ms / 1000.0,
                  "note": "sdv_draft_tree under a silent chunk: one verify forward per draft position, the branches "
                          "as a tree under the chunk's last row; chunk_budget_frac = time / the 1 s chunk",
                  "roofline": {"bound": "hbm", "bytes": nbytes, "achieved_GBs": nbytes / (ms * 1e-3) / 1e9,
                               "peak_GBs": HBM_PEAK_GBS, "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}}
    return main, branch, timing


# -- the single-sequence verify workloads (toy, 1.7B, 8B tree) ----------------------------

def bench_verify(args, wl, w=None, model=None):
    import torch
    import speculative_decoding_verify_amd as sdv
    from synth import make_weights, make_random_kv, uniform_tokens

    sh = wl.shape if w is None else w.shape
    C = wl.ctx[0]
    T, L_a, gamma = wl.T, wl.L_a, wl.gamma
    t0 = time.time()
    if w is None:
        w = make_weights(sh, seed=wl.seed)
    if model is None:
        model = sdv.DeviceModel(w)
    kv_host = None if wl.kv_init == "prefill" else make_random_kv(sh, [C], capacity=C + T, seed=wl.seed + 1000)
    kv = sdv.PagedKV(sh, 1, C + T + 64)
    if kv_host is not None:
        kv.load(kv_host)
    else:
        # prefill the context through the model itself (chunks of 128 rows)
        sdv.prefill(model, kv, uniform_tokens(C, sh.vocab, wl.seed + 2000, "ctx")[None, :])
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    if args.no_drafting:
        # uniform draft tokens: the verify pass has the same shapes and kernels
        drafts = uniform_tokens(gamma, sh.vocab, wl.seed + 5000, "draft")
        branch = uniform_tokens(wl.n_branch, sh.vocab, wl.seed + 5001, "branch") if wl.n_branch else []
        drafting = None
    else:
        drafts, branch, drafting = draft_under_silence(sdv, model, kv, C, L_a, gamma, wl.silence_id, wl.n_branch,
                                                       reps=5)
    parent = wl.parent()
    audio = np.full(L_a, wl.silence_id, dtype=np.int32) if args.scenario == "silence" else \
        uniform_tokens(L_a, sh.vocab, wl.seed + 4000, "audio")
    tokens = np.concatenate([audio, np.asarray(drafts, np.int32), np.asarray(branch, np.int32)]).astype(np.int32)
    rows = wl.logit_rows()
    R = len(rows)
    ver = sdv.Verifier(model, kv, T, L_a, rows, parent=parent, max_ctx=C, want_logits=True)
    ver.set_tokens(tokens[None, :])
    keep_c = torch.tensor([C], dtype=torch.int32, device="cuda")
    acc_out = None

    def step(stream=None):
        nonlocal acc_out
        sdv.kv_rollback(model, kv, keep_c, stream=stream)
        res = ver.forward(stream)
        acc_out = sdv.accept_greedy(1, T, L_a, ver.tokens, ver.parent, ver.logit_rows, res.argmax,
                                    base_len=kv.seq_len, out=acc_out, stream=stream)
        sdv.kv_rollback(model, kv, acc_out["keep"], acc_out["move_src"], acc_out["move_dst"], acc_out["err"],
                        stream=stream)

    graph = None
    if args.graph:
        for _ in range(max(1, args.warmup)):
            step()
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
    ms, dist = timed_steps(graph.replay if graph is not None else step, args.steps, args.warmup)
    n_acc = int(acc_out["n"][0])
    assert int(acc_out["err"][0]) == 0 and int(ver.err[0]) == 0, "device error during bench"

    us = live_kernel_times(sdv, ver, sh, step, args.steps, "lm_head")
    # the other scenario's committed count: one more pass of the same shapes (so the same
    # passes/s) with the chunk's audio swapped between silence and uniform random ids
    committed = {args.scenario: n_acc + 1}
    other = "random" if args.scenario == "silence" else "silence"
    audio_o = np.full(L_a, wl.silence_id, dtype=np.int32) if other == "silence" else \
        uniform_tokens(L_a, sh.vocab, wl.seed + 4000, "audio")
    ver.set_tokens(np.concatenate([audio_o, tokens[L_a:]]).astype(np.int32)[None, :])
    step()
    torch.cuda.synchronize()
    assert int(acc_out["err"][0]) == 0 and int(ver.err[0]) == 0, "device error during bench"
    committed[other] = int(acc_out["n"][0]) + 1
    ver.set_tokens(tokens[None, :])
    work = launch_work(sh, 1, T, R, [C], parent, "lm")
    table, dom = kernel_table(sh, us, work, wl.shape.name, "lm_head")
    nbytes = pass_bytes(sh, T, R, [C])
    flops = sum(fl * (1 if k == "lm_head" else sh.n_layers) for k, (nb, fl) in work.items())
    passes_s = 1e3 / ms
    out = {
        "metric": METRIC,
        "value": T * passes_s,
        "unit": "verified tokens/s",
        "ms_per_step": ms,
        "per_step_ms": dist,
        "dtype": "bf16" if sh.dtype == "bf16" else "f32",
        "config": {"workload": f"{wl.shape.name} verify: {sh.n_layers} layers d={sh.d} {sh.n_heads}x{sh.head_dim} "
                               f"q heads / {sh.n_kv_heads} kv heads FFN {sh.ffn} V={sh.vocab}; C={C}; "
                               f"{L_a} audio + {gamma} drafts" + (f" + {wl.n_branch}-token branch (tree mask)"
                                                                  if wl.n_branch else ""),
                   "batch": 1, "T": T, "R": R, "context": C, "scenario": args.scenario,
                   "graph": bool(args.graph)},
        "passes_per_s": passes_s,
        "committed_tokens_per_pass": n_acc + 1,
        "committed_tokens_per_s": (n_acc + 1) * passes_s,
        "committed_by_scenario": {k: {"per_pass": v, "per_s": v * passes_s} for k, v in committed.items()},
        "roofline": table[dom],
        "pass_roofline": {"bound": "hbm", "bytes": nbytes, "achieved_GBs": nbytes / (ms * 1e-3) / 1e9,
                          "peak_GBs": HBM_PEAK_GBS, "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                          "flops": flops, "mfma_frac": flops / (ms * 1e-3) / 1e12 / mfma_peak(sh)},
        "kernels": {k: {"avg_launch_us": v["avg_launch_us"], "launches_per_pass": v["launches_per_pass"],
                        "bound": v["bound"], "frac": v["frac"]} for k, v in table.items()},
        "drafting": drafting,
        "setup_s": setup_s,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_verify(w, kv_host, wl, sh, tokens, parent, rows, T)
    return out


def cpu_baseline_verify(w, kv_host, wl, sh, tokens, parent, rows, T):
    """The oracle (fp64 NumPy; bf16 rounding mode for bf16 models) timed on the host: full
    passes (verify + greedy acceptance + commit plan) of the same workload, repeated
    until about 10 s of CPU time (at least one pass, at most 20)."""
    from oracle import BF16_KV, EXACT
    from oracle import accept as oacc
    from oracle import decoder as odec
    from synth import make_random_kv
    C = wl.ctx[0]
    if kv_host is None:  # prefilled context: synthetic KV of the same shape for the timing sample
        kv_host = make_random_kv(sh, [C], capacity=C + T, seed=wl.seed + 1000)
    mode = BF16_KV if sh.dtype == "bf16" else EXACT
    cache = odec.Cache(kv_host.k, kv_host.v)
    times = []
    while True:
        t0 = time.perf_counter()
        res = odec.verify_forward(w, cache, tokens[None, :], parent, rows, mode)
        am = [oacc.argmax_lowest(r) for r in res["logits"][0]]
        n, nxt, path = oacc.accept_greedy(list(tokens), parent, wl.L_a, rows, am)
        oacc.commit_plan(C, wl.L_a, path)
        times.append(time.perf_counter() - t0)
        if sum(times) > 10.0 or len(times) >= 20:
            break
    dt = float(np.median(times))
    return cpu_record(T / dt, "verified tokens/s",
                      f"{len(times)} full verify pass(es) of the same workload (median {dt:.3f} s), fp64 oracle "
                      f"({mode} mode)")


# -- the batched multi-codebook workload --------------------------------------------------

def bench_c5(args, wl, w=None, model=None):
    """Batched multi-codebook verify: 32 sessions x (conditional, unconditional) rows on
    the 8B-shape backbone with 8 codebook heads, guidance w = 2, acceptance on codebook 0.
    One step = kv_rollback(C) -> verify_forward -> accept_greedy -> kv_rollback."""
    import torch
    import speculative_decoding_verify_amd as sdv
    from synth import HashedKV, make_weights, page_table, uniform_tokens
    sh = wl.shape
    B, T, L_a = wl.batch, wl.T, wl.L_a
    S, Vc = sh.n_codebooks, sh.codebook_size
    base = sh.vocab - S * Vc
    ctx = list(wl.ctx)
    t0 = time.time()
    if w is None:
        w = make_weights(sh, seed=wl.seed)
    if model is None:
        model = sdv.DeviceModel(w)
    table, n_blocks = page_table(ctx, T + 16, 16, seed=wl.seed + 7)
    kv = sdv.PagedKV(sh, B, 0, table=table, n_blocks=n_blocks)
    kv_seed = wl.seed + 1000
    kv.load(HashedKV(sh, ctx, 0, seed=kv_seed, device=kv.device))
    tokens = np.empty((B, T), dtype=np.int32)
    for s_ in range(B // 2):   # uniform codes; both rows of a session get the same ids
        tokens[2 * s_] = tokens[2 * s_ + 1] = base + uniform_tokens(T, Vc, wl.seed * 1000 + s_, "c5codes") - 1
    rows = wl.logit_rows()
    R = len(rows)
    ver = sdv.Verifier(model, kv, T, L_a, rows, max_ctx=max(ctx), want_logits=False, head=sdv.HEAD_CODEBOOK,
                       cfg_partner=[b ^ 1 for b in range(B)], cfg_w=wl.cfg_w)
    ver.set_tokens(tokens)
    keep_c = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    setup_s = time.time() - t0
    acc_out = None

    def step():
        nonlocal acc_out
        sdv.kv_rollback(model, kv, keep_c)
        res = ver.forward()
        acc_out = sdv.accept_greedy(B, T, L_a, ver.tokens, None, ver.logit_rows, res.argmax, base_len=kv.seq_len,
                                    out=acc_out)
        sdv.kv_rollback(model, kv, acc_out["keep"], acc_out["move_src"], acc_out["move_dst"], acc_out["err"])

    ms, dist = timed_steps(step, args.steps, args.warmup)
    assert int(acc_out["err"].abs().sum()) == 0 and int(ver.err.abs().sum()) == 0, "device error during bench"
    us = live_kernel_times(sdv, ver, sh, step, max(3, args.steps // 4), "codebook_head")
    work = launch_work(sh, B, T, R, ctx, None, "codebook")
    ktable, dom = kernel_table(sh, us, work, "c5-codebook", "codebook_head")
    M = B * T
    nbytes = pass_bytes(sh, T, R, ctx, head_rows=B * R * S, head_cols=Vc)
    flops = sum(fl * (1 if k == "codebook_head" else sh.n_layers) for k, (nb, fl) in work.items())
    passes_s = 1e3 / ms
    n_acc = acc_out["n"].cpu().numpy()
    del kv
    out = {
        "metric": METRIC, "value": (B // 2) * T * passes_s, "unit": "verified session tokens/s",
        "ms_per_step": ms, "per_step_ms": dist, "dtype": "bf16",
        "config": {"workload": f"batched multi-codebook verify: {B // 2} sessions x 2 guidance rows, 8B-shape "
                               f"backbone, {S} codebooks x {Vc}, contexts {min(ctx)}..{max(ctx)}, "
                               f"{L_a} audio + {wl.gamma} drafts, w={wl.cfg_w}",
                   "rows": B, "T": T, "R": R, "cached_tokens": sum(ctx)},
        "passes_per_s": passes_s, "row_tokens_per_s": B * T * passes_s,
        "committed_tokens_per_pass": int((n_acc + 1).sum()) // 2,
        "roofline": ktable[dom],
        "pass_roofline": {"bound": "mfma", "bytes": nbytes, "achieved_GBs": nbytes / (ms * 1e-3) / 1e9,
                          "peak_GBs": HBM_PEAK_GBS, "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                          "flops": flops, "mfma_frac": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_TFLOPS,
                          "note": "the pass is MFMA-bound (HBM roof 12.7 ms < MFMA roof 20.3 ms): frac is the "
                                  "HBM fraction, mfma_frac the matrix-core fraction"},
        "kernels": {k: {"avg_launch_us": v["avg_launch_us"], "launches_per_pass": v["launches_per_pass"],
                        "bound": v["bound"], "frac": v["frac"]} for k, v in ktable.items()},
        "setup_s": setup_s,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_c5(w, wl, tokens, rows, kv_seed, work_per_row=_c5_row_flops(sh, T, ctx))
    return out


def _c5_row_flops(sh, T, ctx):
    """Oracle work per row of the batched pass: decoder GEMMs (same for every row) plus
    attention over its own cached length, in FLOPs."""
    gemm = 2.0 * T * (sh.n_layers * (sh.layer_params() - 2 * sh.d))
    attn = [4.0 * sh.n_layers * sh.n_heads * sh.head_dim * attn_visible_keys(T, C, None) for C in ctx]
    return [gemm + a for a in attn]


def cpu_baseline_c5(w, wl, tokens, rows, kv_seed, work_per_row):
    """The oracle (cfg.verify_codebook, BF16_KV mode) on one guidance pair, the session
    with the shortest context, timed on the host (verify + merge + greedy acceptance);
    the time of the whole 64-row pass is extrapolated linearly in the rows' FLOPs."""
    from oracle import BF16_KV
    from oracle import accept as oacc
    from oracle import cfg
    from oracle import decoder as odec
    from synth import HashedKV
    sh = wl.shape
    ctx = list(wl.ctx)
    S, Vc = sh.n_codebooks, sh.codebook_size
    base = sh.vocab - S * Vc
    s = min(range(len(ctx) // 2), key=lambda i: ctx[2 * i])
    r2 = [2 * s, 2 * s + 1]
    hk = HashedKV(sh, [ctx[b] for b in r2], 0, seed=kv_seed, streams=r2)
    cache = odec.Cache([[hk.block(i, l, 0) for l in range(sh.n_layers)] for i in range(2)],
                       [[hk.block(i, l, 1) for l in range(sh.n_layers)] for i in range(2)])
    t0 = time.perf_counter()
    o = cfg.verify_codebook(w, cache, tokens[r2], None, rows, [1, 0], wl.cfg_w, base, BF16_KV)
    for i in range(2):
        oacc.accept_greedy(list(tokens[r2[i]]), None, wl.L_a, rows, list(o["token"][i]))
    dt = time.perf_counter() - t0
    scale = sum(work_per_row) / (work_per_row[r2[0]] + work_per_row[r2[1]])
    pass_s = dt * scale
    B, T = wl.batch, wl.T
    return cpu_record((B // 2) * T / pass_s, "verified session tokens/s",
                      f"1 guidance pair (session {s}, context {ctx[2 * s]}) of the same pass in {dt:.1f} s, fp64 "
                      f"oracle (bf16-kv mode); the 64-row pass extrapolated linearly in the rows' FLOPs "
                      f"(x{scale:.1f}: {pass_s:.0f} s per pass)")


# -- speculative-sampling acceptance ------------------------------------------------------

def bench_sample(args):
    import torch
    import speculative_decoding_verify_amd as sdv
    from synth import SAMPLE_FULL, make_sample_inputs
    wl = SAMPLE_FULL
    t0 = time.time()
    si = make_sample_inputs(wl)
    B, k, V = wl.batch, wl.k, wl.vocab
    # two resident copies of the inputs, alternated, so consecutive steps do not hit
    # the 256 MB last-level cache with the previous step's data
    copies = [dict(tgt=torch.from_numpy(si.target_logits).cuda(), drf=torch.from_numpy(si.draft_logits).cuda(),
                   drafts=torch.from_numpy(si.drafts).cuda()) for _ in range(2)]
    smp = sdv.Sampler(B, k, V)
    setup_s = time.time() - t0
    it = [0]

    def step():
        c = copies[it[0] & 1]
        it[0] += 1
        smp(c["tgt"], c["drf"], c["drafts"], si.seed)

    ms, dist = timed_steps(step, args.steps, args.warmup)
    nbytes = si.target_logits.nbytes + si.draft_logits.nbytes
    # live duration of the row-statistics launch (it reads every logit once), from two
    # HIP events the library records on the launch stream, over K more steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    stats_ms = []
    for i in range(args.steps):
        c = copies[i & 1]
        smp(c["tgt"], c["drf"], c["drafts"], si.seed, prof_events=ev)
        torch.cuda.synchronize()
        stats_ms.append(ev[0].elapsed_time(ev[1]))
    stats_us = float(np.mean(stats_ms)) * 1e3
    rows = B * (2 * k + 1)
    stats_bytes = nbytes + rows * (4 + 8)           # logits in; row maximum (fp32) and sum (fp64) out
    achieved = stats_bytes / (stats_us * 1e-6) / 1e9
    out = {
        "metric": METRIC, "value": B * k / (ms * 1e-3), "unit": "draft positions/s", "ms_per_step": ms,
        "per_step_ms": dist, "dtype": "f32",
        "config": {"workload": f"speculative-sampling acceptance: {B} seqs x {k} drafts, V={V}, fp32, "
                               f"Philox4x32-10 uniforms drawn in the kernel"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": stored_traffic("sample", "row_stats"),
                     "kernel": "spec_row_stats_kernel (maximum and exponential sum of every logit row)",
                     "bytes_per_launch": stats_bytes, "avg_launch_us": stats_us, "launches_per_pass": 1},
        "pass_roofline": {"bound": "hbm", "bytes": nbytes, "achieved_GBs": nbytes / (ms * 1e-3) / 1e9,
                          "peak_GBs": HBM_PEAK_GBS, "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "setup_s": setup_s,
    }
    if not args.no_cpu_baseline:
        from oracle import spec_sampling as ss
        tgt64, drf64 = si.target_logits.astype(np.float64), si.draft_logits.astype(np.float64)
        reps, dt = 0, 0.0
        while dt < 10.0 and reps < 100:      # full batches until about 10 s of CPU work
            t0 = time.perf_counter()
            ss.accept_sample(tgt64, drf64, si.drafts, si.u_accept, si.u_sample)
            dt += time.perf_counter() - t0
            reps += 1
        out["cpu_baseline"] = cpu_record(reps * B * k / dt, "draft positions/s",
                                         f"{reps} full batches ({B}x{k}, V={V}) in {dt:.1f} s")
    return out


# -- hypothesis pool ------------------------------------------------------------------

def bench_pool(args, n_drafts=2000, draft_len=32, vocab=151936, B=64, max_n=8, max_out=32):
    """A session's hypothesis pool: n_drafts drafts of draft_len tokens inserted one by
    one, then batches of B longest-suffix lookups (suffixes of 16 tokens, half of them
    ending inside a stored draft)."""
    import torch
    import speculative_decoding_verify_amd as sdv
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([9, 0x9001])))
    drafts = rng.integers(0, vocab, size=(n_drafts, draft_len)).astype(np.int32)
    dev = torch.from_numpy(drafts).cuda()
    pool = sdv.HypothesisPool(capacity=n_drafts * draft_len, n_slots=1 << 20, max_n=max_n)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n_drafts):
        pool.insert(dev[i])
    torch.cuda.synchronize()
    insert_us = (time.perf_counter() - t0) / n_drafts * 1e6
    cap = 16
    suf = rng.integers(0, vocab, size=(B, cap)).astype(np.int32)
    for q in range(0, B, 2):
        d, e = int(rng.integers(0, n_drafts)), int(rng.integers(4, draft_len))
        suf[q, cap - 4:] = drafts[d, e - 4:e]
    suf_t, len_t = torch.from_numpy(suf).cuda(), torch.full((B,), cap, dtype=torch.int32, device="cuda")
    ms, dist = timed_steps(lambda: pool.lookup(suf_t, len_t, max_out), args.steps * 10, args.warmup)
    out = {"workload": f"hypothesis pool: {n_drafts} drafts x {draft_len} tokens indexed by n-grams n <= {max_n}, "
                       f"batches of {B} longest-suffix lookups (continuation <= {max_out})",
           "lookup_batch_us": ms * 1e3, "per_batch_ms": dist, "lookups_per_s": B / (ms * 1e-3), "insert_us_per_draft": insert_us,
           "pool_err": int(pool.err[0])}
    if not args.no_cpu_baseline:
        from oracle.pool import Pool
        op = Pool(max_n)
        for d in drafts:
            op.insert(d)
        t0, n = time.perf_counter(), 0
        while time.perf_counter() - t0 < 5.0 and n < B:
            op.lookup(list(suf[n]), max_out)
            n += 1
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = cpu_record(n / dt, "lookups/s", f"{n} oracle lookups (a scan of every stored position)")
    return out


# -- everything in one line ----------------------------------------------------------------

def bench_all(args):
    """Every workload, largest first.  The 8B backbone (with its codebook heads) is
    generated once and serves the batched pass and the 8B tree pass."""
    import torch
    import speculative_decoding_verify_amd as sdv
    from synth import make_weights
    from synth.configs import WORKLOADS
    c5wl = WORKLOADS["c5-codebook"]()
    t0 = time.time()
    w8 = make_weights(c5wl.shape, seed=c5wl.seed)
    model8 = sdv.DeviceModel(w8)
    _log(f"8B weights ready ({time.time() - t0:.0f} s)")
    head = bench_c5(args, c5wl, w8, model8)
    torch.cuda.empty_cache()
    _log(f"c5-codebook done ({time.time() - t0:.0f} s): {head['ms_per_step']:.2f} ms/pass")
    subs = {}
    subs["8b-bf16-tree"] = bench_verify(args, WORKLOADS["8b-bf16-tree"](), w8, model8)
    _log(f"8b-bf16-tree done ({time.time() - t0:.0f} s): {subs['8b-bf16-tree']['ms_per_step']:.3f} ms/pass")
    del model8, w8
    torch.cuda.empty_cache()
    subs["1.7b-bf16"] = bench_verify(args, WORKLOADS["1.7b-bf16"]())
    _log(f"1.7b-bf16 done ({time.time() - t0:.0f} s): {subs['1.7b-bf16']['ms_per_step']:.3f} ms/pass")
    torch.cuda.empty_cache()
    subs["sample"] = bench_sample(args)
    _log(f"sample done ({time.time() - t0:.0f} s)")
    subs["toy-f32"] = bench_verify(args, WORKLOADS["toy-f32"]())
    _log(f"toy-f32 done ({time.time() - t0:.0f} s)")
    subs["hypothesis-pool"] = bench_pool(args)
    _log(f"hypothesis-pool done ({time.time() - t0:.0f} s)")
    head["configs"] = subs
    head["wall_s"] = time.time() - t0
    return head


def copy_calibration(nbytes=256 << 20, reps=10):
    """A plain device-to-device copy of known size: the reference for scaling the
    FETCH_SIZE / WRITE_SIZE counters of the kernels to bytes."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    return {"copy_bytes": nbytes, "reps": reps, "us_per_copy": dt * 1e6, "GBs": 2 * nbytes / dt / 1e9}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all",
                    choices=["all", "c5-codebook", "8b-bf16-tree", "1.7b-bf16", "toy-f32", "sample"])
    ap.add_argument("--scenario", default="silence", choices=["silence", "random"])
    ap.add_argument("--graph", action="store_true", help="replay the step from a captured HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-drafting", action="store_true",
                    help="verify uniform draft tokens instead of drafting them on the GPU first (same pass shapes; "
                         "for counter runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time a plain 256 MiB device-to-device copy (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "bench.py runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU"}))
        sys.exit(1)
    if args.copy_calibration:
        print(json.dumps(copy_calibration()), flush=True)
        return
    import speculative_decoding_verify_amd as sdv
    sdv.lib()  # fail loudly if the HIP library is not built
    from synth.configs import WORKLOADS
    if args.workload == "all":
        out = bench_all(args)
    elif args.workload == "sample":
        out = bench_sample(args)
    elif args.workload == "c5-codebook":
        out = bench_c5(args, WORKLOADS[args.workload]())
    else:
        out = bench_verify(args, WORKLOADS[args.workload]())
    line = {"metric": out.pop("metric"), "value": out.pop("value"), "unit": out.pop("unit"), "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": out.pop("ms_per_step"),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": out.pop("dtype"),
            "data": "synthetic (seeded N(0,0.02) weights, unit-variance synthetic KV, drafts greedy under silence "
                    "or uniform codes)"}
    line.update(out)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
