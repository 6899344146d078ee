"""Benchmark of the single-forward verify step on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  kv_rollback(C)  ->  verify_forward([audio chunk ; drafts])  ->  accept_greedy  ->
  kv_rollback(C + L_a + n)
(the speculative-sampling workload times accept_sample alone).  Inputs are resident
in HBM before timing.  Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1.7b-bf16|8b-bf16-tree|toy-f32|sample]
                  [--graph] [--no-cpu-baseline]
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

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
METRIC = "verified tokens/s per verify pass (chunk+draft) at 1 GPU; % of HBM roofline"


def pass_bytes(sh, T, R, C, n_branch_rows=0):
    """Algorithmic HBM bytes of one verify pass: every weight read once (embedding:
    the T gathered rows), KV read (C cached rows), KV written (T rows), fp32 logits
    of the R rows acceptance needs."""
    eb = sh.elem_bytes
    w = sh.n_layers * (sh.layer_params() - 2 * sh.d) * eb + sh.vocab * sh.d * eb
    w += sh.n_layers * 2 * sh.d * 4 + sh.d * 4          # fp32 norm gains
    w += T * sh.d * eb                                   # gathered embedding rows
    kv_row = sh.n_layers * 2 * sh.kv_dim * eb
    return w + C * kv_row + T * kv_row + R * sh.vocab * 4


def gate_up_launch_bytes(sh, M):
    """Algorithmic HBM bytes of one gate/up projection launch (the pass's dominant
    kernel): the gate and up weights read once, the M normed rows read (4 bytes per
    value) and the M SwiGLU rows written (4 bytes per value)."""
    return 2 * sh.ffn * sh.d * sh.elem_bytes + M * sh.d * 4 + M * sh.ffn * 4


# HBM traffic of the gate/up kernel from rocprofv3 counters (FETCH_SIZE, then WRITE_SIZE
# in separate runs of `bench.py --steps 5 --warmup 2 --no-cpu-baseline`), per dispatch,
# each scaled by what the same counter reads for a plain 256 MiB device copy
# (`bench.py --copy-calibration`).  Valid only for the workload and the kernel sources
# they were taken on: both are checked at run time, else traffic is null.
GATE_UP_TRAFFIC = {"workload": "1.7b-bf16", "sha256": "1f2e20b165ea0707cce46f9d32e44eb39ca284dd8af7f3b6fb72fb9ac882fa1e",
                   "fetch_kib": 34365.5, "fetch_factor": 262144.0 / 131084.0,
                   "write_kib": 1344.0, "write_factor": 262144.0 / 262144.0}
GEMM_SOURCES = ("speculative_decoding_verify_amd/csrc/gemm.hip", "speculative_decoding_verify_amd/csrc/common.h",
                "speculative_decoding_verify_amd/csrc/kernels.h")


# the same for the row-statistics launch of the speculative-sampling acceptance
# (64 x 7 drafts, V = 151936)
ROW_STATS_TRAFFIC = {"workload": "sample", "sha256": "fbfca9f7a64e4cc888b3ebe1372631ccdd6ee92218f7685a8541ddb198a3834f",
                     "fetch_kib": 284937.3, "fetch_factor": 262144.0 / 131084.0,
                     "write_kib": 60.0, "write_factor": 262144.0 / 262144.0}
SAMPLE_SOURCES = ("speculative_decoding_verify_amd/csrc/accept.hip", "speculative_decoding_verify_amd/csrc/common.h",
                  "speculative_decoding_verify_amd/csrc/kernels.h")


def source_sha(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def gemm_source_sha():
    return source_sha(GEMM_SOURCES)


def counter_traffic(t, workload, files):
    """HBM bytes per launch from stored counter readings, or None once the kernel's
    sources differ from those the counters were taken on."""
    if not t or t["workload"] != workload or t["sha256"] != source_sha(files):
        return None
    return (t["fetch_kib"] * t["fetch_factor"] + t["write_kib"] * t["write_factor"]) * 1024.0


def gate_up_traffic(workload):
    return counter_traffic(GATE_UP_TRAFFIC, workload, GEMM_SOURCES)


def cpu_threads():
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        n = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
        return int(n)
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


def draft_under_silence(sdv, model, kv, C, L_a, gamma, silence_id=0):
    """Greedy drafting on the GPU path (untimed setup): feed L_a silence tokens, then
    decode gamma tokens one at a time; roll the cache back to C afterwards."""
    import torch
    ver = sdv.Verifier(model, kv, L_a, L_a, [L_a - 1], max_ctx=C, want_logits=False)
    ver.set_tokens(np.full((1, L_a), silence_id))
    res = ver.forward()
    keep = torch.tensor([C + L_a], dtype=torch.int32, device="cuda")
    sdv.kv_rollback(model, kv, keep)
    drafts = [int(res.argmax[0, 0])]
    step = sdv.Verifier(model, kv, 1, 1, [0], max_ctx=C + L_a + gamma, want_logits=False)
    for i in range(gamma - 1):
        step.set_tokens(np.array([[drafts[-1]]]))
        r = step.forward()
        keep = torch.tensor([C + L_a + i + 1], dtype=torch.int32, device="cuda")
        sdv.kv_rollback(model, kv, keep)
        drafts.append(int(r.argmax[0, 0]))
    sdv.kv_rollback(model, kv, torch.tensor([C], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    return drafts


def bench_verify(args, wl):
    import torch
    import speculative_decoding_verify_amd as sdv
    from synth import make_weights, make_random_kv, uniform_tokens

    sh = wl.shape
    C = wl.ctx[0]
    T, L_a, gamma = wl.T, wl.L_a, wl.gamma
    t0 = time.time()
    w = make_weights(sh, seed=wl.seed)
    if wl.kv_init == "prefill":
        kv_host = None
    else:
        kv_host = make_random_kv(sh, [C], capacity=C + T, seed=wl.seed + 1000)
    model = sdv.DeviceModel(w)
    kv = sdv.PagedKV(sh, 1, C + T + 64)
    if kv_host is not None:
        kv.load(kv_host)
    else:
        # prefill the context through the model itself (chunks of 128 rows)
        ctx = uniform_tokens(C, sh.vocab, wl.seed + 2000, "ctx")
        done = 0
        while done < C:
            n = min(128, C - done)
            pv = sdv.Verifier(model, kv, n, n, [n - 1], max_ctx=done, want_logits=False)
            pv.set_tokens(ctx[None, done:done + n])
            pv.forward()
            done += n
            sdv.kv_rollback(model, kv, torch.tensor([done], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    # drafts: greedy under silence on the GPU path; main draft + runner-up branch
    drafts = draft_under_silence(sdv, model, kv, C, L_a, gamma, wl.silence_id)
    parent = wl.parent()
    branch = []
    if wl.n_branch:
        # runner-up first token: the second-best token of the first draft position,
        # continued greedily (untimed setup; uses the GPU path's logits)
        ver0 = sdv.Verifier(model, kv, L_a, L_a, [L_a - 1], max_ctx=C, want_logits=True)
        ver0.set_tokens(np.full((1, L_a), wl.silence_id))
        lg = ver0.forward().logits[0, 0].clone()
        lg[drafts[0]] = -float("inf")
        branch = [int(torch.argmax(lg))] + list(uniform_tokens(wl.n_branch - 1, sh.vocab, wl.seed + 3000, "br"))
        sdv.kv_rollback(model, kv, torch.tensor([C], dtype=torch.int32, device="cuda"))
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

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    graph = None
    if args.graph:
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

    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms = elapsed / args.steps * 1e3
    n_acc = int(acc_out["n"][0])
    assert int(acc_out["err"][0]) == 0 and int(ver.err[0]) == 0, "device error during bench"

    # live per-launch timing of the GEMMs with HIP events that the library records on
    # the launch stream around each GEMM launch (per layer: q/k/v, o, gate/up, down;
    # then the LM head), over K more steps of the same pass
    n_gemm = 4 * sh.n_layers + 1
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_gemm)]
    ver.set_profile_events(ev)
    gemm_ms = []
    for _ in range(args.steps):
        step()
        torch.cuda.synchronize()
        per = [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(n_gemm)]
        gemm_ms.append(per)
    ver.set_profile_events(None)
    gemm_ms = np.asarray(gemm_ms)                      # [steps, launches]
    per_layer = gemm_ms[:, :4 * sh.n_layers].reshape(args.steps, sh.n_layers, 4)
    launch_us = {name: float(per_layer[:, :, i].mean()) * 1e3 for i, name in enumerate(("qkv", "o", "gate_up", "down"))}
    launch_us["lm_head"] = float(gemm_ms[:, -1].mean()) * 1e3
    gu_us = launch_us["gate_up"]
    gu_bytes = gate_up_launch_bytes(sh, T)
    achieved = gu_bytes / (gu_us * 1e-6) / 1e9
    traffic = gate_up_traffic(args.workload)
    lm_bytes = sh.vocab * sh.d * sh.elem_bytes

    nbytes = pass_bytes(sh, T, R, C)
    passes_s = 1e3 / ms
    out = {
        "metric": METRIC,
        "value": T * passes_s,
        "unit": "verified tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if sh.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,0.02) weights, unit-variance synthetic KV, drafts greedy under silence)",
        "config": {"workload": f"{wl.shape.name} verify: {sh.n_layers} layers d={sh.d} {sh.n_heads}x{sh.head_dim} "
                               f"q heads / {sh.n_kv_heads} kv heads FFN {sh.ffn} V={sh.vocab}; C={C}; "
                               f"{L_a} audio + {gamma} drafts" + (f" + {wl.n_branch}-token branch (tree mask)"
                                                                  if wl.n_branch else ""),
                   "batch": 1, "T": T, "R": R, "context": C, "scenario": args.scenario,
                   "graph": bool(args.graph)},
        "passes_per_s": passes_s,
        "committed_tokens_per_pass": n_acc + 1,
        "committed_tokens_per_s": (n_acc + 1) * passes_s,
        "pass_roofline": {"bound": "hbm", "bytes": nbytes, "achieved_GBs": nbytes / (ms * 1e-3) / 1e9,
                          "peak_GBs": HBM_PEAK_GBS, "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "roofline": {"bound": "hbm", "kernel": "gemm_stream, SwiGLU epilogue (gate/up projection)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "bytes_per_launch": gu_bytes, "avg_launch_us": gu_us,
                     "launches_per_pass": sh.n_layers},
        "gemm_launch_us": launch_us,
        "lm_head": {"avg_launch_us": launch_us["lm_head"], "GBs": lm_bytes / (launch_us["lm_head"] * 1e-6) / 1e9},
        "setup_s": setup_s,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_verify(w, kv_host, wl, tokens, parent, rows, T)
    return out


def cpu_baseline_verify(w, kv_host, wl, tokens, parent, rows, T):
    """The oracle (fp64 NumPy, bf16 rounding mode for bf16 models) timed on the host:
    one full pass (verify + greedy acceptance + commit plan)."""
    from oracle import BF16_KV, EXACT
    from oracle import accept as oacc
    from oracle import decoder as odec
    from synth import make_random_kv
    sh = wl.shape
    C = wl.ctx[0]
    if kv_host is None:  # prefilled context: use synthetic KV of the same shape for the timing sample
        kv_host = make_random_kv(sh, [C], capacity=C + T, seed=wl.seed + 1000)
    mode = BF16_KV if sh.dtype == "bf16" else EXACT
    cache = odec.Cache(kv_host.k, kv_host.v)
    reps = 0
    t0 = time.perf_counter()
    while True:
        res = odec.verify_forward(w, cache, tokens[None, :], parent, rows, mode)
        am = [oacc.argmax_lowest(r) for r in res["logits"][0]]
        n, nxt, path = oacc.accept_greedy(list(tokens), parent, wl.L_a, rows, am)
        oacc.commit_plan(C, wl.L_a, path)
        reps += 1
        if time.perf_counter() - t0 > 10.0 or reps >= 3:
            break
    dt = (time.perf_counter() - t0) / reps
    return {"value": T / dt, "unit": "verified tokens/s", "cores": cpu_threads(), "kind": "oracle",
            "sample": f"{reps} full verify pass(es) of the same workload, fp64 oracle ({mode} mode), "
                      f"{dt:.2f} s per pass"}


def bench_c5(args, wl):
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
    w = make_weights(sh, seed=wl.seed)
    model = sdv.DeviceModel(w)
    del w
    table, n_blocks = page_table(ctx, T + 16, 16, seed=wl.seed + 7)
    kv = sdv.PagedKV(sh, B, 0, table=table, n_blocks=n_blocks)
    kv.load(HashedKV(sh, ctx, 0, seed=wl.seed + 1000, device=kv.device))
    tokens = np.empty((B, T), dtype=np.int32)
    for s_ in range(B // 2):   # uniform codes; both rows of a session get the same ids
        tokens[2 * s_] = tokens[2 * s_ + 1] = base + uniform_tokens(T, Vc, wl.seed * 1000 + s_, "c5codes") - 1
    rows = wl.logit_rows()
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

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t_start) / args.steps * 1e3
    assert int(acc_out["err"].abs().sum()) == 0 and int(ver.err.abs().sum()) == 0, "device error during bench"
    n_gemm = 4 * sh.n_layers + 1
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_gemm)]
    ver.set_profile_events(ev)
    step()
    torch.cuda.synchronize()
    per = [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(n_gemm)]
    ver.set_profile_events(None)
    per_layer = np.asarray(per[:4 * sh.n_layers]).reshape(sh.n_layers, 4)
    launch_us = {name: float(per_layer[:, i].mean()) * 1e3 for i, name in enumerate(("qkv", "o", "gate_up", "down"))}
    launch_us["codebook_head"] = per[-1] * 1e3
    M = B * T
    gu_flops = 2.0 * M * (2 * sh.ffn) * sh.d
    achieved = gu_flops / (launch_us["gate_up"] * 1e-6) / 1e12
    kv_bytes = sum(ctx) * sh.n_layers * 2 * sh.kv_dim * sh.elem_bytes
    # weights read once (decoder, codebook matrix, gathered embedding rows)
    w_bytes = (sh.n_layers * (sh.layer_params() - 2 * sh.d) + Vc * sh.d + B * T * sh.d) * sh.elem_bytes
    nbytes = w_bytes + kv_bytes + M * sh.n_layers * 2 * sh.kv_dim * sh.elem_bytes
    passes_s = 1e3 / ms
    n_acc = acc_out["n"].cpu().numpy()
    return {
        "metric": METRIC, "value": (B // 2) * T * passes_s, "unit": "verified session tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights, coordinate-hashed unit-variance KV generated on the device, "
                "uniform draft codes)",
        "config": {"workload": f"batched multi-codebook verify: {B // 2} sessions x 2 guidance rows, 8B-shape "
                               f"backbone, {S} codebooks x {Vc}, contexts {min(ctx)}..{max(ctx)}, "
                               f"{L_a} audio + {wl.gamma} drafts, w={wl.cfg_w}",
                   "rows": B, "T": T, "R": len(rows), "cached_tokens": sum(ctx)},
        "passes_per_s": passes_s, "row_tokens_per_s": B * T * passes_s,
        "committed_tokens_per_pass": int((n_acc + 1).sum()) // 2,
        "pass_roofline": {"bound": "hbm", "bytes": nbytes, "achieved_GBs": nbytes / (ms * 1e-3) / 1e9,
                          "peak_GBs": HBM_PEAK_GBS, "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "roofline": {"bound": "mfma", "kernel": "gemm_tiled, SwiGLU epilogue (gate/up projection), 2624 rows",
                     "achieved": achieved, "peak": 2500.0, "unit": "TFLOP/s", "frac": achieved / 2500.0,
                     "traffic": None, "flops_per_launch": gu_flops, "avg_launch_us": launch_us["gate_up"]},
        "gemm_launch_us": launch_us, "setup_s": setup_s,
    }


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
    copies = []
    for c in range(2):
        copies.append(dict(tgt=torch.from_numpy(si.target_logits).cuda(), drf=torch.from_numpy(si.draft_logits).cuda(),
                           drafts=torch.from_numpy(si.drafts).cuda()))
    smp = sdv.Sampler(B, k, V)
    setup_s = time.time() - t0

    def step(i):
        c = copies[i & 1]
        smp(c["tgt"], c["drf"], c["drafts"], si.seed)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t_start) / args.steps * 1e3
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
        "metric": METRIC, "value": B * k / (ms * 1e-3), "unit": "draft positions/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"speculative-sampling acceptance: {B} seqs x {k} drafts, V={V}, fp32"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": counter_traffic(ROW_STATS_TRAFFIC, "sample", SAMPLE_SOURCES),
                     "kernel": "spec_row_stats_kernel (maximum and exponential sum of every logit row)",
                     "bytes_per_launch": stats_bytes, "avg_launch_us": stats_us},
        "pass_roofline": {"bound": "hbm", "bytes": nbytes, "achieved_GBs": nbytes / (ms * 1e-3) / 1e9,
                          "peak_GBs": HBM_PEAK_GBS, "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "setup_s": setup_s,
    }
    if not args.no_cpu_baseline:
        from oracle import spec_sampling as ss
        tgt64, drf64 = si.target_logits.astype(np.float64), si.draft_logits.astype(np.float64)
        # repeat the full batch until about 10 s of CPU work have been timed
        reps, dt = 0, 0.0
        while dt < 10.0 and reps < 100:
            t0 = time.perf_counter()
            ss.accept_sample(tgt64, drf64, si.drafts, si.u_accept, si.u_sample)
            dt += time.perf_counter() - t0
            reps += 1
        out["cpu_baseline"] = {"value": reps * B * k / dt, "unit": "draft positions/s", "cores": cpu_threads(),
                               "kind": "oracle",
                               "sample": f"{reps} full batches ({B}x{k}, V={V}) in {dt:.1f} s"}
    return out


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
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="1.7b-bf16",
                    choices=["1.7b-bf16", "8b-bf16-tree", "toy-f32", "sample", "c5-codebook"])
    ap.add_argument("--scenario", default="silence", choices=["silence", "random"])
    ap.add_argument("--graph", action="store_true", help="replay the step from a captured HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time a plain 256 MiB device-to-device copy (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
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
    if args.workload == "sample":
        out = bench_sample(args)
    elif args.workload == "c5-codebook":
        out = bench_c5(args, WORKLOADS[args.workload]())
    else:
        out = bench_verify(args, WORKLOADS[args.workload]())
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
