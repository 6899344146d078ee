"""Helpers of the GPU parity tests: run one verify pass on both sides and compare.

Tolerances (written into the checks below):
  * logits: per-row max-abs error over max-abs oracle logit <= 2e-2 for bf16 models
    (against the oracle's BF16_KV mode: bf16 weights and cache, exact elsewhere) and
    <= 1e-5 for fp32 models (against the exact fp64 mode);
  * argmax and greedy acceptance: bit-exact, except rows whose oracle top-2 margin is
    below 1e-3 (flagged, excluded and counted); acceptance is compared only when no
    row on the oracle's accepted path (or the row deciding the stop) is flagged;
  * keys/values written: layer 0 within 1 bf16 ulp (bf16) / 1e-5 relative (fp32);
    deeper layers within the logits' relative tolerance.
"""
from __future__ import annotations

import numpy as np
import torch

import speculative_decoding_verify_amd as sdv
from oracle import BF16_KV, EXACT
from oracle import accept as oacc
from oracle import decoder as odec

MARGIN_FLAG = 1e-3


def logit_tol(shape) -> float:
    return 2e-2 if shape.dtype == "bf16" else 1e-5


def mode_of(shape) -> str:
    """bf16 models: weights and KV cache in bf16, activations at fp32 precision."""
    return BF16_KV if shape.dtype == "bf16" else EXACT


def run_pair(w, kv_host, tokens, L_a, parent=None, logit_rows=None, perm_seed=None, model=None,
             want_hidden=True, max_ctx=None, extra_capacity=16, oracle_attn=False):
    """tokens [B, T].  Returns (gpu dict, oracle dict, Verifier, PagedKV)."""
    sh = w.shape
    tokens = np.asarray(tokens, dtype=np.int32)
    B, T = tokens.shape
    rows = list(range(L_a - 1, T)) if logit_rows is None else list(logit_rows)
    cap = max(kv_host.lens) + T + extra_capacity
    perm = None
    if perm_seed is not None:
        from synth.gen import page_permutation
        mb = (cap + 15) // 16
        perm = page_permutation(B * mb, perm_seed)
    model = model or sdv.DeviceModel(w)
    kv = sdv.PagedKV(sh, B, cap, perm=perm)
    kv.load(kv_host)
    ver = sdv.Verifier(model, kv, T, L_a, rows, parent=parent,
                       max_ctx=max(kv_host.lens) if max_ctx is None else max_ctx,
                       want_logits=True, want_hidden=want_hidden)
    ver.set_tokens(tokens)
    res = ver.forward()
    torch.cuda.synchronize()
    g = dict(logits=res.logits.cpu().numpy().astype(np.float64), argmax=res.argmax.cpu().numpy(),
             margin=res.margin.cpu().numpy(), lse=res.lse.cpu().numpy(), err=res.err.cpu().numpy(),
             hidden=None if res.hidden is None else res.hidden.cpu().numpy().astype(np.float64))
    cache = odec.Cache(kv_host.k, kv_host.v)
    o = odec.verify_forward(w, cache, tokens, parent, rows, mode_of(sh), want_attn=oracle_attn)
    return g, o, ver, kv


def compare_logits(sh, g, o, max_flag_frac=0.05):
    """Returns (max row rel err, n flagged, n compared) and asserts parity.  Rows whose
    oracle top-2 margin is below 1e-3 are flagged (excluded from the argmax check); at
    most max_flag_frac of the rows (and at least one) may be flagged: random-weight
    logits put about 1 % of rows below the band on the small shapes, and none of the
    full-size rows of the seeded workloads."""
    tol = logit_tol(sh)
    gl, ol = g["logits"], o["logits"]
    B, R, V = ol.shape
    err = np.max(np.abs(gl - ol), axis=2) / np.max(np.abs(ol), axis=2)
    assert np.all(np.isfinite(gl)), "non-finite GPU logits"
    assert err.max() <= tol, f"logit rel err {err.max():.3e} > {tol}"
    flagged = 0
    for b in range(B):
        for r in range(R):
            m = oacc.top2_margin(ol[b, r])
            if m < MARGIN_FLAG:
                flagged += 1
                continue
            assert g["argmax"][b, r] == oacc.argmax_lowest(ol[b, r]), (b, r)
            # margin and log-sum-exp of the GPU agree with its own logits' definition
            srt = np.sort(ol[b, r])
            assert abs(g["margin"][b, r] - (srt[-1] - srt[-2])) <= tol * np.max(np.abs(ol[b, r])) * 2 + 1e-6
    assert flagged <= max(1, int(max_flag_frac * B * R)), f"{flagged} of {B * R} rows flagged"
    lse = np.log(np.sum(np.exp(ol - ol.max(axis=2, keepdims=True)), axis=2)) + ol.max(axis=2)
    assert np.max(np.abs(g["lse"] - lse)) <= max(1e-4, 4 * tol * np.max(np.abs(ol))), "lse mismatch"
    return float(err.max()), flagged, B * R


def compare_kv(sh, kv, o, lens, T):
    """Keys/values written for the chunk rows vs the oracle's.  Layer 0 sees identical
    inputs on both sides, so its bf16 K/V agree to one bf16 ulp (fp32: every element
    within 1e-5 of the tensor's largest magnitude -- fp32 accumulation over K terms
    leaves an absolute error that grows with K, so small elements are not held to a
    fixed absolute floor); deeper layers see a residual stream that already carries
    rounding differences and are held to the logits' per-row relative tolerance."""
    tol = logit_tol(sh)
    for b in range(len(lens)):
        for l in range(sh.n_layers):
            k, v = kv.gather(b, l, lens[b], lens[b] + T)
            for gt, ot in ((k.cpu().numpy(), o["k_new"][b][l]), (v.cpu().numpy(), o["v_new"][b][l])):
                if l == 0 and sh.dtype == "bf16":
                    bad = np.abs(gt - ot) > np.abs(ot) * 2.0 ** -7 + 1e-6
                    assert bad.mean() < 1e-3 and not np.any(np.abs(gt - ot) > np.abs(ot) * 2.0 ** -6 + 1e-5), \
                        f"K/V mismatch b={b} l={l}: {bad.sum()} elements beyond 1 ulp"
                elif l == 0:
                    np.testing.assert_allclose(gt, ot, rtol=1e-5, atol=1e-5 * np.max(np.abs(ot)))
                else:
                    rel = np.max(np.abs(gt - ot)) / np.max(np.abs(ot))
                    assert rel <= tol, f"K/V mismatch b={b} l={l}: rel {rel:.2e}"


def greedy_expectation(tokens_b, parent, L_a, rows, ol_b):
    """Oracle acceptance plus whether any deciding row is flagged."""
    am = [oacc.argmax_lowest(r) for r in ol_b]
    n, nxt, path = oacc.accept_greedy(list(tokens_b), parent, L_a, rows, am)
    rmap = {row: i for i, row in enumerate(rows)}
    deciding = [L_a - 1] + path
    flagged = any(oacc.top2_margin(ol_b[rmap[row]]) < MARGIN_FLAG for row in deciding)
    return n, nxt, path, flagged
