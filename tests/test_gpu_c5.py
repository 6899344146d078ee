"""GPU parity of the batched multi-codebook verify at its full size: the 8B-shape
backbone with 8 codebook heads of 1024 ("An Efficient vLLM-Based Inference Pipeline
for Unified Audio Understanding and Generation", page 2: stream embeddings, shared
codebook matrix, paired guidance with w = 2 and the same token on both rows), 32
sessions x (conditional, unconditional) rows, cached contexts in [2048, 16384] paged
over one permuted block pool (about 91 GB of bf16 KV, generated on the device from the
coordinate-hashed recipe), 25 audio + 16 draft codes per session.

Checked for every row: no device error; both rows of a pair see bit-identical guided
logits and accept the same count.  Checked against the oracle (BF16_KV mode) on the
sessions with the shortest and the longest context and two seeded random sessions:
guided logits per (row, codebook) within 2e-2 of the largest oracle logit, argmax codes
bit-exact where the oracle's top-2 margin is at least 1e-3 (at most 2 % of the
(row, codebook) pairs flagged), committed token and accepted count where no deciding
row is flagged.
The draft codes are uniform (the recipe's greedy drafts change only how many are
accepted, not what the pass computes).
"""
import time

import numpy as np
import pytest
import torch

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import speculative_decoding_verify_amd as sdv  # noqa: E402
from oracle import BF16_KV  # noqa: E402
from oracle import accept as oacc  # noqa: E402
from oracle import cfg  # noqa: E402
from oracle import decoder as odec  # noqa: E402
from synth import HashedKV, make_weights, page_table, uniform_tokens  # noqa: E402
from synth.configs import c5_workload  # noqa: E402
from tests.gpu_helpers import MARGIN_FLAG  # noqa: E402


def _log(msg):
    print(msg, flush=True)


@pytest.mark.timeout(1500)
def test_c5_full_size_codebook_guidance():
    wl = c5_workload()
    sh = wl.shape
    B, T, L_a = wl.batch, wl.T, wl.L_a
    S, Vc = sh.n_codebooks, sh.codebook_size
    base = sh.vocab - S * Vc
    rows = wl.logit_rows()
    ctx = list(wl.ctx)
    _log(f"C5: {B} rows, contexts {min(ctx)}..{max(ctx)}, {sum(ctx)} cached tokens")
    t0 = time.time()
    w = make_weights(sh, seed=wl.seed)
    model = sdv.DeviceModel(w)
    _log(f"weights on the device ({time.time() - t0:.0f} s)")
    table, n_blocks = page_table(ctx, T + 16, 16, seed=wl.seed + 7)
    kv = sdv.PagedKV(sh, B, 0, table=table, n_blocks=n_blocks)
    kv_seed = wl.seed + 1000
    kv.load(HashedKV(sh, ctx, 0, seed=kv_seed, device=kv.device))
    torch.cuda.synchronize()
    _log(f"KV filled on the device: {n_blocks} blocks ({time.time() - t0:.0f} s)")

    # the device-generated cache equals the host recipe (row 5, two layers, a page-crossing slice)
    for l in (0, sh.n_layers - 1):
        k_dev, v_dev = kv.gather(5, l, ctx[5] - 40, ctx[5])
        hk = HashedKV(sh, ctx, 0, seed=kv_seed)
        k_host = hk.block(5, l, 0)[ctx[5] - 40:]
        v_host = hk.block(5, l, 1)[ctx[5] - 40:]
        assert np.array_equal(k_dev.cpu().numpy(), odec.bits_to_f64(k_host).astype(np.float32))
        assert np.array_equal(v_dev.cpu().numpy(), odec.bits_to_f64(v_host).astype(np.float32))

    tokens = np.empty((B, T), dtype=np.int32)
    for s in range(B // 2):
        codes = uniform_tokens(T, Vc, wl.seed * 1000 + s, "c5codes") - 1     # uniform on [0, Vc - 1)
        tokens[2 * s] = tokens[2 * s + 1] = base + codes
    partner = [b ^ 1 for b in range(B)]
    ver = sdv.Verifier(model, kv, T, L_a, rows, max_ctx=max(ctx), want_logits=True, head=sdv.HEAD_CODEBOOK,
                       cfg_partner=partner, cfg_w=wl.cfg_w)
    ver.set_tokens(tokens)
    res = ver.forward()
    acc = sdv.accept_greedy(B, T, L_a, ver.tokens, None, ver.logit_rows, res.argmax)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ver.forward()
    torch.cuda.synchronize()
    _log(f"verify pass on the device: {(time.perf_counter() - t1) * 1e3:.1f} ms")
    g_logits = res.logits.cpu().numpy()
    g_cb = res.cb_argmax.cpu().numpy()
    g_tok = res.argmax.cpu().numpy()
    g_n = acc["n"].cpu().numpy()
    assert (res.err.cpu().numpy() == 0).all()
    assert (acc["err"].cpu().numpy() == 0).all()
    for s in range(B // 2):
        assert np.array_equal(g_logits[2 * s], g_logits[2 * s + 1]), s
        assert g_n[2 * s] == g_n[2 * s + 1], s

    # oracle on the sessions with the shortest and the longest context and two seeded
    # random ones (the longest merges two non-empty key splits over ~1000 pages)
    by_len = sorted(range(B // 2), key=lambda s: ctx[2 * s])
    rest = [s for s in range(B // 2) if s not in (by_len[0], by_len[-1])]
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, 0xC5C5])))
    sessions = [by_len[0], by_len[-1]] + [int(x) for x in rng.choice(rest, size=2, replace=False)]
    for s in sessions:
        r2 = [2 * s, 2 * s + 1]
        _log(f"oracle: session {s}, context {ctx[2 * s]}")
        hk = HashedKV(sh, [ctx[b] for b in r2], 0, seed=kv_seed, streams=r2)
        cache = odec.Cache([[hk.block(i, l, 0) for l in range(sh.n_layers)] for i in range(2)],
                           [[hk.block(i, l, 1) for l in range(sh.n_layers)] for i in range(2)])
        o = cfg.verify_codebook(w, cache, tokens[r2], None, rows, [1, 0], wl.cfg_w, base, BF16_KV)
        flagged = 0
        for i, b in enumerate(r2):
            for r in range(len(rows)):
                for c in range(S):
                    ol, gl = o["logits"][i, r, c], g_logits[b, r, c].astype(np.float64)
                    err = np.abs(gl - ol).max() / np.abs(ol).max()
                    assert err <= 2e-2, (b, r, c, err)
                    if oacc.top2_margin(ol) < MARGIN_FLAG:
                        flagged += 1
                        continue
                    assert g_cb[b, r, c] == o["argmax"][i, r, c], (b, r, c)
                if o["margin"][i, r] >= MARGIN_FLAG:
                    assert g_tok[b, r] == o["token"][i, r], (b, r)
            n, nxt, path = oacc.accept_greedy(list(tokens[b]), None, L_a, rows, list(o["token"][i]))
            deciding = [L_a - 1 + j for j in range(n + 1)]
            if all(o["margin"][i, rows.index(row)] >= MARGIN_FLAG for row in deciding):
                assert g_n[b] == n, (b, g_n[b], n)
        _log(f"session {s}: flagged {flagged}/{2 * len(rows) * S}")
        assert flagged <= max(1, 2 * len(rows) * S // 50)
