"""GPU parity of the codebook-head verify with classifier-free guidance pairs
("An Efficient vLLM-Based Inference Pipeline for Unified Audio Understanding and
Generation", page 2: stream embedding + shared codebook matrix, per-codebook merge
u + w (c - u) on paired rows that accept the same tokens) against oracle.cfg.

Tolerances as in gpu_helpers: guided logits per (row, codebook) within 2e-2 (bf16,
against BF16_KV) or 1e-5 (fp32, against EXACT) relative to the largest oracle logit;
argmax codes bit-exact where the oracle's top-2 margin is at least 1e-3.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import speculative_decoding_verify_amd as sdv
from oracle import accept as oacc
from oracle import cfg
from oracle import decoder as odec
from synth import make_random_kv, make_weights, uniform_tokens
from synth.configs import MINI_BF16, MINI_BF16_D128, MINI_F32
from tests.gpu_helpers import MARGIN_FLAG, logit_tol, mode_of

pytestmark = pytest.mark.gpu

CB_BF16 = replace(MINI_BF16, name="mini-bf16-cb", n_codebooks=4, codebook_size=64)
CB_F32 = replace(MINI_F32, name="mini-f32-cb", n_codebooks=3, codebook_size=48)
CB_D128 = replace(MINI_BF16_D128, name="mini-bf16-dh128-cb", n_codebooks=2, codebook_size=100)


def _run(shape, partner, ctx, seed, L_a=4, gamma=5, w_cfg=2.0):
    w = make_weights(shape, seed=seed)
    B, T = len(ctx), L_a + gamma
    rows = list(range(L_a - 1, T))
    base = shape.vocab - shape.n_codebooks * shape.codebook_size
    tokens = np.empty((B, T), dtype=np.int32)
    for b in range(B):   # token sync: the lower row of a (mutual) pair decides the tokens of both
        p = partner[b]
        src = min(b, p) if p >= 0 and partner[p] == b else b
        tokens[b] = base + uniform_tokens(T, shape.codebook_size, seed * 100 + src, "cbt")
    kv_host = make_random_kv(shape, ctx, capacity=max(ctx) + T, seed=seed + 1)
    model = sdv.DeviceModel(w)
    kv = sdv.PagedKV(shape, B, max(ctx) + T + 16)
    kv.load(kv_host)
    ver = sdv.Verifier(model, kv, T, L_a, rows, max_ctx=max(ctx), want_logits=True, head=sdv.HEAD_CODEBOOK,
                       cfg_partner=partner, cfg_w=w_cfg)
    ver.set_tokens(tokens)
    res = ver.forward()
    acc = sdv.accept_greedy(B, T, L_a, ver.tokens, None, ver.logit_rows, res.argmax)
    torch.cuda.synchronize()
    g = dict(logits=res.logits.cpu().numpy().astype(np.float64), cb=res.cb_argmax.cpu().numpy(),
             argmax=res.argmax.cpu().numpy(), err=res.err.cpu().numpy(), n=acc["n"].cpu().numpy())
    return w, tokens, rows, base, kv_host, g


@pytest.mark.parametrize("shape", [CB_BF16, CB_F32, CB_D128], ids=lambda s: s.name)
def test_codebook_guidance_parity(shape):
    partner = [1, 0, 3, 2, -1, -1]
    ctx = [9, 9, 20, 20, 5, 13]
    w, tokens, rows, base, kv_host, g = _run(shape, partner, ctx, seed=31)
    assert (g["err"] == 0).all()
    o = cfg.verify_codebook(w, odec.Cache(kv_host.k, kv_host.v), tokens, None, rows, partner, 2.0, base,
                            mode_of(shape))
    B, R, S, Vc = o["logits"].shape
    tol = logit_tol(shape)
    flagged = 0
    for b in range(B):
        for r in range(R):
            for s in range(S):
                ol, gl = o["logits"][b, r, s], g["logits"][b, r, s]
                err = np.abs(gl - ol).max() / np.abs(ol).max()
                assert err <= tol, (b, r, s, err)
                if oacc.top2_margin(ol) < MARGIN_FLAG:
                    flagged += 1
                    continue
                assert g["cb"][b, r, s] == o["argmax"][b, r, s], (b, r, s)
            if o["margin"][b, r] >= MARGIN_FLAG:
                assert g["argmax"][b, r] == o["token"][b, r]
    # both rows of a pair see bit-identical guided logits and accept the same count
    for c, u in ((0, 1), (2, 3)):
        assert np.array_equal(g["logits"][c], g["logits"][u])
        assert g["n"][c] == g["n"][u]
    print(f"{shape.name}: flagged {flagged}/{B * R * S}")


def test_guidance_weight_one_is_the_conditional_head():
    shape = CB_F32
    partner = [1, 0]
    w, tokens, rows, base, kv_host, g = _run(shape, partner, [11, 11], seed=41, w_cfg=1.0)
    w2, tokens2, rows2, base2, kv2, g_own = _run(shape, [-1, -1], [11, 11], seed=41)
    np.testing.assert_allclose(g["logits"][1], g_own["logits"][0], rtol=0,
                               atol=1e-5 * np.abs(g_own["logits"][0]).max())


def test_non_mutual_partner_is_reported_and_row_uses_its_own_head():
    shape = CB_F32
    partner = [1, 2, 0]          # 0 -> 1 -> 2 -> 0: no pair is mutual
    w, tokens, rows, base, kv_host, g = _run(shape, partner, [6, 6, 6], seed=51)
    assert (g["err"] & 0x20).all()
    w2, tokens2, rows2, base2, kv2, g_own = _run(shape, [-1, -1, -1], [6, 6, 6], seed=51)
    assert np.array_equal(g["logits"], g_own["logits"])


@pytest.mark.parametrize("shape", [CB_BF16, CB_F32], ids=lambda s: s.name)
def test_guided_greedy_drafts_are_accepted_in_full(shape):
    """Drafts that are the guided greedy continuation (the oracle's codebook-0 argmax of
    the merged logits, one token at a time from the audio chunk) are accepted in full on
    both rows of every pair, with the corrected token equal to the oracle's next one."""
    partner = [1, 0, 3, 2]
    ctx = [9, 9, 20, 20]
    L_a, gamma, seed = 4, 5, 61
    w = make_weights(shape, seed=seed)
    B = len(partner)
    base = shape.vocab - shape.n_codebooks * shape.codebook_size
    kv_host = make_random_kv(shape, ctx, capacity=max(ctx) + L_a + gamma, seed=seed + 1)
    tokens = np.empty((B, L_a), dtype=np.int32)
    for b in range(B):
        tokens[b] = base + uniform_tokens(L_a, shape.codebook_size, seed * 100 + min(b, partner[b]), "cbt")
    mode = mode_of(shape)
    near = np.zeros(B, dtype=bool)   # a guided decision along the drafts within the margin band
    for i in range(gamma + 1):
        o = cfg.verify_codebook(w, odec.Cache(kv_host.k, kv_host.v), tokens, None, [tokens.shape[1] - 1], partner,
                                2.0, base, mode)
        near |= o["margin"][:, 0] < MARGIN_FLAG
        nxt = o["token"][:, 0].astype(np.int32)
        if i == gamma:
            break
        tokens = np.concatenate([tokens, nxt[:, None]], axis=1)
    T = L_a + gamma
    rows = list(range(L_a - 1, T))
    model = sdv.DeviceModel(w)
    kv = sdv.PagedKV(shape, B, max(ctx) + T + 16)
    kv.load(kv_host)
    ver = sdv.Verifier(model, kv, T, L_a, rows, max_ctx=max(ctx), want_logits=True, head=sdv.HEAD_CODEBOOK,
                       cfg_partner=partner, cfg_w=2.0)
    ver.set_tokens(tokens)
    res = ver.forward()
    acc = sdv.accept_greedy(B, T, L_a, ver.tokens, None, ver.logit_rows, res.argmax)
    torch.cuda.synchronize()
    n, nx = acc["n"].cpu().numpy(), acc["next"].cpu().numpy()
    assert near.sum() <= 1, f"{near.sum()} rows of {B} within the margin band"
    for c, u in ((0, 1), (2, 3)):
        assert n[c] == n[u] and nx[c] == nx[u]
        if not (near[c] or near[u]):
            assert n[c] == gamma, (c, n[c])
            assert nx[c] == nxt[c], (c, nx[c], nxt[c])
    print(f"{shape.name}: accepted {list(n)} of {gamma}, near {list(near)}")
