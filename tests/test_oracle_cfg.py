"""Pins of oracle.cfg (codebook heads and guidance merge) against closed forms and
invariants: "An Efficient vLLM-Based Inference Pipeline for Unified Audio
Understanding and Generation" (page 2), Figure 1 (stream embedding + shared head)
and the paired-guidance section (per-codebook interpolation with weight w)."""
from dataclasses import replace

import numpy as np
import pytest

from oracle import BF16_KV, EXACT
from oracle import accept as oacc
from oracle import cfg
from oracle import decoder as odec
from synth import make_random_kv, make_weights, uniform_tokens
from synth.configs import MINI_BF16, MINI_F32

CB_F32 = replace(MINI_F32, name="mini-f32-cb", n_codebooks=3, codebook_size=48)
CB_BF16 = replace(MINI_BF16, name="mini-bf16-cb", n_codebooks=4, codebook_size=64)


def test_merge_closed_forms():
    rng = np.random.default_rng(0)
    c, u = rng.standard_normal(200) * 4, rng.standard_normal(200) * 4
    np.testing.assert_allclose(cfg.cfg_merge(c, u, 1.0), c, rtol=0, atol=1e-14)   # w = 1: conditional
    assert np.array_equal(cfg.cfg_merge(c, u, 0.0), u)                            # w = 0: unconditional
    assert np.array_equal(cfg.cfg_merge(c, c, 2.0), c)                            # c = u: unchanged
    # w = 2 extrapolates away from u: merged - c = c - u
    np.testing.assert_allclose(cfg.cfg_merge(c, u, 2.0) - c, c - u, atol=1e-13)


def test_guidance_can_flip_the_argmax():
    c = np.array([1.0, 1.1])   # conditional prefers 1
    u = np.array([0.0, 1.2])   # unconditional prefers 1 even more
    merged = cfg.cfg_merge(c, u, 2.0)   # [2.0, 1.0]
    assert oacc.argmax_lowest(c) == 1 and oacc.argmax_lowest(merged) == 0
    np.testing.assert_allclose(merged, [2.0, 1.0], atol=1e-15)


def test_stream_embedding_enters_linearly():
    w = make_weights(CB_F32, seed=11)
    h = np.random.default_rng(1).standard_normal((5, CB_F32.d))
    l = cfg.codebook_logits(w, h)                                  # [5, S, Vc]
    wcb = np.asarray(w.codebook, np.float64)
    e = np.asarray(w.stream_emb, np.float64)
    for s in range(1, CB_F32.n_codebooks):
        want = wcb @ (e[s] - e[0])                                  # the same for every row
        for n in range(5):
            np.testing.assert_allclose(l[n, s] - l[n, 0], want, rtol=0, atol=1e-12)


def test_shared_matrix_orientation_with_identity_head():
    # a head whose row v selects coordinate v gives logits = normalised h + e_s
    sh = replace(CB_F32, codebook_size=CB_F32.d)
    w = make_weights(sh, seed=12)
    w.codebook = np.eye(sh.d, dtype=np.float32)
    w.final_norm = np.ones(sh.d, dtype=np.float32)
    h = np.random.default_rng(2).standard_normal((3, sh.d))
    l = cfg.codebook_logits(w, h)
    hn = h / np.sqrt((h * h).mean(axis=1, keepdims=True) + sh.eps)
    for s in range(sh.n_codebooks):
        np.testing.assert_allclose(l[:, s], hn + np.asarray(w.stream_emb[s], np.float64), atol=1e-12)


def test_head_is_scale_invariant_through_the_final_norm():
    w = make_weights(CB_F32, seed=13)
    h = np.random.default_rng(3).standard_normal((4, CB_F32.d))
    np.testing.assert_allclose(cfg.codebook_logits(w, 7.5 * h), cfg.codebook_logits(w, h), rtol=0, atol=1e-5)


@pytest.mark.parametrize("shape,mode", [(CB_F32, EXACT), (CB_BF16, BF16_KV)])
def test_verify_codebook_pairs(shape, mode):
    w = make_weights(shape, seed=21)
    B, L_a, gamma = 5, 3, 3
    T = L_a + gamma
    ctx = [7, 7, 12, 12, 4]          # rows (0,1) and (2,3) are pairs of equal length; row 4 alone
    kv = make_random_kv(shape, ctx, capacity=max(ctx) + T, seed=22)
    cache = odec.Cache(kv.k, kv.v)
    base = shape.vocab - shape.n_codebooks * shape.codebook_size
    toks = base + uniform_tokens(2 * T, shape.codebook_size - 1, 23, "cb").reshape(2, T)
    tokens = np.stack([toks[0], toks[0], toks[1], toks[1], toks[0]])   # token sync inside a pair
    rows = list(range(L_a - 1, T))
    partner = [1, 0, 3, 2, -1]
    out = cfg.verify_codebook(w, cache, tokens, None, rows, partner, 2.0, base, mode)
    own = np.stack([cfg.codebook_logits(w, out["res"]["hidden"][b][rows]) for b in range(B)])
    for c, u in ((0, 1), (2, 3)):
        assert np.array_equal(out["logits"][c], out["logits"][u])       # both rows see the same distribution
        np.testing.assert_allclose(out["logits"][c], own[u] + 2.0 * (own[c] - own[u]), atol=1e-12)
    assert np.array_equal(out["logits"][4], own[4])
    assert np.array_equal(out["token"], base + out["argmax"][:, :, 0])
    # w = 1 reproduces the conditional rows' own head
    out1 = cfg.verify_codebook(w, cache, tokens, None, rows, partner, 1.0, base, mode)
    np.testing.assert_allclose(out1["logits"][1], own[0], atol=1e-12)
    # acceptance on codebook 0 commits the same count to both rows of a pair
    for c, u in ((0, 1), (2, 3)):
        nc = oacc.accept_greedy(list(tokens[c]), None, L_a, rows, list(out["token"][c]))[0]
        nu = oacc.accept_greedy(list(tokens[u]), None, L_a, rows, list(out["token"][u]))[0]
        assert nc == nu


def test_partners_must_be_mutual():
    with pytest.raises(ValueError):
        cfg.check_partners([1, 2, 0])
    cfg.check_partners([1, 0, -1])
