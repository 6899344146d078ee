"""Pins of the oracle decoder, greedy acceptance and rollback (CPU only).

What the pages fix (page 1, "Decode Before You Hear", prerequisites and method
step 4): greedy verification commits exactly the tokens token-by-token greedy
decoding would; at least one token per forward; n follows the printed min
formula.  What mathematics fixes: closed forms of RoPE, RMSNorm and one-key
attention; a verify pass equals recomputation without a cache; a tree branch
equals a linear chunk of its own path; rounding equals torch's bf16 cast.
"""
import itertools
import math

import numpy as np
import pytest
import torch

from oracle import BF16, BF16_KV, EXACT
from oracle import accept as acc
from oracle import decoder as dec
from oracle.numerics import round_bf16, round_f32, bits_to_f64
from synth.configs import ModelShape
from synth.gen import make_weights, uniform_tokens, to_bf16_bits

TINY = ModelShape("tiny", n_layers=2, d=32, n_heads=4, n_kv_heads=2, head_dim=8,
                  ffn=48, vocab=8, dtype="f32")
SMALL = ModelShape("small", n_layers=2, d=48, n_heads=4, n_kv_heads=2, head_dim=12,
                   ffn=64, vocab=61, dtype="f32")
SMALL_BF = ModelShape("small-bf", n_layers=2, d=48, n_heads=4, n_kv_heads=2, head_dim=12,
                      ffn=64, vocab=61, dtype="bf16")


def _model(shape, seed=0, **kw):
    # larger weights than N(0, 0.02) so tiny models have non-trivial attention and logits
    return make_weights(shape, seed, std=kw.pop("std", 0.3), **kw)


def _prefilled(w, n_ctx, seed=1, mode=EXACT):
    sh = w.shape
    cache = dec.Cache.empty(1, sh.n_layers, sh.n_kv_heads, sh.head_dim)
    if n_ctx:
        ctx = uniform_tokens(n_ctx, sh.vocab, seed, "ctx")[None, :]
        dec.prefill(w, cache, ctx, mode, chunk=7)
    return cache


# -- numerics ---------------------------------------------------------------------

def test_round_bf16_equals_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000),
                        1.0 + np.arange(-4, 5) * 2.0 ** -9,        # exact ties around 1
                        [0.0, -0.0, 3.0, -1.5, 2.0 ** -100]])
    x32 = x.astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(round_bf16(x32.astype(np.float64)), ref)
    assert round_f32(1.0 + 2.0 ** -30) == 1.0
    # the synthetic-input encoder agrees with it too (independent bit manipulation)
    np.testing.assert_array_equal(bits_to_f64(to_bf16_bits(x32)), ref)


# -- closed forms -------------------------------------------------------------------

def test_rope_identity_at_zero_and_relative_position():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 1, 16))
    k = rng.standard_normal((1, 1, 16))
    np.testing.assert_allclose(dec.rope(q, np.array([0]), 10000.0), q, rtol=0, atol=0)
    dots = []
    for m, n in [(5, 2), (13, 10), (103, 100), (3, 0)]:
        dots.append(float(np.sum(dec.rope(q, np.array([m]), 10000.0) * dec.rope(k, np.array([n]), 10000.0))))
    np.testing.assert_allclose(dots, dots[0], rtol=1e-12)
    # rotation preserves the norm
    r = dec.rope(q, np.array([77]), 10000.0)
    assert np.linalg.norm(r) == pytest.approx(np.linalg.norm(q), rel=1e-14)
    # rotate-half pairing: element i and i + dh/2 rotate together by pos * theta^(-2i/dh)
    e = np.zeros((1, 1, 16))
    e[0, 0, 1] = 1.0
    r = dec.rope(e, np.array([3]), 10000.0)[0, 0]
    ang = 3 * 10000.0 ** (-2.0 / 16)
    assert r[1] == pytest.approx(np.cos(ang)) and r[9] == pytest.approx(np.sin(ang))


def test_rmsnorm_constant_vector():
    g = np.linspace(0.5, 2.0, 10)
    for c in (3.0, -0.25):
        out = dec.rmsnorm(np.full(10, c), g, 0.0)
        np.testing.assert_allclose(out, np.sign(c) * g, rtol=1e-15)


def test_single_key_attention_returns_value():
    """Empty cache, one row: softmax over a single key is 1, so the attention output of
    query head h is the value of kv head h // G."""
    w = _model(SMALL, 3)
    cache = dec.Cache.empty(1, SMALL.n_layers, SMALL.n_kv_heads, SMALL.head_dim)
    res = dec.verify_forward(w, cache, np.array([[5]]), None, [0], EXACT, want_attn=True)
    G = SMALL.n_heads // SMALL.n_kv_heads
    for l in range(SMALL.n_layers):
        o = res["attn"][0][l].reshape(SMALL.n_heads, SMALL.head_dim)
        v = res["v_new"][0][l][0]
        for h in range(SMALL.n_heads):
            np.testing.assert_allclose(o[h], v[h // G], rtol=1e-15)


def test_gqa_head_mapping():
    """Query head h reads kv head h // G.  Head h is steered onto cached key h (keys are
    unit vectors), and kv head g stores value 100 g + j at key j, so head h outputs
    100 (h // G) + h."""
    H, Hkv, dh, C = 4, 2, 8, 4
    Kc = np.zeros((C, Hkv, dh))
    Vc = np.zeros((C, Hkv, dh))
    for j in range(C):
        Kc[j, :, j] = 1.0
        for g in range(Hkv):
            Vc[j, g, :] = 100.0 * g + j
    q = np.zeros((1, H, dh))
    for h in range(H):
        q[0, h, h] = 200.0
    empty = np.zeros((1, Hkv, dh))
    o = dec.attend(q, Kc, Vc, empty - 1e4, empty, np.zeros((1, 1), bool)).reshape(H, dh)
    np.testing.assert_allclose(o[:, 0], [0.0, 1.0, 102.0, 103.0], atol=1e-9)


# -- verify == decoding ---------------------------------------------------------------

@pytest.mark.parametrize("mode", [EXACT, BF16, BF16_KV])
def test_verify_equals_token_by_token(mode):
    shape = SMALL if mode == EXACT else SMALL_BF
    w = _model(shape, 4)
    cache = _prefilled(w, 23, mode=mode)
    toks = uniform_tokens(11, shape.vocab, 5, "chunk")
    res = dec.verify_forward(w, cache, toks[None, :], None, range(11), mode)
    c2 = cache.copy()
    for j in range(11):
        r1 = dec.verify_forward(w, c2, toks[None, j:j + 1], None, [0], mode)
        np.testing.assert_allclose(r1["logits"][0, 0], res["logits"][0, j], rtol=1e-11, atol=1e-12)
        for l in range(shape.n_layers):
            np.testing.assert_allclose(r1["k_new"][0][l][0], res["k_new"][0][l][j], rtol=1e-11, atol=1e-12)
        dec.commit_rows(c2, 0, r1, [0])


def test_verify_equals_recompute_without_cache():
    w = _model(SMALL, 6)
    ctx = uniform_tokens(30, SMALL.vocab, 7, "ctx")
    chunk = uniform_tokens(9, SMALL.vocab, 8, "chunk")
    cache = dec.Cache.empty(1, SMALL.n_layers, SMALL.n_kv_heads, SMALL.head_dim)
    dec.prefill(w, cache, ctx[None, :], EXACT, chunk=30)
    res = dec.verify_forward(w, cache, chunk[None, :], None, range(9), EXACT)
    full = np.concatenate([ctx, chunk])
    empty = dec.Cache.empty(1, SMALL.n_layers, SMALL.n_kv_heads, SMALL.head_dim)
    ref = dec.verify_forward(w, empty, full[None, :], None, range(30, 39), EXACT)
    np.testing.assert_allclose(res["logits"], ref["logits"], rtol=1e-11, atol=1e-12)


def test_chunked_prefill_equals_one_shot():
    w = _model(SMALL, 9)
    ctx = uniform_tokens(40, SMALL.vocab, 10, "ctx")[None, :]
    a = dec.Cache.empty(1, SMALL.n_layers, SMALL.n_kv_heads, SMALL.head_dim)
    b = dec.Cache.empty(1, SMALL.n_layers, SMALL.n_kv_heads, SMALL.head_dim)
    dec.prefill(w, a, ctx, EXACT, chunk=40)
    dec.prefill(w, b, ctx, EXACT, chunk=6)
    for l in range(SMALL.n_layers):
        np.testing.assert_allclose(a.k[0][l], b.k[0][l], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(a.v[0][l], b.v[0][l], rtol=1e-11, atol=1e-12)


def test_tree_branch_equals_linear_chunk():
    """Rows of a runner-up branch see the audio rows and their own branch only, at
    positions C + depth: identical to a linear verify of [audio ; branch]."""
    w = _model(SMALL, 12)
    cache = _prefilled(w, 17)
    L_a, gamma, nb = 4, 5, 3
    audio = uniform_tokens(L_a, SMALL.vocab, 13, "a")
    main = uniform_tokens(gamma, SMALL.vocab, 14, "m")
    branch = uniform_tokens(nb, SMALL.vocab, 15, "b")
    toks = np.concatenate([audio, main, branch])
    T = len(toks)
    parent = [j - 1 for j in range(T)]
    parent[L_a + gamma] = L_a - 1
    res = dec.verify_forward(w, cache, toks[None, :], parent, range(T), EXACT)
    lin_b = dec.verify_forward(w, cache, np.concatenate([audio, branch])[None, :], None, range(L_a + nb), EXACT)
    lin_m = dec.verify_forward(w, cache, np.concatenate([audio, main])[None, :], None, range(L_a + gamma), EXACT)
    np.testing.assert_allclose(res["logits"][0, L_a + gamma:], lin_b["logits"][0, L_a:], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(res["logits"][0, :L_a + gamma], lin_m["logits"][0], rtol=1e-11, atol=1e-12)
    for l in range(SMALL.n_layers):
        np.testing.assert_allclose(res["k_new"][0][l][L_a + gamma:], lin_b["k_new"][0][l][L_a:], rtol=1e-11, atol=1e-12)


# -- greedy acceptance ----------------------------------------------------------------

def test_greedy_chain_walk_equals_min_formula():
    rng = np.random.default_rng(3)
    for _ in range(300):
        gamma = int(rng.integers(1, 9))
        L_a = int(rng.integers(1, 4))
        drafts = list(rng.integers(0, 3, gamma))
        am = list(rng.integers(0, 3, gamma + 1))
        toks = list(rng.integers(0, 3, L_a)) + drafts
        n, nxt, path = acc.accept_greedy(toks, None, L_a, range(L_a - 1, L_a + gamma), am)
        assert n == acc.greedy_n_chain(drafts, am[:gamma])
        assert nxt == am[n] and path == list(range(L_a, L_a + n))
        assert 0 <= n <= gamma  # at least one token (n accepted + the correction) per pass


def _ar_continuation(w, cache, audio, n):
    c = cache.copy()
    out, _ = dec.greedy_decode(w, c, audio, n, EXACT)
    return out


def test_brute_force_all_drafts_tiny_vocab():
    """V = 8, L_a = 2, gamma = 3: for all 8^3 drafts, verify + greedy acceptance accepts
    exactly the longest prefix that matches greedy decoding, and commits the AR tokens."""
    w = _model(TINY, 21, std=0.5)
    cache = _prefilled(w, 9)
    audio = np.array([3, 6])
    ar = _ar_continuation(w, cache, audio, 4)
    for drafts in itertools.product(range(8), repeat=3):
        toks = np.concatenate([audio, drafts])
        res = dec.verify_forward(w, cache, toks[None, :], None, range(1, 5), EXACT)
        am = [acc.argmax_lowest(r) for r in res["logits"][0]]
        n, nxt, _ = acc.accept_greedy(list(toks), None, 2, range(1, 5), am)
        expect = 0
        while expect < 3 and drafts[expect] == ar[expect]:
            expect += 1
        assert n == expect
        assert list(drafts[:n]) + [nxt] == ar[:n + 1]


def test_corrupted_draft_and_silence_scenarios():
    w = _model(SMALL, 31)
    cache = _prefilled(w, 20)
    sil = np.zeros(5, dtype=np.int64)
    gamma = 6
    drafts = _ar_continuation(w, cache, sil, gamma + 1)
    # audio == silence, drafts == greedy decoding under silence: full acceptance + bonus
    toks = np.concatenate([sil, drafts[:gamma]])
    rows = list(range(4, 4 + gamma + 1))
    res = dec.verify_forward(w, cache, toks[None, :], None, rows, EXACT)
    am = [acc.argmax_lowest(r) for r in res["logits"][0]]
    n, nxt, _ = acc.accept_greedy(list(toks), None, 5, rows, am)
    assert n == gamma and nxt == drafts[gamma]
    # draft j replaced: n = j - 1 (1-based j)
    for j in range(1, gamma + 1):
        bad = list(drafts[:gamma])
        bad[j - 1] = (bad[j - 1] + 1) % SMALL.vocab
        toks = np.concatenate([sil, bad])
        res = dec.verify_forward(w, cache, toks[None, :], None, rows, EXACT)
        am = [acc.argmax_lowest(r) for r in res["logits"][0]]
        n, nxt, _ = acc.accept_greedy(list(toks), None, 5, rows, am)
        assert n == j - 1 and nxt == drafts[j - 1]


def test_tree_acceptance_takes_the_runner_up_branch():
    w = _model(SMALL, 41)
    cache = _prefilled(w, 15)
    audio = uniform_tokens(4, SMALL.vocab, 42, "a")
    ar = _ar_continuation(w, cache, audio, 4)          # the true continuation
    main = [(ar[0] + 1) % SMALL.vocab, 7, 8]            # wrong first token
    branch = ar[:3]                                     # runner-up branch = truth
    toks = np.concatenate([audio, main, branch])
    T = len(toks)
    parent = [j - 1 for j in range(T)]
    parent[7] = 3
    rows = list(range(3, T))
    res = dec.verify_forward(w, cache, toks[None, :], parent, rows, EXACT)
    am = [acc.argmax_lowest(r) for r in res["logits"][0]]
    n, nxt, path = acc.accept_greedy(list(toks), parent, 4, rows, am)
    assert n == 3 and path == [7, 8, 9] and nxt == ar[3]
    keep, moves = acc.commit_plan(15, 4, path)
    assert keep == 15 + 4 + 3 and moves == [(15 + 7, 15 + 4), (15 + 8, 15 + 5), (15 + 9, 15 + 6)]


def test_commit_then_decode_equals_feeding_committed_tokens():
    """After the commit (including a branch compaction), decoding one more token from the
    rolled-back cache equals decoding from a cache built by feeding the committed tokens."""
    w = _model(SMALL, 51)
    cache = _prefilled(w, 12)
    C = cache.length(0)
    audio = uniform_tokens(3, SMALL.vocab, 52, "a")
    ar = _ar_continuation(w, cache, audio, 3)
    main = [(ar[0] + 5) % SMALL.vocab, 1]
    branch = ar[:2]
    toks = np.concatenate([audio, main, branch])
    T = len(toks)
    parent = [j - 1 for j in range(T)]
    parent[5] = 2
    rows = list(range(2, T))
    res = dec.verify_forward(w, cache, toks[None, :], parent, rows, EXACT)
    am = [acc.argmax_lowest(r) for r in res["logits"][0]]
    n, nxt, path = acc.accept_greedy(list(toks), parent, 3, rows, am)
    assert n == 2 and nxt == ar[2]
    keep, moves = acc.commit_plan(C, 3, path)
    rolled = cache.copy()
    for l in range(SMALL.n_layers):
        k = np.concatenate([cache.k[0][l], res["k_new"][0][l]])
        v = np.concatenate([cache.v[0][l], res["v_new"][0][l]])
        rolled.k[0][l], rolled.v[0][l] = acc.apply_rollback(k, v, keep, moves)
    fed = cache.copy()
    dec.prefill(w, fed, np.concatenate([audio, branch])[None, :], EXACT, chunk=1)
    for l in range(SMALL.n_layers):
        np.testing.assert_allclose(rolled.k[0][l], fed.k[0][l], rtol=1e-11, atol=1e-12)
    a = dec.verify_forward(w, rolled, np.array([[nxt]]), None, [0], EXACT)["logits"]
    b = dec.verify_forward(w, fed, np.array([[nxt]]), None, [0], EXACT)["logits"]
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)
    # idempotent
    k2, v2 = acc.apply_rollback(rolled.k[0][0], rolled.v[0][0], keep, [])
    np.testing.assert_array_equal(k2, rolled.k[0][0])


def test_bf16_mode_rounds_stored_values():
    w = _model(SMALL_BF, 61, std=0.1)
    cache = _prefilled(w, 10, mode=BF16)
    res = dec.verify_forward(w, cache, uniform_tokens(5, SMALL_BF.vocab, 62)[None, :], None, range(5), BF16,
                             want_attn=True)
    for l in range(SMALL_BF.n_layers):
        for arr in (res["k_new"][0][l], res["v_new"][0][l], res["attn"][0][l]):
            np.testing.assert_array_equal(arr, round_bf16(arr))
    h = res["hidden"]
    np.testing.assert_array_equal(h, round_f32(h))
    # the KV-only mode rounds exactly the cache entries
    kv_only = dec.verify_forward(w, cache, uniform_tokens(5, SMALL_BF.vocab, 62)[None, :], None, range(5), BF16_KV,
                                 want_attn=True)
    for l in range(SMALL_BF.n_layers):
        for arr in (kv_only["k_new"][0][l], kv_only["v_new"][0][l]):
            np.testing.assert_array_equal(arr, round_bf16(arr))
    assert not np.array_equal(kv_only["attn"][0][0], round_bf16(kv_only["attn"][0][0]))
    # and the bf16 pass stays close to the exact one on the same (bf16-valued) weights
    ex = dec.verify_forward(w, cache, uniform_tokens(5, SMALL_BF.vocab, 62)[None, :], None, range(5), EXACT)
    assert np.max(np.abs(ex["logits"] - res["logits"])) < 0.05 * np.max(np.abs(ex["logits"]))


# -- the activation and the attention scale --------------------------------------------

def test_silu_closed_forms():
    """silu(x) = x * sigmoid(x).  Because sigmoid(x) + sigmoid(-x) = 1, silu(x) - silu(-x)
    equals x exactly; silu(x) / x tends to 1 for large x and silu(x) to 0 for very
    negative x (a swapped sign would give the opposite limits); its minimum sits at
    x = -(1 + W(1/e)) with value -W(1/e), W the Lambert W function (scipy)."""
    from scipy.optimize import minimize_scalar
    from scipy.special import lambertw
    x = np.linspace(-12.0, 12.0, 97)
    np.testing.assert_allclose(dec.silu(x) - dec.silu(-x), x, rtol=0, atol=1e-14)
    assert dec.silu(np.array(0.0)) == 0.0
    np.testing.assert_allclose(dec.silu(np.array([40.0, 60.0])) / np.array([40.0, 60.0]), 1.0, rtol=1e-15)
    assert abs(float(dec.silu(np.array(-60.0)))) < 1e-20
    w = float(lambertw(np.exp(-1.0)).real)
    r = minimize_scalar(lambda t: float(dec.silu(np.array(t))), bracket=(-3.0, -1.0, 0.0), tol=1e-12)
    assert abs(r.x + 1.0 + w) < 1e-6 and abs(r.fun + w) < 1e-12


@pytest.mark.parametrize("dh", [8, 64, 128])
def test_attention_scale_is_inverse_sqrt_head_dim(dh):
    """One query against two cached keys with dot products a and b: the two attention
    weights are softmax([a, b] / sqrt(dh)), so with values e_0 and e_1 the output is
    (sigmoid((a - b) / sqrt(dh)), sigmoid((b - a) / sqrt(dh))).  A scale of 1/dh or none
    at all gives other weights at every head dimension tested."""
    a, b = 6.0, -2.0
    q = np.zeros((1, 1, dh))
    q[0, 0, 0] = 1.0
    Kc = np.zeros((2, 1, dh))
    Kc[0, 0, 0] = a
    Kc[1, 0, 0] = b
    Kc[1, 0, 1] = 3.0            # orthogonal to q: does not change q . k
    Vc = np.zeros((2, 1, dh))
    Vc[0, 0, 0] = 1.0
    Vc[1, 0, 1] = 1.0
    empty = np.zeros((1, 1, dh))
    o = dec.attend(q, Kc, Vc, empty, empty, np.zeros((1, 1), bool))[0]
    w0 = 1.0 / (1.0 + math.exp(-(a - b) / math.sqrt(dh)))
    np.testing.assert_allclose(o[:2], [w0, 1.0 - w0], rtol=0, atol=1e-15)
    for wrong in (1.0 / dh, 1.0):
        assert abs(o[0] - 1.0 / (1.0 + math.exp(-(a - b) * wrong))) > 1e-3
