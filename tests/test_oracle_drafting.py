"""Pins of the oracle's idle-window drafting (CPU only).

Page 1 ("Decode Before You Hear"), method steps 1-2: the greedy draft under a
hypothesised chunk, and a runner-up branch from the best first token other than the
greedy one; its weaknesses / future-directions sections: a top-k first-token tree.
Pinned against: plain greedy decoding (branch 0), greedy decoding with the top token
excluded (branch 1), the ranking's definition by counting, and a recompute of every
drafted token's distribution from scratch without a cache.
"""
import numpy as np
import pytest

from oracle import BF16_KV, EXACT
from oracle import decoder as dec
from oracle import drafting as dr
from synth.configs import ModelShape
from synth.gen import make_weights, uniform_tokens

TINY = ModelShape("tiny-draft", n_layers=2, d=32, n_heads=4, n_kv_heads=2, head_dim=8, ffn=48, vocab=23,
                  dtype="f32")
TINY_BF = ModelShape("tiny-draft-bf", n_layers=2, d=32, n_heads=4, n_kv_heads=2, head_dim=8, ffn=48, vocab=23,
                     dtype="bf16")


def _setup(shape, n_ctx=9, seed=5):
    w = make_weights(shape, seed, std=0.4)
    cache = dec.Cache.empty(1, shape.n_layers, shape.n_kv_heads, shape.head_dim)
    ctx = uniform_tokens(n_ctx, shape.vocab, seed + 1, "ctx")
    dec.prefill(w, cache, ctx[None, :], EXACT, chunk=4)
    return w, cache, ctx


def test_ranking_by_counting():
    """The k-th pick has exactly k entries ranking before it: larger values, or equal
    values at lower indices."""
    rng = np.random.default_rng(1)
    for _ in range(20):
        z = rng.integers(-3, 4, size=40).astype(np.float64)      # many ties
        picks = dr.ranked(z, 12)
        assert len(set(picks)) == 12
        for k, i in enumerate(picks):
            before = sum(1 for j in range(len(z)) if z[j] > z[i] or (z[j] == z[i] and j < i))
            assert before == k


@pytest.mark.parametrize("shape,mode", [(TINY, EXACT), (TINY_BF, BF16_KV)])
def test_main_branch_is_greedy_decoding(shape, mode):
    w, cache, _ = _setup(shape)
    chunk = np.zeros(4, dtype=np.int64)
    drafts, _, _ = dr.draft_tree(w, cache, chunk, [6], mode)
    ref, _ = dec.greedy_decode(w, cache.copy(), chunk, 6, mode)
    assert drafts[0] == ref


def test_runner_up_is_greedy_decoding_without_the_top_token():
    w, cache, _ = _setup(TINY)
    chunk = np.zeros(3, dtype=np.int64)
    drafts, _, _ = dr.draft_tree(w, cache, chunk, [5, 4], EXACT)
    ref, _ = dec.greedy_decode(w, cache.copy(), chunk, 4, EXACT, exclude_first=drafts[0][0])
    assert drafts[1] == ref
    assert drafts[0][0] != drafts[1][0]


def test_every_draft_token_is_the_argmax_of_a_cache_free_recompute():
    """Branch k's token i+1 is the argmax of p(. | context, chunk, branch[:i+1]) computed
    from scratch (empty cache, the whole sequence as one chunk); its first token has rank
    k under the chunk's last row, recomputed the same way."""
    w, cache, ctx = _setup(TINY)
    chunk = np.array([0, 0, 7], dtype=np.int64)
    lens = [4, 3, 2, 2]
    drafts, margins, gaps = dr.draft_tree(w, cache, chunk, lens, EXACT)
    empty = dec.Cache.empty(1, TINY.n_layers, TINY.n_kv_heads, TINY.head_dim)
    seq = np.concatenate([ctx, chunk])
    p1 = dec.verify_forward(w, empty, seq[None, :], None, [len(seq) - 1], EXACT)["logits"][0, 0]
    firsts = [d[0] for d in drafts]
    for k, t in enumerate(firsts):
        assert sum(1 for j in range(TINY.vocab) if p1[j] > p1[t] or (p1[j] == p1[t] and j < t)) == k
    for k, d in enumerate(drafts):
        assert len(d) == lens[k] and len(margins[k]) == lens[k]
        for i in range(1, len(d)):
            full = np.concatenate([seq, d[:i]])
            lg = dec.verify_forward(w, empty, full[None, :], None, [len(full) - 1], EXACT)["logits"][0, 0]
            assert d[i] == int(np.argmax(lg))
            srt = np.sort(lg)
            assert margins[k][i] == pytest.approx(srt[-1] - srt[-2], abs=1e-12)
    assert len(gaps) == 4 and all(g >= 0 for g in gaps)
