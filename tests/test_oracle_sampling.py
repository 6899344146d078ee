"""Pins of the oracle's speculative-sampling acceptance (CPU only).

Checked against what page 3 ("speculative-decoding-omni") fixes: the worked
example of section 2, the identities P(accept) = 1 - TV and output == p, the
chain formula and printed numbers of section 3, and the special cases that
reduce to greedy acceptance.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import spec_sampling as ss
from synth.gen import philox_uniforms

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _enumerate_first_token(p, q, n_acc=4096, n_smp=512):
    """Exact distribution of the first emitted token for k = 1 over a midpoint grid of
    both uniforms, with the draft x drawn from q by enumeration.  Returns (dist, P(accept)).

    Given a rejection the replacement depends only on the sampling uniform; the grid of
    that uniform is enumerated under two different rejecting acceptance uniforms, which
    must agree."""
    V = len(p)
    tgt = np.log(np.stack([p, p]))       # softmax(log p) = p
    drf = np.log(np.asarray(q))[None, :]
    dist = np.zeros(V)
    acc = 0.0
    ua = (np.arange(n_acc) + 0.5) / n_acc
    us = (np.arange(n_smp) + 0.5) / n_smp
    for x in range(V):
        if q[x] == 0:
            continue
        rejecting = []
        for a in ua:
            n, _, _ = ss.accept_one_sequence(tgt, drf, [x], [a], [0.5, 0.5])
            if n == 1:
                dist[x] += q[x] / n_acc
                acc += q[x] / n_acc
            else:
                rejecting.append(a)
        if rejecting:
            hists = []
            for a in (rejecting[0], rejecting[-1]):
                h = np.zeros(V)
                for s in us:
                    _, tok, _ = ss.accept_one_sequence(tgt, drf, [x], [a], [s, 0.5])
                    h[tok] += 1.0 / n_smp
                hists.append(h)
            assert np.array_equal(hists[0], hists[1])
            dist += q[x] * len(rejecting) / n_acc * hists[0]
    return dist, acc


def test_worked_example_exact():
    g = _load("p3_worked_example.json")
    p, q = np.array(g["p"]), np.array(g["q"])
    assert ss.total_variation(p, q) == pytest.approx(g["tv"], abs=1e-15)
    dist, acc = _enumerate_first_token(p, q, n_acc=4096, n_smp=64)
    assert acc == pytest.approx(g["alpha"], abs=1e-12)
    np.testing.assert_allclose(dist, g["output_distribution"], atol=1e-12)
    # drafting B: accepted with probability 0.75; the rejected mass all goes to A
    tgt, drf = np.log(np.stack([p, p])), np.log(q)[None, :]
    ua = (np.arange(4096) + 0.5) / 4096
    accB = np.mean([ss.accept_one_sequence(tgt, drf, [1], [a], [0.5, 0.5])[0] for a in ua])
    assert accB == pytest.approx(g["accept_prob_of_B"], abs=1e-12)
    for s in (0.01, 0.5, 0.99):
        n, tok, _ = ss.accept_one_sequence(tgt, drf, [1], [0.9], [s, 0.5])
        assert n == 0 and tok == 0


def test_worked_example_monte_carlo_philox():
    g = _load("p3_worked_example.json")
    p, q = np.array(g["p"]), np.array(g["q"])
    N = 60000
    u0, u1 = philox_uniforms(1234, np.arange(N), np.zeros(N, dtype=np.int64), stream=0)
    _, u2 = philox_uniforms(1234, np.arange(N), np.zeros(N, dtype=np.int64), stream=2)
    # draft x ~ q by inverse transform of an independent uniform
    xs = np.searchsorted(np.cumsum(q), u2, side="right")
    tgt, drf = np.log(np.stack([p, p])), np.log(q)[None, :]
    first = np.empty(N, dtype=np.int64)
    acc = 0
    for t in range(N):
        n, tok, _ = ss.accept_one_sequence(tgt, drf, [int(xs[t])], [u0[t]], [u1[t], 0.5])
        first[t] = xs[t] if n == 1 else tok
        acc += n
    rate = acc / N
    sigma = math.sqrt(0.9 * 0.1 / N)
    assert abs(rate - 0.9) < 4 * sigma
    counts = np.bincount(first, minlength=3)
    chi2 = float(np.sum((counts - N * p) ** 2 / (N * p)))
    assert chi2 < 13.8  # chi-square, 2 dof, p = 0.001


@pytest.mark.parametrize("seed", range(6))
def test_tiny_vocab_output_equals_p_and_accept_is_one_minus_tv(seed):
    rng = np.random.default_rng(seed)
    V = 2 + seed % 5
    p = rng.dirichlet(np.ones(V))
    q = rng.dirichlet(np.ones(V))
    dist, acc = _enumerate_first_token(p, q, n_acc=2048, n_smp=1024)
    # grid quantisation: each uniform is resolved to 1/n
    assert acc == pytest.approx(1.0 - ss.total_variation(p, q), abs=2.0 / 2048)
    np.testing.assert_allclose(dist, p, atol=3.0 / 1024)


def test_special_cases():
    rng = np.random.default_rng(7)
    V = 5
    p = rng.dirichlet(np.ones(V))
    # q one-hot at x: the draft is always x and is accepted with probability p(x)
    x = 3
    q = np.full(V, 1e-300)
    q[x] = 1.0
    tgt, drf = np.log(np.stack([p, p])), np.log(q)[None, :]
    ua = (np.arange(4096) + 0.5) / 4096
    acc = np.mean([ss.accept_one_sequence(tgt, drf, [x], [a], [0.5, 0.5])[0] for a in ua])
    assert acc == pytest.approx(p[x], abs=1.0 / 4096)
    # p one-hot (temperature -> 0): accept exactly when the draft is p's argmax, and the
    # replacement is that argmax: greedy acceptance
    z = np.array([0.0, 5.0, 1.0, -2.0, 0.5]) * 1e4
    q2 = rng.dirichlet(np.ones(V))
    for x in range(V):
        for a in (0.01, 0.5, 0.99):
            n, tok, _ = ss.accept_one_sequence(np.stack([z, z]), np.log(q2)[None, :], [x], [a], [0.3, 0.3])
            assert (n == 1) == (x == 1)
            if n == 0:
                assert tok == 1
    # p == q: every draft accepted (ratio 1 > u), then a bonus token from p
    k = 4
    zz = rng.standard_normal((k + 1, V))
    for a in (0.0, 0.999999):
        n, tok, _ = ss.accept_one_sequence(zz, zz[:k], [0, 1, 2, 3], [a] * k, [0.2] * (k + 1))
        assert n == k
        assert tok == int(np.searchsorted(np.cumsum(ss.softmax(zz[k])), 0.2, side="right"))


def test_chain_numbers_of_page3():
    g = _load("p3_chain_numbers.json")
    a = g["per_position_accept"]
    # independent product model: sum of products ~ 1.62 accepted tokens
    assert ss.expected_tokens_per_pass(a) - 1.0 == pytest.approx(g["independent_sum_of_products"], abs=0.005)
    # constant alpha 0.8 over k = 7 gives accept_len 3.16, i.e. 4.16 tokens per pass
    k = g["k"]
    t = ss.expected_tokens_per_pass([g["equivalent_constant_alpha"]] * k)
    assert t - 1.0 == pytest.approx(g["reported_accept_len"], abs=0.005)
    alpha = g["equivalent_constant_alpha"]
    assert t == pytest.approx((1 - alpha ** (k + 1)) / (1 - alpha), rel=1e-12)  # closed form
    for c, s in g["net_speedup"].items():
        assert ss.net_speedup(g["tokens_per_pass"], k, float(c)) == pytest.approx(s, abs=0.005)
    tv = g["tv_vs_accept"]
    assert 1 - tv["raw_tv"] == pytest.approx(tv["accept_rate_epoch"], abs=1e-12)


def test_chain_mean_matches_product_formula():
    """k positions with fixed (p_i, q_i); drafts drawn from q_i; E[n] = sum_i prod_{j<=i} alpha_j
    with alpha_j = 1 - TV(p_j, q_j) (the acceptance events are independent here)."""
    rng = np.random.default_rng(11)
    V, k, N = 6, 4, 20000
    zp = rng.standard_normal((k + 1, V)) * 1.5
    zq = zp[:k] + 0.7 * rng.standard_normal((k, V))
    alphas = [1 - ss.total_variation(ss.softmax(zp[i]), ss.softmax(zq[i])) for i in range(k)]
    expect_n = ss.expected_tokens_per_pass(alphas) - 1.0
    u0, _ = philox_uniforms(99, np.arange(N)[:, None], np.arange(k)[None, :], stream=0)
    _, u1 = philox_uniforms(99, np.arange(N)[:, None], np.arange(k + 1)[None, :], stream=1)
    u2, _ = philox_uniforms(99, np.arange(N)[:, None], np.arange(k)[None, :], stream=3)
    cq = [np.cumsum(ss.softmax(zq[i])) for i in range(k)]
    tot = 0
    per_pos_acc = np.zeros(k)
    per_pos_tries = np.zeros(k)
    for t in range(N):
        xs = [min(int(np.searchsorted(cq[i], u2[t, i], side="right")), V - 1) for i in range(k)]
        n, _, _ = ss.accept_one_sequence(zp, zq, xs, u0[t], u1[t])
        tot += n
        per_pos_tries[: min(n + 1, k)] += 1
        per_pos_acc[:n] += 1
    mean = tot / N
    assert abs(mean - expect_n) < 0.03
    # per position, acceptance given the position was tried equals 1 - TV
    np.testing.assert_allclose(per_pos_acc / per_pos_tries, alphas, atol=0.02)


def test_inverse_cdf_is_smallest_index_over_threshold():
    w = np.array([0.0, 0.25, 0.0, 0.5, 0.25])
    assert ss.inverse_cdf(w, 0.0)[0] == 1
    assert ss.inverse_cdf(w, 0.2)[0] == 1
    assert ss.inverse_cdf(w, 0.26)[0] == 3
    assert ss.inverse_cdf(w, 0.76)[0] == 4
    assert ss.inverse_cdf(w, 0.999999)[0] == 4


@pytest.mark.parametrize("seed", range(4))
def test_masked_vocabulary_entries(seed):
    """Logits of -inf (masked entries) have probability 0: the emitted token still has
    distribution p (section 2's losslessness, now with zeros in p and q), so a token
    masked in p is never emitted, and a draft outside q's support is accepted exactly
    when p can produce it."""
    rng = np.random.default_rng(40 + seed)
    V = 5 + seed % 2
    p = rng.dirichlet(np.ones(V))
    q = rng.dirichlet(np.ones(V))
    p[rng.choice(V, 2, replace=False)] = 0.0
    q[rng.choice(V, 2, replace=False)] = 0.0
    p /= p.sum()
    q /= q.sum()
    with np.errstate(divide="ignore"):
        dist, acc = _enumerate_first_token(p, q, n_acc=2048, n_smp=1024)
        assert np.all(dist[p == 0.0] == 0.0)
        assert acc == pytest.approx(1.0 - ss.total_variation(p, q), abs=2.0 / 2048)
        np.testing.assert_allclose(dist, p, atol=3.0 / 1024)
        tgt, drf = np.log(np.stack([p, p])), np.log(q)[None, :]
    for x in np.nonzero(q == 0.0)[0]:
        n, tok, _ = ss.accept_one_sequence(tgt, drf, [int(x)], [0.999], [0.5, 0.5])
        assert n == (1 if p[x] > 0.0 else 0)
        assert p[tok] > 0.0


# -- temperature ------------------------------------------------------------------------

def test_temperature_to_infinity_gives_uniform_distributions():
    """p = softmax(z / T): as T grows both distributions become uniform over V, so every
    ratio p(x)/q(x) is 1 and every draft is accepted (u < 1); the bonus draw of a uniform
    distribution over V at u is floor(u V).  A temperature that multiplied the logits
    instead would make p and q one-hot and reject."""
    rng = np.random.default_rng(7)
    V, k = 11, 4
    tgt = rng.standard_normal((k + 1, V)) * 3.0
    drf = rng.standard_normal((k, V)) * 3.0
    drafts = rng.integers(0, V, size=k)
    u_acc = np.full(k, 1.0 - 1e-9)
    for us in (0.0, 0.3, 0.95):
        n, tok, _ = ss.accept_one_sequence(tgt, drf, drafts, u_acc, [0.5] * k + [us], temperature=1e12)
        assert n == k and tok == int(us * V)


def test_temperature_two_on_two_tokens():
    """V = 2, T = 2: p(0) = sigmoid((z0 - z1) / 2), and likewise q.  The acceptance of draft
    0 switches exactly where u crosses p(0)/q(0)."""
    zp, zq = np.array([0.2, 0.9]), np.array([2.2, 0.1])
    p0 = 1.0 / (1.0 + math.exp(-(zp[0] - zp[1]) / 2.0))
    q0 = 1.0 / (1.0 + math.exp(-(zq[0] - zq[1]) / 2.0))
    ratio = p0 / q0
    assert ratio < 1.0
    tgt, drf = np.stack([zp, zp]), zq[None, :]
    for u, want in ((ratio - 1e-9, 1), (ratio + 1e-9, 0)):
        n, _, _ = ss.accept_one_sequence(tgt, drf, [0], [u], [0.5, 0.5], temperature=2.0)
        assert n == want
    # at T = 1 the same u decides differently (the ratio moves)
    r1 = (1.0 / (1.0 + math.exp(-(zp[0] - zp[1])))) / (1.0 / (1.0 + math.exp(-(zq[0] - zq[1]))))
    assert abs(r1 - ratio) > 1e-3


def test_temperature_to_zero_is_greedy_acceptance():
    """As T -> 0 the target is one-hot at its argmax: a draft equal to the argmax is
    accepted (p(x)/q(x) >= 1 with q one-hot too), any other draft is rejected and the
    replacement is the argmax (the residual max(0, p - q) is one-hot there)."""
    rng = np.random.default_rng(3)
    V, k = 9, 3
    tgt = rng.standard_normal((k + 1, V))
    am = tgt.argmax(axis=1)
    drf = tgt[:k].copy()
    drafts = am[:k].copy()
    drafts[2] = (am[2] + 1) % V
    drf[2, drafts[2]] = tgt[2].max() + 1.0   # q prefers the wrong token
    n, tok, _ = ss.accept_one_sequence(tgt, drf, drafts, [0.5] * k, [0.5] * (k + 1), temperature=1e-6)
    assert n == 2 and tok == am[2]


def test_philox_known_answer_vectors():
    """Philox4x32-10 against the known-answer vectors published with the Random123
    library (Salmon et al., SC'11): zero counter and key, all-ones, and the pi-digit
    counter and key."""
    from synth.gen import philox4x32_10
    cases = [([0, 0, 0, 0], [0, 0], [0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8]),
             ([0xffffffff] * 4, [0xffffffff] * 2, [0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd]),
             ([0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344], [0xa4093822, 0x299f31d0],
              [0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1])]
    for ctr, key, want in cases:
        got = philox4x32_10(np.array(ctr, dtype=np.uint32), np.array(key, dtype=np.uint32))
        assert [int(x) for x in got] == want
