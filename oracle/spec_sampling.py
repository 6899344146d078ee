"""Oracle speculative-sampling acceptance (test infrastructure only).

"speculative-decoding-omni" (page 3), section 2 (why it is lossless): for each
draft token x_i in order, accept with probability min(1, p(x_i)/q(x_i)); on
the first rejection draw a replacement from norm(max(0, p - q)) and drop the
remaining drafts; if all k drafts are accepted draw one bonus token from p.
p is the target distribution and q the draft distribution; the same section
shows the output is distributed exactly as p and that one position accepts with
probability 1 - TV(p, q).  Section 3 gives the chain length
1 + sum_{i<=k} alpha^i = (1 - alpha^{k+1}) / (1 - alpha) for a constant alpha.

The random numbers are inputs: u_accept[b, i] decides position i and
u_sample[b, j] drives the inverse-CDF draw made at position j (residual at a
rejection, bonus at j = k).
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

# decisions closer than this to the threshold are reported as flagged
FLAG_TOL = 1e-6


def softmax(z: np.ndarray, temperature: float = 1.0) -> np.ndarray:
    y = np.asarray(z, dtype=np.float64) / temperature
    y = y - y.max()
    e = np.exp(y)
    return e / e.sum()


def inverse_cdf(weights: np.ndarray, u: float):
    """Smallest index x with sum_{y<=x} w_y > u * sum(w) (w >= 0, not all zero).
    Returns (x, distance of the threshold u*S to the nearest partial sum)."""
    c = np.cumsum(weights)
    target = u * c[-1]
    x = int(np.searchsorted(c, target, side="right"))
    x = min(x, len(c) - 1)
    dist = float(np.min(np.abs(c - target)))
    return x, dist


def accept_one_sequence(tgt: np.ndarray, drf: np.ndarray, drafts: Sequence[int],
                        u_acc: Sequence[float], u_smp: Sequence[float], temperature: float = 1.0):
    """tgt [k+1, V], drf [k, V] logits; drafts [k].  Returns (n, token, flagged)."""
    k = len(drafts)
    flagged = False
    for i in range(k):
        p = softmax(tgt[i], temperature)
        q = softmax(drf[i], temperature)
        x = int(drafts[i])
        if q[x] > 0.0:
            ratio = p[x] / q[x]
            accept = u_acc[i] < ratio
            flagged |= abs(u_acc[i] - ratio) < FLAG_TOL
        else:  # a draft outside q's support: accept only if p can produce it
            accept = p[x] > 0.0
        if not accept:
            resid = np.maximum(0.0, p - q)
            if resid.sum() <= 0.0:  # p == q up to rounding: the residual is empty
                resid = p
            tok, dist = inverse_cdf(resid, u_smp[i])
            flagged |= dist < FLAG_TOL
            return i, tok, flagged
    p = softmax(tgt[k], temperature)
    tok, dist = inverse_cdf(p, u_smp[k])
    flagged |= dist < FLAG_TOL
    return k, tok, flagged


def accept_sample(tgt: np.ndarray, drf: np.ndarray, drafts: np.ndarray, u_acc: np.ndarray,
                  u_smp: np.ndarray, temperature: float = 1.0):
    """Batched: tgt [B, k+1, V], drf [B, k, V], drafts [B, k], u_acc [B, k], u_smp [B, k+1].
    Returns n [B], token [B], flagged [B] (bool)."""
    B = tgt.shape[0]
    n = np.zeros(B, dtype=np.int64)
    tok = np.zeros(B, dtype=np.int64)
    fl = np.zeros(B, dtype=bool)
    for b in range(B):
        n[b], tok[b], fl[b] = accept_one_sequence(tgt[b], drf[b], drafts[b], u_acc[b], u_smp[b], temperature)
    return n, tok, fl


def total_variation(p: np.ndarray, q: np.ndarray) -> float:
    return 0.5 * float(np.abs(np.asarray(p) - np.asarray(q)).sum())


def expected_tokens_per_pass(alphas: Sequence[float]) -> float:
    """1 + sum_i prod_{j<=i} alpha_j: tokens produced per target pass when position i
    is accepted with probability alpha_i given all earlier ones were (page 3, section 3)."""
    total, run = 1.0, 1.0
    for a in alphas:
        run *= a
        total += run
    return total


def net_speedup(tokens_per_pass: float, k: int, c: float) -> float:
    """tokens per pass / (1 + k c), c = draft cost relative to one target pass (page 3, section 3)."""
    return tokens_per_pass / (1.0 + k * c)
