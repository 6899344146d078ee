"""Oracle drafting in the idle window (test infrastructure only).

"Decode Before You Hear: Speculative Listening" (page 1), section "Method steps":
step 1 drafts greedily under a hypothesised silent chunk,
y~_i = argmax_y p(y | x_{<t}, a_sil, y~_{<i}); step 2 starts a runner-up branch from
argmax over V minus {y~_1} of p(. | x_{<t}, a_sil) and decodes it the same way.  The
weaknesses and future-directions sections of the same page name a top-k first-token
tree as the generalisation: branch k starts from the (k+1)-th ranked first token.

Every branch is decoded here token by token (autoregressively, one row per forward
on a copy of the cache), the plain definition; ranks order larger logits first and
lower indices first among equal logits (the argmax tie rule).
"""
from __future__ import annotations

from typing import List, Sequence

import numpy as np

from . import EXACT
from .decoder import Cache, commit_rows, verify_forward


def ranked(logits: np.ndarray, k: int) -> List[int]:
    """The k best indices of a row: larger value first, lower index first on ties."""
    order = sorted(range(len(logits)), key=lambda i: (-float(logits[i]), i))
    return order[:k]


def rank_gaps(logits: np.ndarray, k: int) -> List[float]:
    """Gaps between the values at ranks j and j + 1 for j < k (how far each of the k
    picks is from changing places with the next one)."""
    top = np.sort(np.asarray(logits, dtype=np.float64))[::-1][:k + 1]
    return [float(top[j] - top[j + 1]) for j in range(min(k, len(top) - 1))]


def draft_tree(w, cache: Cache, chunk: Sequence[int], branch_len: Sequence[int], mode: str = EXACT):
    """Drafts of one sequence (B = 1) under the chunk `chunk` (1-D tokens).

    Returns (drafts, margins, gaps): drafts[k] is branch k's token list; margins[k][i]
    the top-2 margin of the distribution token i of branch k was chosen from (for
    i >= 1; margins[k][0] is the rank gap of its first token); gaps the first row's
    rank gaps.  The cache is not modified."""
    K = len(branch_len)
    base = cache.copy()
    res = verify_forward(w, base, np.asarray(chunk, dtype=np.int64)[None, :], None, [len(chunk) - 1], mode)
    commit_rows(base, 0, res, range(len(chunk)))
    p1 = res["logits"][0, 0]
    first = ranked(p1, K)
    gaps = rank_gaps(p1, K)
    drafts, margins = [], []
    for k in range(K):
        c = base.copy()
        toks = [first[k]]
        marg = [gaps[k] if k < len(gaps) else np.inf]
        if k > 0:
            marg[0] = min(marg[0], gaps[k - 1])
        while len(toks) < branch_len[k]:
            r = verify_forward(w, c, np.array([[toks[-1]]], dtype=np.int64), None, [0], mode)
            commit_rows(c, 0, r, [0])
            lg = r["logits"][0, 0]
            nxt = int(np.argmax(lg))
            srt = np.sort(lg)
            marg.append(float(srt[-1] - srt[-2]))
            toks.append(nxt)
        drafts.append(toks)
        margins.append(marg)
    return drafts, margins, gaps
