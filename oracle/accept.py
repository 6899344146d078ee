"""Oracle greedy acceptance and KV commit (test infrastructure only).

"Decode Before You Hear: Speculative Listening" (page 1), section "Method
steps", step 4: accept n = min({i-1 : 1 <= i <= gamma, y~_i != argmax p_i} U
{gamma}) draft tokens and commit the correction argmax p_{n+1}; the pipeline
commits at least one token per forward (same section, closing sentence).

With a runner-up branch (step 2) the chunk is a tree: starting at the last audio
row, the child whose token equals the current row's argmax is accepted and the
walk descends into it; siblings carry distinct tokens, so at most one matches.
On a chain this walk is exactly the min formula above (`greedy_n_chain`).
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np


def argmax_lowest(row: np.ndarray) -> int:
    """Index of the largest value; the lowest such index on ties."""
    return int(np.argmax(row))


def top2_margin(row: np.ndarray) -> float:
    """Largest minus second-largest value (0 when the maximum is attained twice)."""
    i = int(np.argmax(row))
    rest = np.delete(row, i)
    return float(row[i] - rest.max())


def greedy_n_chain(drafts: Sequence[int], argmax_p: Sequence[int]) -> int:
    """n = min({i-1 : 1<=i<=gamma, drafts_i != argmax p_i} U {gamma}); 1-based i as printed."""
    gamma = len(drafts)
    cands = [i - 1 for i in range(1, gamma + 1) if drafts[i - 1] != argmax_p[i - 1]]
    return min(cands + [gamma])


def accept_greedy(tokens: Sequence[int], parent: Optional[Sequence[int]], L_a: int,
                  logit_rows: Sequence[int], argmax_rows: Sequence[int]) -> Tuple[int, int, List[int]]:
    """Tree walk for one sequence.  tokens: the T chunk tokens; argmax_rows[r] is the
    argmax of the distribution at chunk row logit_rows[r].

    Returns (n, next_token, path): n accepted draft rows, the correction/bonus token
    argmax at the last accepted row, and the accepted rows in order."""
    T = len(tokens)
    rmap = {row: r for r, row in enumerate(logit_rows)}
    par = [j - 1 for j in range(T)] if parent is None else list(parent)
    node = L_a - 1
    path: List[int] = []
    while True:
        a = argmax_rows[rmap[node]]
        kids = [j for j in range(L_a, T) if par[j] == node]
        match = [j for j in kids if tokens[j] == a]
        if len(match) > 1:
            raise ValueError("sibling rows carry the same token")
        if not match:
            return len(path), int(a), path
        node = match[0]
        path.append(node)


def commit_plan(C: int, L_a: int, path: Sequence[int]):
    """KV bookkeeping after acceptance.  Chunk row j was written at slot C + j.  The
    committed length is C + L_a + n; accepted row path[i] must end at slot C + L_a + i,
    so rows that are elsewhere (a winning runner-up branch) are moved.
    Returns (keep_len, [(src_slot, dst_slot), ...])."""
    moves = [(C + row, C + L_a + i) for i, row in enumerate(path) if row != L_a + i]
    return C + L_a + len(path), moves


def apply_rollback(k: np.ndarray, v: np.ndarray, keep_len: int, moves) -> Tuple[np.ndarray, np.ndarray]:
    """Apply a commit plan to logical slot arrays k, v ([slots, ...] for one layer):
    copy every move's source slot to its destination, then keep the first keep_len slots."""
    k, v = k.copy(), v.copy()
    for src, dst in moves:
        k[dst] = k[src]
        v[dst] = v[src]
    return k[:keep_len], v[:keep_len]
