"""Oracle hypothesis pool (test infrastructure only).

"Decode Before You Hear: Speculative Listening" (page 1), section "Method steps":
step 3 stores each chunk's draft together with every earlier draft of the session
in an N-gram-indexed pool; step 5 looks up the longest N-gram that matches the end of
what has been output so far and splices its continuation into the next forward.

Readings where the page is silent (the plainest ones): n-grams are taken inside one
draft and count only when at least one token of that draft follows them; among
occurrences of the matched n-gram the most recent one wins (latest draft, latest
position); the continuation runs to the end of that draft, capped at max_out tokens.

This is the definition written out as a scan over every stored position (no index).
"""
from __future__ import annotations

from typing import List, Sequence, Tuple


class Pool:
    def __init__(self, max_n: int):
        self.max_n = max_n
        self.drafts: List[List[int]] = []

    def insert(self, draft: Sequence[int]) -> None:
        self.drafts.append([int(t) for t in draft])

    def lookup(self, suffix: Sequence[int], max_out: int) -> Tuple[List[int], int]:
        """Returns (continuation, n matched); ([], 0) when no n-gram of the suffix is stored."""
        suffix = [int(t) for t in suffix]
        for n in range(min(self.max_n, len(suffix)), 0, -1):
            gram = suffix[len(suffix) - n:]
            best = None
            for d in self.drafts:            # in insertion order: later occurrences replace earlier
                for p in range(n - 1, len(d) - 1):
                    if d[p - n + 1:p + 1] == gram:
                        best = d[p + 1:]
            if best is not None:
                return best[:max_out], n
        return [], 0
