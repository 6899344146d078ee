"""Pins of the oracle hypothesis pool (CPU only): page 1 ("Decode Before You Hear"),
method steps 3 and 5, and its case study of a tool call whose arguments were already
drafted in earlier chunks while the user was still talking.  Worked examples written
out by hand from the definition (longest n-gram of the output's suffix, most recent
occurrence, continuation to the end of its draft), plus properties checked by brute
force on random pools."""
import numpy as np

from oracle.pool import Pool


def test_case_study_tool_call_already_drafted():
    """Tokens: 1 'find', 2 '(', 3 'TYO', 4 ',', 5 'Fri', 6 ')', 9 filler.  An early chunk
    drafted the call; once the output reads '... find (' the pool continues with the rest
    of the call."""
    pool = Pool(max_n=4)
    pool.insert([9, 9, 1, 2, 3, 4, 5, 6])
    pool.insert([9, 7, 9])
    cont, n = pool.lookup([9, 8, 1, 2], max_out=16)
    assert cont == [3, 4, 5, 6] and n == 2
    assert pool.lookup([1, 2], max_out=2) == ([3, 4], 2)


def test_longest_match_and_most_recent_occurrence():
    pool = Pool(max_n=3)
    pool.insert([5, 6, 7, 1])          # 6 7 -> 1
    pool.insert([4, 6, 7, 2, 3])       # 4 6 7 -> 2 3 ; 6 7 -> 2 3 (more recent)
    pool.insert([7, 8])                # 7 -> 8 (most recent for the 1-gram 7)
    assert pool.lookup([5, 6, 7], 10) == ([1], 3)          # the 3-gram 5 6 7 exists only in draft 0
    assert pool.lookup([0, 6, 7], 10) == ([2, 3], 2)       # 2-gram, most recent occurrence
    assert pool.lookup([0, 0, 7], 10) == ([8], 1)          # 1-gram 7: latest draft wins
    assert pool.lookup([0, 0, 3], 10) == ([], 0)           # 3 ends its draft: nothing follows it
    assert pool.lookup([], 10) == ([], 0)


def test_random_pools_against_brute_force_properties():
    """On random pools: the continuation follows a true occurrence of the matched n-gram
    inside one draft, no longer suffix n-gram occurs with a follower, and no later
    occurrence of the matched n-gram exists."""
    rng = np.random.default_rng(3)
    for _ in range(200):
        pool = Pool(max_n=5)
        drafts = [list(rng.integers(0, 6, size=rng.integers(1, 12))) for _ in range(rng.integers(1, 6))]
        for d in drafts:
            pool.insert(d)
        suffix = list(rng.integers(0, 6, size=rng.integers(0, 8)))
        cont, n = pool.lookup(suffix, max_out=4)
        occ = {}
        for di, d in enumerate(drafts):
            for m in range(1, 6):
                for p in range(m - 1, len(d) - 1):
                    occ.setdefault((m, tuple(d[p - m + 1:p + 1])), []).append((di, p))
        longest = 0
        for m in range(1, min(5, len(suffix)) + 1):
            if (m, tuple(suffix[len(suffix) - m:])) in occ:
                longest = m
        assert n == longest
        if n:
            di, p = max(occ[(n, tuple(suffix[len(suffix) - n:]))])
            assert cont == drafts[di][p + 1:p + 5]
        else:
            assert cont == []
