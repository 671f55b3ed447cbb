"""Pins for the oracle's top-k selection: keep the k highest-scoring entries
("闪电索引机制（对应步骤二）"), lowest entry index winning ties, output in
ascending index order padded with -1."""
import itertools

import numpy as np

import oracle


def _dominance_subset(s, valid, kk):
    """The unique subset S of size kk whose members all beat every non-member
    (score higher, or equal score and lower index), found by enumeration."""
    n = len(s)
    found = []
    for S in itertools.combinations([j for j in range(n) if valid[j]], kk):
        inside = set(S)
        ok = all((s[i] > s[j]) or (s[i] == s[j] and i < j)
                 for i in inside for j in range(n) if valid[j] and j not in inside)
        if ok:
            found.append(sorted(S))
    assert len(found) == 1
    return found[0]


def test_exhaustive_small_with_ties():
    rng = np.random.default_rng(0)
    for trial in range(60):
        n = int(rng.integers(1, 10))
        s = rng.integers(-2, 3, size=n).astype(np.float64)  # many ties
        valid = rng.random(n) > 0.2
        s[~valid] = -np.inf
        for k in range(1, n + 3):
            idx, cnt = oracle.topk(s[None, :], k)
            kk = min(k, int(valid.sum()))
            want = _dominance_subset(s, valid, kk)
            assert cnt[0] == kk
            assert list(idx[0, :kk]) == want
            assert np.all(idx[0, kk:] == -1)


def test_matches_numpy_lexsort_large():
    rng = np.random.default_rng(1)
    s = np.round(rng.standard_normal((3, 5000)) * 4) / 4  # quantised -> ties
    s[1, ::7] = -np.inf
    for k in (1, 100, 777, 4999, 6000):
        idx, cnt = oracle.topk(s, k)
        for q in range(3):
            valid = np.flatnonzero(np.isfinite(s[q]))
            order = valid[np.lexsort((valid, -s[q, valid]))]
            want = np.sort(order[:k])
            assert cnt[q] == len(want)
            assert np.array_equal(idx[q, : len(want)], want)
            assert np.all(idx[q, len(want):] == -1)


def test_candidate_mapping_and_tie_rule():
    # slots hold entries 40, 10, 30, 20 (a pool); equal scores -> lower entry wins
    s = np.array([[1.0, 1.0, 2.0, 1.0]])
    cand = np.array([[40, 10, 30, 20]], dtype=np.int32)
    idx, cnt = oracle.topk(s, 2, cand=cand)
    assert list(idx[0]) == [10, 30] and cnt[0] == 2
    cand2 = np.array([[40, -1, 30, 20]], dtype=np.int32)
    idx, cnt = oracle.topk(s, 3, cand=cand2)
    assert list(idx[0]) == [20, 30, 40] and cnt[0] == 3


def test_negative_zero_ties_positive_zero():
    s = np.array([[0.0, -0.0, 0.0, -1.0]])
    idx, _ = oracle.topk(s, 2)
    assert list(idx[0]) == [0, 1]
