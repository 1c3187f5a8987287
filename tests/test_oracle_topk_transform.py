"""Pins for the top-k and page-transform oracles: numpy's sort and partition
as independent selections, the identity case, and the two forms of the
page-table transform."""

import numpy as np
import pytest

from oracle import topk as K
from oracle import transform as X


@pytest.mark.parametrize("n,k", [(1000, 64), (5000, 2048), (300, 256), (256, 256), (17, 256), (0, 8)])
def test_topk_against_sort_and_partition(n, k):
    rng = np.random.default_rng(n + k)
    row = rng.normal(size=n + 50)           # entries past n must be ignored
    row[n:] = 1e9
    sel = K.topk_row(row, n, k)
    m = min(n, k)
    assert (sel[m:] == -1).all()
    valid = sel[:m]
    assert len(set(valid.tolist())) == m
    assert ((valid >= 0) & (valid < n)).all()
    if n > k:
        kth = np.sort(row[:n])[::-1][k - 1]
        assert row[valid].min() >= kth
        part = np.argpartition(-row[:n], k - 1)[:k]
        assert set(part.tolist()) == set(valid.tolist())   # distinct scores
    else:
        np.testing.assert_array_equal(np.sort(valid), np.arange(n))


def _kth_by_counting(row, n, k):
    """The k-th largest of row[:n] from its definition alone: the value v of
    the row such that fewer than k entries exceed v and at least k reach it
    (O(n^2) comparisons, no sort)."""
    x = np.asarray(row[:n], np.float64)
    for v in x:
        if (x > v).sum() < k <= (x >= v).sum():
            return v
    raise AssertionError("no k-th largest")


@pytest.mark.parametrize("n,k", [(40, 1), (40, 7), (40, 39), (200, 64), (17, 16)])
def test_kth_largest_against_definition_and_partition(n, k):
    # kth_largest is the acceptance threshold of every top-k check; it is
    # pinned by the counting definition, numpy's partition (a selection
    # algorithm, not a sort) and the minimum of argpartition's k-set
    rng = np.random.default_rng(100 * n + k)
    row = np.concatenate([rng.normal(size=n), [1e30, -1e30]])   # tail ignored
    got = K.kth_largest(row, n, k)
    assert got == _kth_by_counting(row, n, k)
    assert got == -np.partition(-row[:n], k - 1)[k - 1]
    assert got == row[:n][np.argpartition(-row[:n], k - 1)[:k]].min()


def test_kth_largest_hand_rows():
    assert K.kth_largest([3.0, 1.0, 2.0], 3, 2) == 2.0
    assert K.kth_largest([3.0, 1.0, 2.0], 3, 1) == 3.0
    assert K.kth_largest([5.0, 5.0, 5.0, 1.0], 4, 2) == 5.0       # ties count
    assert K.kth_largest([5.0, 5.0, 5.0, 1.0], 4, 3) == 5.0
    assert K.kth_largest([-np.inf, 0.0, -1.0, 2.0], 4, 3) == -1.0
    assert K.kth_largest([0.5, 9.0, 7.0, 8.0], 3, 2) == 7.0       # position 3 ignored
    assert K.kth_largest([1.0, 2.0], 2, 2) == -np.inf              # keeps every position
    assert K.kth_largest([1.0, 2.0], 2, 5) == -np.inf
    # with ties, exactly the positions scoring >= the k-th value number >= k
    row = np.array([4.0, 4.0, 3.0, 4.0, 1.0, 3.0])
    v = K.kth_largest(row, 6, 4)
    assert v == 3.0 and (row > v).sum() < 4 <= (row >= v).sum()


def test_topk_ties_resolved_by_position():
    row = np.array([1.0, 5.0, 3.0, 3.0, 3.0, 0.0])
    np.testing.assert_array_equal(K.topk_row(row, 6, 3), [1, 2, 3])
    np.testing.assert_array_equal(K.topk_row(row, 6, 2), [1, 2])


def test_topk_rows_and_lengths():
    rng = np.random.default_rng(2)
    logits = rng.normal(size=(3, 400))
    out = K.topk(logits, [400, 10, 0], 16)
    assert out.shape == (3, 16)
    np.testing.assert_array_equal(np.sort(out[1, :10]), np.arange(10))
    assert (out[1, 10:] == -1).all() and (out[2] == -1).all()


def _aligned_tables(lens, page=64, seed=0):
    rng = np.random.default_rng(seed)
    npg = [(n + page - 1) // page for n in lens]
    perm = rng.permutation(sum(npg) + 3)
    width = max(npg) * page
    wide = np.zeros((len(lens), width), np.int64)
    compact = np.zeros((len(lens), max(npg)), np.int64)
    p0 = 0
    for r, n in enumerate(npg):
        pg = perm[p0:p0 + n]
        p0 += n
        wide[r, :n * page] = (pg[:, None] * page + np.arange(page)).reshape(-1)
        compact[r, :n] = pg
    return wide, compact


def test_wide_and_compact_transforms_agree():
    lens = [700, 300, 64]
    wide, compact = _aligned_tables(lens)
    rng = np.random.default_rng(9)
    t2r = np.array([0, 0, 1, 2, 1])
    idx = np.full((5, 40), -1, np.int64)
    for t, r in enumerate(t2r):
        m = min(lens[r], 30 + t)
        idx[t, :m] = rng.choice(lens[r], size=m, replace=False)
    a = X.transform_wide(idx, wide, t2r)
    b = X.transform_compact(idx, compact, t2r)
    np.testing.assert_array_equal(a, b)
    assert ((a == -1) == (idx == -1)).all()
    # a hand-checked entry: position 130 of request 0 is page 2, offset 2
    i = np.array([[130, -1]])
    assert X.transform_compact(i, compact, [0])[0, 0] == compact[0, 2] * 64 + 2
    assert X.transform_wide(i, wide, [0])[0, 1] == -1
