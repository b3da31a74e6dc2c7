"""Pins of the oracle's top-k (the ranking rule of the rerank's consumer): score
descending, ties by lower doc index, -0 equal to +0, NaN after everything, (-inf, -1)
past the end. Checked pairwise by brute force, independently of the oracle's sort."""

from __future__ import annotations

import itertools

import numpy as np
import pytest

import oracle


def _before(a, i, b, j):
    """True when entry (a, i) ranks strictly before (b, j), written out case by case."""
    a_nan, b_nan = np.isnan(a), np.isnan(b)
    if a_nan and b_nan:
        return i < j
    if a_nan:
        return False
    if b_nan:
        return True
    if a > b:
        return True
    if a < b:
        return False
    return i < j


def _check(vals, k):
    ts, ti = oracle.topk(vals, k)
    n = len(vals)
    m = min(k, n)
    assert ts.dtype == np.float32 and ti.dtype == np.int32 and len(ts) == len(ti) == k
    assert np.all(ti[m:] == -1) and np.all(ts[m:] == -np.inf)
    chosen = [int(x) for x in ti[:m]]
    assert len(set(chosen)) == m and all(0 <= x < n for x in chosen)
    for x, y in zip(chosen, chosen[1:]):          # listed in rank order
        assert _before(vals[x], x, vals[y], y)
    rest = set(range(n)) - set(chosen)
    for x, y in itertools.product(chosen, rest):  # every chosen entry beats every other
        assert _before(vals[x], x, vals[y], y)
    assert np.array_equal(ts[:m].view(np.uint32), vals[chosen].view(np.uint32))


@pytest.mark.parametrize("seed", range(6))
def test_topk_pairwise(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 60))
    pool = np.array([0.0, -0.0, 1.0, -1.0, 2.5, np.inf, -np.inf, np.nan, 1e-30, -3.0], np.float32)
    vals = np.where(rng.random(n) < 0.5, rng.choice(pool, n), rng.standard_normal(n).astype(np.float32))
    vals = vals.astype(np.float32)
    for k in (0, 1, 3, n // 2, n, n + 5):
        _check(vals, k)


def test_topk_ties_and_signed_zero():
    vals = np.array([0.0, -0.0, 0.0, 5.0, 5.0, np.nan, -np.inf], np.float32)
    ts, ti = oracle.topk(vals, 7)
    assert list(ti) == [3, 4, 0, 1, 2, 6, 5]
    assert np.signbit(ts[3]) and not np.signbit(ts[2])
