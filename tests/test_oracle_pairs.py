"""Pins of the oracle's multi-query forms: "pairs" (each doc with its own query) and
shared docs (every query against every doc).

The Flash-MaxSim rerank page (docs.vllm.ai, vllm.v1.pool.flash_maxsim.
flash_maxsim_rerank, kernel section `_maxsim_rerank_kernel`) names a pairs kernel without
showing it. The reading pinned here: doc i's score is the single-query MaxSim score for
query doc_query[i], whose rows are [q_offsets[j], q_offsets[j] + q_lengths[j]) of the
stacked query rows; a doc whose query is invalid scores NaN. Each test checks the
oracle against exact rational brute force of that definition, doc by doc, computed
without the oracle.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from brute import brute_scores


def _exact_per_doc(w, max_lq):
    """Brute force of each doc against its own query's rows, NaN for invalid queries."""
    out = []
    nq, q_rows = w.q_offsets.shape[0], w.Q.shape[0]
    for i in range(w.B):
        j = int(w.doc_query[i])
        if not 0 <= j < nq:
            out.append(float("nan"))
            continue
        lo, n = int(w.q_offsets[j]), int(w.q_lengths[j])
        if lo < 0 or n < 0 or n > max_lq or lo + n > q_rows:
            out.append(float("nan"))
            continue
        e = brute_scores(w.dtype, w.Q[lo:lo + n], w.X, w.offsets[i:i + 1], w.lengths[i:i + 1], w.d)[0]
        out.append(e)
    return out


def _check(got, exact):
    assert len(got) == len(exact)
    for g, e in zip(got, exact):
        if isinstance(e, float) and np.isnan(e):
            assert np.isnan(g)
        elif e == float("-inf"):
            assert g == float("-inf")
        else:
            assert abs(g - float(e)) <= 1e-12 * (1 + abs(float(e))), (g, e)


def _pairs_scores(w, max_lq=None):
    return oracle.maxsim_pairs(w.dtype, w.Q, w.q_offsets, w.q_lengths, w.X, w.offsets, w.lengths,
                               w.doc_query, w.Lq if max_lq is None else max_lq, d=w.d)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("interleave", [False, True])
def test_pairs_brute_force(fmt, interleave):
    rng = np.random.default_rng([11, len(fmt), int(interleave)])
    q_lengths = [3, 0, 5, 1, 2]
    per = [3, 2, 4, 2, 3]
    lengths = rng.integers(0, 9, size=sum(per))
    lengths[0] = 0
    w = workloads.custom_pairs(q_lengths, 8, per, lengths, dtype=fmt, seed=21, interleave=interleave,
                               order="shuffled", gap=(0, 2), stride=16)
    _check(_pairs_scores(w), _exact_per_doc(w, w.Lq))


def test_pairs_queries_are_not_mixed_up():
    """Docs of different queries must use their own query's rows: swapping two queries'
    row blocks without remapping changes exactly the scores of those queries' docs."""
    w = workloads.custom_pairs([4, 4, 4], 16, [5, 5, 5], np.full(15, 6), seed=3, interleave=True)
    base = _pairs_scores(w)
    swapped = w.Q.copy()
    swapped[0:4], swapped[4:8] = w.Q[4:8], w.Q[0:4]
    w2 = workloads.custom_pairs([4, 4, 4], 16, [5, 5, 5], np.full(15, 6), seed=3, interleave=True)
    w2.Q = swapped
    got = _pairs_scores(w2)
    moved = np.isin(w.doc_query, [0, 1])
    assert np.all(got[~moved] == base[~moved])
    assert np.all(got[moved] != base[moved])
    # ...and remapping the doc -> query table undoes the swap.
    w2.doc_query = np.where(w.doc_query == 0, 1, np.where(w.doc_query == 1, 0, w.doc_query)).astype(np.int32)
    assert np.array_equal(_pairs_scores(w2), base)


def test_pairs_invalid_queries_are_nan():
    w = workloads.custom_pairs([3, 2], 8, [2, 2], np.array([4, 0, 5, 1]), seed=4)
    q_rows = w.Q.shape[0]
    w.doc_query = np.array([0, 1, 2, -1], np.int32)  # index nq and -1 are outside [0, nq)
    _check(_pairs_scores(w), _exact_per_doc(w, w.Lq))
    assert np.isnan(_pairs_scores(w)[2:]).all() and not np.isnan(_pairs_scores(w)[:2]).any()
    for q_off, q_len, max_lq in ((-1, 2, 3), (0, -1, 3), (q_rows - 1, 2, 3), (0, 3, 2)):
        w.doc_query = np.array([0, 1, 1, 0], np.int32)
        w.q_offsets = np.array([0, q_off], np.int32)
        w.q_lengths = np.array([min(3, max_lq), q_len], np.int32)
        got = _pairs_scores(w, max_lq)
        _check(got, _exact_per_doc(w, max_lq))
        assert np.isnan(got[1:3]).all()


def test_pairs_empty_query_scores_zero_even_for_empty_docs():
    w = workloads.custom_pairs([0, 2], 8, [3, 1], np.array([0, 3, 1, 0]), seed=6)
    got = _pairs_scores(w)
    assert list(got[:3]) == [0.0, 0.0, 0.0]
    assert got[3] == float("-inf")


def test_pairs_single_query_equals_maxsim():
    """nq = 1 with every doc on query 0 is the single-query score, bit for bit."""
    w = workloads.tiny()
    ref = oracle.maxsim_workload(w)
    w.q_offsets = np.array([0], np.int32)
    w.q_lengths = np.array([w.Lq], np.int32)
    w.doc_query = np.zeros(w.B, np.int32)
    assert np.array_equal(oracle.maxsim_workload(w), ref)


def test_pairs_workload_shape():
    w = workloads.custom_pairs([16, 32, 20], 32, [10, 5, 7], np.full(22, 9), seed=9, interleave=True)
    assert w.multi_query and w.nq == 3 and w.Lq == 32 and w.Q.shape == (68, 32)
    assert list(w.q_offsets) == [0, 16, 48]
    assert sorted(np.bincount(w.doc_query).tolist()) == [5, 7, 10]


# ------------------------------------------------------------------ shared docs


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_multi_brute_force(fmt):
    """Several queries against the same docs: scores[j, i] is query j's score of doc i."""
    rng = np.random.default_rng([13, len(fmt)])
    q_lengths = [2, 0, 4, 1]
    lengths = rng.integers(0, 8, size=6)
    lengths[0] = 0
    w = workloads.custom_multi(q_lengths, 8, lengths, dtype=fmt, seed=17, order="shuffled", gap=(0, 2),
                               stride=16)
    got = oracle.maxsim_multi(fmt, w.Q, w.q_lengths, w.X, w.offsets, w.lengths, d=w.d)
    assert got.shape == (4, 6)
    lo = 0
    for j, n in enumerate(q_lengths):
        exact = brute_scores(fmt, w.Q[lo:lo + n], w.X, w.offsets, w.lengths, w.d)
        _check(got[j], exact)
        lo += n
    assert np.all(got[1] == 0.0)  # the empty query


def test_multi_matches_workload_and_rows_are_queries():
    w = workloads.custom_multi([3, 5], 16, np.full(7, 4), seed=2)
    assert w.shared_docs and not w.multi_query and w.nq == 2 and w.Q.shape == (8, 16)
    got = oracle.maxsim_workload(w)
    assert got.shape == (2, 7)
    swapped = np.concatenate([w.Q[3:8], w.Q[0:3]])  # query 1 first, then query 0
    w.Q, w.q_lengths = swapped, np.array([5, 3], np.int32)
    got2 = oracle.maxsim_workload(w)
    assert np.array_equal(got2[::-1], got)
