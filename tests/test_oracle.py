"""Pins of the fp64 oracle against facts fixed by the page and by mathematics.

The score being pinned is the one the Flash-MaxSim rerank page (docs.vllm.ai,
vllm.v1.pool.flash_maxsim.flash_maxsim_rerank) defines: for each doc, the sum over
query rows of the best dot product with any of the doc's rows. Each test below checks
the oracle against something other than itself: library conversions, exact rational
brute force, closed forms and invariants.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from brute import brute_scores, int_brute_scores
from cases import (
    bits_of,
    doc_rows,
    one_hot_case,
    one_hot_expected,
    repack,
    small_int_case,
    with_random_values,
)

ORC = None


def orc():
    global ORC
    if ORC is None:
        oracle.build(force=False)
        ORC = oracle.Oracle(oracle.LIBRARY)
    return ORC


def scores(w, o=None):
    o = o or orc()
    return o.maxsim(w.dtype, w.Q, w.X, w.offsets, w.lengths, d=w.d)


def close(a, b, rel=1e-12):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    ok = same_inf | (np.abs(a - b) <= rel * (1.0 + np.abs(b)))
    return bool(np.all(ok))


# ----------------------------------------------------------------- decoders


def test_decode_f16_all_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc().decode(bits, "f16")
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_decode_bf16_all_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc().decode(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


# ----------------------------------------------------------------- exact brute force


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("Lq", [0, 1, 2, 3, 5])
@pytest.mark.parametrize("d", [1, 3, 8, 16])
def test_brute_force_exact(fmt, Lq, d):
    rng = np.random.default_rng([Lq, d, len(fmt)])
    lengths = rng.integers(0, 21, size=7)
    lengths[0] = 0  # always one empty doc
    stride = d + int(rng.integers(0, 6))
    for values in ("unit", "wide"):
        w = workloads.custom(Lq, d, lengths, dtype=fmt, seed=int(rng.integers(1 << 30)),
                             stride=stride, order="shuffled", gap=(0, 3), gap_fill="nan")
        if values == "wide":
            w = with_random_values(w, seed=Lq * 100 + d)
            w.X[:, d:] = workloads.F16_NAN if fmt == "f16" else workloads.BF16_NAN
        exact = brute_scores(fmt, w.Q, w.X, w.offsets, w.lengths, d)
        got = scores(w)
        for g, e in zip(got, exact):
            if e == float("-inf"):
                assert g == float("-inf")
            else:
                assert abs(g - float(e)) <= 1e-12 * (1 + abs(float(e))), (g, e)


# ----------------------------------------------------------------- closed forms


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_single_query_row_is_max_dot(fmt):
    """Lq = 1: the score is the largest dot product of q with the doc's rows."""
    w = workloads.custom(1, 64, np.arange(1, 41), dtype=fmt, seed=5, order="shuffled",
                         gap=(1, 4), stride=72)
    q = _vals(w.Q, fmt)[0]
    X = _vals(w.X[:, : w.d], fmt)
    ref = np.array([(X[o : o + n] @ q).max() for o, n in zip(w.offsets, w.lengths)])
    assert close(scores(w), ref)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_single_token_doc_is_sum_of_dots(fmt):
    """A one-row doc t: the max is over one row, so the score is sum_q q.t = (sum_q q).t."""
    w = workloads.custom(29, 96, np.ones(50, np.int64), dtype=fmt, seed=6, order="shuffled",
                         gap=(0, 2))
    Qs = _vals(w.Q, fmt).sum(axis=0)
    X = _vals(w.X[:, : w.d], fmt)
    ref = X[w.offsets.astype(np.int64)] @ Qs
    assert close(scores(w), ref, rel=1e-12)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_integer_inputs_exact(fmt):
    """Integer entries in [-2, 2]: every sum is a small integer, exact in fp64."""
    rng = np.random.default_rng(7)
    w, Qi, Xi = small_int_case(rng, 6, 24, rng.integers(0, 12, size=20), fmt, gap=(0, 3),
                               stride=32)
    ref = int_brute_scores(Qi, Xi, w.offsets, w.lengths, 24)
    got = scores(w)
    assert [float(x) for x in ref] == list(got)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_one_hot_counts_matching_columns(fmt):
    """Q[q] = e_a(q), doc rows e_b(t): score = #{q : a(q) is a hot column of the doc}."""
    rng = np.random.default_rng(8)
    Lq, d = 13, 32
    lengths = rng.integers(0, 9, size=40)
    w, a, b = one_hot_case(rng, Lq, d, lengths, fmt, gap=(0, 2))
    assert np.array_equal(scores(w), one_hot_expected(Lq, a, b, w.offsets, w.lengths))


def test_special_cases():
    """Lq = 0 -> 0 (empty sum); a doc with no rows -> -inf (max over nothing); B = 0."""
    w = workloads.custom(4, 16, [0, 3, 0, 1], seed=9)
    s = scores(w)
    assert s[0] == -np.inf and s[2] == -np.inf and np.isfinite(s[1]) and np.isfinite(s[3])
    w0 = workloads.custom(0, 16, [0, 3, 5], seed=9)
    assert np.array_equal(scores(w0), np.zeros(3))
    out = orc().maxsim("f16", w.Q, w.X, np.zeros(0, np.int32), np.zeros(0, np.int32))
    assert out.shape == (0,)


# ----------------------------------------------------------------- invariants


def _vals(bits, fmt):
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if fmt == "f16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_token_permutation_and_duplication_invariant(fmt):
    w = workloads.custom(11, 48, np.random.default_rng(10).integers(1, 30, size=25),
                         dtype=fmt, seed=10, order="shuffled", gap=(1, 5))
    base = scores(w)
    rng = np.random.default_rng(11)
    perm_rows = [doc_rows(w, i)[rng.permutation(w.lengths[i])] for i in range(w.B)]
    assert np.array_equal(scores(repack(w, perm_rows)), base)
    dup_rows = []
    for i in range(w.B):
        r = doc_rows(w, i)
        extra = r[rng.integers(0, len(r), size=int(rng.integers(1, 5)))]
        dup_rows.append(np.concatenate([r, extra])[rng.permutation(len(r) + len(extra))])
    assert np.array_equal(scores(repack(w, dup_rows)), base)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_scattered_equals_contiguous_and_doc_order(fmt):
    w = workloads.custom(9, 40, np.random.default_rng(12).integers(0, 25, size=30),
                         dtype=fmt, seed=12, order="shuffled", gap=(1, 9), stride=56,
                         gap_fill="nan", pad_fill="nan")
    base = scores(w)
    packed = repack(w, [doc_rows(w, i) for i in range(w.B)])
    assert np.array_equal(scores(packed), base)
    perm = np.random.default_rng(13).permutation(w.B)
    got = orc().maxsim(fmt, w.Q, w.X, w.offsets[perm], w.lengths[perm], d=w.d)
    assert np.array_equal(got, base[perm])


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_rows_outside_docs_never_matter(fmt):
    """NaN in gap rows and in stride padding changes nothing."""
    kw = dict(dtype=fmt, seed=14, order="shuffled", gap=(1, 6), stride=40)
    lens = np.random.default_rng(14).integers(0, 20, size=30)
    a = workloads.custom(7, 32, lens, gap_fill="nan", pad_fill="nan", **kw)
    b = workloads.custom(7, 32, lens, gap_fill="random", pad_fill="zero", **kw)
    assert np.array_equal(scores(a), scores(b))


def test_scaling_query_doubles_score():
    """Q -> 2Q is exact in fp16 for unit rows; every dot, max and sum doubles exactly."""
    w = workloads.custom(17, 64, np.random.default_rng(15).integers(1, 40, size=30), seed=15)
    base = scores(w)
    w.Q = workloads.round_f16(2.0 * w.Q.view(np.float16).astype(np.float32))
    assert np.array_equal(scores(w), 2.0 * base)


def test_appending_a_token_never_lowers_the_score():
    w = workloads.custom(8, 32, np.random.default_rng(16).integers(1, 20, size=40), seed=16)
    base = scores(w)
    rng = np.random.default_rng(17)
    extra = workloads.custom(1, 32, [w.B], seed=18).X
    grown = repack(w, [np.concatenate([doc_rows(w, i), extra[i : i + 1]]) for i in range(w.B)])
    assert np.all(scores(grown) >= base)
    del rng


def test_query_row_permutation_within_rounding():
    w = workloads.custom(31, 128, np.random.default_rng(19).integers(1, 60, size=30), seed=19)
    base = scores(w)
    w.Q = w.Q[np.random.default_rng(20).permutation(w.Lq)]
    assert close(scores(w), base, rel=1e-13)


def test_cauchy_schwarz_bound():
    """|score| <= sum_q |q| * max_t |t| for every doc."""
    w = workloads.custom(16, 64, np.random.default_rng(21).integers(1, 50, size=40), seed=21)
    Q = _vals(w.Q, "f16")
    X = _vals(w.X[:, : w.d], "f16")
    qn = np.linalg.norm(Q, axis=1).sum()
    s = scores(w)
    for i in range(w.B):
        o, n = int(w.offsets[i]), int(w.lengths[i])
        tn = np.linalg.norm(X[o : o + n], axis=1).max()
        assert abs(s[i]) <= qn * tn * (1 + 1e-12)


def test_planted_near_duplicate_raises_score():
    """A doc holding unit(Q[q] + 0.02 z) gets a term >= ~0.97 for that query row, far
    above what unrelated unit rows in 128 dimensions reach."""
    w = workloads.custom(32, 128, np.random.default_rng(22).integers(64, 200, size=200),
                         seed=22)
    workloads._plant(w, 0.05, 0.02)
    s = scores(w)
    planted = np.zeros(w.B, bool)
    planted[w.planted] = True
    assert s[planted].min() > s[~planted].max() - 0.5
    assert np.median(s[planted]) > np.median(s[~planted]) + 0.5
