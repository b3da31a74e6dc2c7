"""Property-based pins (hypothesis, derandomised so that every run draws the same cases).

1. The oracle against exact rational brute force on arbitrary finite fp16 / bf16 bit
   patterns: subnormals, signed zeros, values up to the formats' largest, strided rows,
   overlapping and empty docs. fp64 rounds each dot product and the sum over query rows,
   so the two agree within (d + Lq) 2^-52 times the sum of the terms' magnitudes
   (cancellation can make the score itself much smaller than its terms).
2. The range kernel's cut and its prologue's search for each range's first doc (the
   model in test_range_model.py) on random length laws and wave counts.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

import oracle  # noqa: E402
from brute import brute_scores, exact_values  # noqa: E402
from test_range_model import active, prologue_first_docs, range_start, walk  # noqa: E402

SETTINGS = dict(derandomize=True, deadline=None, suppress_health_check=[HealthCheck.too_slow])


def finite_bits(fmt):
    """Raw 16-bit patterns of finite values: every exponent but the all-ones one."""
    if fmt == "f16":
        return st.integers(0, 0xFFFF).filter(lambda b: (b >> 10) & 0x1F != 0x1F)
    return st.integers(0, 0xFFFF).filter(lambda b: (b >> 7) & 0xFF != 0xFF)


@st.composite
def cases(draw):
    fmt = draw(st.sampled_from(["f16", "bf16"]))
    Lq = draw(st.integers(0, 4))
    d = draw(st.integers(1, 9))
    stride = d + draw(st.integers(0, 3))
    T = draw(st.integers(1, 14))
    bits = finite_bits(fmt)
    Q = np.array(draw(st.lists(bits, min_size=Lq * d, max_size=Lq * d)), np.uint16).reshape(Lq, d)
    X = np.array(draw(st.lists(bits, min_size=T * stride, max_size=T * stride)), np.uint16).reshape(T, stride)
    B = draw(st.integers(1, 5))
    offsets, lengths = [], []
    for _ in range(B):
        off = draw(st.integers(0, T - 1))
        offsets.append(off)
        lengths.append(draw(st.integers(0, T - off)))
    return fmt, Q, X, np.array(offsets, np.int32), np.array(lengths, np.int32), d


@settings(max_examples=400, **SETTINGS)
@given(cases())
def test_oracle_equals_exact_brute_force(case):
    fmt, Q, X, offsets, lengths, d = case
    got = oracle.maxsim(fmt, Q, X, offsets, lengths, d=d)
    exact = brute_scores(fmt, Q, X, offsets, lengths, d)
    Qv, Xv = exact_values(Q, fmt), exact_values(X, fmt)
    Lq = Q.shape[0]
    for i, (g, e) in enumerate(zip(got, exact)):
        if Lq == 0:
            assert g == 0.0
            continue
        if e == float("-inf"):
            assert g == float("-inf")
            continue
        off, n = int(offsets[i]), int(lengths[i])
        mag = sum(max(sum(abs(Fraction(float(Qv[q, k])) * Fraction(float(Xv[off + t, k]))) for k in range(d))
                      for t in range(n)) for q in range(Lq))
        bound = (d + Lq) * 2.0 ** -52 * float(mag)
        assert abs(Fraction(g) - e) <= Fraction(bound), (fmt, i, g, float(e), bound)


@st.composite
def length_laws(draw):
    B = draw(st.integers(1, 8192))
    kind = draw(st.sampled_from(["short", "mixed", "sparse", "long"]))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    r = np.random.default_rng(seed)
    if kind == "short":
        L = r.integers(0, 40, size=B)
    elif kind == "mixed":
        L = r.integers(0, 600, size=B)
    elif kind == "sparse":
        L = np.where(r.random(B) < 0.9, 0, r.integers(1, 9000, size=B))
    else:
        L = np.clip(np.rint(np.exp(r.normal(np.log(1024), 0.6, size=B))), 32, 4096).astype(np.int64)
    W = draw(st.sampled_from([256, 1024, 2048, 3072, 4096]))
    return L.astype(np.int64), W


@settings(max_examples=40, **SETTINGS)
@given(length_laws())
def test_range_cut_and_first_doc_search(law):
    lengths, W = law
    nt = np.array([(int(n) + 15) // 16 if n > 0 else 0 for n in lengths], np.int64)
    S = np.concatenate([[0], np.cumsum(nt)])
    T = int(S[-1])
    found, reads, nch = prologue_first_docs(lengths, W)
    assert max(reads) < 4 * 256 * nch
    if T == 0:
        assert not found
        return
    wact = active(T, W)
    for w, (doc, first_tile) in found.items():
        rb = range_start(w, T, wact)
        want = int(np.searchsorted(S, rb, side="right") - 1)
        assert (doc, first_tile) == (want, int(S[want])) and nt[doc] > 0
    # every tile issued exactly once over the waves' walks
    if len(lengths) <= 2048:
        _, _, T2, _, _, issued = walk(lengths, W)
        assert T2 == T and sorted(issued) == list(range(T))
