"""Exact rational brute force of the MaxSim score, for tiny inputs only.

Independent of the oracle: values come from numpy's own float16 / float32 bit
conversions (not the oracle's decoders) and every product and sum is an exact
``fractions.Fraction``. Pure-Python loops, so keep inputs to a few thousand
multiply-adds.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

NEG_INF = float("-inf")


def exact_values(bits: np.ndarray, fmt: str) -> np.ndarray:
    """float64 value of each raw 16-bit pattern, via numpy's conversions."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if fmt == "f16":
        return bits.view(np.float16).astype(np.float64)
    if fmt == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(fmt)


def brute_scores(fmt, Q, X, offsets, lengths, d):
    """Exact scores: a Fraction per doc, or -inf for a doc with no rows (Lq > 0)."""
    Qv = exact_values(Q, fmt)
    Xv = exact_values(X, fmt)
    Lq = Qv.shape[0]
    qf = [[Fraction(float(Qv[q, k])) for k in range(d)] for q in range(Lq)]
    out = []
    for off, n in zip(np.asarray(offsets, np.int64), np.asarray(lengths, np.int64)):
        rows = [[Fraction(float(Xv[off + t, k])) for k in range(d)] for t in range(n)]
        total = Fraction(0)
        empty = False
        for q in range(Lq):
            if n == 0:
                empty = True
                break
            best = max(sum(a * b for a, b in zip(qf[q], r)) for r in rows)
            total += best
        out.append(NEG_INF if empty else total)
    return out


def int_brute_scores(Qi, Xi, offsets, lengths, d):
    """Exact integer scores for integer-valued inputs (Python ints), -inf if empty."""
    out = []
    Lq = len(Qi)
    for off, n in zip(offsets, lengths):
        if Lq and n == 0:
            out.append(NEG_INF)
            continue
        total = 0
        for q in range(Lq):
            total += max(
                sum(int(Qi[q][k]) * int(Xi[off + t][k]) for k in range(d)) for t in range(n)
            )
        out.append(total)
    return out
