"""Input builders shared by the oracle pins and the GPU parity tests.

They only lay out and transform inputs (which rows a doc owns, where it sits in the
packed tensor, what its entries are); none of them computes a score.
"""

from __future__ import annotations

import numpy as np

import workloads
from workloads import Workload


def bits_of(values, fmt: str) -> np.ndarray:
    """Raw bits of float values that are exact in the format (e.g. small integers)."""
    v = np.asarray(values, dtype=np.float32)
    return workloads.round_f16(v) if fmt == "f16" else workloads.round_bf16(v)


def random_finite_bits(rng: np.random.Generator, shape, fmt: str) -> np.ndarray:
    """Random finite patterns with |x| < 4, subnormals and both zeros included."""
    n = int(np.prod(shape))
    sign = rng.integers(0, 2, size=n, dtype=np.uint16)
    if fmt == "f16":
        expo = rng.integers(0, 17, size=n, dtype=np.uint16)  # 2^(16-15) * 1.x < 4
        frac = rng.integers(0, 1024, size=n, dtype=np.uint16)
        bits = (sign << 15) | (expo << 10) | frac
    else:
        expo = rng.integers(100, 129, size=n, dtype=np.uint16)
        expo[rng.random(n) < 0.1] = 0  # subnormals / zeros
        frac = rng.integers(0, 128, size=n, dtype=np.uint16)
        bits = (sign << 15) | (expo << 7) | frac
    return bits.astype(np.uint16).reshape(shape)


def with_random_values(w: Workload, seed: int) -> Workload:
    """Replace Q and every doc row's first d entries by random finite patterns."""
    rng = np.random.default_rng([seed, 99])
    w.Q = random_finite_bits(rng, w.Q.shape, w.dtype)
    w.X[:, : w.d] = random_finite_bits(rng, (w.T, w.d), w.dtype)
    return w


def small_int_case(rng, Lq, d, lengths, fmt, lo=-2, hi=2, stride=None, gap=None,
                   order="shuffled"):
    """Workload whose Q and doc entries are integers in [lo, hi] (exact in fp16/bf16),
    plus the integer matrices themselves."""
    w = workloads.custom(Lq, d, lengths, dtype=fmt, seed=int(rng.integers(1 << 30)),
                         stride=stride, order=order, gap=gap, gap_fill="nan")
    Qi = rng.integers(lo, hi + 1, size=(Lq, d))
    Xi = rng.integers(lo, hi + 1, size=(w.T, d))
    w.Q = bits_of(Qi, fmt).reshape(Lq, d)
    w.X[:, :d] = bits_of(Xi, fmt).reshape(w.T, d)
    return w, Qi, Xi


def one_hot_case(rng, Lq, d, lengths, fmt, stride=None, gap=None):
    """Q[q] = e_a(q), doc row t = e_b(t). Returns the workload, a and b."""
    w = workloads.custom(Lq, d, lengths, dtype=fmt, seed=int(rng.integers(1 << 30)),
                         stride=stride, order="shuffled", gap=gap, gap_fill="nan")
    a = rng.integers(0, d, size=Lq)
    b = rng.integers(0, d, size=w.T)
    Qf = np.zeros((Lq, d), np.float32)
    Qf[np.arange(Lq), a] = 1.0
    Xf = np.zeros((w.T, d), np.float32)
    Xf[np.arange(w.T), b] = 1.0
    w.Q = bits_of(Qf, fmt)
    w.X[:, :d] = bits_of(Xf, fmt)
    return w, a, b


def one_hot_expected(Lq, a, b, offsets, lengths):
    """#{q : a(q) is among the hot columns of the doc's rows}; -inf for an empty doc."""
    out = []
    for off, n in zip(offsets, lengths):
        if Lq and n == 0:
            out.append(float("-inf"))
            continue
        hot = set(int(x) for x in b[off : off + n])
        out.append(float(sum(1 for q in range(Lq) if int(a[q]) in hot)))
    return np.array(out, np.float64)


def doc_rows(w: Workload, i: int) -> np.ndarray:
    o, n = int(w.offsets[i]), int(w.lengths[i])
    return w.X[o : o + n]


def repack(w: Workload, row_lists, stride=None, pad_bits=0) -> Workload:
    """New workload with doc i's rows = row_lists[i] (arrays [n_i, >=d] of bits),
    packed back to back in doc order with the given stride."""
    stride = w.d if stride is None else stride
    lens = np.array([len(r) for r in row_lists], np.int64)
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]]) if len(lens) else lens
    T = int(lens.sum())
    X = np.full((max(T, 1), stride), pad_bits, np.uint16)
    for o, r in zip(offs, row_lists):
        X[o : o + len(r), : w.d] = r[:, : w.d]
    return Workload(name=w.name + "_repacked", dtype=w.dtype, Lq=w.Lq, d=w.d,
                    stride=stride, Q=w.Q.copy(), X=X, offsets=offs.astype(np.int32),
                    lengths=lens.astype(np.int32), seed=w.seed)


def load_golden(path: str):
    """Parse a tests/golden/*.txt fixture: returns (fmt, Q bits, X bits, d, offsets,
    lengths, expected scores)."""
    fmt = None
    d = stride = None
    section = None
    Q, X, docs = [], [], []
    with open(path) as fh:
        for raw in fh:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            head = line.split()
            if head[0] == "format":
                fmt = head[1]
            elif head[0] == "d":
                d = int(head[1])
            elif head[0] == "stride":
                stride = int(head[1])
            elif head[0] in ("Q", "X", "docs") and len(head) == 1:
                section = head[0]
            elif section == "Q":
                Q.append([float(v) for v in head])
            elif section == "X":
                X.append([float(v) for v in head])
            elif section == "docs":
                docs.append((int(head[0]), int(head[1]), float(head[2])))
    Qb = bits_of(np.array(Q, np.float32).reshape(len(Q), d), fmt)
    Xb = bits_of(np.array(X, np.float32).reshape(len(X), stride), fmt)
    offs = np.array([x[0] for x in docs], np.int32)
    lens = np.array([x[1] for x in docs], np.int32)
    exp = np.array([x[2] for x in docs], np.float64)
    return fmt, Qb, Xb, d, offs, lens, exp
