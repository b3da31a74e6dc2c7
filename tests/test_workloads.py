"""The seeded generators: reproducible, the stated shapes and laws, valid layouts."""

import numpy as np
import pytest
import torch

import workloads


def _no_overlap(w):
    order = np.argsort(w.offsets, kind="stable")
    ends = w.offsets[order].astype(np.int64) + w.lengths[order]
    return bool(np.all(ends[:-1] <= w.offsets[order][1:]))


def test_rounding_matches_library_casts():
    x = np.random.default_rng(0).standard_normal(100_000).astype(np.float32) * 3
    assert np.array_equal(workloads.round_f16(x), x.astype(np.float16).view(np.uint16))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(workloads.round_bf16(x), ref)


def test_reproducible_and_thread_independent():
    a = workloads.custom(5, 32, [300_000], seed=3, threads=1)
    b = workloads.custom(5, 32, [300_000], seed=3, threads=4)
    assert np.array_equal(a.X, b.X) and np.array_equal(a.Q, b.Q)
    c = workloads.custom(5, 32, [300_000], seed=4, threads=4)
    assert not np.array_equal(a.X, c.X)


def test_rows_are_unit_norm():
    w = workloads.tiny()
    x = w.X.view(np.float16).astype(np.float64)
    n = np.linalg.norm(x, axis=1)
    assert np.all(np.abs(n - 1) < 2e-3)


@pytest.mark.parametrize("name,Lq,d,B,lo,hi,dtype", [
    ("tiny", 32, 128, 64, 16, 128, "f16"),
    ("colbert", 32, 128, 1000, 64, 300, "f16"),
    ("long_doc", 128, 128, 256, 32, 4096, "bf16"),
    ("scattered", 37, 96, 8192, 1, 512, "f16"),
])
def test_named_workloads(name, Lq, d, B, lo, hi, dtype):
    w = workloads.make(name)
    assert (w.Lq, w.d, w.B, w.dtype, w.stride) == (Lq, d, B, dtype, d)
    assert w.Q.shape == (Lq, d) and w.X.shape == (w.T, d)
    assert w.lengths.min() >= lo and w.lengths.max() <= hi
    assert _no_overlap(w)
    assert int((w.offsets.astype(np.int64) + w.lengths).max()) <= w.T


def test_scattered_layout():
    w = workloads.scattered()
    assert w.lengths.min() == 1  # length-1 docs present
    order = np.argsort(w.offsets)
    assert not np.array_equal(order, np.arange(w.B))  # shuffled memory order
    gaps = w.offsets[order][1:] - (w.offsets[order][:-1] + w.lengths[order][:-1])
    assert gaps.min() >= 1 and gaps.max() <= 48
    last = order[-1]
    assert w.offsets[last] + w.lengths[last] == w.T  # last doc ends on the last row
    assert 1 <= w.offsets[order[0]] <= 48


def test_long_doc_lengths_law():
    w = workloads.long_doc()
    med = np.median(w.lengths)
    assert 850 < med < 1200
    assert w.lengths.max() <= 4096 and w.lengths.min() >= 32


def test_nan_gap_fill_only_touches_gaps():
    a = workloads.custom(4, 16, [3, 5, 2], seed=1, order="shuffled", gap=(1, 3), stride=24)
    b = workloads.custom(4, 16, [3, 5, 2], seed=1, order="shuffled", gap=(1, 3), stride=24,
                         gap_fill="nan")
    for o, n in zip(a.offsets, a.lengths):
        assert np.array_equal(a.X[o:o + n, :16], b.X[o:o + n, :16])
    assert np.all(b.X[:, 16:] == workloads.F16_NAN)
