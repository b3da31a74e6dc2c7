"""Pins of the oracle's FP8 E4M3 doc path (docs stored as E4M3 bytes with one fp32 scale
for the doc tensor; the sparse prefill pages page, docs.vllm.ai, `stage_prefill_pages`,
dequantises FP8 E4M3 caches with per-tensor scales). Each pin compares with something
other than the oracle: torch's float8_e4m3fn conversion, exact rational brute force, the
pinned fp16 path on values that are exact in fp16, and one-hot closed forms."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from pin_suite import (_e4m3_vals, _fp8_case, pin_e4m3_decoder, pin_fp8_brute_force,
                       pin_fp8_equals_f16_path)


def _orc():
    oracle.build(force=False)
    return oracle.Oracle(oracle.LIBRARY)


def test_e4m3_decoder_all_patterns():
    pin_e4m3_decoder(_orc())


def test_fp8_brute_force():
    pin_fp8_brute_force(_orc())


def test_fp8_equals_f16_path_on_exact_values():
    pin_fp8_equals_f16_path(_orc())


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_fp8_one_hot(fmt):
    """Q[q] = e_a(q): the score is sum_q max_t scale * x[t][a(q)]."""
    rng = np.random.default_rng(3)
    Lq, d = 6, 32
    w = _fp8_case(fmt, Lq, d, [5, 1, 0, 9, 4], seed=8, scale=0.25, all_patterns=True)
    a = rng.integers(0, d, size=Lq)
    one = 0x3C00 if fmt == "f16" else 0x3F80
    w.Q = np.zeros((Lq, d), np.uint16)
    w.Q[np.arange(Lq), a] = one
    vals = _e4m3_vals(w.X8[:, :d]) * w.doc_scale
    ref = []
    for o_, n in zip(w.offsets, w.lengths):
        ref.append(float("-inf") if n == 0 else sum(vals[o_:o_ + n, a[q]].max() for q in range(Lq)))
    got = oracle.maxsim_fp8(fmt, w.Q, w.X8, w.offsets, w.lengths, w.doc_scale, d=d)
    assert np.array_equal(got, np.array(ref))


def test_fp8_workload_quantisation():
    """to_fp8 keeps the layout (offsets, lengths, NaN outside docs) and rounds each value
    to the nearest E4M3 step of value / scale."""
    w = workloads.custom(4, 32, [3, 5, 2], seed=2, gap=(1, 2), gap_fill="nan", stride=40)
    x = workloads._bits_to_f32(w.X[:, :32], "f16")
    workloads.to_fp8(w, doc_scale=1 / 256)
    assert w.X8.shape == (w.T, 32)
    v = _e4m3_vals(w.X8)
    in_doc = np.zeros(w.T, bool)
    for o_, n in zip(w.offsets, w.lengths):
        in_doc[o_:o_ + n] = True
    assert np.isnan(v[~in_doc]).all() and not np.isnan(v[in_doc]).any()
    err = np.abs(v[in_doc] * w.doc_scale - x[in_doc])
    assert np.all(err <= np.abs(x[in_doc]) * 2.0 ** -4 + 2.0 ** -9 * w.doc_scale)
