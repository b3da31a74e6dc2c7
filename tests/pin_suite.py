"""A compact set of oracle pins that can run against any build of the oracle library.

Used in two ways: tests/test_oracle_mutants.py runs it in a subprocess against copies
of the oracle with planted mistakes (each must fail at least one pin), and against the
unmodified oracle (which must pass all of them).

    python tests/pin_suite.py path/to/liboracle.so   -> exit 0 iff every pin holds
"""

from __future__ import annotations

import glob
import os
import sys
import tempfile

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)

import oracle  # noqa: E402
import workloads  # noqa: E402
from brute import brute_scores  # noqa: E402
from cases import load_golden, one_hot_case, one_hot_expected, with_random_values  # noqa: E402


def _vals(bits, fmt):
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        if fmt == "f16":
            return bits.view(np.float16).astype(np.float64)
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _close(a, b, rel=1e-12):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        return bool(np.all(same_inf | (np.abs(a - b) <= rel * (1 + np.abs(b)))))


def pin_decoders(o):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for fmt in ("f16", "bf16"):
        got = o.decode(bits, fmt)
        ref = _vals(bits, fmt)
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan), fmt
        assert np.array_equal(got[~nan], ref[~nan]), fmt
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan])), fmt


def pin_brute_force(o):
    for fmt in ("f16", "bf16"):
        for Lq, d in ((1, 3), (3, 8), (5, 16)):
            rng = np.random.default_rng([Lq, d, 7])
            lengths = rng.integers(0, 12, size=6)
            lengths[0] = 0
            for wide in (False, True):
                w = workloads.custom(Lq, d, lengths, dtype=fmt, seed=Lq * 10 + d,
                                     stride=d + 3, order="shuffled", gap=(0, 3),
                                     gap_fill="nan")
                if wide:
                    w = with_random_values(w, seed=Lq + d)
                exact = brute_scores(fmt, w.Q, w.X, w.offsets, w.lengths, d)
                got = o.maxsim(fmt, w.Q, w.X, w.offsets, w.lengths, d=d)
                assert _close(got, [float(e) for e in exact]), (fmt, Lq, d, wide)


def pin_golden(o):
    paths = sorted(glob.glob(os.path.join(HERE, "golden", "handworked_*.txt")))
    assert paths
    for p in paths:
        fmt, Q, X, d, offs, lens, exp = load_golden(p)
        assert np.array_equal(o.maxsim(fmt, Q, X, offs, lens, d=d), exp), p


def pin_closed_forms(o):
    for fmt in ("f16", "bf16"):
        w = workloads.custom(1, 32, np.arange(1, 20), dtype=fmt, seed=3, order="shuffled",
                             gap=(1, 3))
        q = _vals(w.Q, fmt)[0]
        X = _vals(w.X[:, : w.d], fmt)
        ref = [(X[a : a + n] @ q).max() for a, n in zip(w.offsets, w.lengths)]
        assert _close(o.maxsim(fmt, w.Q, w.X, w.offsets, w.lengths, d=w.d), ref), fmt
        w = workloads.custom(7, 40, np.ones(12, np.int64), dtype=fmt, seed=4, gap=(0, 2))
        ref = _vals(w.X[:, : w.d], fmt)[w.offsets.astype(np.int64)] @ _vals(w.Q, fmt).sum(0)
        assert _close(o.maxsim(fmt, w.Q, w.X, w.offsets, w.lengths, d=w.d), ref), fmt


def pin_one_hot(o):
    rng = np.random.default_rng(5)
    for fmt in ("f16", "bf16"):
        w, a, b = one_hot_case(rng, 9, 16, rng.integers(0, 7, size=20), fmt, gap=(0, 2))
        got = o.maxsim(fmt, w.Q, w.X, w.offsets, w.lengths, d=w.d)
        assert np.array_equal(got, one_hot_expected(9, a, b, w.offsets, w.lengths)), fmt


def pin_int64_addressing(o):
    """Docs whose element offset (row * stride) is past 2**31 and 2**32 score exactly
    as the same rows placed at the front of a small tensor. X is a sparse file mapping,
    so only the doc rows take memory."""
    d = stride = 128
    T = (1 << 33) // stride + 64  # 2**33 elements: 16 GiB apparent, a few KB resident
    small = workloads.custom(6, d, [5, 3, 7], seed=11)
    rows = [small.X[a : a + n] for a, n in zip(small.offsets, small.lengths)]
    starts = [(1 << 31) // stride + 1, (1 << 32) // stride + 3, T - 7]
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "x.bin")
        X = np.memmap(path, dtype=np.uint16, mode="w+", shape=(T, stride))
        for s, r in zip(starts, rows):
            X[s : s + len(r)] = r
        X.flush()
        got = o.maxsim("f16", small.Q, X, np.array(starts, np.int32), small.lengths, d=d)
        del X
    ref = o.maxsim("f16", small.Q, small.X, small.offsets, small.lengths, d=d)
    assert np.array_equal(got, ref), (got, ref)


def _e4m3_vals(bits):
    """float64 of FP8 E4M3 bytes by torch's float8_e4m3fn (not the oracle's decoder)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def pin_e4m3_decoder(o):
    bits = np.arange(256, dtype=np.uint8)
    got = o.decode_e4m3(bits)
    ref = _e4m3_vals(bits)
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def _fp8_case(fmt, Lq, d, lengths, seed, scale, all_patterns=False):
    w = workloads.custom(Lq, d, lengths, dtype=fmt, seed=seed, order="shuffled", gap=(0, 3),
                         gap_fill="nan")
    workloads.to_fp8(w, doc_scale=scale, stride8=d + 5)
    if all_patterns:  # every finite byte somewhere in the docs
        rng = np.random.default_rng(seed)
        finite = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], np.uint8)
        for o_, n in zip(w.offsets, w.lengths):
            w.X8[o_:o_ + n, :d] = rng.choice(finite, size=(n, d))
    return w


def pin_fp8_brute_force(o):
    from fractions import Fraction

    for fmt in ("f16", "bf16"):
        for scale in (1.0, 0.37, 2.0 ** -7):
            w = _fp8_case(fmt, 3, 8, [0, 4, 1, 6, 3], seed=int(scale * 100) + len(fmt), scale=scale,
                          all_patterns=True)
            Qv = _vals(w.Q, fmt)
            Xv = _e4m3_vals(w.X8)
            sc = Fraction(float(np.float32(scale)))
            got = o.maxsim_fp8(fmt, w.Q, w.X8, w.offsets, w.lengths, w.doc_scale, d=w.d)
            for i, (a, n) in enumerate(zip(w.offsets, w.lengths)):
                if n == 0:
                    assert got[i] == float("-inf")
                    continue
                tot = Fraction(0)
                for q in range(w.Lq):
                    tot += max(sum(Fraction(float(Qv[q, k])) * sc * Fraction(float(Xv[a + t, k]))
                                   for k in range(w.d)) for t in range(n))
                assert abs(got[i] - float(tot)) <= 1e-12 * (1 + abs(float(tot))), (fmt, scale, i)


def pin_fp8_equals_f16_path(o):
    """With a power-of-two scale every doc value is exact in fp16: the FP8 score equals
    the fp16 oracle on those values, bit for bit (same loop order)."""
    w = _fp8_case("f16", 5, 24, [3, 0, 7, 1, 9], seed=21, scale=2.0 ** -6, all_patterns=True)
    vals = _e4m3_vals(w.X8[:, : w.d]) * w.doc_scale
    vals[np.isnan(vals)] = 0.0
    X16 = np.ascontiguousarray(vals.astype(np.float16)).view(np.uint16)
    assert np.array_equal(X16.view(np.float16).astype(np.float64), vals)
    got = o.maxsim_fp8("f16", w.Q, w.X8, w.offsets, w.lengths, w.doc_scale, d=w.d)
    ref = o.maxsim("f16", w.Q, X16, w.offsets, w.lengths, d=w.d)
    assert np.array_equal(got, ref)


PINS = [pin_decoders, pin_brute_force, pin_golden, pin_closed_forms, pin_one_hot,
        pin_int64_addressing, pin_e4m3_decoder, pin_fp8_brute_force, pin_fp8_equals_f16_path]


def run(o) -> list[str]:
    failed = []
    for pin in PINS:
        try:
            pin(o)
        except AssertionError as e:
            failed.append(f"{pin.__name__}: {e}")
    return failed


def main(argv) -> int:
    o = oracle.Oracle(argv[1])
    failed = run(o)
    for f in failed:
        print("FAILED", f)
    print("pins failed:", len(failed), "of", len(PINS))
    return 1 if failed else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
