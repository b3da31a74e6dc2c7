"""fp64 CPU oracle for Flash-MaxSim reranking (ctypes wrapper over maxsim_oracle.c).

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU-baseline
leg import this package. The GPU library never imports, links or calls it, and the
two share no code.

Functions and what pins each of them (the pins live in tests/test_oracle.py,
tests/test_oracle_golden.py and tests/test_oracle_mutants.py):

- ``decode(bits, fmt)``: the oracle's own binary16 / bfloat16 decoders. Pinned on
  all 65,536 bit patterns of each format against numpy's float16 and torch's
  bfloat16 conversions.
- ``maxsim(...)``: the score definition of the Flash-MaxSim rerank page (docs.vllm.ai,
  vllm.v1.pool.flash_maxsim.flash_maxsim_rerank, module description and the
  ``flash_maxsim_rerank_direct`` parameters), in fp64. Pinned by exact rational brute
  force on tiny inputs, the single-query-row and single-token closed forms, integer
  and one-hot inputs with exact answers, invariances (token permutation and
  duplication, packing, doc order, contents of rows and columns outside the docs,
  scaling), the empty-doc / empty-query special cases, and by hand-worked golden
  examples. A mutation test plants plausible mistakes in a copy of the C source and
  checks that the pins catch each one.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

__all__ = ["FMT", "build", "Oracle", "decode", "maxsim", "maxsim_workload", "max_threads"]

FMT = {"f16": 0, "bf16": 1}

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "maxsim_oracle.c")
LIBRARY = os.path.join(_HERE, "libmaxsim_oracle.so")

_lock = threading.Lock()
_default = None


def compile_source(src: str, out: str) -> None:
    """Compile one oracle C source into a shared library with gcc."""
    cmd = [
        "gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
        "-std=c11", "-Wall", "-o", out + ".tmp", src, "-lm",
    ]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(out + ".tmp", out)


def build(force: bool = True) -> str:
    """Compile maxsim_oracle.c into libmaxsim_oracle.so next to it."""
    with _lock:
        if force or not os.path.exists(LIBRARY) or (
            os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE)
        ):
            compile_source(SOURCE, LIBRARY)
    return LIBRARY


class Oracle:
    """One loaded copy of the oracle library (the mutation test loads mutants)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        lib.oracle_decode_f16.restype = ctypes.c_double
        lib.oracle_decode_f16.argtypes = [ctypes.c_uint16]
        lib.oracle_decode_bf16.restype = ctypes.c_double
        lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
        lib.oracle_decode_table.restype = ctypes.c_int
        lib.oracle_decode_table.argtypes = [ctypes.c_int, ctypes.c_void_p]
        lib.maxsim_oracle_f64.restype = ctypes.c_int
        lib.maxsim_oracle_f64.argtypes = [
            ctypes.c_int, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int32, ctypes.c_void_p, ctypes.c_int,
        ]
        lib.oracle_max_threads.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def decode(self, bits: np.ndarray, fmt: str) -> np.ndarray:
        table = np.empty(65536, np.float64)
        rc = self.lib.oracle_decode_table(FMT[fmt], table.ctypes.data)
        if rc:
            raise ValueError(f"oracle_decode_table failed ({rc})")
        return table[np.asarray(bits, dtype=np.uint16)]

    def maxsim(self, fmt: str, Q: np.ndarray, X: np.ndarray, offsets, lengths,
               d: int | None = None, threads: int = 0) -> np.ndarray:
        """fp64 scores for docs (offsets[i], lengths[i]) of the row tensor X.

        Q: uint16 [Lq, d] bits. X: uint16 [T, stride] bits (row stride = X.shape[1]).
        """
        Q = np.ascontiguousarray(Q, dtype=np.uint16)
        X = np.ascontiguousarray(X, dtype=np.uint16)
        if Q.ndim != 2 or X.ndim != 2:
            raise ValueError("Q and X must be 2-D")
        Lq = Q.shape[0]
        d = Q.shape[1] if d is None else int(d)
        if Q.shape[1] != d:
            raise ValueError("Q width must equal d")
        offs = np.ascontiguousarray(offsets, dtype=np.int32)
        lens = np.ascontiguousarray(lengths, dtype=np.int32)
        B = offs.shape[0]
        if lens.shape[0] != B:
            raise ValueError("offsets and lengths differ in length")
        out = np.empty(B, np.float64)
        if B == 0:
            return out
        rc = self.lib.maxsim_oracle_f64(
            FMT[fmt], Q.ctypes.data, Lq, d, X.ctypes.data, X.shape[1],
            offs.ctypes.data, lens.ctypes.data, B, out.ctypes.data, int(threads),
        )
        if rc:
            raise ValueError(f"maxsim_oracle_f64 failed ({rc})")
        return out


def _get() -> Oracle:
    global _default
    if _default is None:
        build(force=False)
        _default = Oracle(LIBRARY)
    return _default


def decode(bits: np.ndarray, fmt: str) -> np.ndarray:
    """The oracle's decoding of raw 16-bit patterns to float64."""
    return _get().decode(bits, fmt)


def maxsim(fmt, Q, X, offsets, lengths, d=None, threads: int = 0) -> np.ndarray:
    return _get().maxsim(fmt, Q, X, offsets, lengths, d=d, threads=threads)


def maxsim_workload(w, docs=None, threads: int = 0) -> np.ndarray:
    """fp64 scores of a workloads.Workload, for all docs or for the doc ids `docs`."""
    offs, lens = w.offsets, w.lengths
    if docs is not None:
        docs = np.asarray(docs, dtype=np.int64)
        offs, lens = offs[docs], lens[docs]
    return maxsim(w.dtype, w.Q, w.X, offs, lens, d=w.d, threads=threads)


def max_threads() -> int:
    return int(_get().lib.oracle_max_threads())
