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
- ``maxsim_pairs(...)``: the batch form with several queries, each doc scored against
  its own query. The pages name a pairs kernel without defining it; the reading taken
  is that doc i's score is the single-query score above for query doc_query[i], and a
  doc whose query index or rows are invalid scores NaN. Written as that selection plus
  ``maxsim``. Pinned by exact brute force per doc on tiny batches with interleaved,
  repeated, empty and invalid queries (tests/test_oracle_pairs.py).
- ``maxsim_multi(...)``: several queries against the same docs, scores [nq, B]: the
  single-query score per (query, doc). Pinned by exact brute force per (query, doc)
  (tests/test_oracle_pairs.py).
- ``decode_e4m3(bits)`` and ``maxsim_fp8(...)``: docs stored as FP8 E4M3 bits with one
  fp32 scale for the doc tensor (element = scale * e4m3), the query fp16 or bf16, as
  FP8 caches are dequantised with a per-tensor scale on the sparse prefill pages page
  (`stage_prefill_pages`). The decoder is pinned on all 256 patterns against torch's
  float8_e4m3fn; the score by exact brute force, one-hot closed forms and the
  equality with ``maxsim`` on the decoded values (tests/test_oracle_fp8.py).
- ``topk(scores, k)``: the k best docs of a score array under the ranking rule (score
  descending, ties by lower doc index; -0 ties with +0, NaN ranks below everything,
  -inf below every finite score); past B the slots hold (-inf, -1). A plain sort,
  pinned by pairwise brute force on small arrays with ties, zeros of both signs,
  infinities and NaN (tests/test_oracle_topk.py).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

__all__ = ["FMT", "build", "Oracle", "decode", "decode_e4m3", "maxsim", "maxsim_fp8",
           "maxsim_pairs", "maxsim_multi", "maxsim_workload", "max_threads", "topk"]

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
        lib.oracle_decode_e4m3_table.restype = None
        lib.oracle_decode_e4m3_table.argtypes = [ctypes.c_void_p]
        lib.maxsim_oracle_fp8_f64.restype = ctypes.c_int
        lib.maxsim_oracle_fp8_f64.argtypes = [
            ctypes.c_int, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int32, ctypes.c_double, ctypes.c_void_p, ctypes.c_int,
        ]
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

    def decode_e4m3(self, bits: np.ndarray) -> np.ndarray:
        table = np.empty(256, np.float64)
        self.lib.oracle_decode_e4m3_table(table.ctypes.data)
        return table[np.asarray(bits, dtype=np.uint8)]

    def maxsim_fp8(self, qfmt: str, Q: np.ndarray, X8: np.ndarray, offsets, lengths, doc_scale: float,
                   d: int | None = None, threads: int = 0) -> np.ndarray:
        """fp64 scores: Q uint16 [Lq, d] bits (fp16 or bf16), X8 uint8 [T, stride] E4M3
        bits, doc element = doc_scale * e4m3."""
        Q = np.ascontiguousarray(Q, dtype=np.uint16)
        X8 = np.ascontiguousarray(X8, dtype=np.uint8)
        if Q.ndim != 2 or X8.ndim != 2:
            raise ValueError("Q and X8 must be 2-D")
        Lq = Q.shape[0]
        d = Q.shape[1] if d is None else int(d)
        offs = np.ascontiguousarray(offsets, dtype=np.int32)
        lens = np.ascontiguousarray(lengths, dtype=np.int32)
        B = offs.shape[0]
        out = np.empty(B, np.float64)
        if B == 0:
            return out
        rc = self.lib.maxsim_oracle_fp8_f64(
            FMT[qfmt], Q.ctypes.data, Lq, d, X8.ctypes.data, X8.shape[1], offs.ctypes.data,
            lens.ctypes.data, B, float(doc_scale), out.ctypes.data, int(threads),
        )
        if rc:
            raise ValueError(f"maxsim_oracle_fp8_f64 failed ({rc})")
        return out


def _get() -> Oracle:
    """The oracle library: libmaxsim_oracle.so, or the build MAXSIM_ORACLE_LIBRARY names
    (the same source built otherwise, e.g. address-sanitised)."""
    global _default
    if _default is None:
        path = os.environ.get("MAXSIM_ORACLE_LIBRARY")
        if not path:
            build(force=False)
            path = LIBRARY
        _default = Oracle(path)
    return _default


def decode(bits: np.ndarray, fmt: str) -> np.ndarray:
    """The oracle's decoding of raw 16-bit patterns to float64."""
    return _get().decode(bits, fmt)


def maxsim(fmt, Q, X, offsets, lengths, d=None, threads: int = 0) -> np.ndarray:
    return _get().maxsim(fmt, Q, X, offsets, lengths, d=d, threads=threads)


def decode_e4m3(bits: np.ndarray) -> np.ndarray:
    """The oracle's decoding of FP8 E4M3 bytes to float64."""
    return _get().decode_e4m3(bits)


def maxsim_fp8(qfmt, Q, X8, offsets, lengths, doc_scale, d=None, threads: int = 0) -> np.ndarray:
    return _get().maxsim_fp8(qfmt, Q, X8, offsets, lengths, doc_scale, d=d, threads=threads)


def maxsim_pairs(fmt, Qs, q_offsets, q_lengths, X, offsets, lengths, doc_query, max_lq,
                 d=None, threads: int = 0, X8=None, doc_scale: float = 1.0) -> np.ndarray:
    """fp64 scores of docs that each take their own query.

    Query j is rows [q_offsets[j], q_offsets[j] + q_lengths[j]) of Qs (uint16 bits,
    [q_rows, d]); doc i is scored, as by ``maxsim``, against query doc_query[i]. A doc
    gets NaN when its query index is outside [0, nq) or that query has a negative
    offset or length, more than max_lq rows, or rows past the end of Qs. With X8 (FP8
    E4M3 bytes) the docs are X8 with doc_scale, as by ``maxsim_fp8``, and X is unused.
    """
    Qs = np.ascontiguousarray(Qs, dtype=np.uint16)
    d = Qs.shape[1] if d is None else int(d)
    q_offsets = np.asarray(q_offsets, np.int64)
    q_lengths = np.asarray(q_lengths, np.int64)
    offsets = np.asarray(offsets, np.int64)
    lengths = np.asarray(lengths, np.int64)
    doc_query = np.asarray(doc_query, np.int64)
    nq, q_rows = q_offsets.shape[0], Qs.shape[0]
    out = np.full(offsets.shape[0], np.nan)
    for j in np.unique(doc_query):
        if not 0 <= j < nq:
            continue
        lo, n = int(q_offsets[j]), int(q_lengths[j])
        if lo < 0 or n < 0 or n > max_lq or lo + n > q_rows:
            continue
        sel = np.nonzero(doc_query == j)[0]
        if X8 is not None:
            out[sel] = maxsim_fp8(fmt, Qs[lo:lo + n], X8, offsets[sel], lengths[sel], doc_scale, d=d,
                                  threads=threads)
        else:
            out[sel] = maxsim(fmt, Qs[lo:lo + n], X, offsets[sel], lengths[sel], d=d, threads=threads)
    return out


def maxsim_multi(fmt, Qs, q_lengths, X, offsets, lengths, d=None, threads: int = 0, X8=None,
                 doc_scale: float = 1.0) -> np.ndarray:
    """fp64 scores [nq, B]: query j (rows sum(q_lengths[:j]) .. + q_lengths[j] - 1 of
    Qs) against every doc, as by ``maxsim`` (or ``maxsim_fp8`` with X8, doc_scale)."""
    Qs = np.ascontiguousarray(Qs, dtype=np.uint16)
    q_lengths = np.asarray(q_lengths, np.int64)
    out = np.empty((q_lengths.shape[0], np.asarray(offsets).shape[0]), np.float64)
    lo = 0
    for j, n in enumerate(q_lengths.tolist()):
        if X8 is not None:
            out[j] = maxsim_fp8(fmt, Qs[lo:lo + n], X8, offsets, lengths, doc_scale, d=d, threads=threads)
        else:
            out[j] = maxsim(fmt, Qs[lo:lo + n], X, offsets, lengths, d=d, threads=threads)
        lo += n
    return out


def maxsim_workload(w, docs=None, threads: int = 0) -> np.ndarray:
    """fp64 scores of a workloads.Workload, for all docs or for the doc ids `docs`
    ([nq, len(docs)] when several queries share the docs)."""
    offs, lens = w.offsets, w.lengths
    dq = w.doc_query
    if docs is not None:
        docs = np.asarray(docs, dtype=np.int64)
        offs, lens = offs[docs], lens[docs]
        dq = None if dq is None else dq[docs]
    if w.q_lengths is not None and dq is None:
        return maxsim_multi(w.dtype, w.Q, w.q_lengths, w.X, offs, lens, d=w.d, threads=threads, X8=w.X8,
                            doc_scale=w.doc_scale)
    if dq is not None:
        return maxsim_pairs(w.dtype, w.Q, w.q_offsets, w.q_lengths, w.X, offs, lens, dq, w.Lq,
                            d=w.d, threads=threads, X8=w.X8, doc_scale=w.doc_scale)
    if w.X8 is not None:
        return maxsim_fp8(w.dtype, w.Q, w.X8, offs, lens, w.doc_scale, d=w.d, threads=threads)
    return maxsim(w.dtype, w.Q, w.X, offs, lens, d=w.d, threads=threads)


def max_threads() -> int:
    return int(_get().lib.oracle_max_threads())


def topk(scores, k: int):
    """(top_scores, top_ids) of the k best entries of a float32 score array: higher score
    first, equal scores (-0 equal to +0) by lower index, NaN after everything. Slots
    past the array's end hold (-inf, -1)."""
    vals = np.asarray(scores, dtype=np.float32)

    def rank_key(i):
        v = float(vals[i])
        return (1, 0.0, i) if v != v else (0, -v, i)  # NaN last; 0.0 == -0.0 compare equal

    order = sorted(range(vals.shape[0]), key=rank_key)[:k]
    top_ids = np.full(k, -1, np.int32)
    top_scores = np.full(k, -np.inf, np.float32)
    top_ids[: len(order)] = order
    top_scores[: len(order)] = vals[order]
    return top_scores, top_ids
