"""Seeded synthetic MaxSim rerank workloads.

Builds, for one query, the inputs that the Flash-MaxSim rerank page ("Flash-MaxSim
rerank: one query vs variable-length docs in a packed tensor", module docstring and the
`flash_maxsim_rerank_direct` parameter list) describes: a query ``Q[Lq, d]``, a packed
doc-row tensor ``X[T, stride]`` holding every doc's tokens (possibly scattered, with
unrelated rows between them) and one int32 ``(offset, length)`` pair per doc.

This module holds none of the method's arithmetic. It only draws random numbers,
scales each row to unit length, rounds rows to the storage format (IEEE binary16 or
bfloat16, round to nearest even) and lays docs out in memory. Both the GPU path's tests
and the CPU oracle's tests take their inputs from here; neither side's arithmetic lives
here.

All arrays hold raw 16-bit patterns (``uint16``), whatever the storage format, so both
sides decode the very same bits.

Seeding: every draw comes from ``numpy.random.default_rng([seed, stream, ...])``
(PCG64), with one stream for the doc table (lengths, order, gaps, planted rows), one for
Q, and one per 2**18-row chunk of X, so the result does not depend on thread count.
"""

from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Workload",
    "CONFIGS",
    "make",
    "custom",
    "tiny",
    "colbert",
    "long_doc",
    "scattered",
    "large",
    "pairs",
    "custom_pairs",
    "shared",
    "custom_multi",
    "large_fp8",
    "shared_fp8",
    "to_fp8",
    "E4M3_NAN",
    "round_f16",
    "round_bf16",
    "F16_NAN",
    "BF16_NAN",
]

F16_NAN = 0x7E00
BF16_NAN = 0x7FC0
E4M3_NAN = 0x7F
_CHUNK_ROWS = 1 << 18

_S_META, _S_Q, _S_ROWS, _S_PLANT = 0, 1, 2, 3


@dataclass
class Workload:
    """One query and a packed, possibly scattered doc collection."""

    name: str
    dtype: str  # "f16" or "bf16": storage format of Q and X
    Lq: int
    d: int
    stride: int  # elements between consecutive rows of X (>= d)
    Q: np.ndarray  # uint16 [Lq, d], raw bits
    X: np.ndarray  # uint16 [T, stride], raw bits
    offsets: np.ndarray  # int32 [B], first row of each doc in X
    lengths: np.ndarray  # int32 [B], rows per doc
    seed: int = 0
    planted: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))
    notes: str = ""
    # Several queries in one batch (None: one query, Q itself). Query j is rows
    # [q_offsets[j], q_offsets[j] + q_lengths[j]) of Q; Lq is then the longest query.
    # With doc_query, doc i takes query doc_query[i] ("pairs"); without it, every
    # query scores every doc (shared docs, scores [nq, B]).
    q_offsets: np.ndarray | None = None  # int32 [nq]
    q_lengths: np.ndarray | None = None  # int32 [nq]
    doc_query: np.ndarray | None = None  # int32 [B]
    # Docs stored as FP8 E4M3 bits (None: X holds them): element = doc_scale * e4m3.
    X8: np.ndarray | None = None         # uint8 [T, stride8]
    doc_scale: float = 1.0

    @property
    def B(self) -> int:
        return int(self.offsets.shape[0])

    @property
    def multi_query(self) -> bool:
        return self.doc_query is not None

    @property
    def shared_docs(self) -> bool:
        return self.q_lengths is not None and self.doc_query is None

    @property
    def nq(self) -> int:
        return 1 if self.q_offsets is None else int(self.q_offsets.shape[0])

    @property
    def T(self) -> int:
        return int((self.X8 if self.X8 is not None else self.X).shape[0])

    @property
    def doc_tokens(self) -> int:
        return int(self.lengths.astype(np.int64).sum())

    @property
    def doc_bytes(self) -> int:
        """Bytes of doc rows the method must read: 2*d per doc token (d with FP8 docs)."""
        return self.doc_tokens * (1 if self.X8 is not None else 2) * self.d


# --------------------------------------------------------------------------- rounding


def round_f16(x: np.ndarray) -> np.ndarray:
    """fp32 -> IEEE binary16 bits, round to nearest even (numpy's cast)."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bits, round to nearest even on the fp32 bit pattern.

    bfloat16 is the upper half of a binary32 word; rounding adds 0x7FFF plus the
    lowest kept bit before truncating. Only finite inputs are produced here.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _round(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return round_f16(x)
    if dtype == "bf16":
        return round_bf16(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def _bits_to_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float32)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _nan_bits(dtype: str) -> int:
    return F16_NAN if dtype == "f16" else BF16_NAN


# --------------------------------------------------------------------------- rows


def _unit_rows(rng: np.random.Generator, n: int, d: int) -> np.ndarray:
    """n rows drawn N(0, I_d) in fp32, each scaled to unit L2 norm in fp32."""
    x = rng.standard_normal((n, d), dtype=np.float32)
    nrm = np.sqrt(np.einsum("ij,ij->i", x, x, dtype=np.float32))
    nrm[nrm == 0] = 1.0
    x /= nrm[:, None]
    return x


def _fill_rows(X: np.ndarray, d: int, dtype: str, seed: int, threads: int | None) -> None:
    """Fill X[:, :d] with rounded unit rows, one independent RNG stream per chunk."""
    T = X.shape[0]
    nchunks = (T + _CHUNK_ROWS - 1) // _CHUNK_ROWS

    def one(c: int) -> None:
        r0 = c * _CHUNK_ROWS
        r1 = min(T, r0 + _CHUNK_ROWS)
        rng = np.random.default_rng([seed, _S_ROWS, c])
        X[r0:r1, :d] = _round(_unit_rows(rng, r1 - r0, d), dtype)

    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    if nchunks <= 1 or threads <= 1:
        for c in range(nchunks):
            one(c)
    else:
        with _cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, range(nchunks)))


# --------------------------------------------------------------------------- layout


def _layout(
    lengths: np.ndarray,
    order: np.ndarray,
    gaps: np.ndarray,
    lead: int,
) -> tuple[np.ndarray, int]:
    """Place docs in memory in `order`, with `gaps[k]` rows after the k-th placed doc.

    Returns (offsets indexed by doc id, total rows T).
    """
    B = lengths.shape[0]
    offsets = np.zeros(B, np.int64)
    pos = int(lead)
    for k, i in enumerate(order):
        offsets[i] = pos
        pos += int(lengths[i]) + (int(gaps[k]) if k < len(gaps) else 0)
    return offsets, pos


def custom(
    Lq: int,
    d: int,
    lengths,
    *,
    dtype: str = "f16",
    seed: int = 0,
    stride: int | None = None,
    order: str = "in_order",
    gap: tuple[int, int] | None = None,
    lead_gap: int | None = None,
    trailing_gap: int = 0,
    gap_fill: str = "random",
    pad_fill: str = "nan",
    name: str = "custom",
    threads: int | None = None,
) -> Workload:
    """General builder.

    order: "in_order" (doc i placed i-th) or "shuffled" (random memory order).
    gap: inclusive integer range of unrelated rows between consecutive docs in memory
        (None = packed back to back); lead_gap rows before the first doc (default: one
        draw from `gap`, or 0); trailing_gap rows after the last one.
    gap_fill: "random" (unit rows, like other tokens of a batch) or "nan".
    pad_fill: contents of columns d..stride-1: "nan" or "zero".
    """
    stride = d if stride is None else int(stride)
    if stride < d:
        raise ValueError("stride must be >= d")
    lengths = np.asarray(lengths, dtype=np.int64)
    B = int(lengths.shape[0])
    meta = np.random.default_rng([seed, _S_META, 1])
    if order == "in_order":
        perm = np.arange(B)
    elif order == "shuffled":
        perm = meta.permutation(B)
    else:
        raise ValueError(f"unknown order {order!r}")
    if gap is None:
        gaps = np.zeros(max(B - 1, 0), np.int64)
        lead = 0 if lead_gap is None else lead_gap
    else:
        gaps = meta.integers(gap[0], gap[1], size=max(B - 1, 0), endpoint=True)
        lead = int(meta.integers(gap[0], gap[1], endpoint=True)) if lead_gap is None else lead_gap
    offsets, T = _layout(lengths, perm, gaps, lead)
    T += int(trailing_gap)

    X = np.zeros((T, stride), np.uint16)
    _fill_rows(X, d, dtype, seed, threads)
    nan = _nan_bits(dtype)
    if stride > d:
        X[:, d:] = nan if pad_fill == "nan" else 0
    if gap_fill == "nan" and B:
        in_doc = np.zeros(T, bool)
        for o, n in zip(offsets, lengths):
            in_doc[o : o + n] = True
        X[~in_doc, :d] = nan

    qrng = np.random.default_rng([seed, _S_Q])
    Q = _round(_unit_rows(qrng, Lq, d), dtype) if Lq else np.zeros((0, d), np.uint16)
    return Workload(
        name=name,
        dtype=dtype,
        Lq=int(Lq),
        d=int(d),
        stride=stride,
        Q=Q,
        X=X,
        offsets=offsets.astype(np.int32),
        lengths=lengths.astype(np.int32),
        seed=seed,
    )


# --------------------------------------------------------------------------- configs


def tiny(seed: int = 0, **kw) -> Workload:
    """Lq 32, d 128, B 64, lengths U[16,128], packed back to back in doc order, fp16."""
    meta = np.random.default_rng([seed, _S_META, 0])
    lengths = meta.integers(16, 128, size=64, endpoint=True)
    return custom(32, 128, lengths, dtype="f16", seed=seed, name="tiny", **kw)


def colbert(seed: int = 1, **kw) -> Workload:
    """ColBERT-shaped: Lq 32, d 128, B 1000, lengths U[64,300], packed in a random
    doc order, fp16."""
    meta = np.random.default_rng([seed, _S_META, 0])
    lengths = meta.integers(64, 300, size=1000, endpoint=True)
    return custom(32, 128, lengths, dtype="f16", seed=seed, order="shuffled",
                  name="colbert", **kw)


def long_doc(seed: int = 2, **kw) -> Workload:
    """Long docs: Lq 128, d 128, B 256, lengths rint(exp(N(ln 1024, 0.6^2))) clipped
    to [32, 4096], packed in doc order, bf16."""
    meta = np.random.default_rng([seed, _S_META, 0])
    raw = np.rint(np.exp(meta.normal(np.log(1024.0), 0.6, size=256)))
    lengths = np.clip(raw, 32, 4096).astype(np.int64)
    return custom(128, 128, lengths, dtype="bf16", seed=seed, name="long_doc", **kw)


def scattered(seed: int = 3, gap_fill: str = "random", **kw) -> Workload:
    """Scattered ragged: Lq 37, d 96, B 8192, lengths U[1,512], random memory order,
    U[1,48] unrelated rows before the first doc and between consecutive docs, none after
    the last (the last doc ends on the tensor's last row), fp16.

    The workload text asks for a 2,000,000-token tensor, but 8192 docs of mean length
    256.5 already hold ~2.1 M tokens; B, the length law, Lq, d and dtype are kept and
    the tensor grows to fit (~2.3 M rows).
    """
    meta = np.random.default_rng([seed, _S_META, 0])
    lengths = meta.integers(1, 512, size=8192, endpoint=True)
    return custom(37, 96, lengths, dtype="f16", seed=seed, order="shuffled",
                  gap=(1, 48), trailing_gap=0, gap_fill=gap_fill, name="scattered", **kw)


def large(seed: int = 4, plant_frac: float = 0.01, noise: float = 0.02, **kw) -> Workload:
    """Large, int64-addressed: Lq 32, d 128, B 80,000, lengths U[64,448] (~20.5 M rows,
    ~5.2 GB fp16, row offset * d past 2**31), packed in doc order, fp16.

    For plant_frac of the docs (chosen at random) one random token row is replaced by a
    near-duplicate of a random query row: unit(Q[q] + noise * z), z ~ N(0, I_d).
    """
    meta = np.random.default_rng([seed, _S_META, 0])
    lengths = meta.integers(64, 448, size=80_000, endpoint=True)
    w = custom(32, 128, lengths, dtype="f16", seed=seed, name="large", **kw)
    _plant(w, plant_frac, noise)
    return w


def _plant(w: Workload, frac: float, noise: float) -> None:
    nplant = int(round(frac * w.B))
    if nplant == 0:
        return
    rng = np.random.default_rng([w.seed, _S_PLANT])
    docs = np.sort(rng.choice(w.B, size=nplant, replace=False))
    toks = rng.integers(0, w.lengths[docs].astype(np.int64))
    qrows = rng.integers(0, w.Lq, size=nplant)
    z = rng.standard_normal((nplant, w.d), dtype=np.float32)
    qf = _bits_to_f32(w.Q, w.dtype)
    rows = qf[qrows] + np.float32(noise) * z
    rows /= np.sqrt(np.einsum("ij,ij->i", rows, rows, dtype=np.float32))[:, None]
    w.X[w.offsets[docs].astype(np.int64) + toks, : w.d] = _round(rows, w.dtype)
    w.planted = docs.astype(np.int64)


def custom_pairs(
    q_lengths,
    d: int,
    docs_per_query,
    doc_lengths,
    *,
    dtype: str = "f16",
    seed: int = 0,
    interleave: bool = False,
    name: str = "custom_pairs",
    **kw,
) -> Workload:
    """A batch of several queries, each with its own docs.

    q_lengths[j]: rows of query j (its rows follow query j-1's in Q).
    docs_per_query[j]: docs of query j; doc_lengths: one length per doc, in doc order.
    Docs are numbered query by query (all of query 0's, then query 1's, ...), unless
    interleave, which shuffles the doc -> query assignment. Other keywords go to
    custom() and shape the doc-row tensor.
    """
    q_lengths = np.asarray(q_lengths, dtype=np.int64)
    docs_per_query = np.asarray(docs_per_query, dtype=np.int64)
    if q_lengths.shape != docs_per_query.shape:
        raise ValueError("one docs_per_query entry per query")
    w = custom(0, d, doc_lengths, dtype=dtype, seed=seed, name=name, **kw)
    if int(docs_per_query.sum()) != w.B:
        raise ValueError("docs_per_query must sum to the number of docs")
    doc_query = np.repeat(np.arange(q_lengths.shape[0]), docs_per_query)
    if interleave:
        doc_query = np.random.default_rng([seed, _S_META, 2]).permutation(doc_query)
    q_offsets = np.concatenate([[0], np.cumsum(q_lengths)[:-1]]) if q_lengths.size else q_lengths
    rows = int(q_lengths.sum())
    qrng = np.random.default_rng([seed, _S_Q])
    w.Q = _round(_unit_rows(qrng, rows, d), dtype) if rows else np.zeros((0, d), np.uint16)
    w.Lq = int(q_lengths.max()) if q_lengths.size else 0
    w.q_offsets = q_offsets.astype(np.int32)
    w.q_lengths = q_lengths.astype(np.int32)
    w.doc_query = doc_query.astype(np.int32)
    return w


def pairs(seed: int = 5, **kw) -> Workload:
    """A serving batch of 64 queries with lengths U[16,32], each with 1000 ColBERT-
    shaped docs (lengths U[64,300]), d 128, fp16: 64,000 docs, ~11.3 M rows packed
    query by query, each query's docs in a random memory order."""
    meta = np.random.default_rng([seed, _S_META, 0])
    nq, per = 64, 1000
    q_lengths = meta.integers(16, 32, size=nq, endpoint=True)
    lengths = meta.integers(64, 300, size=nq * per, endpoint=True)
    perm = np.concatenate([j * per + meta.permutation(per) for j in range(nq)])
    w = custom_pairs(q_lengths, 128, np.full(nq, per), lengths, dtype="f16", seed=seed,
                     name="pairs", **kw)
    # Re-lay docs so that each query's docs sit together in memory, shuffled within.
    offsets, T = _layout(w.lengths.astype(np.int64), perm, np.zeros(nq * per - 1, np.int64), 0)
    assert T == w.T
    w.offsets = offsets.astype(np.int32)
    return w


def to_fp8(w: Workload, doc_scale: float = 2.0 ** -8, stride8: int | None = None,
           keep_x: bool = True) -> Workload:
    """Store w's docs as FP8 E4M3: X8 = e4m3(decode(X) / doc_scale), round to nearest
    even by torch's float8_e4m3fn conversion (no value reaches 448 for unit rows at
    the default scale). Rows are stride8 bytes apart (default: the row width rounded
    up to 16); bytes past d hold the E4M3 NaN pattern, as do rows that held NaN.
    The scale is stored rounded to fp32."""
    import torch

    d = w.d
    stride8 = ((d + 15) // 16) * 16 if stride8 is None else int(stride8)
    if stride8 < d:
        raise ValueError("stride8 must be >= d")
    doc_scale = float(np.float32(doc_scale))
    X8 = np.full((w.T, stride8), E4M3_NAN, np.uint8)
    for r0 in range(0, w.T, _CHUNK_ROWS):
        r1 = min(w.T, r0 + _CHUNK_ROWS)
        v = _bits_to_f32(np.ascontiguousarray(w.X[r0:r1, :d]), w.dtype) / np.float32(doc_scale)
        X8[r0:r1, :d] = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    w.X8 = X8
    w.doc_scale = doc_scale
    if not keep_x:
        w.X = np.zeros((0, w.stride), np.uint16)
    return w


def large_fp8(seed: int = 4, **kw) -> Workload:
    """The large workload (same docs, query and seed) with docs stored as FP8 E4M3,
    doc scale 2^-8, rows 128 bytes apart (~2.6 GB)."""
    w = large(seed=seed, **kw)
    w.name = "large_fp8"
    return to_fp8(w, keep_x=False)


def shared_fp8(seed: int = 6, **kw) -> Workload:
    """The shared workload (8 queries of 32 rows, the same 80,000 docs) with docs stored
    as FP8 E4M3 bytes, doc scale 2^-8, rows 128 bytes apart (~2.6 GB)."""
    w = shared(seed=seed, **kw)
    w.name = "shared_fp8"
    return to_fp8(w, keep_x=False)


def custom_multi(q_lengths, d: int, doc_lengths, *, dtype: str = "f16", seed: int = 0,
                 name: str = "custom_multi", **kw) -> Workload:
    """Several queries (rows back to back in Q, lengths q_lengths) that all score the
    same docs. Other keywords go to custom() and shape the doc-row tensor."""
    q_lengths = np.asarray(q_lengths, dtype=np.int64)
    w = custom(0, d, doc_lengths, dtype=dtype, seed=seed, name=name, **kw)
    rows = int(q_lengths.sum())
    qrng = np.random.default_rng([seed, _S_Q])
    w.Q = _round(_unit_rows(qrng, rows, d), dtype) if rows else np.zeros((0, d), np.uint16)
    w.Lq = int(q_lengths.max()) if q_lengths.size else 0
    q_offsets = np.concatenate([[0], np.cumsum(q_lengths)[:-1]]) if q_lengths.size else q_lengths
    w.q_offsets = q_offsets.astype(np.int32)
    w.q_lengths = q_lengths.astype(np.int32)
    return w


def shared(seed: int = 6, **kw) -> Workload:
    """8 queries of 32 rows against the same 80,000 fp16 docs of U[64,448] rows, d 128,
    packed back to back in doc order (~20.5 M rows, 5.2 GB): e.g. query variants or
    several users over one candidate set."""
    meta = np.random.default_rng([seed, _S_META, 0])
    lengths = meta.integers(64, 448, size=80_000, endpoint=True)
    return custom_multi(np.full(8, 32), 128, lengths, dtype="f16", seed=seed, name="shared", **kw)


CONFIGS = {
    "tiny": tiny,
    "colbert": colbert,
    "long_doc": long_doc,
    "scattered": scattered,
    "large": large,
    "pairs": pairs,
    "shared": shared,
    "large_fp8": large_fp8,
    "shared_fp8": shared_fp8,
}


def make(name: str, **kw) -> Workload:
    """Build one of the named workloads."""
    return CONFIGS[name](**kw)
