"""GPU-side helpers for the parity tests: upload a workload, run the HIP path through the
C ABI, and compare with the oracle under the acceptance rules."""

from __future__ import annotations

import numpy as np
import torch

import late_interaction_reranking_amd as lir

DEV = torch.device("cuda:0")
RTOL = 1e-3  # |gpu - oracle| <= RTOL * (1 + |oracle|)


def tdtype(fmt: str):
    return torch.float16 if fmt == "f16" else torch.bfloat16


def upload(w, dev=DEV):
    """(Q, X view [T, d] with the workload's row stride, offsets, lengths) on the GPU."""
    t = tdtype(w.dtype)
    Q = torch.from_numpy(np.ascontiguousarray(w.Q).view(np.int16)).to(dev).view(t)
    X = torch.from_numpy(w.X.view(np.int16)).to(dev).view(t)[:, : w.d]
    offs = torch.from_numpy(np.ascontiguousarray(w.offsets, dtype=np.int32)).to(dev)
    lens = torch.from_numpy(np.ascontiguousarray(w.lengths, dtype=np.int32)).to(dev)
    return Q, X, offs, lens


def upload8(w, dev=DEV):
    """(Q, FP8 doc bytes [T, d] with the workload's byte stride, offsets, lengths)."""
    t = tdtype(w.dtype)
    Q = torch.from_numpy(np.ascontiguousarray(w.Q).view(np.int16)).to(dev).view(t)
    X8 = torch.from_numpy(w.X8).to(dev)[:, : w.d]
    offs = torch.from_numpy(np.ascontiguousarray(w.offsets, dtype=np.int32)).to(dev)
    lens = torch.from_numpy(np.ascontiguousarray(w.lengths, dtype=np.int32)).to(dev)
    return Q, X8, offs, lens


def gpu_scores(w, dev=DEV) -> np.ndarray:
    Q, X, offs, lens = upload(w, dev)
    s = lir.rerank(Q, X, offs, lens)
    torch.cuda.synchronize(dev)
    return s.cpu().numpy().astype(np.float64)


def parity_report(got: np.ndarray, ref: np.ndarray) -> tuple[bool, float, int]:
    """(ok, max scaled error over finite refs, number of violations)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    inf = np.isinf(ref)
    inf_ok = np.array_equal(np.isinf(got), inf) and np.array_equal(got[inf], ref[inf])
    fin = ~inf
    if fin.any():
        err = np.abs(got[fin] - ref[fin]) / (1.0 + np.abs(ref[fin]))
        bad = int(np.sum(~(err <= RTOL)))
        mx = float(np.nanmax(err)) if np.all(np.isfinite(err)) else float("inf")
    else:
        bad, mx = 0, 0.0
    return inf_ok and bad == 0, mx, bad + (0 if inf_ok else 1)


def assert_parity(got, ref, what=""):
    ok, mx, bad = parity_report(got, ref)
    assert ok, f"{what}: {bad} docs outside |err| <= {RTOL}(1+|s|) (max scaled err {mx:.3e})"
    return mx


def top_k(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k best scores, descending, ties by lower index."""
    order = np.lexsort((np.arange(len(scores)), -np.asarray(scores, np.float64)))
    return order[:k]


def top10_ok(got: np.ndarray, ref_of, ref_sorted_top: np.ndarray, k: int = 10) -> bool:
    """The GPU's top-k, scored by the oracle (ref_of maps doc ids to oracle scores),
    reproduces the oracle's sorted top-k scores within tolerance rank by rank: swaps
    happen only between oracle near-ties."""
    gtop = top_k(got, k)
    if len(set(gtop.tolist())) != k:
        return False
    mine = np.asarray(ref_of(gtop), np.float64)
    want = np.asarray(ref_sorted_top[:k], np.float64)
    return bool(np.all(np.abs(mine - want) <= RTOL * (1.0 + np.abs(want))))
