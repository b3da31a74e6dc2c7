"""Device top-k (maxsim_topk, maxsim_rerank_topk) on the GPU.

The selection is integer work on the float bits: given the same score array, the GPU's
(ids, score bits) must equal the oracle's top-k exactly (score descending, ties by lower
index, -0 equal to +0, NaN last, (-inf, -1) past the end). Through the rerank, the ids
must equal the exact top-k of the GPU's own scores, and, scored by the oracle, reproduce
the oracle's sorted top-k within the parity tolerance (swaps only at near-ties)."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

if torch.cuda.is_available():
    import late_interaction_reranking_amd as lir
    from devio import DEV, RTOL, gpu_scores, upload


def _say(msg):
    print(msg, flush=True)


def gpu_topk(vals, k):
    s = torch.from_numpy(np.ascontiguousarray(vals, dtype=np.float32)).to(DEV)
    ts, ti = lir.maxsim_topk(s, k)
    torch.cuda.synchronize()
    return ts.cpu().numpy(), ti.cpu().numpy()


def assert_same_topk(vals, k):
    ts, ti = gpu_topk(vals, k)
    rs, ri = oracle.topk(vals, k)
    assert np.array_equal(ti, ri), (ti[:20], ri[:20])
    assert np.array_equal(ts.view(np.uint32), rs.view(np.uint32))


def spiky(rng, n):
    pool = np.array([0.0, -0.0, 1.0, -1.0, 2.5, np.inf, -np.inf, np.nan, 7.0], np.float32)
    v = rng.standard_normal(n).astype(np.float32)
    pick = rng.random(n) < 0.3
    v[pick] = rng.choice(pool, int(pick.sum()))
    return v


@pytest.mark.parametrize("B", [0, 1, 7, 4095, 4096, 4097, 20000, 80000])
@pytest.mark.parametrize("k", [1, 10, 100, 1024])
def test_topk_exact(B, k):
    _say(f"[topk] B={B} k={k}")
    rng = np.random.default_rng([B, k])
    assert_same_topk(spiky(rng, B), k)


def test_topk_all_ties_and_many_levels():
    _say("[topk] ties, 1.3 M scores")
    assert_same_topk(np.full(10000, 3.0, np.float32), 1024)
    rng = np.random.default_rng(1)
    v = np.round(rng.standard_normal(1_300_000), 2).astype(np.float32)  # heavy ties
    for k in (1, 64, 1000, 1024):
        assert_same_topk(v, k)


@pytest.mark.parametrize("name", ["tiny", "colbert", "long_doc", "scattered"])
def test_rerank_topk_matches_scores_and_oracle(name):
    _say(f"[topk] rerank {name}")
    w = workloads.make(name)
    k = min(100, w.B)
    Q, X, offs, lens = upload(w)
    ts, ti = lir.maxsim_rerank_topk(Q, X, offs, lens, k)
    torch.cuda.synchronize()
    ts, ti = ts.cpu().numpy(), ti.cpu().numpy()
    got = gpu_scores(w).astype(np.float32)
    rs, ri = oracle.topk(got, k)                      # exact selection on the GPU's scores
    assert np.array_equal(ti, ri) and np.array_equal(ts.view(np.uint32), rs.view(np.uint32))
    ref = oracle.maxsim_workload(w)                   # ranking vs the fp64 oracle
    want = np.sort(ref)[::-1][:k]
    mine = ref[ti]
    assert np.all(np.abs(mine - want) <= RTOL * (1 + np.abs(want)))


def test_rerank_topk_k_past_batch_and_empty():
    _say("[topk] k > B, B = 0")
    w = workloads.custom(16, 64, [5, 0, 9], seed=2)
    Q, X, offs, lens = upload(w)
    ts, ti = lir.maxsim_rerank_topk(Q, X, offs, lens, 6)
    ts, ti = ts.cpu().numpy(), ti.cpu().numpy()
    got = gpu_scores(w).astype(np.float32)
    rs, ri = oracle.topk(got, 6)
    assert np.array_equal(ti, ri) and list(ti[3:]) == [-1, -1, -1]
    assert ti[2] == 1 and ts[2] == -np.inf          # the empty doc ranks last among docs
    ts, ti = lir.maxsim_rerank_topk(Q, X, offs[:0], lens[:0], 4)
    assert list(ti.cpu().numpy()) == [-1] * 4


def test_topk_errors_raise():
    s = torch.zeros(10, dtype=torch.float32, device=DEV)
    with pytest.raises(lir.MaxSimError):
        lir.maxsim_topk(s, 1025)
    with pytest.raises(ValueError):
        lir.maxsim_topk(s.double(), 3)
    with pytest.raises(ValueError):
        lir.maxsim_topk(s, -1)
