"""Several queries against the same docs ("shared docs") on the GPU, through the C ABI.

Each pass of up to 128 query rows (64 when d > 128) reads every doc tile once. Scores
[nq, B] are compared with the oracle under the usual rule, |gpu - oracle| <=
1e-3 (1 + |oracle|) with -inf where the oracle has it, and each query's row must equal,
bit for bit, what the single-query entry point gives for that query alone: every query
starts on a 16-row tile, so its rows meet the same lanes in the same order.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

if torch.cuda.is_available():
    import late_interaction_reranking_amd as lir
    from devio import DEV, assert_parity, gpu_scores, upload


def _say(msg):
    print(msg, flush=True)


def multi_scores(w):
    Q, X, offs, lens = upload(w)
    s = lir.rerank_multi(Q, w.q_lengths, X, offs, lens)
    torch.cuda.synchronize()
    return s.cpu().numpy().astype(np.float64)


def alone(w, j):
    lo, n = int(w.q_offsets[j]), int(w.q_lengths[j])
    wj = workloads.Workload(**{**w.__dict__, "Q": np.ascontiguousarray(w.Q[lo:lo + n]), "Lq": n,
                               "q_offsets": None, "q_lengths": None, "doc_query": None})
    return gpu_scores(wj)


def ragged_docs(seed, n=120, max_len=300, long_docs=0):
    rng = np.random.default_rng(seed)
    lengths = rng.integers(0, max_len, size=n)
    lengths[:5] = [0, 1, 15, 16, 17]
    if long_docs:
        lengths[rng.choice(n, long_docs, replace=False)] = rng.integers(2000, 6000, long_docs)
    return lengths


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("d,stride", [(128, 128), (96, 104), (256, 264), (32, 40)])
def test_multi_parity_and_each_query_alone(fmt, d, stride):
    _say(f"[multi] parity {fmt} d={d}")
    q_lengths = [32, 0, 1, 17, 16, 100, 5, 64, 33, 200, 8, 32]
    w = workloads.custom_multi(q_lengths, d, ragged_docs(d, long_docs=3), dtype=fmt, seed=d + len(fmt),
                               stride=stride, order="shuffled", gap=(0, 4), gap_fill="nan")
    got = multi_scores(w)
    ref = oracle.maxsim_workload(w)
    assert got.shape == (len(q_lengths), w.B)
    for j in range(len(q_lengths)):
        assert_parity(got[j], ref[j], f"query {j} (Lq={q_lengths[j]})")
        assert np.array_equal(got[j], alone(w, j)), f"query {j} alone"


def test_multi_single_query_equals_rerank():
    _say("[multi] nq = 1")
    w = workloads.colbert()
    ref = gpu_scores(w)
    got = multi_scores(workloads.Workload(**{**w.__dict__, "q_offsets": np.array([0], np.int32),
                                             "q_lengths": np.array([w.Lq], np.int32)}))
    assert np.array_equal(got[0], ref)


def test_multi_many_queries_and_empty_runs():
    """More queries than one pass holds, and a run of 130 empty queries between two
    non-empty ones (the pass's score-row offset stays small)."""
    _say("[multi] many queries")
    q_lengths = [5] + [0] * 130 + [5] + [32] * 9 + [3] * 20
    w = workloads.custom_multi(q_lengths, 64, ragged_docs(3, n=60), seed=4)
    got = multi_scores(w)
    ref = oracle.maxsim_workload(w)
    for j in range(len(q_lengths)):
        assert_parity(got[j], ref[j], f"query {j}")
    assert np.all(got[1:131] == 0.0)


def test_multi_empty_cases():
    _say("[multi] empty")
    w = workloads.custom_multi([0, 0], 64, ragged_docs(5, n=10), seed=5)
    assert np.array_equal(multi_scores(w), np.zeros((2, 10)))
    Q, X, offs, lens = upload(w)
    assert lir.rerank_multi(Q, [], X, offs, lens).shape == (0, 10)
    assert lir.rerank_multi(Q, [0, 0], X, offs[:0], lens[:0]).shape == (2, 0)


def test_multi_long_docs_split():
    _say("[multi] long docs, split")
    w = workloads.custom_multi([32, 32, 20, 7], 128, np.array([8000, 3000, 5000, 7, 0, 6000]), seed=9,
                               order="shuffled", gap=(1, 3), gap_fill="nan")
    got = multi_scores(w)
    ref = oracle.maxsim_workload(w)
    for j in range(4):
        assert_parity(got[j], ref[j], f"query {j}")
        assert np.array_equal(got[j], alone(w, j))


def test_multi_errors_raise():
    _say("[multi] errors")
    w = workloads.custom_multi([4, 4], 64, ragged_docs(6, n=10), seed=6)
    Q, X, offs, lens = upload(w)
    with pytest.raises(ValueError):
        lir.rerank_multi(Q, [4, 5], X, offs, lens)  # rows do not add up
    Qbig = torch.zeros((300, 64), dtype=torch.float16, device=DEV)
    with pytest.raises(lir.MaxSimError):
        lir.rerank_multi(Qbig, [257, 43], X, offs, lens)
    with pytest.raises(lir.MaxSimError):
        lir.rerank_multi(Qbig, [301, -1], X, offs, lens)
    with pytest.raises(TypeError):
        lir.maxsim_rerank_multi_bf16(Q, [4, 4], X, offs, lens)


@pytest.mark.slow
def test_multi_shared_workload_sampled():
    """8 queries x 80,000 docs (~20.5 M rows): a sample of docs for every query."""
    _say("[multi] shared workload (generating ~5.2 GB)")
    w = workloads.make("shared")
    got = multi_scores(w)
    rng = np.random.default_rng(1)
    sample = np.unique(np.concatenate([rng.choice(w.B, 1500, replace=False), [0, w.B - 1]]))
    ref = oracle.maxsim_workload(w, docs=sample)
    for j in range(w.nq):
        assert_parity(got[j][sample], ref[j], f"shared query {j}")
