"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on the GPU.

Acceptance: per doc |gpu - oracle| <= 1e-3 (1 + |oracle|), an oracle -inf must be a GPU
-inf, and the GPU's top-10 must reproduce the oracle's sorted top-10 scores rank by rank
within that tolerance. Inputs whose every partial sum is exact (integers, one-hot rows)
must match bitwise; so must results that the method leaves unchanged (token order,
packing, doc order, chunking of long docs).
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from cases import doc_rows, one_hot_case, one_hot_expected, repack, small_int_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

if torch.cuda.is_available():
    import late_interaction_reranking_amd as lir
    from devio import DEV, assert_parity, gpu_scores, top10_ok, top_k, upload


def _say(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------ named workloads


@pytest.mark.parametrize("name", ["tiny", "colbert", "long_doc", "scattered"])
def test_named_workload_full_parity(name):
    _say(f"[parity] workload {name}")
    w = workloads.make(name)
    got = gpu_scores(w)
    ref = oracle.maxsim_workload(w)
    mx = assert_parity(got, ref, name)
    order = top_k(ref, 10)
    assert top10_ok(got, lambda ids: ref[ids], ref[order]), name
    _say(f"[parity] {name}: B={w.B} tokens={w.doc_tokens} max scaled err {mx:.2e}")


def test_scattered_with_nan_gaps_matches_random_gaps():
    _say("[parity] scattered, NaN gap rows")
    a = gpu_scores(workloads.scattered(gap_fill="nan"))
    b = gpu_scores(workloads.scattered(gap_fill="random"))
    assert np.array_equal(a, b)


@pytest.mark.slow
def test_large_int64_workload_sampled():
    """~20.5 M rows, 5.2 GB: offsets times d pass 2^31. Compared doc by doc on a sample
    (all planted docs, 3000 random ones, and every doc near the GPU's top-10)."""
    _say("[parity] workload large (generating ~5.2 GB)")
    w = workloads.large()
    assert int(w.offsets.max()) * w.d > 2**31
    got = gpu_scores(w)
    rng = np.random.default_rng(0)
    g10 = np.sort(got)[-10]
    band = 2 * 1e-3 * (1 + abs(g10))
    cand = np.nonzero(got >= g10 - band)[0]
    sample = np.unique(np.concatenate([w.planted, rng.choice(w.B, 3000, replace=False), cand,
                                       [0, w.B - 1]]))
    ref = oracle.maxsim_workload(w, docs=sample)
    assert_parity(got[sample], ref, "large (sample)")
    # Every doc that can be in the oracle's top-10 is a candidate (given per-doc parity).
    ref_of = dict(zip(sample.tolist(), ref.tolist()))
    cand_ref = np.array([ref_of[i] for i in cand])
    ref_top = np.sort(cand_ref)[::-1]
    assert len(ref_top) >= 10
    assert top10_ok(got, lambda ids: np.array([ref_of[int(i)] for i in ids]), ref_top)
    planted = np.zeros(w.B, bool)
    planted[w.planted] = True
    assert got[planted].mean() > got[~planted].mean() + 0.5
    _say(f"[parity] large: sample {len(sample)} docs, candidates {len(cand)}")


# ------------------------------------------------------------------ shapes and edges


SHAPES = [
    # (Lq, d, stride)
    (1, 128, 128), (15, 128, 136), (16, 64, 64), (17, 96, 96), (37, 96, 104), (32, 128, 128),
    (128, 128, 128), (129, 128, 128), (200, 128, 136), (256, 256, 256), (64, 256, 264),
    (33, 8, 8), (20, 40, 48), (45, 200, 208), (7, 160, 160), (100, 32, 32), (200, 200, 200),
    (129, 256, 256),
    # 18 query tiles in 3 groups (lq_pad 288: more than 64 four-row cells per slot)
    (256, 160, 160), (250, 136, 136),
]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("Lq,d,stride", SHAPES)
def test_shapes_ragged(fmt, Lq, d, stride):
    _say(f"[parity] shape Lq={Lq} d={d} stride={stride} {fmt}")
    rng = np.random.default_rng([Lq, d, stride])
    lengths = rng.integers(0, 90, size=60)
    lengths[:8] = [0, 1, 15, 16, 17, 31, 32, 33]
    w = workloads.custom(Lq, d, lengths, dtype=fmt, seed=Lq * 7 + d, stride=stride,
                         order="shuffled", gap=(0, 5), gap_fill="nan", pad_fill="nan")
    assert_parity(gpu_scores(w), oracle.maxsim_workload(w), f"Lq={Lq} d={d} {fmt}")


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("Lq,d", [(64, 128), (256, 160)])
def test_long_docs_split_and_tail(fmt, Lq, d):
    _say(f"[parity] long docs Lq={Lq} d={d} {fmt}")
    lengths = np.array([4096, 4095, 1, 2049, 0, 3000, 17, 5000, 16, 8191])
    w = workloads.custom(Lq, d, lengths, dtype=fmt, seed=3, order="shuffled", gap=(1, 3),
                         gap_fill="nan")
    assert_parity(gpu_scores(w), oracle.maxsim_workload(w), "long docs")


def test_query_with_no_rows_and_empty_batch():
    _say("[parity] Lq=0, B=0")
    w = workloads.custom(0, 64, [0, 5, 9], seed=1)
    assert np.array_equal(gpu_scores(w), np.zeros(3))
    w = workloads.custom(8, 64, [3], seed=1)
    Q, X, offs, lens = upload(w)
    out = lir.maxsim_rerank(Q, X, offs[:0], lens[:0])
    assert out.shape == (0,)


def test_overlapping_and_duplicate_docs():
    _say("[parity] overlapping docs")
    w = workloads.custom(32, 128, [100, 50, 70], seed=2)
    offs = np.array([0, 0, 10, 100, 30, 0], np.int32)
    lens = np.array([100, 100, 50, 50, 120, 1], np.int32)
    w.offsets, w.lengths = offs, lens
    got = gpu_scores(w)
    assert got[0] == got[1]
    assert_parity(got, oracle.maxsim_workload(w), "overlap")


def test_last_doc_ends_on_last_row():
    _say("[parity] doc flush with the end of the tensor")
    w = workloads.custom(16, 128, [33, 7, 1, 250], seed=4, order="in_order")
    assert int(w.offsets[-1] + w.lengths[-1]) == w.T
    assert_parity(gpu_scores(w), oracle.maxsim_workload(w), "flush")


# ------------------------------------------------------------------ exact inputs


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("Lq,d", [(32, 128), (37, 96), (128, 128), (5, 40), (200, 64)])
def test_integer_inputs_bitwise(fmt, Lq, d):
    """Entries in [-2, 2]: every product and partial sum is an integer below 2^24, so fp32
    is exact and the GPU must equal the oracle bit for bit."""
    _say(f"[parity] integer inputs Lq={Lq} d={d} {fmt}")
    rng = np.random.default_rng([Lq, d])
    w, _, _ = small_int_case(rng, Lq, d, rng.integers(0, 70, size=80), fmt, gap=(0, 3))
    assert np.array_equal(gpu_scores(w), oracle.maxsim_workload(w))


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("Lq,d", [(32, 128), (37, 96), (64, 256), (17, 8)])
def test_one_hot_layout(fmt, Lq, d):
    """Q[q] = e_a(q), doc rows e_b(t): score = #{q : a(q) hot in the doc}. Pins which lane
    holds which query row and which doc row in the MFMA output."""
    _say(f"[parity] one-hot Lq={Lq} d={d} {fmt}")
    rng = np.random.default_rng([Lq, d, 1])
    w, a, b = one_hot_case(rng, Lq, d, rng.integers(0, 40, size=100), fmt, gap=(0, 2))
    assert np.array_equal(gpu_scores(w), one_hot_expected(Lq, a, b, w.offsets, w.lengths))


# ------------------------------------------------------------------ invariances


def test_token_order_packing_and_doc_order_bitwise():
    _say("[parity] invariances")
    w = workloads.custom(37, 96, np.random.default_rng(9).integers(1, 200, size=300), seed=9,
                         order="shuffled", gap=(1, 20), stride=104)
    base = gpu_scores(w)
    rng = np.random.default_rng(10)
    perm = repack(w, [doc_rows(w, i)[rng.permutation(w.lengths[i])] for i in range(w.B)])
    assert np.array_equal(gpu_scores(perm), base)
    packed = repack(w, [doc_rows(w, i) for i in range(w.B)])
    assert np.array_equal(gpu_scores(packed), base)
    order = rng.permutation(w.B)
    w2 = workloads.Workload(**{**w.__dict__, "offsets": w.offsets[order], "lengths": w.lengths[order]})
    assert np.array_equal(gpu_scores(w2), base[order])


def test_chunking_does_not_change_scores():
    """A long doc scored alone is split into many chunks; among ~2.5 M other rows it gets
    a coarser split. The per-row maxima are exact and the final sum has one fixed order,
    so the score is bitwise the same."""
    _say("[parity] chunking independence")
    long_len = 4000
    alone = workloads.custom(64, 128, [long_len], seed=11)
    many = workloads.custom(64, 128, [long_len] + [256] * 10_000, seed=11)
    assert np.array_equal(alone.X[:long_len], many.X[:long_len])
    a = gpu_scores(alone)[0]
    b = gpu_scores(many)[0]
    assert a == b
    assert_parity([a], oracle.maxsim_workload(alone), "long doc")


def test_combine_mixed_workgroup_and_wave_docs():
    """Split docs with many chunk slots are combined by a whole workgroup, those with few
    by one wave: a batch with both (three docs of 6,000-8,000 rows cut into 256 chunks,
    300 of 65-199 rows cut into 2-8) gets every score within tolerance."""
    _say("[parity] combine: workgroup and wave docs in one launch")
    rng = np.random.default_rng(21)
    lengths = np.concatenate([[8000, 6000, 7777], rng.integers(65, 200, size=300)])
    w = workloads.custom(64, 128, lengths, seed=21, order="shuffled")
    assert_parity(gpu_scores(w), oracle.maxsim_workload(w), "mixed combine")


def test_query_row_permutation_within_tolerance():
    w = workloads.custom(37, 96, np.random.default_rng(12).integers(1, 100, size=100), seed=12)
    base = gpu_scores(w)
    w.Q = w.Q[np.random.default_rng(13).permutation(w.Lq)]
    assert_parity(gpu_scores(w), base, "Q permutation")


# ------------------------------------------------------------------ runtime behaviour


def test_deterministic_and_guards_intact():
    _say("[parity] determinism and guard regions")
    w = workloads.colbert()
    Q, X, offs, lens = upload(w)
    B = w.B
    buf = torch.full((B + 2048,), 12345.0, dtype=torch.float32, device=DEV)
    out = buf[1024 : 1024 + B]
    lir.maxsim_rerank(Q, X, offs, lens, scores=out)
    first = out.clone()
    lir.maxsim_rerank(Q, X, offs, lens, scores=out)
    torch.cuda.synchronize()
    assert torch.equal(first, out)
    assert bool((buf[:1024] == 12345.0).all()) and bool((buf[1024 + B :] == 12345.0).all())


def test_staged_api_matches_one_shot_on_a_side_stream():
    _say("[parity] staged API")
    w = workloads.long_doc()
    Q, X, offs, lens = upload(w)
    ref = lir.rerank(Q, X, offs, lens)
    nbytes = lir.maxsim_workspace_size(w.Lq, w.d, w.B)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lir.maxsim_plan(offs, lens, w.Lq, w.d, ws)
        got = lir.maxsim_score(Q, X, offs, lens, ws)
        lir.maxsim_finish(Q, w.B, ws, got)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


def test_errors_raise():
    w = workloads.custom(8, 64, [3, 4], seed=1)
    Q, X, offs, lens = upload(w)
    with pytest.raises(TypeError):
        lir.maxsim_rerank(Q, X, offs.long(), lens)
    with pytest.raises(TypeError):
        lir.maxsim_rerank_bf16(Q, X, offs, lens)
    big = torch.zeros((4, 264), dtype=torch.float16, device=DEV)
    with pytest.raises(lir.MaxSimError):
        lir.maxsim_rerank(big[:2, :264].contiguous(), big, offs, lens)


def test_graph_replay_tracks_inputs_changed_in_place():
    """The staged form (caller workspace, no allocation) captured once in a HIP graph and
    replayed after Q, offsets and lengths change in place: every replay equals an eager
    run on the same inputs."""
    _say("[parity] graph capture and replay")
    w = workloads.custom(37, 96, np.random.default_rng(30).integers(0, 300, size=500), seed=30,
                         order="shuffled", gap=(1, 9), stride=104)
    Q, X, offs, lens = upload(w)
    B = w.B
    nbytes = lir.maxsim_workspace_size(w.Lq, w.d, B)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    out = torch.empty(B, dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm up (occupancy queries, code loading) before capture
        lir.maxsim_plan(offs, lens, w.Lq, w.d, ws)
        lir.maxsim_score(Q, X, offs, lens, ws, scores=out)
        lir.maxsim_finish(Q, B, ws, out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        lir.maxsim_plan(offs, lens, w.Lq, w.d, ws)
        lir.maxsim_score(Q, X, offs, lens, ws, scores=out)
        lir.maxsim_finish(Q, B, ws, out)
    rng = np.random.default_rng(31)
    for it in range(4):
        if it:
            Q.copy_(Q[torch.from_numpy(rng.permutation(w.Lq)).to(DEV)])
            perm = torch.from_numpy(rng.permutation(B)).to(DEV)
            new_offs, new_lens = offs[perm].clone(), lens[perm].clone()
            new_lens[: B // 4] = torch.clamp(new_lens[: B // 4] // 2, min=0)
            offs.copy_(new_offs)
            lens.copy_(new_lens)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = lir.rerank(Q, X, offs, lens)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {it}"


def test_more_than_a_million_docs():
    """B past 2^20 makes each plan block take several rounds of 1024 docs."""
    _say("[parity] 1.1 M docs")
    B = 1_100_000
    lengths = np.random.default_rng(32).integers(0, 4, size=B)
    w = workloads.custom(4, 32, lengths, seed=32, order="shuffled")
    got = gpu_scores(w)
    sample = np.random.default_rng(33).choice(B, 20000, replace=False)
    sample = np.unique(np.concatenate([sample, [0, B - 1], np.nonzero(lengths == 0)[0][:50]]))
    assert_parity(got[sample], oracle.maxsim_workload(w, docs=sample), "1.1 M docs")
