"""Parity of the one-launch short-doc path (maxsim_rerank_short: one workgroup per doc,
no schedule, no workspace) against the oracle, and bitwise against the scheduled path,
whose max is the same exact max and whose sum runs in the same order."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

if torch.cuda.is_available():
    import late_interaction_reranking_amd as lir
    from devio import assert_parity, top10_ok, top_k, upload, upload8


def _say(msg):
    print(msg, flush=True)


def _both(w):
    Q, X, offs, lens = upload(w)
    short = lir.rerank_short(Q, X, offs, lens)
    sched = lir.rerank(Q, X, offs, lens)
    torch.cuda.synchronize()
    return short.cpu().numpy().astype(np.float64), sched.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("name", ["tiny", "colbert", "long_doc", "scattered"])
def test_named_workloads(name):
    _say(f"[short] workload {name}")
    w = workloads.make(name)
    got, sched = _both(w)
    ref = oracle.maxsim_workload(w)
    assert_parity(got, ref, name)
    assert top10_ok(got, lambda ids: ref[ids], ref[top_k(ref, 10)]), name
    assert np.array_equal(got, sched), name


SHAPES = [
    # (Lq, d, stride): every query fits one register group
    (1, 128, 128), (15, 128, 136), (17, 96, 96), (37, 96, 104), (32, 128, 128), (128, 128, 128),
    (33, 8, 8), (20, 40, 48), (45, 200, 208), (7, 160, 160), (96, 160, 168), (100, 32, 32),
    (64, 256, 264), (128, 64, 64), (16, 64, 64),
]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("Lq,d,stride", SHAPES)
def test_shapes_ragged(fmt, Lq, d, stride):
    _say(f"[short] shape Lq={Lq} d={d} stride={stride} {fmt}")
    rng = np.random.default_rng([Lq, d, stride, 7])
    lengths = rng.integers(0, 150, size=70)
    lengths[:10] = [0, 1, 15, 16, 17, 31, 32, 33, 63, 65]
    w = workloads.custom(Lq, d, lengths, dtype=fmt, seed=Lq * 11 + d, stride=stride, order="shuffled",
                         gap=(0, 5), gap_fill="nan", pad_fill="nan")
    got, sched = _both(w)
    assert_parity(got, oracle.maxsim_workload(w), f"Lq={Lq} d={d} {fmt}")
    assert np.array_equal(got, sched)


def test_long_and_unequal_docs_are_still_exact():
    """A launch lasts as long as its longest doc, but the scores stay exact."""
    _say("[short] long docs")
    lengths = np.array([5000, 1, 0, 2049, 17, 4096, 300])
    w = workloads.custom(64, 128, lengths, seed=8, order="shuffled", gap=(1, 3), gap_fill="nan")
    got, sched = _both(w)
    assert_parity(got, oracle.maxsim_workload(w), "long docs")
    assert np.array_equal(got, sched)


def test_more_docs_than_resident_workgroups():
    """Each workgroup takes docs b, b + grid, ... once the batch exceeds four rounds of
    resident workgroups (a few thousand)."""
    _say("[short] 20,000 docs")
    lengths = np.random.default_rng(12).integers(1, 40, size=20_000)
    w = workloads.custom(32, 128, lengths, seed=12, order="shuffled")
    got, sched = _both(w)
    assert_parity(got, oracle.maxsim_workload(w), "20k docs")
    assert np.array_equal(got, sched)


def test_empty_query_batch_and_unsupported_shapes():
    w = workloads.custom(32, 128, [5, 0, 9], seed=1)
    Q, X, offs, lens = upload(w)
    assert lir.rerank_short(Q[:0], X, offs, lens).cpu().tolist() == [0.0, 0.0, 0.0]
    empty = lir.rerank_short(Q, X, offs[:0], lens[:0])
    assert empty.numel() == 0
    w2 = workloads.custom(129, 128, [5, 9], seed=2)
    Q2, X2, o2, l2 = upload(w2)
    with pytest.raises(lir.MaxSimError):
        lir.rerank_short(Q2, X2, o2, l2)
    torch.cuda.synchronize()


def test_graph_capture_and_replay():
    """No allocation inside: captured once, replayed after the inputs change in place."""
    _say("[short] graph capture")
    w = workloads.custom(32, 128, np.random.default_rng(3).integers(0, 300, size=1000), seed=3,
                         order="shuffled")
    Q, X, offs, lens = upload(w)
    out = torch.empty(w.B, dtype=torch.float32, device=Q.device)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        lir.rerank_short(Q, X, offs, lens, scores=out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        lir.rerank_short(Q, X, offs, lens, scores=out)
    rng = np.random.default_rng(4)
    for it in range(3):
        if it:
            Q.copy_(Q[torch.from_numpy(rng.permutation(w.Lq)).to(Q.device)] * 0.5)
            lens.copy_(torch.clamp(lens - 11 * it, min=0))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = lir.rerank(Q, X, offs, lens)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {it}"


# ------------------------------------------------------------------ FP8 E4M3 docs


def _both8(w):
    Q, X8, offs, lens = upload8(w)
    short = lir.maxsim_rerank_short_fp8(Q, X8, offs, lens, w.doc_scale)
    sched = lir.maxsim_rerank_fp8(Q, X8, offs, lens, w.doc_scale)
    torch.cuda.synchronize()
    return short.cpu().numpy().astype(np.float64), sched.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("name", ["tiny", "colbert", "long_doc", "scattered"])
def test_fp8_named_workloads(name):
    _say(f"[short fp8] workload {name}")
    w = workloads.to_fp8(workloads.make(name), doc_scale=1 / 300)
    got, sched = _both8(w)
    assert_parity(got, oracle.maxsim_workload(w), name)
    assert np.array_equal(got, sched), name


FP8_SHAPES = [
    # (Lq, d, row stride in bytes): one register group, d % 16 == 0
    (1, 128, 128), (32, 16, 16), (7, 32, 48), (37, 48, 64), (32, 128, 128), (128, 128, 144),
    (64, 256, 256), (17, 160, 176), (96, 64, 80), (45, 208, 224),
]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("Lq,d,stride8", FP8_SHAPES)
def test_fp8_shapes_ragged(fmt, Lq, d, stride8):
    _say(f"[short fp8] shape Lq={Lq} d={d} stride={stride8} {fmt}")
    rng = np.random.default_rng([Lq, d, stride8, 9])
    lengths = rng.integers(0, 120, size=60)
    lengths[:10] = [0, 1, 15, 16, 17, 31, 32, 33, 63, 65]
    w = workloads.custom(Lq, d, lengths, dtype=fmt, seed=Lq + 3 * d, order="shuffled", gap=(0, 5),
                         gap_fill="nan")
    workloads.to_fp8(w, doc_scale=0.0123, stride8=stride8)
    got, sched = _both8(w)
    assert_parity(got, oracle.maxsim_workload(w), f"Lq={Lq} d={d} {fmt}")
    assert np.array_equal(got, sched)


FINITE = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], np.uint8)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_fp8_one_hot_every_byte_exact(fmt):
    """One-hot query rows pick single E4M3 values, so every score is exact: equal to the
    oracle's bit for bit (every finite byte appears in some doc row)."""
    _say(f"[short fp8] one-hot all bytes {fmt}")
    rng = np.random.default_rng([5, len(fmt)])
    Lq, d = 6, 64
    lengths = rng.integers(0, 40, size=80)
    lengths[:3] = [0, 1, 17]
    w = workloads.custom(Lq, d, lengths, dtype=fmt, seed=5, order="shuffled", gap=(0, 3), gap_fill="nan")
    workloads.to_fp8(w, doc_scale=1.0, stride8=d + 16)
    for o_, n in zip(w.offsets, w.lengths):
        w.X8[o_:o_ + n, :d] = rng.choice(FINITE, size=(n, d))
    o0 = int(w.offsets[np.argmax(w.lengths)])
    flat = w.X8[o0:o0 + int(w.lengths.max()), :d].reshape(-1)
    flat[: FINITE.size] = FINITE
    w.X8[o0:o0 + int(w.lengths.max()), :d] = flat.reshape(-1, d)
    a = rng.integers(0, d, size=Lq)
    w.Q = np.zeros((Lq, d), np.uint16)
    w.Q[np.arange(Lq), a] = 0x3C00 if fmt == "f16" else 0x3F80
    got, sched = _both8(w)
    assert np.array_equal(got, oracle.maxsim_workload(w))
    assert np.array_equal(got, sched)


def test_fp8_errors_and_empty():
    w = workloads.to_fp8(workloads.custom(32, 128, [5, 0, 9], seed=1), doc_scale=0.5)
    Q, X8, offs, lens = upload8(w)
    assert lir.maxsim_rerank_short_fp8(Q[:0], X8, offs, lens, 0.5).cpu().tolist() == [0.0, 0.0, 0.0]
    assert lir.maxsim_rerank_short_fp8(Q, X8, offs[:0], lens[:0], 0.5).numel() == 0
    with pytest.raises(lir.MaxSimError):
        lir.maxsim_rerank_short_fp8(Q, X8, offs, lens, 0.0)
    Q129 = torch.zeros((129, 128), dtype=torch.float16, device=Q.device)
    with pytest.raises(lir.MaxSimError):
        lir.maxsim_rerank_short_fp8(Q129, X8, offs, lens, 0.5)
    with pytest.raises(TypeError):
        lir.maxsim_rerank_short_fp8(Q, X8.to(torch.float16), offs, lens, 0.5)
    torch.cuda.synchronize()


@pytest.mark.slow
def test_fp8_large_sampled():
    """The FP8 rerank workload at full size (80,000 docs of 64 to 448 rows, offsets past
    2**31 bytes) in one launch."""
    _say("[short fp8] large_fp8 (generating)")
    w = workloads.make("large_fp8")
    got, sched = _both8(w)
    assert np.array_equal(got, sched)
    rng = np.random.default_rng(1)
    sample = np.unique(np.concatenate([w.planted, rng.choice(w.B, 2000, replace=False), [0, w.B - 1]]))
    assert_parity(got[sample], oracle.maxsim_workload(w, docs=sample), "large_fp8 (sample)")
