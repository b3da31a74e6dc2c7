"""The self-scheduling range path that maxsim_rerank takes for a single query of at most
8192 docs (one register group of query tiles): oracle parity within the tolerance, and
bit-for-bit equality with the scheduled path (plan, score, combine on a caller
workspace), which splits docs differently. Batches with empty docs, one-row docs, docs
far longer than a wave's share, runs of empty docs longer than a 64-doc window, every
query width up to 128 rows, bf16 and FP8 docs, prologue blocks of 1 to 32 docs per
thread, and the 8192/8193-doc boundary."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

if torch.cuda.is_available():
    import late_interaction_reranking_amd as lir
    from devio import DEV, assert_parity, upload, upload8


def _say(msg):
    print(msg, flush=True)


def staged(Q, X, offs, lens):
    """The scheduled path on a fresh caller workspace."""
    B = int(offs.shape[0])
    ws = torch.empty(lir.maxsim_workspace_size(Q.shape[0], Q.shape[1], B), dtype=torch.uint8, device=DEV)
    lir.maxsim_plan(offs, lens, Q.shape[0], Q.shape[1], ws)
    out = lir.maxsim_score(Q, X, offs, lens, ws)
    lir.maxsim_finish(Q, B, ws, out)
    return out


def staged8(Q, X8, offs, lens, scale):
    B = int(offs.shape[0])
    ws = torch.empty(lir.maxsim_workspace_size(Q.shape[0], Q.shape[1], B), dtype=torch.uint8, device=DEV)
    lir.maxsim_plan(offs, lens, Q.shape[0], Q.shape[1], ws)
    out = lir.maxsim_score_fp8(Q, X8, offs, lens, scale, ws)
    lir.maxsim_finish_fp8(Q, B, scale, ws, out)
    return out


def check(w, what):
    U = upload(w)
    got = lir.rerank(*U)
    ref_staged = staged(*U)
    torch.cuda.synchronize()
    g = got.cpu().numpy().astype(np.float64)
    assert_parity(g, oracle.maxsim_workload(w), what)
    assert torch.equal(got, ref_staged), f"{what}: range path differs from the scheduled path"


LENGTH_LAWS = {
    "short": lambda r, B: r.integers(0, 40, size=B),
    "colbert": lambda r, B: r.integers(64, 301, size=B),
    "lognormal": lambda r, B: np.clip(np.rint(np.exp(r.normal(np.log(1024), 0.6, size=B))), 32, 4096),
    "sparse_long": lambda r, B: np.where(r.random(B) < 0.9, 0, r.integers(1, 9000, size=B)),
    "ones": lambda r, B: np.ones(B, np.int64),
}


# Every law up to 1024 docs (one 4-doc chunk per prologue thread); above that (2 to 8
# chunks, offsets in LDS or, where they do not fit, from global memory) the laws whose
# batches stay a few million rows.
LAW_CASES = [(law, B) for law in sorted(LENGTH_LAWS) for B in (1, 7, 300, 1024)] + [
    (law, B) for law in ("colbert", "ones", "short", "sparse_long") for B in (1025, 3000, 5000, 8192)]


@pytest.mark.parametrize("law,B", LAW_CASES)
def test_length_laws(law, B):
    _say(f"[range] {law} B={B}")
    r = np.random.default_rng(hash((law, B)) % 2**32)
    w = workloads.custom(32, 128, LENGTH_LAWS[law](r, B), seed=B + 3, order="shuffled", gap=(0, 3),
                         gap_fill="nan")
    check(w, f"{law} B={B}")


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("Lq,d,stride", [(1, 8, 8), (16, 32, 40), (17, 64, 64), (37, 96, 104), (48, 128, 128),
                                         (100, 128, 136), (128, 128, 128), (64, 256, 264), (5, 160, 160)])
def test_query_and_row_shapes(fmt, Lq, d, stride):
    _say(f"[range] {fmt} Lq={Lq} d={d} stride={stride}")
    r = np.random.default_rng(Lq * 131 + d)
    lens = np.concatenate([r.integers(0, 200, size=500), [0, 1, 15, 16, 17, 4000, 0]])
    w = workloads.custom(Lq, d, lens, dtype=fmt, seed=Lq + d, order="shuffled", stride=stride, gap=(1, 4),
                         gap_fill="nan")
    check(w, f"{fmt} Lq={Lq} d={d}")


def test_runs_of_empty_docs_beyond_a_window():
    """Non-empty docs hundreds of indices apart: each wave's walk to the next doc with a
    tile crosses several 64-doc windows."""
    _say("[range] long runs of empty docs")
    lens = np.zeros(1024, np.int64)
    lens[[0, 3, 200, 201, 450, 777, 1023]] = [70, 5, 3000, 1, 900, 33, 260]
    w = workloads.custom(32, 128, lens, seed=9, order="shuffled", gap=(1, 3))
    check(w, "empty runs")
    lens2 = np.zeros(1000, np.int64)
    lens2[999] = 50
    check(workloads.custom(32, 128, lens2, seed=10), "one doc at the end")
    # (a few unrelated rows, so that the doc tensor itself is not empty)
    check(workloads.custom(32, 128, np.zeros(64, np.int64), seed=11, trailing_gap=5), "all empty")


def test_boundary_at_8192_docs():
    _say("[range] 8192 and 8193 docs")
    r = np.random.default_rng(12)
    lens = r.integers(0, 200, size=8193)
    w_in = workloads.custom(32, 128, lens[:8192], seed=12, order="shuffled")
    w_out = workloads.custom(32, 128, lens, seed=12, order="shuffled")
    check(w_in, "8192 docs (range path)")
    check(w_out, "8193 docs (scheduled path)")


def test_named_small_workloads_bitwise_with_the_scheduled_path():
    for name in ("tiny", "colbert", "long_doc", "scattered"):
        _say(f"[range] {name}")
        check(workloads.make(name), name)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_fp8_docs(fmt):
    _say(f"[range] FP8 docs, {fmt} query")
    r = np.random.default_rng(13)
    w = workloads.to_fp8(workloads.custom(32, 128, np.concatenate([r.integers(0, 700, size=900), [0, 1, 5000]]),
                                          dtype=fmt, seed=13, order="shuffled"), doc_scale=0.01)
    Q, X8, offs, lens = upload8(w)
    got = lir.maxsim_rerank_fp8(Q, X8, offs, lens, w.doc_scale)
    ref = staged8(Q, X8, offs, lens, w.doc_scale)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    assert_parity(got.cpu().numpy().astype(np.float64), oracle.maxsim_workload(w), "fp8 range")


def test_topk_on_the_range_path():
    _say("[range] top-k")
    r = np.random.default_rng(14)
    w = workloads.custom(32, 128, r.integers(0, 400, size=800), seed=14, order="shuffled")
    U = upload(w)
    ts, ti = lir.maxsim_rerank_topk(*U, 37)
    rs, ri = lir.maxsim_topk(staged(*U), 37)
    torch.cuda.synchronize()
    assert torch.equal(ts, rs) and torch.equal(ti, ri)


def test_repeated_calls_and_streams_are_deterministic():
    _say("[range] repeated calls on two streams")
    r = np.random.default_rng(15)
    w = workloads.custom(32, 128, r.integers(0, 2000, size=700), seed=15, order="shuffled")
    U = upload(w)
    ref = staged(*U)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(5):
        for s in (s1, s2):
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                outs.append(lir.rerank(*U))
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, ref)


def test_rows_past_the_32_bit_byte_offsets():
    """Docs placed from row 2^24 + 5 of a zero-filled 4.3 GB device tensor (row offset
    times 256 bytes passes 2^32): the range kernel forms its addresses in 64 bits. The
    oracle scores the same rows at their original offsets (scores do not depend on where
    the rows sit)."""
    _say("[range] rows past 2^32 bytes")
    w = workloads.custom(32, 128, np.random.default_rng(13).integers(0, 300, size=600), seed=13,
                         order="shuffled", gap=(1, 5))
    Q, X, offs, lens = upload(w)
    base = (1 << 24) + 5
    big = torch.zeros((base + X.shape[0], 128), dtype=X.dtype, device=DEV)
    big[base:] = X
    far = offs + base
    assert int(far.max()) * 128 * 2 > 2 ** 32
    got = lir.rerank(Q, big, far, lens)
    ref_staged = staged(Q, big, far, lens)
    torch.cuda.synchronize()
    assert_parity(got.cpu().numpy().astype(np.float64), oracle.maxsim_workload(w), "far rows")
    assert torch.equal(got, ref_staged), "far rows: range path differs from the scheduled path"
    del big
    torch.cuda.empty_cache()
