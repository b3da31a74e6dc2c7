"""Concurrency and capture on the GPU: reranks running at the same time on two streams
give the same bits as run alone, and the one-shot entry points (which allocate their
workspace stream-ordered) captured in a HIP graph and replayed after their inputs change
in place give the same bits as eager calls on the same inputs, replay after replay."""

from __future__ import annotations

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

if torch.cuda.is_available():
    import late_interaction_reranking_amd as lir
    from devio import DEV, upload


def _say(msg):
    print(msg, flush=True)


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def test_two_streams_at_once():
    _say("[streams] two streams")
    wa = workloads.custom(32, 128, np.random.default_rng(1).integers(1, 400, size=3000), seed=1, order="shuffled")
    wb = workloads.custom(37, 96, np.random.default_rng(2).integers(1, 3000, size=300), seed=2, dtype="bf16",
                          order="shuffled", gap=(1, 5), stride=104)
    A, B = upload(wa), upload(wb)
    ref_a = lir.rerank(*A)
    ref_b = lir.rerank(*B)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(6):
        with torch.cuda.stream(s1):
            oa = lir.rerank(*A)
        with torch.cuda.stream(s2):
            ob = lir.rerank(*B)
        outs.append((oa, ob))
    torch.cuda.synchronize()
    for oa, ob in outs:
        assert torch.equal(oa, ref_a) and torch.equal(ob, ref_b)


def _capture(fn, s):
    with torch.cuda.stream(s):  # warm up before capture (occupancy queries, code loading)
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    return g


def _replays(g, change, eager, out, n=3):
    for it in range(n):
        if it:
            change(it)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = eager()
        torch.cuda.synchronize()
        got = out() if callable(out) else out
        if isinstance(ref, tuple):
            for a, b in zip(got, ref):
                assert torch.equal(a, b), f"replay {it}"
        else:
            assert torch.equal(got, ref), f"replay {it}"


def test_graph_one_shot_rerank_and_topk():
    _say("[graph] one-shot rerank + top-k")
    w = workloads.custom(32, 128, np.random.default_rng(3).integers(0, 500, size=2000), seed=3, order="shuffled")
    Q, X, offs, lens = upload(w)
    out = torch.empty(w.B, dtype=torch.float32, device=DEV)
    holder = {}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())

    def fn():
        lir.rerank(Q, X, offs, lens, scores=out)
        holder["tk"] = lir.maxsim_rerank_topk(Q, X, offs, lens, 50)

    g = _capture(fn, s)
    rng = np.random.default_rng(4)

    def change(it):
        Q.copy_(Q[torch.from_numpy(rng.permutation(w.Lq)).to(DEV)] * 0.5)
        lens.copy_(torch.clamp(lens - it * 7, min=0))

    _replays(g, change, lambda: lir.rerank(Q, X, offs, lens), out)
    _replays(g, change, lambda: lir.maxsim_rerank_topk(Q, X, offs, lens, 50), lambda: holder["tk"])


def test_graph_pairs_multi_fp8():
    _say("[graph] pairs, shared docs, FP8 docs")
    rng = np.random.default_rng(5)
    wp = workloads.custom_pairs([16, 32, 8], 64, [200, 100, 150], rng.integers(1, 300, size=450), seed=5,
                                interleave=True)
    Qp, Xp, offp, lenp = upload(wp)
    qo, ql, dq = _i32(wp.q_offsets), _i32(wp.q_lengths), _i32(wp.doc_query)
    wm = workloads.custom_multi([32, 32, 32, 32, 16], 128, rng.integers(1, 400, size=600), seed=6)
    Qm, Xm, offm, lenm = upload(wm)
    wf = workloads.to_fp8(workloads.custom(32, 128, rng.integers(1, 400, size=700), seed=7), doc_scale=0.01)
    Qf = torch.from_numpy(wf.Q.view(np.int16)).to(DEV).view(torch.float16)
    Xf = torch.from_numpy(wf.X8).to(DEV)[:, : wf.d]
    offf, lenf = _i32(wf.offsets), _i32(wf.lengths)
    op = torch.empty(wp.B, dtype=torch.float32, device=DEV)
    om = torch.empty((wm.nq, wm.B), dtype=torch.float32, device=DEV)
    of = torch.empty(wf.B, dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())

    def fn():
        lir.rerank_pairs(Qp, qo, ql, wp.Lq, Xp, offp, lenp, dq, scores=op)
        lir.rerank_multi(Qm, wm.q_lengths, Xm, offm, lenm, scores=om)
        lir.maxsim_rerank_fp8(Qf, Xf, offf, lenf, wf.doc_scale, scores=of)

    g = _capture(fn, s)

    def change(it):
        dq.copy_(dq[torch.from_numpy(rng.permutation(wp.B)).to(DEV)])
        lenm.copy_(torch.clamp(lenm - 5 * it, min=0))
        Qf.mul_(-1.0)

    def eager():
        return (lir.rerank_pairs(Qp, qo, ql, wp.Lq, Xp, offp, lenp, dq),
                lir.rerank_multi(Qm, wm.q_lengths, Xm, offm, lenm),
                lir.maxsim_rerank_fp8(Qf, Xf, offf, lenf, wf.doc_scale))

    _replays(g, change, eager, (op, om, of))


def _staged(Q, X, offs, lens):
    """Scores from the staged path on a fresh caller workspace (no library cache)."""
    B = int(offs.shape[0])
    ws = torch.empty(lir.maxsim_workspace_size(Q.shape[0], Q.shape[1], B), dtype=torch.uint8, device=DEV)
    lir.maxsim_plan(offs, lens, Q.shape[0], Q.shape[1], ws)
    out = lir.maxsim_score(Q, X, offs, lens, ws)
    lir.maxsim_finish(Q, B, ws, out)
    return out


def test_one_shot_workspace_cache_reuse_growth_eviction():
    """The one-shot entry points keep a workspace per stream: batches that grow and
    shrink on one stream with no synchronisation between calls, then more streams than
    the library keeps workspaces for (so workspaces are evicted and freed while other
    streams run), every result bitwise the staged path's on its own workspace."""
    _say("[streams] one-shot workspace cache")
    rng = np.random.default_rng(11)
    shapes = [(300, 500), (3000, 2000), (50, 40), (1000, 9000), (200, 100), (4000, 300)]
    ws = [workloads.custom(32, 128, rng.integers(0, n, size=b), seed=20 + i, order="shuffled")
          for i, (n, b) in enumerate(shapes)]
    ups = [upload(w) for w in ws]
    refs = [_staged(*u) for u in ups]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    outs = []
    with torch.cuda.stream(s):
        for _ in range(3):
            for k, u in enumerate(ups):
                outs.append((k, lir.rerank(*u)))
    torch.cuda.synchronize()
    for k, o in outs:
        assert torch.equal(o, refs[k]), f"same stream, batch {k}"
    streams = [torch.cuda.Stream() for _ in range(21)]
    outs = []
    for rep in range(3):
        for j, st in enumerate(streams):
            st.wait_stream(torch.cuda.current_stream())
            k = (j + rep) % len(ups)
            with torch.cuda.stream(st):
                outs.append((k, lir.rerank(*ups[k])))
                outs.append((-1 - k, lir.maxsim_rerank_topk(*ups[k], 20)))
    torch.cuda.synchronize()
    for k, o in outs:
        if k >= 0:
            assert torch.equal(o, refs[k]), f"many streams, batch {k}"
        else:
            ref_s, ref_i = lir.maxsim_topk(refs[-1 - k], 20)
            assert torch.equal(o[0], ref_s) and torch.equal(o[1], ref_i), f"top-k, batch {-1 - k}"


def test_eager_calls_after_a_captured_one_shot_on_the_same_stream():
    """A graph captured on a stream that already holds a cached workspace refers only to
    its own graph memory: eager calls on that stream between replays, with other inputs,
    leave the replays' results intact, and the replays leave theirs."""
    _say("[graph] captured one-shot next to eager calls on the same stream")
    rng = np.random.default_rng(12)
    wa = workloads.custom(32, 128, rng.integers(0, 700, size=1500), seed=30, order="shuffled")
    wb = workloads.custom(32, 128, rng.integers(0, 2500, size=600), seed=31, order="shuffled")
    A, Bw = upload(wa), upload(wb)
    ref_a, ref_b = _staged(*A), _staged(*Bw)
    out = torch.empty(wa.B, dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = _capture(lambda: lir.rerank(*A, scores=out), s)
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            eb = lir.rerank(*Bw)
            g.replay()
            eb2 = lir.rerank(*Bw)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_a)
        assert torch.equal(eb, ref_b) and torch.equal(eb2, ref_b)
