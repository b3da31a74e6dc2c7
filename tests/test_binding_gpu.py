"""The binding refuses output tensors on the wrong device before the library is called:
a score tensor in host memory passed to any GPU entry would be stored through as if it
were device memory."""

from __future__ import annotations

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

if torch.cuda.is_available():
    import late_interaction_reranking_amd as lir
    from devio import DEV, upload, upload8


def test_host_scores_and_workspace_are_refused():
    print("[binding] host tensors refused", flush=True)
    w = workloads.custom(32, 128, [5, 9, 0, 40], seed=1)
    Q, X, offs, lens = upload(w)
    B = w.B
    host = torch.empty(B, dtype=torch.float32)
    ws = torch.empty(lir.maxsim_workspace_size(w.Lq, w.d, B), dtype=torch.uint8, device=DEV)
    ws_host = torch.empty(ws.numel(), dtype=torch.uint8)
    qo = torch.zeros(1, dtype=torch.int32, device=DEV)
    ql = torch.full((1,), w.Lq, dtype=torch.int32, device=DEV)
    dq = torch.zeros(B, dtype=torch.int32, device=DEV)
    w8 = workloads.to_fp8(workloads.custom(32, 128, [5, 9, 0, 40], seed=1))
    Q8, X8, offs8, lens8 = upload8(w8)
    calls = [
        lambda: lir.rerank(Q, X, offs, lens, scores=host),
        lambda: lir.maxsim_rerank_short(Q, X, offs, lens, scores=host),
        lambda: lir.maxsim_score(Q, X, offs, lens, ws, scores=host),
        lambda: lir.maxsim_finish(Q, B, ws, host),
        lambda: lir.rerank_pairs(Q, qo, ql, w.Lq, X, offs, lens, dq, scores=host),
        lambda: lir.rerank_multi(Q, [w.Lq], X, offs, lens, scores=host.view(1, B)),
        lambda: lir.maxsim_rerank_fp8(Q8, X8, offs8, lens8, w8.doc_scale, scores=host),
        lambda: lir.maxsim_rerank_short_fp8(Q8, X8, offs8, lens8, w8.doc_scale, scores=host),
        lambda: lir.maxsim_rerank_pairs_fp8(Q8, qo, ql, w.Lq, X8, offs8, lens8, dq, w8.doc_scale, scores=host),
        lambda: lir.maxsim_rerank_multi_fp8(Q8, [w.Lq], X8, offs8, lens8, w8.doc_scale, scores=host.view(1, B)),
        lambda: lir.maxsim_score(Q, X, offs, lens, ws_host),
        lambda: lir.maxsim_plan(offs, lens, w.Lq, w.d, ws_host),
    ]
    for i, c in enumerate(calls):
        with pytest.raises(ValueError):
            c()
    torch.cuda.synchronize()
    good = lir.rerank(Q, X, offs, lens)
    torch.cuda.synchronize()
    assert np.isneginf(good[2].item())
