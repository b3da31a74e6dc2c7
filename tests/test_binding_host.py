"""Host-side checks of the Python binding (no GPU): a caller-supplied score tensor or
workspace on the wrong device is refused before any call into the library, since the
kernels would store through its pointer."""

from __future__ import annotations

import ast
import inspect

import pytest
import torch

from late_interaction_reranking_amd import maxsim


def test_scores_out_refuses_the_host_and_other_gpus():
    gpu0 = torch.device("cuda:0")
    with pytest.raises(ValueError, match="must live on cuda:0"):
        maxsim._scores_out(torch.empty(5, dtype=torch.float32), (5,), gpu0)
    with pytest.raises(ValueError, match="must live on cuda:1"):
        maxsim._scores_out(torch.empty(5, dtype=torch.float32), (5,), torch.device("cuda:1"))
    with pytest.raises(ValueError, match="contiguous float32"):
        maxsim._scores_out(torch.empty(5, dtype=torch.float64), (5,), gpu0)
    with pytest.raises(ValueError, match="contiguous float32"):
        maxsim._scores_out(torch.empty(6, dtype=torch.float32), (5,), gpu0)
    with pytest.raises(ValueError, match="contiguous float32"):
        maxsim._scores_out(torch.empty((5, 2), dtype=torch.float32).t(), (2, 5), gpu0)
    cpu = torch.empty(3, dtype=torch.float32)
    assert maxsim._scores_out(cpu, (3,), torch.device("cpu")) is cpu


def test_workspace_on_another_device_is_refused():
    ws = torch.empty(256, dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU tensor"):
        maxsim._ws(ws)
    with pytest.raises(ValueError, match="GPU tensor"):
        maxsim._ws(ws, torch.device("cuda:0"))


def test_every_scores_argument_goes_through_the_check():
    """Every public wrapper that takes `scores` either checks it with _scores_out or
    hands it to another wrapper that does."""
    checked = set()
    pending = {}
    for name in maxsim.__all__:
        fn = getattr(maxsim, name, None)
        if not callable(fn) or not hasattr(fn, "__code__"):
            continue
        if "scores" not in inspect.signature(fn).parameters or name == "maxsim_topk":
            continue  # (maxsim_topk only reads its scores, a GPU tensor it checks)
        src = inspect.getsource(fn)
        # names the body refers to (a wrapper may pick the function it calls first)
        calls = {n.id for n in ast.walk(ast.parse(src.lstrip())) if isinstance(n, ast.Name)}
        if "_scores_out" in calls:
            checked.add(name)
        else:
            pending[name] = calls
    helpers = {"_rerank", "_rerank_pairs", "_rerank_multi"}
    for h in helpers:
        src = inspect.getsource(getattr(maxsim, h))
        assert "_scores_out(" in src, h
    ok = checked | helpers
    changed = True
    while changed:
        changed = False
        for name, calls in list(pending.items()):
            if calls & ok:
                ok.add(name)
                del pending[name]
                changed = True
    assert not pending, f"wrappers passing `scores` on unchecked: {sorted(pending)}"
