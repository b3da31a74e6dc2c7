"""The C-ABI library without a GPU: it loads, exports every declared symbol, and rejects
bad arguments on the host before any HIP call."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

import late_interaction_reranking_amd as lir

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "maxsim.h")

OK, INVALID, UNSUPPORTED, HIP, WORKSPACE = 0, 1, 2, 3, 4


def declared_functions() -> list[str]:
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"MAXSIM_API\s+[\w\s\*]*?\b(maxsim_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return lir.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("maxsim_rerank", "maxsim_rerank_bf16", "maxsim_status_string",
              "maxsim_workspace_size", "maxsim_plan", "maxsim_score", "maxsim_finish",
              "maxsim_version", "maxsim_rerank_pairs", "maxsim_rerank_pairs_bf16",
              "maxsim_plan_pairs", "maxsim_rerank_multi", "maxsim_rerank_multi_bf16",
              "maxsim_rerank_fp8", "maxsim_rerank_fp8_bf16", "maxsim_score_fp8", "maxsim_finish_fp8",
              "maxsim_topk_workspace_size", "maxsim_topk", "maxsim_rerank_topk", "maxsim_rerank_topk_bf16",
              "maxsim_rerank_pairs_fp8", "maxsim_rerank_multi_fp8", "maxsim_rerank_short",
              "maxsim_rerank_noalloc",
              "maxsim_rerank_short_fp8"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_only_declared_symbols_are_exported():
    import subprocess

    out = subprocess.run(["nm", "-D", "--defined-only", lir.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = sorted({ln.split()[-1] for ln in out.splitlines() if " T " in ln})
    assert exported == declared_functions()


def test_status_strings(lib):
    for code in (OK, INVALID, UNSUPPORTED, HIP, WORKSPACE, 99, -1):
        s = lir.maxsim_status_string(code)
        assert isinstance(s, str) and s
    assert lir.maxsim_status_string(99) == "unknown status"
    assert lir.maxsim_version() == 100


FAKE = 0x7F0000000000  # 256-byte aligned stand-in for a device address; never dereferenced


def call(lib, fn="maxsim_rerank", Q=FAKE, Lq=32, d=128, docs=FAKE, stride=128, offs=FAKE,
         lens=FAKE + 1024, B=10, scores=FAKE + 4096):
    return getattr(lib, fn)(Q, Lq, d, docs, stride, offs, lens, B, scores, None)


@pytest.mark.parametrize("fn", ["maxsim_rerank", "maxsim_rerank_bf16"])
@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), INVALID),
    (dict(Lq=-1), INVALID),
    (dict(d=0), INVALID),
    (dict(stride=64), INVALID),          # stride < d
    (dict(docs=None), INVALID),
    (dict(offs=None), INVALID),
    (dict(lens=None), INVALID),
    (dict(scores=None), INVALID),
    (dict(Q=None), INVALID),
    (dict(d=12, stride=16), UNSUPPORTED),   # d % 8
    (dict(d=264, stride=264), UNSUPPORTED),  # d > 256
    (dict(Lq=257), UNSUPPORTED),
    (dict(stride=132), UNSUPPORTED),         # stride % 8
    (dict(stride=(1 << 24) + 8), UNSUPPORTED),
    (dict(docs=FAKE + 8), UNSUPPORTED),      # docs not 16-byte aligned
    (dict(Q=FAKE + 4), UNSUPPORTED),         # Q not 16-byte aligned
    (dict(offs=FAKE + 2), INVALID),          # int32 arrays not 4-byte aligned
    (dict(scores=FAKE + 2), INVALID),
    (dict(B=0, docs=None, offs=None, lens=None, scores=None), OK),  # nothing to do
])
def test_host_validation(lib, fn, kw, code):
    assert call(lib, fn, **kw) == code


def call_short(lib, dtype=0, **kw):
    args = dict(Q=FAKE, Lq=32, d=128, docs=FAKE, stride=128, offs=FAKE, lens=FAKE + 1024, B=10,
                scores=FAKE + 4096)
    args.update(kw)
    return lib.maxsim_rerank_short(dtype, args["Q"], args["Lq"], args["d"], args["docs"], args["stride"],
                                   args["offs"], args["lens"], args["B"], args["scores"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), INVALID),
    (dict(dtype=-1), INVALID),
    (dict(B=-1), INVALID),
    (dict(stride=64), INVALID),
    (dict(scores=None), INVALID),
    (dict(d=12, stride=16), UNSUPPORTED),
    (dict(Lq=257), UNSUPPORTED),
    (dict(Q=FAKE + 4), UNSUPPORTED),
    # more than one register group of query tiles
    (dict(Lq=129, d=128), UNSUPPORTED),
    (dict(Lq=65, d=256, stride=256), UNSUPPORTED),
    (dict(Lq=97, d=160, stride=160), UNSUPPORTED),   # 7 query tiles of 5 K-steps: 35 > 32
    (dict(Lq=129, d=128, B=0), UNSUPPORTED),         # the envelope is checked before B
    (dict(B=0, docs=None, offs=None, lens=None, scores=None), OK),
    (dict(dtype=1, B=0, docs=None, offs=None, lens=None, scores=None), OK),
])
def test_short_validation(lib, kw, code):
    assert call_short(lib, **kw) == code


def call_noalloc(lib, dtype=0, **kw):
    args = dict(Q=FAKE, Lq=32, d=128, docs=FAKE, stride=128, offs=FAKE, lens=FAKE + 1024, B=10,
                scores=FAKE + 4096)
    args.update(kw)
    return lib.maxsim_rerank_noalloc(dtype, args["Q"], args["Lq"], args["d"], args["docs"], args["stride"],
                                     args["offs"], args["lens"], args["B"], args["scores"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), INVALID),
    (dict(dtype=-1), INVALID),
    (dict(B=-1), INVALID),
    (dict(Lq=-1), INVALID),
    (dict(stride=64), INVALID),
    (dict(scores=None), INVALID),
    (dict(docs=None), INVALID),
    (dict(offs=FAKE + 2), INVALID),
    (dict(d=12, stride=16), UNSUPPORTED),
    (dict(Lq=257), UNSUPPORTED),
    (dict(Q=FAKE + 4), UNSUPPORTED),
    (dict(stride=(1 << 24) + 8), UNSUPPORTED),
    (dict(B=0, docs=None, offs=None, lens=None, scores=None), OK),
    (dict(dtype=1, B=0, docs=None, offs=None, lens=None, scores=None), OK),
])
def test_noalloc_validation(lib, kw, code):
    """maxsim_rerank_noalloc checks its arguments on the host, as maxsim_rerank does,
    before it touches the GPU or its scratch."""
    assert call_noalloc(lib, **kw) == code


def test_scratch_status_string(lib):
    assert "64 MiB" in lir.maxsim_status_string(5)


def call_short_fp8(lib, dtype=0, scale=1.0, **kw):
    args = dict(Q=FAKE, Lq=32, d=128, docs=FAKE, stride=128, offs=FAKE, lens=FAKE + 1024, B=10,
                scores=FAKE + 4096)
    args.update(kw)
    fn = lib.maxsim_rerank_short_fp8
    fn.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                   ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_float,
                   ctypes.c_void_p, ctypes.c_void_p]
    return fn(dtype, args["Q"], args["Lq"], args["d"], args["docs"], args["stride"], args["offs"],
              args["lens"], args["B"], scale, args["scores"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), INVALID),                        # a format flag is not a query format
    (dict(dtype=3), INVALID),
    (dict(scale=0.0), INVALID),
    (dict(scale=-1.0), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(scale=float("inf")), INVALID),
    (dict(d=24, stride=32), UNSUPPORTED),            # d % 16
    (dict(stride=136), UNSUPPORTED),                 # stride % 16 (bytes)
    (dict(Lq=129, d=128), UNSUPPORTED),              # more than one register group
    (dict(B=-1), INVALID),
    (dict(docs=None), INVALID),
    (dict(B=0, docs=None, offs=None, lens=None, scores=None), OK),
    (dict(dtype=1, B=0, docs=None, offs=None, lens=None, scores=None), OK),
])
def test_short_fp8_validation(lib, kw, code):
    assert call_short_fp8(lib, **kw) == code


def test_staged_validation(lib):
    P = ctypes.c_void_p
    # unknown element format
    assert lib.maxsim_score(7, FAKE, 32, 128, FAKE, 128, FAKE, FAKE, 4, FAKE, FAKE, 1 << 20, None) == INVALID
    # workspace missing / misaligned (checked before the device is touched)
    assert lib.maxsim_score(0, FAKE, 32, 128, FAKE, 128, FAKE, FAKE, 4, FAKE, None, 1 << 20, None) == WORKSPACE
    assert lib.maxsim_score(0, FAKE, 32, 128, FAKE, 128, FAKE, FAKE, 4, FAKE, FAKE + 16, 1 << 20, None) == WORKSPACE
    assert lib.maxsim_plan(FAKE, FAKE, 4, 32, 128, None, 1 << 20, None) == WORKSPACE
    assert lib.maxsim_plan(FAKE, FAKE, 4, 32, 128, FAKE + 64, 1 << 20, None) == WORKSPACE
    assert lib.maxsim_plan(None, FAKE, 4, 32, 128, FAKE, 1 << 20, None) == INVALID
    assert lib.maxsim_plan(FAKE, FAKE, -2, 32, 128, FAKE, 1 << 20, None) == INVALID
    assert lib.maxsim_plan(FAKE, FAKE, 4, 32, 100, FAKE, 1 << 20, None) == UNSUPPORTED
    assert lib.maxsim_plan(FAKE, FAKE, 0, 32, 128, None, 0, None) == OK
    assert lib.maxsim_finish(5, 32, 128, 4, FAKE, FAKE, 1 << 20, None) == INVALID
    assert lib.maxsim_finish(0, 32, 128, -4, FAKE, FAKE, 1 << 20, None) == INVALID
    assert lib.maxsim_finish(0, 32, 128, 4, None, FAKE, 1 << 20, None) == INVALID
    assert lib.maxsim_finish(0, 32, 100, 4, FAKE, FAKE, 1 << 20, None) == UNSUPPORTED
    assert lib.maxsim_finish(0, 32, 128, 4, FAKE, None, 1 << 20, None) == WORKSPACE
    assert lib.maxsim_finish(0, 32, 128, 0, None, None, 0, None) == OK
    n = ctypes.c_size_t(0)
    assert lib.maxsim_workspace_size(32, 128, -1, ctypes.byref(n)) == INVALID
    assert lib.maxsim_workspace_size(32, 128, 10, None) == INVALID
    assert lib.maxsim_workspace_size(32, 100, 10, ctypes.byref(n)) == UNSUPPORTED
    del P


def call_pairs(lib, fn="maxsim_rerank_pairs", Qs=FAKE, q_rows=64, d=128, qo=FAKE + 8192,
               ql=FAKE + 12288, nq=4, max_lq=32, docs=FAKE, stride=128, offs=FAKE,
               lens=FAKE + 1024, dq=FAKE + 16384, B=10, scores=FAKE + 4096):
    return getattr(lib, fn)(Qs, q_rows, d, qo, ql, nq, max_lq, docs, stride, offs, lens, dq, B,
                            scores, None)


@pytest.mark.parametrize("fn", ["maxsim_rerank_pairs", "maxsim_rerank_pairs_bf16"])
@pytest.mark.parametrize("kw,code", [
    (dict(nq=-1), INVALID),
    (dict(q_rows=-1), INVALID),
    (dict(max_lq=-1), INVALID),
    (dict(max_lq=257), UNSUPPORTED),
    (dict(dq=None), INVALID),
    (dict(qo=None), INVALID),
    (dict(ql=None), INVALID),
    (dict(dq=FAKE + 2), INVALID),
    (dict(qo=FAKE + 1), INVALID),
    (dict(Qs=None), INVALID),
    (dict(Qs=FAKE + 4), UNSUPPORTED),
    (dict(d=12, stride=16), UNSUPPORTED),
    (dict(stride=64), INVALID),
    (dict(docs=None), INVALID),
    (dict(scores=None), INVALID),
    (dict(B=-3), INVALID),
    (dict(nq=0, qo=None, ql=None, B=0, docs=None, offs=None, lens=None, dq=None, scores=None), OK),
    (dict(B=0), OK),
])
def test_pairs_host_validation(lib, fn, kw, code):
    assert call_pairs(lib, fn, **kw) == code


def test_plan_pairs_validation(lib):
    def plan(offs=FAKE, lens=FAKE, dq=FAKE, B=4, qo=FAKE, ql=FAKE, nq=2, q_rows=40, max_lq=32, d=128,
             ws=FAKE, nbytes=1 << 20):
        return lib.maxsim_plan_pairs(offs, lens, dq, B, qo, ql, nq, q_rows, max_lq, d, ws, nbytes, None)

    assert plan(max_lq=0) == INVALID        # staged score/finish read Lq = 0 as "no rows"
    assert plan(max_lq=257) == UNSUPPORTED
    assert plan(dq=None) == INVALID
    assert plan(offs=None) == INVALID
    assert plan(nq=-1) == INVALID
    assert plan(d=100) == UNSUPPORTED
    assert plan(ws=None) == WORKSPACE
    assert plan(ws=FAKE + 128) == WORKSPACE
    assert plan(B=0, offs=None, lens=None, dq=None, ws=None) == OK


@pytest.mark.parametrize("fn", ["maxsim_rerank_multi", "maxsim_rerank_multi_bf16"])
def test_multi_host_validation(lib, fn):
    ql = (ctypes.c_int32 * 3)(32, 0, 17)

    def m(Qs=FAKE, q=ql, nq=3, d=128, docs=FAKE, stride=128, offs=FAKE, lens=FAKE + 1024, B=10,
          scores=FAKE + 4096):
        qp = ctypes.cast(q, ctypes.c_void_p) if q is not None else None
        return getattr(lib, fn)(Qs, qp, nq, d, docs, stride, offs, lens, B, scores, None)

    assert m(nq=-1) == INVALID
    assert m(q=None) == INVALID
    assert m(q=(ctypes.c_int32 * 3)(32, -1, 3)) == INVALID
    assert m(q=(ctypes.c_int32 * 3)(32, 257, 3)) == UNSUPPORTED
    assert m(Qs=None) == INVALID
    assert m(Qs=FAKE + 8) == UNSUPPORTED
    assert m(d=100, stride=104) == UNSUPPORTED
    assert m(docs=None) == INVALID
    assert m(scores=None) == INVALID
    assert m(B=0) == OK
    assert m(nq=0, q=None) == OK
    assert m(nq=0, q=None, scores=None) == OK      # zero queries write nothing
    assert m(Qs=None, q=(ctypes.c_int32 * 3)(0, 0, 0), B=0) == OK


@pytest.mark.parametrize("fn", ["maxsim_rerank_fp8", "maxsim_rerank_fp8_bf16"])
@pytest.mark.parametrize("kw,code", [
    (dict(scale=0.0), INVALID),
    (dict(scale=-1.0), INVALID),
    (dict(scale=float("inf")), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(d=24, stride=32), UNSUPPORTED),     # d % 16
    (dict(stride=136), UNSUPPORTED),          # stride % 16
    (dict(d=264, stride=272), UNSUPPORTED),
    (dict(Lq=257), UNSUPPORTED),
    (dict(stride=64), INVALID),               # stride < d
    (dict(docs=None), INVALID),
    (dict(Q=FAKE + 4), UNSUPPORTED),
    (dict(B=0, docs=None, offs=None, lens=None, scores=None), OK),
])
def test_fp8_host_validation(lib, fn, kw, code):
    a = dict(Q=FAKE, Lq=32, d=128, docs=FAKE, stride=128, offs=FAKE, lens=FAKE + 1024, B=10, scale=0.01,
             scores=FAKE + 4096)
    a.update(kw)
    assert getattr(lib, fn)(a["Q"], a["Lq"], a["d"], a["docs"], a["stride"], a["offs"], a["lens"], a["B"],
                            ctypes.c_float(a["scale"]), a["scores"], None) == code


def test_fp8_staged_validation(lib):
    f = ctypes.c_float
    assert lib.maxsim_score_fp8(2, FAKE, 32, 128, FAKE, 128, FAKE, FAKE, 4, f(1.0), FAKE, FAKE, 1 << 20, None) == INVALID
    assert lib.maxsim_score_fp8(0, FAKE, 32, 128, FAKE, 128, FAKE, FAKE, 4, f(0.0), FAKE, FAKE, 1 << 20, None) == INVALID
    assert lib.maxsim_score_fp8(0, FAKE, 32, 120, FAKE, 128, FAKE, FAKE, 4, f(1.0), FAKE, FAKE, 1 << 20, None) == UNSUPPORTED
    assert lib.maxsim_score_fp8(0, FAKE, 32, 128, FAKE, 128, FAKE, FAKE, 4, f(1.0), FAKE, None, 1 << 20, None) == WORKSPACE
    assert lib.maxsim_score_fp8(1, FAKE, 32, 128, FAKE, 128, FAKE, FAKE, 0, f(1.0), None, None, 0, None) == OK
    assert lib.maxsim_finish_fp8(0, 32, 128, 4, f(-2.0), FAKE, FAKE, 1 << 20, None) == INVALID
    assert lib.maxsim_finish_fp8(0, 32, 120, 4, f(1.0), FAKE, FAKE, 1 << 20, None) == UNSUPPORTED
    assert lib.maxsim_finish_fp8(0, 32, 128, 4, f(1.0), FAKE, None, 1 << 20, None) == WORKSPACE
    assert lib.maxsim_finish_fp8(0, 32, 128, 0, f(1.0), None, None, 0, None) == OK


def test_topk_validation(lib):
    n = ctypes.c_size_t(0)
    assert lib.maxsim_topk_workspace_size(100, 10, ctypes.byref(n)) == OK and n.value >= 256
    assert lib.maxsim_topk_workspace_size(80000, 100, ctypes.byref(n)) == OK
    assert n.value >= 2 * 20 * 100 * 8
    assert lib.maxsim_topk_workspace_size(-1, 10, ctypes.byref(n)) == INVALID
    assert lib.maxsim_topk_workspace_size(10, 1025, ctypes.byref(n)) == UNSUPPORTED
    assert lib.maxsim_topk_workspace_size(10, 10, None) == INVALID

    def tk(scores=FAKE, B=100, k=10, ts=FAKE + 4096, ti=FAKE + 8192, ws=FAKE + 65536, nb=1 << 20):
        return lib.maxsim_topk(scores, B, k, ts, ti, ws, nb, None)

    assert tk(k=-1) == INVALID
    assert tk(B=-1) == INVALID
    assert tk(k=1025) == UNSUPPORTED
    assert tk(k=0, scores=None, ts=None, ti=None, ws=None) == OK
    assert tk(scores=None) == INVALID
    assert tk(ts=None) == INVALID
    assert tk(ti=FAKE + 2) == INVALID
    assert tk(ws=None) == WORKSPACE
    assert tk(ws=FAKE + 128) == WORKSPACE
    assert tk(B=80000, k=100, nb=256) == WORKSPACE


@pytest.mark.parametrize("fn", ["maxsim_rerank_topk", "maxsim_rerank_topk_bf16"])
def test_rerank_topk_validation(lib, fn):
    def rt(Q=FAKE, Lq=32, d=128, docs=FAKE, stride=128, offs=FAKE, lens=FAKE + 1024, B=10, k=5,
           ts=FAKE + 4096, ti=FAKE + 8192):
        return getattr(lib, fn)(Q, Lq, d, docs, stride, offs, lens, B, k, ts, ti, None)

    assert rt(k=-1) == INVALID
    assert rt(k=1025) == UNSUPPORTED
    assert rt(ts=None) == INVALID
    assert rt(ti=FAKE + 1) == INVALID
    assert rt(d=12, stride=16) == UNSUPPORTED
    assert rt(docs=None) == INVALID
    assert rt(B=-1) == INVALID
    assert rt(k=0, ts=None, ti=None) == OK


def test_fp8_batch_forms_validation(lib):
    f = ctypes.c_float
    ql = (ctypes.c_int32 * 2)(32, 16)
    qp = ctypes.cast(ql, ctypes.c_void_p)

    def multi(dtype=0, d=128, stride=128, scale=0.5, B=10, docs=FAKE):
        return lib.maxsim_rerank_multi_fp8(dtype, FAKE, qp, 2, d, docs, stride, FAKE, FAKE + 1024, B, f(scale),
                                           FAKE + 4096, None)

    assert multi(dtype=2) == INVALID
    assert multi(scale=0.0) == INVALID
    assert multi(d=120, stride=128) == UNSUPPORTED
    assert multi(stride=136) == UNSUPPORTED
    assert multi(docs=None) == INVALID
    assert multi(B=0) == OK

    def pairs(dtype=1, d=128, stride=128, scale=0.5, B=10, max_lq=32):
        return lib.maxsim_rerank_pairs_fp8(dtype, FAKE, 64, d, FAKE + 8192, FAKE + 12288, 4, max_lq, FAKE, stride,
                                           FAKE, FAKE + 1024, FAKE + 16384, B, f(scale), FAKE + 4096, None)

    assert pairs(dtype=-1) == INVALID
    assert pairs(scale=float("inf")) == INVALID
    assert pairs(d=48, stride=56) == UNSUPPORTED
    assert pairs(max_lq=300) == UNSUPPORTED
    assert pairs(B=0) == OK
