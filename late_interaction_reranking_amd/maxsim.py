"""Python binding of libmaxsim.so (ctypes). Argument marshalling only: every step of
the computation runs in the library's HIP kernels; PyTorch supplies device memory and
the current stream.

The functions carry the C ABI's names (include/maxsim.h) and take torch tensors:

    maxsim_rerank(Q, docs, doc_offsets, doc_lengths)       fp16 Q and docs
    maxsim_rerank_bf16(Q, docs, doc_offsets, doc_lengths)  bf16 Q and docs
    maxsim_workspace_size(Lq, d, B) -> bytes
    maxsim_plan(doc_offsets, doc_lengths, Lq, d, workspace)
    maxsim_score(Q, docs, doc_offsets, doc_lengths, workspace, scores=None)
    maxsim_finish(Q, B, workspace, scores)
    rerank(...)  picks maxsim_rerank or maxsim_rerank_bf16 from Q's dtype

    maxsim_rerank_pairs(Qs, q_offsets, q_lengths, max_lq, docs, doc_offsets,
                        doc_lengths, doc_query)                 fp16, many queries
    maxsim_rerank_pairs_bf16(...)                               bf16, many queries
    maxsim_plan_pairs(doc_offsets, doc_lengths, doc_query, q_offsets, q_lengths,
                      q_rows, max_lq, d, workspace)
    rerank_pairs(...)  picks the fp16 or bf16 pairs entry from Qs's dtype

    maxsim_rerank_multi(Qs, q_lengths, docs, doc_offsets, doc_lengths)
                       fp16, several queries against the same docs -> [nq, B]
    maxsim_rerank_multi_bf16(...)                               bf16
    rerank_multi(...)  picks one of the two from Qs's dtype

    maxsim_rerank_fp8(Q, docs8, doc_offsets, doc_lengths, doc_scale)
                       FP8 E4M3 docs (uint8 or float8_e4m3fn), fp16 or bf16 Q
    maxsim_rerank_short_fp8(...)  the same in one launch, one workgroup per doc
    maxsim_score_fp8(...), maxsim_finish_fp8(...)   staged form, after maxsim_plan

    maxsim_rerank_pairs_fp8(Qs, ..., doc_query, doc_scale)      pairs over FP8 docs
    maxsim_rerank_multi_fp8(Qs, q_lengths, docs8, ..., doc_scale) shared docs, FP8

    maxsim_topk(scores, k) -> (top_scores [k], top_ids [k])   device top-k
    maxsim_rerank_topk(Q, docs, doc_offsets, doc_lengths, k)  scores + top-k, one call

Q is [Lq, d] and contiguous; docs is a 2-D view whose rows are docs.stride(0) elements
apart with unit column stride (a column slice of a wider tensor works: its extra
columns are never read); doc_offsets and doc_lengths are int32 [B] on the same device.
The scores are fp32 [B] (Flash-MaxSim rerank page, docs.vllm.ai,
vllm.v1.pool.flash_maxsim.flash_maxsim_rerank, `flash_maxsim_rerank_direct`).
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = [
    "MaxSimError",
    "library_path",
    "load",
    "maxsim_rerank",
    "maxsim_rerank_bf16",
    "maxsim_status_string",
    "maxsim_workspace_size",
    "maxsim_plan",
    "maxsim_score",
    "maxsim_finish",
    "maxsim_version",
    "rerank",
    "maxsim_rerank_short",
    "rerank_short",
    "maxsim_rerank_noalloc",
    "maxsim_rerank_pairs",
    "maxsim_rerank_pairs_bf16",
    "maxsim_plan_pairs",
    "rerank_pairs",
    "maxsim_rerank_multi",
    "maxsim_rerank_multi_bf16",
    "rerank_multi",
    "maxsim_rerank_fp8",
    "maxsim_rerank_short_fp8",
    "maxsim_score_fp8",
    "maxsim_finish_fp8",
    "maxsim_topk",
    "maxsim_rerank_topk",
    "maxsim_rerank_pairs_fp8",
    "maxsim_rerank_multi_fp8",
    "MAXSIM_F16",
    "MAXSIM_BF16",
]

MAXSIM_OK = 0
MAXSIM_F16 = 0
MAXSIM_BF16 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_lock = threading.Lock()
_lib = None


class MaxSimError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status}: {maxsim_status_string(status)}")


def library_path() -> str:
    """libmaxsim.so next to this file, or the build MAXSIM_LIBRARY names (another build of
    the same sources, e.g. one with the host code address-sanitised)."""
    return os.environ.get("MAXSIM_LIBRARY") or os.path.join(_HERE, "libmaxsim.so")


def load() -> ctypes.CDLL:
    """Load libmaxsim.so (built in-tree by late_interaction_reranking_amd.build)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with `python -m late_interaction_reranking_amd.build`"
            )
        lib = ctypes.CDLL(path)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        rr = [P, I32, I32, P, I64, P, P, I32, P, P]
        for name in ("maxsim_rerank", "maxsim_rerank_bf16"):
            fn = getattr(lib, name)
            fn.restype = ctypes.c_int
            fn.argtypes = rr
        lib.maxsim_rerank_short.restype = ctypes.c_int
        lib.maxsim_rerank_short.argtypes = [ctypes.c_int, *rr]
        lib.maxsim_rerank_noalloc.restype = ctypes.c_int
        lib.maxsim_rerank_noalloc.argtypes = [ctypes.c_int, *rr]
        lib.maxsim_status_string.restype = ctypes.c_char_p
        lib.maxsim_status_string.argtypes = [ctypes.c_int]
        lib.maxsim_workspace_size.restype = ctypes.c_int
        lib.maxsim_workspace_size.argtypes = [I32, I32, I32, ctypes.POINTER(SZ)]
        lib.maxsim_plan.restype = ctypes.c_int
        lib.maxsim_plan.argtypes = [P, P, I32, I32, I32, P, SZ, P]
        lib.maxsim_score.restype = ctypes.c_int
        lib.maxsim_score.argtypes = [ctypes.c_int, P, I32, I32, P, I64, P, P, I32, P, P, SZ, P]
        lib.maxsim_finish.restype = ctypes.c_int
        lib.maxsim_finish.argtypes = [ctypes.c_int, I32, I32, I32, P, P, SZ, P]
        pr = [P, I32, I32, P, P, I32, I32, P, I64, P, P, P, I32, P, P]
        for name in ("maxsim_rerank_pairs", "maxsim_rerank_pairs_bf16"):
            fn = getattr(lib, name)
            fn.restype = ctypes.c_int
            fn.argtypes = pr
        mr = [P, P, I32, I32, P, I64, P, P, I32, P, P]
        for name in ("maxsim_rerank_multi", "maxsim_rerank_multi_bf16"):
            fn = getattr(lib, name)
            fn.restype = ctypes.c_int
            fn.argtypes = mr
        F32 = ctypes.c_float
        for name in ("maxsim_rerank_fp8", "maxsim_rerank_fp8_bf16"):
            fn = getattr(lib, name)
            fn.restype = ctypes.c_int
            fn.argtypes = [P, I32, I32, P, I64, P, P, I32, F32, P, P]
        lib.maxsim_rerank_short_fp8.restype = ctypes.c_int
        lib.maxsim_rerank_short_fp8.argtypes = [ctypes.c_int, P, I32, I32, P, I64, P, P, I32, F32, P, P]
        lib.maxsim_score_fp8.restype = ctypes.c_int
        lib.maxsim_score_fp8.argtypes = [ctypes.c_int, P, I32, I32, P, I64, P, P, I32, F32, P, P, SZ, P]
        lib.maxsim_finish_fp8.restype = ctypes.c_int
        lib.maxsim_finish_fp8.argtypes = [ctypes.c_int, I32, I32, I32, F32, P, P, SZ, P]
        lib.maxsim_rerank_pairs_fp8.restype = ctypes.c_int
        lib.maxsim_rerank_pairs_fp8.argtypes = [ctypes.c_int, P, I32, I32, P, P, I32, I32, P, I64, P, P, P, I32,
                                                F32, P, P]
        lib.maxsim_rerank_multi_fp8.restype = ctypes.c_int
        lib.maxsim_rerank_multi_fp8.argtypes = [ctypes.c_int, P, P, I32, I32, P, I64, P, P, I32, F32, P, P]
        lib.maxsim_topk_workspace_size.restype = ctypes.c_int
        lib.maxsim_topk_workspace_size.argtypes = [I32, I32, ctypes.POINTER(SZ)]
        lib.maxsim_topk.restype = ctypes.c_int
        lib.maxsim_topk.argtypes = [P, I32, I32, P, P, P, SZ, P]
        for name in ("maxsim_rerank_topk", "maxsim_rerank_topk_bf16"):
            fn = getattr(lib, name)
            fn.restype = ctypes.c_int
            fn.argtypes = [P, I32, I32, P, I64, P, P, I32, I32, P, P, P]
        lib.maxsim_plan_pairs.restype = ctypes.c_int
        lib.maxsim_plan_pairs.argtypes = [P, P, P, I32, P, P, I32, I32, I32, I32, P, SZ, P]
        lib.maxsim_version.restype = ctypes.c_int
        lib.maxsim_version.argtypes = []
        _lib = lib
        return lib


def maxsim_status_string(status: int) -> str:
    return load().maxsim_status_string(int(status)).decode()


def maxsim_version() -> int:
    return int(load().maxsim_version())


def _check(status: int, where: str) -> None:
    if status != MAXSIM_OK:
        raise MaxSimError(status, where)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _marshal(Q, docs, doc_offsets, doc_lengths, dtype):
    if Q.dim() != 2 or docs.dim() != 2:
        raise ValueError("Q and docs must be 2-D")
    if Q.dtype != dtype or docs.dtype != dtype:
        raise TypeError(f"Q and docs must both be {dtype}")
    if doc_offsets.dtype != torch.int32 or doc_lengths.dtype != torch.int32:
        raise TypeError("doc_offsets and doc_lengths must be int32")
    if doc_offsets.dim() != 1 or doc_offsets.shape != doc_lengths.shape:
        raise ValueError("doc_offsets and doc_lengths must be 1-D of equal length")
    dev = docs.device
    for name, t in (("Q", Q), ("docs", docs), ("doc_offsets", doc_offsets), ("doc_lengths", doc_lengths)):
        if t.device != dev or dev.type != "cuda":
            raise ValueError(f"{name} must live on the GPU, with docs")
    if not Q.is_contiguous() or not doc_offsets.is_contiguous() or not doc_lengths.is_contiguous():
        raise ValueError("Q, doc_offsets and doc_lengths must be contiguous")
    if docs.shape[0] > 0 and docs.stride(1) != 1:
        raise ValueError("docs must have unit column stride")
    if Q.shape[1] != docs.shape[1]:
        raise ValueError("Q and docs must have the same width d")
    Lq, d = int(Q.shape[0]), int(Q.shape[1])
    stride = int(docs.stride(0)) if docs.shape[0] > 1 else max(int(docs.stride(0)), d)
    return Lq, d, stride, int(doc_offsets.shape[0])


def _scores_out(scores, shape, dev) -> torch.Tensor:
    """A new fp32 score tensor of `shape` on `dev`, or the caller's after checking that it
    is one: contiguous fp32 of that shape on the same GPU as the docs (the kernels store
    through its pointer, so a tensor on the host or on another GPU must never reach them)."""
    if scores is None:
        return torch.empty(shape, dtype=torch.float32, device=dev)
    if scores.dtype != torch.float32 or tuple(scores.shape) != tuple(shape) or not scores.is_contiguous():
        raise ValueError(f"scores must be a contiguous float32 {list(shape)} tensor")
    if scores.device != dev:
        raise ValueError(f"scores must live on {dev}, with docs (got {scores.device})")
    return scores


def _rerank(fn_name, dtype, Q, docs, doc_offsets, doc_lengths, scores=None):
    Lq, d, stride, B = _marshal(Q, docs, doc_offsets, doc_lengths, dtype)
    scores = _scores_out(scores, (B,), docs.device)
    with torch.cuda.device(docs.device):
        st = getattr(load(), fn_name)(
            Q.data_ptr(), Lq, d, docs.data_ptr(), stride, doc_offsets.data_ptr(),
            doc_lengths.data_ptr(), B, scores.data_ptr(), _stream(docs),
        )
    _check(st, fn_name)
    return scores


def maxsim_rerank(Q, docs, doc_offsets, doc_lengths, scores=None) -> torch.Tensor:
    """fp32 [B] MaxSim scores, fp16 inputs."""
    return _rerank("maxsim_rerank", torch.float16, Q, docs, doc_offsets, doc_lengths, scores)


def maxsim_rerank_bf16(Q, docs, doc_offsets, doc_lengths, scores=None) -> torch.Tensor:
    """fp32 [B] MaxSim scores, bf16 inputs."""
    return _rerank("maxsim_rerank_bf16", torch.bfloat16, Q, docs, doc_offsets, doc_lengths, scores)


def rerank(Q, docs, doc_offsets, doc_lengths, scores=None) -> torch.Tensor:
    """maxsim_rerank or maxsim_rerank_bf16, chosen by Q's dtype."""
    if Q.dtype == torch.bfloat16:
        return maxsim_rerank_bf16(Q, docs, doc_offsets, doc_lengths, scores)
    return maxsim_rerank(Q, docs, doc_offsets, doc_lengths, scores)


def maxsim_rerank_short(Q, docs, doc_offsets, doc_lengths, scores=None) -> torch.Tensor:
    """fp32 [B] MaxSim scores in one launch, one workgroup per doc (for batches of short
    docs); fp16 or bf16 by Q's dtype. Bitwise equal to maxsim_rerank."""
    dtype = torch.bfloat16 if Q.dtype == torch.bfloat16 else torch.float16
    Lq, d, stride, B = _marshal(Q, docs, doc_offsets, doc_lengths, dtype)
    scores = _scores_out(scores, (B,), docs.device)
    code = MAXSIM_BF16 if dtype == torch.bfloat16 else MAXSIM_F16
    with torch.cuda.device(docs.device):
        st = load().maxsim_rerank_short(
            code, Q.data_ptr(), Lq, d, docs.data_ptr(), stride, doc_offsets.data_ptr(),
            doc_lengths.data_ptr(), B, scores.data_ptr(), _stream(docs),
        )
    _check(st, "maxsim_rerank_short")
    return scores


rerank_short = maxsim_rerank_short


def maxsim_rerank_noalloc(Q, docs, doc_offsets, doc_lengths, scores=None) -> torch.Tensor:
    """maxsim_rerank's scores (bitwise) with the library's fixed per-GPU scratch as the
    workspace: the call allocates no device memory (pass `scores` to allocate nothing
    at all). Calls that overlap on one GPU race; fp16 or bf16 by Q's dtype."""
    dtype = torch.bfloat16 if Q.dtype == torch.bfloat16 else torch.float16
    Lq, d, stride, B = _marshal(Q, docs, doc_offsets, doc_lengths, dtype)
    scores = _scores_out(scores, (B,), docs.device)
    code = MAXSIM_BF16 if dtype == torch.bfloat16 else MAXSIM_F16
    with torch.cuda.device(docs.device):
        st = load().maxsim_rerank_noalloc(
            code, Q.data_ptr(), Lq, d, docs.data_ptr(), stride, doc_offsets.data_ptr(),
            doc_lengths.data_ptr(), B, scores.data_ptr(), _stream(docs),
        )
    _check(st, "maxsim_rerank_noalloc")
    return scores


def maxsim_workspace_size(Lq: int, d: int, B: int, device=None) -> int:
    """Bytes of workspace maxsim_plan / maxsim_score need on `device` (current by default)."""
    n = ctypes.c_size_t(0)
    dev = torch.device("cuda") if device is None else torch.device(device)
    with torch.cuda.device(dev):
        st = load().maxsim_workspace_size(int(Lq), int(d), int(B), ctypes.byref(n))
    _check(st, "maxsim_workspace_size")
    return int(n.value)


def _ws(workspace: torch.Tensor, dev=None) -> tuple[int, int]:
    """Pointer and size of a caller workspace: a contiguous uint8 tensor on the GPU, on
    `dev` (the device of the tensors the call reads or writes) when given."""
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous() or workspace.device.type != "cuda":
        raise ValueError("workspace must be a contiguous uint8 GPU tensor")
    if dev is not None and workspace.device != dev:
        raise ValueError(f"workspace must live on {dev}, with the other tensors (got {workspace.device})")
    return workspace.data_ptr(), int(workspace.numel())


def maxsim_plan(doc_offsets, doc_lengths, Lq: int, d: int, workspace: torch.Tensor) -> None:
    """Enqueue the length-binned schedule into `workspace` on the current stream."""
    if doc_offsets.dtype != torch.int32 or doc_lengths.dtype != torch.int32:
        raise TypeError("doc_offsets and doc_lengths must be int32")
    if doc_offsets.device != workspace.device or doc_lengths.device != workspace.device:
        raise ValueError("doc_offsets and doc_lengths must live on the workspace's GPU")
    ptr, nbytes = _ws(workspace)
    with torch.cuda.device(workspace.device):
        st = load().maxsim_plan(doc_offsets.data_ptr(), doc_lengths.data_ptr(), int(doc_offsets.shape[0]),
                                int(Lq), int(d), ptr, nbytes, _stream(workspace))
    _check(st, "maxsim_plan")


def maxsim_score(Q, docs, doc_offsets, doc_lengths, workspace: torch.Tensor, scores=None,
                 Lq: int | None = None) -> torch.Tensor:
    """Enqueue the score kernel over a schedule maxsim_plan (or maxsim_plan_pairs) wrote
    into `workspace`. Docs the schedule split are completed by maxsim_finish. Lq
    defaults to Q's row count; after maxsim_plan_pairs pass its max_lq."""
    dtype = torch.bfloat16 if Q.dtype == torch.bfloat16 else torch.float16
    q_rows, d, stride, B = _marshal(Q, docs, doc_offsets, doc_lengths, dtype)
    Lq = q_rows if Lq is None else int(Lq)
    scores = _scores_out(scores, (B,), docs.device)
    ptr, nbytes = _ws(workspace, docs.device)
    code = MAXSIM_BF16 if dtype == torch.bfloat16 else MAXSIM_F16
    with torch.cuda.device(docs.device):
        st = load().maxsim_score(code, Q.data_ptr(), Lq, d, docs.data_ptr(), stride,
                                 doc_offsets.data_ptr(), doc_lengths.data_ptr(), B,
                                 scores.data_ptr(), ptr, nbytes, _stream(docs))
    _check(st, "maxsim_score")
    return scores


def maxsim_finish(Q, B: int, workspace: torch.Tensor, scores: torch.Tensor,
                  Lq: int | None = None) -> torch.Tensor:
    """Enqueue the combine step: the scores of docs the schedule split into several
    work items. Q only supplies d, the element format and, unless given, Lq."""
    if Q.dim() != 2:
        raise ValueError("Q must be 2-D")
    if scores is None or scores.device.type != "cuda":
        raise ValueError("scores must be a GPU tensor")
    scores = _scores_out(scores, (B,), scores.device)
    code = MAXSIM_BF16 if Q.dtype == torch.bfloat16 else MAXSIM_F16
    ptr, nbytes = _ws(workspace, scores.device)
    with torch.cuda.device(workspace.device):
        st = load().maxsim_finish(code, int(Q.shape[0]) if Lq is None else int(Lq), int(Q.shape[1]),
                                  int(B), scores.data_ptr(),
                                  ptr, nbytes, _stream(workspace))
    _check(st, "maxsim_finish")
    return scores


def _int32_vec(t, name, dev):
    if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous 1-D int32 tensor")
    if t.device != dev:
        raise ValueError(f"{name} must live on the GPU, with docs")


def _rerank_pairs(fn_name, dtype, Qs, q_offsets, q_lengths, max_lq, docs, doc_offsets, doc_lengths,
                  doc_query, scores=None):
    _, d, stride, B = _marshal(Qs, docs, doc_offsets, doc_lengths, dtype)
    dev = docs.device
    for name, t in (("q_offsets", q_offsets), ("q_lengths", q_lengths), ("doc_query", doc_query)):
        _int32_vec(t, name, dev)
    if q_offsets.shape != q_lengths.shape:
        raise ValueError("q_offsets and q_lengths must have one entry per query")
    if doc_query.shape[0] != B:
        raise ValueError("doc_query must have one entry per doc")
    scores = _scores_out(scores, (B,), dev)
    with torch.cuda.device(dev):
        st = getattr(load(), fn_name)(
            Qs.data_ptr(), int(Qs.shape[0]), d, q_offsets.data_ptr(), q_lengths.data_ptr(),
            int(q_offsets.shape[0]), int(max_lq), docs.data_ptr(), stride, doc_offsets.data_ptr(),
            doc_lengths.data_ptr(), doc_query.data_ptr(), B, scores.data_ptr(), _stream(docs),
        )
    _check(st, fn_name)
    return scores


def maxsim_rerank_pairs(Qs, q_offsets, q_lengths, max_lq: int, docs, doc_offsets, doc_lengths,
                        doc_query, scores=None) -> torch.Tensor:
    """fp32 [B] scores, doc i against query doc_query[i] (rows q_offsets[j] ..
    q_offsets[j] + q_lengths[j] - 1 of Qs); fp16 inputs. max_lq bounds q_lengths."""
    return _rerank_pairs("maxsim_rerank_pairs", torch.float16, Qs, q_offsets, q_lengths, max_lq,
                         docs, doc_offsets, doc_lengths, doc_query, scores)


def maxsim_rerank_pairs_bf16(Qs, q_offsets, q_lengths, max_lq: int, docs, doc_offsets, doc_lengths,
                             doc_query, scores=None) -> torch.Tensor:
    """maxsim_rerank_pairs with bf16 inputs."""
    return _rerank_pairs("maxsim_rerank_pairs_bf16", torch.bfloat16, Qs, q_offsets, q_lengths, max_lq,
                         docs, doc_offsets, doc_lengths, doc_query, scores)


def rerank_pairs(Qs, q_offsets, q_lengths, max_lq: int, docs, doc_offsets, doc_lengths, doc_query,
                 scores=None) -> torch.Tensor:
    """maxsim_rerank_pairs or maxsim_rerank_pairs_bf16, chosen by Qs's dtype."""
    fn = maxsim_rerank_pairs_bf16 if Qs.dtype == torch.bfloat16 else maxsim_rerank_pairs
    return fn(Qs, q_offsets, q_lengths, max_lq, docs, doc_offsets, doc_lengths, doc_query, scores)


def maxsim_plan_pairs(doc_offsets, doc_lengths, doc_query, q_offsets, q_lengths, q_rows: int,
                      max_lq: int, d: int, workspace: torch.Tensor) -> None:
    """Enqueue the schedule of a multi-query batch into `workspace`, sized by
    maxsim_workspace_size(max_lq, d, B). The batch is then scored by
    maxsim_score(Qs, ..., Lq=max_lq) and maxsim_finish(Qs, B, workspace, scores,
    Lq=max_lq). max_lq must be at least 1."""
    dev = workspace.device
    for name, t in (("doc_offsets", doc_offsets), ("doc_lengths", doc_lengths), ("doc_query", doc_query),
                    ("q_offsets", q_offsets), ("q_lengths", q_lengths)):
        _int32_vec(t, name, dev)
    ptr, nbytes = _ws(workspace)
    with torch.cuda.device(dev):
        st = load().maxsim_plan_pairs(doc_offsets.data_ptr(), doc_lengths.data_ptr(), doc_query.data_ptr(),
                                      int(doc_offsets.shape[0]), q_offsets.data_ptr(), q_lengths.data_ptr(),
                                      int(q_offsets.shape[0]), int(q_rows), int(max_lq), int(d), ptr, nbytes,
                                      _stream(workspace))
    _check(st, "maxsim_plan_pairs")


def _rerank_multi(fn_name, dtype, Qs, q_lengths, docs, doc_offsets, doc_lengths, scores=None):
    _, d, stride, B = _marshal(Qs, docs, doc_offsets, doc_lengths, dtype)
    ql = [int(x) for x in (q_lengths.tolist() if hasattr(q_lengths, "tolist") else q_lengths)]
    nq = len(ql)
    if sum(ql) != Qs.shape[0]:
        raise ValueError("Qs must hold exactly the rows of the queries, back to back")
    host = (ctypes.c_int32 * max(nq, 1))(*ql)
    scores = _scores_out(scores, (nq, B), docs.device)
    with torch.cuda.device(docs.device):
        st = getattr(load(), fn_name)(
            Qs.data_ptr(), ctypes.cast(host, ctypes.c_void_p), nq, d, docs.data_ptr(), stride,
            doc_offsets.data_ptr(), doc_lengths.data_ptr(), B, scores.data_ptr(), _stream(docs),
        )
    _check(st, fn_name)
    return scores


def maxsim_rerank_multi(Qs, q_lengths, docs, doc_offsets, doc_lengths, scores=None) -> torch.Tensor:
    """fp32 [nq, B] scores of nq queries (rows back to back in Qs, lengths q_lengths,
    a host sequence) against the same B docs; fp16 inputs. Each doc tile is read once
    per pass of up to 128 query rows (64 when d > 128)."""
    return _rerank_multi("maxsim_rerank_multi", torch.float16, Qs, q_lengths, docs, doc_offsets,
                         doc_lengths, scores)


def maxsim_rerank_multi_bf16(Qs, q_lengths, docs, doc_offsets, doc_lengths, scores=None) -> torch.Tensor:
    """maxsim_rerank_multi with bf16 inputs."""
    return _rerank_multi("maxsim_rerank_multi_bf16", torch.bfloat16, Qs, q_lengths, docs, doc_offsets,
                         doc_lengths, scores)


def rerank_multi(Qs, q_lengths, docs, doc_offsets, doc_lengths, scores=None) -> torch.Tensor:
    """maxsim_rerank_multi or maxsim_rerank_multi_bf16, chosen by Qs's dtype."""
    fn = maxsim_rerank_multi_bf16 if Qs.dtype == torch.bfloat16 else maxsim_rerank_multi
    return fn(Qs, q_lengths, docs, doc_offsets, doc_lengths, scores)


def _check_fp8_args(Q, docs, doc_offsets, doc_lengths):
    if docs.dtype not in (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8)):
        raise TypeError("docs must hold FP8 E4M3 bytes (uint8 or float8_e4m3fn)")
    if Q.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("Q must be float16 or bfloat16")
    if Q.dim() != 2 or docs.dim() != 2:
        raise ValueError("Q and docs must be 2-D")
    if doc_offsets.dtype != torch.int32 or doc_lengths.dtype != torch.int32:
        raise TypeError("doc_offsets and doc_lengths must be int32")
    if doc_offsets.dim() != 1 or doc_offsets.shape != doc_lengths.shape:
        raise ValueError("doc_offsets and doc_lengths must be 1-D of equal length")
    dev = docs.device
    for name, t in (("Q", Q), ("docs", docs), ("doc_offsets", doc_offsets), ("doc_lengths", doc_lengths)):
        if t.device != dev or dev.type != "cuda":
            raise ValueError(f"{name} must live on the GPU, with docs")
    if not Q.is_contiguous() or not doc_offsets.is_contiguous() or not doc_lengths.is_contiguous():
        raise ValueError("Q, doc_offsets and doc_lengths must be contiguous")
    if docs.shape[0] > 0 and docs.stride(1) != 1:
        raise ValueError("docs must have unit column stride")
    if Q.shape[1] != docs.shape[1]:
        raise ValueError("Q and docs must have the same width d")
    Lq, d = int(Q.shape[0]), int(Q.shape[1])
    stride = int(docs.stride(0)) if docs.shape[0] > 1 else max(int(docs.stride(0)), d)
    return Lq, d, stride, int(doc_offsets.shape[0])


def maxsim_rerank_fp8(Q, docs, doc_offsets, doc_lengths, doc_scale: float, scores=None) -> torch.Tensor:
    """fp32 [B] MaxSim scores with docs stored as FP8 E4M3 bytes (element = doc_scale *
    e4m3) and an fp16 or bf16 query; d and the row stride (bytes) multiples of 16."""
    Lq, d, stride, B = _check_fp8_args(Q, docs, doc_offsets, doc_lengths)
    scores = _scores_out(scores, (B,), docs.device)
    name = "maxsim_rerank_fp8_bf16" if Q.dtype == torch.bfloat16 else "maxsim_rerank_fp8"
    with torch.cuda.device(docs.device):
        st = getattr(load(), name)(Q.data_ptr(), Lq, d, docs.data_ptr(), stride, doc_offsets.data_ptr(),
                                   doc_lengths.data_ptr(), B, float(doc_scale), scores.data_ptr(),
                                   _stream(docs))
    _check(st, name)
    return scores


def maxsim_rerank_short_fp8(Q, docs, doc_offsets, doc_lengths, doc_scale: float, scores=None) -> torch.Tensor:
    """maxsim_rerank_fp8's scores in one launch, one workgroup per doc (for batches of
    short docs); bitwise equal to maxsim_rerank_fp8 with the same query dtype."""
    Lq, d, stride, B = _check_fp8_args(Q, docs, doc_offsets, doc_lengths)
    scores = _scores_out(scores, (B,), docs.device)
    code = MAXSIM_BF16 if Q.dtype == torch.bfloat16 else MAXSIM_F16
    with torch.cuda.device(docs.device):
        st = load().maxsim_rerank_short_fp8(code, Q.data_ptr(), Lq, d, docs.data_ptr(), stride,
                                            doc_offsets.data_ptr(), doc_lengths.data_ptr(), B,
                                            float(doc_scale), scores.data_ptr(), _stream(docs))
    _check(st, "maxsim_rerank_short_fp8")
    return scores


def maxsim_score_fp8(Q, docs, doc_offsets, doc_lengths, doc_scale: float, workspace: torch.Tensor,
                     scores=None) -> torch.Tensor:
    """Staged score kernel for FP8 E4M3 docs over a schedule maxsim_plan wrote."""
    Lq, d, stride, B = _check_fp8_args(Q, docs, doc_offsets, doc_lengths)
    scores = _scores_out(scores, (B,), docs.device)
    ptr, nbytes = _ws(workspace, docs.device)
    code = MAXSIM_BF16 if Q.dtype == torch.bfloat16 else MAXSIM_F16
    with torch.cuda.device(docs.device):
        st = load().maxsim_score_fp8(code, Q.data_ptr(), Lq, d, docs.data_ptr(), stride, doc_offsets.data_ptr(),
                                     doc_lengths.data_ptr(), B, float(doc_scale), scores.data_ptr(), ptr, nbytes,
                                     _stream(docs))
    _check(st, "maxsim_score_fp8")
    return scores


def maxsim_finish_fp8(Q, B: int, doc_scale: float, workspace: torch.Tensor, scores: torch.Tensor) -> torch.Tensor:
    """Staged combine step for FP8 E4M3 docs (Q supplies Lq, d and its format)."""
    if Q.dim() != 2:
        raise ValueError("Q must be 2-D")
    if scores is None or scores.device.type != "cuda":
        raise ValueError("scores must be a GPU tensor")
    scores = _scores_out(scores, (B,), scores.device)
    code = MAXSIM_BF16 if Q.dtype == torch.bfloat16 else MAXSIM_F16
    ptr, nbytes = _ws(workspace, scores.device)
    with torch.cuda.device(workspace.device):
        st = load().maxsim_finish_fp8(code, int(Q.shape[0]), int(Q.shape[1]), int(B), float(doc_scale),
                                      scores.data_ptr(), ptr, nbytes, _stream(workspace))
    _check(st, "maxsim_finish_fp8")
    return scores


def maxsim_topk(scores: torch.Tensor, k: int, workspace: torch.Tensor | None = None):
    """(top_scores fp32 [k], top_ids int32 [k]) of a contiguous fp32 score vector on the
    GPU: score descending, ties by lower index, NaN last; (-inf, -1) past the end."""
    if scores.dtype != torch.float32 or scores.dim() != 1 or not scores.is_contiguous():
        raise ValueError("scores must be a contiguous 1-D float32 tensor")
    if scores.device.type != "cuda":
        raise ValueError("scores must live on the GPU")
    B, k = int(scores.shape[0]), int(k)
    if k < 0:
        raise ValueError("k must be >= 0")
    dev = scores.device
    n = ctypes.c_size_t(0)
    _check(load().maxsim_topk_workspace_size(B, k, ctypes.byref(n)), "maxsim_topk_workspace_size")
    if workspace is None:
        workspace = torch.empty(int(n.value), dtype=torch.uint8, device=dev)
    ptr, nbytes = _ws(workspace, dev)
    top_scores = torch.empty(k, dtype=torch.float32, device=dev)
    top_ids = torch.empty(k, dtype=torch.int32, device=dev)
    with torch.cuda.device(dev):
        st = load().maxsim_topk(scores.data_ptr(), B, k, top_scores.data_ptr(), top_ids.data_ptr(), ptr, nbytes,
                                _stream(scores))
    _check(st, "maxsim_topk")
    return top_scores, top_ids


def maxsim_rerank_topk(Q, docs, doc_offsets, doc_lengths, k: int):
    """The k best docs of a single-query rerank, (top_scores [k], top_ids [k]), without
    materialising the scores outside the library (fp16 or bf16 from Q's dtype)."""
    dtype = torch.bfloat16 if Q.dtype == torch.bfloat16 else torch.float16
    Lq, d, stride, B = _marshal(Q, docs, doc_offsets, doc_lengths, dtype)
    k = int(k)
    if k < 0:
        raise ValueError("k must be >= 0")
    top_scores = torch.empty(k, dtype=torch.float32, device=docs.device)
    top_ids = torch.empty(k, dtype=torch.int32, device=docs.device)
    name = "maxsim_rerank_topk_bf16" if dtype == torch.bfloat16 else "maxsim_rerank_topk"
    with torch.cuda.device(docs.device):
        st = getattr(load(), name)(Q.data_ptr(), Lq, d, docs.data_ptr(), stride, doc_offsets.data_ptr(),
                                   doc_lengths.data_ptr(), B, k, top_scores.data_ptr(), top_ids.data_ptr(),
                                   _stream(docs))
    _check(st, name)
    return top_scores, top_ids


def maxsim_rerank_pairs_fp8(Qs, q_offsets, q_lengths, max_lq: int, docs, doc_offsets, doc_lengths, doc_query,
                            doc_scale: float, scores=None) -> torch.Tensor:
    """maxsim_rerank_pairs over docs stored as FP8 E4M3 bytes (element = doc_scale *
    e4m3); Qs fp16 or bf16."""
    _, d, stride, B = _check_fp8_args(Qs, docs, doc_offsets, doc_lengths)
    dev = docs.device
    for name, t in (("q_offsets", q_offsets), ("q_lengths", q_lengths), ("doc_query", doc_query)):
        _int32_vec(t, name, dev)
    if q_offsets.shape != q_lengths.shape or doc_query.shape[0] != B:
        raise ValueError("q_offsets / q_lengths: one entry per query; doc_query: one per doc")
    scores = _scores_out(scores, (B,), dev)
    code = MAXSIM_BF16 if Qs.dtype == torch.bfloat16 else MAXSIM_F16
    with torch.cuda.device(dev):
        st = load().maxsim_rerank_pairs_fp8(
            code, Qs.data_ptr(), int(Qs.shape[0]), d, q_offsets.data_ptr(), q_lengths.data_ptr(),
            int(q_offsets.shape[0]), int(max_lq), docs.data_ptr(), stride, doc_offsets.data_ptr(),
            doc_lengths.data_ptr(), doc_query.data_ptr(), B, float(doc_scale), scores.data_ptr(), _stream(docs))
    _check(st, "maxsim_rerank_pairs_fp8")
    return scores


def maxsim_rerank_multi_fp8(Qs, q_lengths, docs, doc_offsets, doc_lengths, doc_scale: float,
                            scores=None) -> torch.Tensor:
    """maxsim_rerank_multi over docs stored as FP8 E4M3 bytes (element = doc_scale *
    e4m3); Qs fp16 or bf16; q_lengths a host sequence. Returns [nq, B]."""
    _, d, stride, B = _check_fp8_args(Qs, docs, doc_offsets, doc_lengths)
    ql = [int(x) for x in (q_lengths.tolist() if hasattr(q_lengths, "tolist") else q_lengths)]
    nq = len(ql)
    if sum(ql) != Qs.shape[0]:
        raise ValueError("Qs must hold exactly the rows of the queries, back to back")
    host = (ctypes.c_int32 * max(nq, 1))(*ql)
    scores = _scores_out(scores, (nq, B), docs.device)
    code = MAXSIM_BF16 if Qs.dtype == torch.bfloat16 else MAXSIM_F16
    with torch.cuda.device(docs.device):
        st = load().maxsim_rerank_multi_fp8(code, Qs.data_ptr(), ctypes.cast(host, ctypes.c_void_p), nq, d,
                                            docs.data_ptr(), stride, doc_offsets.data_ptr(), doc_lengths.data_ptr(),
                                            B, float(doc_scale), scores.data_ptr(), _stream(docs))
    _check(st, "maxsim_rerank_multi_fp8")
    return scores
