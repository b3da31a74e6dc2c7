"""MI355X (gfx950) MaxSim late-interaction rerank.

One query Q[Lq, d] is scored against B variable-length documents read in place from a
packed, possibly scattered row tensor by per-document (offset, length) pairs:
score_i = sum over query rows of the best dot product with any of document i's rows
(Flash-MaxSim rerank page, docs.vllm.ai, vllm.v1.pool.flash_maxsim.flash_maxsim_rerank).
The pairs entry points score a batch of many queries in one launch, each document
against its own query; the multi entry points score several queries against the same
documents, reading each document tile once for a pass of up to 128 query rows; the
fp8 entry points read documents stored as FP8 E4M3 bytes with one scale.

The computation lives in libmaxsim.so (hand-written HIP, C ABI in include/maxsim.h);
this package is its ctypes binding. Build the library with
``python -m late_interaction_reranking_amd.build``.
"""

from .maxsim import (  # noqa: F401
    MAXSIM_BF16,
    MAXSIM_F16,
    MaxSimError,
    library_path,
    load,
    maxsim_plan,
    maxsim_plan_pairs,
    maxsim_rerank,
    maxsim_rerank_bf16,
    maxsim_rerank_multi,
    maxsim_rerank_multi_bf16,
    maxsim_rerank_multi_fp8,
    maxsim_rerank_pairs,
    maxsim_rerank_pairs_bf16,
    maxsim_rerank_pairs_fp8,
    maxsim_rerank_short,
    maxsim_rerank_noalloc,
    maxsim_rerank_topk,
    maxsim_topk,
    maxsim_finish,
    maxsim_finish_fp8,
    maxsim_rerank_fp8,
    maxsim_rerank_short_fp8,
    maxsim_score,
    maxsim_score_fp8,
    maxsim_status_string,
    maxsim_version,
    maxsim_workspace_size,
    rerank,
    rerank_multi,
    rerank_pairs,
    rerank_short,
)
