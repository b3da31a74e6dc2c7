/*
 * maxsim.h -- C ABI of the MI355X (gfx950) MaxSim rerank library, libmaxsim.so.
 *
 * Operation (Flash-MaxSim rerank page, docs.vllm.ai,
 * vllm.v1.pool.flash_maxsim.flash_maxsim_rerank: the module description and the
 * parameters and return value of `flash_maxsim_rerank_direct`): one query Q of Lq
 * token rows, each d wide, is scored against B documents whose token rows sit in a
 * packed row tensor. Document i is the run of doc_lengths[i] consecutive rows that
 * starts at row doc_offsets[i]; documents may be scattered, in any order, with
 * unrelated rows between them, and may overlap. For each document
 *
 *     scores[i] = sum over q < Lq of  max over t < doc_lengths[i] of  Q[q] . row(doc_offsets[i] + t)
 *
 * computed from fp16 or bf16 inputs with fp32 products and sums. Nothing is padded
 * or copied and no [B, Lq, len] similarity tensor is formed.
 *
 * Conventions shared by every entry point:
 *   - Pointers named Q, docs, doc_offsets, doc_lengths, scores and workspace are
 *     DEVICE pointers (any allocator, including PyTorch's caching allocator). The
 *     caller owns every buffer; the library keeps no pointer after the call returns.
 *   - Scratch of the one-shot entry points (those that take no workspace argument and
 *     need one: maxsim_rerank[_bf16], _pairs, _multi, _fp8, _topk): the library keeps
 *     its own workspace per (device, stream), allocated stream-ordered on that stream
 *     the first time it is needed (and again, larger, when a call needs more), and
 *     reuses it for every later call on the stream, whose stream order places their
 *     kernels after the earlier ones. Up to 16 streams per device keep one; a 17th
 *     stream takes the least recently used stream's, freed stream-ordered after an
 *     event that follows that stream's last use. A call on a stream that is being
 *     captured into a HIP graph allocates and frees its workspace inside the capture
 *     instead (graph memory nodes), so a graph never refers to the cached memory. The
 *     memory is held until the process ends.
 *   - Q: [Lq, d] row-major, contiguous, same element format as docs, 16-byte aligned.
 *   - docs: rows of `stride` elements (row r starts at element r*stride), unit column
 *     stride, 16-byte aligned. Only columns 0..d-1 of rows inside documents are read;
 *     every other row or column may hold anything, NaN included.
 *   - doc_offsets, doc_lengths: int32 [B]. Row addresses are formed in 64 bits, so
 *     offset*stride may exceed 2^31 (the page widens the offset before multiplying;
 *     kernel section `_maxsim_rerank_kernel`).
 *   - scores: fp32 [B]; every element is written exactly once. It must not alias the
 *     inputs.
 *   - stream: a hipStream_t passed as void* (NULL = the default stream). Work is
 *     enqueued on it and the call returns without waiting; the caller synchronises.
 *     No entry point reads device memory on the host.
 *   - Special values: B == 0 writes nothing; Lq == 0 gives scores 0 (an empty sum);
 *     a document of length 0 gives -inf (its max is over no rows, as in the page's
 *     kernel, whose running max starts at minus infinity).
 *   - Preconditions that are not checked (checking would read device memory):
 *     0 <= doc_offsets[i], 0 <= doc_lengths[i], and doc_offsets[i] + doc_lengths[i]
 *     rows lie inside the docs allocation. Breaking them is undefined behaviour.
 *   - Return value: MAXSIM_OK, or an error code; on any error nothing has been
 *     enqueued, except MAXSIM_ERR_HIP, which reports a failed HIP call (allocation or
 *     launch) after which the contents of scores are unspecified.
 *
 * Supported envelope (MAXSIM_ERR_UNSUPPORTED outside it): 1 <= d <= 256 with
 * d % 8 == 0; Lq <= 256; stride % 8 == 0 and stride <= 2^24; Q and docs 16-byte
 * aligned (each lane reads 8 consecutive elements, 16 bytes, of one row at a time).
 */
#ifndef MAXSIM_H
#define MAXSIM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Symbols of this header are the library's only exports. */
#if defined(__GNUC__) || defined(__clang__)
#define MAXSIM_API __attribute__((visibility("default")))
#else
#define MAXSIM_API
#endif

/* Status codes. */
#define MAXSIM_OK 0
#define MAXSIM_ERR_INVALID_ARG 1 /* null pointer, negative size, stride < d, bad dtype  */
#define MAXSIM_ERR_UNSUPPORTED 2 /* outside the supported envelope above                */
#define MAXSIM_ERR_HIP 3         /* a HIP call failed (no device, allocation, launch)   */
#define MAXSIM_ERR_WORKSPACE 4   /* caller workspace null, misaligned or too small      */
#define MAXSIM_ERR_SCRATCH 5     /* batch needs more than maxsim_rerank_noalloc's scratch */

/* Element formats of Q and docs for the staged entry points. */
#define MAXSIM_F16 0
#define MAXSIM_BF16 1

/*
 * MaxSim scores, fp16 Q and docs (IEEE binary16).
 * Uses the stream's one-shot workspace (conventions above), so concurrent calls on
 * different streams do not interfere; calls from several host threads are safe.
 * Launches: for 1 <= B <= 8192 with ceil(Lq / 16) <= 8 and
 * ceil(Lq / 16) * ceil(d / 32) <= 32 (the query held in registers at once), a
 * self-scheduling kernel that cuts the docs' 16-row tiles into equal contiguous
 * ranges per wave, then a combine launch for the docs it split; otherwise the staged
 * plan, score and finish below. Both give bitwise the same scores.
 */
MAXSIM_API int maxsim_rerank(const void *Q, int32_t Lq, int32_t d,
                  const void *docs, int64_t stride,
                  const int32_t *doc_offsets, const int32_t *doc_lengths, int32_t B,
                  float *scores, void *stream);

/* Same as maxsim_rerank, bf16 Q and docs (computed in bf16, never converted). */
MAXSIM_API int maxsim_rerank_bf16(const void *Q, int32_t Lq, int32_t d,
                       const void *docs, int64_t stride,
                       const int32_t *doc_offsets, const int32_t *doc_lengths, int32_t B,
                       float *scores, void *stream);

/*
 * The same scores in a single launch, with no schedule and no scratch space: one
 * workgroup per doc, its four waves taking the doc's 16-row tiles in turn (one program
 * per doc, as in the Flash-MaxSim rerank page's kernel, section
 * `_maxsim_rerank_kernel`, with the doc's tiles shared by four waves). For small
 * batches of short docs, such as a ColBERT-style rerank of about a thousand docs of a
 * few hundred rows, the scheduled maxsim_rerank spends most of its time in its three
 * dependent launches. A launch here lasts as long as its longest doc, so long or very
 * unequal docs belong on maxsim_rerank.
 * dtype: MAXSIM_F16 or MAXSIM_BF16 (Q and docs). Scores are bitwise those of
 * maxsim_rerank: the max is exact and the sum runs in the same order. Allocates
 * nothing; can be captured in a graph.
 * Errors: as maxsim_rerank, plus MAXSIM_ERR_UNSUPPORTED when the query needs more than
 * one register group of query tiles (more than 32 16x32 query fragments: Lq > 128 at
 * d <= 128, Lq > 64 at d <= 256, in general ceil(Lq/16) * ceil(d/32) > 32 or
 * ceil(Lq/16) > 8).
 */
MAXSIM_API int maxsim_rerank_short(int dtype, const void *Q, int32_t Lq, int32_t d,
                        const void *docs, int64_t stride,
                        const int32_t *doc_offsets, const int32_t *doc_lengths, int32_t B,
                        float *scores, void *stream);

/*
 * maxsim_rerank for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. The same kernels as
 * maxsim_rerank (the self-scheduling kernel and its combine, or plan, score and
 * combine, chosen as there), so the same scores bit for bit, with a fixed scratch
 * array in device memory as their workspace instead of an allocation: 64 MiB
 * per GPU, reserved when the library is first used on that GPU and held until the
 * process ends. The call allocates nothing (no hipMalloc, hipMallocAsync or hipFree).
 * dtype: MAXSIM_F16 or MAXSIM_BF16 (Q and docs); other arguments as maxsim_rerank.
 * Every call on one GPU shares that GPU's scratch and leaves its contents there: calls
 * that overlap on one GPU (on different streams, or from several host threads before
 * the earlier call's kernels finish) race and give wrong scores; the caller must
 * serialise them, e.g. by issuing them all on one stream.
 * Limit: the schedule must fit in the 64 MiB (the self-scheduling kernel's always
 * does: 8 bytes per doc and two slots per wave). Otherwise 32 bytes per doc, plus the
 * split docs' partial maxima, at most (8 W + min(B, 8 W)) slots of 4 bytes per padded query row (W
 * the score launch's waves; about 6.3 MB at Lq 32 on MI355X, 8.5 MB for 256 docs at
 * Lq 128), i.e. about 1.8 million docs at Lq <= 32. A larger batch returns
 * MAXSIM_ERR_SCRATCH with nothing enqueued.
 */
MAXSIM_API int maxsim_rerank_noalloc(int dtype, const void *Q, int32_t Lq, int32_t d,
                          const void *docs, int64_t stride,
                          const int32_t *doc_offsets, const int32_t *doc_lengths, int32_t B,
                          float *scores, void *stream);

/*
 * Many queries in one launch ("pairs": each doc is scored against its own query).
 * The Flash-MaxSim rerank page (docs.vllm.ai, vllm.v1.pool.flash_maxsim.
 * flash_maxsim_rerank, kernel section `_maxsim_rerank_kernel`) refers to a pairs
 * kernel that widens doc offsets to 64 bits the same way, without showing it; this is
 * that batch form of the operation above, read as: doc i, with query
 * j = doc_query[i], gets
 *
 *     scores[i] = sum over q < q_lengths[j] of  max over t < doc_lengths[i] of
 *                 Qs[q_offsets[j] + q] . row(doc_offsets[i] + t)
 *
 * Qs:        [q_rows, d] row-major, contiguous: the rows of every query (device).
 * q_offsets, q_lengths: int32 [nq] (device): query j is rows
 *            [q_offsets[j], q_offsets[j] + q_lengths[j]) of Qs. Queries may overlap or
 *            share rows, and a query may be empty (its docs score 0).
 * max_lq:    an upper bound on q_lengths, 0 <= max_lq <= 256; it picks the kernel
 *            configuration, so a tight bound is faster.
 * doc_query: int32 [B] (device): the query of each doc; docs of one query need not
 *            be adjacent.
 * Other arguments as for maxsim_rerank. A doc whose query index is outside [0, nq),
 * or whose query has a negative offset or length, is longer than max_lq or reaches
 * past row q_rows, gets NaN (these are checked on the device, per doc). Each doc's
 * score equals the one maxsim_rerank gives for that query alone.
 */
MAXSIM_API int maxsim_rerank_pairs(const void *Qs, int32_t q_rows, int32_t d,
                        const int32_t *q_offsets, const int32_t *q_lengths, int32_t nq,
                        int32_t max_lq, const void *docs, int64_t stride,
                        const int32_t *doc_offsets, const int32_t *doc_lengths,
                        const int32_t *doc_query, int32_t B, float *scores, void *stream);

/* Same as maxsim_rerank_pairs, bf16 Qs and docs. */
MAXSIM_API int maxsim_rerank_pairs_bf16(const void *Qs, int32_t q_rows, int32_t d,
                             const int32_t *q_offsets, const int32_t *q_lengths, int32_t nq,
                             int32_t max_lq, const void *docs, int64_t stride,
                             const int32_t *doc_offsets, const int32_t *doc_lengths,
                             const int32_t *doc_query, int32_t B, float *scores, void *stream);

/*
 * Several queries scored against the same documents, in passes that read each doc
 * tile once for all the queries of a pass. Prior art for reading a tile once per group
 * of query rows: the request-segmented QSA scorer page (ReVolta pull request 59,
 * "Change" section), which multiplies each loaded key tile by the rows of one request
 * together. The operation is maxsim_rerank's, once per query:
 *
 *     scores[j * B + i] = MaxSim score of query j against doc i
 *
 * Qs:        [sum of q_lengths, d] (device): the queries' rows back to back, query j
 *            starting right after query j-1; contiguous, 16-byte aligned.
 * q_lengths: int32 [nq], a HOST array: rows of each query, 0 <= q_lengths[j] <= 256 (an
 *            empty query scores 0 against every doc). Read during the call only.
 * scores:    fp32 [nq, B] row-major (device).
 * Other arguments as for maxsim_rerank. Query j's scores equal, bit for bit, those
 * maxsim_rerank gives for query j alone. Uses the stream's one-shot workspace.
 */
MAXSIM_API int maxsim_rerank_multi(const void *Qs, const int32_t *q_lengths, int32_t nq, int32_t d,
                        const void *docs, int64_t stride,
                        const int32_t *doc_offsets, const int32_t *doc_lengths, int32_t B,
                        float *scores, void *stream);

/* Same as maxsim_rerank_multi, bf16 Qs and docs. */
MAXSIM_API int maxsim_rerank_multi_bf16(const void *Qs, const int32_t *q_lengths, int32_t nq,
                             int32_t d, const void *docs, int64_t stride,
                             const int32_t *doc_offsets, const int32_t *doc_lengths, int32_t B,
                             float *scores, void *stream);

/*
 * Docs stored as FP8 E4M3 ("e4m3fn": 4 exponent bits, bias 7, 3 fraction bits,
 * largest finite 448, S.1111.111 = NaN) with one fp32 scale for the whole doc tensor:
 * doc element = doc_scale * e4m3(byte). Half the bytes of fp16 docs on a path bound by
 * reading them. FP8 caches dequantised with per-tensor scales are the sparse prefill
 * pages page's (docs.vllm.ai, `stage_prefill_pages`: FP8 E4M3 pages with k/v scales).
 * The query stays fp16 (maxsim_rerank_fp8) or bf16 (maxsim_rerank_fp8_bf16); each doc
 * value is converted exactly to the query's format, products and sums are fp32 as in
 * maxsim_rerank, and the sum is multiplied by doc_scale.
 *
 * docs:      FP8 E4M3 bytes, row r at docs + r * stride (stride in bytes = elements),
 *            16-byte aligned.
 * doc_scale: finite, > 0 (MAXSIM_ERR_INVALID_ARG otherwise).
 * Envelope: d % 16 == 0 and stride % 16 == 0 (MAXSIM_ERR_UNSUPPORTED otherwise), the
 * rest as for maxsim_rerank. Quantising docs to E4M3 is the caller's step.
 */
MAXSIM_API int maxsim_rerank_fp8(const void *Q, int32_t Lq, int32_t d,
                      const void *docs, int64_t stride,
                      const int32_t *doc_offsets, const int32_t *doc_lengths, int32_t B,
                      float doc_scale, float *scores, void *stream);

/* Same as maxsim_rerank_fp8 with a bf16 query. */
MAXSIM_API int maxsim_rerank_fp8_bf16(const void *Q, int32_t Lq, int32_t d,
                           const void *docs, int64_t stride,
                           const int32_t *doc_offsets, const int32_t *doc_lengths, int32_t B,
                           float doc_scale, float *scores, void *stream);

/*
 * maxsim_rerank_fp8's operation in maxsim_rerank_short's single launch (one workgroup
 * per doc, no schedule, nothing allocated). dtype is the query format, MAXSIM_F16 or
 * MAXSIM_BF16 (MAXSIM_ERR_INVALID_ARG otherwise). Scores are bitwise those of
 * maxsim_rerank_fp8 (for dtype MAXSIM_BF16, maxsim_rerank_fp8_bf16); the FP8 envelope
 * and scale checks of maxsim_rerank_fp8 and the one-register-group limit of
 * maxsim_rerank_short apply.
 */
MAXSIM_API int maxsim_rerank_short_fp8(int dtype, const void *Q, int32_t Lq, int32_t d,
                            const void *docs, int64_t stride,
                            const int32_t *doc_offsets, const int32_t *doc_lengths, int32_t B,
                            float doc_scale, float *scores, void *stream);

/*
 * Top-k of a score array on the GPU (the rerank's consumer: the Flash-MaxSim rerank page
 * returns raw per-doc scores, `flash_maxsim_rerank_direct` return value, and the caller
 * keeps the best docs). Order: score descending; equal scores (-0 equal to +0) by
 * lower doc index; NaN after every number; so the k results are unique.
 *
 * scores:     fp32 [B] (device).
 * k:          0 <= k <= 1024 (MAXSIM_ERR_UNSUPPORTED above).
 * top_scores: fp32 [k] (device): the selected scores, bit for bit as in `scores`.
 * top_ids:    int32 [k] (device): their indices; slots past B hold (-inf, -1).
 * workspace:  device, 256-byte aligned, maxsim_topk_workspace_size(B, k) bytes.
 * Enqueued on `stream` without host synchronisation.
 */
MAXSIM_API int maxsim_topk_workspace_size(int32_t B, int32_t k, size_t *bytes);

MAXSIM_API int maxsim_topk(const float *scores, int32_t B, int32_t k, float *top_scores,
                int32_t *top_ids, void *workspace, size_t workspace_bytes, void *stream);

/*
 * maxsim_rerank followed by maxsim_topk in one call: the scores stay in the stream's
 * one-shot workspace and only the k best (score, doc index) pairs are written. Arguments
 * as for maxsim_rerank and maxsim_topk.
 */
MAXSIM_API int maxsim_rerank_topk(const void *Q, int32_t Lq, int32_t d,
                       const void *docs, int64_t stride,
                       const int32_t *doc_offsets, const int32_t *doc_lengths, int32_t B,
                       int32_t k, float *top_scores, int32_t *top_ids, void *stream);

/* Same as maxsim_rerank_topk, bf16 Q and docs. */
MAXSIM_API int maxsim_rerank_topk_bf16(const void *Q, int32_t Lq, int32_t d,
                            const void *docs, int64_t stride,
                            const int32_t *doc_offsets, const int32_t *doc_lengths, int32_t B,
                            int32_t k, float *top_scores, int32_t *top_ids, void *stream);

/*
 * The pairs batch and the shared-doc multi-query form over FP8 E4M3 docs with one scale
 * (the operations of maxsim_rerank_pairs and maxsim_rerank_multi, doc elements as in
 * maxsim_rerank_fp8). dtype is the query format, MAXSIM_F16 or MAXSIM_BF16
 * (MAXSIM_ERR_INVALID_ARG otherwise); the FP8 envelope and scale checks apply.
 */
MAXSIM_API int maxsim_rerank_pairs_fp8(int dtype, const void *Qs, int32_t q_rows, int32_t d,
                            const int32_t *q_offsets, const int32_t *q_lengths, int32_t nq,
                            int32_t max_lq, const void *docs, int64_t stride,
                            const int32_t *doc_offsets, const int32_t *doc_lengths,
                            const int32_t *doc_query, int32_t B, float doc_scale, float *scores,
                            void *stream);

MAXSIM_API int maxsim_rerank_multi_fp8(int dtype, const void *Qs, const int32_t *q_lengths,
                            int32_t nq, int32_t d, const void *docs, int64_t stride,
                            const int32_t *doc_offsets, const int32_t *doc_lengths, int32_t B,
                            float doc_scale, float *scores, void *stream);

/* Static, NUL-terminated description of a status code (never NULL). */
MAXSIM_API const char *maxsim_status_string(int status);

/*
 * Staged form of the same operation, with a caller-owned workspace, for callers that
 * manage scratch memory themselves or time the stages apart. The three stages must run
 * in order on one stream, with the same Lq, d, B and dtype; maxsim_rerank is exactly
 * plan + score + finish.
 *
 * maxsim_workspace_size: bytes of device workspace the stages need for these sizes
 *   on the current device (depends on the device's compute-unit count). Writes
 *   *bytes. Queries the current device: MAXSIM_ERR_HIP without one.
 *
 * maxsim_plan: the length-binned doc schedule. Reads doc_offsets and doc_lengths and
 *   writes the schedule into `workspace` (one kernel launch when B <= 1024, else two).
 *   The workspace must be 256-byte aligned and at least maxsim_workspace_size bytes.
 *
 * maxsim_score: the score kernel (one launch). Writes the score of every doc the
 *   schedule kept whole; for docs it split into several work items (long docs, when
 *   the batch is small for the GPU) it writes per-row partial maxima into the
 *   workspace instead. dtype is MAXSIM_F16 or MAXSIM_BF16.
 *
 * maxsim_finish: combines those partial maxima and writes the remaining scores (one
 *   launch; returns at once on the GPU when no doc was split).
 *
 * A workspace must not be shared by work that may run concurrently.
 */
MAXSIM_API int maxsim_workspace_size(int32_t Lq, int32_t d, int32_t B, size_t *bytes);

MAXSIM_API int maxsim_plan(const int32_t *doc_offsets, const int32_t *doc_lengths, int32_t B,
                int32_t Lq, int32_t d,
                void *workspace, size_t workspace_bytes, void *stream);

/*
 * maxsim_plan_pairs: the schedule of a multi-query batch (the operation of
 *   maxsim_rerank_pairs, same argument meanings). Size the workspace with
 *   maxsim_workspace_size(max_lq, d, B); then call maxsim_score and maxsim_finish with
 *   Q = Qs and Lq = max_lq. Here max_lq must be at least 1 (MAXSIM_ERR_INVALID_ARG
 *   otherwise; 1 is a valid bound when every query is empty), because maxsim_score and
 *   maxsim_finish with Lq = 0 write zeros without reading a plan.
 */
MAXSIM_API int maxsim_plan_pairs(const int32_t *doc_offsets, const int32_t *doc_lengths,
                      const int32_t *doc_query, int32_t B,
                      const int32_t *q_offsets, const int32_t *q_lengths, int32_t nq,
                      int32_t q_rows, int32_t max_lq, int32_t d,
                      void *workspace, size_t workspace_bytes, void *stream);

MAXSIM_API int maxsim_score(int dtype, const void *Q, int32_t Lq, int32_t d,
                 const void *docs, int64_t stride,
                 const int32_t *doc_offsets, const int32_t *doc_lengths, int32_t B,
                 float *scores, void *workspace, size_t workspace_bytes, void *stream);

MAXSIM_API int maxsim_finish(int dtype, int32_t Lq, int32_t d, int32_t B, float *scores,
                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * Staged score and finish for FP8 E4M3 docs (maxsim_rerank_fp8's operation; dtype is
 * the query's format, MAXSIM_F16 or MAXSIM_BF16). The plan and the workspace are the
 * same as above (maxsim_plan, maxsim_workspace_size).
 */
MAXSIM_API int maxsim_score_fp8(int dtype, const void *Q, int32_t Lq, int32_t d,
                     const void *docs, int64_t stride,
                     const int32_t *doc_offsets, const int32_t *doc_lengths, int32_t B,
                     float doc_scale, float *scores,
                     void *workspace, size_t workspace_bytes, void *stream);

MAXSIM_API int maxsim_finish_fp8(int dtype, int32_t Lq, int32_t d, int32_t B, float doc_scale,
                      float *scores, void *workspace, size_t workspace_bytes, void *stream);

/* Library version as major*10000 + minor*100 + patch. */
MAXSIM_API int maxsim_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MAXSIM_H */
