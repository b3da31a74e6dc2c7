// C ABI of the MaxSim rerank library (declared in include/maxsim.h): argument checks,
// the plan (length-binned doc schedule) kernels, the combine kernels (split docs), and
// the launches of the score kernel for every entry point: one query, a pairs batch
// (each doc with its own query), several queries over the same docs (passes of query
// tiles), and FP8 E4M3 docs. One query against at most 8192 docs takes the
// self-scheduling range kernel (maxsim_range.h) and its combine instead. The one-shot
// entry points keep a workspace per (device, stream); maxsim_rerank_noalloc uses a
// static per-device scratch. The top-k selection lives in maxsim_topk.hip.
#include "maxsim.h"

#include <string.h>

#include <mutex>
#include <vector>

#include "maxsim_common.h"
#include "maxsim_range.h"
#include "maxsim_sched.h"
#include "maxsim_topk.h"

using namespace maxsim;

// Instance lookups, one per (format, K-steps) file built from maxsim_score_inst.hip.
#define MAXSIM_DECLARE_LOOKUPS(fmt)                                                 \
    const void *maxsim_score_kernel_##fmt##_k1(int);                               \
    const void *maxsim_score_kernel_##fmt##_k2(int);                               \
    const void *maxsim_score_kernel_##fmt##_k3(int);                               \
    const void *maxsim_score_kernel_##fmt##_k4(int);                               \
    const void *maxsim_score_kernel_##fmt##_k5(int);                               \
    const void *maxsim_score_kernel_##fmt##_k6(int);                               \
    const void *maxsim_score_kernel_##fmt##_k7(int);                               \
    const void *maxsim_score_kernel_##fmt##_k8(int);                               \
    const void *maxsim_score_kernel_##fmt(int nks, int nqt)                        \
    {                                                                              \
        switch (nks) {                                                             \
        case 1: return maxsim_score_kernel_##fmt##_k1(nqt);                        \
        case 2: return maxsim_score_kernel_##fmt##_k2(nqt);                        \
        case 3: return maxsim_score_kernel_##fmt##_k3(nqt);                        \
        case 4: return maxsim_score_kernel_##fmt##_k4(nqt);                        \
        case 5: return maxsim_score_kernel_##fmt##_k5(nqt);                        \
        case 6: return maxsim_score_kernel_##fmt##_k6(nqt);                        \
        case 7: return maxsim_score_kernel_##fmt##_k7(nqt);                        \
        case 8: return maxsim_score_kernel_##fmt##_k8(nqt);                        \
        default: return nullptr;                                                   \
        }                                                                          \
    }
MAXSIM_DECLARE_LOOKUPS(f16)
MAXSIM_DECLARE_LOOKUPS(bf16)
MAXSIM_DECLARE_LOOKUPS(f16_fp8)
MAXSIM_DECLARE_LOOKUPS(bf16_fp8)
#undef MAXSIM_DECLARE_LOOKUPS

// One-launch short-doc kernels, one lookup per (format, K-steps) file.
#define MAXSIM_DECLARE_SHORT(fmt)                                                   \
    const void *maxsim_short_kernel_##fmt##_k1(int);                               \
    const void *maxsim_short_kernel_##fmt##_k2(int);                               \
    const void *maxsim_short_kernel_##fmt##_k3(int);                               \
    const void *maxsim_short_kernel_##fmt##_k4(int);                               \
    const void *maxsim_short_kernel_##fmt##_k5(int);                               \
    const void *maxsim_short_kernel_##fmt##_k6(int);                               \
    const void *maxsim_short_kernel_##fmt##_k7(int);                               \
    const void *maxsim_short_kernel_##fmt##_k8(int);                               \
    const void *maxsim_short_kernel_##fmt(int nks, int nqt)                        \
    {                                                                              \
        switch (nks) {                                                             \
        case 1: return maxsim_short_kernel_##fmt##_k1(nqt);                        \
        case 2: return maxsim_short_kernel_##fmt##_k2(nqt);                        \
        case 3: return maxsim_short_kernel_##fmt##_k3(nqt);                        \
        case 4: return maxsim_short_kernel_##fmt##_k4(nqt);                        \
        case 5: return maxsim_short_kernel_##fmt##_k5(nqt);                        \
        case 6: return maxsim_short_kernel_##fmt##_k6(nqt);                        \
        case 7: return maxsim_short_kernel_##fmt##_k7(nqt);                        \
        case 8: return maxsim_short_kernel_##fmt##_k8(nqt);                        \
        default: return nullptr;                                                   \
        }                                                                          \
    }
MAXSIM_DECLARE_SHORT(f16)
MAXSIM_DECLARE_SHORT(bf16)
MAXSIM_DECLARE_SHORT(f16_fp8)
MAXSIM_DECLARE_SHORT(bf16_fp8)
#undef MAXSIM_DECLARE_SHORT

// Self-scheduling range kernels (small single-query batches), one lookup per file.
#define MAXSIM_DECLARE_RANGE(fmt)                                                   \
    const void *maxsim_range_kernel_##fmt##_k1(int);                               \
    const void *maxsim_range_kernel_##fmt##_k2(int);                               \
    const void *maxsim_range_kernel_##fmt##_k3(int);                               \
    const void *maxsim_range_kernel_##fmt##_k4(int);                               \
    const void *maxsim_range_kernel_##fmt##_k5(int);                               \
    const void *maxsim_range_kernel_##fmt##_k6(int);                               \
    const void *maxsim_range_kernel_##fmt##_k7(int);                               \
    const void *maxsim_range_kernel_##fmt##_k8(int);                               \
    const void *maxsim_range_kernel_##fmt(int nks, int nqt)                        \
    {                                                                              \
        switch (nks) {                                                             \
        case 1: return maxsim_range_kernel_##fmt##_k1(nqt);                        \
        case 2: return maxsim_range_kernel_##fmt##_k2(nqt);                        \
        case 3: return maxsim_range_kernel_##fmt##_k3(nqt);                        \
        case 4: return maxsim_range_kernel_##fmt##_k4(nqt);                        \
        case 5: return maxsim_range_kernel_##fmt##_k5(nqt);                        \
        case 6: return maxsim_range_kernel_##fmt##_k6(nqt);                        \
        case 7: return maxsim_range_kernel_##fmt##_k7(nqt);                        \
        case 8: return maxsim_range_kernel_##fmt##_k8(nqt);                        \
        default: return nullptr;                                                   \
        }                                                                          \
    }
MAXSIM_DECLARE_RANGE(f16)
MAXSIM_DECLARE_RANGE(bf16)
MAXSIM_DECLARE_RANGE(f16_fp8)
MAXSIM_DECLARE_RANGE(bf16_fp8)
#undef MAXSIM_DECLARE_RANGE

namespace {

// ---------------------------------------------------------------- plan kernels
//
// The schedule: docs grouped by tile-count bin (bin_of), highest bin first, docs of one
// bin in index order. The score kernel hands them out in that order, so the longest
// docs start first and the short ones fill in the tail.
//
// Pass 1 (count) writes, per plan block, the number of its docs in each bin and the
// sum of their tile counts. Pass 2
// (scatter) sums those rows to get each bin's start and the block's place inside it,
// then writes every doc's descriptor at its slot. Block 0 of pass 2 also writes the
// bin totals and the total tile count to the header.

__device__ __forceinline__ uint32_t tiles_of(int32_t len)
{
    return len > 0 ? ((uint32_t)len + (kTileRows - 1)) / kTileRows : 0u;
}

__global__ void __launch_bounds__(kPlanBlock)
plan_count_kernel(const int32_t *__restrict__ lengths, int32_t B, uint32_t docs_per_block,
                  uint32_t *__restrict__ hist)
{
    __shared__ uint32_t cnt[kNumBins];
    __shared__ unsigned long long tiles;
    if (threadIdx.x < kNumBins) cnt[threadIdx.x] = 0;
    if (threadIdx.x == 0) tiles = 0;
    __syncthreads();

    const int64_t first = (int64_t)blockIdx.x * docs_per_block;
    const int64_t last = first + docs_per_block < (int64_t)B ? first + docs_per_block : (int64_t)B;
    unsigned long long my_tiles = 0;
    for (int64_t i = first + threadIdx.x; i < last; i += kPlanBlock) {
        const uint32_t nt = tiles_of(lengths[i]);
        atomicAdd(&cnt[bin_of(nt)], 1u);
        my_tiles += nt;
    }
    for (int o = 32; o > 0; o >>= 1) my_tiles += __shfl_xor(my_tiles, o);
    if ((threadIdx.x & (kWave - 1)) == 0) atomicAdd(&tiles, my_tiles);
    __syncthreads();

    uint32_t *row = hist + (size_t)blockIdx.x * kHistStride;
    if (threadIdx.x < kNumBins) row[threadIdx.x] = cnt[threadIdx.x];
    if (threadIdx.x == kNumBins) row[kNumBins] = (uint32_t)tiles;
    if (threadIdx.x == kNumBins + 1) row[kNumBins + 1] = (uint32_t)(tiles >> 32);
}

// With a single plan block (B <= kPlanBlock docs), the scatter kernel counts its own
// docs (self_count) and the count kernel is not launched.
//
// The kernel is a chain of dependent memory round trips on a small grid, so it issues
// its first round's length, offset and query loads at entry, where they overlap the
// histogram sums, and each round prefetches the next one's.
__global__ void __launch_bounds__(kPlanBlock)
plan_scatter_kernel(const int32_t *__restrict__ offsets, const int32_t *__restrict__ lengths,
                    int32_t B, uint32_t docs_per_block, const uint32_t *__restrict__ hist,
                    uint32_t nblocks, int self_count, const QueryTable qt, Header *__restrict__ hdr,
                    DocDesc *__restrict__ desc)
{
    constexpr int kRowGroups = kPlanBlock / kHistStride;  // 32
    __shared__ unsigned long long part_tot[kRowGroups][kHistStride];
    __shared__ uint32_t part_before[kRowGroups][kHistStride];
    __shared__ uint32_t bin_next[kNumBins];  // next free slot of each bin for this block
    __shared__ uint32_t wave_cnt[kPlanBlock / kWave][kNumBins];
    __shared__ uint32_t used_bins;           // bit b: some doc of the batch is in bin b

    const int64_t first = (int64_t)blockIdx.x * docs_per_block;
    const int64_t last = first + docs_per_block < (int64_t)B ? first + docs_per_block : (int64_t)B;
    struct DocIn {
        int32_t len, off, q;
    };
    auto load_doc = [&](int64_t i) {
        DocIn v{0, 0, 0};
        if (i < last) {
            v.len = lengths[i];
            v.off = offsets[i];
            v.q = qt.doc_query ? qt.doc_query[i] : 0;
        }
        return v;
    };
    DocIn cur = load_doc(first + threadIdx.x);

    if (self_count) {
        // One block holds every doc (first = 0, last = B <= kPlanBlock): bin counts and
        // tile total straight from the lengths already loaded.
        if (threadIdx.x < kHistStride) {
            part_tot[0][threadIdx.x] = 0;
            part_before[0][threadIdx.x] = 0;
        }
        __syncthreads();
        unsigned long long my_tiles = 0;
        if ((int64_t)threadIdx.x < last) {
            const uint32_t nt = tiles_of(cur.len);
            atomicAdd(&part_tot[0][bin_of(nt)], 1ull);
            my_tiles = nt;
        }
        for (int o = 32; o > 0; o >>= 1) my_tiles += __shfl_xor(my_tiles, o);
        if ((threadIdx.x & (kWave - 1)) == 0) atomicAdd(&part_tot[0][kNumBins], my_tiles);
        __syncthreads();
    } else {
    // Column c of the hist table summed over all blocks, and over blocks before ours.
    {
        const int c = threadIdx.x % kHistStride;
        const int rg = threadIdx.x / kHistStride;
        unsigned long long tot = 0;
        uint32_t before = 0;
#pragma unroll 4
        for (uint32_t k = rg; k < nblocks; k += kRowGroups) {
            const uint32_t v = hist[(size_t)k * kHistStride + c];
            tot += v;
            if (k < blockIdx.x) before += v;
        }
        part_tot[rg][c] = tot;
        part_before[rg][c] = before;
    }
    __syncthreads();
    if (threadIdx.x < kHistStride) {
        const int c = threadIdx.x;
        unsigned long long tot = 0;
        uint32_t before = 0;
        for (int rg = 0; rg < kRowGroups; ++rg) {
            tot += part_tot[rg][c];
            before += part_before[rg][c];
        }
        part_tot[0][c] = tot;
        part_before[0][c] = before;
    }
    __syncthreads();
    }
    if (threadIdx.x == 0) {
        uint32_t start = 0;  // bins in descending order
        uint32_t used = 0;
        for (int b = kNumBins - 1; b >= 0; --b) {
            bin_next[b] = start + part_before[0][b];
            start += (uint32_t)part_tot[0][b];
            if (part_tot[0][b] != 0) used |= 1u << b;
        }
        used_bins = used;
        if (blockIdx.x == 0) {
            for (int b = 0; b < kNumBins; ++b) hdr->bin_count[b] = (uint32_t)part_tot[0][b];
            hdr->total_tiles = part_tot[0][kNumBins] + (part_tot[0][kNumBins + 1] << 32);
            hdr->multi_query = qt.doc_query ? 1u : 0u;
        }
    }
    __syncthreads();

    // Stable placement: rounds of kPlanBlock consecutive docs; inside a round, rank by
    // (wave, lane) with one ballot per bin that holds docs of the batch (the others
    // hold none of this block's docs either, and their counts are never read).
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const unsigned long long lanes_below = (1ull << lane) - 1ull;
    const uint32_t used = used_bins;
    for (int64_t base = first; base < last; base += kPlanBlock) {
        const int64_t i = base + threadIdx.x;
        const bool valid = i < last;
        const DocIn in = cur;
        cur = load_doc(i + kPlanBlock);  // the next round's docs, in flight meanwhile
        const int32_t len = in.len;
        const uint32_t nt = tiles_of(len);
        const int bin = valid ? bin_of(nt) : -1;
        uint32_t rank = 0;
        for (uint32_t m_bins = used; m_bins != 0u; m_bins &= m_bins - 1u) {
            const int b = __builtin_ctz(m_bins);
            const unsigned long long m = __ballot(bin == b);
            if (lane == 0) wave_cnt[wave][b] = (uint32_t)__popcll(m);
            if (bin == b) rank = (uint32_t)__popcll(m & lanes_below);
        }
        __syncthreads();
        if (valid) {
            uint32_t slot = bin_next[bin] + rank;
            for (int w = 0; w < wave; ++w) slot += wave_cnt[w][bin];
            DocDesc dd;
            dd.doc = (int32_t)i;
            dd.offset = in.off;
            dd.length = len > 0 ? len : 0;
            dd.tiles = (int32_t)nt;
            // The doc's query, checked here once so the score kernel needs no host
            // check: an index outside [0, nq), rows outside Q or a query longer than
            // the launch was built for make the doc's score NaN.
            const int32_t q = in.q;
            int32_t q_off = 0, q_len = -1;
            if (q >= 0 && q < qt.nq) {
                q_off = qt.q_offsets ? qt.q_offsets[q] : 0;
                q_len = qt.q_lengths ? qt.q_lengths[q] : qt.Lq;
                if (q_off < 0 || q_len < 0 || q_len > qt.max_lq || (int64_t)q_off + q_len > qt.q_rows) {
                    q_off = 0;
                    q_len = -1;
                }
            }
            dd.query = q;
            dd.q_offset = q_off;
            dd.q_length = q_len;
            dd.reserved = 0;
            desc[slot] = dd;
        }
        __syncthreads();
        if (threadIdx.x < kNumBins && ((used >> threadIdx.x) & 1u)) {
            uint32_t add = 0;
            for (int w = 0; w < kPlanBlock / kWave; ++w) add += wave_cnt[w][threadIdx.x];
            bin_next[threadIdx.x] += add;
        }
        __syncthreads();
    }
}

// Split docs: max over each doc's chunk slots, then the score kernel's fixed-order sum
// (lane l adds, per query tile, rows 4 (l / 16) + 0..3; then lanes 0, 16, 32, 48), so a
// split doc's score is bitwise the one it would get unsplit. The slots are read as cells
// of 4 consecutive query rows (16 bytes) of one slot, every cell of a doc in one round of
// independent loads: a doc of at most kSoloCells cells is reduced by one wave, lanes over
// (row quad, slot), and a larger one by a whole workgroup. Docs sit in descending bin
// order and a bin's chunk count grows with the bin, so the larger docs come first.
constexpr int kSoloCells = 8 * kWave;
constexpr int kMaxQuads = kMaxLqPad / 4;
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 max4(f32x4 a, f32x4 b)
{
    f32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = a[i] > b[i] ? a[i] : b[i];
    return r;
}

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Max over slots k = k0, k0 + step, ... < K of cell `quad` (8 loads in flight).
__device__ __forceinline__ f32x4 slot_max(const float *base, int lq_pad, int quad, uint32_t k0, uint32_t step,
                                          uint32_t K)
{
    constexpr float NEG_INF = -__builtin_huge_valf();
    constexpr int U = 8;
    f32x4 m = {NEG_INF, NEG_INF, NEG_INF, NEG_INF};
    for (uint32_t k = k0; k < K; k += U * step) {
        f32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t ku = k + u * step;
            v[u] = ku < K ? *reinterpret_cast<const f32x4 *>(base + (size_t)ku * lq_pad + quad * 4)
                          : f32x4{NEG_INF, NEG_INF, NEG_INF, NEG_INF};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) m = max4(m, v[u]);
    }
    return m;
}

// One wave: the score kernel's per-query sums of the row maxima in rmax (lq_pad rows as
// quads), in its order (query tiles ascending, lane groups last), stored as it stores them.
__device__ __forceinline__ void combine_sums(const CombineArgs &a, const f32x4 *rmax, const DocDesc &dd,
                                             bool pairs, int lane)
{
    const int kgroup = lane >> 4;
    const int ntiles = a.ngroups * a.nqt;
    float lane_sum = 0.0f;
    for (int T = 0; T < ntiles; ++T) {
        int nr, end;
        if (pairs) {
            const int left = dd.q_length - T * kTileRows;
            nr = left < 0 ? 0 : (left > kTileRows ? kTileRows : left);
            end = T == ntiles - 1 ? 0 : -1;
        } else {
            nr = a.qt.rows(T);
            end = a.qt.end(T);
        }
        const f32x4 m = rmax[T * 4 + kgroup];
#pragma unroll
        for (int i = 0; i < 4; ++i) lane_sum += kgroup * 4 + i < nr ? m[i] : 0.0f;
        if (end >= 0) {
            const int ls = __builtin_bit_cast(int, lane_sum);
            const float s0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ls, 0));
            const float s1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ls, 16));
            const float s2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ls, 32));
            const float s3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ls, 48));
            // NaN for an invalid query, chosen and stored as bits (the library is
            // compiled without NaN semantics for its max steps).
            const float sum = (((s0 + s1) + s2) + s3) * a.doc_scale;
            const uint32_t v = pairs && dd.q_length < 0 ? kNaNBits : __builtin_bit_cast(uint32_t, sum);
            if (lane == 0) reinterpret_cast<uint32_t *>(a.scores)[(size_t)end * a.qt.score_stride + dd.doc] = v;
            lane_sum = 0.0f;
        }
    }
}

__global__ void __launch_bounds__(kScoreBlock)
combine_kernel(const CombineArgs a)
{
    __shared__ BinTables tab;
    __shared__ f32x4 s_red[kScoreBlock];            // per-thread maxima over its slots
    __shared__ f32x4 s_quad[kScoreWaves][kMaxQuads];  // a doc's row maxima, per wave
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = (int)__builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (wave == 0) fill_bin_tables(a.hdr, a.score_waves, a.nqt, tab, lane);
    __syncthreads();
    const LaneBins L = lane_bins(tab, lane);
    const uint32_t split = tab.split_docs;
    const int lq_pad = a.lq_pad;
    const int nquads = lq_pad / 4;
    const bool pairs = a.hdr->multi_query != 0u;
    // Workgroup docs: those of the bins whose docs have more than kSoloCells cells; the
    // lowest such bin b ends at the start of bin b - 1 (bin 0 is never split).
    const unsigned long long big =
        __ballot(lane < kNumBins && L.chunks > 1u && (uint64_t)L.chunks * (uint64_t)nquads > kSoloCells);
    uint32_t coop_end = 0;
    if (big) {
        const int b = __builtin_ctzll(big);
        coop_end = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(L.desc_start, b - 1));
    }
    if (coop_end > split) coop_end = split;

    // Workgroup docs: thread t takes cell t % nquads of the slots t / nquads + j S.
    const int t = threadIdx.x;
    for (uint32_t di = blockIdx.x; di < coop_end; di += gridDim.x) {
        const Item it = locate_doc(L, lane, di);
        const DocDesc dd = load_desc(a.desc, di);
        const float *base = a.partials + (size_t)it.first * lq_pad;
        const uint32_t S = (uint32_t)(kScoreBlock / nquads);
        const int quad = t % nquads;
        const uint32_t sl = (uint32_t)(t / nquads);
        constexpr float NEG_INF = -__builtin_huge_valf();
        f32x4 m = {NEG_INF, NEG_INF, NEG_INF, NEG_INF};
        if (sl < S) m = slot_max(base, lq_pad, quad, sl, S, it.K);
        s_red[t] = m;
        __syncthreads();
        if (t < nquads) {
            f32x4 r = s_red[t];
            for (uint32_t k = 1; k < S; ++k) r = max4(r, s_red[k * nquads + t]);
            s_quad[0][t] = r;
        }
        __syncthreads();
        if (wave == 0) combine_sums(a, s_quad[0], dd, pairs, lane);
        __syncthreads();
    }

    // One wave per doc: lane l takes cell l % nquads of the slots l / nquads + j S, or,
    // with more than 64 cells per slot, cells l and l + 64 of every slot.
    const uint32_t nw = gridDim.x * kScoreWaves;
    f32x4 *red = s_red + wave * kWave;
    f32x4 *rq = s_quad[wave];
    for (uint32_t di = coop_end + blockIdx.x * kScoreWaves + wave; di < split; di += nw) {
        const Item it = locate_doc(L, lane, di);
        const DocDesc dd = load_desc(a.desc, di);
        const float *base = a.partials + (size_t)it.first * lq_pad;
        if (nquads <= kWave) {
            const uint32_t S = (uint32_t)(kWave / nquads);
            const int quad = lane % nquads;
            const uint32_t sl = (uint32_t)(lane / nquads);
            constexpr float NEG_INF = -__builtin_huge_valf();
            f32x4 m = {NEG_INF, NEG_INF, NEG_INF, NEG_INF};
            if (sl < S) m = slot_max(base, lq_pad, quad, sl, S, it.K);
            red[lane] = m;
            wave_lds_sync();
            if (lane < nquads) {
                f32x4 r = red[lane];
                for (uint32_t k = 1; k < S; ++k) r = max4(r, red[k * nquads + lane]);
                rq[lane] = r;
            }
        } else {
            rq[lane] = slot_max(base, lq_pad, lane, 0, 1, it.K);
            if (lane + kWave < nquads) rq[lane + kWave] = slot_max(base, lq_pad, lane + kWave, 0, 1, it.K);
        }
        wave_lds_sync();
        combine_sums(a, rq, dd, pairs, lane);
        wave_lds_sync();
    }
}

}  // namespace

namespace maxsim {

// Scores of the docs a range launch split (csrc/maxsim_range.h): one wave per doc. Doc
// i's pieces are the tail slot of the wave holding its first tile and the head slots of
// the following waves up to the one holding its last tile; their max is exact, and the
// sum runs in the score kernel's fixed order (query tiles ascending, then lanes 0, 16,
// 32, 48), so the score is bitwise the one an unsplit doc gets.
__global__ void __launch_bounds__(kScoreBlock)
range_combine_kernel(const RangeCombineArgs a)
{
    __shared__ f32x4 s_red[kScoreBlock];
    __shared__ f32x4 s_quad[kScoreWaves][kMaxQuads];
    typedef __attribute__((address_space(4))) const unsigned long long ConstU64;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = (int)__builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    // The tile total and the first doc's scan entries in one round of loads.
    const int di0 = (int)blockIdx.x * kScoreWaves + wave;
    const unsigned long long T = ((ConstU64 *)a.scan)[a.B];
    unsigned long long s0 = 0, e0 = 0;
    if (di0 < a.B) {
        s0 = ((ConstU64 *)a.scan)[di0];
        e0 = ((ConstU64 *)a.scan)[di0 + 1];
    }
    if (T == 0ull) return;  // every doc empty: no pieces
    const uint32_t wact = range_active_waves(T, a.waves);
    const int kgroup = lane >> 4;
    const int lq_pad = a.nqt * kTileRows;
    const int nquads = lq_pad / 4;
    const uint32_t S = (uint32_t)(kWave / nquads);
    const int quad = lane % nquads;
    const uint32_t sl = (uint32_t)(lane / nquads);
    f32x4 *red = s_red + wave * kWave;
    f32x4 *rq = s_quad[wave];
    constexpr float NEG_INF = -__builtin_huge_valf();
    for (int di = di0; di < a.B; di += (int)gridDim.x * kScoreWaves) {
        const unsigned long long s = di == di0 ? s0 : ((ConstU64 *)a.scan)[di];
        const unsigned long long e = di == di0 ? e0 : ((ConstU64 *)a.scan)[di + 1];
        if (e <= s || e > T) continue;  // no tile (e > T: not a scan the range kernel wrote)
        const uint32_t w_lo = range_wave(s, T, wact);
        const uint32_t w_hi = range_wave(e - 1ull, T, wact);
        if (w_lo == w_hi) continue;
        const uint32_t K = w_hi - w_lo + 1u;
        // Piece k's slot: the tail slot of wave w_lo for k = 0, else the head slot of wave
        // w_lo + k. Eight loads in flight per lane before their max.
        constexpr int U = 8;
        f32x4 m = {NEG_INF, NEG_INF, NEG_INF, NEG_INF};
        if (sl < S) {
            for (uint32_t k0 = sl; k0 < K; k0 += U * S) {
                f32x4 v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const uint32_t k = k0 + u * S;
                    const uint32_t slot = k == 0u ? wact + w_lo : w_lo + k;
                    v[u] = k < K ? *reinterpret_cast<const f32x4 *>(a.partials + (size_t)slot * lq_pad + quad * 4)
                                 : f32x4{NEG_INF, NEG_INF, NEG_INF, NEG_INF};
                }
#pragma unroll
                for (int u = 0; u < U; ++u) m = max4(m, v[u]);
            }
        }
        red[lane] = m;
        wave_lds_sync();
        if (lane < nquads) {
            f32x4 r = red[lane];
            for (uint32_t k = 1; k < S; ++k) r = max4(r, red[k * nquads + lane]);
            rq[lane] = r;
        }
        wave_lds_sync();
        float lane_sum = 0.0f;
        for (int t = 0; t < a.nqt; ++t) {
            const int left = a.Lq - t * kTileRows;
            const int nr = left < 0 ? 0 : (left > kTileRows ? kTileRows : left);
            const f32x4 v = rq[t * 4 + kgroup];
#pragma unroll
            for (int i = 0; i < 4; ++i) lane_sum += kgroup * 4 + i < nr ? v[i] : 0.0f;
        }
        const int ls = __builtin_bit_cast(int, lane_sum);
        const float s0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ls, 0));
        const float s1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ls, 16));
        const float s2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ls, 32));
        const float s3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ls, 48));
        const float sum = (((s0 + s1) + s2) + s3) * a.doc_scale;
        if (lane == 0) a.scores[di] = sum;
        wave_lds_sync();
    }
}

}  // namespace maxsim

namespace {

__global__ void fill_kernel(float *__restrict__ out, int32_t n, float v)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        out[i] = v;
}

// ---------------------------------------------------------------- device facts

struct DeviceFacts {
    int cus = 0;
    int waves_per_cu = 0;  // most resident waves per CU
    int status = MAXSIM_ERR_HIP;
};

constexpr int kMaxDevices = 64;
std::once_flag g_facts_once[kMaxDevices];
DeviceFacts g_facts[kMaxDevices];

int current_facts(DeviceFacts *out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MAXSIM_ERR_HIP;
    std::call_once(g_facts_once[dev], [dev] {
        DeviceFacts f;
        int cus = 0, threads = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            hipDeviceGetAttribute(&threads, hipDeviceAttributeMaxThreadsPerMultiProcessor, dev) == hipSuccess &&
            cus > 0 && threads >= kWave) {
            f.cus = cus;
            f.waves_per_cu = threads / kWave;
            f.status = MAXSIM_OK;
        }
        g_facts[dev] = f;
    });
    *out = g_facts[dev];
    return out->status;
}

// Per-kernel occupancy (resident score workgroups per CU), cached by kernel and LDS.
struct OccEntry {
    const void *fn;
    int dev;
    size_t lds;
    int blocks;
};
std::mutex g_occ_mu;
OccEntry g_occ[512];
int g_occ_n = 0;

int score_blocks_per_cu(const void *fn, size_t lds, int *blocks)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MAXSIM_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_occ_mu);
    for (int i = 0; i < g_occ_n; ++i)
        if (g_occ[i].fn == fn && g_occ[i].dev == dev && g_occ[i].lds == lds) {
            *blocks = g_occ[i].blocks;
            return MAXSIM_OK;
        }
    if (lds > 48 * 1024 &&
        hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return MAXSIM_ERR_HIP;
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, kScoreBlock, lds) != hipSuccess || nb < 1)
        return MAXSIM_ERR_HIP;
    if (g_occ_n < (int)(sizeof(g_occ) / sizeof(g_occ[0]))) g_occ[g_occ_n++] = OccEntry{fn, dev, lds, nb};
    *blocks = nb;
    return MAXSIM_OK;
}

// ---------------------------------------------------------------- configuration

struct Config {
    int nks;      // K-steps of 32 columns: ceil(d / 32)
    int nqt;      // query tiles per register group
    int ngroups;  // register groups covering all query tiles
    int lq_pad;   // ngroups * nqt * 16
};

Config choose_config(int32_t Lq, int32_t d)
{
    Config c;
    c.nks = (d + kStepK - 1) / kStepK;
    const int tiles = (Lq + kTileRows - 1) / kTileRows;
    int max_nqt = kMaxFragsPerGroup / c.nks;
    if (max_nqt > kMaxQTilesPerGroup) max_nqt = kMaxQTilesPerGroup;
    if (tiles == 0) {
        c.ngroups = 1;
        c.nqt = 1;
    } else {
        c.ngroups = (tiles + max_nqt - 1) / max_nqt;
        c.nqt = (tiles + c.ngroups - 1) / c.ngroups;
    }
    c.lq_pad = c.ngroups * c.nqt * kTileRows;
    return c;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

size_t q_lds_bytes(const Config &c) { return (size_t)c.lq_pad * (c.nks * kStepK + 8) * 2; }

// Kernel formats: bit 0 = bf16 query (MAXSIM_BF16), bit 1 = docs stored as FP8 E4M3.
constexpr int kFmtFp8Docs = 2;

// Whether a launch stages the query tiles in LDS: whenever the padded tile fits the
// budget. The reservation depends on the configuration alone, never on the plan, so the
// score kernel's occupancy (and the chunking derived from it) is the same for every plan
// and the staged maxsim_score / maxsim_finish serve both; under a multi-query plan the
// kernel reads each wave's current query from global memory instead.
bool q_staged(const Config &c) { return q_lds_bytes(c) <= kMaxQLdsBytes; }

// Dynamic LDS of the score kernel: P LDS-DMA tile slots per wave (dma_pipe,
// dma_tile_bytes); a query of several register groups stays staged in front of them,
// while a single group's fragments are loaded once per wave at the start and the slots
// then reuse the query's LDS.
size_t score_lds_bytes(const Config &c, int32_t d, int fmt)
{
    (void)d;
    const bool fp8 = (fmt & kFmtFp8Docs) != 0;
    const size_t q = q_staged(c) ? q_lds_bytes(c) : 0;
    const int sub = score_sub(fp8);
    const size_t slots = (size_t)kScoreWaves * dma_pipe(c.nks, c.nqt, fp8, sub) * sub * dma_tile_bytes(c.nks, fp8);
    if (c.ngroups > 1) return q + slots;
    return q > slots ? q : slots;
}

const void *score_fn(int fmt, const Config &c)
{
    switch (fmt) {
    case MAXSIM_F16: return maxsim_score_kernel_f16(c.nks, c.nqt);
    case MAXSIM_BF16: return maxsim_score_kernel_bf16(c.nks, c.nqt);
    case MAXSIM_F16 | kFmtFp8Docs: return maxsim_score_kernel_f16_fp8(c.nks, c.nqt);
    case MAXSIM_BF16 | kFmtFp8Docs: return maxsim_score_kernel_bf16_fp8(c.nks, c.nqt);
    default: return nullptr;
    }
}

// scores_needed = false: no score is written (zero queries), so scores may be null.
int check_common(const void *Q, int32_t Lq, int32_t d, const void *docs, int64_t stride,
                 const int32_t *offsets, const int32_t *lengths, int32_t B, const float *scores,
                 bool scores_needed = true)
{
    if (B < 0 || Lq < 0 || d < 1 || stride < d) return MAXSIM_ERR_INVALID_ARG;
    if (B > 0 && (!docs || !offsets || !lengths || (scores_needed && !scores))) return MAXSIM_ERR_INVALID_ARG;
    if (B > 0 && Lq > 0 && !Q) return MAXSIM_ERR_INVALID_ARG;
    if (d > kMaxD || d % 8 != 0 || Lq > kMaxLq) return MAXSIM_ERR_UNSUPPORTED;
    if (stride % 8 != 0 || stride > kMaxStride) return MAXSIM_ERR_UNSUPPORTED;
    if (B > 0 && !aligned16(docs)) return MAXSIM_ERR_UNSUPPORTED;
    if (B > 0 && Lq > 0 && !aligned16(Q)) return MAXSIM_ERR_UNSUPPORTED;
    if (B > 0 && (((uintptr_t)offsets | (uintptr_t)lengths | (uintptr_t)scores) & 3u))
        return MAXSIM_ERR_INVALID_ARG;
    return MAXSIM_OK;
}

int workspace_layout(int32_t Lq, int32_t d, int32_t B, Layout *L)
{
    DeviceFacts f;
    if (current_facts(&f) != MAXSIM_OK) return MAXSIM_ERR_HIP;
    const Config c = choose_config(Lq, d);
    *L = make_layout(c.lq_pad, B, (uint32_t)(f.cus * f.waves_per_cu));
    return MAXSIM_OK;
}

// The query table of a launch over one query of Lq rows: every doc takes query 0.
QueryTable single_query(int32_t Lq)
{
    QueryTable qt;
    qt.doc_query = nullptr;
    qt.q_offsets = nullptr;
    qt.q_lengths = nullptr;
    qt.nq = 1;
    qt.q_rows = Lq;
    qt.Lq = Lq;
    qt.max_lq = Lq;
    return qt;
}

int launch_plan(const int32_t *offsets, const int32_t *lengths, int32_t B, const Layout &L,
                const QueryTable &qt, char *ws, hipStream_t stream)
{
    uint32_t *hist = reinterpret_cast<uint32_t *>(ws + L.hist);
    Header *hdr = reinterpret_cast<Header *>(ws + L.header);
    DocDesc *desc = reinterpret_cast<DocDesc *>(ws + L.desc);
    const int self_count = L.plan_blocks == 1 && (uint32_t)B <= (uint32_t)kPlanBlock;
    if (!self_count) {
        hipLaunchKernelGGL(plan_count_kernel, dim3(L.plan_blocks), dim3(kPlanBlock), 0, stream,
                           lengths, B, L.docs_per_plan_block, hist);
        if (hipGetLastError() != hipSuccess) return MAXSIM_ERR_HIP;
    }
    hipLaunchKernelGGL(plan_scatter_kernel, dim3(L.plan_blocks), dim3(kPlanBlock), 0, stream,
                       offsets, lengths, B, L.docs_per_plan_block, hist, L.plan_blocks, self_count,
                       qt, hdr, desc);
    if (hipGetLastError() != hipSuccess) return MAXSIM_ERR_HIP;
    return MAXSIM_OK;
}

int launch_fill(float *scores, int32_t B, float v, hipStream_t stream)
{
    const int blocks = (B + 255) / 256 < 1024 ? (B + 255) / 256 : 1024;
    hipLaunchKernelGGL(fill_kernel, dim3(blocks), dim3(256), 0, stream, scores, B, v);
    return hipGetLastError() == hipSuccess ? MAXSIM_OK : MAXSIM_ERR_HIP;
}

// Query tiles of one query of Lq rows, whose scores are one row.
QueryTiles single_tiles(int32_t Lq)
{
    QueryTiles t{};
    t.score_stride = 0;
    const int nt = (Lq + kTileRows - 1) / kTileRows;
    for (int T = 0; T < kMaxQTiles; ++T) {
        const int left = Lq - T * kTileRows;
        t.set(T, T < nt ? T * kTileRows : 0, left <= 0 ? 0 : (left > kTileRows ? kTileRows : left),
              T == nt - 1 ? 0 : -1);
    }
    return t;
}

// Lq: rows of the one query, the longest query of a pairs plan, or 16 x the query
// tiles of a launch over several queries sharing the docs (qt describes them).
// fmt: kernel format (query format | kFmtFp8Docs); doc_scale multiplies FP8 doc sums.
int launch_score(int fmt, const void *Q, int32_t Lq, int32_t d, const void *docs, int64_t stride,
                 float *scores, const Layout &L, char *ws, const QueryTiles &qt, float doc_scale,
                 hipStream_t stream)
{
    const Config c = choose_config(Lq, d);
    if (c.lq_pad > kMaxLqPad || c.nqt * c.nks > kMaxFragsPerGroup) return MAXSIM_ERR_UNSUPPORTED;
    const void *fn = score_fn(fmt, c);
    if (!fn) return MAXSIM_ERR_UNSUPPORTED;
    const bool q_in_lds = q_staged(c);
    const size_t lds = score_lds_bytes(c, d, fmt);
    int per_cu = 0;
    if (score_blocks_per_cu(fn, lds, &per_cu) != MAXSIM_OK) return MAXSIM_ERR_HIP;
    DeviceFacts f;
    if (current_facts(&f) != MAXSIM_OK) return MAXSIM_ERR_HIP;
    ScoreArgs a;
    a.Q = static_cast<const uint16_t *>(Q);
    a.docs = static_cast<const char *>(docs);
    a.stride_bytes = stride * ((fmt & kFmtFp8Docs) ? 1 : 2);
    a.hdr = reinterpret_cast<const Header *>(ws + L.header);
    a.desc = reinterpret_cast<const DocDesc *>(ws + L.desc);
    a.partials = reinterpret_cast<float *>(ws + L.partials);
    a.scores = scores;
    a.d = d;
    a.ngroups = c.ngroups;
    a.lq_pad = c.lq_pad;
    a.q_in_lds = q_in_lds ? 1 : 0;
    a.qt = qt;
    a.doc_scale = doc_scale;
    void *args[] = {&a};
    const dim3 grid((unsigned)(f.cus * per_cu));
    if (hipLaunchKernel(fn, grid, dim3(kScoreBlock), args, lds, stream) != hipSuccess) return MAXSIM_ERR_HIP;
    return hipGetLastError() == hipSuccess ? MAXSIM_OK : MAXSIM_ERR_HIP;
}

// The combine kernel recomputes the score kernel's chunking, which depends on that
// launch's wave count: the same instance and occupancy are looked up here.
int launch_finish(int fmt, int32_t Lq, int32_t d, float *scores, const Layout &L, char *ws,
                  const QueryTiles &qt, float doc_scale, hipStream_t stream)
{
    const Config c = choose_config(Lq, d);
    if (c.lq_pad > kMaxLqPad || c.nqt * c.nks > kMaxFragsPerGroup) return MAXSIM_ERR_UNSUPPORTED;
    const void *fn = score_fn(fmt, c);
    if (!fn) return MAXSIM_ERR_UNSUPPORTED;
    int per_cu = 0;
    if (score_blocks_per_cu(fn, score_lds_bytes(c, d, fmt), &per_cu) != MAXSIM_OK) return MAXSIM_ERR_HIP;
    DeviceFacts f;
    if (current_facts(&f) != MAXSIM_OK) return MAXSIM_ERR_HIP;
    CombineArgs ca;
    ca.hdr = reinterpret_cast<const Header *>(ws + L.header);
    ca.desc = reinterpret_cast<const DocDesc *>(ws + L.desc);
    ca.partials = reinterpret_cast<const float *>(ws + L.partials);
    ca.scores = scores;
    ca.score_waves = (uint32_t)(f.cus * per_cu * kScoreWaves);
    ca.nqt = c.nqt;
    ca.ngroups = c.ngroups;
    ca.lq_pad = c.lq_pad;
    ca.qt = qt;
    ca.doc_scale = (fmt & kFmtFp8Docs) ? doc_scale : 1.0f;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)f.cus * 8u), dim3(kScoreBlock), 0, stream, ca);
    return hipGetLastError() == hipSuccess ? MAXSIM_OK : MAXSIM_ERR_HIP;
}

// ---------------------------------------------------------------- one-shot workspaces
//
// The one-shot entry points need scratch space for the schedule and for the per-row
// maxima of split docs. Taken from hipMallocAsync on every call, that memory is mapped
// again on every call once the default pool has given it back, which it does at every
// synchronisation (a 256-doc rerank with a sync per call took 375 us that way, against
// 56 us with a caller-owned workspace). So the library keeps one workspace per (device,
// stream) it is called on and reuses it: stream order puts every later call's kernels
// after the earlier calls' kernels that used it. A workspace that is too small is freed
// and allocated again, both stream-ordered on its stream.
//
// A call on a stream that is being captured into a graph does not use it: its
// workspace is allocated and freed inside the capture (graph memory nodes), so a graph
// never refers to memory that an eager call reuses or that the cache frees.
//
// kWsSlots streams per device keep a workspace; a new stream takes the least recently
// used slot. The memory of an evicted slot is freed on the new stream after that stream
// waits for an event recorded after the slot's last use, so the free is ordered after
// every kernel that read or wrote it. One lock covers the lookup and the enqueueing of a
// whole call (host side only: the GPU work of different streams still overlaps).
constexpr int kWsSlots = 16;

struct WsSlot {
    hipStream_t stream = nullptr;
    void *buf = nullptr;
    size_t bytes = 0;
    hipEvent_t done = nullptr;  // recorded on `stream` after the last call that used buf
    uint64_t last = 0;          // use stamp; 0: the slot is free
};

std::mutex g_ws_mu;
WsSlot g_ws[kMaxDevices][kWsSlots];
uint64_t g_ws_clock = 0;

// Whether work enqueued on s now would be captured. An error of the query (for instance
// on the legacy default stream while another stream captures) counts as capturing: the
// per-call path needs nothing from the cache.
bool stream_capturing(hipStream_t s)
{
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &st) != hipSuccess) {
        (void)hipGetLastError();  // do not leave the failed query as the last error
        return true;
    }
    return st != hipStreamCaptureStatusNone;
}

// Under g_ws_mu: the slot of (current device, s), holding at least `need` bytes.
int ws_acquire(hipStream_t s, size_t need, WsSlot **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MAXSIM_ERR_HIP;
    WsSlot *tab = g_ws[dev];
    WsSlot *slot = nullptr;
    for (int i = 0; i < kWsSlots && !slot; ++i)
        if (tab[i].last != 0 && tab[i].stream == s) slot = &tab[i];
    if (!slot) {
        slot = &tab[0];  // free slots (last == 0) first, then the least recently used
        for (int i = 1; i < kWsSlots; ++i)
            if (tab[i].last < slot->last) slot = &tab[i];
        if (slot->buf) {
            if (hipStreamWaitEvent(s, slot->done, 0) != hipSuccess) return MAXSIM_ERR_HIP;
            if (hipFreeAsync(slot->buf, s) != hipSuccess) return MAXSIM_ERR_HIP;
            slot->buf = nullptr;
            slot->bytes = 0;
        }
        if (!slot->done && hipEventCreateWithFlags(&slot->done, hipEventDisableTiming) != hipSuccess) {
            slot->done = nullptr;
            return MAXSIM_ERR_HIP;
        }
        slot->stream = s;
    }
    slot->last = ++g_ws_clock;
    if (slot->bytes < need) {
        if (slot->buf) {
            if (hipFreeAsync(slot->buf, s) != hipSuccess) return MAXSIM_ERR_HIP;
            slot->buf = nullptr;
            slot->bytes = 0;
        }
        // A quarter more than asked, in whole MiB, so that a slowly growing batch does
        // not reallocate on every call.
        const size_t want = ((need + need / 4) + ((size_t)1 << 20) - 1) & ~(((size_t)1 << 20) - 1);
        void *p = nullptr;
        if (hipMallocAsync(&p, want, s) != hipSuccess) return MAXSIM_ERR_HIP;
        slot->buf = p;
        slot->bytes = want;
    }
    *out = slot;
    return MAXSIM_OK;
}

// Runs enqueue(w) with w a 256-byte aligned workspace of at least `need` bytes on s.
template <class F>
int with_workspace(hipStream_t s, size_t need, F &&enqueue)
{
    if (need == 0) need = 256;
    if (stream_capturing(s)) {
        void *ws = nullptr;
        if (hipMallocAsync(&ws, need, s) != hipSuccess) return MAXSIM_ERR_HIP;
        int rc = enqueue(static_cast<char *>(ws));
        if (hipFreeAsync(ws, s) != hipSuccess && rc == MAXSIM_OK) rc = MAXSIM_ERR_HIP;
        return rc;
    }
    std::lock_guard<std::mutex> lock(g_ws_mu);
    WsSlot *slot = nullptr;
    int rc = ws_acquire(s, need, &slot);
    if (rc != MAXSIM_OK) return rc;
    rc = enqueue(static_cast<char *>(slot->buf));
    if (hipEventRecord(slot->done, s) != hipSuccess && rc == MAXSIM_OK) rc = MAXSIM_ERR_HIP;
    return rc;
}

// ---------------------------------------------------------------- static scratch
//
// maxsim_rerank_noalloc's workspace: a fixed array in device memory. Each GPU the
// library runs on holds its own copy, at its own address, until the process ends. In
// host code the array's name is only a stand-in for it, never an address: a GPU's copy
// is reached through the pointer hipGetSymbolAddress returns, taken once per device with
// that device current. Every call on a GPU shares that GPU's copy, so calls that overlap
// on one GPU race (the caller serialises them). Nothing in it needs to start at zero:
// the plan kernels write the header, the histogram rows and every descriptor before the
// score and combine kernels read them, and a split doc's slots are written by its chunks
// before the combine kernel reads them.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

std::once_flag g_scratch_once[kMaxDevices];
char *g_scratch_ptr[kMaxDevices];
int g_scratch_status[kMaxDevices];

int scratch_of_current_device(char **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MAXSIM_ERR_HIP;
    std::call_once(g_scratch_once[dev], [dev] {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e == hipSuccess && p) {
            g_scratch_ptr[dev] = static_cast<char *>(p);
            g_scratch_status[dev] = MAXSIM_OK;
        } else {
            (void)hipGetLastError();
            g_scratch_ptr[dev] = nullptr;
            g_scratch_status[dev] = MAXSIM_ERR_HIP;
        }
    });
    *out = g_scratch_ptr[dev];
    return g_scratch_status[dev];
}

// Waves of the score launch of format fmt for (Lq, d): the grid launch_score uses
// (CUs x resident workgroups of that instance x 4 waves), from the same occupancy query.
int score_launch_waves(int fmt, int32_t Lq, int32_t d, uint32_t *waves)
{
    const Config c = choose_config(Lq, d);
    if (c.lq_pad > kMaxLqPad || c.nqt * c.nks > kMaxFragsPerGroup) return MAXSIM_ERR_UNSUPPORTED;
    const void *fn = score_fn(fmt, c);
    if (!fn) return MAXSIM_ERR_UNSUPPORTED;
    int per_cu = 0;
    if (score_blocks_per_cu(fn, score_lds_bytes(c, d, fmt), &per_cu) != MAXSIM_OK) return MAXSIM_ERR_HIP;
    DeviceFacts f;
    if (current_facts(&f) != MAXSIM_OK) return MAXSIM_ERR_HIP;
    *waves = (uint32_t)(f.cus * per_cu * kScoreWaves);
    return MAXSIM_OK;
}

// ---------------------------------------------------------------- range launches
//
// A single-query batch of at most kRangeMaxDocs (8192) docs whose query fits one register group
// runs as two launches: the self-scheduling range kernel (csrc/maxsim_range.h), which
// cuts the docs' tiles into equal contiguous ranges per wave, and range_combine_kernel
// for the docs it split. No plan launch. Its workspace holds the tile prefix sums (the
// last is the tile total) and 2 W slots of per-row maxima.
bool range_eligible(int32_t Lq, int32_t d, int32_t B)
{
    if (B < 1 || B > kRangeMaxDocs || Lq < 1) return false;
    if (choose_config(Lq, d).ngroups != 1) return false;
    // The range kernel's grid has a wave for each of the prologue's 256 doc blocks (at
    // least one workgroup of 4 waves on each of 64 compute units); a smaller device
    // takes the scheduled path.
    DeviceFacts f;
    return current_facts(&f) == MAXSIM_OK && f.cus * kScoreWaves >= kScoreBlock;
}

const void *range_fn(int fmt, const Config &c)
{
    switch (fmt) {
    case MAXSIM_F16: return maxsim_range_kernel_f16(c.nks, c.nqt);
    case MAXSIM_BF16: return maxsim_range_kernel_bf16(c.nks, c.nqt);
    case MAXSIM_F16 | kFmtFp8Docs: return maxsim_range_kernel_f16_fp8(c.nks, c.nqt);
    case MAXSIM_BF16 | kFmtFp8Docs: return maxsim_range_kernel_bf16_fp8(c.nks, c.nqt);
    default: return nullptr;
    }
}

// Dynamic LDS: the query tile, then (in the prologue) the doc lengths, 1024 per 4-doc
// chunk a thread takes, and the doc offsets in 256-doc pieces where they fit without
// growing the allocation (always for at most 1024 docs: 4 KB); then the same tile slots
// as the score kernel over all of it.
struct RangeLds {
    size_t len, off, bytes;  // byte offsets of the lengths and offsets (off 0: not in LDS); size
};

RangeLds range_lds(const Config &c, int fmt, int32_t B)
{
    const bool fp8 = (fmt & kFmtFp8Docs) != 0;
    RangeLds r;
    r.len = (q_lds_bytes(c) + 15) & ~size_t(15);
    const size_t nch = ((size_t)B + kRangeDocsPerChunkRow - 1) / kRangeDocsPerChunkRow;
    const size_t pro = r.len + 4 * kRangeDocsPerChunkRow * nch;
    const size_t off_bytes = (size_t)4 * 4 * kWave * (((size_t)B + 4 * kWave - 1) / (4 * kWave));
    const size_t slots = (size_t)kScoreWaves * dma_pipe(c.nks, c.nqt, fp8) * dma_tile_bytes(c.nks, fp8);
    const size_t base = pro > slots ? pro : slots;
    r.off = 0;
    r.bytes = base;
    if (pro + off_bytes <= base || B <= kRangeDocsPerChunkRow) {
        r.off = pro;
        r.bytes = pro + off_bytes > base ? pro + off_bytes : base;
    }
    return r;
}

struct RangePlan {
    const void *fn;
    size_t lds;
    uint32_t blocks;
    size_t scan, partials, bytes;  // workspace layout
};

int range_plan(int fmt, int32_t Lq, int32_t d, int32_t B, RangePlan *rp)
{
    const Config c = choose_config(Lq, d);
    if (c.ngroups != 1 || c.nqt * c.nks > kMaxFragsPerGroup) return MAXSIM_ERR_UNSUPPORTED;
    rp->fn = range_fn(fmt, c);
    if (!rp->fn) return MAXSIM_ERR_UNSUPPORTED;
    rp->lds = range_lds(c, fmt, B).bytes;
    int per_cu = 0;
    if (score_blocks_per_cu(rp->fn, rp->lds, &per_cu) != MAXSIM_OK) return MAXSIM_ERR_HIP;
    DeviceFacts f;
    if (current_facts(&f) != MAXSIM_OK) return MAXSIM_ERR_HIP;
    // (W < 2^16 keeps the cut's 64-bit products in range: the grid is at most 16383
    // workgroups, more than any device holds at once.)
    const long long blocks = (long long)f.cus * per_cu;
    rp->blocks = (uint32_t)(blocks < 16383 ? blocks : 16383);
    const size_t waves = (size_t)rp->blocks * kScoreWaves;
    rp->scan = 0;
    rp->partials = align256((size_t)8 * (B + 1));
    rp->bytes = align256(rp->partials + 2 * waves * (size_t)c.lq_pad * 4);
    return MAXSIM_OK;
}

int enqueue_range(int fmt, const RangePlan &rp, const void *Q, int32_t Lq, int32_t d, const void *docs,
                  int64_t stride, const int32_t *offsets, const int32_t *lengths, int32_t B, float *scores,
                  float doc_scale, char *w, hipStream_t stream)
{
    const Config c = choose_config(Lq, d);
    const bool fp8 = (fmt & kFmtFp8Docs) != 0;
    RangeArgs a;
    a.Q = static_cast<const uint16_t *>(Q);
    a.docs = static_cast<const char *>(docs);
    a.stride_bytes = stride * (fp8 ? 1 : 2);
    a.offsets = offsets;
    a.lengths = lengths;
    a.scores = scores;
    a.scan = reinterpret_cast<unsigned long long *>(w + rp.scan);
    a.partials = reinterpret_cast<float *>(w + rp.partials);
    a.B = B;
    a.d = d;
    a.Lq = Lq;
    const RangeLds rl = range_lds(c, fmt, B);
    a.len_lds = (uint32_t)rl.len;
    a.off_lds = (uint32_t)rl.off;
    a.doc_scale = fp8 ? doc_scale : 1.0f;
    void *args[] = {&a};
    if (hipLaunchKernel(rp.fn, dim3(rp.blocks), dim3(kScoreBlock), args, rp.lds, stream) != hipSuccess)
        return MAXSIM_ERR_HIP;
    if (hipGetLastError() != hipSuccess) return MAXSIM_ERR_HIP;
    RangeCombineArgs ca;
    ca.scan = a.scan;
    ca.partials = a.partials;
    ca.scores = scores;
    ca.B = B;
    ca.Lq = Lq;
    ca.nqt = c.nqt;
    ca.waves = rp.blocks * kScoreWaves;
    ca.doc_scale = a.doc_scale;
    hipLaunchKernelGGL(range_combine_kernel, dim3((unsigned)((B + kScoreWaves - 1) / kScoreWaves)),
                       dim3(kScoreBlock), 0, stream, ca);
    return hipGetLastError() == hipSuccess ? MAXSIM_OK : MAXSIM_ERR_HIP;
}

// Plan, score and combine into the workspace w (layout L); qt.max_lq sizes the kernel
// configuration.
int enqueue_all(int fmt, const void *Q, const QueryTable &qt, int32_t d, const void *docs, int64_t stride,
                const int32_t *offsets, const int32_t *lengths, int32_t B, float *scores, float doc_scale,
                const Layout &L, char *w, hipStream_t stream)
{
    const QueryTiles tiles = single_tiles(qt.max_lq);  // (a pairs plan ignores them)
    int rc = launch_plan(offsets, lengths, B, L, qt, w, stream);
    if (rc == MAXSIM_OK)
        rc = launch_score(fmt, Q, qt.max_lq, d, docs, stride, scores, L, w, tiles, doc_scale, stream);
    if (rc == MAXSIM_OK) rc = launch_finish(fmt, qt.max_lq, d, scores, L, w, tiles, doc_scale, stream);
    return rc;
}

// Plan, score and combine with the stream's one-shot workspace.
int run_all(int fmt, const void *Q, const QueryTable &qt, int32_t d, const void *docs,
            int64_t stride, const int32_t *offsets, const int32_t *lengths, int32_t B, float *scores,
            float doc_scale, hipStream_t stream)
{
    Layout L;
    if (workspace_layout(qt.max_lq, d, B, &L) != MAXSIM_OK) return MAXSIM_ERR_HIP;
    return with_workspace(stream, L.total, [&](char *w) {
        return enqueue_all(fmt, Q, qt, d, docs, stride, offsets, lengths, B, scores, doc_scale, L, w, stream);
    });
}

int rerank(int dtype, const void *Q, int32_t Lq, int32_t d, const void *docs, int64_t stride,
           const int32_t *offsets, const int32_t *lengths, int32_t B, float *scores, void *stream_ptr)
{
    const int st = check_common(Q, Lq, d, docs, stride, offsets, lengths, B, scores);
    if (st != MAXSIM_OK) return st;
    if (B == 0) return MAXSIM_OK;
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    if (Lq == 0) return launch_fill(scores, B, 0.0f, stream);
    if (range_eligible(Lq, d, B)) {
        RangePlan rp;
        const int rc = range_plan(dtype, Lq, d, B, &rp);
        if (rc != MAXSIM_OK) return rc;
        return with_workspace(stream, rp.bytes, [&](char *w) {
            return enqueue_range(dtype, rp, Q, Lq, d, docs, stride, offsets, lengths, B, scores, 1.0f, w, stream);
        });
    }
    return run_all(dtype, Q, single_query(Lq), d, docs, stride, offsets, lengths, B, scores, 1.0f, stream);
}

// maxsim_rerank's plan, score and combine with the static scratch as the workspace. Its
// partial-maxima slots are sized with the score launch's own wave count (the bound grows
// with W, so the launch's W is enough), which keeps the schedule of a large batch well
// inside the array.
int rerank_noalloc(int dtype, const void *Q, int32_t Lq, int32_t d, const void *docs, int64_t stride,
                   const int32_t *offsets, const int32_t *lengths, int32_t B, float *scores, void *stream_ptr)
{
    if (dtype != MAXSIM_F16 && dtype != MAXSIM_BF16) return MAXSIM_ERR_INVALID_ARG;
    const int st = check_common(Q, Lq, d, docs, stride, offsets, lengths, B, scores);
    if (st != MAXSIM_OK) return st;
    if (B == 0) return MAXSIM_OK;
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    if (Lq == 0) return launch_fill(scores, B, 0.0f, stream);
    if (range_eligible(Lq, d, B)) {
        RangePlan rp;
        int rc = range_plan(dtype, Lq, d, B, &rp);
        if (rc != MAXSIM_OK) return rc;
        if (rp.bytes > kScratchBytes) return MAXSIM_ERR_SCRATCH;
        char *w = nullptr;
        if ((rc = scratch_of_current_device(&w)) != MAXSIM_OK) return rc;
        return enqueue_range(dtype, rp, Q, Lq, d, docs, stride, offsets, lengths, B, scores, 1.0f, w, stream);
    }
    uint32_t waves = 0;
    int rc = score_launch_waves(dtype, Lq, d, &waves);
    if (rc != MAXSIM_OK) return rc;
    const Layout L = make_layout(choose_config(Lq, d).lq_pad, B, waves);
    if (L.total > kScratchBytes) return MAXSIM_ERR_SCRATCH;
    char *w = nullptr;
    if ((rc = scratch_of_current_device(&w)) != MAXSIM_OK) return rc;
    return enqueue_all(dtype, Q, single_query(Lq), d, docs, stride, offsets, lengths, B, scores, 1.0f, L, w,
                       stream);
}

// A usable scale of FP8 docs: positive and at most 3.4e38 (so finite), never NaN. The
// test runs on the bit pattern: a positive float's bits grow with its value, and zero,
// negative values, infinity and NaN all fall outside (0, bits(3.4e38)]. No compare of
// floats is involved, so no assumption a compiler may make about NaN can change it.
bool valid_scale(float s)
{
    uint32_t bits;
    memcpy(&bits, &s, sizeof bits);
    constexpr uint32_t kMaxScaleBits = 0x7F7FC99Eu;  // 3.4e38f
    return bits - 1u < kMaxScaleBits;
}

// Extra checks for docs stored as FP8 E4M3 bytes: whole 16-byte chunks per row and a
// finite positive scale.
int check_fp8(int32_t d, int64_t stride, float doc_scale)
{
    if (!valid_scale(doc_scale)) return MAXSIM_ERR_INVALID_ARG;
    if (d % 16 != 0 || stride % 16 != 0) return MAXSIM_ERR_UNSUPPORTED;
    return MAXSIM_OK;
}

// One launch, one workgroup per doc (csrc/maxsim_short.h); the query must fit one
// register group. fmt: query format, | kFmtFp8Docs for FP8 E4M3 docs with doc_scale.
int rerank_short(int fmt, const void *Q, int32_t Lq, int32_t d, const void *docs, int64_t stride,
                 const int32_t *offsets, const int32_t *lengths, int32_t B, float doc_scale, float *scores,
                 void *stream_ptr)
{
    const int dtype = fmt & ~kFmtFp8Docs;
    const bool fp8 = (fmt & kFmtFp8Docs) != 0;
    if (dtype != MAXSIM_F16 && dtype != MAXSIM_BF16) return MAXSIM_ERR_INVALID_ARG;
    int st = check_common(Q, Lq, d, docs, stride, offsets, lengths, B, scores);
    if (st != MAXSIM_OK) return st;
    if (fp8 && (st = check_fp8(d, stride, doc_scale)) != MAXSIM_OK) return st;
    const Config c = choose_config(Lq, d);
    if (Lq > 0 && c.ngroups != 1) return MAXSIM_ERR_UNSUPPORTED;
    if (B == 0) return MAXSIM_OK;
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    if (Lq == 0) return launch_fill(scores, B, 0.0f, stream);
    const void *fn = fp8 ? (dtype == MAXSIM_BF16 ? maxsim_short_kernel_bf16_fp8(c.nks, c.nqt)
                                                 : maxsim_short_kernel_f16_fp8(c.nks, c.nqt))
                         : (dtype == MAXSIM_BF16 ? maxsim_short_kernel_bf16(c.nks, c.nqt)
                                                 : maxsim_short_kernel_f16(c.nks, c.nqt));
    if (!fn) return MAXSIM_ERR_UNSUPPORTED;
    // The query tile first, then the tile slots over it (the same LDS-DMA rule as the
    // scheduled kernel).
    const size_t slots = (size_t)kScoreWaves * dma_pipe(c.nks, c.nqt, fp8) * dma_tile_bytes(c.nks, fp8);
    const size_t lds = q_lds_bytes(c) > slots ? q_lds_bytes(c) : slots;
    int per_cu = 0;
    if (score_blocks_per_cu(fn, lds, &per_cu) != MAXSIM_OK) return MAXSIM_ERR_HIP;
    DeviceFacts f;
    if (current_facts(&f) != MAXSIM_OK) return MAXSIM_ERR_HIP;
    // One workgroup per doc, up to four rounds of resident workgroups (each stages the
    // query once, then takes docs b, b + grid, ...).
    const int64_t cap = (int64_t)f.cus * per_cu * 4;
    const unsigned grid = (unsigned)((int64_t)B < cap ? (int64_t)B : cap);
    ShortArgs a;
    a.Q = static_cast<const uint16_t *>(Q);
    a.docs = static_cast<const char *>(docs);
    a.stride_bytes = fp8 ? stride : stride * 2;
    a.offsets = offsets;
    a.lengths = lengths;
    a.scores = scores;
    a.B = B;
    a.d = d;
    a.Lq = Lq;
    a.doc_scale = fp8 ? doc_scale : 1.0f;
    void *args[] = {&a};
    if (hipLaunchKernel(fn, dim3(grid), dim3(kScoreBlock), args, lds, stream) != hipSuccess) return MAXSIM_ERR_HIP;
    return hipGetLastError() == hipSuccess ? MAXSIM_OK : MAXSIM_ERR_HIP;
}

// Scores into the stream's one-shot workspace, then the device top-k of them.
int rerank_topk(int dtype, const void *Q, int32_t Lq, int32_t d, const void *docs, int64_t stride,
                const int32_t *offsets, const int32_t *lengths, int32_t B, int32_t k, float *top_scores,
                int32_t *top_ids, void *stream_ptr)
{
    if (k < 0) return MAXSIM_ERR_INVALID_ARG;
    if (k > kTopkMaxK) return MAXSIM_ERR_UNSUPPORTED;
    if (k > 0 && (!top_scores || !top_ids)) return MAXSIM_ERR_INVALID_ARG;
    if (((uintptr_t)top_scores | (uintptr_t)top_ids) & 3u) return MAXSIM_ERR_INVALID_ARG;
    // The score arguments are checked as maxsim_rerank checks them (scores is internal).
    int st = check_common(Q, Lq, d, docs, stride, offsets, lengths, B, nullptr, false);
    if (st != MAXSIM_OK) return st;
    if (k == 0) return MAXSIM_OK;
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    // Workspace: the rerank's (when there is one), then the scores, then the top-k's.
    Layout L{};
    RangePlan rp{};
    const bool ranked = B > 0 && Lq > 0;
    const bool ranged = ranked && range_eligible(Lq, d, B);
    if (ranged) {
        const int rc = range_plan(dtype, Lq, d, B, &rp);
        if (rc != MAXSIM_OK) return rc;
    } else if (ranked && workspace_layout(Lq, d, B, &L) != MAXSIM_OK) {
        return MAXSIM_ERR_HIP;
    }
    const size_t score_at = ranged ? rp.bytes : (ranked ? L.total : 0);
    const size_t score_bytes = ((size_t)(B > 0 ? B : 1) * 4 + 255) & ~size_t(255);
    const size_t need = score_at + score_bytes + topk_workspace_bytes(B, k);
    return with_workspace(stream, need, [&](char *w) {
        float *scores = reinterpret_cast<float *>(w + score_at);
        int rc = MAXSIM_OK;
        if (B > 0) {
            if (!ranked)
                rc = launch_fill(scores, B, 0.0f, stream);
            else if (ranged)
                rc = enqueue_range(dtype, rp, Q, Lq, d, docs, stride, offsets, lengths, B, scores, 1.0f, w, stream);
            else
                rc = enqueue_all(dtype, Q, single_query(Lq), d, docs, stride, offsets, lengths, B, scores, 1.0f, L,
                                 w, stream);
        }
        if (rc == MAXSIM_OK) rc = launch_topk(scores, B, k, top_scores, top_ids, w + score_at + score_bytes, stream);
        return rc;
    });
}

int rerank_fp8(int dtype, const void *Q, int32_t Lq, int32_t d, const void *docs, int64_t stride,
               const int32_t *offsets, const int32_t *lengths, int32_t B, float doc_scale, float *scores,
               void *stream_ptr)
{
    int st = check_common(Q, Lq, d, docs, stride, offsets, lengths, B, scores);
    if (st != MAXSIM_OK) return st;
    if ((st = check_fp8(d, stride, doc_scale)) != MAXSIM_OK) return st;
    if (B == 0) return MAXSIM_OK;
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    if (Lq == 0) return launch_fill(scores, B, 0.0f, stream);
    if (range_eligible(Lq, d, B)) {
        RangePlan rp;
        const int rc = range_plan(dtype | kFmtFp8Docs, Lq, d, B, &rp);
        if (rc != MAXSIM_OK) return rc;
        return with_workspace(stream, rp.bytes, [&](char *w) {
            return enqueue_range(dtype | kFmtFp8Docs, rp, Q, Lq, d, docs, stride, offsets, lengths, B, scores,
                                 doc_scale, w, stream);
        });
    }
    return run_all(dtype | kFmtFp8Docs, Q, single_query(Lq), d, docs, stride, offsets, lengths, B, scores,
                   doc_scale, stream);
}

// Host checks of a query table (the per-doc checks run in the plan kernel).
int check_queries(const int32_t *q_offsets, const int32_t *q_lengths, int32_t nq, int32_t q_rows,
                  int32_t max_lq, const int32_t *doc_query, int32_t B, QueryTable *qt)
{
    if (q_rows < 0 || nq < 0 || max_lq < 0) return MAXSIM_ERR_INVALID_ARG;
    if (max_lq > kMaxLq) return MAXSIM_ERR_UNSUPPORTED;
    if (B > 0 && (!doc_query || (nq > 0 && (!q_offsets || !q_lengths)))) return MAXSIM_ERR_INVALID_ARG;
    if (((uintptr_t)doc_query | (uintptr_t)q_offsets | (uintptr_t)q_lengths) & 3u) return MAXSIM_ERR_INVALID_ARG;
    qt->doc_query = doc_query;
    qt->q_offsets = q_offsets;
    qt->q_lengths = q_lengths;
    qt->nq = nq;
    qt->q_rows = q_rows;
    qt->Lq = 0;
    qt->max_lq = max_lq;
    return MAXSIM_OK;
}

// fmt: kernel format (query format, | kFmtFp8Docs for FP8 E4M3 docs with doc_scale).
int rerank_pairs(int fmt, const void *Qs, int32_t q_rows, int32_t d, const int32_t *q_offsets,
                 const int32_t *q_lengths, int32_t nq, int32_t max_lq, const void *docs, int64_t stride,
                 const int32_t *offsets, const int32_t *lengths, const int32_t *doc_query, int32_t B,
                 float doc_scale, float *scores, void *stream_ptr)
{
    QueryTable qt;
    int st = check_queries(q_offsets, q_lengths, nq, q_rows, max_lq, doc_query, B, &qt);
    if (st != MAXSIM_OK) return st;
    st = check_common(Qs, max_lq, d, docs, stride, offsets, lengths, B, scores);
    if (st != MAXSIM_OK) return st;
    if ((fmt & kFmtFp8Docs) && (st = check_fp8(d, stride, doc_scale)) != MAXSIM_OK) return st;
    if (B == 0) return MAXSIM_OK;
    return run_all(fmt, Qs, qt, d, docs, stride, offsets, lengths, B, scores, doc_scale,
                   static_cast<hipStream_t>(stream_ptr));
}

// Several queries against the same docs: the queries (rows back to back in Qs, lengths
// on the host) are packed in order into passes of at most one register group of query
// tiles, each query starting on a tile; a query longer than a group has a pass of its
// own. One plan serves every pass; each pass is one score launch and one combine
// launch, reading the docs once for all of its queries. Empty queries score 0.
int rerank_multi(int fmt, const void *Qs, const int32_t *q_lengths, int32_t nq, int32_t d,
                 const void *docs, int64_t stride, const int32_t *offsets, const int32_t *lengths,
                 int32_t B, float doc_scale, float *scores, void *stream_ptr)
{
    if (nq < 0 || (nq > 0 && !q_lengths)) return MAXSIM_ERR_INVALID_ARG;
    int64_t total_rows = 0;
    for (int32_t j = 0; j < nq; ++j) {
        if (q_lengths[j] < 0) return MAXSIM_ERR_INVALID_ARG;
        if (q_lengths[j] > kMaxLq) return MAXSIM_ERR_UNSUPPORTED;
        total_rows += q_lengths[j];
    }
    int st = check_common(Qs, total_rows > 0 ? 1 : 0, d, docs, stride, offsets, lengths, B, scores, nq > 0);
    if (st != MAXSIM_OK) return st;
    if ((fmt & kFmtFp8Docs) && (st = check_fp8(d, stride, doc_scale)) != MAXSIM_OK) return st;
    if (B == 0 || nq == 0) return MAXSIM_OK;
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);

    struct Pass {
        int32_t j0, j1;    // queries [j0, j1)
        int64_t row0;      // first row of query j0 in Qs
        int tiles;
    };
    const int nks = (d + kStepK - 1) / kStepK;
    int group_tiles = kMaxFragsPerGroup / nks;
    if (group_tiles > kMaxQTilesPerGroup) group_tiles = kMaxQTilesPerGroup;
    std::vector<Pass> passes;
    int max_pad = 0;
    {
        int64_t row = 0;
        Pass cur{0, 0, 0, 0};
        auto close = [&](int32_t j_end) {
            if (cur.tiles > 0) {
                cur.j1 = j_end;
                passes.push_back(cur);
                const int pad = choose_config(cur.tiles * kTileRows, d).lq_pad;
                if (pad > max_pad) max_pad = pad;
            }
            cur.tiles = 0;
        };
        for (int32_t j = 0; j < nq; ++j) {
            const int t = (q_lengths[j] + kTileRows - 1) / kTileRows;
            if (t > 0) {
                // A new pass when this query does not fit, or when the score row
                // offset inside the pass would outgrow the table's int8.
                if (cur.tiles > 0 && (cur.tiles + t > group_tiles || j - cur.j0 > 127)) close(j);
                if (cur.tiles == 0) {
                    cur.j0 = j;
                    cur.row0 = row;
                }
                cur.tiles += t;
                if (cur.tiles >= group_tiles) close(j + 1);
            }
            row += q_lengths[j];
        }
        close(nq);
    }

    int rc = MAXSIM_OK;
    for (int32_t j = 0; j < nq && rc == MAXSIM_OK; ++j)
        if (q_lengths[j] == 0) rc = launch_fill(scores + (size_t)j * B, B, 0.0f, stream);
    if (rc != MAXSIM_OK || passes.empty()) return rc;

    DeviceFacts f;
    if (current_facts(&f) != MAXSIM_OK) return MAXSIM_ERR_HIP;
    const Layout L = make_layout(max_pad, B, (uint32_t)(f.cus * f.waves_per_cu));
    return with_workspace(stream, L.total, [&](char *w) {
        int rc = launch_plan(offsets, lengths, B, L, single_query(0), w, stream);
        const char *qbytes = static_cast<const char *>(Qs);
        for (size_t p = 0; p < passes.size() && rc == MAXSIM_OK; ++p) {
            const Pass &ps = passes[p];
            QueryTiles qt{};
            qt.score_stride = B;
            for (int T = 0; T < kMaxQTiles; ++T) qt.set(T, 0, 0, -1);
            int T = 0;
            int64_t rel = 0;  // row of query j relative to the pass
            for (int32_t j = ps.j0; j < ps.j1; ++j) {
                const int Lj = q_lengths[j];
                const int t = (Lj + kTileRows - 1) / kTileRows;
                for (int k = 0; k < t; ++k, ++T) {
                    const int left = Lj - k * kTileRows;
                    qt.set(T, (int)(rel + k * kTileRows), left > kTileRows ? kTileRows : left,
                           k == t - 1 ? j - ps.j0 : -1);
                }
                rel += Lj;
            }
            const void *Qp = qbytes + (size_t)ps.row0 * (size_t)d * 2;
            float *sp = scores + (size_t)ps.j0 * (size_t)B;
            const int rows = ps.tiles * kTileRows;
            rc = launch_score(fmt, Qp, rows, d, docs, stride, sp, L, w, qt, doc_scale, stream);
            if (rc == MAXSIM_OK) rc = launch_finish(fmt, rows, d, sp, L, w, qt, doc_scale, stream);
        }
        return rc;
    });
}

// Bodies of the staged score and finish entries; fmt is already checked.
int staged_score(int fmt, const void *Q, int32_t Lq, int32_t d, const void *docs, int64_t stride,
                 const int32_t *doc_offsets, const int32_t *doc_lengths, int32_t B, float *scores,
                 void *workspace, size_t workspace_bytes, float doc_scale, hipStream_t s)
{
    const int st = check_common(Q, Lq, d, docs, stride, doc_offsets, doc_lengths, B, scores);
    if (st != MAXSIM_OK) return st;
    if (B == 0) return MAXSIM_OK;
    if (Lq == 0) return launch_fill(scores, B, 0.0f, s);
    if (!workspace || ((uintptr_t)workspace & 255u)) return MAXSIM_ERR_WORKSPACE;
    Layout L;
    if (workspace_layout(Lq, d, B, &L) != MAXSIM_OK) return MAXSIM_ERR_HIP;
    if (workspace_bytes < L.total) return MAXSIM_ERR_WORKSPACE;
    return launch_score(fmt, Q, Lq, d, docs, stride, scores, L, static_cast<char *>(workspace), single_tiles(Lq),
                        doc_scale, s);
}

int staged_finish(int fmt, int32_t Lq, int32_t d, int32_t B, float *scores, void *workspace,
                  size_t workspace_bytes, float doc_scale, hipStream_t s)
{
    if (B < 0 || Lq < 0 || d < 1) return MAXSIM_ERR_INVALID_ARG;
    if (B > 0 && !scores) return MAXSIM_ERR_INVALID_ARG;
    if (d > kMaxD || d % 8 != 0 || Lq > kMaxLq) return MAXSIM_ERR_UNSUPPORTED;
    if (B > 0 && ((uintptr_t)scores & 3u)) return MAXSIM_ERR_INVALID_ARG;
    if (B == 0 || Lq == 0) return MAXSIM_OK;
    if (!workspace || ((uintptr_t)workspace & 255u)) return MAXSIM_ERR_WORKSPACE;
    Layout L;
    if (workspace_layout(Lq, d, B, &L) != MAXSIM_OK) return MAXSIM_ERR_HIP;
    if (workspace_bytes < L.total) return MAXSIM_ERR_WORKSPACE;
    return launch_finish(fmt, Lq, d, scores, L, static_cast<char *>(workspace), single_tiles(Lq), doc_scale, s);
}

}  // namespace

extern "C" {

int maxsim_rerank(const void *Q, int32_t Lq, int32_t d, const void *docs, int64_t stride,
                  const int32_t *doc_offsets, const int32_t *doc_lengths, int32_t B, float *scores,
                  void *stream)
{
    return rerank(MAXSIM_F16, Q, Lq, d, docs, stride, doc_offsets, doc_lengths, B, scores, stream);
}

int maxsim_rerank_bf16(const void *Q, int32_t Lq, int32_t d, const void *docs, int64_t stride,
                       const int32_t *doc_offsets, const int32_t *doc_lengths, int32_t B,
                       float *scores, void *stream)
{
    return rerank(MAXSIM_BF16, Q, Lq, d, docs, stride, doc_offsets, doc_lengths, B, scores, stream);
}

int maxsim_rerank_noalloc(int dtype, const void *Q, int32_t Lq, int32_t d, const void *docs, int64_t stride,
                          const int32_t *doc_offsets, const int32_t *doc_lengths, int32_t B, float *scores,
                          void *stream)
{
    return rerank_noalloc(dtype, Q, Lq, d, docs, stride, doc_offsets, doc_lengths, B, scores, stream);
}

int maxsim_rerank_short(int dtype, const void *Q, int32_t Lq, int32_t d, const void *docs, int64_t stride,
                        const int32_t *doc_offsets, const int32_t *doc_lengths, int32_t B, float *scores,
                        void *stream)
{
    if (dtype != MAXSIM_F16 && dtype != MAXSIM_BF16) return MAXSIM_ERR_INVALID_ARG;
    return rerank_short(dtype, Q, Lq, d, docs, stride, doc_offsets, doc_lengths, B, 1.0f, scores, stream);
}

int maxsim_rerank_short_fp8(int dtype, const void *Q, int32_t Lq, int32_t d, const void *docs, int64_t stride,
                            const int32_t *doc_offsets, const int32_t *doc_lengths, int32_t B, float doc_scale,
                            float *scores, void *stream)
{
    if (dtype != MAXSIM_F16 && dtype != MAXSIM_BF16) return MAXSIM_ERR_INVALID_ARG;
    return rerank_short(dtype | kFmtFp8Docs, Q, Lq, d, docs, stride, doc_offsets, doc_lengths, B, doc_scale,
                        scores, stream);
}

int maxsim_rerank_pairs(const void *Qs, int32_t q_rows, int32_t d, const int32_t *q_offsets,
                        const int32_t *q_lengths, int32_t nq, int32_t max_lq, const void *docs,
                        int64_t stride, const int32_t *doc_offsets, const int32_t *doc_lengths,
                        const int32_t *doc_query, int32_t B, float *scores, void *stream)
{
    return rerank_pairs(MAXSIM_F16, Qs, q_rows, d, q_offsets, q_lengths, nq, max_lq, docs, stride,
                        doc_offsets, doc_lengths, doc_query, B, 1.0f, scores, stream);
}

int maxsim_rerank_pairs_bf16(const void *Qs, int32_t q_rows, int32_t d, const int32_t *q_offsets,
                             const int32_t *q_lengths, int32_t nq, int32_t max_lq, const void *docs,
                             int64_t stride, const int32_t *doc_offsets, const int32_t *doc_lengths,
                             const int32_t *doc_query, int32_t B, float *scores, void *stream)
{
    return rerank_pairs(MAXSIM_BF16, Qs, q_rows, d, q_offsets, q_lengths, nq, max_lq, docs, stride,
                        doc_offsets, doc_lengths, doc_query, B, 1.0f, scores, stream);
}

int maxsim_rerank_multi(const void *Qs, const int32_t *q_lengths, int32_t nq, int32_t d, const void *docs,
                        int64_t stride, const int32_t *doc_offsets, const int32_t *doc_lengths, int32_t B,
                        float *scores, void *stream)
{
    return rerank_multi(MAXSIM_F16, Qs, q_lengths, nq, d, docs, stride, doc_offsets, doc_lengths, B, 1.0f,
                        scores, stream);
}

int maxsim_rerank_multi_bf16(const void *Qs, const int32_t *q_lengths, int32_t nq, int32_t d,
                             const void *docs, int64_t stride, const int32_t *doc_offsets,
                             const int32_t *doc_lengths, int32_t B, float *scores, void *stream)
{
    return rerank_multi(MAXSIM_BF16, Qs, q_lengths, nq, d, docs, stride, doc_offsets, doc_lengths, B, 1.0f,
                        scores, stream);
}

int maxsim_rerank_fp8(const void *Q, int32_t Lq, int32_t d, const void *docs, int64_t stride,
                      const int32_t *doc_offsets, const int32_t *doc_lengths, int32_t B, float doc_scale,
                      float *scores, void *stream)
{
    return rerank_fp8(MAXSIM_F16, Q, Lq, d, docs, stride, doc_offsets, doc_lengths, B, doc_scale, scores, stream);
}

int maxsim_rerank_fp8_bf16(const void *Q, int32_t Lq, int32_t d, const void *docs, int64_t stride,
                           const int32_t *doc_offsets, const int32_t *doc_lengths, int32_t B, float doc_scale,
                           float *scores, void *stream)
{
    return rerank_fp8(MAXSIM_BF16, Q, Lq, d, docs, stride, doc_offsets, doc_lengths, B, doc_scale, scores,
                      stream);
}

int maxsim_rerank_topk(const void *Q, int32_t Lq, int32_t d, const void *docs, int64_t stride,
                       const int32_t *doc_offsets, const int32_t *doc_lengths, int32_t B, int32_t k,
                       float *top_scores, int32_t *top_ids, void *stream)
{
    return rerank_topk(MAXSIM_F16, Q, Lq, d, docs, stride, doc_offsets, doc_lengths, B, k, top_scores, top_ids,
                       stream);
}

int maxsim_rerank_topk_bf16(const void *Q, int32_t Lq, int32_t d, const void *docs, int64_t stride,
                            const int32_t *doc_offsets, const int32_t *doc_lengths, int32_t B, int32_t k,
                            float *top_scores, int32_t *top_ids, void *stream)
{
    return rerank_topk(MAXSIM_BF16, Q, Lq, d, docs, stride, doc_offsets, doc_lengths, B, k, top_scores, top_ids,
                       stream);
}

int maxsim_rerank_pairs_fp8(int dtype, const void *Qs, int32_t q_rows, int32_t d, const int32_t *q_offsets,
                            const int32_t *q_lengths, int32_t nq, int32_t max_lq, const void *docs,
                            int64_t stride, const int32_t *doc_offsets, const int32_t *doc_lengths,
                            const int32_t *doc_query, int32_t B, float doc_scale, float *scores, void *stream)
{
    if (dtype != MAXSIM_F16 && dtype != MAXSIM_BF16) return MAXSIM_ERR_INVALID_ARG;
    return rerank_pairs(dtype | kFmtFp8Docs, Qs, q_rows, d, q_offsets, q_lengths, nq, max_lq, docs, stride,
                        doc_offsets, doc_lengths, doc_query, B, doc_scale, scores, stream);
}

int maxsim_rerank_multi_fp8(int dtype, const void *Qs, const int32_t *q_lengths, int32_t nq, int32_t d,
                            const void *docs, int64_t stride, const int32_t *doc_offsets,
                            const int32_t *doc_lengths, int32_t B, float doc_scale, float *scores, void *stream)
{
    if (dtype != MAXSIM_F16 && dtype != MAXSIM_BF16) return MAXSIM_ERR_INVALID_ARG;
    return rerank_multi(dtype | kFmtFp8Docs, Qs, q_lengths, nq, d, docs, stride, doc_offsets, doc_lengths, B,
                        doc_scale, scores, stream);
}

const char *maxsim_status_string(int status)
{
    switch (status) {
    case MAXSIM_OK: return "ok";
    case MAXSIM_ERR_INVALID_ARG: return "invalid argument (null pointer, negative size, stride < d or bad format)";
    case MAXSIM_ERR_UNSUPPORTED: return "unsupported shape or alignment (need d <= 256 and d % 8 == 0, Lq <= 256, stride % 8 == 0 and <= 2^24, 16-byte aligned Q and docs)";
    case MAXSIM_ERR_HIP: return "HIP call failed (no device, allocation or launch failure)";
    case MAXSIM_ERR_WORKSPACE: return "workspace null, not 256-byte aligned, or too small";
    case MAXSIM_ERR_SCRATCH: return "the batch needs more scratch than maxsim_rerank_noalloc's static 64 MiB per GPU holds";
    default: return "unknown status";
    }
}

int maxsim_workspace_size(int32_t Lq, int32_t d, int32_t B, size_t *bytes)
{
    if (!bytes || B < 0 || Lq < 0 || d < 1) return MAXSIM_ERR_INVALID_ARG;
    if (d > kMaxD || d % 8 != 0 || Lq > kMaxLq) return MAXSIM_ERR_UNSUPPORTED;
    Layout L;
    if (workspace_layout(Lq, d, B, &L) != MAXSIM_OK) return MAXSIM_ERR_HIP;
    *bytes = L.total;
    return MAXSIM_OK;
}

int maxsim_plan(const int32_t *doc_offsets, const int32_t *doc_lengths, int32_t B, int32_t Lq,
                int32_t d, void *workspace, size_t workspace_bytes, void *stream)
{
    if (B < 0 || Lq < 0 || d < 1) return MAXSIM_ERR_INVALID_ARG;
    if (B > 0 && (!doc_offsets || !doc_lengths)) return MAXSIM_ERR_INVALID_ARG;
    if (d > kMaxD || d % 8 != 0 || Lq > kMaxLq) return MAXSIM_ERR_UNSUPPORTED;
    if (B == 0 || Lq == 0) return MAXSIM_OK;
    if (!workspace || ((uintptr_t)workspace & 255u)) return MAXSIM_ERR_WORKSPACE;
    Layout L;
    if (workspace_layout(Lq, d, B, &L) != MAXSIM_OK) return MAXSIM_ERR_HIP;
    if (workspace_bytes < L.total) return MAXSIM_ERR_WORKSPACE;
    return launch_plan(doc_offsets, doc_lengths, B, L, single_query(Lq), static_cast<char *>(workspace),
                       static_cast<hipStream_t>(stream));
}

int maxsim_plan_pairs(const int32_t *doc_offsets, const int32_t *doc_lengths, const int32_t *doc_query,
                      int32_t B, const int32_t *q_offsets, const int32_t *q_lengths, int32_t nq,
                      int32_t q_rows, int32_t max_lq, int32_t d, void *workspace, size_t workspace_bytes,
                      void *stream)
{
    if (B < 0 || d < 1) return MAXSIM_ERR_INVALID_ARG;
    if (B > 0 && (!doc_offsets || !doc_lengths)) return MAXSIM_ERR_INVALID_ARG;
    QueryTable qt;
    const int st = check_queries(q_offsets, q_lengths, nq, q_rows, max_lq, doc_query, B, &qt);
    if (st != MAXSIM_OK) return st;
    if (d > kMaxD || d % 8 != 0) return MAXSIM_ERR_UNSUPPORTED;
    // maxsim_score and maxsim_finish take Lq = 0 to mean "no query rows at all" and
    // write zeros without reading a plan, which would hide invalid queries.
    if (max_lq < 1) return MAXSIM_ERR_INVALID_ARG;
    if (B == 0) return MAXSIM_OK;
    if (!workspace || ((uintptr_t)workspace & 255u)) return MAXSIM_ERR_WORKSPACE;
    Layout L;
    if (workspace_layout(max_lq, d, B, &L) != MAXSIM_OK) return MAXSIM_ERR_HIP;
    if (workspace_bytes < L.total) return MAXSIM_ERR_WORKSPACE;
    return launch_plan(doc_offsets, doc_lengths, B, L, qt, static_cast<char *>(workspace),
                       static_cast<hipStream_t>(stream));
}

int maxsim_score(int dtype, const void *Q, int32_t Lq, int32_t d, const void *docs, int64_t stride,
                 const int32_t *doc_offsets, const int32_t *doc_lengths, int32_t B, float *scores,
                 void *workspace, size_t workspace_bytes, void *stream)
{
    if (dtype != MAXSIM_F16 && dtype != MAXSIM_BF16) return MAXSIM_ERR_INVALID_ARG;
    return staged_score(dtype, Q, Lq, d, docs, stride, doc_offsets, doc_lengths, B, scores, workspace,
                        workspace_bytes, 1.0f, static_cast<hipStream_t>(stream));
}

int maxsim_score_fp8(int dtype, const void *Q, int32_t Lq, int32_t d, const void *docs, int64_t stride,
                     const int32_t *doc_offsets, const int32_t *doc_lengths, int32_t B, float doc_scale,
                     float *scores, void *workspace, size_t workspace_bytes, void *stream)
{
    if (dtype != MAXSIM_F16 && dtype != MAXSIM_BF16) return MAXSIM_ERR_INVALID_ARG;
    const int st = check_fp8(d, stride, doc_scale);
    if (st != MAXSIM_OK) return st;
    return staged_score(dtype | kFmtFp8Docs, Q, Lq, d, docs, stride, doc_offsets, doc_lengths, B, scores,
                        workspace, workspace_bytes, doc_scale, static_cast<hipStream_t>(stream));
}

int maxsim_finish(int dtype, int32_t Lq, int32_t d, int32_t B, float *scores, void *workspace,
                  size_t workspace_bytes, void *stream)
{
    if (dtype != MAXSIM_F16 && dtype != MAXSIM_BF16) return MAXSIM_ERR_INVALID_ARG;
    return staged_finish(dtype, Lq, d, B, scores, workspace, workspace_bytes, 1.0f,
                         static_cast<hipStream_t>(stream));
}

int maxsim_finish_fp8(int dtype, int32_t Lq, int32_t d, int32_t B, float doc_scale, float *scores,
                      void *workspace, size_t workspace_bytes, void *stream)
{
    if (dtype != MAXSIM_F16 && dtype != MAXSIM_BF16) return MAXSIM_ERR_INVALID_ARG;
    if (!valid_scale(doc_scale)) return MAXSIM_ERR_INVALID_ARG;
    if (d % 16 != 0) return MAXSIM_ERR_UNSUPPORTED;
    return staged_finish(dtype | kFmtFp8Docs, Lq, d, B, scores, workspace, workspace_bytes, doc_scale,
                         static_cast<hipStream_t>(stream));
}

int maxsim_version(void) { return 100; }

}  // extern "C"
