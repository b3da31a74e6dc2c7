// Internal layout shared by the library's host code and its kernels: the scratch
// workspace, the doc schedule it holds, and the score kernel's argument block.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace maxsim {

// ---------------------------------------------------------------- shapes
constexpr int kWave = 64;
constexpr int kScoreBlock = 256;              // score kernel workgroup: 4 waves
constexpr int kScoreWaves = kScoreBlock / kWave;
constexpr int kTileRows = 16;                 // doc rows per tile (N of the 16x16x32 MFMA)
constexpr int kStepK = 32;                    // K of one MFMA
constexpr int kMaxD = 256;
constexpr int kMaxLq = 256;
constexpr int64_t kMaxStride = int64_t(1) << 24;
constexpr int kMaxQTilesPerGroup = 8;         // query tiles held in registers at once
constexpr int kMaxFragsPerGroup = 32;         // NQT * NKS <= 32 -> <= 128 VGPRs of Q
// Padded query rows: g groups of ceil(tiles / g) tiles, tiles <= 16, g <= 4 (a group
// holds >= 4 tiles), so at most tiles + g - 1 <= 19 tiles.
constexpr int kMaxLqPad = 19 * kTileRows;
constexpr int kMaxQTiles = kMaxLqPad / kTileRows;
constexpr uint32_t kNaNBits = 0x7FC00000u;    // fp32 quiet NaN: the score of a doc whose query is invalid

// ---------------------------------------------------------------- schedule
// Docs are binned by tile count nt = ceil(len / 16): bin 0 holds nt <= 1, bin b >= 1
// holds 2^(b-1) < nt <= 2^b. len < 2^31 gives nt <= 2^27, so 28 bins.
constexpr int kNumBins = 28;
constexpr int kPlanBlock = 1024;              // plan kernels: threads per block
constexpr int kPlanMaxBlocks = 1024;          // docs per plan block grows past 2^20 docs
constexpr int kHistStride = 32;               // words per plan block: 28 counts, tiles lo, hi
constexpr int kItemsPerWave = 4;              // target work items per score wave
constexpr uint32_t kDealPeriod = 12;          // deal rounds per period; odd-XCD waves sit out one
constexpr int kMinChunkTiles = 2;              // and at least the query tiles per register group

struct Header {
    unsigned long long total_tiles;          // sum over docs of ceil(len / 16)
    uint32_t bin_count[kNumBins];            // docs per bin
    uint32_t multi_query;                    // docs carry their own queries (no Q staging)
};

struct alignas(16) DocDesc {
    int32_t doc;       // index into scores
    int32_t offset;    // first row in docs
    int32_t length;    // rows
    int32_t tiles;     // ceil(length / 16)
    int32_t query;     // query the doc is scored against
    int32_t q_offset;  // its first row in Q
    int32_t q_length;  // its rows; -1 marks an invalid query (the doc's score is NaN)
    int32_t reserved;
};

__host__ __device__ inline int bin_of(uint32_t nt)
{
    return nt <= 1 ? 0 : 32 - __builtin_clz(nt - 1);
}

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Layout {
    size_t header, hist, partials, desc, total;
    uint32_t plan_blocks, docs_per_plan_block;
    uint32_t partial_slots;
    int lq_pad;
};

// A doc is split when its bin's upper bound 2^b exceeds the chunk size CT, so every
// split doc has nt > 2^(b-1) >= CT / 2 tiles: there are fewer than 2 T / CT of them,
// and, since CT >= T / (kItemsPerWave * W), fewer than S = 2 * kItemsPerWave * W; there
// are also at most B. Each gets ceil(2^b / CT) < 2 nt / CT + 1 chunks, so all of them
// together have fewer than 2 T / CT + (split docs) <= S + min(B, S) chunks. Split docs
// come first in the claim order (their bins are the highest), so a split chunk's claim
// index serves as its slot of per-row maxima. Any W at least the score launch's wave
// count gives enough slots (the bound grows with W).
inline uint32_t partial_slots_for(int32_t B, uint32_t waves)
{
    const uint64_t s = 2ull * kItemsPerWave * waves;
    const uint64_t b = B > 0 ? (uint64_t)B : 0ull;
    return (uint32_t)(s + (b < s ? b : s));
}

inline Layout make_layout(int lq_pad, int32_t B, uint32_t waves_max)
{
    Layout L{};
    uint32_t rounds = 1;
    while ((uint64_t)rounds * kPlanBlock * kPlanMaxBlocks < (uint64_t)(B > 0 ? B : 0)) rounds *= 2;
    L.docs_per_plan_block = rounds * kPlanBlock;
    L.plan_blocks = B > 0 ? (uint32_t)(((uint64_t)B + L.docs_per_plan_block - 1) / L.docs_per_plan_block) : 1;
    L.partial_slots = partial_slots_for(B, waves_max);
    L.lq_pad = lq_pad;
    size_t off = 0;
    L.header = off;   off = align256(off + sizeof(Header));
    L.hist = off;     off = align256(off + (size_t)L.plan_blocks * kHistStride * 4);
    L.partials = off; off = align256(off + (size_t)L.partial_slots * (size_t)lq_pad * 4);
    L.desc = off;     off = align256(off + (size_t)(B > 0 ? B : 0) * sizeof(DocDesc));
    L.total = off;
    return L;
}

// ---------------------------------------------------------------- score kernel
// The query rows of one score launch as 16-row query tiles: the one query of a
// single-query launch, or several queries that score the same docs, each starting on
// a tile boundary (a tile never mixes two queries, so each query's rows meet the lanes
// exactly as they would alone). Tile T holds rows src(T) .. src(T) + rows(T) - 1 of Q;
// end(T) >= 0 says that tile T is its query's last and gives that query's score row
// (scores + end(T) * score_stride). Not used under a multi-query "pairs" plan, whose
// docs carry their own query rows.
// One 32-bit word per tile, so that a kernel reads an entry at a wave-uniform index with
// one scalar load (narrower fields would need vector loads, whose waits also wait for
// the doc tiles already in flight).
struct QueryTiles {
    int64_t score_stride;           // elements between the score rows of two queries
    uint32_t tile[kMaxQTiles];      // src (bits 0-15), rows 0..16 (16-23), end as int8 (24-31)

    __host__ __device__ int src(int T) const { return (int)(tile[T] & 0xFFFFu); }
    __host__ __device__ int rows(int T) const { return (int)((tile[T] >> 16) & 0xFFu); }
    __host__ __device__ int end(int T) const { return (int)(int8_t)(uint8_t)(tile[T] >> 24); }
    __host__ __device__ void set(int T, int src_row, int nrows, int end_row)
    {
        tile[T] = (uint32_t)(src_row & 0xFFFF) | ((uint32_t)(nrows & 0xFF) << 16) |
                  ((uint32_t)(uint8_t)(int8_t)end_row << 24);
    }
};

struct ScoreArgs {
    const uint16_t *Q;        // query rows [*, d]
    const char *docs;         // row r at docs + r * stride_bytes
    int64_t stride_bytes;
    const Header *hdr;
    const DocDesc *desc;
    float *partials;          // [partial_slots, lq_pad]
    float *scores;
    int32_t d, ngroups, lq_pad;
    int32_t q_in_lds;         // LDS holds room for the Q tile; used unless the plan is multi-query
    float doc_scale;          // FP8 docs: value = doc_scale * e4m3 (unused otherwise)
    QueryTiles qt;
};

// Q is staged in LDS when its padded tile takes at most this many bytes; a larger
// query (up to 256 x 256) would leave no room for the per-wave doc tiles, so its
// fragments are read from global memory (L2-resident) instead.
constexpr size_t kMaxQLdsBytes = 64 * 1024;

// ---------------------------------------------------------------- doc-tile pipeline
// Doc tiles go from memory straight into LDS (LDS-DMA buffer loads, 16 bytes per lane,
// no registers in flight). A 16-row tile is kept as rows of dma_row_chunks 16-byte
// chunks: a power of two covering the K-steps' columns (8 elements per chunk for 16-bit
// docs, 16 for FP8 docs), the chunks past a row's d columns filled with zeros by
// out-of-range loads. Each wave owns P such slots. These rules fix an instance's
// pipeline depth and the occupancy it is built for; the host sizes the kernel's LDS
// with the same functions.
constexpr int kLdsPerCu = 160 * 1024;
constexpr int kScoreStaticLds = 1024;             // bin tables and other static LDS, rounded up

constexpr int dma_row_chunks(int nks, bool fp8)
{
    const int need = fp8 ? 2 * nks : 4 * nks;  // chunks the NKS K-steps read
    return need <= 4 ? 4 : (need <= 8 ? 8 : (need <= 16 ? 16 : 32));
}
constexpr int dma_tile_bytes(int nks, bool fp8) { return kTileRows * dma_row_chunks(nks, fp8) * 16; }
// 16-row MFMA row blocks per slot of the scheduled score kernel: FP8 rows are half as
// wide, so a slot holds 32 of them (the bytes of a 16-bit tile), and every slot's fixed
// cost (descriptor, waits, loop) is paid once per 4 KB at d = 128 in both formats.
constexpr int score_sub(bool fp8) { return fp8 ? 2 : 1; }
// Swizzle of slot row r: its chunk c sits at r * CP + (c ^ dma_swizzle(r, CP)). The 16
// rows of one fragment read land in distinct 16-byte bank groups, modulo 8 and modulo
// 16 groups, whichever the LDS serves a read in.
__host__ __device__ constexpr int dma_swizzle(int r, int cp) { return (r % cp) ^ ((r / cp) & 1); }
// Registers of one wave: query fragments, one B-fragment set, running maxima,
// accumulators, addressing and loop state (and the FP8 conversion's temporaries).
constexpr int dma_regs(int nks, int nqt, bool fp8) { return 4 * nqt * nks + 4 * nks + 4 * nqt + 56 + (fp8 ? 8 : 0); }
constexpr int dma_waves_per_simd(int nks, int nqt, bool fp8)
{
    return dma_regs(nks, nqt, fp8) <= 128 ? 4 : (dma_regs(nks, nqt, fp8) <= 168 ? 3 : (dma_regs(nks, nqt, fp8) <= 256 ? 2 : 1));
}
// Workgroups per CU an instance is built for: what its registers allow, at most 3 (four
// workgroups of LDS-DMA streams per CU read slower than three, measured), and fewer if
// two tiles in flight per wave would not fit their LDS.
// (sub: 16-row blocks per slot; a slot holds sub * dma_tile_bytes bytes.)
constexpr int dma_blocks(int nks, int nqt, bool fp8, int sub = 1)
{
    int b = dma_waves_per_simd(nks, nqt, fp8) < 3 ? dma_waves_per_simd(nks, nqt, fp8) : 3;
    while (b > 1 && kScoreWaves * 2 * sub * dma_tile_bytes(nks, fp8) > kLdsPerCu / b - kScoreStaticLds) --b;
    return b;
}
// Slots in flight per wave: up to 16 KB (8 slots), within a workgroup's share of LDS.
constexpr int dma_pipe(int nks, int nqt, bool fp8, int sub = 1)
{
    int p = 16384 / (sub * dma_tile_bytes(nks, fp8));
    if (p > 8) p = 8;
    while (p > 1 && kScoreWaves * p * sub * dma_tile_bytes(nks, fp8) >
                        kLdsPerCu / dma_blocks(nks, nqt, fp8, sub) - kScoreStaticLds)
        --p;
    return p;
}

// ---------------------------------------------------------------- one-launch short-doc kernel
struct ShortArgs {
    const uint16_t *Q;        // [Lq, d]
    const char *docs;         // row r at docs + r * stride_bytes
    int64_t stride_bytes;
    const int32_t *offsets;   // [B]
    const int32_t *lengths;   // [B]
    float *scores;            // [B]
    int32_t B, d, Lq;
    float doc_scale;          // FP8 docs: multiplies each sum (unused otherwise)
};

// ---------------------------------------------------------------- combine kernel
struct CombineArgs {
    const Header *hdr;
    const DocDesc *desc;
    const float *partials;
    float *scores;
    uint32_t score_waves;     // W of the score launch (fixes the chunking)
    int32_t nqt, ngroups, lq_pad;
    float doc_scale;          // multiplies each sum (1 for 16-bit docs)
    QueryTiles qt;            // as in ScoreArgs
};

// What the plan kernels need to know about the queries. A single query is nq = 1 with
// doc_query, q_offsets and q_lengths null and Lq rows.
struct QueryTable {
    const int32_t *doc_query;  // [B] query of each doc (null: all query 0)
    const int32_t *q_offsets;  // [nq] first row of each query in Q (null: 0)
    const int32_t *q_lengths;  // [nq] rows of each query (null: Lq)
    int32_t nq;
    int32_t q_rows;            // rows of Q; a query must lie inside them
    int32_t Lq;                // rows of the single query
    int32_t max_lq;            // longest query the launch is built for
};

}  // namespace maxsim

// Kernel entry lookup implemented by the per-(format, K-steps) instance files.
// Returns nullptr when (nqt) is not instantiated.
const void *maxsim_score_kernel_f16(int nks, int nqt);
const void *maxsim_score_kernel_bf16(int nks, int nqt);
