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

// ---------------------------------------------------------------- schedule
// Docs are binned by tile count nt = ceil(len / 16): bin 0 holds nt <= 1, bin b >= 1
// holds 2^(b-1) < nt <= 2^b. len < 2^31 gives nt <= 2^27, so 28 bins.
constexpr int kNumBins = 28;
constexpr int kPlanBlock = 1024;              // plan kernels: threads per block
constexpr int kPlanMaxBlocks = 1024;          // docs per plan block grows past 2^20 docs
constexpr int kHistStride = 32;               // words per plan block: 28 counts, tiles lo, hi
constexpr int kItemsPerWave = 4;              // target work items per score wave
constexpr int kMinChunkTiles = 2;

struct Header {
    unsigned long long total_tiles;          // sum over docs of ceil(len / 16)
    uint32_t bin_count[kNumBins];            // docs per bin
};

struct alignas(16) DocDesc {
    int32_t doc;     // index into scores
    int32_t offset;  // first row in docs
    int32_t length;  // rows
    int32_t tiles;   // ceil(length / 16)
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
// and, since CT >= T / (kItemsPerWave * W), fewer than 2 * kItemsPerWave * W. Each gets
// ceil(2^b / CT) < 2 nt / CT + 1 chunks, fewer than 4 * kItemsPerWave * W in all.
// Split docs come first in the claim order (their bins are the highest), so a split
// chunk's claim index serves as its slot of per-row maxima.
inline Layout make_layout(int lq_pad, int32_t B, uint32_t waves_max)
{
    Layout L{};
    uint32_t rounds = 1;
    while ((uint64_t)rounds * kPlanBlock * kPlanMaxBlocks < (uint64_t)(B > 0 ? B : 0)) rounds *= 2;
    L.docs_per_plan_block = rounds * kPlanBlock;
    L.plan_blocks = B > 0 ? (uint32_t)(((uint64_t)B + L.docs_per_plan_block - 1) / L.docs_per_plan_block) : 1;
    L.partial_slots = 4u * kItemsPerWave * waves_max;
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
struct ScoreArgs {
    const uint16_t *Q;        // [Lq, d]
    const char *docs;         // row r at docs + r * stride_bytes
    int64_t stride_bytes;
    const Header *hdr;
    const DocDesc *desc;
    float *partials;          // [partial_slots, lq_pad]
    float *scores;
    int32_t Lq, d, ngroups, lq_pad;
    int32_t q_in_lds;         // Q staged in LDS (else fragments come from global)
};

// Q is staged in LDS when its padded tile takes at most this many bytes; a larger
// query (up to 256 x 256) would leave no room for the per-wave doc tiles, so its
// fragments are read from global memory (L2-resident) instead.
constexpr size_t kMaxQLdsBytes = 64 * 1024;

// ---------------------------------------------------------------- combine kernel
struct CombineArgs {
    const Header *hdr;
    const DocDesc *desc;
    const float *partials;
    float *scores;
    uint32_t score_waves;     // W of the score launch (fixes the chunking)
    int32_t Lq, nqt, ngroups, lq_pad;
};

}  // namespace maxsim

// Kernel entry lookup implemented by the per-(format, K-steps) instance files.
// Returns nullptr when (nqt) is not instantiated.
const void *maxsim_score_kernel_f16(int nks, int nqt);
const void *maxsim_score_kernel_bf16(int nks, int nqt);
