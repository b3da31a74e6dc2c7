// Work-item arithmetic of the length-binned schedule, shared by the score kernel and
// the combine kernel (device side).
//
// The plan kernels leave, in the workspace header, the number of docs in each tile-count
// bin and the total tile count T; the doc descriptors sit in `desc`, bins in descending
// order. A kernel turns that into work items:
//   - chunk size CT = max(2, NQT, ceil(T / (kItemsPerWave * W))) tiles, W = score
//     waves, NQT = query tiles per register group (an item's fixed cost, the per-row
//     maxima across lanes and their store or sum, grows with NQT);
//   - a doc of bin b is cut into K_b = ceil(2^b / CT) chunks when 2^b > CT (else 1);
//     chunk c covers its tiles [c nt / K_b, (c + 1) nt / K_b), never empty since
//     nt > 2^(b-1) >= K_b;
//   - claims (work items) run bin 27 first ... bin 0 last, a doc's chunks adjacent.
#pragma once

#include "maxsim_common.h"

namespace maxsim {

struct BinTables {
    uint32_t claim_end[kNumBins];   // claims of bins >= b
    uint32_t desc_start[kNumBins];  // first desc index of bin b
    uint32_t chunks[kNumBins];      // K_b
    uint32_t total_claims;
    uint32_t split_docs;            // docs with K_b > 1: desc indices [0, split_docs)
};

// Wave 0 of a workgroup fills the tables (lane b computes bin b, lane 0 scans the
// bins in descending order); the caller publishes them with a barrier.
__device__ inline void fill_bin_tables(const Header *hdr, uint32_t waves, int nqt, BinTables &t, int lane)
{
    const unsigned long long T = hdr->total_tiles;
    const unsigned long long per = (unsigned long long)waves * kItemsPerWave;
    unsigned long long ct = (T + per - 1) / per;
    if (ct < kMinChunkTiles) ct = kMinChunkTiles;
    if (ct < (unsigned long long)nqt) ct = (unsigned long long)nqt;
    if (ct > (1ull << 28)) ct = 1ull << 28;  // above every bin's 2^b: no splits
    const uint32_t ct32 = (uint32_t)ct;
    if (lane < kNumBins) {
        const uint32_t cnt = hdr->bin_count[lane];
        const uint32_t cap = 1u << lane;  // most tiles a doc of bin `lane` has
        const uint32_t K = cap > ct32 ? (cap + ct32 - 1u) / ct32 : 1u;
        t.chunks[lane] = K;
        t.desc_start[lane] = cnt;       // counts for now, turned into starts below
        t.claim_end[lane] = cnt * K;    // claims of the bin for now
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane == 0) {
        uint32_t claims = 0, descs = 0, split = 0;
        for (int b = kNumBins - 1; b >= 0; --b) {
            const uint32_t cnt = t.desc_start[b];
            if (t.chunks[b] > 1) split += cnt;
            t.desc_start[b] = descs;
            descs += cnt;
            claims += t.claim_end[b];
            t.claim_end[b] = claims;
        }
        t.total_claims = claims;
        t.split_docs = split;
    }
}

// Per-lane copy of the tables (lane b < kNumBins holds bin b) for ballot searches.
struct LaneBins {
    uint32_t claim_end, desc_start, chunks;
};

__device__ inline LaneBins lane_bins(const BinTables &t, int lane)
{
    LaneBins L;
    L.claim_end = lane < kNumBins ? t.claim_end[lane] : 0u;
    L.desc_start = lane < kNumBins ? t.desc_start[lane] : 0xFFFFFFFFu;
    L.chunks = lane < kNumBins ? t.chunks[lane] : 1u;
    return L;
}

struct Item {
    uint32_t di;     // desc index of the doc
    uint32_t c;      // chunk of the doc
    uint32_t K;      // chunks of the doc
    uint32_t first;  // claim index of the doc's chunk 0
};

// Work item of claim g (< total claims). g < claim_end[b] holds exactly for
// b <= bin(g), so the bin is the highest set bit of the ballot.
__device__ inline Item locate_claim(const LaneBins &L, int lane, uint32_t g)
{
    const unsigned long long below = __ballot(lane < kNumBins && g < L.claim_end);
    const int b = 63 - __builtin_clzll(below);
    const uint32_t begin = b + 1 < kNumBins ? __builtin_amdgcn_readlane(L.claim_end, b + 1) : 0u;
    Item it;
    it.K = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(L.chunks, b));
    const uint32_t local = g - __builtin_amdgcn_readfirstlane(begin);
    const uint32_t j = local / it.K;
    it.c = local - j * it.K;
    it.di = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(L.desc_start, b)) + j;
    it.first = g - it.c;
    return it;
}

// Work items of the doc at desc index di. di >= desc_start[b] holds exactly for
// b >= bin(di), so the bin is the lowest set bit of the ballot.
__device__ inline Item locate_doc(const LaneBins &L, int lane, uint32_t di)
{
    const unsigned long long above = __ballot(lane < kNumBins && di >= L.desc_start);
    const int b = __builtin_ctzll(above);
    const uint32_t begin = b + 1 < kNumBins ? __builtin_amdgcn_readlane(L.claim_end, b + 1) : 0u;
    Item it;
    it.K = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(L.chunks, b));
    const uint32_t j = di - __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(L.desc_start, b));
    it.di = di;
    it.c = 0;
    it.first = __builtin_amdgcn_readfirstlane(begin) + j * it.K;
    return it;
}

// The doc descriptors, written by the plan kernels before the score and combine
// launches, are read-only while those run: read through the constant address space, a
// descriptor at a wave-uniform index comes in one scalar load, whose wait leaves the
// vector loads in flight alone.
typedef __attribute__((address_space(4))) const DocDesc ConstDocDesc;

__device__ __forceinline__ DocDesc load_desc(const DocDesc *desc, uint32_t i)
{
    ConstDocDesc *c = (ConstDocDesc *)desc + i;
    DocDesc d;
    d.doc = c->doc;
    d.offset = c->offset;
    d.length = c->length;
    d.tiles = c->tiles;
    d.query = c->query;
    d.q_offset = c->q_offset;
    d.q_length = c->q_length;
    d.reserved = c->reserved;
    return d;
}

}  // namespace maxsim
