// MaxSim score kernel for gfx950 (CDNA4), one instance per (format, K-steps, query
// tiles per group).
//
// Operation (Flash-MaxSim rerank page, docs.vllm.ai,
// vllm.v1.pool.flash_maxsim.flash_maxsim_rerank, module description and section
// `_maxsim_rerank_kernel`): score_i = sum over query rows q of the max over doc i's
// rows t of Q[q] . X[off_i + t], fp16/bf16 inputs, fp32 products and sums.
//
// Mapping onto the hardware:
//   - Persistent workgroups of 4 waves, as many as fit on every CU. Each wave claims
//     work items (a doc, or a chunk of a long doc's tiles) from the length-binned
//     schedule that the plan kernels wrote, longest bins first, through one atomic
//     counter.
//   - Q is staged once per workgroup into LDS, zero-padded to 16-row tiles and
//     32-column K-steps. Each wave keeps its MFMA A-fragments of one group of up to
//     NQT query tiles in registers; with one group (every Lq * d that fits 128 VGPRs)
//     they are loaded once for the kernel's lifetime.
//   - Doc rows are read in 16-row tiles. Lane l owns row (l % 16) of the tile and, in
//     K-step s, the 8 contiguous elements starting at column 8 * (4 s + l / 16): one
//     128-bit buffer load per lane per K-step, i.e. exactly the B-fragment layout of
//     v_mfma_f32_16x16x32_{f16,bf16}. A and B use the same lane -> column mapping, so
//     the dot products are exact dot products whatever the order inside a fragment.
//   - The row address is a 64-bit scalar base (doc offset widened to int64 before it
//     is multiplied by the stride, as the page's kernel does) plus a 32-bit per-lane
//     offset. Each tile gets a buffer descriptor whose size covers only the tile's
//     valid rows, so rows past the end of the doc read as zero and are never fetched;
//     K-chunks past d are pushed out of range the same way.
//   - S = Qtile . Dtile^T lands with lane l holding doc row (l % 16) and query rows
//     4 (l / 16) + j, j < 4. Invalid doc rows are set to -inf (only on a partial
//     tile), then an element-wise running max per lane; at the end of the item four
//     DPP row_ror steps (8, 4, 2, 1) take the max over the 16 doc-row lanes.
//   - Query rows past Lq (zero padding) are masked to 0 and the per-row maxima are
//     summed in one fixed order (ascending query tile, then j, then the four lane
//     groups), whether the doc was scored in one item or several, so scores do not
//     depend on how the schedule chunked the doc.
//   - A doc split into K chunks: each chunk writes its per-row maxima to its own slot,
//     bumps the doc's arrival counter, and the chunk that arrives last takes the max
//     over the K slots (exact, so order-free) and does the fixed-order sum.
#pragma once

#include "maxsim_common.h"

namespace maxsim {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor word 3 for raw (unswizzled, unformatted) access on gfx9-family.
constexpr int kBufferWord3 = 0x00020000;

template <bool BF16>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c)
{
    if constexpr (BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <int CTRL>
__device__ __forceinline__ float dpp_move(float v)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float fmax_plain(float a, float b) { return a > b ? a : b; }

// Max over the 16 lanes of each DPP row (row_ror:8, 4, 2, 1); every lane of the row
// ends with the row's max.
__device__ __forceinline__ float row16_max(float v)
{
    v = fmax_plain(v, dpp_move<0x128>(v));
    v = fmax_plain(v, dpp_move<0x124>(v));
    v = fmax_plain(v, dpp_move<0x122>(v));
    v = fmax_plain(v, dpp_move<0x121>(v));
    return v;
}

__device__ __forceinline__ uint32_t wave_uniform(uint32_t v)
{
    return __builtin_amdgcn_readfirstlane(v);
}

template <int NKS, int NQT, bool BF16, int P>
__global__ void __launch_bounds__(kScoreBlock)
score_kernel(const ScoreArgs a)
{
    constexpr int DPAD = NKS * kStepK;
    constexpr int LDQ = DPAD + 8;  // LDS row pitch (halves): 16 B skew against bank conflicts
    constexpr float NEG_INF = -__builtin_huge_valf();

    extern __shared__ __attribute__((aligned(16))) uint16_t qs[];  // [lq_pad][LDQ]
    __shared__ uint32_t s_claim_end[kNumBins];   // claims of bins >= b (descending order)
    __shared__ uint32_t s_desc_start[kNumBins];  // first desc index of bin b
    __shared__ uint32_t s_chunks[kNumBins];      // chunks per doc in bin b
    __shared__ float s_comb[kScoreWaves][kMaxLqPad];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int Lq = a.Lq;
    const int lq_pad = a.lq_pad;

    // ---- stage Q (zero-padded) into LDS
    {
        constexpr int CPR = DPAD / 8;  // 16-byte chunks per padded row
        const int n = lq_pad * CPR;
        for (int e = threadIdx.x; e < n; e += kScoreBlock) {
            const int r = e / CPR;
            const int c = e - r * CPR;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (r < Lq && c * 8 < a.d)
                v = *reinterpret_cast<const u32x4 *>(a.Q + (size_t)r * a.d + c * 8);
            *reinterpret_cast<u32x4 *>(qs + r * LDQ + c * 8) = v;
        }
    }

    // ---- schedule: chunk size from the total tile count and this grid's wave count
    if (threadIdx.x == 0) {
        const unsigned long long T = a.hdr->total_tiles;
        const unsigned long long per = (unsigned long long)gridDim.x * kScoreWaves * kItemsPerWave;
        unsigned long long ct = (T + per - 1) / per;
        if (ct < kMinChunkTiles) ct = kMinChunkTiles;
        uint32_t claims = 0, descs = 0;
        for (int b = kNumBins - 1; b >= 0; --b) {
            const uint32_t cnt = a.hdr->bin_count[b];
            const uint32_t cap = 1u << b;  // most tiles a doc of bin b has
            // cap > ct implies ct < 2^27: 32-bit division suffices.
            const uint32_t K = cap > ct ? (cap + (uint32_t)ct - 1u) / (uint32_t)ct : 1u;
            s_desc_start[b] = descs;
            s_chunks[b] = K;
            descs += cnt;
            claims += cnt * K;
            s_claim_end[b] = claims;
        }
    }
    __syncthreads();

    // Per-lane copies of the bin tables (lane b holds bin b), for a ballot search.
    const uint32_t my_claim_end = lane < kNumBins ? s_claim_end[lane] : 0u;
    const uint32_t my_desc_start = lane < kNumBins ? s_desc_start[lane] : 0u;
    const uint32_t my_chunks = lane < kNumBins ? s_chunks[lane] : 1u;
    const uint32_t total_claims = wave_uniform(__builtin_amdgcn_readlane(my_claim_end, 0));

    // ---- per-lane load geometry
    const uint32_t stride_bytes = (uint32_t)a.stride_bytes;
    const int row_in_tile = lane & 15;
    const int kgroup = lane >> 4;
    const uint32_t voff = (uint32_t)row_in_tile * stride_bytes + (uint32_t)kgroup * 16u;
    // K-step NKS-1 may hold 8-column chunks past d; those lanes point at row 16 of the
    // tile, which no tile descriptor covers (it spans at most 16 rows), so they read 0.
    const bool last_chunk_ok = ((NKS - 1) * 4 + kgroup) * 8 < a.d;
    const uint32_t voff_last = last_chunk_ok ? voff + (NKS - 1) * 64u : (uint32_t)kTileRows * stride_bytes;

    u32x4 qf[NQT][NKS];
    auto load_q = [&](int grp) {
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
            for (int s = 0; s < NKS; ++s) {
                const int row = (grp * NQT + qt) * kTileRows + row_in_tile;
                const int col = (s * 4 + kgroup) * 8;
                qf[qt][s] = *reinterpret_cast<const u32x4 *>(qs + row * LDQ + col);
            }
    };
    if (a.ngroups == 1) load_q(0);

    for (;;) {
        uint32_t g = 0;
        if (lane == 0) g = atomicAdd(a.claim, 1u);
        g = wave_uniform(__builtin_amdgcn_readlane(g, 0));
        if (g >= total_claims) break;

        // Bin of claim g: claims run bin 27 first, ..., bin 0 last; g < claim_end[b]
        // holds exactly for b <= bin(g).
        const unsigned long long below = __ballot(lane < kNumBins && g < my_claim_end);
        const int b = 63 - __builtin_clzll(below);
        const uint32_t bin_end = __builtin_amdgcn_readlane(my_claim_end, b);
        const uint32_t K = wave_uniform(__builtin_amdgcn_readlane(my_chunks, b));
        const uint32_t bin_begin = b + 1 < kNumBins ? __builtin_amdgcn_readlane(my_claim_end, b + 1) : 0u;
        const uint32_t local = g - wave_uniform(bin_begin);
        (void)bin_end;
        const uint32_t j = local / K;
        const uint32_t c = local - j * K;
        const uint32_t di = wave_uniform(__builtin_amdgcn_readlane(my_desc_start, b)) + j;
        const DocDesc dd = a.desc[di];
        const int doc = (int)wave_uniform((uint32_t)dd.doc);
        const int64_t off = (int64_t)(int32_t)wave_uniform((uint32_t)dd.offset);
        const int len = (int)wave_uniform((uint32_t)dd.length);
        const uint32_t nt = wave_uniform((uint32_t)dd.tiles);

        // Tiles [t_begin, t_end) of the doc's nt tiles; never empty (nt >= K).
        const uint32_t t_begin = (uint32_t)(((unsigned long long)c * nt) / K);
        const uint32_t t_end = (uint32_t)(((unsigned long long)(c + 1) * nt) / K);
        const int ntiles = (int)(t_end - t_begin);
        const int row0 = (int)t_begin * kTileRows;
        const int nrows = (len < (int)t_end * kTileRows ? len : (int)t_end * kTileRows) - row0;
        const char *chunk_base = a.docs + (off + row0) * a.stride_bytes;

        float lane_sum = 0.0f;
        for (int grp = 0; grp < a.ngroups; ++grp) {
            if (a.ngroups > 1) load_q(grp);

            float rmax[NQT][4];
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
                for (int r = 0; r < 4; ++r) rmax[qt][r] = NEG_INF;

            u32x4 buf[P][NKS];
            auto issue = [&](int slot, int t) {
                const int left = nrows - t * kTileRows;
                const uint32_t rows = left <= 0 ? 0u : (left >= kTileRows ? (uint32_t)kTileRows : (uint32_t)left);
                // Every field of the descriptor is wave-uniform; say so, so that it
                // lives in scalar registers.
                const uint64_t base = (uint64_t)(uintptr_t)chunk_base + (uint64_t)t * kTileRows * stride_bytes;
                const uint64_t ubase = (uint64_t)wave_uniform((uint32_t)base) |
                                       ((uint64_t)wave_uniform((uint32_t)(base >> 32)) << 32);
                const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
                    reinterpret_cast<void *>((uintptr_t)ubase), (short)0,
                    (int)wave_uniform(rows * stride_bytes), kBufferWord3);
#pragma unroll
                for (int s = 0; s < NKS; ++s) {
                    const uint32_t vo = s == NKS - 1 ? voff_last : voff + s * 64u;
                    buf[slot][s] = __builtin_bit_cast(
                        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)vo, 0, 0));
                }
            };
            auto consume = [&](int slot, int t) {
                const int left = nrows - t * kTileRows;
#pragma unroll
                for (int qt = 0; qt < NQT; ++qt) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < NKS; ++s) acc = mfma16x16x32<BF16>(qf[qt][s], buf[slot][s], acc);
                    if (left < kTileRows) {
                        const bool ok = row_in_tile < left;
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[r] = ok ? acc[r] : NEG_INF;
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) rmax[qt][r] = fmax_plain(rmax[qt][r], acc[r]);
                }
            };

            // Software pipeline, P tiles deep: the loads of tile t + P are issued as
            // soon as tile t has been consumed. The scheduling barriers keep the
            // issue order fixed, so each consume waits only for its own tile's loads.
#pragma unroll
            for (int p = 0; p < P; ++p) {
                issue(p, p);
                __builtin_amdgcn_sched_barrier(0);
            }
            for (int t0 = 0; t0 < ntiles; t0 += P) {
#pragma unroll
                for (int p = 0; p < P; ++p) {
                    consume(p, t0 + p);
                    __builtin_amdgcn_sched_barrier(0);
                    issue(p, t0 + p + P);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }

#pragma unroll
            for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
                for (int r = 0; r < 4; ++r) rmax[qt][r] = row16_max(rmax[qt][r]);

            if (K == 1) {
#pragma unroll
                for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int q = (grp * NQT + qt) * kTileRows + kgroup * 4 + r;
                        lane_sum += q < Lq ? rmax[qt][r] : 0.0f;
                    }
            } else if (row_in_tile == 0) {
#pragma unroll
                for (int qt = 0; qt < NQT; ++qt) {
                    const int q = (grp * NQT + qt) * kTileRows + kgroup * 4;
                    f32x4 v = {rmax[qt][0], rmax[qt][1], rmax[qt][2], rmax[qt][3]};
                    *reinterpret_cast<f32x4 *>(a.partials + (size_t)g * lq_pad + q) = v;
                }
            }
        }

        if (K > 1) {
            // Publish this chunk's maxima, then count it in; the last chunk combines.
            __threadfence();
            uint32_t prev = 0;
            if (lane == 0) prev = atomicAdd(a.arrive + di, 1u);
            prev = wave_uniform(__builtin_amdgcn_readlane(prev, 0));
            if (prev != K - 1) continue;
            __threadfence();
            const uint32_t first = g - c;
            for (int q = lane; q < lq_pad; q += kWave) {
                float m = NEG_INF;
                for (uint32_t k = 0; k < K; ++k)
                    m = fmax_plain(m, __builtin_nontemporal_load(a.partials + (size_t)(first + k) * lq_pad + q));
                s_comb[wave][q] = m;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            for (int grp = 0; grp < a.ngroups; ++grp)
#pragma unroll
                for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int q = (grp * NQT + qt) * kTileRows + kgroup * 4 + r;
                        lane_sum += q < Lq ? s_comb[wave][q] : 0.0f;
                    }
            __builtin_amdgcn_wave_barrier();
        }

        // Fixed-order sum over the four lane groups.
        const float s0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lane_sum), 0));
        const float s1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lane_sum), 16));
        const float s2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lane_sum), 32));
        const float s3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lane_sum), 48));
        if (lane == 0) a.scores[doc] = ((s0 + s1) + s2) + s3;
    }
}

}  // namespace maxsim
