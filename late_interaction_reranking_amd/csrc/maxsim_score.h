// MaxSim score kernel for gfx950 (CDNA4), one instance per (format, K-steps, query
// tiles per group).
//
// Operation (Flash-MaxSim rerank page, docs.vllm.ai,
// vllm.v1.pool.flash_maxsim.flash_maxsim_rerank, module description and section
// `_maxsim_rerank_kernel`): score_i = sum over query rows q of the max over doc i's
// rows t of Q[q] . X[off_i + t], fp16/bf16 inputs, fp32 products and sums.
//
// Mapping onto the hardware:
//   - Persistent workgroups of 4 waves, as many as fit on every CU. The work items (a
//     doc, or a chunk of a long doc's tiles) of the length-binned schedule that the
//     plan kernels wrote, longest bins first, are dealt to the W waves in rounds, in
//     alternating direction (round r gives item r W + w to wave w, or to wave W-1-w
//     when r is odd), so every wave gets a similar mix of long and short items. No
//     atomics: a shared claim counter serialises across the chip's eight XCDs.
//     Each wave loads the descriptor of its next item while it scores the current one.
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
//   - A doc split into K chunks: each chunk writes its per-row maxima to its own slot
//     with plain stores; the combine kernel, launched next on the same stream, takes
//     the max over the K slots (exact, so order-free) and does the same fixed-order
//     sum. The kernel boundary is the only synchronisation: no fences in the hot loop
//     (on this chip a device-scope fence writes back and invalidates the XCD's L2).
#pragma once

#include "maxsim_common.h"
#include "maxsim_sched.h"

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
    __shared__ BinTables tab;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int Lq = a.Lq;
    const int lq_pad = a.lq_pad;
    const uint32_t W = gridDim.x * kScoreWaves;
    const uint32_t wid = blockIdx.x * kScoreWaves + wave;

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
    if (threadIdx.x == 0) fill_bin_tables(a.hdr, W, tab);
    __syncthreads();

    const LaneBins L = lane_bins(tab, lane);
    const uint32_t total = tab.total_claims;

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

    // Round r deals item r W + w to wave w (r even) or to wave W-1-w (r odd).
    auto claim_of = [&](uint32_t r) -> uint32_t {
        return r * W + ((r & 1u) ? (W - 1u - wid) : wid);
    };
    uint32_t r = 0;
    uint32_t g = claim_of(0);
    Item nit{};
    DocDesc nd{};
    if (g < total) {
        nit = locate_claim(L, lane, g);
        nd = a.desc[nit.di];
    }

    while (g < total) {
        const Item it = nit;
        const int doc = (int)wave_uniform((uint32_t)nd.doc);
        const int64_t off = (int64_t)(int32_t)wave_uniform((uint32_t)nd.offset);
        const int len = (int)wave_uniform((uint32_t)nd.length);
        const uint32_t nt = wave_uniform((uint32_t)nd.tiles);
        const uint32_t K = it.K;
        const uint32_t c = it.c;
        const uint32_t g_cur = g;

        // Next item's descriptor, in flight while this one is scored.
        g = claim_of(++r);
        if (g < total) {
            nit = locate_claim(L, lane, g);
            nd = a.desc[nit.di];
        }

        // Tiles [t_begin, t_end) of the doc's nt tiles; never empty unless nt == 0.
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
                for (int i = 0; i < 4; ++i) rmax[qt][i] = NEG_INF;

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
                        for (int i = 0; i < 4; ++i) acc[i] = ok ? acc[i] : NEG_INF;
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) rmax[qt][i] = fmax_plain(rmax[qt][i], acc[i]);
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
                for (int i = 0; i < 4; ++i) rmax[qt][i] = row16_max(rmax[qt][i]);

            if (K == 1) {
#pragma unroll
                for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int q = (grp * NQT + qt) * kTileRows + kgroup * 4 + i;
                        lane_sum += q < Lq ? rmax[qt][i] : 0.0f;
                    }
            } else if (row_in_tile == 0) {
#pragma unroll
                for (int qt = 0; qt < NQT; ++qt) {
                    const int q = (grp * NQT + qt) * kTileRows + kgroup * 4;
                    f32x4 v = {rmax[qt][0], rmax[qt][1], rmax[qt][2], rmax[qt][3]};
                    *reinterpret_cast<f32x4 *>(a.partials + (size_t)g_cur * lq_pad + q) = v;
                }
            }
        }
        if (K > 1) continue;  // the combine kernel finishes split docs

        // Fixed-order sum over the four lane groups.
        const float s0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lane_sum), 0));
        const float s1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lane_sum), 16));
        const float s2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lane_sum), 32));
        const float s3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lane_sum), 48));
        if (lane == 0) a.scores[doc] = ((s0 + s1) + s2) + s3;
    }
}

}  // namespace maxsim
