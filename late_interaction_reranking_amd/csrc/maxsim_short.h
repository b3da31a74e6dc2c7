// One-launch MaxSim for batches of short docs: one workgroup per doc, no schedule, no
// combine launch and no workspace.
//
// Operation (Flash-MaxSim rerank page, docs.vllm.ai,
// vllm.v1.pool.flash_maxsim.flash_maxsim_rerank, module description and section
// `_maxsim_rerank_kernel`): score_i = sum over query rows q of the max over doc i's rows
// t of Q[q] . X[off_i + t]; one program per doc, as in the page's kernel.
//
// Workgroup b scores doc b: its four waves take the doc's 16-row tiles round robin
// (wave w: tiles w, w + 4, ...), each streaming them through its own LDS-DMA slots
// exactly as the scheduled score kernel does (same slot layout, same MFMA fragments,
// same running max), then the waves' per-row maxima meet in LDS and wave 0 sums them in
// the scheduled kernel's fixed order. The max is exact and the order of the sum is the
// same, so a score is bitwise the one the scheduled path gives. The query must fit one
// register group (NQT query tiles of NKS K-steps). The time of a launch follows its
// longest doc: long or very unequal docs belong on the scheduled path.
//
// FP8D: docs stored as FP8 E4M3 bytes, staged and converted to Q's format per fragment
// as in the score kernel; the sum is multiplied by a.doc_scale after the same fixed-order
// sum, as the scheduled path does.
#pragma once

#include "maxsim_score.h"

namespace maxsim {

template <int NKS, int NQT, bool BF16, bool FP8D, int P, int MINW>
__global__ void __launch_bounds__(kScoreBlock, MINW)
short_kernel(const ShortArgs a)
{
    constexpr int DPAD = NKS * kStepK;
    constexpr int LDQ = DPAD + 8;                 // Q row pitch in LDS (halves), as the score kernel's
    constexpr int CP = dma_row_chunks(NKS, FP8D);
    constexpr int NLDD = CP / 4;
    constexpr int TILE_CHUNKS = kTileRows * CP;
    constexpr int LQP = NQT * kTileRows;          // padded query rows
    constexpr float NEG_INF = -__builtin_huge_valf();

    extern __shared__ __attribute__((aligned(16))) uint16_t qs[];  // Q tile, then the tile slots over it
    __shared__ float part[kScoreWaves][LQP];                       // per-wave row maxima of the doc

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = (int)wave_uniform(threadIdx.x / kWave);
    const int row_in_tile = lane & 15;
    const int kgroup = lane >> 4;

    // ---- the query: zero-padded tile in LDS, then each wave's A-fragments in registers
    {
        constexpr int CPR = DPAD / 8;
        for (int e = threadIdx.x; e < LQP * CPR; e += kScoreBlock) {
            const int r = e / CPR;
            const int c = e - r * CPR;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (r < a.Lq && c * 8 < a.d) v = *reinterpret_cast<const u32x4 *>(a.Q + (size_t)r * a.d + c * 8);
            *reinterpret_cast<u32x4 *>(qs + r * LDQ + c * 8) = v;
        }
    }
    __syncthreads();
    u32x4 qf[NQT][NKS];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
        for (int s = 0; s < NKS; ++s)
            qf[qt][s] = *reinterpret_cast<const u32x4 *>(qs + (qt * kTileRows + row_in_tile) * LDQ + (s * 4 + kgroup) * 8);
    __syncthreads();  // the tile slots reuse the query's LDS

    // ---- LDS-DMA slots and fragment addresses (the score kernel's layout)
    const uint32_t stride_bytes = (uint32_t)a.stride_bytes;
    const uint32_t tile_bytes = (uint32_t)kTileRows * stride_bytes;
    const int C = FP8D ? a.d / 16 : a.d / 8;  // 16-byte chunks per doc row
    u32x4 *const slots = reinterpret_cast<u32x4 *>(qs) + wave * (P * TILE_CHUNKS);
    uint32_t dma_off[NLDD];
#pragma unroll
    for (int s = 0; s < NLDD; ++s) {
        const int q = s * kWave + lane;
        const int row = q / CP;
        const int c = (q % CP) ^ dma_swizzle(row, CP);
        dma_off[s] = c < C ? (uint32_t)row * stride_bytes + (uint32_t)c * 16u : (uint32_t)kTileRows * stride_bytes;
    }
    // B fragment of K-step s: 16-bit docs, chunk kgroup + 4 s; FP8 docs, the 8 bytes at
    // half kgroup % 2 of chunk kgroup / 2 + 2 s.
    int rd_dma[NKS];
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
        const int c = FP8D ? (kgroup >> 1) + 2 * s : kgroup + 4 * s;
        rd_dma[s] = row_in_tile * CP + (c ^ dma_swizzle(row_in_tile, CP));
    }
    const int rd_half = (kgroup & 1) * 8;

    for (uint32_t doc = blockIdx.x; doc < (uint32_t)a.B; doc += gridDim.x) {
        typedef __attribute__((address_space(4))) const int32_t ConstI32;
        const int64_t off = (int64_t)((ConstI32 *)a.offsets)[doc];
        const int32_t len_raw = ((ConstI32 *)a.lengths)[doc];
        const int len = len_raw > 0 ? len_raw : 0;
        const int nt = (len + kTileRows - 1) / kTileRows;
        const int cnt = nt > wave ? (nt - wave + kScoreWaves - 1) / kScoreWaves : 0;  // this wave's tiles
        const uint64_t base = (uint64_t)(uintptr_t)a.docs + (uint64_t)(off * a.stride_bytes);

        // Tile k of this wave (doc tile wave + 4 k) into slot `slot`; zero-size past its tiles.
        auto issue = [&](int slot, int k) {
            const int t = wave + kScoreWaves * k;
            // Valid rows, clamped in two steps on scalar registers (as in the score kernel).
            const int left = (int)wave_uniform((uint32_t)(k < cnt ? len - t * kTileRows : 0));
            const int lo = (int)wave_uniform((uint32_t)(left > 0 ? left : 0));
            const uint32_t rows = (uint32_t)(lo < kTileRows ? lo : kTileRows);
            const uint64_t ub = wave_uniform64(base + (uint64_t)(uint32_t)(k < cnt ? t : 0) * (uint64_t)tile_bytes);
            const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
                reinterpret_cast<void *>((uintptr_t)ub), (short)0, (int)(rows * stride_bytes), kBufferWord3);
            __builtin_amdgcn_s_waitcnt(kWaitAllLgkm);
#pragma unroll
            for (int s = 0; s < NLDD; ++s)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rsrc, (__attribute__((address_space(3))) void *)(slots + slot * TILE_CHUNKS + s * kWave), 16,
                    (int)dma_off[s], 0, 0, kDocLoadPolicy);
        };

        float rmax[NQT][4];
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
            for (int i = 0; i < 4; ++i) rmax[qt][i] = NEG_INF;

        auto consume = [&](int slot, int k) {
            const int left = len - (wave + kScoreWaves * k) * kTileRows;
            __builtin_amdgcn_s_waitcnt(wait_vmcnt(NLDD * (P - 1)));
            u32x4 bf[NKS];
#pragma unroll
            for (int s = 0; s < NKS; ++s) {
                if constexpr (FP8D) {
                    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                    const u32x2 v = *reinterpret_cast<const u32x2 *>(
                        reinterpret_cast<const char *>(slots + slot * TILE_CHUNKS + rd_dma[s]) + rd_half);
                    bf[s] = e4m3x8_to_16<BF16>(v[0], v[1]);
                } else {
                    bf[s] = slots[slot * TILE_CHUNKS + rd_dma[s]];
                }
            }
            const float c0 = row_in_tile < left ? 0.0f : NEG_INF;
            // Tile qt's products in one accumulator while tile qt - 1's are folded into
            // the running max (as in the score kernel).
            f32x4 acc[2];
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt) {
                f32x4 r = {c0, c0, c0, c0};
#pragma unroll
                for (int s = 0; s < NKS; ++s) r = mfma16x16x32<BF16>(qf[qt][s], bf[s], r);
                acc[qt & 1] = r;
                if (qt > 0) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        rmax[qt - 1][i] = __builtin_fmaxf(rmax[qt - 1][i], acc[(qt - 1) & 1][i]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) rmax[NQT - 1][i] = __builtin_fmaxf(rmax[NQT - 1][i], acc[(NQT - 1) & 1][i]);
        };

        // P tiles deep; every slot is refilled in turn (zero-size loads past the wave's
        // tiles), so each consume waits for exactly its own loads.
#pragma unroll
        for (int p = 0; p < P; ++p) {
            issue(p, p);
            __builtin_amdgcn_sched_barrier(0);
        }
        const int ntp = (cnt + P - 1) / P * P;
        for (int k0 = 0; k0 < ntp; k0 += P) {
#pragma unroll
            for (int p = 0; p < P; ++p) {
                if (k0 + p < cnt) consume(p, k0 + p);
                __builtin_amdgcn_sched_barrier(0);
                issue(p, k0 + p + P);
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        // ---- the doc's row maxima: over the 16 doc-row lanes, then over the 4 waves
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
            for (int i = 0; i < 4; ++i) rmax[qt][i] = row16_max(rmax[qt][i]);
        if (row_in_tile == 0) {
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
                for (int i = 0; i < 4; ++i) part[wave][qt * kTileRows + kgroup * 4 + i] = rmax[qt][i];
        }
        __syncthreads();
        if (wave == 0) {
            // The scheduled kernel's sum: lanes add their rows, query tiles ascending,
            // rows past Lq adding nothing; then lanes 0, 16, 32, 48 in that order.
            float lane_sum = 0.0f;
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt) {
                const int left = a.Lq - qt * kTileRows;
                const int nr = left < 0 ? 0 : (left > kTileRows ? kTileRows : left);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int q = qt * kTileRows + kgroup * 4 + i;
                    float m = part[0][q];
#pragma unroll
                    for (int w = 1; w < kScoreWaves; ++w) m = fmax_plain(m, part[w][q]);
                    lane_sum += kgroup * 4 + i < nr ? m : 0.0f;
                }
            }
            const int ls = __builtin_bit_cast(int, lane_sum);
            const float s0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ls, 0));
            const float s1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ls, 16));
            const float s2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ls, 32));
            const float s3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ls, 48));
            float sum = ((s0 + s1) + s2) + s3;
            if constexpr (FP8D) sum *= a.doc_scale;
            if (lane == 0) a.scores[doc] = sum;
        }
        __syncthreads();  // part is reused by the next doc
    }
}

}  // namespace maxsim
