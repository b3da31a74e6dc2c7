// MaxSim score kernel for gfx950 (CDNA4), one instance per (query format, doc storage,
// K-steps, query tiles per group).
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
//   - Each wave runs its items as one continuous stream of tiles: the last pipeline
//     slots of one item already load the next item's first tiles, and descriptors are
//     fetched two items ahead, so the load pipeline never drains between items.
//   - Q is staged once per workgroup into LDS, zero-padded to 16-row tiles and
//     32-column K-steps (when the padded tile fits 64 KB; a larger query's fragments
//     are read from global memory). Each wave keeps its MFMA A-fragments of one group
//     of up to NQT query tiles in registers; with one group (every Lq * d that fits
//     128 VGPRs) they are loaded once, at the start, and the doc-tile slots then reuse
//     the query's LDS.
//   - Doc rows are read in 16-row tiles with non-temporal LDS-DMA buffer loads
//     (buffer_load ... lds): 16 bytes per lane go straight into the wave's LDS slot,
//     lane-ordered, so no registers hold tiles in flight and the pipeline depth is set
//     by LDS. Each lane fetches the global chunk that belongs at its LDS position under
//     an XOR-swizzled row layout (conflict-free fragment reads); 16 lanes still read
//     one contiguous run of a row. Lanes then read the B-fragment layout of
//     v_mfma_f32_16x16x32_{f16,bf16}: lane l, K-step s gets row (l % 16), columns
//     8 (4 s + l / 16) .. +7. A and B use the same lane -> column mapping, so the dot
//     products are exact dot products whatever the order inside a fragment.
//   - The row address is a 64-bit scalar base (doc offset widened to int64 before it
//     is multiplied by the stride, as the page's kernel does) plus a 32-bit per-lane
//     offset. Each tile gets a buffer descriptor whose size covers only the tile's
//     valid rows, so rows past the end of the doc are never fetched and land as zeros;
//     chunks past the row's d columns are pushed out of range the same way.
//   - Docs may be stored as FP8 E4M3 (half the bytes of the bandwidth-bound stream):
//     tiles are loaded as bytes, and each lane converts its 8-byte B fragment to Q's
//     format with the hardware converter (exact), so the MFMA and the fp32
//     accumulation are the 16-bit path's; the doc tensor's scale multiplies the sum.
//   - S = Qtile . Dtile^T lands with lane l holding doc row (l % 16) and query rows
//     4 (l / 16) + j, j < 4. The accumulator of an invalid doc row (past the doc's
//     end) starts at -inf instead of 0, which keeps it at -inf; then an element-wise
//     running max per lane; at the end of the item four DPP row_ror steps
//     (8, 4, 2, 1) take the max over the 16 doc-row lanes.
//   - Several queries may score the same docs in one launch: their rows are stacked,
//     each query starting on a 16-row tile, so every doc tile is loaded once and
//     multiplied by all of them; a table of query tiles says where each query ends.
//   - Or several queries may share a launch with each doc scored against its own (a
//     "pairs" plan: the descriptor carries the query's rows); a wave then reloads its
//     query fragments only when the query changes between its items.
//   - Query rows past their query's end (zero padding) are masked to 0 and each
//     query's per-row maxima are summed in one fixed order (ascending query tile, then
//     j, then the four lane groups), whether the doc was scored in one item or several,
//     so scores do not depend on how the schedule chunked the doc, nor on which other
//     queries shared the launch.
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
// Cache policy of the doc-row loads: non-temporal (streaming). Every doc byte is read
// exactly once; with the default policy the same stream runs ~12 % slower on MI355X
// (6.2 vs 6.9 TB/s measured for plain 1 KB-per-instruction reads).
constexpr int kDocLoadPolicy = 2;
// s_waitcnt operands (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt
// 11:8; a counter at its maximum is not waited for).
constexpr int wait_vmcnt(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
constexpr int kWaitAllVmem = wait_vmcnt(0);
constexpr int kWaitAllLgkm = 0xC07F;  // lgkmcnt 0

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

__device__ __forceinline__ uint64_t wave_uniform64(uint64_t v)
{
    return (uint64_t)wave_uniform((uint32_t)v) | ((uint64_t)wave_uniform((uint32_t)(v >> 32)) << 32);
}

// Eight FP8 E4M3 values (two words, lowest byte first) to the eight fp16 or bf16
// halves of one MFMA fragment, exactly (every E4M3 value is representable in both).
template <bool BF16>
__device__ __forceinline__ u32x4 e4m3x8_to_16(uint32_t lo, uint32_t hi)
{
    u32x4 r;
    if constexpr (BF16) {
        r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
        r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
        r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
        r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
    } else {
        r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false));
        r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true));
        r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false));
        r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true));
    }
    return r;
}

// Issue priority from a wave's progress through its share of the static deal: a wave
// that has started fewer of its rounds issues first. The SIMD arbiter otherwise favours
// the oldest waves, so the last workgroup placed on a CU would finish its equal share
// last; this feeds back toward all waves ending together.
__device__ __forceinline__ void progress_priority(uint32_t started, uint32_t rounds)
{
    const uint32_t q = rounds ? (4u * started) / rounds : 3u;
    if (q == 0u) __builtin_amdgcn_s_setprio(3);
    else if (q == 1u) __builtin_amdgcn_s_setprio(2);
    else if (q == 2u) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
}

// MINW: waves per SIMD the register allocation must allow (512 / MINW registers).
// BF16: element format of Q (and of the MFMA). FP8D: docs stored as FP8 E4M3 bytes
// (converted to Q's format per fragment; the score is multiplied by a.doc_scale).
template <int NKS, int NQT, bool BF16, bool FP8D, int P, int MINW>
__global__ void __launch_bounds__(kScoreBlock, MINW)
score_kernel(const ScoreArgs a)
{
    constexpr int DPAD = NKS * kStepK;
    // Doc rows are loaded with LDS-DMA straight into the wave's P slots. A slot holds SUB
    // 16-row MFMA blocks: 16 rows of 16-bit docs, 32 of FP8 docs (the same bytes).
    constexpr int SUB = score_sub(FP8D);
    constexpr int SROWS = SUB * kTileRows;         // doc rows per slot
    constexpr int CP = dma_row_chunks(NKS, FP8D);  // slot row: 16-byte chunks
    constexpr int TILE_CHUNKS = SROWS * CP;        // 16-byte chunks per slot
    constexpr int NLDD = TILE_CHUNKS / kWave;      // LDS-DMA loads per slot, 64 chunks each
    constexpr int LDQ = DPAD + 8;  // LDS row pitch (halves): 16 B skew against bank conflicts
    constexpr float NEG_INF = -__builtin_huge_valf();

    extern __shared__ __attribute__((aligned(16))) uint16_t qs[];  // [lq_pad][LDQ], then per-wave tiles
    __shared__ BinTables tab;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = (int)wave_uniform(threadIdx.x / kWave);  // uniform: claims and descriptors stay scalar
    const int lq_pad = a.lq_pad;
    const int ngroups = a.ngroups;
    const uint32_t W = gridDim.x * kScoreWaves;
    const uint32_t wid = blockIdx.x * kScoreWaves + wave;

    // ---- stage the query tiles (zero-padded) into LDS when they fit; under a
    // multi-query "pairs" plan every wave reads its current query from global memory.
    const bool pairs = a.hdr->multi_query != 0u;
    const bool stage_q = a.q_in_lds && !pairs;
    if (stage_q) {
        constexpr int CPR = DPAD / 8;  // 16-byte chunks per padded row
        const int n = lq_pad * CPR;
        for (int e = threadIdx.x; e < n; e += kScoreBlock) {
            const int r = e / CPR;
            const int c = e - r * CPR;
            const int T = r / kTileRows;
            const int ri = r - T * kTileRows;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (ri < a.qt.rows(T) && c * 8 < a.d)
                v = *reinterpret_cast<const u32x4 *>(a.Q + ((size_t)a.qt.src(T) + ri) * a.d + c * 8);
            *reinterpret_cast<u32x4 *>(qs + r * LDQ + c * 8) = v;
        }
    }
    if (wave == 0) fill_bin_tables(a.hdr, W, NQT, tab, lane);
    __syncthreads();

    const LaneBins L = lane_bins(tab, lane);
    const uint32_t total = tab.total_claims;

    // ---- per-lane load and staging geometry
    const uint32_t stride_bytes = (uint32_t)a.stride_bytes;
    const uint32_t tile_bytes = (uint32_t)SROWS * stride_bytes;  // bytes between slots of a doc
    const int row_in_tile = lane & 15;
    const int kgroup = lane >> 4;
    const int C = FP8D ? a.d / 16 : a.d / 8;  // 16-byte chunks per doc row
    // The staged query stays in LDS for the whole launch for FP8 docs and for a query of
    // several register groups; otherwise (one group, 16-bit docs) the waves load their
    // fragments right away and the doc-tile slots reuse its LDS.
    const bool q_keep = a.q_in_lds && ngroups > 1;
    u32x4 *const tiles = reinterpret_cast<u32x4 *>(qs + (q_keep ? lq_pad * LDQ : 0));

    // Slot row r keeps its chunk c at position r * CP + (c ^ dma_swizzle(r, CP)), so the
    // 16 rows that one fragment read touches fall in distinct banks; load s, lane l fills
    // position 64 s + l (LDS-DMA writes lane-ordered). Chunks past the row (c >= C) and
    // rows past the tile's valid rows are outside the descriptor's range and land as
    // zeros, so K-columns past d need no masking.
    u32x4 *const slots = tiles + wave * (P * TILE_CHUNKS);
    uint32_t dma_off[NLDD];
#pragma unroll
    for (int s = 0; s < NLDD; ++s) {
        const int q = s * kWave + lane;
        const int row = q / CP;
        const int c = (q % CP) ^ dma_swizzle(row, CP);
        dma_off[s] = c < C ? (uint32_t)row * stride_bytes + (uint32_t)c * 16u : (uint32_t)SROWS * stride_bytes;
    }
    // B fragment of K-step s, row row_in_tile of block h: 16-bit docs, chunk kgroup + 4 s
    // (8 columns); FP8 docs, the 8 bytes at half kgroup % 2 of chunk kgroup / 2 + 2 s.
    int rd_dma[SUB][NKS];
#pragma unroll
    for (int h = 0; h < SUB; ++h)
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            const int c = FP8D ? (kgroup >> 1) + 2 * s : kgroup + 4 * s;
            const int row = h * kTileRows + row_in_tile;
            rd_dma[h][s] = row * CP + (c ^ dma_swizzle(row, CP));
        }
    const int rd_half = (kgroup & 1) * 8;  // FP8 docs: byte offset in the chunk

    // Query fragments of register group grp: from LDS when the query tiles are staged
    // there, else from global memory, by the tile table or, under a pairs plan, for the
    // item's query at rows [q_off, q_off + q_len) of Q.
    u32x4 qf[NQT][NKS];
    auto load_q = [&](int grp, int q_off, int q_len) {
        if (stage_q) {
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt) {
                const int row = (grp * NQT + qt) * kTileRows + row_in_tile;
#pragma unroll
                for (int s = 0; s < NKS; ++s)
                    qf[qt][s] = *reinterpret_cast<const u32x4 *>(qs + row * LDQ + (s * 4 + kgroup) * 8);
            }
        } else {
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt) {
                const int T = grp * NQT + qt;
                const int row = T * kTileRows + row_in_tile;
                const bool row_ok = pairs ? row < q_len : row_in_tile < a.qt.rows(T);
                const size_t src = pairs ? (size_t)q_off + row : (size_t)a.qt.src(T) + row_in_tile;
#pragma unroll
                for (int s = 0; s < NKS; ++s) {
                    const int col = (s * 4 + kgroup) * 8;
                    u32x4 v = {0u, 0u, 0u, 0u};
                    if (row_ok && col < a.d) v = *reinterpret_cast<const u32x4 *>(a.Q + src * a.d + col);
                    qf[qt][s] = v;
                }
            }
            // The fragments are waited for here, on this path alone. Otherwise the
            // compiler's wait-count analysis, which cannot tell the two paths apart where
            // they meet at the tile loop, makes every pass of that loop wait for all of
            // the wave's loads in flight, its prefetched doc tiles too.
            __builtin_amdgcn_s_waitcnt(kWaitAllVmem);
        }
    };
    int loaded_query = -1;  // query whose fragments qf holds (one register group only)

    // ---- the wave's items: round r deals item r W + w to wave w (r even) or to wave
    // W-1-w (r odd). Workgroups are placed on the eight XCDs round robin (block b on XCD
    // b % 8), and waves on the odd-numbered XCDs stream HBM ~8 % slower, so when the grid
    // is a multiple of 8 blocks the rounds come in periods of kDealPeriod: in the last
    // round of a period only the waves of even blocks take an item (numbered by their
    // rank among those waves). A slow wave then gets 11 items for a fast wave's 12. Not
    // under a pairs plan: its waves wait for each new query's fragments with the tile
    // loads drained, a latency that the XCDs share alike (measured: the weighting made
    // a pairs batch ~1 % slower, single-query launches ~1 % faster).
    const bool weighted = !pairs && (gridDim.x & 7u) == 0u;
    const bool slow = weighted && (blockIdx.x & 1u);
    const uint32_t per_period = weighted ? (kDealPeriod - 1u) * W + W / 2u : W;
    const uint32_t my_rounds = weighted ? (slow ? kDealPeriod - 1u : kDealPeriod) : 1u;
    const uint32_t fast_rank = (blockIdx.x >> 1) * kScoreWaves + wave;
    auto claim_of = [&](uint32_t r) -> uint32_t {
        const uint32_t p = r / my_rounds;
        const uint32_t j = r - p * my_rounds;
        unsigned long long g;
        if (!weighted) {
            g = (unsigned long long)r * W + ((r & 1u) ? (W - 1u - wid) : wid);
        } else {
            const uint32_t round = p * kDealPeriod + j;  // parity sets the direction
            g = (unsigned long long)p * per_period;
            if (j < kDealPeriod - 1u)
                g += (unsigned long long)j * W + ((round & 1u) ? (W - 1u - wid) : wid);
            else
                g += (unsigned long long)(kDealPeriod - 1u) * W + ((round & 1u) ? (W / 2u - 1u - fast_rank) : fast_rank);
        }
        return g < 0xFFFFFFFFull ? (uint32_t)g : 0xFFFFFFFFu;  // past the last claim: invalid
    };
    struct Span {  // one work item, resolved to rows; every field wave-uniform
        uint64_t base;   // address of its first row
        int nrows;
        int ntiles;
        int doc;
        uint32_t K;      // chunks of its doc (1: the item is the whole doc)
        uint32_t g;      // claim index (slot of its partial maxima when K > 1)
        int query;       // its doc's query: rows [q_off, q_off + q_len) of Q
        int q_off;
        int q_len;       // -1: invalid query, the doc's score is NaN
        bool valid;
    };
    auto fetch = [&](uint32_t g, Item &it, DocDesc &dd) {
        if (g < total) {
            it = locate_claim(L, lane, g);
            dd = load_desc(a.desc, it.di);
        }
    };
    auto resolve = [&](uint32_t g, const Item &it, const DocDesc &dd) -> Span {
        Span sp;
        sp.valid = g < total;
        sp.g = g;
        if (!sp.valid) {
            sp.base = (uint64_t)(uintptr_t)a.docs;
            sp.nrows = sp.ntiles = sp.doc = 0;
            sp.query = sp.q_off = sp.q_len = 0;
            sp.K = 1;
            return sp;
        }
        sp.doc = (int)wave_uniform((uint32_t)dd.doc);
        sp.query = (int)wave_uniform((uint32_t)dd.query);
        sp.q_off = (int)wave_uniform((uint32_t)dd.q_offset);
        sp.q_len = (int)wave_uniform((uint32_t)dd.q_length);
        const int64_t off = (int64_t)(int32_t)wave_uniform((uint32_t)dd.offset);
        const int len = (int)wave_uniform((uint32_t)dd.length);
        const uint32_t nt = wave_uniform((uint32_t)dd.tiles);
        sp.K = it.K;
        // Tiles [t_begin, t_end) of the doc's nt tiles; never empty unless nt == 0.
        const uint32_t t_begin = (uint32_t)(((unsigned long long)it.c * nt) / it.K);
        const uint32_t t_end = (uint32_t)(((unsigned long long)(it.c + 1) * nt) / it.K);
        sp.ntiles = (int)(t_end - t_begin);
        const int row0 = (int)t_begin * kTileRows;
        sp.nrows = (len < (int)t_end * kTileRows ? len : (int)t_end * kTileRows) - row0;
        sp.base = (uint64_t)(uintptr_t)a.docs + (uint64_t)((off + row0) * a.stride_bytes);
        return sp;
    };

    // Loads of slot-tile t (rows [t SROWS, (t + 1) SROWS) of a span) into pipeline slot
    // `slot`. The descriptor covers only the valid rows (none for t past the span, or
    // for an invalid span).
    auto issue = [&](int slot, uint64_t base, int nrows, int t) {
        // Valid rows, clamped in two steps on scalar registers (one clamp would become a
        // vector med3, a vector multiply and a readfirstlane).
        const int left = (int)wave_uniform((uint32_t)(nrows - t * SROWS));
        const int lo = (int)wave_uniform((uint32_t)(left > 0 ? left : 0));
        const uint32_t rows = (uint32_t)(lo < SROWS ? lo : SROWS);
        // t < 2^27 and a slot is at most 32 rows of 2^24 bytes: a 32 x 32 -> 64-bit product.
        const uint64_t ub = wave_uniform64(base + (uint64_t)(uint32_t)t * (uint64_t)tile_bytes);
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            reinterpret_cast<void *>((uintptr_t)ub), (short)0, (int)(rows * stride_bytes), kBufferWord3);
        // The slot's previous tile has been read (its products were issued after the
        // reads completed); the wait makes that explicit before it is overwritten.
        __builtin_amdgcn_s_waitcnt(kWaitAllLgkm);
#pragma unroll
        for (int s = 0; s < NLDD; ++s)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc, (__attribute__((address_space(3))) void *)(slots + slot * TILE_CHUNKS + s * kWave), 16,
                (int)dma_off[s], 0, 0, kDocLoadPolicy);
    };

    float rmax[NQT][4];
    // Slot-tile t (in slot `slot`) of a span with `nrows` rows: stage, multiply, max, one
    // 16-row block at a time (a block past the span's rows is skipped, except the first).
    auto consume = [&](int slot, int nrows, int t) {
        // Every slot is refilled in turn, so exactly NLDD (P - 1) loads were issued after
        // this slot's; once no more are in flight, its rows are in LDS.
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(NLDD * (P - 1)));
#pragma unroll
        for (int h = 0; h < SUB; ++h) {
            const int left = (int)wave_uniform((uint32_t)(nrows - (t * SUB + h) * kTileRows));
            if (h > 0 && left <= 0) break;
            u32x4 bf[NKS];
#pragma unroll
            for (int s = 0; s < NKS; ++s) {
                if constexpr (FP8D) {
                    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                    const u32x2 v = *reinterpret_cast<const u32x2 *>(
                        reinterpret_cast<const char *>(slots + slot * TILE_CHUNKS + rd_dma[h][s]) + rd_half);
                    bf[s] = e4m3x8_to_16<BF16>(v[0], v[1]);
                } else {
                    bf[s] = slots[slot * TILE_CHUNKS + rd_dma[h][s]];
                }
            }
            // The accumulator starts at 0 for this lane's doc row if the row is valid and
            // at -inf if not (past the doc end): -inf + a finite dot stays -inf, so invalid
            // rows never win the max and need no masking.
            const float c0 = row_in_tile < left ? 0.0f : NEG_INF;
            // Query tile qt's products go into one accumulator while tile qt - 1's, in the
            // other, are folded into the running max: the max waits on finished MFMAs.
            f32x4 acc[2];
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt) {
                f32x4 a = {c0, c0, c0, c0};
#pragma unroll
                for (int s = 0; s < NKS; ++s) a = mfma16x16x32<BF16>(qf[qt][s], bf[s], a);
                acc[qt & 1] = a;
                if (qt > 0) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        rmax[qt - 1][i] = __builtin_fmaxf(rmax[qt - 1][i], acc[(qt - 1) & 1][i]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) rmax[NQT - 1][i] = __builtin_fmaxf(rmax[NQT - 1][i], acc[(NQT - 1) & 1][i]);
        }
    };

    // Descriptor queue: cur and nxt resolved, the one after that in flight.
    uint32_t r = 0;
    Item i0{}, i1{}, i2{};
    DocDesc d0{}, d1{}, d2{};
    const uint32_t g0 = claim_of(r++);
    const uint32_t g1 = claim_of(r++);
    fetch(g0, i0, d0);
    fetch(g1, i1, d1);
    Span cur = resolve(g0, i0, d0);
    Span nxt = resolve(g1, i1, d1);
    uint32_t g2 = g1;

    if (stage_q && !q_keep) {
        // One register group over a staged query: load it now, before the tile slots
        // overwrite its LDS (every wave has its fragments once the barrier is passed).
        load_q(0, 0, 0);
        loaded_query = 0;
        __syncthreads();
    }

#pragma unroll
    for (int p = 0; p < P; ++p) {
        issue(p, cur.base, cur.nrows, p);
        __builtin_amdgcn_sched_barrier(0);
    }

    // Sub-items: (item, query group). The tiles of a sub-item run as one pipelined
    // stream that ends by loading the first tiles of the next sub-item (the same item's
    // next query group, or the next item).
    int grp = 0;
    float lane_sum = 0.0f;
    // Items this wave gets in the deal, about total * my_rounds / per_period.
    const uint32_t rounds =
        (uint32_t)(((unsigned long long)total * my_rounds + per_period - 1u) / per_period);
    while (wave_uniform(cur.valid ? 1u : 0u)) {
        if (grp == 0) {
            g2 = claim_of(r++);
            fetch(g2, i2, d2);
            progress_priority(r, rounds);
        }
        if (ngroups > 1 || cur.query != loaded_query) {
            load_q(grp, cur.q_off, cur.q_len);
            loaded_query = ngroups > 1 ? -1 : cur.query;
        }
        // Everything that steers the tile loop is wave-uniform; restate it so that it
        // stays in scalar registers (the loads' descriptors are built from it).
        const bool more_groups = grp + 1 < ngroups;
        const uint64_t c_base = wave_uniform64(cur.base);
        const int c_rows = (int)wave_uniform((uint32_t)cur.nrows);
        // An empty doc runs as one slot with no valid rows (zero-size loads, all
        // accumulators -inf): its maxima stay -inf, and the loop shape never changes.
        // The span's 16-row tiles fill ceil(ntiles / SUB) slots.
        const int c_tiles = (int)wave_uniform((uint32_t)(cur.ntiles > 0 ? (cur.ntiles + SUB - 1) / SUB : 1));
        const uint64_t n_base = wave_uniform64(more_groups ? cur.base : nxt.base);
        const int n_rows = (int)wave_uniform((uint32_t)(more_groups ? cur.nrows : nxt.nrows));

#pragma unroll
        for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
            for (int i = 0; i < 4; ++i) rmax[qt][i] = NEG_INF;

        // Software pipeline, P tiles deep, over the span's tiles rounded up to P; the
        // scheduling barriers keep the issue order fixed, so each tile waits only for
        // its own loads.
        const int ntp = (c_tiles + P - 1) / P * P;
        for (int t0 = 0; t0 < ntp; t0 += P) {
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const int t = t0 + p;
                if (t < c_tiles) consume(p, c_rows, t);
                __builtin_amdgcn_sched_barrier(0);
                // Tile t + P of this sub-item, or, past its end, of the next one.
                const int ti = t + P;
                const bool tail = ti >= ntp;
                issue(p, tail ? n_base : c_base, tail ? n_rows : c_rows, tail ? ti - ntp : ti);
                __builtin_amdgcn_sched_barrier(0);
            }
        }

#pragma unroll
        for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
            for (int i = 0; i < 4; ++i) rmax[qt][i] = row16_max(rmax[qt][i]);

        if (cur.K == 1) {
            // Rows past the end of their query add nothing; each query's sum is stored
            // at its last tile: lanes add their rows in ascending order, then the four
            // lane groups in a fixed order.
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt) {
                const int T = grp * NQT + qt;
                int nr, end;
                if (pairs) {
                    const int left = cur.q_len - T * kTileRows;
                    nr = left < 0 ? 0 : (left > kTileRows ? kTileRows : left);
                    end = T == ngroups * NQT - 1 ? 0 : -1;
                } else {
                    nr = a.qt.rows(T);
                    end = a.qt.end(T);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) lane_sum += kgroup * 4 + i < nr ? rmax[qt][i] : 0.0f;
                if (end >= 0) {
                    const int ls = __builtin_bit_cast(int, lane_sum);
                    const float s0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ls, 0));
                    const float s1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ls, 16));
                    const float s2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ls, 32));
                    const float s3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ls, 48));
                    // NaN for an invalid query, chosen and stored as bits (this code is
                    // compiled without NaN semantics for its max steps).
                    float sum = ((s0 + s1) + s2) + s3;
                    if constexpr (FP8D) sum *= a.doc_scale;
                    const uint32_t v = pairs && cur.q_len < 0 ? kNaNBits : __builtin_bit_cast(uint32_t, sum);
                    if (lane == 0)
                        reinterpret_cast<uint32_t *>(a.scores)[(size_t)end * a.qt.score_stride + cur.doc] = v;
                    lane_sum = 0.0f;
                }
            }
        } else if (row_in_tile == 0) {
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt) {
                const int q = (grp * NQT + qt) * kTileRows + kgroup * 4;
                f32x4 v = {rmax[qt][0], rmax[qt][1], rmax[qt][2], rmax[qt][3]};
                *reinterpret_cast<f32x4 *>(a.partials + (size_t)cur.g * lq_pad + q) = v;
            }
        }
        if (more_groups) {
            ++grp;
            continue;
        }
        // (split docs: the combine kernel finishes them)
        lane_sum = 0.0f;
        grp = 0;
        cur = nxt;
        nxt = resolve(g2, i2, d2);
    }
}

}  // namespace maxsim
