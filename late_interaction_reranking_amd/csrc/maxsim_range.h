// MaxSim score kernel for single-query batches of at most kRangeMaxDocs docs (one
// register group of query tiles) that schedules itself: one launch, no plan launch.
//
// Operation (Flash-MaxSim rerank page, docs.vllm.ai,
// vllm.v1.pool.flash_maxsim.flash_maxsim_rerank, module description and section
// `_maxsim_rerank_kernel`): score_i = sum over query rows q of the max over doc i's rows
// t of Q[q] . X[off_i + t], fp16/bf16 inputs, fp32 products and sums.
//
// Schedule. The docs' 16-row tiles, taken in doc index order, form one sequence of T
// tiles: doc i holds tiles [S_i, S_i + nt_i), nt_i = ceil(len_i / 16), S the exclusive
// prefix sums. It is cut into W_act ranges of equal size (to one tile): wave w takes
// tiles [floor(w T / W_act), floor((w + 1) T / W_act)), W_act = min(W, T / kMinRangeTiles)
// (at least 1). Every workgroup loads the lengths and forms the cut itself: each thread
// sums the tiles of a contiguous block of up to 32 docs, a block-wide scan gives each
// block's first tile, and each wave finds the block holding its first tile (a count over
// the 256 block starts) and the doc within it (a scan over the block's docs).
// So nothing runs before this launch, and the balance is exact: with a few tiles per
// wave, a deal of whole docs or of chunks leaves the slowest wave about twice the average.
//
// Pieces. A wave's range holds whole docs and, at its two ends, pieces of docs that
// other waves also cover. A whole doc is summed and stored here, as the score kernel
// does. A piece stores its per-row maxima in a slot: the piece that opens the range (a
// doc begun by an earlier wave) in head slot w, the piece that closes it (a doc that a
// later wave continues) in tail slot W_act + w. range_combine_kernel then finds a split
// doc's pieces by the same arithmetic (the tail slot of the wave holding its first tile,
// the head slots of the next waves up to the one holding its last tile), takes the max
// (exact, order-free) and sums in the same fixed order, so the score is bitwise the one
// any other schedule gives.
//
// Pipeline. Each wave runs its range as one stream of tiles through P LDS-DMA slots
// (the score kernel's slot layout, fragments and running max). The issue side walks the
// docs P tiles ahead of the consume side and leaves, per slot, what the consume side
// needs: the tile's valid rows, whether it ends a piece, and the piece's doc and slot.
// Doc boundaries therefore cost no pipeline bubble. The doc lengths and offsets come
// from a window of 64 docs held one per lane (the first filled by the prologue, later
// ones loaded). Tile positions are 64-bit: docs may overlap, so T is bounded only by
// B * 2^27.
#pragma once

#include <type_traits>

#include "maxsim_score.h"

namespace maxsim {

constexpr int kRangeChunksPerThread = 8;                            // most 4-doc chunks a prologue thread sums
constexpr int kRangeMaxBlockDocs = 4 * kRangeChunksPerThread;       // most docs in a thread's block: 32
constexpr int kRangeDocsPerChunkRow = 4 * kScoreBlock;              // docs covered per chunk a thread takes
constexpr int kRangeMaxDocs = kRangeMaxBlockDocs * kScoreBlock;     // docs of a range launch: 8192
constexpr uint32_t kMinRangeTiles = 2;                              // fewest tiles per active wave

struct RangeArgs {
    const uint16_t *Q;             // [Lq, d]
    const char *docs;              // row r at docs + r * stride_bytes
    int64_t stride_bytes;
    const int32_t *offsets;        // [B]
    const int32_t *lengths;        // [B]
    float *scores;                 // [B]
    unsigned long long *scan;      // workspace: S_0 .. S_B (S_B = T) for the combine kernel
    float *partials;               // workspace: [2 W][16 NQT] head slots, then tail slots
    int32_t B, d, Lq;
    uint32_t len_lds;              // byte offset of the prologue's doc lengths in the dynamic LDS
    uint32_t off_lds;              // and of its doc offsets (0: the offsets stay in global memory)
    float doc_scale;               // FP8 docs: multiplies each sum (unused otherwise)
};

struct RangeCombineArgs {
    const unsigned long long *scan;
    const float *partials;
    float *scores;
    int32_t B, Lq, nqt;
    uint32_t waves;                // W of the range launch
    float doc_scale;
};

// Wave w's first tile when T tiles are cut into W_act ranges (T <= B 2^27 <= 2^40 and
// w, W_act < 2^16: the products stay below 2^56).
__host__ __device__ inline unsigned long long range_start(uint32_t w, unsigned long long T, uint32_t wact)
{
    return ((unsigned long long)w * T) / wact;
}

// The wave whose range holds tile t (t < T): the largest w with range_start(w) <= t.
__host__ __device__ inline uint32_t range_wave(unsigned long long t, unsigned long long T, uint32_t wact)
{
    return (uint32_t)(((t + 1ull) * wact + T - 1ull) / T) - 1u;
}

__host__ __device__ inline uint32_t range_active_waves(unsigned long long T, uint32_t waves)
{
    unsigned long long w = T / kMinRangeTiles;
    if (w < 1) w = 1;
    return w < waves ? (uint32_t)w : waves;
}

// Lane l of a DPP move with control C into rows R (others 0; lanes with no source 0).
template <int C, int R>
__device__ __forceinline__ unsigned long long dpp_move64(unsigned long long v)
{
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, C, R, 0xf, true);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), C, R, 0xf, true);
    return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Inclusive prefix sum over the wave's 64 lanes, on the VALU: shifts by 1, 2, 4 and 8
// lanes within each row of 16, then lane 15 of each row added into the row after it (rows
// 1 and 3) and lane 31 into rows 2 and 3.
__device__ __forceinline__ unsigned long long wave_scan_incl64(unsigned long long x)
{
    x += dpp_move64<0x111, 0xf>(x);  // row_shr:1
    x += dpp_move64<0x112, 0xf>(x);  // row_shr:2
    x += dpp_move64<0x114, 0xf>(x);  // row_shr:4
    x += dpp_move64<0x118, 0xf>(x);  // row_shr:8
    x += dpp_move64<0x142, 0xa>(x);  // row_bcast:15
    x += dpp_move64<0x143, 0xc>(x);  // row_bcast:31
    return x;
}

template <int NKS, int NQT, bool BF16, bool FP8D, int P, int MINW>
__global__ void __launch_bounds__(kScoreBlock, MINW)
range_kernel(const RangeArgs a)
{
    constexpr int DPAD = NKS * kStepK;
    constexpr int LDQ = DPAD + 8;                 // Q row pitch in LDS (halves), as the score kernel's
    constexpr int CP = dma_row_chunks(NKS, FP8D);
    constexpr int NLDD = CP / 4;
    constexpr int TILE_CHUNKS = kTileRows * CP;
    constexpr int LQP = NQT * kTileRows;          // padded query rows
    constexpr float NEG_INF = -__builtin_huge_valf();

    extern __shared__ __attribute__((aligned(16))) uint16_t qs[];  // Q tile | lengths | offsets; then the tile slots
    __shared__ unsigned long long wave_tiles[kScoreWaves];          // tiles of each wave's docs
    __shared__ unsigned long long blk_excl[kScoreBlock];            // each block's first tile within its wave's

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = (int)wave_uniform(threadIdx.x / kWave);
    const int row_in_tile = lane & 15;
    const int kgroup = lane >> 4;
    const uint32_t W = gridDim.x * kScoreWaves;
    const uint32_t wid = blockIdx.x * kScoreWaves + wave;
    const int B = a.B;

    // ---- prologue: one round of loads. The lengths (and, when the LDS has room, the
    // offsets) go to LDS by DMA, 256 docs per wave instruction; the query's chunks go to
    // registers and from there to LDS.
    const int nch = (B + kRangeDocsPerChunkRow - 1) / kRangeDocsPerChunkRow;  // 4-doc chunks per thread
    const int dpt = 4 * nch;                                                  // docs per thread block
    int32_t *lds_len = reinterpret_cast<int32_t *>(reinterpret_cast<char *>(qs) + a.len_lds);
    int32_t *lds_off = reinterpret_cast<int32_t *>(reinterpret_cast<char *>(qs) + a.off_lds);
    {
        const int pieces = (B + 4 * kWave - 1) / (4 * kWave);
        const __amdgpu_buffer_rsrc_t rlen = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<int32_t *>(a.lengths), (short)0, B * 4, kBufferWord3);
        const __amdgpu_buffer_rsrc_t roff = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<int32_t *>(a.offsets), (short)0, B * 4, kBufferWord3);
        for (int p = wave; p < pieces; p += kScoreWaves) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rlen, (__attribute__((address_space(3))) void *)(lds_len + p * 4 * kWave), 16,
                p * 16 * kWave + lane * 16, 0, 0, 0);
            if (a.off_lds)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    roff, (__attribute__((address_space(3))) void *)(lds_off + p * 4 * kWave), 16,
                    p * 16 * kWave + lane * 16, 0, 0, 0);
        }
    }
    constexpr int CPR = DPAD / 8;                                        // 16-byte chunks per query row
    constexpr int QL = (LQP * CPR + kScoreBlock - 1) / kScoreBlock;     // query chunks per thread
    u32x4 qv[QL];
#pragma unroll
    for (int k = 0; k < QL; ++k) {
        const int e = (int)threadIdx.x + k * kScoreBlock;
        const int r = e / CPR;
        const int c = e - r * CPR;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (e < LQP * CPR && r < a.Lq && c * 8 < a.d) v = *reinterpret_cast<const u32x4 *>(a.Q + (size_t)r * a.d + c * 8);
        qv[k] = v;
    }
    __builtin_amdgcn_s_waitcnt(kWaitAllVmem);
    __syncthreads();  // every wave's lengths are in LDS

    // ---- the schedule. Thread t's block of docs is [t dpt, (t + 1) dpt); its tiles are
    // summed chunk by chunk, starting at chunk t mod nch (the threads of a wave then read
    // distinct banks); a block-wide scan gives each block's first tile.
    auto tiles_of_len = [](int32_t len) -> uint32_t {
        return len > 0 ? ((uint32_t)len + (kTileRows - 1)) / kTileRows : 0u;
    };
    // N chunk reads (N >= nch) issued together; a read past the thread's nch chunks
    // repeats one and is not counted.
    auto block_tiles = [&](auto n) -> unsigned long long {
        constexpr int N = decltype(n)::value;
        const int t = (int)threadIdx.x;
        int c = t % nch;
        int4 v[N];
#pragma unroll
        for (int j = 0; j < N; ++j) {
            v[j] = *reinterpret_cast<const int4 *>(lds_len + t * dpt + 4 * c);
            c = c + 1 == nch ? 0 : c + 1;
        }
        unsigned long long sum = 0;
        c = t % nch;
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const int i0 = t * dpt + 4 * c;
            uint32_t nt = tiles_of_len(i0 < B ? v[j].x : 0) + tiles_of_len(i0 + 1 < B ? v[j].y : 0);
            unsigned long long pair = (unsigned long long)nt +
                                      tiles_of_len(i0 + 2 < B ? v[j].z : 0) + tiles_of_len(i0 + 3 < B ? v[j].w : 0);
            sum += j < nch ? pair : 0ull;
            c = c + 1 == nch ? 0 : c + 1;
        }
        return sum;
    };
    const unsigned long long mine = nch <= 2 ? block_tiles(std::integral_constant<int, 2>{})
                                             : block_tiles(std::integral_constant<int, kRangeChunksPerThread>{});
    const unsigned long long incl = wave_scan_incl64(mine);
    blk_excl[threadIdx.x] = incl - mine;
    if (lane == kWave - 1) wave_tiles[wave] = incl;
    // The query tile, zero-padded, into LDS (behind the same barrier as the scan).
#pragma unroll
    for (int k = 0; k < QL; ++k) {
        const int e = (int)threadIdx.x + k * kScoreBlock;
        const int r = e / CPR;
        const int c = e - r * CPR;
        if (e < LQP * CPR) *reinterpret_cast<u32x4 *>(qs + r * LDQ + c * 8) = qv[k];
    }
    __syncthreads();
    // Tiles of each wave's blocks (wave-uniform), all tiles, and the first tile of wave
    // v's blocks (a sum of selects: an array indexed at run time would go to scratch).
    static_assert(kScoreWaves == 4, "four waves per workgroup");
    const unsigned long long wt0 = wave_uniform64(wave_tiles[0]), wt1 = wave_uniform64(wave_tiles[1]),
                             wt2 = wave_uniform64(wave_tiles[2]), wt3 = wave_uniform64(wave_tiles[3]);
    const unsigned long long T = wt0 + wt1 + wt2 + wt3;
    auto wave_first_of = [&](int v) -> unsigned long long {
        return (v > 0 ? wt0 : 0ull) + (v > 1 ? wt1 : 0ull) + (v > 2 ? wt2 : 0ull);
    };

    // Lane l of block k: doc k dpt + l's length (0 past the block or the batch), tiles and
    // first tile.
    auto block_len = [&](int k) -> int32_t {
        const int i = k * dpt + lane;
        return lane < dpt && i < B ? lds_len[i] : 0;
    };
    auto block_first = [&](int k, uint32_t nt) -> unsigned long long {
        return wave_first_of(k / kWave) + blk_excl[k] + wave_scan_incl64(nt) - nt;
    };

    // ---- this wave's range and its first doc: the block holding the range's first
    // tile (the last block whose first tile is at most it), then the doc within it.
    const uint32_t wact = range_active_waves(T, W);
    unsigned long long r_begin = 0, r_end = 0;
    if (wid < wact) {
        r_begin = range_start(wid, T, wact);
        r_end = wid + 1 == wact ? T : range_start(wid + 1, T, wact);
    }
    r_begin = wave_uniform64(r_begin);
    r_end = wave_uniform64(r_end);
    int first_doc = 0;
    unsigned long long first_tile = 0;  // tile position of first_doc's first tile
    if (r_end > r_begin) {
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < kScoreBlock / kWave; ++j)
            cnt += __popcll(__ballot(wave_first_of(j) + blk_excl[j * kWave + lane] <= r_begin));
        const int k = cnt > 0 ? cnt - 1 : 0;  // (cnt >= 1: block 0 starts at tile 0 <= r_begin)
        const uint32_t nt = tiles_of_len(block_len(k));
        const unsigned long long first = block_first(k, nt);
        // Exactly one lane's tiles hold r_begin. The tile walk below stays inside each doc
        // it takes whatever the scan gave, and with no such lane the wave takes no range.
        const unsigned long long hit = __ballot(nt > 0u && first <= r_begin && r_begin < first + nt);
        if (hit) {
            const int l = __builtin_ctzll(hit);
            first_doc = k * dpt + l;
            first_tile = __shfl(first, l);
        } else {
            r_end = r_begin;
        }
    }
    first_doc = (int)wave_uniform((uint32_t)first_doc);
    first_tile = wave_uniform64(first_tile);
    // The first window of lengths and offsets (doc first_doc + l in lane l).
    int32_t wlen = 0, woff = 0;
    {
        const int i = first_doc + lane;
        if (i < B) {
            wlen = lds_len[i];
            woff = a.off_lds ? lds_off[i] : a.offsets[i];
        }
    }

    u32x4 qf[NQT][NKS];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
        for (int s = 0; s < NKS; ++s)
            qf[qt][s] = *reinterpret_cast<const u32x4 *>(qs + (qt * kTileRows + row_in_tile) * LDQ + (s * 4 + kgroup) * 8);
    // Block wid's lengths, for the scan output written once the first tiles are in flight.
    const int32_t out_len = (int)wid < kScoreBlock ? block_len((int)wid) : 0;
    __syncthreads();  // the tile slots now reuse the query's LDS (and the prologue's)

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
    int rd_dma[NKS];
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
        const int c = FP8D ? (kgroup >> 1) + 2 * s : kgroup + 4 * s;
        rd_dma[s] = row_in_tile * CP + (c ^ dma_swizzle(row_in_tile, CP));
    }
    const int rd_half = (kgroup & 1) * 8;

    // ---- doc lengths and offsets: a window of 64 docs, doc win + l in lane l; later
    // windows come from global memory
    int win = first_doc;
    auto load_window = [&](int base) {
        win = base;
        const int i = base + lane;
        wlen = i < B ? a.lengths[i] : 0;
        woff = i < B ? a.offsets[i] : 0;
        // Waited for here, on this path alone: otherwise the compiler's wait analysis
        // would make every later pass of the tile loop wait for all loads in flight.
        __builtin_amdgcn_s_waitcnt(kWaitAllVmem);
    };
    // Length and offset of doc j (wave-uniform): from the window, moved forward when j
    // leaves it (the walk only moves forward).
    auto doc_info = [&](int j, int32_t &len, int32_t &off) {
        if (j - win >= kWave) load_window(j);
        len = __builtin_amdgcn_readlane(wlen, j - win);
        off = __builtin_amdgcn_readlane(woff, j - win);
    };
    // The next doc after j that has a tile.
    auto next_doc = [&](int j) -> int {
        for (;;) {
            ++j;
            if (j >= B) return B;
            if (j - win >= kWave) load_window(j);
            const unsigned long long has = __ballot(lane >= j - win && wlen > 0);
            if (has) return win + __builtin_ctzll(has);
            j = win + kWave - 1;  // none left in the window: continue past it
        }
    };

    // ---- issue side: walks the range, P tiles ahead of the consume side
    // Piece kinds: 0 whole doc (store the score), 1 head slot, 2 tail slot.
    int i_doc = B;                 // doc of the next tile to issue (B: none left)
    uint32_t i_t = 0, i_tend = 0;  // its tile in the doc, and the end of its piece there
    uint32_t i_kind = 0;
    int32_t i_len = 0;
    uint64_t i_base = 0;
    // Tile position of the issue side in the whole sequence: the first tile of doc i_doc
    // is i_pos - i_t.
    unsigned long long i_pos = r_begin;
    auto start_doc = [&](int j, uint32_t t_begin, unsigned long long doc_first_tile) {
        int32_t len, off;
        doc_info(j, len, off);
        const uint32_t nt = ((uint32_t)len + (kTileRows - 1)) / kTileRows;
        i_doc = j;
        i_t = t_begin;
        i_len = len;
        i_base = wave_uniform64((uint64_t)(uintptr_t)a.docs + (uint64_t)((int64_t)off * a.stride_bytes));
        const unsigned long long doc_end = doc_first_tile + nt;
        i_tend = (uint32_t)((doc_end <= r_end ? doc_end : r_end) - doc_first_tile);
        i_kind = t_begin > 0 ? 1u : (i_tend < nt ? 2u : 0u);
    };
    if (r_end > r_begin) start_doc(first_doc, (uint32_t)(r_begin - first_tile), first_tile);

    // Next tile of the walk into slot `slot` (a zero-size load once the range is done);
    // returns its info word: rows | end-of-piece << 5 | kind << 6 | valid << 8 | doc << 16.
    auto issue = [&](uint32_t slot) -> uint32_t {
        uint32_t rows = 0, inf = 0;
        uint64_t ub = (uint64_t)(uintptr_t)a.docs;
        if (i_doc < B) {
            const int left = i_len - (int)i_t * kTileRows;
            rows = (uint32_t)(left < kTileRows ? left : kTileRows);
            ub = wave_uniform64(i_base + (uint64_t)i_t * (uint64_t)tile_bytes);
            const bool last = i_t + 1 == i_tend;
            inf = rows | (last ? 1u << 5 : 0u) | (i_kind << 6) | (1u << 8) | ((uint32_t)i_doc << 16);
            ++i_t;
            ++i_pos;
            if (last) {
                // the next piece: the next doc with a tile, if the range goes on
                if (i_pos < r_end) start_doc(next_doc(i_doc), 0, i_pos);
                else i_doc = B;
            }
        }
        rows = wave_uniform(rows);
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
        return wave_uniform(inf);
    };

    float rmax[NQT][4];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
        for (int i = 0; i < 4; ++i) rmax[qt][i] = NEG_INF;

    auto consume = [&](uint32_t slot, uint32_t rows) {
        // Every slot is refilled in turn, so exactly NLDD (P - 1) loads were issued after
        // this slot's; once no more are in flight, its tile is in LDS.
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(NLDD * (P - 1)));
        const u32x4 *tile = slots + slot * TILE_CHUNKS;
        u32x4 bf[NKS];
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            if constexpr (FP8D) {
                typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                const u32x2 v = *reinterpret_cast<const u32x2 *>(reinterpret_cast<const char *>(tile + rd_dma[s]) + rd_half);
                bf[s] = e4m3x8_to_16<BF16>(v[0], v[1]);
            } else {
                bf[s] = tile[rd_dma[s]];
            }
        }
        // The accumulator of a row past the doc end starts at -inf, which keeps it out
        // of the max; tile qt's products go into one accumulator while tile qt - 1's are
        // folded into the running max.
        const float c0 = row_in_tile < (int)rows ? 0.0f : NEG_INF;
        f32x4 acc[2];
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) {
            f32x4 r = {c0, c0, c0, c0};
#pragma unroll
            for (int s = 0; s < NKS; ++s) r = mfma16x16x32<BF16>(qf[qt][s], bf[s], r);
            acc[qt & 1] = r;
            if (qt > 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) rmax[qt - 1][i] = __builtin_fmaxf(rmax[qt - 1][i], acc[(qt - 1) & 1][i]);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) rmax[NQT - 1][i] = __builtin_fmaxf(rmax[NQT - 1][i], acc[(NQT - 1) & 1][i]);
    };

    // A piece ends: its row maxima over the 16 doc-row lanes, then the doc's score (a
    // whole doc, summed in the score kernel's order) or the piece's slot.
    auto finish_piece = [&](uint32_t inf) {
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
            for (int i = 0; i < 4; ++i) rmax[qt][i] = row16_max(rmax[qt][i]);
        const uint32_t kind = (inf >> 6) & 3u;
        const int doc = (int)(inf >> 16);
        if (kind == 0u) {
            float lane_sum = 0.0f;
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt) {
                const int left = a.Lq - qt * kTileRows;
                const int nr = left < 0 ? 0 : (left > kTileRows ? kTileRows : left);
#pragma unroll
                for (int i = 0; i < 4; ++i) lane_sum += kgroup * 4 + i < nr ? rmax[qt][i] : 0.0f;
            }
            const int ls = __builtin_bit_cast(int, lane_sum);
            const float s0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ls, 0));
            const float s1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ls, 16));
            const float s2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ls, 32));
            const float s3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ls, 48));
            float sum = ((s0 + s1) + s2) + s3;
            if constexpr (FP8D) sum *= a.doc_scale;
            if (lane == 0) a.scores[doc] = sum;
        } else if (row_in_tile == 0) {
            const uint32_t slot = kind == 1u ? wid : wact + wid;
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt) {
                f32x4 v = {rmax[qt][0], rmax[qt][1], rmax[qt][2], rmax[qt][3]};
                *reinterpret_cast<f32x4 *>(a.partials + (size_t)slot * LQP + qt * kTileRows + kgroup * 4) = v;
            }
        }
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
            for (int i = 0; i < 4; ++i) rmax[qt][i] = NEG_INF;
    };

    // The stream: slot k % P holds tile k of the walk. info[0] is the oldest slot's, the
    // one consumed next; each step consumes it, refills its slot with the tile P ahead
    // and shifts the queue. Tiles are issued in walk order, so once the oldest slot
    // holds no tile, none does.
    uint32_t info[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        info[p] = issue((uint32_t)p);
        __builtin_amdgcn_sched_barrier(0);
    }
    // For the combine kernel, while the first tiles arrive: S_0 .. S_B (S_B = T), and -inf
    // for empty docs (no tile, so no piece and no combine); wave w < 256 writes block w
    // (the host launches at least 256 waves).
    if (wid < (uint32_t)kScoreBlock) {
        const int k = (int)wid;
        const uint32_t nt = tiles_of_len(out_len);
        const unsigned long long first = block_first(k, nt);
        const int i = k * dpt + lane;
        if (lane < dpt && i < B) {
            a.scan[i] = first;
            if (nt == 0u) a.scores[i] = NEG_INF;
        }
        if (k == 0 && lane == 0) a.scan[B] = T;
    }
    uint32_t slot = 0;
    while (info[0] & (1u << 8)) {
        const uint32_t inf = info[0];
        consume(slot, inf & 31u);
        __builtin_amdgcn_sched_barrier(0);
        const uint32_t fresh = issue(slot);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int p = 0; p + 1 < P; ++p) info[p] = info[p + 1];
        info[P - 1] = fresh;
        if (inf & (1u << 5)) finish_piece(inf);
        slot = slot + 1u == (uint32_t)P ? 0u : slot + 1u;
    }
    // Every load has landed before the wave ends (the last ones were zero-size loads,
    // which still write their LDS slot).
    __builtin_amdgcn_s_waitcnt(kWaitAllVmem);
}

// Scores of the docs a range launch split: one wave per doc, the max over its pieces'
// slots, then the score kernel's fixed-order sum.
__global__ void __launch_bounds__(kScoreBlock)
range_combine_kernel(const RangeCombineArgs a);

}  // namespace maxsim
