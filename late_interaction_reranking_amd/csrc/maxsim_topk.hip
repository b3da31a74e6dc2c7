// Top-k selection over a score array on the GPU: the ranking the rerank's consumer needs
// (the Flash-MaxSim rerank page returns raw per-doc scores, section
// `flash_maxsim_rerank_direct`, return value; choosing the best docs is the next step).
//
// Order: score descending, equal scores (-0 equal to +0) by lower doc index, NaN after
// everything. Each entry becomes one 64-bit key, (order-preserving score bits << 32) |
// (2^32 - 1 - index), so the order is a strict total order on keys: the top k are
// unique and the selection is exact. Selection runs in levels: every block holds 4096
// keys in registers, finds its k-th largest by radix selection on an LDS histogram and
// keeps the k keys at or above it; the survivors (k per block) are the next level's
// input, until one block remains, which places each of its k survivors at its rank
// (the number of survivors above it, counted in LDS) and writes the results.
// Everything stays on the stream; nothing is read back to the host.
#include "maxsim.h"

#include "maxsim_topk.h"

namespace maxsim {
namespace {

constexpr int kChunk = 4096;    // keys per block (>= 4 kTopkMaxK, a multiple of kThreads)
constexpr int kThreads = 1024;

__device__ __forceinline__ uint64_t rank_key(float v, uint32_t idx)
{
    uint32_t u = __builtin_bit_cast(uint32_t, v);
    uint32_t key;
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u) {
        key = 0u;  // NaN: below every number
    } else {
        if (u == 0x80000000u) u = 0u;  // -0 ranks as +0
        key = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    }
    return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}

// One level: block b takes keys [b * kChunk, (b + 1) * kChunk) of the level's input (the
// scores themselves when in_keys is null), finds its k-th largest key T by radix
// selection in LDS (passes of 8 bits from the highest bit in which the block's keys
// differ; keys are unique apart from the zero padding), and keeps the k keys >= T: unordered in out_keys[b * k ..], or, on
// the last level (out_keys null), ranked (descending) into the final (score, index)
// pairs.
__global__ void __launch_bounds__(kThreads)
topk_level_kernel(const float *__restrict__ scores, const uint64_t *__restrict__ in_keys, int64_t n,
                  int32_t k, uint64_t *__restrict__ out_keys, int32_t B, float *__restrict__ top_scores,
                  int32_t *__restrict__ top_ids)
{
    constexpr int PER = kChunk / kThreads;
    __shared__ uint32_t hist[256];
    __shared__ uint64_t sel[kTopkMaxK];  // the final level's survivors
    __shared__ uint64_t sh_prefix, sh_and, sh_or;
    __shared__ uint32_t sh_need, sh_cnt, sh_done;
    const int tid = threadIdx.x;
    const int lane = tid & 63;

    uint64_t key[PER];
    const int64_t base = (int64_t)blockIdx.x * kChunk;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int64_t g = base + tid + j * kThreads;
        uint64_t v = 0;  // padding: below every real entry (whose low word is >= 2^31)
        if (g < n) v = in_keys ? in_keys[g] : rank_key(scores[g], (uint32_t)g);
        key[j] = v;
    }
    // Bits that all of the block's keys share need no histogram pass (scores of one
    // batch share their leading exponent bits, which would put every key in one bin).
    uint64_t vand = ~(uint64_t)0, vor = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        vand &= key[j];
        vor |= key[j];
    }
    for (int o = 32; o > 0; o >>= 1) {
        vand &= __shfl_xor(vand, o);
        vor |= __shfl_xor(vor, o);
    }
    for (int i = tid; i < 256; i += kThreads) hist[i] = 0u;
    if (tid == 0) {
        sh_and = ~(uint64_t)0;
        sh_or = 0;
        sh_need = (uint32_t)k;
        sh_cnt = 0u;
        sh_done = 0u;
    }
    __syncthreads();
    if (lane == 0) {
        atomicAnd(&sh_and, vand);
        atomicOr(&sh_or, vor);
    }
    __syncthreads();
    const uint64_t diff = sh_and ^ sh_or;
    const int top = diff ? 64 - __builtin_clzll(diff) : 0;  // bits [top, 64) are common
    uint64_t mask = top < 64 ? ~(uint64_t)0 << top : 0;
    if (tid == 0) sh_prefix = sh_and & mask;
    __syncthreads();

    // Radix selection of the k-th largest key, 8 bits per pass below the common bits:
    // `prefix` holds its bits above the current digit. It stops early when the chosen
    // bin holds exactly the keys still needed: then every key whose bits under `mask`
    // reach `prefix` is selected, without resolving the rest of the threshold.
    for (int hi = top; hi > 0; hi -= 8) {
        const int shift = hi >= 8 ? hi - 8 : 0;
        const uint32_t dmask = (1u << (hi - shift)) - 1u;
        const uint64_t prefix = sh_prefix;
#pragma unroll
        for (int j = 0; j < PER; ++j)
            if ((key[j] & mask) == prefix) atomicAdd(&hist[(uint32_t)(key[j] >> shift) & dmask], 1u);
        __syncthreads();
        if (tid < 64) {
            // Bins in descending order, four per lane; find the one that holds the
            // need-th largest remaining key, and clear the histogram for the next pass.
            const uint32_t need = sh_need;
            uint32_t c[4], tot = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int b = 255 - 4 * lane - i;
                c[i] = hist[b];
                hist[b] = 0u;
                tot += c[i];
            }
            uint32_t incl = tot;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t up = __shfl_up(incl, o);
                if (lane >= o) incl += up;
            }
            uint32_t acc = incl - tot;
            if (acc < need && need <= incl) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (acc + c[i] >= need) {
                        sh_prefix = prefix | ((uint64_t)(255 - 4 * lane - i) << shift);
                        sh_need = need - acc;
                        if (acc + c[i] == need) sh_done = 1u;
                        break;
                    }
                    acc += c[i];
                }
            }
        }
        mask |= (uint64_t)dmask << shift;
        __syncthreads();
        if (sh_done) break;
    }

    // Keep the keys above the threshold prefix, then fill the remaining places with keys
    // on it (after an early stop they fill them exactly; after a full selection only the
    // zero padding can repeat the threshold key).
    const uint64_t T = sh_prefix;
    uint64_t *dst = out_keys ? out_keys + (int64_t)blockIdx.x * k : sel;
#pragma unroll
    for (int j = 0; j < PER; ++j)
        if ((key[j] & mask) > T) dst[atomicAdd(&sh_cnt, 1u)] = key[j];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < PER; ++j)
        if ((key[j] & mask) == T) {
            const uint32_t pos = atomicAdd(&sh_cnt, 1u);
            if (pos < (uint32_t)k) dst[pos] = key[j];
        }
    if (out_keys) return;

    // Last level: each survivor's place in the output is its rank, the number of
    // survivors above it (keys are unique apart from the zero padding, whose equal keys
    // are ranked by position). One pass of k LDS reads per thread, one barrier.
    __syncthreads();
    for (int j = tid; j < k; j += kThreads) {
        const uint64_t v = sel[j];
        int rank = 0;
        for (int i = 0; i < k; ++i) {
            const uint64_t u = sel[i];
            rank += (u > v || (u == v && i < j)) ? 1 : 0;
        }
        const uint32_t idx = 0xFFFFFFFFu - (uint32_t)v;
        const bool real = v != 0u && idx < (uint32_t)B;
        top_ids[rank] = real ? (int32_t)idx : -1;
        top_scores[rank] = real ? scores[idx] : -__builtin_huge_valf();
    }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

size_t topk_workspace_bytes(int32_t B, int32_t k)
{
    const int64_t nb = ((int64_t)(B > 0 ? B : 0) + kChunk - 1) / kChunk;
    if (nb <= 1 || k <= 0) return 256;
    return 2 * align256((size_t)nb * (size_t)k * sizeof(uint64_t));
}

int launch_topk(const float *scores, int32_t B, int32_t k, float *top_scores, int32_t *top_ids, char *ws,
                hipStream_t stream)
{
    const size_t half = topk_workspace_bytes(B, k) / 2;
    uint64_t *buf[2] = {reinterpret_cast<uint64_t *>(ws), reinterpret_cast<uint64_t *>(ws + half)};
    int64_t n = B;
    const uint64_t *in = nullptr;
    int cur = 0;
    for (;;) {
        int64_t nb = (n + kChunk - 1) / kChunk;
        if (nb < 1) nb = 1;
        const bool last = nb == 1;
        hipLaunchKernelGGL(topk_level_kernel, dim3((unsigned)nb), dim3(kThreads), 0, stream, scores, in, n, k,
                           last ? nullptr : buf[cur], B, top_scores, top_ids);
        if (hipGetLastError() != hipSuccess) return MAXSIM_ERR_HIP;
        if (last) return MAXSIM_OK;
        in = buf[cur];
        n = nb * k;
        cur ^= 1;
    }
}

}  // namespace maxsim

extern "C" {

int maxsim_topk_workspace_size(int32_t B, int32_t k, size_t *bytes)
{
    if (!bytes || B < 0 || k < 0) return MAXSIM_ERR_INVALID_ARG;
    if (k > maxsim::kTopkMaxK) return MAXSIM_ERR_UNSUPPORTED;
    *bytes = maxsim::topk_workspace_bytes(B, k);
    return MAXSIM_OK;
}

int maxsim_topk(const float *scores, int32_t B, int32_t k, float *top_scores, int32_t *top_ids,
                void *workspace, size_t workspace_bytes, void *stream)
{
    if (B < 0 || k < 0) return MAXSIM_ERR_INVALID_ARG;
    if (k > maxsim::kTopkMaxK) return MAXSIM_ERR_UNSUPPORTED;
    if (k == 0) return MAXSIM_OK;
    if ((B > 0 && !scores) || !top_scores || !top_ids) return MAXSIM_ERR_INVALID_ARG;
    if (((uintptr_t)scores | (uintptr_t)top_scores | (uintptr_t)top_ids) & 3u) return MAXSIM_ERR_INVALID_ARG;
    if (!workspace || ((uintptr_t)workspace & 255u)) return MAXSIM_ERR_WORKSPACE;
    if (workspace_bytes < maxsim::topk_workspace_bytes(B, k)) return MAXSIM_ERR_WORKSPACE;
    return maxsim::launch_topk(scores, B, k, top_scores, top_ids, static_cast<char *>(workspace),
                               static_cast<hipStream_t>(stream));
}

}  // extern "C"
