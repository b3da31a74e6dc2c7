// Read-only streaming probe: the rate at which this device reads a large buffer once,
// in order, with nothing else to do. It is the measured ceiling that the score kernel's
// HBM bandwidth is set against (the published 8 TB/s is the other reference). Not part of
// the rerank library: built as libmaxsim_probe.so and loaded by the benchmark only.
//
// Both modes read 1 KB of consecutive bytes per wave instruction (16 bytes per lane),
// non-temporal, over a persistent grid of workgroups of 4 waves. Wave w reads the 4 KB
// tiles [T c(w) / c(W), T c(w + 1) / c(W)) of the T = ceil(bytes / 4096) tiles, c being
// the running sum of the waves' weights. Workgroups sit on the eight XCDs round robin
// (block b on XCD b % 8) and the odd-numbered XCDs read ~8 % slower, so when the grid
// is a multiple of 8 blocks a wave of an odd block weighs 11 and one of an even block 12
// (the split the score kernel's deal also makes); otherwise every wave weighs 1.
//   - mode 0, LDS-DMA: buffer_load_dwordx4 ... lds into 3 tile slots per wave, as the
//     score kernel loads its 16-bit doc tiles (at 3 workgroups per CU, the score kernel's
//     own occupancy on a 128-column query of 32 rows); nothing reads the tiles.
//   - mode 1, registers: 16-byte loads into VGPRs folded into an xor, which each lane
//     stores once at the end so that no load can be dropped.
// Every access stays inside [buf, buf + bytes): the LDS-DMA descriptors cover only a
// tile's bytes inside the buffer; register loads of whole tiles are in range by
// construction, and those of a partial last tile are guarded per lane (bytes is a
// multiple of 16).
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kBlock = kWave * kWaves;
constexpr int kTile = 4096;                   // bytes per tile: 4 loads of 1 KB
constexpr int kLoads = kTile / (kWave * 16);  // 4
constexpr int kSlots = 3;                     // tiles in flight per wave (LDS-DMA mode)
constexpr int kBufferWord3 = 0x00020000;      // raw buffer access, gfx9 family
constexpr int kNonTemporal = 2;
constexpr int kWaitLoadsButOneSlot = 0x0F70 | (kLoads * (kSlots - 1));  // s_waitcnt vmcnt(8)
constexpr int kWaitAllVmem = 0x0F70;                                      // s_waitcnt vmcnt(0)

// readfirstlane returns a signed int: each half goes through uint32_t before it is
// widened, or a low half with bit 31 set would sign-extend over the high half.
__device__ __forceinline__ uint32_t uniform32(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ uint64_t uniform64(uint64_t v)
{
    return (uint64_t)uniform32((uint32_t)v) | ((uint64_t)uniform32((uint32_t)(v >> 32)) << 32);
}

// Running sum of the weights of waves [0, v).
__device__ __forceinline__ uint64_t weight_before(uint64_t v, bool weighted)
{
    if (!weighted) return v;
    const uint64_t pairs = v / (2 * kWaves), r = v % (2 * kWaves);  // an even block, then an odd one
    return pairs * (kWaves * 12 + kWaves * 11) + (r < kWaves ? r * 12 : kWaves * 12 + (r - kWaves) * 11);
}

__device__ __forceinline__ uint64_t first_tile(uint64_t v, uint64_t W, uint64_t T)
{
    const bool weighted = (gridDim.x & 7u) == 0u;
    return T * weight_before(v, weighted) / weight_before(W, weighted);
}

__global__ void __launch_bounds__(kBlock) probe_lds_kernel(const char *buf, uint64_t bytes, uint32_t *sink)
{
    __shared__ __attribute__((aligned(16))) u32x4 slots[kWaves * kSlots * kTile / 16];
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t wave = uniform32(threadIdx.x / kWave);
    const uint64_t W = (uint64_t)gridDim.x * kWaves;
    const uint64_t wid = (uint64_t)blockIdx.x * kWaves + wave;
    const uint64_t T = (bytes + kTile - 1) / kTile;
    const uint64_t t0 = uniform64(first_tile(wid, W, T));
    const uint64_t t1 = uniform64(first_tile(wid + 1, W, T));
    u32x4 *const mine = slots + wave * (kSlots * kTile / 16);

    // Loads of tile t into slot `slot`; a tile past the wave's range loads nothing (its
    // descriptor has size 0, so every lane is out of range and no byte is fetched).
    auto issue = [&](int slot, uint64_t t) {
        uint32_t n = 0;
        if (t < t1) {
            const uint64_t left = bytes - t * kTile;
            n = left < (uint64_t)kTile ? (uint32_t)left : (uint32_t)kTile;
        }
        n = uniform32(n);
        const uint64_t base = uniform64((uint64_t)(uintptr_t)buf + (t < t1 ? t : t0) * kTile);
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>((uintptr_t)base), (short)0, (int)n, kBufferWord3);
#pragma unroll
        for (int s = 0; s < kLoads; ++s)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc, (__attribute__((address_space(3))) void *)(mine + slot * (kTile / 16) + s * kWave), 16,
                (lane + s * kWave) * 16, 0, 0, kNonTemporal);
    };

#pragma unroll
    for (int p = 0; p < kSlots; ++p) {
        issue(p, t0 + p);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (uint64_t t = t0; t < t1; t += kSlots) {
#pragma unroll
        for (int p = 0; p < kSlots; ++p) {
            // The slot's tile has landed once no more than the younger slots' loads are
            // in flight; then the slot is refilled with the tile kSlots further on.
            __builtin_amdgcn_s_waitcnt(kWaitLoadsButOneSlot);
            __builtin_amdgcn_sched_barrier(0);
            issue(p, t + p + kSlots);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __builtin_amdgcn_s_waitcnt(kWaitAllVmem);
    __syncthreads();
    // One word per lane of what landed in LDS: the loads' results are used.
    sink[wid * kWave + lane] = mine[lane].x;
}

__global__ void __launch_bounds__(kBlock) probe_reg_kernel(const char *buf, uint64_t bytes, uint32_t *sink)
{
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t wave = uniform32(threadIdx.x / kWave);
    const uint64_t W = (uint64_t)gridDim.x * kWaves;
    const uint64_t wid = (uint64_t)blockIdx.x * kWaves + wave;
    const uint64_t T = (bytes + kTile - 1) / kTile;
    const uint64_t t0 = uniform64(first_tile(wid, W, T));
    const uint64_t t1 = uniform64(first_tile(wid + 1, W, T));
    u32x4 acc = {0u, 0u, 0u, 0u};
    // Whole tiles in groups of kGroup, loads first and xors after, so that the group's
    // 16 loads are in flight together; then single whole tiles; then the buffer's partial
    // last tile, if this wave has it, lane by lane.
    constexpr int kGroup = 4;
    const uint64_t whole = bytes / kTile;
    const uint64_t tw = t1 < whole ? t1 : whole;
    const char *p = buf + (uint64_t)lane * 16;
    uint64_t t = t0;
    for (; t + kGroup <= tw; t += kGroup) {
        u32x4 v[kGroup * kLoads];
#pragma unroll
        for (int i = 0; i < kGroup * kLoads; ++i)
            v[i] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4 *>(p + (t + i / kLoads) * kTile + (i % kLoads) * kWave * 16));
#pragma unroll
        for (int i = 0; i < kGroup * kLoads; ++i) acc ^= v[i];
    }
    for (; t < tw; ++t) {
#pragma unroll
        for (int s = 0; s < kLoads; ++s)
            acc ^= __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p + t * kTile + s * kWave * 16));
    }
    if (t < t1) {  // t == whole: the partial tile
        for (int s = 0; s < kLoads; ++s) {
            const uint64_t off = t * kTile + (uint64_t)(lane + s * kWave) * 16;
            if (off < bytes) acc ^= __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(buf + off));
        }
    }
    sink[wid * kWave + lane] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

extern "C" {

// Workgroups of the probe's persistent grid: 3 per compute unit of the current device,
// or -1 when the device cannot be queried.
__attribute__((visibility("default"))) int maxsim_probe_blocks(void)
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
    return 3 * cus;
}

// Reads bytes of device memory at buf (16-byte aligned, bytes a multiple of 16) once with
// `blocks` workgroups; mode 0 LDS-DMA, 1 registers. sink: device memory of at least
// blocks * 256 32-bit words, overwritten. Enqueued on stream (a hipStream_t, NULL for the
// default stream). Returns 0, 1 for an invalid argument (nothing enqueued), 2 for a
// failed launch.
__attribute__((visibility("default"))) int maxsim_probe_read(const void *buf, uint64_t bytes, int mode,
                                                             int blocks, uint32_t *sink, void *stream)
{
    if (!buf || !sink || bytes == 0 || bytes % 16 != 0 || ((uintptr_t)buf & 15u) != 0 || blocks < 1 ||
        blocks > 65535 || (mode != 0 && mode != 1))
        return 1;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (mode == 0)
        hipLaunchKernelGGL(probe_lds_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, s,
                           static_cast<const char *>(buf), bytes, sink);
    else
        hipLaunchKernelGGL(probe_reg_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, s,
                           static_cast<const char *>(buf), bytes, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
