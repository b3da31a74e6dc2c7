// Score kernel instances for one query format, one doc storage and one K-step count,
// chosen by -DMAXSIM_BF16=0|1 -DMAXSIM_FP8=0|1 -DMAXSIM_NKS=1..8 (the build compiles
// this file once per triple, in parallel). Query tiles per group NQT run 1..8 with
// NQT * NKS <= 32. Each file also holds the one-launch short-doc kernel and the
// self-scheduling range kernel of its triple.
#include "maxsim_range.h"
#include "maxsim_score.h"
#include "maxsim_short.h"

#ifndef MAXSIM_BF16
#error "define MAXSIM_BF16"
#endif
#ifndef MAXSIM_NKS
#error "define MAXSIM_NKS"
#endif
#ifndef MAXSIM_FP8
#error "define MAXSIM_FP8"
#endif

namespace {

constexpr int NKS = MAXSIM_NKS;
constexpr bool BF = MAXSIM_BF16 != 0;
constexpr bool FP8 = MAXSIM_FP8 != 0;
// Pipeline depth in doc tiles and occupancy target (workgroups of 4 waves per CU,
// i.e. waves per SIMD) for the register allocation: the LDS-DMA rule shared with the
// host (maxsim::dma_pipe, maxsim::dma_blocks).
// (sub: 16-row blocks per slot; the scheduled score kernel's FP8 slots hold 32 rows,
// the one-launch kernels' 16.)
template <int NQT, int SUB = 1>
constexpr int pipe_depth()
{
    return maxsim::dma_pipe(NKS, NQT, FP8, SUB);
}

template <int NQT, int SUB = 1>
constexpr int min_waves()
{
    return maxsim::dma_blocks(NKS, NQT, FP8, SUB);
}

template <int NQT>
const void *short_entry()
{
    if constexpr (NQT * NKS <= maxsim::kMaxFragsPerGroup)
        return reinterpret_cast<const void *>(
            &maxsim::short_kernel<NKS, NQT, BF, FP8, pipe_depth<NQT>(), min_waves<NQT>()>);
    else
        return nullptr;
}

template <int NQT>
const void *range_entry()
{
    if constexpr (NQT * NKS <= maxsim::kMaxFragsPerGroup)
        return reinterpret_cast<const void *>(
            &maxsim::range_kernel<NKS, NQT, BF, FP8, pipe_depth<NQT>(), min_waves<NQT>()>);
    else
        return nullptr;
}

template <int NQT>
const void *entry()
{
    if constexpr (NQT * NKS <= maxsim::kMaxFragsPerGroup)
        return reinterpret_cast<const void *>(
            &maxsim::score_kernel<NKS, NQT, BF, FP8, pipe_depth<NQT, maxsim::score_sub(FP8)>(),
                                  min_waves<NQT, maxsim::score_sub(FP8)>()>);
    else
        return nullptr;
}

}  // namespace

#define MAXSIM_CAT2(a, b) a##b
#define MAXSIM_CAT(a, b) MAXSIM_CAT2(a, b)
#if MAXSIM_BF16 && MAXSIM_FP8
#define MAXSIM_LOOKUP MAXSIM_CAT(maxsim_score_kernel_bf16_fp8_k, MAXSIM_NKS)
#elif MAXSIM_BF16
#define MAXSIM_LOOKUP MAXSIM_CAT(maxsim_score_kernel_bf16_k, MAXSIM_NKS)
#elif MAXSIM_FP8
#define MAXSIM_LOOKUP MAXSIM_CAT(maxsim_score_kernel_f16_fp8_k, MAXSIM_NKS)
#else
#define MAXSIM_LOOKUP MAXSIM_CAT(maxsim_score_kernel_f16_k, MAXSIM_NKS)
#endif

const void *MAXSIM_LOOKUP(int nqt)
{
    switch (nqt) {
    case 1: return entry<1>();
    case 2: return entry<2>();
    case 3: return entry<3>();
    case 4: return entry<4>();
    case 5: return entry<5>();
    case 6: return entry<6>();
    case 7: return entry<7>();
    case 8: return entry<8>();
    default: return nullptr;
    }
}

#if MAXSIM_BF16 && MAXSIM_FP8
#define MAXSIM_SHORT_LOOKUP MAXSIM_CAT(maxsim_short_kernel_bf16_fp8_k, MAXSIM_NKS)
#elif MAXSIM_BF16
#define MAXSIM_SHORT_LOOKUP MAXSIM_CAT(maxsim_short_kernel_bf16_k, MAXSIM_NKS)
#elif MAXSIM_FP8
#define MAXSIM_SHORT_LOOKUP MAXSIM_CAT(maxsim_short_kernel_f16_fp8_k, MAXSIM_NKS)
#else
#define MAXSIM_SHORT_LOOKUP MAXSIM_CAT(maxsim_short_kernel_f16_k, MAXSIM_NKS)
#endif

const void *MAXSIM_SHORT_LOOKUP(int nqt)
{
    switch (nqt) {
    case 1: return short_entry<1>();
    case 2: return short_entry<2>();
    case 3: return short_entry<3>();
    case 4: return short_entry<4>();
    case 5: return short_entry<5>();
    case 6: return short_entry<6>();
    case 7: return short_entry<7>();
    case 8: return short_entry<8>();
    default: return nullptr;
    }
}

#if MAXSIM_BF16 && MAXSIM_FP8
#define MAXSIM_RANGE_LOOKUP MAXSIM_CAT(maxsim_range_kernel_bf16_fp8_k, MAXSIM_NKS)
#elif MAXSIM_BF16
#define MAXSIM_RANGE_LOOKUP MAXSIM_CAT(maxsim_range_kernel_bf16_k, MAXSIM_NKS)
#elif MAXSIM_FP8
#define MAXSIM_RANGE_LOOKUP MAXSIM_CAT(maxsim_range_kernel_f16_fp8_k, MAXSIM_NKS)
#else
#define MAXSIM_RANGE_LOOKUP MAXSIM_CAT(maxsim_range_kernel_f16_k, MAXSIM_NKS)
#endif

const void *MAXSIM_RANGE_LOOKUP(int nqt)
{
    switch (nqt) {
    case 1: return range_entry<1>();
    case 2: return range_entry<2>();
    case 3: return range_entry<3>();
    case 4: return range_entry<4>();
    case 5: return range_entry<5>();
    case 6: return range_entry<6>();
    case 7: return range_entry<7>();
    case 8: return range_entry<8>();
    default: return nullptr;
    }
}
