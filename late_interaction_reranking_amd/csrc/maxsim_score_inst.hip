// Score kernel instances for one query format, one doc storage and one K-step count,
// chosen by -DMAXSIM_BF16=0|1 -DMAXSIM_FP8=0|1 -DMAXSIM_NKS=1..8 (the build compiles
// this file once per triple, in parallel). Query tiles per group NQT run 1..8 with
// NQT * NKS <= 32.
#include "maxsim_score.h"

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
constexpr int NLD = FP8 ? (NKS + 1) / 2 : NKS;  // 1 KB loads per doc tile
// Pipeline depth in doc tiles: 4-8 KB of coalesced loads outstanding per wave (FP8
// tiles are half the bytes, so twice as many).
#ifdef MAXSIM_FORCE_P
constexpr int P = MAXSIM_FORCE_P;
#else
constexpr int P16 = NKS >= 3 ? 2 : (NKS == 2 ? 3 : 4);
constexpr int P = FP8 ? (2 * P16 < 8 ? 2 * P16 : 8) : P16;
#endif

// Occupancy target (waves per SIMD) from an estimate of the registers one wave needs:
// query fragments, P tiles of loads in flight, one staged fragment set, running
// maxima and accumulators, plus addressing and loop state.
template <int NQT>
constexpr int min_waves()
{
#ifdef MAXSIM_FORCE_MINW
    return MAXSIM_FORCE_MINW;
#else
    constexpr int est = 4 * NQT * NKS + 4 * P * NLD + 4 * NKS + 4 * NQT + 48;
    return est <= 128 ? 4 : (est <= 168 ? 3 : (est <= 256 ? 2 : 1));
#endif
}

template <int NQT>
const void *entry()
{
    if constexpr (NQT * NKS <= maxsim::kMaxFragsPerGroup)
        return reinterpret_cast<const void *>(&maxsim::score_kernel<NKS, NQT, BF, FP8, P, min_waves<NQT>()>);
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
