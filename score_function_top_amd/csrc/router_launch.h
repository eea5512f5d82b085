// router_launch.h -- host-side launch tables of the router kernels.
// Internal to the library.
//
// Vector kernels (16-byte loads and stores; E % 4 == 0, aligned arrays) are
// built for lane-group widths LPT = 16, 32, 64 and a list of chunk counts
// NCH each; a row of E elements takes the smallest built NCH with
// NCH*4*LPT >= E.  Element-wise kernels (any E, element-aligned arrays) are
// built for LPT = 64 and NCH in {1, 2, 4, 8, 16}.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "router_grid.h"
#include "router_kernels.h"

namespace rker {

template <int LPT, int NCH, typename TIn, int SCORE, int SEL, bool VEC>
hipError_t fwd_sel(const FwdParams &p, int gm, const Launch &l)
{
    const dim3 b(kBlock);
    if (gm == GROUP_LDS) {
        constexpr auto k = fwd_kernel<LPT, NCH, TIn, SCORE, SEL, GROUP_LDS, VEC>;
        hipLaunchKernelGGL(k, dim3(launch_grid<k>(l)), b, l.smem, l.stream, p);
    } else if (gm == GROUP_REG) {
        // built for vector kernels of up to kGroupRegMaxNch chunks only
        if constexpr (VEC && NCH <= kGroupRegMaxNch) {
            constexpr auto k = fwd_kernel<LPT, NCH, TIn, SCORE, SEL, GROUP_REG, VEC>;
            hipLaunchKernelGGL(k, dim3(launch_grid<k>(l)), b, l.smem, l.stream, p);
        } else {
            return hipErrorInvalidValue;
        }
    } else {
        // waves per block as the host sized the grid and LDS for
        constexpr int W = fwd_waves(LPT, NCH, GROUP_NONE, SEL, VEC);
        if (l.threads != 64u * W)
            return hipErrorInvalidValue;
        constexpr auto k = fwd_kernel<LPT, NCH, TIn, SCORE, SEL, GROUP_NONE, VEC, W>;
        hipLaunchKernelGGL(k, dim3(launch_grid<k>(l)), dim3(64 * W), l.smem, l.stream, p);
    }
    return hipGetLastError();
}

template <int LPT, int NCH, typename TIn, int SCORE, bool VEC>
hipError_t fwd_one(const FwdParams &p, int gm, const Launch &l)
{
    return p.sel == SEL_ARGMAX ? fwd_sel<LPT, NCH, TIn, SCORE, SEL_ARGMAX, VEC>(p, gm, l)
                               : fwd_sel<LPT, NCH, TIn, SCORE, SEL_PRUNE, VEC>(p, gm, l);
}

template <int LPT, int NCH, typename TIn, int SCORE, bool VEC>
hipError_t bwd_one(const BwdParams &p, const Launch &l)
{
    constexpr auto k = bwd_kernel<LPT, NCH, TIn, SCORE, VEC>;
    hipLaunchKernelGGL(k, dim3(launch_grid<k>(l)), dim3(kBlock), 0, l.stream, p);
    return hipGetLastError();
}

// Launches the forward for the first listed N equal to nch.
template <int LPT, bool VEC, int... N>
bool fwd_pick(int nch, int dtype, int score, int gm, const FwdParams &p,
              const Launch &l, hipError_t *err)
{
    auto one = [&](auto nc) {
        constexpr int C = decltype(nc)::value;
        if (dtype == 0)
            *err = score == 0 ? fwd_one<LPT, C, float, 0, VEC>(p, gm, l)
                              : fwd_one<LPT, C, float, 1, VEC>(p, gm, l);
        else
            *err = score == 0 ? fwd_one<LPT, C, uint16_t, 0, VEC>(p, gm, l)
                              : fwd_one<LPT, C, uint16_t, 1, VEC>(p, gm, l);
        return true;
    };
    return ((nch == N && one(std::integral_constant<int, N>{})) || ...);
}

template <int LPT, bool VEC, int... N>
bool bwd_pick(int nch, int dtype, int score, const BwdParams &p, const Launch &l,
              hipError_t *err)
{
    auto one = [&](auto nc) {
        constexpr int C = decltype(nc)::value;
        if (dtype == 0)
            *err = score == 0 ? bwd_one<LPT, C, float, 0, VEC>(p, l)
                              : bwd_one<LPT, C, float, 1, VEC>(p, l);
        else
            *err = score == 0 ? bwd_one<LPT, C, uint16_t, 0, VEC>(p, l)
                              : bwd_one<LPT, C, uint16_t, 1, VEC>(p, l);
        return true;
    };
    return ((nch == N && one(std::integral_constant<int, N>{})) || ...);
}

}  // namespace rker

// Defines fwd_NAME / bwd_NAME for lane width LPT_, vector flag VEC_ and the
// listed chunk counts.
#define ROUTER_DEFINE_PART(NAME, LPT_, VEC_, ...)                                   \
    namespace rker {                                                                \
    bool fwd_##NAME(int lpt, int nch, bool vec, int dtype, int score, int gm,       \
                    const FwdParams &p, const Launch &l, hipError_t *err)           \
    {                                                                               \
        if (lpt != LPT_ || vec != VEC_)                                             \
            return false;                                                           \
        return fwd_pick<LPT_, VEC_, __VA_ARGS__>(nch, dtype, score, gm, p, l,       \
                                                 err);                              \
    }                                                                               \
    bool bwd_##NAME(int lpt, int nch, bool vec, int dtype, int score,               \
                    const BwdParams &p, const Launch &l, hipError_t *err)           \
    {                                                                               \
        if (lpt != LPT_ || vec != VEC_)                                             \
            return false;                                                           \
        return bwd_pick<LPT_, VEC_, __VA_ARGS__>(nch, dtype, score, p, l, err);     \
    }                                                                               \
    }
