// Group-limited forward kernels for rows of 32-expert groups (see
// router_grouped.h), 16- or 32-lane tokens; one translation unit per lane
// width (ROUTER_GROUPED_LPT), so the two compile in parallel.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "router_grid.h"
#include "router_grouped.h"

#ifndef ROUTER_GROUPED_LPT
#error "ROUTER_GROUPED_LPT must be 16 or 32"
#endif

namespace rker {

namespace {

template <typename T>
struct tag {
    using type = T;
};

template <int LPT, int NCH, typename TIn, int SCORE, int Q, bool BIAS>
hipError_t grouped_one(const FwdParams &p, const Launch &l)
{
    constexpr auto k = grouped_fwd_kernel<LPT, NCH, TIn, SCORE, Q, BIAS>;
    hipLaunchKernelGGL(k, dim3(launch_grid<k>(l)), dim3(kBlock), l.smem, l.stream, p);
    return hipGetLastError();
}

template <int LPT, int NCH>
hipError_t grouped_nch(int dtype, int score, int Q, bool bias, const FwdParams &p,
                       const Launch &l)
{
    auto go = [&](auto tin, auto sc) {
        using TIn = typename decltype(tin)::type;
        constexpr int SC = decltype(sc)::value;
        if (Q == 2)
            return bias ? grouped_one<LPT, NCH, TIn, SC, 2, true>(p, l)
                        : grouped_one<LPT, NCH, TIn, SC, 2, false>(p, l);
        return bias ? grouped_one<LPT, NCH, TIn, SC, 4, true>(p, l)
                    : grouped_one<LPT, NCH, TIn, SC, 4, false>(p, l);
    };
    using F = tag<float>;
    using B = tag<uint16_t>;
    using S0 = std::integral_constant<int, SCORE_SOFTMAX>;
    using S1 = std::integral_constant<int, SCORE_SIGMOID>;
    if (dtype == 0)
        return score == SCORE_SOFTMAX ? go(F{}, S0{}) : go(F{}, S1{});
    return score == SCORE_SOFTMAX ? go(B{}, S0{}) : go(B{}, S1{});
}

}  // namespace

#define ROUTER_GROUPED_NAME_(L) fwd_grouped##L
#define ROUTER_GROUPED_NAME(L) ROUTER_GROUPED_NAME_(L)

bool ROUTER_GROUPED_NAME(ROUTER_GROUPED_LPT)(int lpt, int nch, int dtype, int score, int Q,
                                             bool bias, const FwdParams &p, const Launch &l,
                                             hipError_t *err)
{
    constexpr int L = ROUTER_GROUPED_LPT;
    if (lpt != L || (Q != 2 && Q != 4))
        return false;
    switch (nch) {
    case 1: *err = grouped_nch<L, 1>(dtype, score, Q, bias, p, l); return true;
    case 2: *err = grouped_nch<L, 2>(dtype, score, Q, bias, p, l); return true;
    case 4: *err = grouped_nch<L, 4>(dtype, score, Q, bias, p, l); return true;
    default: return false;
    }
}

}  // namespace rker
