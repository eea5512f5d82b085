// Group-limited forward kernels for rows of 32-expert groups (see
// router_grouped.h), 16- or 32-lane tokens; one translation unit per lane
// width (ROUTER_GROUPED_LPT), so the two compile in parallel.
#include <hip/hip_runtime.h>

#include <mutex>
#include <type_traits>

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

// Occupancy-sized grid: the kernel's resident blocks per compute unit
// (hipOccupancyMaxActiveBlocksPerMultiprocessor, read once per device and
// kernel) times the compute units, or fewer when the tokens need fewer.
// Each wave then loops over token groups with the next group's logits in
// flight behind its work.  Measured on MI355X at T=16384, E=256 in 8
// groups, bf16 (5 resident blocks per CU): 1280 blocks 9.4 us; one block
// per two-token wave pair (2048 blocks) 12.3 us; 6 per CU 11.3 us, and 2,
// 3, 4 per CU 14.2, 11.4, 10.5 us.
template <int LPT, int NCH, typename TIn, int SCORE, int Q, bool BIAS>
hipError_t grouped_one(const FwdParams &p, const Launch &l)
{
    const auto kern = grouped_fwd_kernel<LPT, NCH, TIn, SCORE, Q, BIAS>;
    constexpr int kMaxDev = 64;
    static std::once_flag once[kMaxDev];
    static int blocks_per_device[kMaxDev];
    int d = 0;
    hipError_t e = hipGetDevice(&d);
    if (e != hipSuccess)
        return e;
    if (d < 0 || d >= kMaxDev)
        return hipErrorInvalidDevice;
    std::call_once(once[d], [&] {
        int occ = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, kBlock, l.smem) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, d) != hipSuccess)
            occ = cus = 0;
        blocks_per_device[d] = occ * cus;
    });
    const unsigned cap = (unsigned)blocks_per_device[d];
    const unsigned grid = cap > 0 && l.grid > cap ? cap : l.grid;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kBlock), l.smem, l.stream, p);
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
