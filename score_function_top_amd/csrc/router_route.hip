// router_route.hip -- decode-shape routing with expert maps on gfx950: per
// token the score function and the K largest logits in order, then the
// (expert, token)-sorted expert maps of all T*K (token, slot) pairs, in one
// workgroup.
//
// Operation: the fused softmax + top-k + expert-map kernel of "[CUDA] Add
// fused decode routing, single-pass finalize, and PDL overlap for NVFP4
// QMoE" (onnxruntime pull request 33366, Description item 1: up to 4 rows,
// 512 experts, k in {1, 2, 4, 6, 8, 10}), with the map layout of the
// permutation maps in the TensorRT-LLM fused gather/finalize page
// (unpermuted index = token + k * num_rows; expert of each permuted row;
// first permuted row of each expert).  The maths is stated in
// include/router.h.
//
// One wave per token (T <= 16 waves in the block, at least 4) runs the ordered top-K of
// router_topk_wave.h; lane k keeps slot k.  The maps need no sort: each expert's LDS
// word collects a bit per token that chose it, so the expert offsets are an
// exclusive scan of the words' popcounts and pair (t, k) -> expert e lands
// at offset[e] + popcount(word[e] & ((1 << t) - 1)), which is the
// (expert, token) order because a token picks an expert at most once.
#include <hip/hip_runtime.h>

#include "router_io.h"
#include "router_params.h"
#include "router_topk_wave.h"

namespace rker {

namespace {

constexpr int kRouteMaxPairs = kRouteMaxRows * kRouteMaxK;

template <int NCH, typename TIn, bool VEC>
__global__ __launch_bounds__(kRouteMaxRows * 64) void route_maps_kernel(RouteParams p)
{
    __shared__ uint32_t tokmask[kRouteMaxExperts];  // bit t: token t chose expert e
    __shared__ uint32_t offs[kRouteMaxExperts + 1];
    __shared__ int32_t pair_expert[kRouteMaxPairs];  // by unpermuted index t + k*T
    __shared__ uint32_t wave_tot[kRouteMaxRows];
    __shared__ uint64_t cand[kRouteMaxRows][kSortedSlots];

    const int T = p.T, E = p.E, K = p.K, n = T * K;
    const int nthreads = (int)blockDim.x;
    const int tid = (int)threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = lane_id();
    for (int e = tid; e < E; e += nthreads)
        tokmask[e] = 0;
    __syncthreads();

    // ---- one wave per token: scores, ordered top-K, weights
    if (w < T) {
        constexpr uint32_t sz = io<TIn>::kSize;
        const rsrc_t r = make_rsrc((const char *)p.x + (int64_t)w * E * sz, (uint32_t)E * sz);
        int my_id;
        float wgt;
        wave_topk_row<NCH, TIn, VEC>(r, E, K, p.score, p.renorm, cand[w], my_id, wgt);
        if (lane < K) {
            const rsrc_t rw = make_rsrc(p.weights, (uint32_t)n * 4u);
            const rsrc_t ri = make_rsrc(p.ids, (uint32_t)n * 4u);
            const uint32_t o = (uint32_t)(w * K + lane) * 4u;
            __builtin_amdgcn_raw_buffer_store_b32(as_u(wgt), rw, (int)o, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32((uint32_t)my_id, ri, (int)o, 0, 0);
            pair_expert[w + lane * T] = my_id;
            atomicOr(&tokmask[my_id], 1u << w);
        }
    }
    __syncthreads();

    // ---- offsets: exclusive scan of popcount(tokmask[e]) over e < E; thread
    // t owns the contiguous run [t*m, t*m + m) of experts
    const int nwaves = nthreads >> 6;
    const int m = (E + nthreads - 1) / nthreads;  // <= kRouteMaxExperts / 64
    const int e0 = tid * m;
    uint32_t loc = 0;
    for (int i = 0; i < m; i++)
        loc += e0 + i < E ? (uint32_t)__builtin_popcount(tokmask[e0 + i]) : 0u;
    const uint32_t incl = group_incl_scan<64>(loc);
    if (lane == 63)
        wave_tot[w] = incl;
    __syncthreads();
    uint32_t run = incl - loc;
    for (int w2 = 0; w2 < w; w2++)
        run += wave_tot[w2];
    for (int i = 0; i < m; i++) {
        if (e0 + i < E) {
            offs[e0 + i] = run;
            run += (uint32_t)__builtin_popcount(tokmask[e0 + i]);
        }
    }
    if (tid == 0) {
        uint32_t tot = 0;
        for (int w2 = 0; w2 < nwaves; w2++)
            tot += wave_tot[w2];
        offs[E] = tot;  // = T*K
    }
    __syncthreads();

    const rsrc_t ro = make_rsrc(p.offsets, (uint32_t)(E + 1) * 8u);
    for (int e = tid; e <= E; e += nthreads) {
        __attribute__((ext_vector_type(2))) uint32_t v2;
        v2[0] = offs[e];
        v2[1] = 0u;
        __builtin_amdgcn_raw_buffer_store_b64(v2, ro, e * 8, 0, 0);
    }
    const rsrc_t rp2u = make_rsrc(p.perm_to_unperm, (uint32_t)n * 4u);
    const rsrc_t ru2p = make_rsrc(p.unperm_to_perm, (uint32_t)n * 4u);
    const rsrc_t rpe = make_rsrc(p.perm_expert, (uint32_t)n * 4u);
    for (int u = tid; u < n; u += nthreads) {
        const int e = pair_expert[u];
        const int t = u % T;
        const uint32_t pos = offs[e] + (uint32_t)__builtin_popcount(tokmask[e] & ((1u << t) - 1u));
        __builtin_amdgcn_raw_buffer_store_b32(pos, ru2p, u * 4, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)u, rp2u, (int)pos * 4, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)e, rpe, (int)pos * 4, 0, 0);
    }
}

// One wave per token, and at least kRouteMinWaves waves: the waves past T
// skip the top-K and share the per-expert map work (the zeroing, scan and
// offset stores over E), which a single wave did alone for one token
// (E = 512: T = 1 calls 4.4 -> 3.7 us at K = 1, 5.1 -> 4.4 us at K = 10;
// 8 waves measured the same as 4).
constexpr int kRouteMinWaves = 4;

template <int NCH>
hipError_t route_nch(const RouteParams &p, int dtype, bool vec, hipStream_t stream)
{
    const dim3 grid(1), block(64 * (p.T > kRouteMinWaves ? p.T : kRouteMinWaves));
    if (dtype == 0) {
        if (vec)
            hipLaunchKernelGGL((route_maps_kernel<NCH, float, true>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((route_maps_kernel<NCH, float, false>), grid, block, 0, stream, p);
    } else {
        if (vec)
            hipLaunchKernelGGL((route_maps_kernel<NCH, uint16_t, true>), grid, block, 0, stream,
                               p);
        else
            hipLaunchKernelGGL((route_maps_kernel<NCH, uint16_t, false>), grid, block, 0, stream,
                               p);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route_maps(const RouteParams &p, int dtype, bool vec, hipStream_t stream)
{
    if (p.E <= 256)
        return route_nch<1>(p, dtype, vec, stream);
    if (p.E <= 512)
        return route_nch<2>(p, dtype, vec, stream);
    return route_nch<4>(p, dtype, vec, stream);
}

}  // namespace rker
