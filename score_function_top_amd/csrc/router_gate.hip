// router_gate.hip -- routed softmax top-k with the shared-expert sigmoid gate
// folded into the same kernel, on gfx950.
//
// Operation: "[HIP] [Perf] Fold shared-expert gate GEMV into topk_softmax
// kernel" (ROCm aiter pull request 5652): per token the routed top-k slots
// of the softmax over the gating logits, and for each shared expert s the
// gate scale * sigmoid(hidden_states[m,:] . gate_weight[s,:]) with id
// shared_base + s in the columns after the K routed ones.  The maths is
// stated in include/router.h.
//
// shared_gate_kernel: one wave per token (grid-stride over tokens), its
// hidden row of up to 8 pieces per lane requested before the routed half
// (from 8192 tokens on, every load first and the routed half last).
// shared_gate_split_kernel, up to 1024 tokens: one wave per half of a
// token.  The routed half is the ordered top-K of router_topk_wave.h.  The
// gate half is a GEMV with S <= 16
// outputs per token, bound by the hidden-state read (H elements per token,
// S flops each): it runs on the VALU, not on matrix cores.  Lane l owns
// the 16-byte pieces h = c*64*VH + VH*l (VH elements per piece); each piece
// of the hidden row is read once (non-temporal) and dotted with the same
// piece of every gate row (shared by all tokens, so it stays in the caches;
// bf16 pairs through v_dot2_f32_bf16, whose products are exact in fp32),
// then S wave sums give the gate logits.
#include <hip/hip_runtime.h>

#include "router_io.h"
#include "router_params.h"
#include "router_topk_wave.h"

namespace rker {

namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <typename TIn>
__device__ __forceinline__ float dot16(const uint32_t (&a)[4], const uint32_t (&b)[4], float acc)
{
    if constexpr (sizeof(TIn) == 2) {
#pragma unroll
        for (int q = 0; q < 4; q++)
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a[q]),
                                                  __builtin_bit_cast(bf16x2_t, b[q]), acc, false);
    } else {
#pragma unroll
        for (int q = 0; q < 4; q++)
            acc = fmaf(as_f(a[q]), as_f(b[q]), acc);
    }
    return acc;
}

// 16 bytes of a row at element offset h (elements past H read as 0).
template <typename TIn, bool VEC, int POL>
__device__ __forceinline__ void load16(rsrc_t r, int h, int H, uint32_t (&v)[4])
{
    constexpr int VH = 16 / (int)sizeof(TIn);
    constexpr uint32_t sz = (uint32_t)sizeof(TIn);
    if constexpr (VEC) {
        const auto t = __builtin_amdgcn_raw_buffer_load_b128(
            r, (int)(h < H ? (uint32_t)h * sz : kOOB), 0, POL);
#pragma unroll
        for (int q = 0; q < 4; q++)
            v[q] = t[q];
    } else if constexpr (sizeof(TIn) == 2) {
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int h0 = h + 2 * q;
            const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(
                r, (int)(h0 < H ? (uint32_t)h0 * sz : kOOB), 0, POL);
            const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(
                r, (int)(h0 + 1 < H ? (uint32_t)(h0 + 1) * sz : kOOB), 0, POL);
            v[q] = (lo & 0xFFFFu) | (hi << 16);
        }
    } else {
#pragma unroll
        for (int q = 0; q < VH; q++)
            v[q] = __builtin_amdgcn_raw_buffer_load_b32(
                r, (int)(h + q < H ? (uint32_t)(h + q) * sz : kOOB), 0, POL);
    }
}

// Row m of the outputs: K routed slots (lane k < K), then S gates (lane
// K + s).
__device__ __forceinline__ void store_row(const GateParams &p, int64_t m, int lane, int id,
                                          float wt, float gate)
{
    const uint32_t nb = (uint32_t)(p.K + p.S) * 4u;
    const rsrc_t rw = make_rsrc(p.weights + m * p.ld, nb);
    const rsrc_t ri = make_rsrc(p.ids + m * p.ld, nb);
    const bool routed = lane < p.K;
    const bool shared = lane >= p.K && lane < p.K + p.S;
    const uint32_t o = routed || shared ? (uint32_t)lane * 4u : kOOB;
    __builtin_amdgcn_raw_buffer_store_b32(as_u(routed ? wt : gate), rw, (int)o, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32((uint32_t)(routed ? id : p.base + (lane - p.K)), ri,
                                          (int)o, 0, 0);
}

// Hidden-row pieces (16 bytes per lane) requested before the routed half
// when the whole row fits: 4096 bf16 or 2048 fp32 elements.
constexpr int kGatePrefetch = 8;

// LATE (prefetched rows only): every load of the token first -- hidden row,
// the first gate row, gating row -- then the gate half, then the routed
// half on the loaded logits; nothing is held across the routed half (103
// VGPRs against 119 at E=512, bf16).  From two rounds of waves on, other
// waves' loads cover the routed half at the end (on MI355X at E=512,
// hidden 4096: M = 8192 the same within 1%, M = 12288 24.7 -> 24.4 us,
// M = 16384 31.2 -> 30.2); in a single round nothing does (M = 4096
// 10.5 -> 10.6, M = 6144 14.4 -> 15.2).
template <int NCH, typename TIn, bool VEC_G, bool VEC_H, bool PRE, bool LATE = false>
__global__ __launch_bounds__(kBlock) void shared_gate_kernel(GateParams p)
{
    __shared__ uint64_t cand[kWaves][kSortedSlots];
    constexpr uint32_t sz = io<TIn>::kSize;
    constexpr int VH = 16 / (int)sz;  // hidden elements per 16-byte piece
    const int lane = lane_id();
    const int64_t nwaves = (int64_t)gridDim.x * kWaves;
    const int E = p.E, H = p.H, K = p.K, S = p.S;
    const int pieces = (H + 64 * VH - 1) / (64 * VH);
    const rsrc_t rgw = make_rsrc(p.gw, (uint32_t)S * (uint32_t)H * sz);
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));

    for (int64_t m = (int64_t)blockIdx.x * kWaves + wave; m < p.M; m += nwaves) {
        const rsrc_t rh = make_rsrc((const char *)p.hs + m * H * sz, (uint32_t)H * sz);
        if constexpr (PRE && LATE) {
            const rsrc_t rx = make_rsrc((const char *)p.x + m * E * sz, (uint32_t)E * sz);
            uint32_t hrow[kGatePrefetch][4], g0[kGatePrefetch][4];
#pragma unroll
            for (int c = 0; c < kGatePrefetch; c++)
                load16<TIn, VEC_H, kStream>(rh, c * 64 * VH + VH * lane, H, hrow[c]);
#pragma unroll
            for (int c = 0; c < kGatePrefetch; c++)
                load16<TIn, VEC_H, 0>(rgw, c * 64 * VH + VH * lane, H, g0[c]);
            float key[NCH][4];
            wave_topk_load<NCH, TIn, VEC_G>(rx, E, key);
            float gate = 0.0f;
            for (int s = 0; s < S; s++) {
                float acc = 0.0f;
#pragma unroll
                for (int c = 0; c < kGatePrefetch; c++) {
                    const int h = c * 64 * VH + VH * lane;
                    uint32_t gv[4];
                    if (s == 0) {
#pragma unroll
                        for (int q = 0; q < 4; q++)
                            gv[q] = g0[c][q];
                    } else {
                        load16<TIn, VEC_H, 0>(rgw, s * H + h, s * H + H, gv);
                    }
                    acc = dot16<TIn>(hrow[c], gv, acc);
                }
                const float logit = group_sum<64>(acc);
                const float sg = p.scale * sigmoid_fast(logit);
                gate = lane == K + s ? sg : gate;
            }
            int id;
            float wt;
            wave_topk_keys<NCH>(key, K, SCORE_SOFTMAX, p.renorm, cand[wave], id, wt);
            store_row(p, m, lane, id, wt, gate);
            continue;
        }
        [[maybe_unused]] uint32_t hpre[kGatePrefetch][4];
        if constexpr (PRE) {
            // the whole hidden row is requested before the routed half, so
            // its latency hides behind that work
#pragma unroll
            for (int c = 0; c < kGatePrefetch; c++)
                load16<TIn, VEC_H, kStream>(rh, c * 64 * VH + VH * lane, H, hpre[c]);
        }

        // routed half
        const rsrc_t rx = make_rsrc((const char *)p.x + m * E * sz, (uint32_t)E * sz);
        int id;
        float wt;
        wave_topk_row<NCH, TIn, VEC_G>(rx, E, K, SCORE_SOFTMAX, p.renorm, cand[wave], id, wt);

        // gate half: S dot products over the hidden row
        if constexpr (PRE) {
            float gate = 0.0f;
            for (int s = 0; s < S; s++) {
                float acc = 0.0f;
#pragma unroll
                for (int c = 0; c < kGatePrefetch; c++) {
                    const int h = c * 64 * VH + VH * lane;
                    uint32_t gv[4];
                    load16<TIn, VEC_H, 0>(rgw, s * H + h, s * H + H, gv);
                    acc = dot16<TIn>(hpre[c], gv, acc);
                }
                const float logit = group_sum<64>(acc);
                // every lane evaluates it: no lane-divergent branch
                const float sg = p.scale * sigmoid_fast(logit);
                gate = lane == K + s ? sg : gate;
            }
            store_row(p, m, lane, id, wt, gate);
            continue;
        }
        float acc[kGateMaxShared];
#pragma unroll
        for (int s = 0; s < kGateMaxShared; s++)
            acc[s] = 0.0f;
#pragma unroll 8
        for (int c = 0; c < pieces; c++) {
            const int h = c * 64 * VH + VH * lane;
            uint32_t hv[4];
            load16<TIn, VEC_H, kStream>(rh, h, H, hv);
#pragma unroll
            for (int s = 0; s < kGateMaxShared; s++) {
                if (s < S) {
                    uint32_t gv[4];
                    load16<TIn, VEC_H, 0>(rgw, s * H + h, s * H + H, gv);
                    acc[s] = dot16<TIn>(hv, gv, acc[s]);
                }
            }
        }
        float gate = 0.0f;
#pragma unroll
        for (int s = 0; s < kGateMaxShared; s++) {
            if (s < S) {
                const float logit = group_sum<64>(acc[s]);
                const float sg = p.scale * sigmoid_fast(logit);
                gate = lane == K + s ? sg : gate;
            }
        }

        store_row(p, m, lane, id, wt, gate);
    }
}

// Up to this many tokens each token is two wave tasks of one launch, the
// routed half and the gate half, which then run side by side (one round
// of waves at these sizes, so the token's latency is the longer half, not
// the sum: M = 1 4.0 -> 3.7 us, M = 256 4.6 -> 4.2 us on MI355X at E=512,
// hidden 4096, bf16).  Above it one wave takes both halves of a token, its
// hidden row requested before the routed half so that the row's latency
// hides behind that work (M = 4096 10.7 us against 11.9 split, M = 16384
// 30.9 against 32.5).
constexpr int64_t kGateSplitMaxTokens = 1024;
// From this many tokens (two rounds of resident waves at E=512, bf16) the
// prefetched-row kernel takes its routed half last (shared_gate_kernel,
// LATE).
constexpr int64_t kGateLateMinTokens = 8192;

// The gate half over a prefetched hidden row: S dot products, each a wave
// sum; lane K + s returns gate s.
template <typename TIn, bool VEC_H>
__device__ __forceinline__ float gate_prefetched(const GateParams &p, rsrc_t rgw,
                                                 const uint32_t (&hpre)[kGatePrefetch][4], int lane)
{
    constexpr int VH = 16 / (int)io<TIn>::kSize;
    const int H = p.H;
    float gate = 0.0f;
    for (int s = 0; s < p.S; s++) {
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < kGatePrefetch; c++) {
            const int h = c * 64 * VH + VH * lane;
            uint32_t gv[4];
            load16<TIn, VEC_H, 0>(rgw, s * H + h, s * H + H, gv);
            acc = dot16<TIn>(hpre[c], gv, acc);
        }
        const float logit = group_sum<64>(acc);
        // every lane evaluates it: no lane-divergent branch
        const float sg = p.scale * sigmoid_fast(logit);
        gate = lane == p.K + s ? sg : gate;
    }
    return gate;
}

// The gate half for longer rows: the hidden row streamed piece by piece
// against all S gate rows.
template <typename TIn, bool VEC_H>
__device__ __forceinline__ float gate_streamed(const GateParams &p, rsrc_t rgw, rsrc_t rh,
                                               int lane)
{
    constexpr int VH = 16 / (int)io<TIn>::kSize;
    const int H = p.H, S = p.S;
    const int pieces = (H + 64 * VH - 1) / (64 * VH);
    float acc[kGateMaxShared];
#pragma unroll
    for (int s = 0; s < kGateMaxShared; s++)
        acc[s] = 0.0f;
#pragma unroll 8
    for (int c = 0; c < pieces; c++) {
        const int h = c * 64 * VH + VH * lane;
        uint32_t hv[4];
        load16<TIn, VEC_H, kStream>(rh, h, H, hv);
#pragma unroll
        for (int s = 0; s < kGateMaxShared; s++) {
            if (s < S) {
                uint32_t gv[4];
                load16<TIn, VEC_H, 0>(rgw, s * H + h, s * H + H, gv);
                acc[s] = dot16<TIn>(hv, gv, acc[s]);
            }
        }
    }
    float gate = 0.0f;
#pragma unroll
    for (int s = 0; s < kGateMaxShared; s++) {
        if (s < S) {
            const float logit = group_sum<64>(acc[s]);
            const float sg = p.scale * sigmoid_fast(logit);
            gate = lane == p.K + s ? sg : gate;
        }
    }
    return gate;
}

// The whole hidden row of token m (up to kGatePrefetch pieces per lane),
// requested at once.
template <typename TIn, bool VEC_H>
__device__ __forceinline__ void prefetch_row(rsrc_t rh, int H, int lane,
                                             uint32_t (&hpre)[kGatePrefetch][4])
{
    constexpr int VH = 16 / (int)io<TIn>::kSize;
#pragma unroll
    for (int c = 0; c < kGatePrefetch; c++)
        load16<TIn, VEC_H, kStream>(rh, c * 64 * VH + VH * lane, H, hpre[c]);
}

// Row m's K routed slots (lane k < K) alone ...
__device__ __forceinline__ void store_routed(const GateParams &p, int64_t m, int lane, int id,
                                             float wt)
{
    const uint32_t nb = (uint32_t)(p.K + p.S) * 4u;
    const rsrc_t rw = make_rsrc(p.weights + m * p.ld, nb);
    const rsrc_t ri = make_rsrc(p.ids + m * p.ld, nb);
    const uint32_t o = lane < p.K ? (uint32_t)lane * 4u : kOOB;
    __builtin_amdgcn_raw_buffer_store_b32(as_u(wt), rw, (int)o, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32((uint32_t)id, ri, (int)o, 0, 0);
}

// ... and its S gates (lane K + s) alone.
__device__ __forceinline__ void store_gates(const GateParams &p, int64_t m, int lane, float gate)
{
    const uint32_t nb = (uint32_t)(p.K + p.S) * 4u;
    const rsrc_t rw = make_rsrc(p.weights + m * p.ld, nb);
    const rsrc_t ri = make_rsrc(p.ids + m * p.ld, nb);
    const uint32_t o = lane >= p.K && lane < p.K + p.S ? (uint32_t)lane * 4u : kOOB;
    __builtin_amdgcn_raw_buffer_store_b32(as_u(gate), rw, (int)o, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32((uint32_t)(p.base + (lane - p.K)), ri, (int)o, 0, 0);
}

// Grid-stride over 2*M wave tasks: task t is the routed half (t even) or
// the gate half (t odd) of token t/2; the same arithmetic as
// shared_gate_kernel, so the outputs are the same bit for bit.
template <int NCH, typename TIn, bool VEC_G, bool VEC_H, bool PRE>
__global__ __launch_bounds__(kBlock) void shared_gate_split_kernel(GateParams p)
{
    __shared__ uint64_t cand[kWaves][kSortedSlots];
    constexpr uint32_t sz = io<TIn>::kSize;
    const int lane = lane_id();
    const int64_t nwaves = (int64_t)gridDim.x * kWaves;
    const int E = p.E, H = p.H;
    const rsrc_t rgw = make_rsrc(p.gw, (uint32_t)p.S * (uint32_t)H * sz);
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));

    for (int64_t t = (int64_t)blockIdx.x * kWaves + wave; t < 2 * p.M; t += nwaves) {
        const int64_t m = t >> 1;
        if ((t & 1) == 0) {  // wave-uniform
            const rsrc_t rx = make_rsrc((const char *)p.x + m * E * sz, (uint32_t)E * sz);
            int id;
            float wt;
            wave_topk_row<NCH, TIn, VEC_G>(rx, E, p.K, SCORE_SOFTMAX, p.renorm, cand[wave], id,
                                           wt);
            store_routed(p, m, lane, id, wt);
            continue;
        }
        const rsrc_t rh = make_rsrc((const char *)p.hs + m * H * sz, (uint32_t)H * sz);
        float gate;
        if constexpr (PRE) {
            uint32_t hpre[kGatePrefetch][4];
            prefetch_row<TIn, VEC_H>(rh, H, lane, hpre);
            gate = gate_prefetched<TIn, VEC_H>(p, rgw, hpre, lane);
        } else {
            gate = gate_streamed<TIn, VEC_H>(p, rgw, rh, lane);
        }
        store_gates(p, m, lane, gate);
    }
}

// Launch modes: one wave per token, the same with the routed half last
// (LATE), one wave per half of a token (split kernel).
enum GateMode { kGateFused, kGateLate, kGateSplit };

template <int NCH, typename TIn, bool PRE, int MODE>
hipError_t gate_p(const GateParams &p, bool vec_g, bool vec_h, unsigned grid, hipStream_t st)
{
    const dim3 g(grid), b(kBlock);
#define ROUTER_GATE_LAUNCH(VG, VH)                                                             \
    if constexpr (MODE == kGateSplit)                                                        \
        hipLaunchKernelGGL((shared_gate_split_kernel<NCH, TIn, VG, VH, PRE>), g, b, 0, st, p);   \
    else                                                                                     \
        hipLaunchKernelGGL((shared_gate_kernel<NCH, TIn, VG, VH, PRE, MODE == kGateLate>), g, b, \
                           0, st, p);
    if (vec_g && vec_h) {
        ROUTER_GATE_LAUNCH(true, true)
    } else if (vec_g) {
        ROUTER_GATE_LAUNCH(true, false)
    } else if (vec_h) {
        ROUTER_GATE_LAUNCH(false, true)
    } else {
        ROUTER_GATE_LAUNCH(false, false)
    }
#undef ROUTER_GATE_LAUNCH
    return hipGetLastError();
}

template <int NCH, typename TIn>
hipError_t gate_t(const GateParams &p, bool vec_g, bool vec_h, unsigned grid, hipStream_t st)
{
    const int vh = 16 / (int)sizeof(TIn);
    const bool pre = vec_h && p.H <= kGatePrefetch * 64 * vh;
    if (p.M <= kGateSplitMaxTokens)
        return pre ? gate_p<NCH, TIn, true, kGateSplit>(p, vec_g, vec_h, grid, st)
                   : gate_p<NCH, TIn, false, kGateSplit>(p, vec_g, vec_h, grid, st);
    if (pre && p.M >= kGateLateMinTokens)
        return gate_p<NCH, TIn, true, kGateLate>(p, vec_g, vec_h, grid, st);
    return pre ? gate_p<NCH, TIn, true, kGateFused>(p, vec_g, vec_h, grid, st)
               : gate_p<NCH, TIn, false, kGateFused>(p, vec_g, vec_h, grid, st);
}

template <int NCH>
hipError_t gate_nch(const GateParams &p, int dtype, bool vec_g, bool vec_h, unsigned grid,
                    hipStream_t st)
{
    return dtype == 0 ? gate_t<NCH, float>(p, vec_g, vec_h, grid, st)
                      : gate_t<NCH, uint16_t>(p, vec_g, vec_h, grid, st);
}

}  // namespace

hipError_t launch_shared_gate(const GateParams &p, int dtype, bool vec_g, bool vec_h,
                              hipStream_t stream)
{
    if (p.M == 0)
        return hipSuccess;
    const int64_t ntask = p.M <= kGateSplitMaxTokens ? 2 * p.M : p.M;  // wave tasks
    const int64_t blocks = (ntask + kWaves - 1) / kWaves;
    const unsigned grid = (unsigned)(blocks < kGateMaxBlocks ? blocks : kGateMaxBlocks);
    if (p.E <= 256)
        return gate_nch<1>(p, dtype, vec_g, vec_h, grid, stream);
    if (p.E <= 512)
        return gate_nch<2>(p, dtype, vec_g, vec_h, grid, stream);
    return gate_nch<4>(p, dtype, vec_g, vec_h, grid, stream);
}

}  // namespace rker
