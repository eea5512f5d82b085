// router_kernels.h -- forward and backward kernels of the fused MoE router
// for gfx950.
//
// Operations: fused_topk_with_score_function and fused_score_for_moe_aux_loss
// ("[Common] Optimize fused router forward/backward kernels", NVIDIA
// TransformerEngine pull request 3012, "Summary", "Forward kernels",
// "Backward kernels").  The per-token maths is stated in include/router.h.
//
// Work split: one token per lane group of LPT lanes (16, 32 or 64), 64/LPT
// tokens per wave, 4 waves per 256-thread block, grid-stride over tokens.
// Lane l of a group holds NCH chunks of 4 elements.  Vector rows (E a
// multiple of 4, aligned arrays): 4 consecutive elements, j = c*4*LPT +
// 4*l + u for chunk c and component u, so every chunk load or store of a
// group is one contiguous segment.  Element-wise rows (any E or
// alignment): j = c*4*LPT + u*LPT + l, so each of a chunk's four element
// accesses covers LPT consecutive elements (T=8192, E=3070 softmax:
// forward 145 -> 87 us, backward 130 -> 68 us against 4 elements per lane
// at stride 4).  jrel and lane_part hold the two mappings; every index
// the selection compares comes from them.  The whole row lives in
// VGPRs; LDS holds only a 3*LPT-slot candidate list per token (and, for the
// LDS form of group-limited routing, the row's group values).
//
// Selection of the K largest keys (ties to the lower index) is exact and
// reduces to one 64-bit threshold: with pack(j) = key_j << 32 | ~j (unique
// per element), expert j is selected iff pack(j) >= T64, where T64 is the
// K-th largest pack value.  Ways to find it:
//   argmax  K rounds of a group-wide max whose winner is marked (small K);
//   prune   tau = K-th largest lane maximum bounds the K-th largest key from
//           below (K lanes hold a key >= tau), so only keys >= tau compete;
//           they are compacted into LDS (at most 2*LPT of them) and
//           bitonic-sorted across the lanes (K <= LPT);
//   bits    exact bit-by-bit search of the K-th key value, then of the index
//           among equal keys (any K; taken when pruning leaves more than
//           2*LPT candidates, or when K > LPT).
//
// Code shape: no branch depends on a single element.  Padding is encoded in
// the data (key -inf, score 0); stores of masked chunks get a byte offset
// past the buffer's range, which the hardware drops.
#pragma once

#include <type_traits>

#include "router_device.h"
#include "router_io.h"
#include "router_params.h"

namespace rker {

using namespace rdev;

// Row I/O (buffer resources, the io<> element types) lives in router_io.h.


// Element index of chunk c, component u relative to this lane; the lane's
// part, j_lane (lane_part), is added by the caller.  Vector rows: a lane
// holds 4 consecutive elements of each chunk (j = c*4*LPT + 4*lane + u),
// one 4-element access.  Element-wise rows: component u of a chunk is
// element lane of its u-th run of LPT (j = c*4*LPT + u*LPT + lane), so each
// of the four element accesses of a chunk covers LPT consecutive elements.
template <int LPT, bool VEC>
__device__ __forceinline__ constexpr int jrel(int c, int u)
{
    return VEC ? c * 4 * LPT + u : c * 4 * LPT + u * LPT;
}
template <bool VEC>
__device__ __forceinline__ constexpr int lane_part(int lane) { return VEC ? 4 * lane : lane; }

// Loads chunk c of the group's row (element offset goff in the wave's
// buffer).  With VEC one 4-element vector access (lane offset in a VGPR,
// chunk offset in the scalar offset), else four element accesses, each
// over LPT consecutive elements of the group.
// Elements at or past Ev read as `pad`.  A masked access gets the VGPR
// offset kOOB, which is out of range whether or not the hardware adds the
// scalar offset to its range check, so it never touches memory.
template <int LPT, typename T, bool VEC, int POL = kStream>
__device__ __forceinline__ void load_chunk(rsrc_t r, uint32_t goff, int c, int j_lane,
                                           int Ev, float pad, float (&v)[4])
{
    const int j0 = jrel<LPT, VEC>(c, 0) + j_lane;
    if constexpr (VEC) {
        const bool ok = j0 < Ev;
        io<T>::template load4<POL>(r, ok ? (goff + (uint32_t)j_lane) * io<T>::kSize : kOOB,
                                   (uint32_t)jrel<LPT, VEC>(c, 0) * io<T>::kSize, v);
#pragma unroll
        for (int u = 0; u < 4; u++)
            v[u] = ok ? v[u] : pad;
    } else {
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int j = jrel<LPT, VEC>(c, u) + j_lane;
            const bool ok = j < Ev;
            const float t = io<T>::template load1<POL>(
                r, ok ? (goff + (uint32_t)j) * io<T>::kSize : kOOB);
            v[u] = ok ? t : pad;
        }
    }
}

// load_chunk in two halves, so that a row's loads can all be issued before
// the first wait: load_chunk_raw requests the chunk as stored (a masked
// access reads 0; bf16 stays two packed words in v[0], v[1]; element-wise
// rows get their values), and mask_chunk, after the loads, unpacks it and
// applies the padding value.
template <int LPT, typename T, bool VEC, int POL = kStream>
__device__ __forceinline__ void load_chunk_raw(rsrc_t r, uint32_t goff, int c, int j_lane,
                                               int Ev, float pad, float (&v)[4])
{
    if constexpr (VEC) {
        const bool ok = jrel<LPT, VEC>(c, 0) + j_lane < Ev;
        const int off = (int)(ok ? (goff + (uint32_t)j_lane) * io<T>::kSize : kOOB);
        const int soff = (int)((uint32_t)jrel<LPT, VEC>(c, 0) * io<T>::kSize);
        if constexpr (sizeof(T) == 2) {
            const auto t = __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, POL);
            v[0] = as_f(t[0]);
            v[1] = as_f(t[1]);
        } else {
            const auto t = __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, POL);
#pragma unroll
            for (int u = 0; u < 4; u++)
                v[u] = as_f(t[u]);
        }
    } else {
        // element-wise: masked elements read 0 (offset kOOB); the padding
        // value goes in after every load is in flight (mask_chunk)
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int j = jrel<LPT, VEC>(c, u) + j_lane;
            v[u] = io<T>::template load1<POL>(
                r, j < Ev ? (goff + (uint32_t)j) * io<T>::kSize : kOOB);
        }
    }
}

template <int LPT, typename T, bool VEC>
__device__ __forceinline__ void mask_chunk(int c, int j_lane, int Ev, float pad, float (&v)[4])
{
    if constexpr (VEC) {
        if constexpr (sizeof(T) == 2) {
            const uint32_t w0 = as_u(v[0]), w1 = as_u(v[1]);
            v[0] = as_f(w0 << 16);
            v[1] = as_f(w0 & 0xFFFF0000u);
            v[2] = as_f(w1 << 16);
            v[3] = as_f(w1 & 0xFFFF0000u);
        }
        const bool ok = jrel<LPT, VEC>(c, 0) + j_lane < Ev;
#pragma unroll
        for (int u = 0; u < 4; u++)
            v[u] = ok ? v[u] : pad;
    } else {
#pragma unroll
        for (int u = 0; u < 4; u++)
            v[u] = jrel<LPT, VEC>(c, u) + j_lane < Ev ? v[u] : pad;
    }
}

template <int LPT, typename T, bool VEC>
__device__ __forceinline__ void store_chunk(rsrc_t r, uint32_t goff, int c, int j_lane,
                                            int E, const float (&v)[4])
{
    if constexpr (VEC) {
        const int j0 = jrel<LPT, VEC>(c, 0) + j_lane;
        io<T>::store4(r, j0 < E ? (goff + (uint32_t)j0) * io<T>::kSize : kOOB, v);
    } else {
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int j = jrel<LPT, VEC>(c, u) + j_lane;
            io<T>::store1(r, j < E ? (goff + (uint32_t)j) * io<T>::kSize : kOOB, v[u]);
        }
    }
}

// Map bytes of chunk c, little-endian in one u32 (0 past Ev).
template <int LPT, bool VEC>
__device__ __forceinline__ uint32_t load_map_chunk(rsrc_t r, uint32_t goff, int c,
                                                   int j_lane, int Ev)
{
    if constexpr (VEC) {
        const bool ok = jrel<LPT, VEC>(c, 0) + j_lane < Ev;
        const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(
            r, (int)(ok ? goff + (uint32_t)j_lane : kOOB), jrel<LPT, VEC>(c, 0), kStream);
        return ok ? w : 0u;
    } else {
        uint32_t w = 0;
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int j = jrel<LPT, VEC>(c, u) + j_lane;
            const uint32_t b = __builtin_amdgcn_raw_buffer_load_b8(
                r, (int)(j < Ev ? goff + (uint32_t)j : kOOB), 0, kStream);
            w |= b << (8 * u);
        }
        return w;
    }
}

template <int LPT, bool VEC>
__device__ __forceinline__ void store_map_chunk(rsrc_t r, uint32_t goff, int c, int j_lane,
                                                int E, uint32_t w)
{
    if constexpr (VEC) {
        const int j0 = jrel<LPT, VEC>(c, 0) + j_lane;
        __builtin_amdgcn_raw_buffer_store_b32(w, r, (int)(j0 < E ? goff + (uint32_t)j0 : kOOB),
                                              0, kStream);
    } else {
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int j = jrel<LPT, VEC>(c, u) + j_lane;
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(w >> (8 * u)), r,
                                                 (int)(j < E ? goff + (uint32_t)j : kOOB), 0,
                                                 kStream);
        }
    }
}

// Pairwise (tree) sum of N values held in registers.
template <int N, int O = 0>
__device__ __forceinline__ float tree_sum(const float *v)
{
    if constexpr (N == 1) {
        return v[O];
    } else {
        constexpr int H = N / 2;
        return tree_sum<H, O>(v) + tree_sum<N - H, O + H>(v);
    }
}

// IEEE maximum / minimum (v_maximum3 / v_minimum3 on gfx950): unlike
// fmaxf / fminf they need no canonicalisation of their inputs, and they
// agree with them on every value used here (never NaN; where -0 can occur
// the result feeds only comparisons or a +0 canonicalisation).
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmin(float a, float b) { return __builtin_elementwise_minimum(a, b); }

// ------------------------------------------------------------ selection
//
// Selection keys are floats: the logit without a bias, fp32(s + b) with
// one; -inf marks padding and experts outside the kept groups (finite
// logits are a precondition).  Equal keys tie (-0.0 == +0.0) and ties go to
// the lower index.  A selection is described by its threshold (x, j):
// expert j with key k is selected iff k > x, or k == x and j <= j_t.
// Where a total order is needed (sorting, group-wide maxima) a key is packed
// as ord(k) << 32 | ~j: ord is monotone and canonical on +-0, and ~j makes
// the lower index the larger pack.

struct Thresh {
    float x;
    uint32_t j;   // 0xFFFFFFFF: every key equal to x is selected
};

__device__ __forceinline__ uint64_t pack_key(float k, uint32_t j)
{
    return ((uint64_t)ord_key(k + 0.0f) << 32) | (uint32_t)~j;
}

__device__ __forceinline__ Thresh unpack_thresh(uint64_t t64)
{
    return Thresh{ord_key_inv((uint32_t)(t64 >> 32)), ~(uint32_t)t64};
}

// Largest finite float: the lowest threshold a real key can need.
constexpr float kMinKey = -3.4028234663852886e38f;

// argmax: K rounds; each round the group's largest (key, lower index) wins
// and its key becomes NaN (never compares larger again).  Afterwards the
// selected experts are exactly the NaN keys.
template <int LPT, int NCH, bool VEC>
__device__ __forceinline__ void select_argmax(float (&key)[NCH][4], int K, int j_lane)
{
    for (int r = 0; r < K; r++) {
        // lane-local best: first (lowest j) element with the largest key
        float bk = -INFINITY;
        uint32_t bj = 0;
#pragma unroll
        for (int c = 0; c < NCH; c++)
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const bool gt = key[c][u] > bk;
                bk = gt ? key[c][u] : bk;
                bj = gt ? (uint32_t)jrel<LPT, VEC>(c, u) : bj;
            }
        const uint64_t mine = bk == -INFINITY ? 0ull : pack_key(bk, bj + (uint32_t)j_lane);
        const uint64_t best = group_max_u64<LPT>(mine);
        // winner's j relative to this lane; no match when there is no winner
        const uint32_t jw = best ? ~(uint32_t)best - (uint32_t)j_lane : 0xFFFFFFFFu;
#pragma unroll
        for (int c = 0; c < NCH; c++)
#pragma unroll
            for (int u = 0; u < 4; u++)
                key[c][u] = jw == (uint32_t)jrel<LPT, VEC>(c, u) ? __builtin_nanf("") : key[c][u];
    }
}

// bits: exact search, any K.  Finds the K-th largest key value v by a
// bit-by-bit search over its order-preserving u32 code (each candidate code
// is mapped back to a float and compared), then, if more keys equal v than
// the selection needs, the index of the last selected one.
template <int LPT, int NCH, bool VEC>
__device__ __forceinline__ Thresh select_bits(const float (&key)[NCH][4], int K, int j_lane)
{
    uint32_t pref = 0;
    for (int b = 31; b >= 0; b--) {
        const uint32_t cand = pref | (1u << b);
        const float cf = ord_key_inv(cand);  // NaN codes count nothing
        uint32_t cnt = 0;
#pragma unroll
        for (int c = 0; c < NCH; c++)
#pragma unroll
            for (int u = 0; u < 4; u++)
                cnt += key[c][u] >= cf;
        pref = group_sum_u32<LPT>(cnt) >= (uint32_t)K ? cand : pref;
    }
    const float v = ord_key_inv(pref);
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int c = 0; c < NCH; c++)
#pragma unroll
        for (int u = 0; u < 4; u++) {
            gt += key[c][u] > v;
            eq += key[c][u] == v;
        }
    gt = group_sum_u32<LPT>(gt);
    eq = group_sum_u32<LPT>(eq);
    const uint32_t need = (uint32_t)K - gt;
    uint32_t J = 0xFFFFFFFFu;
    if (wave_any(eq != need)) {
        // lowest J with #{key == v, j <= J} >= need
        uint32_t lo = 0;
        for (int b = 31 - __builtin_clz(NCH * 4 * LPT); b >= 0; b--) {
            const int test = (int)(lo + (1u << b) - 1u) - j_lane;  // lane-relative
            uint32_t f = 0;
#pragma unroll
            for (int c = 0; c < NCH; c++)
#pragma unroll
                for (int u = 0; u < 4; u++)
                    f += (key[c][u] == v) & (jrel<LPT, VEC>(c, u) <= test);
            lo = group_sum_u32<LPT>(f) < need ? lo + (1u << b) : lo;
        }
        J = eq != need ? lo : J;
    }
    return Thresh{v, J};
}

// prune: keys >= tau are compacted into this group's LDS list -- raw key
// bits and ~j, 2*LPT slots plus one dummy slot per lane for the writes of
// non-candidates -- read back at most two per lane, packed, bitonic-sorted,
// and the K-th taken.  tau is the K-th largest lane maximum (K lanes hold
// a key >= tau, so the K-th largest key is >= tau), or, with TOP2 and
// 2*K > LPT, the K-th largest of the lanes' two largest keys (2*LPT
// distinct elements, K of them >= tau: the same bound, tighter when K is a
// large share of the lanes, and valid up to K = 2*LPT).  When the (K+1)-th
// candidate has a different key, no tie straddles the threshold and j_t is
// "all".  Falls back to select_bits for the whole wave when a group has
// more than 2*LPT candidates.  Requires K <= LPT, or K <= 2*LPT with TOP2.
// The two-key bound is compiled only into the kernels without groups and
// with 16 or 32 lanes per token: in the group-limited kernels (capped at
// few registers) it cost spills, and 64-lane tokens take K <= 64 anyway.
template <int LPT, int NCH, bool TOP2, bool KEYS32, bool VEC>
__device__ __forceinline__ Thresh select_prune(const float (&key)[NCH][4], int K, int lane,
                                               int j_lane, uint64_t *cand, bool use_bound,
                                               float bound)
{
    float tau;
    if (use_bound) {
        tau = bound;  // from the group stage: at most the K-th largest key
    } else if (!TOP2 || 2 * K <= LPT) {
        float lm = -INFINITY;
#pragma unroll
        for (int c = 0; c < NCH; c++)
#pragma unroll
            for (int u = 0; u < 4; u++)
                lm = fmaxf(lm, key[c][u]);
        tau = ord_key_inv(group_bcast<LPT>(sort_desc32<LPT>(ord_key(lm + 0.0f)), K - 1));
    } else {
        // the lane's two largest keys (two elements; equal values allowed)
        float m1 = -INFINITY, m2 = -INFINITY;
#pragma unroll
        for (int c = 0; c < NCH; c++)
#pragma unroll
            for (int u = 0; u < 4; u++) {
                m2 = fmaxf(m2, fminf(m1, key[c][u]));
                m1 = fmaxf(m1, key[c][u]);
            }
        uint32_t a = ord_key(m1 + 0.0f), b = ord_key(m2 + 0.0f);
        sort_desc32x2<LPT>(a, b);
        tau = ord_key_inv(K <= LPT ? group_bcast<LPT>(a, K - 1)
                                   : group_bcast<LPT>(b, K - 1 - LPT));
    }
    tau = fmaxf(tau, kMinKey);  // padding and excluded experts never compete
    uint32_t cnt = 0;
#pragma unroll
    for (int c = 0; c < NCH; c++)
#pragma unroll
        for (int u = 0; u < 4; u++)
            cnt += key[c][u] >= tau;
    const uint32_t incl = group_incl_scan<LPT>(cnt);
    const uint32_t total = group_bcast<LPT>(incl, LPT - 1);
    if (wave_any(total > 2u * LPT))
        return select_bits<LPT, NCH, VEC>(key, K, j_lane);
    uint32_t pos = incl - cnt;
    const uint32_t dummy = 2u * LPT + (uint32_t)lane;
#pragma unroll
    for (int c = 0; c < NCH; c++)
#pragma unroll
        for (int u = 0; u < 4; u++) {
            // same test as the count, spelled so the compiler recomputes it
            // instead of keeping 36 lane masks alive (keys are never NaN here)
            const bool in = !(key[c][u] < tau);
            cand[in ? pos : dummy] = ((uint64_t)as_u(key[c][u]) << 32) |
                                     (uint32_t)~(uint32_t)(jrel<LPT, VEC>(c, u) + j_lane);
            pos += in;
        }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // Keys alone first: sort the candidates' 32-bit order keys (half the
    // work of the 64-bit words).  When no group of the wave has equal keys
    // at positions K-1 and K, the K-th key alone is the threshold: exactly
    // the K keys at or above it are selected.  Only such a tie needs the
    // indices, i.e. the 64-bit sort further down (the list is still there).
    // Compiled into the 16- and 32-lane kernels without the register group
    // stage only: the register-capped group-limited kernels spilled with it,
    // and the 64-lane forward of 2304 experts ran 2% slower with it (a
    // memory-bound kernel; its candidate sort is not what limits it).
    if constexpr (KEYS32) {
        const uint32_t *ck = reinterpret_cast<const uint32_t *>(cand);
        auto okey = [&](int i) { return ord_key(as_f(ck[2 * i + 1]) + 0.0f); };  // key bits
        uint32_t a0 = (uint32_t)lane < total ? okey(lane) : 0u;
        uint32_t xk, xn;
        if (wave_any(total > (uint32_t)LPT)) {
            uint32_t a1 = (uint32_t)(lane + LPT) < total ? okey(lane + LPT) : 0u;
            sort_desc32x2<LPT>(a0, a1);
            xk = K <= LPT ? group_bcast<LPT>(a0, K - 1)
                          : group_bcast<LPT>(a1, (K - 1 - LPT) & (LPT - 1));
            xn = K < LPT ? group_bcast<LPT>(a0, K)
                         : (K < 2 * LPT ? group_bcast<LPT>(a1, K - LPT) : 0u);
        } else {
            constexpr int H = LPT == 32 ? 16 : LPT;  // as for the 64-bit sort below
            if (H < LPT && !wave_any(total > (uint32_t)H)) {
                a0 = sort_desc32<H>(a0);
                xn = K < H ? group_bcast<LPT>(a0, K) : 0u;
            } else {
                a0 = sort_desc32<LPT>(a0);
                xn = K < LPT ? group_bcast<LPT>(a0, K) : 0u;
            }
            xk = group_bcast<LPT>(a0, K <= LPT ? K - 1 : LPT - 1);
        }
        // candidates' keys are never 0 (finite floats map above it); idle
        // groups have none, so xn == 0 there
        if (!wave_any(xn != 0u && xn == xk)) {
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
            return Thresh{ord_key_inv(xk), 0xFFFFFFFFu};
        }
    }
    auto repack = [](uint64_t raw) {
        return ((uint64_t)ord_key(as_f((uint32_t)(raw >> 32)) + 0.0f) << 32) | (uint32_t)raw;
    };
    uint64_t v0 = cand[lane];
    v0 = (uint32_t)lane < total ? repack(v0) : 0ull;
    uint64_t next, t64 = 0;
    if (wave_any(total > (uint32_t)LPT)) {
        uint64_t v1 = cand[lane + LPT];
        v1 = (uint32_t)(lane + LPT) < total ? repack(v1) : 0ull;
        sort_desc64x2<LPT>(v0, v1);
        // the K-th and (K+1)-th are positions K-1 and K of the 2*LPT slots
        if constexpr (TOP2) {
            if (K > LPT)
                t64 = group_bcast64<LPT>(v1, K - 1 - LPT);
            next = K < LPT ? group_bcast64<LPT>(v0, K)
                           : (K < 2 * LPT ? group_bcast64<LPT>(v1, K - LPT) : 0ull);
        } else {
            next = K < LPT ? group_bcast64<LPT>(v0, K) : group_bcast64<LPT>(v1, 0);
        }
    } else {
        // no group of the wave has more than LPT candidates: every token of
        // the wave has K <= LPT (with K > LPT the wave is idle, past T, and
        // stores nothing).  32-lane groups with at most 16 candidates
        // everywhere sort only their first 16 lanes (the others hold no
        // candidate): positions K-1 and K are then in those lanes, or K is
        // 16 and equals the count, so there is no (K+1)-th.  (Compiled into
        // the 64-lane kernels the same branch slowed the 2304-expert forward
        // by 3%, where it is never taken.)
        constexpr int H = LPT == 32 ? 16 : LPT;
        if (H < LPT && !wave_any(total > (uint32_t)H)) {
            v0 = sort_desc64<H>(v0);
            next = K < H ? group_bcast64<LPT>(v0, K) : 0ull;
        } else {
            v0 = sort_desc64<LPT>(v0);
            next = K < LPT ? group_bcast64<LPT>(v0, K) : 0ull;
        }
    }
    if (!TOP2 || K <= LPT)
        t64 = group_bcast64<LPT>(v0, K - 1);  // in the first half
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    Thresh t = unpack_thresh(t64);
    if ((next >> 32) != (t64 >> 32))
        t.j = 0xFFFFFFFFu;
    return t;
}

// Group-limited routing.  Group g = experts [g*P, (g+1)*P); its score is
// the fp32 sum of its q largest values s + b, largest first; the Kg best
// groups stay (ties keep the lower group) and the keys of every other
// expert become -inf.  The caller first stores each element's value with
// group_value_store into gscr (group_scratch_floats(E, G, LPT) floats of
// LDS for this token group: one padding word after each group so the
// per-group scans touch distinct banks, and a dummy word per lane for
// padding elements).  Requires G <= LPT.

__device__ __forceinline__ int group_of(int j, float invP)
{
    return (int)(((float)j + 0.5f) * invP);  // exact for E <= 2^20
}

__device__ __forceinline__ void group_value_store(float *gscr, int j, bool real, float v,
                                                  const FwdParams &p, float invP, int lane)
{
    gscr[real ? j + group_of(j, invP) : p.E + p.G + lane] = v;
}

template <int LPT, int NCH, bool VEC>
__device__ __forceinline__ void group_limit(float (&key)[NCH][4], const FwdParams &p,
                                            int lane, int j_lane, bool tok, float invP,
                                            const float *gscr)
{
    const int G = p.G, P = p.P;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    float h = -INFINITY;
    if (lane < G && tok) {
        const float *gv = gscr + lane * (P + 1);
        if (p.q <= 4) {
            // one pass keeping the 4 largest values, sorted (insertion by
            // max/min from the bottom up); the sum takes the first q,
            // largest first
            float t0 = -INFINITY, t1 = -INFINITY, t2 = -INFINITY, t3 = -INFINITY;
            for (int i = 0; i < P; i++) {
                const float v = gv[i];
                t3 = fmaxf(t3, fminf(t2, v));
                t2 = fmaxf(t2, fminf(t1, v));
                t1 = fmaxf(t1, fminf(t0, v));
                t0 = fmaxf(t0, v);
            }
            h = t0;
            if (p.q > 1)
                h = h + t1;
            if (p.q > 2)
                h = h + t2;
            if (p.q > 3)
                h = h + t3;
        } else {
            // q rounds, each taking the next largest (value, lower index)
            float acc = 0.0f, pv = INFINITY;
            int pi = -1;
            for (int r = 0; r < p.q; r++) {
                float bv = -INFINITY;
                int bi = P;
                for (int i = 0; i < P; i++) {
                    const float v = gv[i];
                    const bool below = v < pv || (v == pv && i > pi);
                    const bool better = v > bv || (v == bv && i < bi);
                    bv = (below && better) ? v : bv;
                    bi = (below && better) ? i : bi;
                }
                acc = acc + bv;
                pv = bv;
                pi = bi;
            }
            h = acc;
        }
    }
    // rank of group `lane` among the G scores (ties: lower group)
    uint32_t rank = 0;
    for (int g2 = 0; g2 < G; g2++) {
        const float o = as_f(group_bcast<LPT>(as_u(h), g2));
        rank += (o > h) || (o == h && g2 < lane);
    }
    const bool kept = lane < G && rank < (uint32_t)p.Kg;
    const uint64_t gmask = __builtin_amdgcn_ballot_w64(kept) >> (lane_id() & ~(LPT - 1));
#pragma unroll
    for (int c = 0; c < NCH; c++)
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int g = group_of(jrel<LPT, VEC>(c, u) + j_lane, invP);
            const bool in = g < G && ((gmask >> (g & 63)) & 1ull);
            key[c][u] = in ? key[c][u] : -INFINITY;
        }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Group-limited routing in registers, for groups that tile the chunk
// layout: P = 4*L with L a power of two no larger than LPT, so group g
// of a row is lanes [s*L, (s+1)*L) of chunk c with g = c*(LPT/L) + s, and
// each lane's four elements of a chunk share one group.  The same result
// as group_limit (same group scores, bit for bit, and the same kept
// groups), without LDS: each lane sorts its four values, the lists merge
// across the L lanes of the group (the merge steps of group_allreduce_u
// whose lane distance is below L), and every lane ranks its groups against
// all others, read with one cross-lane permute per group slot.
//
// Merge of two descending lists a, b of length Q into the Q largest of
// both, descending: max(a_i, b_{Q-1-i}) holds exactly those values in a
// V-shaped order, which one bitonic pass sorts.  Group values are never
// NaN and never -0 (s >= +0, and s + b rounds an exact zero to +0).
template <int Q>
__device__ __forceinline__ void topq_merge(float (&a)[Q], const float (&b)[Q])
{
    float c[Q];
#pragma unroll
    for (int i = 0; i < Q; i++)
        c[i] = vmax(a[i], b[Q - 1 - i]);
    if constexpr (Q == 2) {
        a[0] = vmax(c[0], c[1]);
        a[1] = vmin(c[0], c[1]);
    } else {
        static_assert(Q == 4, "lists of 2 or 4");
        const float h0 = vmax(c[0], c[2]), l0 = vmin(c[0], c[2]);
        const float h1 = vmax(c[1], c[3]), l1 = vmin(c[1], c[3]);
        a[0] = vmax(h0, h1);
        a[1] = vmin(h0, h1);
        a[2] = vmax(l0, l1);
        a[3] = vmin(l0, l1);
    }
}

// The Q largest of four values, descending.
template <int Q>
__device__ __forceinline__ void topq_of4(const float (&x)[4], float (&t)[Q])
{
    const float a = vmax(x[0], x[1]), b = vmin(x[0], x[1]);
    const float c = vmax(x[2], x[3]), d = vmin(x[2], x[3]);
    if constexpr (Q == 2) {
        t[0] = vmax(a, c);
        t[1] = vmax(vmin(a, c), vmax(b, d));
    } else {
        static_assert(Q == 4, "lists of 2 or 4");
        t[0] = vmax(a, c);
        t[3] = vmin(b, d);
        const float m1 = vmin(a, c), m2 = vmax(b, d);
        t[1] = vmax(m1, m2);
        t[2] = vmin(m1, m2);
    }
}

// One merge step with the list of the lane at distance D (lane ^ D for
// D = 1, 2; the mirror image inside blocks of 2D lanes from D = 4 on, which
// pairs blocks of D lanes that already agree).
template <int D, int Q>
__device__ __forceinline__ void topq_step(float (&t)[Q])
{
    float o[Q];
#pragma unroll
    for (int i = 0; i < Q; i++) {
        const uint32_t v = as_u(t[i]);
        uint32_t w;
        if constexpr (D == 1)
            w = dpp_mov<kQpXor1>(v);
        else if constexpr (D == 2)
            w = dpp_mov<kQpXor2>(v);
        else if constexpr (D == 4)
            w = dpp_mov<kRowHalfMirror>(v);
        else if constexpr (D == 8)
            w = dpp_mov<kRowMirror>(v);
        else
            w = shfl_xor<D>(v);
        o[i] = as_f(w);
    }
    topq_merge<Q>(t, o);
}

// Group stage for 2^LG lanes per group and lists of Q values (q <= Q).
// With BOUND and a bias (keys == group values) it returns a lower bound of
// the K-th largest key: the kept groups' q largest values are Kg*q = K
// distinct experts, so their minimum is at most the K-th largest key;
// otherwise -inf.
template <int LPT, int NCH, int LG, int Q, bool BOUND>
__device__ __forceinline__ float group_limit_reg_t(float (&key)[NCH][4],
                                                   const float (&s)[NCH][4], bool has_bias,
                                                   const FwdParams &p, int lane)
{
    constexpr int L = 1 << LG;
    constexpr int NS = LPT / L;  // groups per chunk
    float h[NCH], tq[NCH];
#pragma unroll
    for (int c = 0; c < NCH; c++) {
        float x[4];
#pragma unroll
        for (int u = 0; u < 4; u++)
            x[u] = has_bias ? key[c][u] : s[c][u];  // s + b (the keys hold it with a bias)
        float t[Q];
        topq_of4<Q>(x, t);
        if constexpr (L > 1)
            topq_step<1, Q>(t);
        if constexpr (L > 2)
            topq_step<2, Q>(t);
        if constexpr (L > 4)
            topq_step<4, Q>(t);
        if constexpr (L > 8)
            topq_step<8, Q>(t);
        if constexpr (L > 16)
            topq_step<16, Q>(t);
        if constexpr (L > 32)
            topq_step<32, Q>(t);
        float a = t[0], v = t[0];
#pragma unroll
        for (int i = 1; i < Q; i++) {
            a = p.q > i ? a + t[i] : a;
            v = p.q > i ? t[i] : v;  // the q-th largest
        }
        h[c] = a;
        tq[c] = BOUND ? v : 0.0f;
    }

    // every lane reads all S = NCH*NS group slots; lane i < S ranks slot i
    // among the G real ones (ties: lower group; slots past G are padding
    // past E), and one ballot hands the kept groups to every lane
    constexpr int S = NCH * NS;
    static_assert(S <= LPT, "one lane per group slot");
    const int base = lane_id() & ~(LPT - 1);
    float o[S];
#pragma unroll
    for (int c2 = 0; c2 < NCH; c2++)
#pragma unroll
        for (int s2 = 0; s2 < NS; s2++)
            o[c2 * NS + s2] = as_f((uint32_t)__builtin_amdgcn_ds_bpermute(
                (base + s2 * L) << 2, (int)as_u(h[c2])));
    float mine = o[0];
#pragma unroll
    for (int g = 1; g < S; g++)
        mine = lane == g ? o[g] : mine;
    uint32_t rank = 0;
#pragma unroll
    for (int g2 = 0; g2 < S; g2++) {
        // bitwise, so no branch per comparison
        const uint32_t beats = (uint32_t)(o[g2] > mine) |
                               ((uint32_t)(o[g2] == mine) & (uint32_t)(g2 < lane));
        rank += g2 < p.G ? beats : 0u;
    }
    const bool kept_slot = (lane < p.G) & (rank < (uint32_t)p.Kg);
    const uint64_t kept = __builtin_amdgcn_ballot_w64(kept_slot) >> base;
    const int seg = lane >> LG;
    float m = INFINITY;
#pragma unroll
    for (int c = 0; c < NCH; c++) {
        const bool in = (kept >> (c * NS + seg)) & 1u;
#pragma unroll
        for (int u = 0; u < 4; u++)
            key[c][u] = in ? key[c][u] : -INFINITY;
        if constexpr (BOUND)
            m = in ? vmin(m, tq[c]) : m;
    }
    if (!BOUND || !has_bias)
        return -INFINITY;
    return as_f(group_allreduce_u<LPT>(as_u(m), [](uint32_t x, uint32_t y) {
        return as_u(vmin(as_f(x), as_f(y)));
    }));
}

// Dispatch on the lanes per group (P / 4, a power of two here) and the
// list length; the host takes this stage only for the combinations built
// here (group_reg_ok).
template <int LPT, int NCH, bool BOUND>
__device__ __forceinline__ float group_limit_reg(float (&key)[NCH][4], const float (&s)[NCH][4],
                                                 bool has_bias, const FwdParams &p, int lane)
{
    float bound = -INFINITY;
    auto run = [&](auto lg) {
        constexpr int LG = decltype(lg)::value;
        if constexpr (group_reg_ok(LPT, NCH, LG)) {
            if (p.q <= 2)
                bound = group_limit_reg_t<LPT, NCH, LG, 2, BOUND>(key, s, has_bias, p, lane);
            else
                bound = group_limit_reg_t<LPT, NCH, LG, 4, BOUND>(key, s, has_bias, p, lane);
        }
    };
    switch (__builtin_ctz((unsigned)p.P) - 2) {
    case 0: run(std::integral_constant<int, 0>{}); break;
    case 1: run(std::integral_constant<int, 1>{}); break;
    case 2: run(std::integral_constant<int, 2>{}); break;
    case 3: run(std::integral_constant<int, 3>{}); break;
    case 4: run(std::integral_constant<int, 4>{}); break;
    case 5: run(std::integral_constant<int, 5>{}); break;
    default: run(std::integral_constant<int, 6>{}); break;
    }
    return bound;
}

// ------------------------------------------------------------ forward

// SEL_ARGMAX kernels run the argmax rounds; SEL_PRUNE kernels run the
// pruned sort, or the bit search when p.sel == SEL_BITS.  GM selects
// group-limited routing (p.G > 0): GROUP_NONE, GROUP_LDS (group_limit, any
// P) or GROUP_REG (group_limit_reg, groups that tile the chunks).
//
// Rows of 16 chunks (3072 < E <= 4096) take the lane index through an
// opaque copy in every token iteration: otherwise the per-chunk offsets and
// range tests derived from it were hoisted out of the token loop and held
// in about 40 registers for the kernel's life, which left one wave per
// SIMD (softmax 306 -> 256 VGPRs, 2 waves per SIMD; T=8192, E=4096: 89.9 ->
// 83.6 us).  The sigmoid rows (262 VGPRs with the copy) also ask for 2
// waves per SIMD, which they reach without scratch (92.9 -> 84.2 us); the
// softmax rows ran slower with that request (92.6 us).  The bf16 rows of
// 6 chunks and more take the copy too, and those of 9 and 12 chunks ask
// for 3 waves per SIMD (a bf16 row moves half the logit bytes, so the
// same per-element arithmetic is less hidden and more rows in flight pay):
// T=8192, bf16 softmax E=1536 25.2 -> 23.5 us, E=2048 33.7 -> 29.3,
// E=2304 38.4 -> 32.4 (K=36; sigmoid 41.1 -> 33.4), E=3072 70.2 -> 43.1
// (K=8; K=36 75.0 -> 43.8, with 20-40 bytes of scratch at 3 waves).  The
// fp32 rows ran slower with the copy at 12 chunks (E=3072: 56.3 -> 58.1
// us) and with 3 waves per SIMD at 9 (E=2304: 44.2 -> 47.5 us).
template <int LPT, int NCH, typename TIn, int SCORE, int SEL, int GM, bool VEC,
          int WPB = kWaves>
__global__ void __launch_bounds__(
    64 * WPB, GM == GROUP_LDS && VEC && NCH <= 4 ? 3
              : GM == GROUP_REG ? (NCH <= 2 && LPT >= 32 ? 5 : 4)
              : GM != GROUP_NONE || !VEC ? 1
              : NCH == 16 && SCORE == SCORE_SIGMOID ? 2
              : (NCH == 9 || NCH == 12) && sizeof(TIn) == 2 ? 3 : 1)
fwd_kernel(FwdParams p)
{
    constexpr int GPW = 64 / LPT;            // token groups per wave
    constexpr int TPB = WPB * GPW;           // tokens per block (WPB waves)
    constexpr int VPL = NCH * 4;
    extern __shared__ uint64_t smem[];

    const int lane64 = lane_id();
    const int lane0 = lane64 & (LPT - 1);
    const int grp = lane64 / LPT;                          // group in wave
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int gslot = wave * GPW + grp;                    // group in block
    uint64_t *cand = smem + gslot * cand_slots(LPT);
    const int E = p.E;
    const uint32_t goff = (uint32_t)(grp * E);             // group row in the wave buffer
    // The host takes an expert bias with the sigmoid only.  The softmax
    // rows of 16 chunks drop the bias code at compile time, which freed
    // registers they need (T=8192, E=4096, K=36: 136 -> 90 us); narrower
    // softmax rows keep the run-time test, which measured faster there
    // (E=512, K=8: 9.8 against 10.7 us; E=3072: 56.6 against 57.4 us).
    const bool has_bias = (SCORE == SCORE_SIGMOID || NCH < 16) && p.bias != nullptr;

    for (int64_t tb = (int64_t)blockIdx.x * TPB; tb < p.T;
         tb += (int64_t)gridDim.x * TPB) {
        int lane = lane0;
        if constexpr (NCH >= 16 || (NCH >= 6 && sizeof(TIn) == 2))
            asm volatile("" : "+v"(lane));  // per iteration: see above
        const int j_lane = lane_part<VEC>(lane);
        const int64_t t0 = tb + wave * GPW;                // first token of the wave
        const int64_t left = p.T - t0;
        const int nval = left <= 0 ? 0 : (left >= GPW ? GPW : (int)left);
        const bool tok = grp < nval;
        const int Ev = tok ? E : 0;
        const int64_t off0 = nval ? t0 * (int64_t)E : 0;
        const uint32_t nel = (uint32_t)(nval * E);
        const rsrc_t rx = make_rsrc(static_cast<const TIn *>(p.x) + off0, nel * io<TIn>::kSize);

        // key[][] holds the logits (-inf on padding) and becomes the keys.
        // The 8- and 9-chunk rows request their logits as stored and mask
        // (and unpack) them only after every load is in flight; with the
        // masking next to each load the compiler waited for a chunk before
        // the later loads were issued.  Measured at T=8192 on one machine:
        // E=1792 38.1 -> 35.4 us, E=2048 40.1 -> 38.7, E=2304 44.4 -> 44.0;
        // at 6 and 12 chunks it was 3-5% slower, so they keep the plain load.
        // The element-wise rows do the same at every width (E=4094: 356 ->
        // 205 us; no change at 4 to 12 chunks).
        float key[NCH][4];
        constexpr bool kRaw = (VEC && LPT == 64 && NCH >= 8 && NCH <= 9) || !VEC;
#pragma unroll
        for (int c = 0; c < NCH; c++) {
            if constexpr (kRaw)
                load_chunk_raw<LPT, TIn, VEC>(rx, goff, c, j_lane, Ev, -INFINITY, key[c]);
            else
                load_chunk<LPT, TIn, VEC>(rx, goff, c, j_lane, Ev, -INFINITY, key[c]);
        }
        __builtin_amdgcn_sched_barrier(0);  // every load in flight before any math
        if constexpr (kRaw) {
#pragma unroll
            for (int c = 0; c < NCH; c++)
                mask_chunk<LPT, TIn, VEC>(c, j_lane, Ev, -INFINITY, key[c]);
        }

        // ---- score function
        float s[NCH][4];
        float mx = 0.0f;
        if constexpr (SCORE == SCORE_SOFTMAX) {
            float m = -INFINITY;
#pragma unroll
            for (int c = 0; c < NCH; c++)
#pragma unroll
                for (int u = 0; u < 4; u++)
                    m = vmax(m, key[c][u]);  // logits: finite, or -inf padding
            mx = group_max<LPT>(m);
            mx = tok ? mx : 0.0f;
        }
        // Sigmoid on padding (key -inf): the vector kernels skip it with a
        // branch (about 3% faster at E = 512 and 2304 than computing and
        // dropping it).  The element-wise kernels compute it on every element
        // and select: there the branch led hipcc to place a register copy of
        // another element's score in the join block ahead of the exec
        // restore (16-chunk forward), so lanes with padding kept a stale
        // value.  A code-generation test rejects that pattern in every kernel.
#pragma unroll
        for (int c = 0; c < NCH; c++)
#pragma unroll
            for (int u = 0; u < 4; u++) {
                if constexpr (SCORE == SCORE_SOFTMAX) {
                    s[c][u] = exp_split(key[c][u] - mx);           // padding: exactly 0
                } else {
                    if constexpr (VEC) {
                        s[c][u] = key[c][u] == -INFINITY ? 0.0f : sigmoid_fast(key[c][u]);
                    } else {
                        const float sg = sigmoid_fast(key[c][u]);
                        s[c][u] = key[c][u] == -INFINITY ? 0.0f : sg;
                    }
                }
            }
        if constexpr (SCORE == SCORE_SOFTMAX) {
            const float z = group_sum<LPT>(tree_sum<VPL>(&s[0][0]));
            // the divisions here run on every lane (idle groups divide by
            // 0 and the select drops the result): kept out of lane-divergent
            // branches, like the sigmoid above
            const float rz0 = 1.0f / z;
            const float rz = tok ? rz0 : 0.0f;
#pragma unroll
            for (int c = 0; c < NCH; c++)
#pragma unroll
                for (int u = 0; u < 4; u++)
                    s[c][u] *= rz;
        }

        // ---- expert bias (selection only) and group values s + b
        [[maybe_unused]] float *gscr = nullptr;
        [[maybe_unused]] float invP = 0.0f;
        if constexpr (GM == GROUP_LDS) {
            gscr = reinterpret_cast<float *>(smem + TPB * cand_slots(LPT)) +
                   gslot * group_scratch_floats(E, p.G, LPT);
            invP = 1.0f / (float)p.P;
        }
        if (has_bias || GM == GROUP_LDS) {
            const rsrc_t rb = make_rsrc(p.bias, has_bias ? (uint32_t)E * 4u : 0u);
#pragma unroll
            for (int c = 0; c < NCH; c++) {
                float b[4];
                // the bias is shared by every token: default cache policy
                load_chunk<LPT, float, VEC, 0>(rb, 0u, c, j_lane, Ev, 0.0f, b);
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    const float r = s[c][u] + b[u];
                    const bool real = key[c][u] != -INFINITY;
                    if constexpr (GM == GROUP_LDS)
                        group_value_store(gscr, jrel<LPT, VEC>(c, u) + j_lane, real, r, p, invP, lane);
                    if (has_bias)
                        key[c][u] = real ? r : -INFINITY;
                }
            }
        }

        // ---- the intermediate is final: store it now, so its writes overlap
        // the selection work (no global load follows in this iteration, so
        // no wait on the memory counter covers these stores; ~6% at E=2304).
        // Probs and map wait for the selection: storing the chunks known to
        // be zero early splits cache lines between two write bursts, which
        // measured 1.7x slower.
        const rsrc_t ri = make_rsrc(p.inter + off0, nel * 4u);
#pragma unroll
        for (int c = 0; c < NCH; c++)
            store_chunk<LPT, float, VEC>(ri, goff, c, j_lane, E, s[c]);

        if constexpr (GM == GROUP_LDS)
            group_limit<LPT, NCH, VEC>(key, p, lane, j_lane, tok, invP, gscr);
        // with a bias, the group stage also bounds the K-th key from below
        // (see group_limit_reg_t), which spares the pruned select its sort
        // of the lane maxima (grouped bf16 forward: 778 -> 740 VALU
        // instructions per wave, 14.4 -> 13.9 us)
        constexpr bool kGroupBound = GM == GROUP_REG && NCH <= 2;
        [[maybe_unused]] float bound = -INFINITY;
        if constexpr (GM == GROUP_REG) {
            // The group stage's lane masks (lane == slot, slot < lane) do not
            // depend on the token, so the compiler hoisted them out of the
            // token loop as SGPR pairs, ran out of SGPRs and reloaded each
            // from a VGPR lane at every use.  An opaque copy of the lane
            // index keeps them per iteration: one compare each (T=16384,
            // E=256, 8 groups, bf16: 884 -> 828 VALU instructions per wave,
            // 15.6 -> 14.7 us).
            int lane_i = lane;
            asm volatile("" : "+v"(lane_i));
            bound = group_limit_reg<LPT, NCH, kGroupBound>(key, s, has_bias, p, lane_i);
        }

        // ---- top-K; the selection lives in the map words (one byte per
        // element, chunk-packed), which the store needs anyway
        uint32_t mw[NCH];
        if constexpr (SEL == SEL_ARGMAX) {
            select_argmax<LPT, NCH, VEC>(key, p.K, j_lane);
#pragma unroll
            for (int c = 0; c < NCH; c++) {
                uint32_t w = 0;
#pragma unroll
                for (int u = 0; u < 4; u++)
                    w |= (uint32_t)(key[c][u] != key[c][u]) << (8 * u);  // NaN: taken
                mw[c] = w;
            }
        } else {
            const Thresh t = p.sel == SEL_BITS
                                 ? select_bits<LPT, NCH, VEC>(key, p.K, j_lane)
                                 : select_prune<LPT, NCH, prune_top2(LPT, GM), GM != GROUP_REG && LPT < 64, VEC>(
                                       key, p.K, lane, j_lane, cand,
                                       // the bound's live values spilled the
                                       // register-capped 4-chunk kernels
                                       kGroupBound && has_bias, bound);
            // idle groups (past T) store nothing; give them a threshold no key meets
            const float tx = tok ? t.x : INFINITY;
            if (!wave_any(t.j != 0xFFFFFFFFu)) {
#pragma unroll
                for (int c = 0; c < NCH; c++) {
                    uint32_t w = 0;
#pragma unroll
                    for (int u = 0; u < 4; u++)
                        w |= (uint32_t)(key[c][u] >= tx) << (8 * u);
                    mw[c] = w;
                }
            } else {
                const int jt = (int)t.j - j_lane;  // lane-relative; "all" stays large
#pragma unroll
                for (int c = 0; c < NCH; c++) {
                    uint32_t w = 0;
#pragma unroll
                    for (int u = 0; u < 4; u++) {
                        const float k = key[c][u];
                        const bool in = k > tx || (k == tx && (t.j == 0xFFFFFFFFu ||
                                                               jrel<LPT, VEC>(c, u) <= jt));
                        w |= (uint32_t)in << (8 * u);
                    }
                    mw[c] = w;
                }
            }
        }

        // ---- weights: out = keep ? s * mult : 0, keep = aux or selected
        const bool all = p.aux != 0;
        const uint32_t keep_all = all ? 0x01010101u : 0u;
        const bool norm = all ? (SCORE == SCORE_SIGMOID && p.renorm)
                              : (p.renorm && (SCORE == SCORE_SOFTMAX || p.K > 1));
        float mult = all ? 1.0f : p.scale;
        if (norm) {
            float part[NCH];
#pragma unroll
            for (int c = 0; c < NCH; c++) {
                const uint32_t kw = mw[c] | keep_all;
                float a4[4];
#pragma unroll
                for (int u = 0; u < 4; u++)
                    a4[u] = ((kw >> (8 * u)) & 0xFFu) ? s[c][u] : 0.0f;
                part[c] = (a4[0] + a4[1]) + (a4[2] + a4[3]);
            }
            const float a = group_sum<LPT>(tree_sum<NCH>(part));
            const float mq = mult / a;
            mult = tok ? mq : 0.0f;
        }

        // ---- stores (tokens past T fall outside the buffers and are dropped)
        const rsrc_t ro = make_rsrc(static_cast<TIn *>(p.out) + off0, nel * io<TIn>::kSize);
        const rsrc_t rm = make_rsrc(p.map + off0, nel);
#pragma unroll
        for (int c = 0; c < NCH; c++) {
            const uint32_t kw = mw[c] | keep_all;
            float o[4];
#pragma unroll
            for (int u = 0; u < 4; u++)
                o[u] = ((kw >> (8 * u)) & 0xFFu) ? s[c][u] * mult : 0.0f;
            store_chunk<LPT, TIn, VEC>(ro, goff, c, j_lane, E, o);
            store_map_chunk<LPT, VEC>(rm, goff, c, j_lane, E, mw[c]);
        }
    }
}

// ------------------------------------------------------------ backward
//
// Every mode is dx = w * (gm - beta) with per-token uniforms:
//   w    = base * alpha * (mask_w ? m : 1),  base = s (softmax) or s(1-s)
//   gm   = mask_g ? m g : g
//   softmax, no renorm:   alpha = c,    beta = B,   mask_g        (aux: c = 1)
//   softmax, renorm:      alpha = c/A,  beta = B/A, mask_w
//   sigmoid, renorm, K>1: alpha = c/A,  beta = B/A, mask_w        (aux: c = 1, m = 1)
//   sigmoid otherwise:    alpha = c,    beta = 0,   mask_w
// with A = sum m s and B = sum g m s over the token.

template <int LPT, int NCH, typename TIn, int SCORE, bool VEC>
__global__ void __launch_bounds__(kBlock)
bwd_kernel(BwdParams p)
{
    constexpr int GPW = 64 / LPT;
    constexpr int TPB = kWaves * GPW;

    const int lane64 = lane_id();
    const int lane0 = lane64 & (LPT - 1);
    const int grp = lane64 / LPT;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int E = p.E;
    const uint32_t goff = (uint32_t)(grp * E);
    const bool aux = p.m == nullptr;
    const bool renorm_mode = p.renorm && (SCORE == SCORE_SOFTMAX ? !aux : (aux || p.K > 1));
    const float c0 = aux ? 1.0f : p.scale;
    const float mask_w = (SCORE == SCORE_SOFTMAX && !renorm_mode) ? 0.0f : 1.0f;
    const float mask_g = 1.0f - mask_w;

    for (int64_t tb = (int64_t)blockIdx.x * TPB; tb < p.T;
         tb += (int64_t)gridDim.x * TPB) {
        // rows of 12 and 16 chunks: an opaque copy of the lane index per
        // iteration keeps the per-chunk offsets and range masks out of
        // registers held across the token loop
        int lane = lane0;
        if constexpr (NCH >= 12)
            asm volatile("" : "+v"(lane));
        const int j_lane = lane_part<VEC>(lane);
        const int64_t t0 = tb + wave * GPW;
        const int64_t left = p.T - t0;
        const int nval = left <= 0 ? 0 : (left >= GPW ? GPW : (int)left);
        const int Ev = grp < nval ? E : 0;
        const int64_t off0 = nval ? t0 * (int64_t)E : 0;
        const uint32_t nel = (uint32_t)(nval * E);
        const rsrc_t rg = make_rsrc(static_cast<const TIn *>(p.g) + off0, nel * io<TIn>::kSize);
        const rsrc_t rs = make_rsrc(p.s + off0, nel * 4u);
        const rsrc_t rm = make_rsrc(aux ? nullptr : p.m + off0, aux ? 0u : nel);

        float g[NCH][4], s[NCH][4];
        uint32_t mw[NCH];
        if constexpr (VEC) {
#pragma unroll
            for (int c = 0; c < NCH; c++) {
                load_chunk<LPT, TIn, VEC>(rg, goff, c, j_lane, Ev, 0.0f, g[c]);
                load_chunk<LPT, float, VEC>(rs, goff, c, j_lane, Ev, 0.0f, s[c]);
                mw[c] = load_map_chunk<LPT, VEC>(rm, goff, c, j_lane, Ev);  // aux: 0
            }
            __builtin_amdgcn_sched_barrier(0);  // every load in flight before any math
        } else {
            // Element-wise rows: every access is issued as stored before any
            // value is used (a masked one reads 0, which is the padding of
            // g, s and the map); widening bf16 or packing the map bytes next
            // to each load let the compiler wait for it before issuing the
            // next one (T=8192, E=2302 softmax: 119.7 -> 52.9 us).
            uint32_t gw[NCH][4], sw[NCH][4], mb[NCH][4];
#pragma unroll
            for (int c = 0; c < NCH; c++)
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    const int j = jrel<LPT, VEC>(c, u) + j_lane;
                    const bool ok = j < Ev;
                    const uint32_t jo = goff + (uint32_t)j;
                    if constexpr (sizeof(TIn) == 2)
                        gw[c][u] = __builtin_amdgcn_raw_buffer_load_b16(
                            rg, (int)(ok ? jo * 2u : kOOB), 0, kStream);
                    else
                        gw[c][u] = __builtin_amdgcn_raw_buffer_load_b32(
                            rg, (int)(ok ? jo * 4u : kOOB), 0, kStream);
                    sw[c][u] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(ok ? jo * 4u : kOOB),
                                                                    0, kStream);
                    mb[c][u] = __builtin_amdgcn_raw_buffer_load_b8(rm, (int)(ok ? jo : kOOB), 0,
                                                                   kStream);
                }
            __builtin_amdgcn_sched_barrier(0);  // every load in flight before any math
#pragma unroll
            for (int c = 0; c < NCH; c++) {
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    g[c][u] = sizeof(TIn) == 2 ? as_f(gw[c][u] << 16) : as_f(gw[c][u]);
                    s[c][u] = as_f(sw[c][u]);
                }
                mw[c] = mb[c][0] | (mb[c][1] << 8) | (mb[c][2] << 16) | (mb[c][3] << 24);
            }
        }
        // aux: every expert routed (padding has s = g = 0 and adds nothing)
        // (element-wise rows: selects, no branch after the loads; see below)
        if constexpr (VEC) {
            if (aux) {
#pragma unroll
                for (int c = 0; c < NCH; c++)
                    mw[c] = 0x01010101u;
            }
        } else {
#pragma unroll
            for (int c = 0; c < NCH; c++)
                mw[c] = aux ? 0x01010101u : mw[c];
        }
        // A and B, and the mode chosen by selects.  With the sigmoid a
        // branch on the mode here let the compiler sink the g and s loads
        // below it, behind a wait for the map (two round trips per row, the
        // map bytes expanded twice, 236 VGPRs at 9 chunks; E=4096, K=16:
        // 152 -> 74 us), so its A and B are always computed.  The softmax
        // needs B always and A for renormalisation only; its branch is
        // harmless in the vector rows (the loads stay above it) and skips a
        // reduction.  The element-wise rows compute A always and set the aux
        // map by a select (T=8192, softmax, E=2302: 223.6 -> 133.8 us,
        // E=3070: 152.7 -> 130.5, E=2046: 86.5 -> 81.0).
        float pa[NCH], pb[NCH];
#pragma unroll
        for (int c = 0; c < NCH; c++) {
            float a4[4], b4[4];
#pragma unroll
            for (int u = 0; u < 4; u++) {
                a4[u] = ((mw[c] >> (8 * u)) & 0xFFu) ? s[c][u] : 0.0f;
                b4[u] = g[c][u] * a4[u];
            }
            pa[c] = (a4[0] + a4[1]) + (a4[2] + a4[3]);
            pb[c] = (b4[0] + b4[1]) + (b4[2] + b4[3]);
        }
        float A = 1.0f;
        if constexpr (SCORE == SCORE_SOFTMAX && VEC) {
            if (renorm_mode)
                A = group_sum<LPT>(tree_sum<NCH>(pa));
        } else {
            A = group_sum<LPT>(tree_sum<NCH>(pa));
        }
        const float B = group_sum<LPT>(tree_sum<NCH>(pb));
        const float rA0 = 1.0f / A;  // every lane: no divergent branch
        const float rA = Ev ? rA0 : 0.0f;
        const float alpha = renorm_mode ? c0 * rA : c0;
        const float beta = renorm_mode ? B * rA : (SCORE == SCORE_SOFTMAX ? B : 0.0f);
        const rsrc_t rd = make_rsrc(static_cast<TIn *>(p.dx) + off0, nel * io<TIn>::kSize);
#pragma unroll
        for (int c = 0; c < NCH; c++) {
            float d[4];
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const float sv = s[c][u];
                const float m = ((mw[c] >> (8 * u)) & 0xFFu) ? 1.0f : 0.0f;
                const float base = SCORE == SCORE_SOFTMAX ? sv : sv * (1.0f - sv);
                const float wm = fmaf(mask_w, m - 1.0f, 1.0f);   // mask_w ? m : 1
                const float gm = g[c][u] * fmaf(mask_g, m - 1.0f, 1.0f);
                d[u] = (base * alpha * wm) * (gm - beta);
            }
            store_chunk<LPT, TIn, VEC>(rd, goff, c, j_lane, E, d);
        }
    }
}

}  // namespace rker
