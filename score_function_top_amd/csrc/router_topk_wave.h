// router_topk_wave.h -- ordered top-K of one logits row per wave (decode
// routing and the routed half of the shared-gate kernel).
//
// Lane l holds elements j = c*256 + 4*l + u (NCH chunks).  Scores are the
// softmax over the row or the logistic sigmoid; the selection is on the
// logits (ties to the lower index).  Each lane packs its keys
// ord(x) << 32 | ~j once and sorts them descending in registers (bitonic
// network); slot k is round k of a wave-wide 64-bit maximum of the lanes'
// heads, and the winning lane pops its head (a masked shift of its list).  Lane k < K ends with slot k:
// its expert and its weight (the score, divided by the sum of the K
// selected scores when `renorm`, except for sigmoid with K == 1).
#pragma once

#include "router_io.h"
#include "router_params.h"

namespace rker {

__device__ __forceinline__ uint64_t route_key(float x, uint32_t j)
{
    return ((uint64_t)ord_key(x + 0.0f) << 32) | (uint32_t)~j;
}

// Smallest K for which the sorted path replaces the rounds.
constexpr int kSortedMinK = 4;
// LDS of the sorted path per wave: 2*64 candidate slots and a dummy per lane.
constexpr int kSortedSlots = 3 * 64;

// The sorted path: true and lane k < K holding slot k's packed key in *slot,
// or false (too many keys tie at or above tau) with nothing decided.
template <int NCH>
__device__ __forceinline__ bool sorted_topk(const float (&key)[NCH][4], int K, uint64_t *cand,
                                            uint64_t &slot)
{
    const int lane = lane_id();
    float lm = -INFINITY;
#pragma unroll
    for (int c = 0; c < NCH; c++)
#pragma unroll
        for (int u = 0; u < 4; u++)
            lm = fmaxf(lm, key[c][u]);
    const float tau =
        fmaxf(ord_key_inv(group_bcast<64>(sort_desc32<64>(ord_key(lm + 0.0f)), K - 1)),
              -3.4028234663852886e38f);  // padding (-inf) never competes
    uint32_t cnt = 0;
#pragma unroll
    for (int c = 0; c < NCH; c++)
#pragma unroll
        for (int u = 0; u < 4; u++)
            cnt += !(key[c][u] < tau);
    const uint32_t incl = group_incl_scan<64>(cnt);
    const uint32_t total = group_bcast<64>(incl, 63);
    if (total > 128u)
        return false;
    uint32_t pos = incl - cnt;
    const uint32_t dummy = 128u + (uint32_t)lane;
#pragma unroll
    for (int c = 0; c < NCH; c++)
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const bool in = !(key[c][u] < tau);
            cand[in ? pos : dummy] = route_key(key[c][u], (uint32_t)(c * 256 + 4 * lane + u));
            pos += in;
        }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    uint64_t v0 = (uint32_t)lane < total ? cand[lane] : 0ull;
    if (total > 64u) {
        uint64_t v1 = (uint32_t)(lane + 64) < total ? cand[lane + 64] : 0ull;
        sort_desc64x2<64>(v0, v1);
    } else {
        v0 = sort_desc64<64>(v0);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    slot = v0;
    return true;
}

// A row of E logits, 4 per lane and chunk (element c*256 + 4*lane + u),
// -inf past E.
template <int NCH, typename TIn, bool VEC, int POL = kStream>
__device__ __forceinline__ void wave_topk_load(rsrc_t r, int E, float (&key)[NCH][4])
{
    const int lane = lane_id();
    constexpr uint32_t sz = io<TIn>::kSize;
#pragma unroll
    for (int c = 0; c < NCH; c++) {
        const int j0 = c * 256 + 4 * lane;
        if constexpr (VEC) {
            io<TIn>::template load4<POL>(r, j0 < E ? (uint32_t)j0 * sz : kOOB, 0, key[c]);
#pragma unroll
            for (int u = 0; u < 4; u++)
                key[c][u] = j0 < E ? key[c][u] : -INFINITY;
        } else {
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const bool ok = j0 + u < E;
                const float v = io<TIn>::template load1<POL>(r, ok ? (uint32_t)(j0 + u) * sz : kOOB);
                key[c][u] = ok ? v : -INFINITY;
            }
        }
    }
}

// The ordered top-K of a loaded row: lane k < K gets slot k's expert and
// weight.
template <int NCH>
__device__ __forceinline__ void wave_topk_keys(float (&key)[NCH][4], int K, int score, int renorm,
                                               uint64_t *cand, int &my_id, float &my_w)
{
    const int lane = lane_id();
    float mx = 0.0f, rz = 0.0f;
    if (score == SCORE_SOFTMAX) {
        float m = -INFINITY;
#pragma unroll
        for (int c = 0; c < NCH; c++)
#pragma unroll
            for (int u = 0; u < 4; u++)
                m = fmaxf(m, key[c][u]);
        mx = group_max<64>(m);
        float z = 0.0f;
#pragma unroll
        for (int c = 0; c < NCH; c++)
#pragma unroll
            for (int u = 0; u < 4; u++)
                z += exp_split(key[c][u] - mx);  // padding: exactly 0
        rz = 1.0f / group_sum<64>(z);
    }
    my_id = 0;
    float my_s = 0.0f;
    uint64_t slot = 0;
    const bool sorted = cand != nullptr && K >= kSortedMinK && sorted_topk<NCH>(key, K, cand, slot);
    if (sorted) {
        const uint32_t jw = ~(uint32_t)slot;
        const float xw = ord_key_inv((uint32_t)(slot >> 32));
        my_id = (int)jw;
        my_s = score == SCORE_SOFTMAX ? exp_split(xw - mx) * rz : sigmoid_fast(xw);
    } else {
        constexpr int V = NCH * 4;
        uint64_t lst[V];
#pragma unroll
        for (int c = 0; c < NCH; c++)
#pragma unroll
            for (int u = 0; u < 4; u++)
                lst[c * 4 + u] = key[c][u] == -INFINITY
                                     ? 0ull
                                     : route_key(key[c][u], (uint32_t)(c * 256 + 4 * lane + u));
#pragma unroll
        for (int k2 = 2; k2 <= V; k2 <<= 1)
#pragma unroll
            for (int j2 = k2 >> 1; j2 > 0; j2 >>= 1)
#pragma unroll
                for (int i = 0; i < V; i++) {
                    const int l2 = i ^ j2;
                    if (l2 > i) {
                        // descending where bit k2 of i is clear, ascending where set
                        const bool desc = (i & k2) == 0;
                        const uint64_t a = lst[i], b = lst[l2];
                        const bool swap = desc ? (b > a) : (a > b);
                        lst[i] = swap ? b : a;
                        lst[l2] = swap ? a : b;
                    }
                }
        // The pops below run on the two 32-bit halves with an opaque all-ones /
        // all-zero mask: a select between neighbouring entries would be folded
        // into a load at a computed index and lowered to compare-and-select
        // chains over the whole list every round.
        uint32_t lo[V], hi[V];
#pragma unroll
        for (int i = 0; i < V; i++) {
            lo[i] = (uint32_t)lst[i];
            hi[i] = (uint32_t)(lst[i] >> 32);
        }
        for (int k = 0; k < K; k++) {
            const uint64_t head = ((uint64_t)hi[0] << 32) | lo[0];
            const uint64_t best = group_max_u64<64>(head);
            uint32_t m = head == best ? 0xFFFFFFFFu : 0u;
            asm volatile("" : "+v"(m));
#pragma unroll
            for (int i = 0; i + 1 < V; i++) {
                lo[i] = (lo[i + 1] & m) | (lo[i] & ~m);
                hi[i] = (hi[i + 1] & m) | (hi[i] & ~m);
            }
            lo[V - 1] &= ~m;
            hi[V - 1] &= ~m;
            const uint32_t jw = ~(uint32_t)best;
            const float xw = ord_key_inv((uint32_t)(best >> 32));
            const float sw = score == SCORE_SOFTMAX ? exp_split(xw - mx) * rz : sigmoid_fast(xw);
            my_id = lane == k ? (int)jw : my_id;
            my_s = lane == k ? sw : my_s;
        }
    }
    my_w = my_s;
    if (renorm && (score == SCORE_SOFTMAX || K > 1)) {
        // the selected scores in slot order, summed sequentially
        float den = 0.0f;
        for (int k = 0; k < K; k++)
            den += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), k));
        my_w = my_s / den;
    }
}

// Both: load the row, then select.
template <int NCH, typename TIn, bool VEC, int POL = kStream>
__device__ __forceinline__ void wave_topk_row(rsrc_t r, int E, int K, int score, int renorm,
                                              uint64_t *cand, int &my_id, float &my_w)
{
    float key[NCH][4];
    wave_topk_load<NCH, TIn, VEC, POL>(r, E, key);
    wave_topk_keys<NCH>(key, K, score, renorm, cand, my_id, my_w);
}

}  // namespace rker
