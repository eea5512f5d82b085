// router_grouped.h -- the group-limited forward of the fused MoE router for
// rows of 32-expert groups on gfx950.
//
// Operation: fused_topk_with_score_function forward with group-limited
// routing ("[Common] Optimize fused router forward/backward kernels", NVIDIA
// TransformerEngine pull request 3012, "Hardening": topk divisible by
// group_topk); the per-token maths is stated in include/router.h.  This is
// the layout of the widely used router of 256 experts in 8 groups (4 groups
// kept, 8 experts chosen), and of E = 64..512 in groups of 32 in general.
//
// Layout: as the general forward (router_kernels.h): one token per LPT
// lanes (16 or 32), lane l holds NCH chunks of 4 consecutive elements,
// j = c*4*LPT + 4*l + u, and E == NCH*4*LPT exactly.  A group of 32 experts
// is then lanes [8s, 8s+8) of one chunk: group g = c*NS + s with NS = LPT/8
// groups per chunk, and each lane's four elements of a chunk share a group.
//
// Differences from the general kernel's group stage, which this kernel
// replaces for these shapes (same results bit for bit):
//  * the group geometry is a compile-time constant (no dispatch on it);
//  * the top-q lists are formed on the selection keys (the logit without a
//    bias, s + b with one), and a group's score is the fp32 sum of the
//    scores of its q largest keys, largest first -- the same values the
//    oracle sums, since the score is monotone in the logit and the scores
//    are recomputed with the forward's own formula; so the kept groups'
//    q-th largest keys bound the K-th key from below with or without a bias
//    and the pruned select always skips its sort of the lane maxima;
//  * a group's rank is counted from packed (score, ~group) words of every
//    group, read with lane shuffles (no LDS);
//  * the pruned select sorts 32-bit order keys first (indices only on a tie
//    at the K-th position).
#pragma once

#include <type_traits>

#include "router_kernels.h"

namespace rker {

// Group-limited forward for 32-expert groups.  Q: length of the per-group
// top lists (q <= Q); BIAS: an expert bias is given.
template <int LPT, int NCH, typename TIn, int SCORE, int Q, bool BIAS>
__global__ void __launch_bounds__(kBlock, NCH <= 2 ? 6 : 4) grouped_fwd_kernel(FwdParams p)
{
    constexpr int GPW = 64 / LPT;            // tokens per wave
    constexpr int TPB = kWaves * GPW;        // tokens per block
    constexpr int VPL = NCH * 4;
    constexpr int NS = LPT / 8;              // groups per chunk
    constexpr int G = NCH * NS;              // groups per row
    static_assert(LPT == 16 || LPT == 32, "two or four 8-lane groups per chunk");
    extern __shared__ uint64_t smem[];

    const int lane64 = lane_id();
    const int lane = lane64 & (LPT - 1);
    const int j_lane = 4 * lane;
    const int grp = lane64 / LPT;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint64_t *cand = smem + (wave * GPW + grp) * cand_slots(LPT);
    const int E = p.E;
    const uint32_t goff = (uint32_t)(grp * E);
    const int seg = lane >> 3;               // group slot within a chunk

    // The expert bias, shared by every token: copied once per block into
    // LDS after the candidate lists and read per token group (no registers
    // held across the loop).
    [[maybe_unused]] const float *bl = reinterpret_cast<const float *>(smem + TPB * cand_slots(LPT));
    if constexpr (BIAS) {
        float *bw = reinterpret_cast<float *>(smem + TPB * cand_slots(LPT));
        for (int j = (int)threadIdx.x; j < E; j += kBlock)
            bw[j] = p.bias[j];
        __syncthreads();
    }

    // Logits of token group tb (this wave's tokens of the block's group), as
    // loaded: RAW words per chunk (bf16: two 32-bit words of two values
    // each; fp32: four values).  Rows have no padding (E == NCH*4*LPT): a
    // masked load (a token past T) reads 0, and that token's outputs are
    // dropped.
    constexpr bool BF = sizeof(TIn) == 2;
    using raw_t = std::conditional_t<BF, uint32_t __attribute__((ext_vector_type(2))),
                                     uint32_t __attribute__((ext_vector_type(4)))>;
    auto load_x = [&](int64_t tb_, raw_t (&dst)[NCH]) {
        const int64_t t0_ = tb_ + wave * GPW;
        const int64_t left_ = p.T - t0_;
        const int nval_ = left_ <= 0 ? 0 : (left_ >= GPW ? GPW : (int)left_);
        const int64_t off_ = nval_ ? t0_ * (int64_t)E : 0;
        const rsrc_t r = make_rsrc(static_cast<const TIn *>(p.x) + off_,
                                   (uint32_t)(nval_ * E) * io<TIn>::kSize);
        const int off = grp < nval_ ? (int)((goff + (uint32_t)j_lane) * io<TIn>::kSize)
                                    : (int)kOOB;
#pragma unroll
        for (int c = 0; c < NCH; c++) {
            const int soff = (int)((uint32_t)jrel<LPT, true>(c, 0) * io<TIn>::kSize);
            if constexpr (BF)
                dst[c] = __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, kStream);
            else
                dst[c] = __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, kStream);
        }
    };
    auto unpack = [](const raw_t &w, float (&v)[4]) {
        if constexpr (BF) {
            v[0] = as_f(w[0] << 16);
            v[1] = as_f(w[0] & 0xFFFF0000u);
            v[2] = as_f(w[1] << 16);
            v[3] = as_f(w[1] & 0xFFFF0000u);
        } else {
            v[0] = as_f(w[0]);
            v[1] = as_f(w[1]);
            v[2] = as_f(w[2]);
            v[3] = as_f(w[3]);
        }
    };

    // Grid-stride over token groups, the next group's logits requested
    // before this group's work: with a grid sized to the resident waves
    // (the host's choice) every wave streams its loads behind its compute.
    const int64_t step = (int64_t)gridDim.x * TPB;
    int64_t tb = (int64_t)blockIdx.x * TPB;
    raw_t xn[NCH];
    load_x(tb, xn);
    for (; tb < p.T; tb += step) {
        const int64_t t0 = tb + wave * GPW;
        const int64_t left = p.T - t0;
        const int nval = left <= 0 ? 0 : (left >= GPW ? GPW : (int)left);
        const bool tok = grp < nval;
        const int64_t off0 = nval ? t0 * (int64_t)E : 0;
        const uint32_t nel = (uint32_t)(nval * E);

        float key[NCH][4];
#pragma unroll
        for (int c = 0; c < NCH; c++)
            unpack(xn[c], key[c]);
        if (tb + step < p.T)
            load_x(tb + step, xn);

        // ---- score function (as the general forward: the same values)
        float s[NCH][4];
        float mx = 0.0f, rz = 0.0f;
        if constexpr (SCORE == SCORE_SOFTMAX) {
            float m = -INFINITY;
#pragma unroll
            for (int c = 0; c < NCH; c++)
#pragma unroll
                for (int u = 0; u < 4; u++)
                    m = vmax(m, key[c][u]);
            mx = group_max<LPT>(m);
            mx = tok ? mx : 0.0f;
#pragma unroll
            for (int c = 0; c < NCH; c++)
#pragma unroll
                for (int u = 0; u < 4; u++)
                    s[c][u] = exp_split(key[c][u] - mx);
            const float z = group_sum<LPT>(tree_sum<VPL>(&s[0][0]));
            const float rz0 = 1.0f / z;
            rz = tok ? rz0 : 0.0f;
#pragma unroll
            for (int c = 0; c < NCH; c++)
#pragma unroll
                for (int u = 0; u < 4; u++)
                    s[c][u] *= rz;
        } else {
#pragma unroll
            for (int c = 0; c < NCH; c++)
#pragma unroll
                for (int u = 0; u < 4; u++)
                    s[c][u] = sigmoid_fast(key[c][u]);
        }
        // the score of one logit, bit for bit as above
        auto score_of = [&](float x) {
            if constexpr (SCORE == SCORE_SOFTMAX)
                return exp_split(x - mx) * rz;
            else
                return sigmoid_fast(x);
        };
        if constexpr (BIAS) {
#pragma unroll
            for (int c = 0; c < NCH; c++) {
                typedef float f4 __attribute__((ext_vector_type(4)));
                const f4 b = *reinterpret_cast<const f4 *>(bl + jrel<LPT, true>(c, 0) + j_lane);
#pragma unroll
                for (int u = 0; u < 4; u++)
                    key[c][u] = s[c][u] + b[u];
            }
        }

        // ---- the intermediate is final: store it now (overlaps the rest)
        const rsrc_t ri = make_rsrc(p.inter + off0, nel * 4u);
#pragma unroll
        for (int c = 0; c < NCH; c++)
            store_chunk<LPT, float, true>(ri, goff, c, j_lane, E, s[c]);

        // ---- group stage: every lane of a group gets the group's sorted
        // top-Q keys (merge steps with the lanes at distance 1, 2 and 4)
        uint64_t pk[NCH];    // (ord(score), ~group): larger = better group
        float tq[NCH];       // the group's q-th largest key
#pragma unroll
        for (int c = 0; c < NCH; c++) {
            float t[Q];
            topq_of4<Q>(key[c], t);
            topq_step<1, Q>(t);
            topq_step<2, Q>(t);
            topq_step<4, Q>(t);
            float h = BIAS ? t[0] : score_of(t[0]);
            float v = t[0];
#pragma unroll
            for (int i = 1; i < Q; i++) {
                if (p.q > i) {
                    h = h + (BIAS ? t[i] : score_of(t[i]));
                    v = t[i];
                }
            }
            tq[c] = v;
            const uint32_t g = (uint32_t)(c * NS + seg);
            pk[c] = ((uint64_t)ord_key(h + 0.0f) << 32) | (uint32_t)~g;
        }

        // rank of each of the lane's groups among the G groups: compare with
        // every chunk's groups in every segment (segment s ^ d of chunk c2
        // holds pk[c2] of that group on this lane after the shuffle)
        uint32_t rank[NCH];
#pragma unroll
        for (int c = 0; c < NCH; c++)
            rank[c] = 0;
#pragma unroll
        for (int c2 = 0; c2 < NCH; c2++) {
#pragma unroll
            for (int d = 0; d < NS; d++) {
                uint64_t o = pk[c2];
                if (d & 1)
                    o = partner_xor64<8>(o);
                if (d & 2)
                    o = partner_xor64<16>(o);
#pragma unroll
                for (int c = 0; c < NCH; c++) {
                    if (d == 0 && c2 == c)
                        continue;
                    rank[c] += o > pk[c] ? 1u : 0u;
                }
            }
        }
        // the K-th key is at least the smallest q-th key of the kept groups
        // (their q largest are Kg*q = K distinct experts); other groups'
        // experts do not compete
        float m = INFINITY;
#pragma unroll
        for (int c = 0; c < NCH; c++) {
            const bool kept = rank[c] < (uint32_t)p.Kg;
            m = kept ? vmin(m, tq[c]) : m;
#pragma unroll
            for (int u = 0; u < 4; u++)
                key[c][u] = kept ? key[c][u] : -INFINITY;
        }
        const float bound = as_f(group_allreduce_u<LPT>(as_u(m), [](uint32_t x, uint32_t y) {
            return as_u(vmin(as_f(x), as_f(y)));
        }));
        static_assert(G <= 16, "at most 16 groups");

        // ---- top-K among the kept groups
        const Thresh t = select_prune<LPT, NCH, false, true, true>(key, p.K, lane, j_lane, cand, true,
                                                              bound);
        // selection as 0/1 floats: the map bytes (one conversion per byte),
        // the renormalisation sum and the probs take them without selects
        const float tx = tok ? t.x : INFINITY;
        float mf[NCH][4];
        if (!wave_any(t.j != 0xFFFFFFFFu)) {
            // no tie straddles any threshold of the wave: one compare each
#pragma unroll
            for (int c = 0; c < NCH; c++)
#pragma unroll
                for (int u = 0; u < 4; u++)
                    mf[c][u] = key[c][u] >= tx ? 1.0f : 0.0f;
        } else {
            // equal keys at the threshold: up to expert j_t (bitwise
            // operators: no short-circuit branches per element)
            const int jt = t.j == 0xFFFFFFFFu ? 0x7FFFFFFF : (int)t.j - j_lane;
#pragma unroll
            for (int c = 0; c < NCH; c++)
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    const float k = key[c][u];
                    const int in = (int)(k > tx) | ((int)(k == tx) & (int)(jrel<LPT, true>(c, u) <= jt));
                    mf[c][u] = in ? 1.0f : 0.0f;
                }
        }
        float sm[NCH][4];    // s on the selected experts, +0 elsewhere (s >= 0)
#pragma unroll
        for (int c = 0; c < NCH; c++)
#pragma unroll
            for (int u = 0; u < 4; u++)
                sm[c][u] = s[c][u] * mf[c][u];

        // ---- weights and stores (as the general forward)
        const bool norm = p.renorm && (SCORE == SCORE_SOFTMAX || p.K > 1);
        float mult = p.scale;
        if (norm) {
            float part[NCH];
#pragma unroll
            for (int c = 0; c < NCH; c++)
                part[c] = (sm[c][0] + sm[c][1]) + (sm[c][2] + sm[c][3]);
            const float a = group_sum<LPT>(tree_sum<NCH>(part));
            const float mq = mult / a;
            mult = tok ? mq : 0.0f;
        }
        const rsrc_t ro = make_rsrc(static_cast<TIn *>(p.out) + off0, nel * io<TIn>::kSize);
        const rsrc_t rm = make_rsrc(p.map + off0, nel);
#pragma unroll
        for (int c = 0; c < NCH; c++) {
            float o[4];
            uint32_t w = 0;
#pragma unroll
            for (int u = 0; u < 4; u++) {
                // s * mult, and +0 (not -0) off the selection for any sign
                // of the scaling factor
                o[u] = fmaf(sm[c][u], mult, 0.0f);
                w = __builtin_amdgcn_cvt_pk_u8_f32(mf[c][u], u, w);
            }
            store_chunk<LPT, TIn, true>(ro, goff, c, j_lane, E, o);
            store_map_chunk<LPT, true>(rm, goff, c, j_lane, E, w);
        }
    }
}

}  // namespace rker
