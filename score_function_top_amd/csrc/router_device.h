// router_device.h -- gfx950 (CDNA4) device building blocks of the fused MoE
// router kernels: lane-group shuffles, reductions, scans and sorts built on
// DPP and the gfx950 permlane swaps, orderable selection keys and bf16
// conversion.
//
// A "lane group" is LPT consecutive lanes of a 64-wide wavefront (LPT = 16,
// 32 or 64) that together hold one token's row of E values.  Every helper
// here works inside each group independently and never reads a lane of
// another group, so a wave processes 64/LPT tokens side by side.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rdev {

// ---------------------------------------------------------------- lanes

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// DPP control words (gfx9 family encoding).
enum : int {
    kQpXor1 = 0xB1,       // quad_perm [1,0,3,2]: lane ^ 1
    kQpXor2 = 0x4E,       // quad_perm [2,3,0,1]: lane ^ 2
    kQpXor3 = 0x1B,       // quad_perm [3,2,1,0]: lane ^ 3
    kRowShr1 = 0x111,     // row_shr:n = 0x110 + n
    kRowShr2 = 0x112,
    kRowShr4 = 0x114,
    kRowShr8 = 0x118,
    kRowRor8 = 0x128,     // row_ror:8: lane ^ 8 inside a 16-lane row
    kRowMirror = 0x140,   // lane ^ 15 inside a row
    kRowHalfMirror = 0x141,  // lane ^ 7 inside an 8-lane half row
    kRowBcast15 = 0x142,  // lane 15 of each row feeds the next row
    kRowBcast31 = 0x143,  // lane 31 feeds rows 2 and 3
};

// Lane permutation inside 16-lane rows; every source lane is valid for the
// controls used here, so no "old" value is needed.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

// Value held by lane (lane ^ J) of the same group; J < LPT.
template <int J>
__device__ __forceinline__ uint32_t shfl_xor(uint32_t v)
{
    static_assert(J == 1 || J == 2 || J == 4 || J == 8 || J == 16 || J == 32,
                  "power-of-two lane distance below 64");
    if constexpr (J == 1) {
        return dpp_mov<kQpXor1>(v);
    } else if constexpr (J == 2) {
        return dpp_mov<kQpXor2>(v);
    } else if constexpr (J == 4) {
        // (lane ^ 7) ^ 3 == lane ^ 4
        return dpp_mov<kQpXor3>(dpp_mov<kRowHalfMirror>(v));
    } else if constexpr (J == 8) {
        return dpp_mov<kRowRor8>(v);
    } else if constexpr (J == 16) {
        // permlane16_swap(v, v) returns {even rows copied to both rows of a
        // pair, odd rows copied to both}; the partner of an odd row is the
        // even row and vice versa.
        auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (lane_id() & 16) ? r[0] : r[1];
    } else {
        auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (lane_id() & 32) ? r[0] : r[1];
    }
}

// Value held by lane (lane ^ (K-1)) of the same group: the mirror image
// inside each block of K lanes.
template <int K>
__device__ __forceinline__ uint32_t shfl_mirror(uint32_t v)
{
    if constexpr (K == 2) {
        return dpp_mov<kQpXor1>(v);
    } else if constexpr (K == 4) {
        return dpp_mov<kQpXor3>(v);
    } else if constexpr (K == 8) {
        return dpp_mov<kRowHalfMirror>(v);
    } else if constexpr (K == 16) {
        return dpp_mov<kRowMirror>(v);
    } else if constexpr (K == 32) {
        return shfl_xor<16>(dpp_mov<kRowMirror>(v));
    } else {
        static_assert(K == 64, "block of 2..64 lanes");
        return shfl_xor<32>(shfl_xor<16>(dpp_mov<kRowMirror>(v)));
    }
}

__device__ __forceinline__ float as_f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __float_as_uint(f); }

// ------------------------------------------------------------ reductions

// All-reduce over the LPT lanes of each group with a commutative,
// associative op; every lane of the group ends with identical bits.
// Steps: lane^1, lane^2 (quad_perm), then the half-row and row mirrors
// (after the first two steps every lane of a quad holds the same value, so
// a mirror pairs each quad with the other one), then the row swaps.
template <int LPT, typename Op>
__device__ __forceinline__ uint32_t group_allreduce_u(uint32_t v, Op op)
{
    v = op(v, dpp_mov<kQpXor1>(v));
    v = op(v, dpp_mov<kQpXor2>(v));
    v = op(v, dpp_mov<kRowHalfMirror>(v));
    v = op(v, dpp_mov<kRowMirror>(v));
    if constexpr (LPT >= 32) {
        auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        v = op(r[0], r[1]);
    }
    if constexpr (LPT >= 64) {
        auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        v = op(r[0], r[1]);
    }
    return v;
}

template <int LPT>
__device__ __forceinline__ float group_sum(float v)
{
    return as_f(group_allreduce_u<LPT>(as_u(v), [](uint32_t a, uint32_t b) {
        return as_u(as_f(a) + as_f(b));
    }));
}

template <int LPT>
__device__ __forceinline__ float group_max(float v)
{
    return as_f(group_allreduce_u<LPT>(as_u(v), [](uint32_t a, uint32_t b) {
        return as_u(fmaxf(as_f(a), as_f(b)));
    }));
}

template <int LPT>
__device__ __forceinline__ uint32_t group_sum_u32(uint32_t v)
{
    return group_allreduce_u<LPT>(v, [](uint32_t a, uint32_t b) { return a + b; });
}

// Two fp32 sums reduced side by side.
template <int LPT>
__device__ __forceinline__ void group_sum2(float &a, float &b)
{
    a = group_sum<LPT>(a);
    b = group_sum<LPT>(b);
}

// Largest 64-bit value over the group.
template <int LPT>
__device__ __forceinline__ uint64_t group_max_u64(uint64_t v)
{
    auto step = [](uint64_t x, uint32_t ph, uint32_t pl) {
        uint64_t p = ((uint64_t)ph << 32) | pl;
        return p > x ? p : x;
    };
    uint32_t h = (uint32_t)(v >> 32), l = (uint32_t)v;
    v = step(v, dpp_mov<kQpXor1>(h), dpp_mov<kQpXor1>(l));
    h = (uint32_t)(v >> 32); l = (uint32_t)v;
    v = step(v, dpp_mov<kQpXor2>(h), dpp_mov<kQpXor2>(l));
    h = (uint32_t)(v >> 32); l = (uint32_t)v;
    v = step(v, dpp_mov<kRowHalfMirror>(h), dpp_mov<kRowHalfMirror>(l));
    h = (uint32_t)(v >> 32); l = (uint32_t)v;
    v = step(v, dpp_mov<kRowMirror>(h), dpp_mov<kRowMirror>(l));
    if constexpr (LPT >= 32) {
        h = (uint32_t)(v >> 32); l = (uint32_t)v;
        v = step(v, shfl_xor<16>(h), shfl_xor<16>(l));
    }
    if constexpr (LPT >= 64) {
        h = (uint32_t)(v >> 32); l = (uint32_t)v;
        v = step(v, shfl_xor<32>(h), shfl_xor<32>(l));
    }
    return v;
}

// Inclusive prefix sum over the lanes of each group (Hillis-Steele inside
// 16-lane rows, then the row broadcasts carry row totals forward).
template <int LPT>
__device__ __forceinline__ uint32_t group_incl_scan(uint32_t v)
{
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kRowShr1, 0xF, 0xF, true);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kRowShr2, 0xF, 0xF, true);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kRowShr4, 0xF, 0xF, true);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kRowShr8, 0xF, 0xF, true);
    if constexpr (LPT >= 32)
        v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kRowBcast15, 0xA, 0xF, false);
    if constexpr (LPT >= 64)
        v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kRowBcast31, 0xC, 0xF, false);
    return v;
}

// Value of lane `src` (0 <= src < LPT, equal on every lane of a group) of
// the caller's group.
template <int LPT>
__device__ __forceinline__ uint32_t group_bcast(uint32_t v, int src)
{
    if constexpr (LPT == 64) {
        return (uint32_t)__builtin_amdgcn_readlane((int)v, src);
    } else {
        int base = lane_id() & ~(LPT - 1);
        return (uint32_t)__builtin_amdgcn_ds_bpermute((base + src) << 2, (int)v);
    }
}

template <int LPT>
__device__ __forceinline__ uint64_t group_bcast64(uint64_t v, int src)
{
    uint32_t h = group_bcast<LPT>((uint32_t)(v >> 32), src);
    uint32_t l = group_bcast<LPT>((uint32_t)v, src);
    return ((uint64_t)h << 32) | l;
}

// True on every lane when `pred` holds on any active lane of the wave.
__device__ __forceinline__ bool wave_any(bool pred)
{
    return __builtin_amdgcn_ballot_w64(pred) != 0;
}

// ----------------------------------------------------------------- sorts
//
// Bitonic sort of one value per lane, descending across the group (lane 0
// holds the largest).  Merge stages use the mirror form: within each block
// of K lanes, lane i meets lane i ^ (K-1), then the half-cleaners meet
// lane ^ J for J = K/4 .. 1; the lower lane of each pair keeps the larger.

template <int J>
__device__ __forceinline__ uint64_t partner_xor64(uint64_t v)
{
    uint32_t h = shfl_xor<J>((uint32_t)(v >> 32));
    uint32_t l = shfl_xor<J>((uint32_t)v);
    return ((uint64_t)h << 32) | l;
}

template <int K>
__device__ __forceinline__ uint64_t partner_mirror64(uint64_t v)
{
    uint32_t h = shfl_mirror<K>((uint32_t)(v >> 32));
    uint32_t l = shfl_mirror<K>((uint32_t)v);
    return ((uint64_t)h << 32) | l;
}

// Compare-exchange: the lower lane of a pair keeps the larger value, the
// upper lane the smaller; i.e. take the partner's value when it is larger
// exactly on the lower lane.
__device__ __forceinline__ uint64_t keep(uint64_t mine, uint64_t other, bool lower)
{
    return ((other > mine) == lower) ? other : mine;
}

__device__ __forceinline__ uint32_t keep32(uint32_t mine, uint32_t other, bool lower)
{
    return ((other > mine) == lower) ? other : mine;
}

template <int J>
__device__ __forceinline__ uint64_t cleaners64(uint64_t v)
{
    if constexpr (J >= 1) {
        v = keep(v, partner_xor64<J>(v), (lane_id() & J) == 0);
        return cleaners64<J / 2>(v);
    } else {
        return v;
    }
}

template <int J>
__device__ __forceinline__ uint32_t cleaners32(uint32_t v)
{
    if constexpr (J >= 1) {
        v = keep32(v, shfl_xor<J>(v), (lane_id() & J) == 0);
        return cleaners32<J / 2>(v);
    } else {
        return v;
    }
}

template <int LPT, int K = 2>
__device__ __forceinline__ uint64_t sort_desc64(uint64_t v)
{
    if constexpr (K <= LPT) {
        v = keep(v, partner_mirror64<K>(v), (lane_id() & (K / 2)) == 0);
        v = cleaners64<K / 4>(v);
        return sort_desc64<LPT, K * 2>(v);
    } else {
        return v;
    }
}

template <int LPT, int K = 2>
__device__ __forceinline__ uint32_t sort_desc32(uint32_t v)
{
    if constexpr (K <= LPT) {
        v = keep32(v, shfl_mirror<K>(v), (lane_id() & (K / 2)) == 0);
        v = cleaners32<K / 4>(v);
        return sort_desc32<LPT, K * 2>(v);
    } else {
        return v;
    }
}

// Sort of 2*LPT values, two per lane: logical position e*LPT + lane holds
// v[e].  Each half is sorted, then the halves merge (mirror step across
// halves, then half-cleaners inside each half).
template <int LPT>
__device__ __forceinline__ void sort_desc64x2(uint64_t &v0, uint64_t &v1)
{
    v0 = sort_desc64<LPT>(v0);
    v1 = sort_desc64<LPT>(v1);
    uint64_t p0 = partner_mirror64<LPT>(v1);  // partner of (0, i) is (1, i^(LPT-1))
    uint64_t p1 = partner_mirror64<LPT>(v0);
    uint64_t n0 = v0 > p0 ? v0 : p0;
    uint64_t n1 = v1 > p1 ? p1 : v1;
    v0 = cleaners64<LPT / 2>(n0);
    v1 = cleaners64<LPT / 2>(n1);
}

// The same for 32-bit values.
template <int LPT>
__device__ __forceinline__ void sort_desc32x2(uint32_t &v0, uint32_t &v1)
{
    v0 = sort_desc32<LPT>(v0);
    v1 = sort_desc32<LPT>(v1);
    const uint32_t p0 = shfl_mirror<LPT>(v1);
    const uint32_t p1 = shfl_mirror<LPT>(v0);
    const uint32_t n0 = v0 > p0 ? v0 : p0;
    const uint32_t n1 = v1 > p1 ? p1 : v1;
    v0 = cleaners32<LPT / 2>(n0);
    v1 = cleaners32<LPT / 2>(n1);
}

// ------------------------------------------------------------ keys, bf16

// Monotone map of a finite float to an unsigned key: a < b  <=>  key(a) <
// key(b), and -0.0 < +0.0.  Every finite float maps above 0x007FFFFF, so 0
// is free to mark "not a candidate".
__device__ __forceinline__ uint32_t ord_key(float f)
{
    uint32_t u = as_u(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float ord_key_inv(uint32_t k)
{
    return as_f((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// ----------------------------------------------------------- exp, sigmoid

// e^y for y <= 88 in ~2 ulp: 2^(y log2 e) on the hardware exp2, with the
// product y*log2(e) carried in two parts (the second, from an FMA, holds the
// rounding error of the first and the tail of the constant) and folded back
// by 2^t ~ 1 + t ln 2.  y below -200 (padding: -inf) gives exactly 0.
// The lower clamp is an IEEE maximum (one instruction; fmaxf would first
// canonicalise its input): the same value for every non-NaN y.
__device__ __forceinline__ float exp_split(float y)
{
    y = __builtin_elementwise_maximum(y, -200.0f);
    const float L = 1.44269502162933349609375f;       // log2(e) rounded to fp32
    const float Llo = 1.925963033500011079e-8f;       // log2(e) - L
    const float th = y * L;
    const float tl = fmaf(y, Llo, fmaf(y, L, -th));
    const float e = __builtin_amdgcn_exp2f(th);
    return fmaf(e, tl * 0.693147180559945309f, e);
}

// Logistic sigmoid 1 / (1 + e^-x) with the hardware reciprocal (~3 ulp);
// for x < -88 the result is below 1e-38 instead of the exact tiny value.
// The exponent -x is clamped to [-200, 88] by one median-of-three (the two
// clamps of exp_split's domain in one instruction; the same value).
__device__ __forceinline__ float sigmoid_fast(float x)
{
    const float y = __builtin_amdgcn_fmed3f(-x, -200.0f, 88.0f);
    const float L = 1.44269502162933349609375f;
    const float Llo = 1.925963033500011079e-8f;
    const float th = y * L;
    const float tl = fmaf(y, Llo, fmaf(y, L, -th));
    const float e = __builtin_amdgcn_exp2f(th);
    return __builtin_amdgcn_rcpf(1.0f + fmaf(e, tl * 0.693147180559945309f, e));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b)
{
    return as_f((uint32_t)b << 16);
}

// Two fp32 values to a packed pair of bf16 (low half from `lo`), rounded
// to nearest even by the gfx950 packed conversion (v_cvt_pk_bf16_f32: one
// instruction for two values, against four integer operations each for
// the rounding done by hand).
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    return (uint16_t)f32x2_to_bf16x2(f, 0.0f);
}

}  // namespace rdev
