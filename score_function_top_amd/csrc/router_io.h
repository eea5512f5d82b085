// router_io.h -- global-memory access of the router kernels on gfx950:
// raw buffer resources and the per-element-type vector loads and stores.
#pragma once

#include "router_device.h"

namespace rker {

using namespace rdev;

// ------------------------------------------------------------ row I/O
//
// Global traffic goes through raw buffer resources: one descriptor per wave
// covering the rows of the wave's tokens (base and byte count in SGPRs) and
// a 32-bit per-lane byte offset.  Loads past the range read 0 and stores
// past it are dropped, which retires the tail tokens of the last wave and
// masked chunks without branches.

typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr uint32_t kOOB = 0x80000000u;  // byte offset outside every buffer

// Cache policy of every row access: non-temporal (the gfx94x/gfx950 "nt"
// bit).  Each byte is touched once, so streaming it past the caches keeps
// them from thrashing; measured on MI355X it lifts the backward from ~5.3
// to ~5.9 TB/s at E=2304.
constexpr int kStream = 2;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    // 0x00020000: raw 32-bit data format word for the gfx9 family
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                             (int)bytes, 0x00020000);
}

template <typename TIn> struct io;

template <> struct io<float> {
    static constexpr uint32_t kSize = 4;
    template <int POL = kStream>
    __device__ static void load4(rsrc_t r, uint32_t off, uint32_t soff, float (&v)[4])
    {
        auto t = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, (int)soff, POL);
        v[0] = as_f(t[0]); v[1] = as_f(t[1]); v[2] = as_f(t[2]); v[3] = as_f(t[3]);
    }
    template <int POL = kStream>
    __device__ static float load1(rsrc_t r, uint32_t off)
    {
        return as_f(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, POL));
    }
    __device__ static void store4(rsrc_t r, uint32_t off, const float (&v)[4])
    {
        __attribute__((ext_vector_type(4))) uint32_t t;
        t[0] = as_u(v[0]); t[1] = as_u(v[1]); t[2] = as_u(v[2]); t[3] = as_u(v[3]);
        __builtin_amdgcn_raw_buffer_store_b128(t, r, (int)off, 0, kStream);
    }
    __device__ static void store1(rsrc_t r, uint32_t off, float v)
    {
        __builtin_amdgcn_raw_buffer_store_b32(as_u(v), r, (int)off, 0, kStream);
    }
};

template <> struct io<uint16_t> {
    static constexpr uint32_t kSize = 2;
    template <int POL = kStream>
    __device__ static void load4(rsrc_t r, uint32_t off, uint32_t soff, float (&v)[4])
    {
        auto t = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, (int)soff, POL);
        v[0] = as_f(t[0] << 16); v[1] = as_f(t[0] & 0xFFFF0000u);
        v[2] = as_f(t[1] << 16); v[3] = as_f(t[1] & 0xFFFF0000u);
    }
    template <int POL = kStream>
    __device__ static float load1(rsrc_t r, uint32_t off)
    {
        return bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, POL));
    }
    __device__ static void store4(rsrc_t r, uint32_t off, const float (&v)[4])
    {
        __attribute__((ext_vector_type(2))) uint32_t t;
        t[0] = f32x2_to_bf16x2(v[0], v[1]);
        t[1] = f32x2_to_bf16x2(v[2], v[3]);
        __builtin_amdgcn_raw_buffer_store_b64(t, r, (int)off, 0, kStream);
    }
    __device__ static void store1(rsrc_t r, uint32_t off, float v)
    {
        __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), r, (int)off, 0, kStream);
    }
};

}  // namespace rker
