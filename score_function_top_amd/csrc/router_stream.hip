// router_stream.hip -- plain data-movement kernels for the bandwidth
// references next to the router's measured bandwidth, with no arithmetic:
//   stream_kernel reads `read_bytes` and writes `write_bytes` with the
//     access style of the router kernels (16-byte buffer loads and stores
//     per lane, non-temporal), one 16-byte unit per thread, so a run at the
//     router's read:write mix gives the bandwidth this device reaches for
//     that mix;
//   row_stream_kernel moves the forward's bytes in the forward's own
//     pattern (one wave per row, the row loaded whole, then three stores
//     per chunk), which is what the forward can reach at best.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "router_io.h"
#include "router_params.h"

namespace rker {

namespace {

// Unit u (16 bytes): src unit u is read when u < nr, dst unit u written when
// u < nw; a written unit holds the unit read at u (or the unit index), so
// every load feeds a store and none is dead code.
__global__ __launch_bounds__(kBlock) void stream_kernel(const void *src, int64_t nr, void *dst,
                                                        int64_t nw)
{
    const int64_t n = nr > nw ? nr : nw;
    const int64_t step = (int64_t)gridDim.x * kBlock;
    for (int64_t u0 = (int64_t)blockIdx.x * kBlock; u0 < n; u0 += step) {
        // one buffer window of kBlock units per block and step: offsets
        // stay 32-bit; units past nr / nw fall outside and are dropped
        const int64_t rr = nr - u0 < kBlock ? (nr > u0 ? nr - u0 : 0) : kBlock;
        const int64_t ww = nw - u0 < kBlock ? (nw > u0 ? nw - u0 : 0) : kBlock;
        const rsrc_t rs = make_rsrc((const char *)src + (rr ? u0 * 16 : 0), (uint32_t)(rr * 16));
        const rsrc_t rd = make_rsrc((char *)dst + (ww ? u0 * 16 : 0), (uint32_t)(ww * 16));
        const uint32_t off = threadIdx.x * 16u;
        float v[4];
        io<float>::load4(rs, off, 0, v);
        if (u0 + (int64_t)threadIdx.x >= nr)
            v[0] = (float)(u0 + threadIdx.x);
        io<float>::store4(rd, off, v);
    }
}

// The forward's memory pattern with no arithmetic: one 64-lane wave per
// row of E = 256*NCH fp32 values, the whole row loaded (16 bytes per lane
// and chunk) before any store, then per chunk a 16-byte store to each of
// two E-float outputs and a 4-byte store to a one-byte-per-element output
// (the sign bits of the four values, so every load feeds a store).  NCH is
// a template constant so that the stores issue back to back, as in the
// forward (with a run-time chunk count every store waited for the one
// before it).
template <int NCH>
__global__ __launch_bounds__(kBlock) void row_stream_kernel(const float *x, float *a, float *b,
                                                            uint8_t *m, int64_t T)
{
    using u32x4 = __attribute__((ext_vector_type(4))) uint32_t;
    constexpr int E = NCH * 256;
    const int lane = threadIdx.x & 63;
    // the wave index in a scalar register: the row's buffer resources are
    // then wave-uniform (a per-lane index makes every access a loop over
    // the distinct resources)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t t = (int64_t)blockIdx.x * kWaves + wave;
    if (t >= T)
        return;
    const rsrc_t rx = make_rsrc(x + t * E, (uint32_t)E * 4u);
    const rsrc_t ra = make_rsrc(a + t * E, (uint32_t)E * 4u);
    const rsrc_t rb = make_rsrc(b + t * E, (uint32_t)E * 4u);
    const rsrc_t rm = make_rsrc(m + t * E, (uint32_t)E);
    u32x4 v[NCH];
#pragma unroll
    for (int c = 0; c < NCH; c++)
        v[c] = __builtin_amdgcn_raw_buffer_load_b128(rx, lane * 16, c * 1024, kStream);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < NCH; c++)
        __builtin_amdgcn_raw_buffer_store_b128(v[c], ra, lane * 16 + c * 1024, 0, kStream);
#pragma unroll
    for (int c = 0; c < NCH; c++) {
        __builtin_amdgcn_raw_buffer_store_b128(v[c], rb, lane * 16 + c * 1024, 0, kStream);
        const uint32_t w = (v[c][0] >> 31) | (v[c][1] >> 31) << 8 | (v[c][2] >> 31) << 16 |
                           (v[c][3] >> 31) << 24;
        __builtin_amdgcn_raw_buffer_store_b32(w, rm, lane * 4 + c * 256, 0, kStream);
    }
}

template <int... N>
hipError_t row_stream_pick(int nch, dim3 grid, const float *x, float *a, float *b, uint8_t *m,
                           int64_t T, hipStream_t stream)
{
    bool done = false;
    auto one = [&](auto c) {
        constexpr int C = decltype(c)::value;
        hipLaunchKernelGGL(row_stream_kernel<C>, grid, dim3(kBlock), 0, stream, x, a, b, m, T);
        return done = true;
    };
    ((nch == N && one(std::integral_constant<int, N>{})) || ...);
    return done ? hipGetLastError() : hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_row_stream(const float *x, float *a, float *b, uint8_t *m, int64_t T, int E,
                             hipStream_t stream)
{
    if (T == 0)
        return hipSuccess;
    const int64_t blocks = (T + kWaves - 1) / kWaves;
    return row_stream_pick<1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16>(
        E / 256, dim3((unsigned)blocks), x, a, b, m, T, stream);
}

hipError_t launch_stream(const void *src, int64_t read_bytes, void *dst, int64_t write_bytes,
                         hipStream_t stream)
{
    const int64_t nr = read_bytes / 16, nw = write_bytes / 16;
    const int64_t n = nr > nw ? nr : nw;
    if (n == 0)
        return hipSuccess;
    int64_t blocks = (n + kBlock - 1) / kBlock;
    if (blocks > 65536)
        blocks = 65536;
    hipLaunchKernelGGL(stream_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, stream, src, nr,
                       dst, nw);
    return hipGetLastError();
}

}  // namespace rker
