// router_stream.hip -- plain data-movement kernels for the bandwidth
// references next to the router's measured bandwidth, with no arithmetic:
//   stream_kernel reads `read_bytes` and writes `write_bytes` with the
//     access style of the router kernels (16-byte buffer loads and stores
//     per lane, non-temporal), 1, 2, 4 or 8 16-byte units per thread, so
//     the fastest of these runs at the router's read:write mix gives the
//     bandwidth this device reaches for that mix;
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
// every load feeds a store and none is dead code.  A thread moves U units
// per step (units i*kBlock + tid of its block's window, every load issued
// before any store): one unit per thread leaves a wave 1 KB in flight, too
// little for a read-heavy mix to reach the bandwidth the router kernels
// reach with a whole row in flight (T=8192, E=2304: read only 14.8 us at
// U=1, 12.1 at U=4; the 4:9 write-heavy mix is fastest at U=1).
template <int U>
__global__ __launch_bounds__(kBlock) void stream_kernel(const void *src, int64_t nr, void *dst,
                                                        int64_t nw)
{
    constexpr int64_t kSpan = (int64_t)kBlock * U;  // units per block and step
    const int64_t n = nr > nw ? nr : nw;
    const int64_t step = (int64_t)gridDim.x * kSpan;
    for (int64_t u0 = (int64_t)blockIdx.x * kSpan; u0 < n; u0 += step) {
        // one buffer window of kSpan units per block and step: offsets
        // stay 32-bit; units past nr / nw fall outside and are dropped
        const int64_t rr = nr - u0 < kSpan ? (nr > u0 ? nr - u0 : 0) : kSpan;
        const int64_t ww = nw - u0 < kSpan ? (nw > u0 ? nw - u0 : 0) : kSpan;
        const rsrc_t rs = make_rsrc((const char *)src + (rr ? u0 * 16 : 0), (uint32_t)(rr * 16));
        const rsrc_t rd = make_rsrc((char *)dst + (ww ? u0 * 16 : 0), (uint32_t)(ww * 16));
        float v[U][4];
#pragma unroll
        for (int i = 0; i < U; i++)
            io<float>::load4(rs, (uint32_t)(i * kBlock + (int)threadIdx.x) * 16u, 0, v[i]);
        __builtin_amdgcn_sched_barrier(0);  // every load in flight before any store
#pragma unroll
        for (int i = 0; i < U; i++) {
            const int64_t u = u0 + i * kBlock + (int64_t)threadIdx.x;
            if (u >= nr)
                v[i][0] = (float)u;
            io<float>::store4(rd, (uint32_t)(i * kBlock + (int)threadIdx.x) * 16u, v[i]);
        }
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
                         int units, hipStream_t stream)
{
    const int64_t nr = read_bytes / 16, nw = write_bytes / 16;
    const int64_t n = nr > nw ? nr : nw;
    if (n == 0)
        return hipSuccess;
    const int64_t span = (int64_t)kBlock * units;
    int64_t blocks = (n + span - 1) / span;
    if (blocks > 65536)
        blocks = 65536;
    const dim3 grid((unsigned)blocks), block(kBlock);
    switch (units) {
    case 1: hipLaunchKernelGGL(stream_kernel<1>, grid, block, 0, stream, src, nr, dst, nw); break;
    case 2: hipLaunchKernelGGL(stream_kernel<2>, grid, block, 0, stream, src, nr, dst, nw); break;
    case 4: hipLaunchKernelGGL(stream_kernel<4>, grid, block, 0, stream, src, nr, dst, nw); break;
    case 8: hipLaunchKernelGGL(stream_kernel<8>, grid, block, 0, stream, src, nr, dst, nw); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace rker
