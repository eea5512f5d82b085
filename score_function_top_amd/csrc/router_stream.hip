// router_stream.hip -- a plain streaming kernel for the bandwidth ceiling
// next to the router's measured bandwidth: it reads `read_bytes` and writes
// `write_bytes` with the access style of the router kernels (16-byte
// buffer loads and stores per lane, non-temporal), so a run at the
// router's read:write mix gives the bandwidth this device reaches for that
// mix with no arithmetic at all.
#include <hip/hip_runtime.h>

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

}  // namespace

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
