// router_loss.hip -- the load-balancing aux loss over the aux scores on
// gfx950: tokens per expert from the routing map, the loss, and its
// gradient.
//
// The fused-router page ("[Common] Optimize fused router forward/backward
// kernels", NVIDIA TransformerEngine pull request 3012, "Files changed")
// names the aux-loss kernel that consumes the aux scores but not its
// formula; the loss implemented is the Switch-Transformer balancing loss
// extended to top-K routing,
//   L = coeff * E / (N^2 K) * sum_i n_i * sum_t scores[t,i],
// n_i = tokens routed to expert i (over the N tokens the counts cover),
// with dL/dscores[t,i] = coeff * E * n_i / (N^2 K).
//
// All three are column reductions or broadcasts over [T,E] and bound by
// HBM.  They share one geometry (ColGeo): a lane owns 4 consecutive columns
// for every row it visits, so its per-column sums and weights live in
// registers, and a wave reads or writes one contiguous row segment per
// step.  The fp64 loss is reduced across blocks through a workspace and a
// second one-block kernel in a fixed order, so it is the same bit for bit
// on every run; the integer counts use atomic adds, exact in any order.
#include <hip/hip_runtime.h>

#include "router_io.h"
#include "router_params.h"

namespace rker {

namespace {

struct LaneCols {
    int col0;      // first of the lane's 4 columns (may be >= E: idle lane)
    int row_lane;  // row of this lane within a wave step
};

__device__ __forceinline__ LaneCols lane_cols(const ColGeo &g, int stripe)
{
    const int lane = lane_id();
    return LaneCols{geo_col0(g, stripe, lane), geo_row_lane(g, lane)};
}

__device__ __forceinline__ int wave_index()
{
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

__device__ __forceinline__ int split_row(const ColGeo &g, int w, int k, int row_lane)
{
    return geo_split_row(g, w, k, row_lane);
}

// Buffer over the rows of split sp: loads past its last row read 0 and
// stores past it are dropped.
__device__ __forceinline__ rsrc_t split_rsrc(const void *base, const ColGeo &g, int64_t sp,
                                             uint32_t esize)
{
    const int64_t r0 = sp * g.rows_per_split;
    const int64_t left = g.T - r0;
    const int64_t rows = left < g.rows_per_split ? left : g.rows_per_split;
    return make_rsrc((const char *)base + r0 * g.E * esize, (uint32_t)(rows * g.E * esize));
}

// Fixed-order block sum of one double per thread (thread 0 gets it).
__device__ __forceinline__ double block_sum(double v, double *lds)
{
    lds[threadIdx.x] = v;
    __syncthreads();
#pragma unroll
    for (int h = kBlock / 2; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h)
            lds[threadIdx.x] += lds[threadIdx.x + h];
        __syncthreads();
    }
    return lds[0];
}

__device__ __forceinline__ void store_one_f32(float *p, float v)
{
    __builtin_amdgcn_raw_buffer_store_b32(as_u(v), make_rsrc(p, 4), 0, 0, 0);
}

// ------------------------------------------------------------ counts

// Bit 0 of each byte := OR of that byte's bits (a byte counts as routed
// when it is nonzero); other bits cleared.
__device__ __forceinline__ uint32_t bytes_nonzero(uint32_t w)
{
    w |= w >> 4;
    w |= w >> 2;
    w |= w >> 1;
    return w & 0x01010101u;
}

// The lane's 16 map bytes of one row as 4 little-endian words (0 past E).
// VW = access width: 16 (one 16-byte load; E % 16 == 0), 4 (four 4-byte
// loads; E % 4 == 0) or 1 (byte loads, any E).
template <int VW>
__device__ __forceinline__ void load_map16(rsrc_t r, uint32_t off, int col0, int E,
                                           uint32_t (&w)[4])
{
    if constexpr (VW == 16) {
        const auto t = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(col0 < E ? off : kOOB), 0,
                                                             kStream);
#pragma unroll
        for (int q = 0; q < 4; q++)
            w[q] = t[q];
    } else if constexpr (VW == 4) {
#pragma unroll
        for (int q = 0; q < 4; q++)
            w[q] = __builtin_amdgcn_raw_buffer_load_b32(
                r, (int)(col0 + 4 * q < E ? off + 4 * q : kOOB), 0, kStream);
    } else {
#pragma unroll
        for (int q = 0; q < 4; q++) {
            w[q] = 0;
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const int c = col0 + 4 * q + u;
                const uint32_t b = __builtin_amdgcn_raw_buffer_load_b8(
                    r, (int)(c < E ? off + 4 * q + u : kOOB), 0, kStream);
                w[q] |= b << (8 * u);
            }
        }
    }
}

// counts[i] = 0 (runs before count_kernel on the same stream).
__global__ __launch_bounds__(kBlock) void zero_counts_kernel(int64_t *counts, int E)
{
    const int i = (int)(blockIdx.x * kBlock + threadIdx.x);
    if (i < E)
        counts[i] = 0;
}

constexpr int kCountThreads = kCountWaves * 64;
constexpr int kCountRegion = 64 << kCountCpl;  // counts one wave holds (16 per lane)

// Adds block b's counts (its splits, the columns of its stripe) to
// counts[] with 64-bit atomic adds.  Integer addition is associative, so
// the totals do not depend on the order the blocks finish in.  Each lane
// owns 16 columns; a split's loads are issued in chunks of CH steps (all
// of them for 16-byte loads) before any is consumed.  Lanes then store
// their counts to their wave's LDS region (lane l at 16*l, which is
// row_lane*width + column-in-stripe), and thread i sums column i over the
// waves and rows of a wave step, so the atomics of a wave hit consecutive
// addresses.
template <int VW>
__global__ __launch_bounds__(kCountThreads) void count_kernel(const uint8_t *map, ColGeo g,
                                                             int64_t *counts)
{
    constexpr int CH = VW == 1 ? 4 : kCountSteps;
    __shared__ uint32_t region[kCountWaves * kCountRegion];
    const int stripe = (int)(blockIdx.x % (unsigned)g.nstripe);
    const int s0 = (int)(blockIdx.x / (unsigned)g.nstripe);
    const int w = wave_index();
    const LaneCols lc = lane_cols(g, stripe);

    uint32_t c[16];
#pragma unroll
    for (int u = 0; u < 16; u++)
        c[u] = 0;
    for (int64_t sp = s0; sp < g.nsplit; sp += g.gsplit) {
        const rsrc_t r = split_rsrc(map, g, sp, 1);
        // bytes b0 and b2 of each word in `lo`, b1 and b3 in `hi`, one
        // 16-bit field each: at most kCountSteps per field
        uint32_t lo[4] = {0, 0, 0, 0}, hi[4] = {0, 0, 0, 0};
        auto chunk = [&](int k0) {
            uint32_t v[CH][4];
#pragma unroll
            for (int k = 0; k < CH; k++)
                load_map16<VW>(r,
                               (uint32_t)split_row(g, w, k0 + k, lc.row_lane) * (uint32_t)g.E +
                                   (uint32_t)lc.col0,
                               lc.col0, g.E, v[k]);
#pragma unroll
            for (int k = 0; k < CH; k++)
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const uint32_t t = bytes_nonzero(v[k][q]);
                    lo[q] += t & 0x00010001u;
                    hi[q] += (t >> 8) & 0x00010001u;
                }
        };
        if constexpr (CH == kCountSteps) {
            chunk(0);
        } else {
#pragma unroll 1
            for (int k0 = 0; k0 < kCountSteps; k0 += CH)
                chunk(k0);
        }
#pragma unroll
        for (int q = 0; q < 4; q++) {
            c[4 * q + 0] += lo[q] & 0xFFFFu;
            c[4 * q + 1] += hi[q] & 0xFFFFu;
            c[4 * q + 2] += lo[q] >> 16;
            c[4 * q + 3] += hi[q] >> 16;
        }
    }
    uint32_t *mine = region + w * kCountRegion + lane_id() * 16;
#pragma unroll
    for (int q = 0; q < 4; q++) {
        __attribute__((ext_vector_type(4))) uint32_t t;
        t[0] = c[4 * q];
        t[1] = c[4 * q + 1];
        t[2] = c[4 * q + 2];
        t[3] = c[4 * q + 3];
        *(decltype(t) *)(mine + 4 * q) = t;
    }
    __syncthreads();
    const int width = geo_width(g);
    const int rpw = 1 << g.rpw_log2;
    for (int i = (int)threadIdx.x; i < width; i += kCountThreads) {
        uint32_t a = 0;
        for (int ww = 0; ww < kCountWaves; ww++)
            for (int rl = 0; rl < rpw; rl++)
                a += region[ww * kCountRegion + rl * width + i];
        const int col = stripe * width + i;
        if (col < g.E && a)
            atomicAdd((unsigned long long *)(counts + col), (unsigned long long)a);
    }
}

// ------------------------------------------------------------ loss

// Block partial sum_{its rows, its columns} n_i * scores[t,i] in fp64.
template <typename TIn, bool VEC>
__global__ __launch_bounds__(kBlock) void loss_kernel(const void *scores,
                                                      const int64_t *counts, ColGeo g,
                                                      double *ws)
{
    __shared__ double lds[kBlock];
    const int stripe = (int)(blockIdx.x % (unsigned)g.nstripe);
    const int s0 = (int)(blockIdx.x / (unsigned)g.nstripe);
    const int w = wave_index();
    const LaneCols lc = lane_cols(g, stripe);
    constexpr uint32_t sz = io<TIn>::kSize;

    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    for (int64_t sp = s0; sp < g.nsplit; sp += g.gsplit) {
        const rsrc_t r = split_rsrc(scores, g, sp, sz);
        float v[kLossSteps][4];
#pragma unroll
        for (int k = 0; k < kLossSteps; k++) {
            const uint32_t e =
                (uint32_t)split_row(g, w, k, lc.row_lane) * (uint32_t)g.E + (uint32_t)lc.col0;
            if constexpr (VEC) {
                io<TIn>::load4(r, lc.col0 < g.E ? e * sz : kOOB, 0, v[k]);
            } else {
#pragma unroll
                for (int u = 0; u < 4; u++)
                    v[k][u] = io<TIn>::load1(r, lc.col0 + u < g.E ? (e + u) * sz : kOOB);
            }
        }
#pragma unroll
        for (int k = 0; k < kLossSteps; k++)
#pragma unroll
            for (int u = 0; u < 4; u++)
                acc[u] += (double)v[k][u];
    }
    double part = 0.0;
#pragma unroll
    for (int u = 0; u < 4; u++)
        if (lc.col0 + u < g.E)
            part += acc[u] * (double)counts[lc.col0 + u];
    const double s = block_sum(part, lds);
    if (threadIdx.x == 0)
        ws[blockIdx.x] = s;
}

// loss = C * sum of the n block partials, in a fixed order.  Thread t sums
// partials t, t + 256, ... in chunks of 8 independent loads.
__global__ __launch_bounds__(kBlock) void loss_final_kernel(const double *ws, int n, double C,
                                                            float *loss)
{
    __shared__ double lds[kBlock];
    double s = 0.0;
    for (int i0 = 0; i0 < n; i0 += 8 * kBlock) {
        double v[8];
#pragma unroll
        for (int q = 0; q < 8; q++) {
            const int i = i0 + q * kBlock + (int)threadIdx.x;
            v[q] = i < n ? ws[i] : 0.0;
        }
#pragma unroll
        for (int q = 0; q < 8; q++)
            s += v[q];
    }
    s = block_sum(s, lds);
    if (threadIdx.x == 0)
        store_one_f32(loss, (float)(s * C));
}

// grad_scores[t,i] = grad_loss * C * n_i.
template <typename TOut, bool VEC>
__global__ __launch_bounds__(kBlock) void loss_bwd_kernel(const float *grad_loss,
                                                          const int64_t *counts, ColGeo g,
                                                          double C, void *dx)
{
    const int stripe = (int)(blockIdx.x % (unsigned)g.nstripe);
    const int s0 = (int)(blockIdx.x / (unsigned)g.nstripe);
    const int w = wave_index();
    const LaneCols lc = lane_cols(g, stripe);
    constexpr uint32_t sz = io<TOut>::kSize;

    const double gc = (double)grad_loss[0] * C;
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; u++)
        v[u] = lc.col0 + u < g.E ? (float)(gc * (double)counts[lc.col0 + u]) : 0.0f;

    for (int64_t sp = s0; sp < g.nsplit; sp += g.gsplit) {
        const rsrc_t r = split_rsrc(dx, g, sp, sz);
#pragma unroll
        for (int k = 0; k < kLossBwdSteps; k++) {
            const uint32_t e =
                (uint32_t)split_row(g, w, k, lc.row_lane) * (uint32_t)g.E + (uint32_t)lc.col0;
            if constexpr (VEC) {
                io<TOut>::store4(r, lc.col0 < g.E ? e * sz : kOOB, v);
            } else {
#pragma unroll
                for (int u = 0; u < 4; u++)
                    io<TOut>::store1(r, lc.col0 + u < g.E ? (e + u) * sz : kOOB, v[u]);
            }
        }
    }
}

unsigned grid_of(const ColGeo &g) { return (unsigned)g.gsplit * (unsigned)g.nstripe; }

}  // namespace

hipError_t launch_count(const uint8_t *map, int vec, const ColGeo &g, int64_t *counts,
                        hipStream_t stream)
{
    hipLaunchKernelGGL(zero_counts_kernel, dim3((g.E + kBlock - 1) / kBlock), dim3(kBlock), 0,
                       stream, counts, g.E);
    if (g.gsplit > 0) {
        const dim3 grid(grid_of(g)), block(kCountThreads);
        if (vec == 16)
            hipLaunchKernelGGL(count_kernel<16>, grid, block, 0, stream, map, g, counts);
        else if (vec == 4)
            hipLaunchKernelGGL(count_kernel<4>, grid, block, 0, stream, map, g, counts);
        else
            hipLaunchKernelGGL(count_kernel<1>, grid, block, 0, stream, map, g, counts);
    }
    return hipGetLastError();
}

hipError_t launch_loss(const void *scores, int dtype, bool vec, const ColGeo &g,
                       const int64_t *counts, double C, double *ws, float *loss,
                       hipStream_t stream)
{
    if (g.gsplit > 0) {
        const dim3 grid(grid_of(g)), block(kBlock);
        if (dtype == 0) {
            if (vec)
                hipLaunchKernelGGL((loss_kernel<float, true>), grid, block, 0, stream, scores,
                                   counts, g, ws);
            else
                hipLaunchKernelGGL((loss_kernel<float, false>), grid, block, 0, stream, scores,
                                   counts, g, ws);
        } else {
            if (vec)
                hipLaunchKernelGGL((loss_kernel<uint16_t, true>), grid, block, 0, stream,
                                   scores, counts, g, ws);
            else
                hipLaunchKernelGGL((loss_kernel<uint16_t, false>), grid, block, 0, stream,
                                   scores, counts, g, ws);
        }
    }
    hipLaunchKernelGGL(loss_final_kernel, dim3(1), dim3(kBlock), 0, stream, ws,
                       (int)grid_of(g), C, loss);
    return hipGetLastError();
}

hipError_t launch_loss_bwd(const float *grad_loss, const int64_t *counts, int dtype, bool vec,
                           const ColGeo &g, double C, void *grad_scores, hipStream_t stream)
{
    if (g.gsplit == 0)
        return hipSuccess;
    const dim3 grid(grid_of(g)), block(kBlock);
    if (dtype == 0) {
        if (vec)
            hipLaunchKernelGGL((loss_bwd_kernel<float, true>), grid, block, 0, stream, grad_loss,
                               counts, g, C, grad_scores);
        else
            hipLaunchKernelGGL((loss_bwd_kernel<float, false>), grid, block, 0, stream,
                               grad_loss, counts, g, C, grad_scores);
    } else {
        if (vec)
            hipLaunchKernelGGL((loss_bwd_kernel<uint16_t, true>), grid, block, 0, stream,
                               grad_loss, counts, g, C, grad_scores);
        else
            hipLaunchKernelGGL((loss_bwd_kernel<uint16_t, false>), grid, block, 0, stream,
                               grad_loss, counts, g, C, grad_scores);
    }
    return hipGetLastError();
}

}  // namespace rker
