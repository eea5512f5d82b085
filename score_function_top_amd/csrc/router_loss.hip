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
// HBM.  They share one geometry (ColGeo): a lane owns consecutive columns
// (4 for the loss, 4 to 16 for the counts) for every row it visits, so its per-column sums and weights live in
// registers, and a wave reads or writes one contiguous row segment per
// step.  The fp64 loss is reduced across blocks through a workspace and a
// second one-block kernel in a fixed order, so it is the same bit for bit
// on every run; the integer counts use atomic adds, exact in any order, and
// the last block of each column stripe writes them out (one launch).
#include <hip/hip_runtime.h>

#include <mutex>
#include <type_traits>

#include "router_io.h"
#include "router_params.h"

namespace rker {

namespace {

struct LaneCols {
    int col0;      // first of the lane's columns (may be >= E: idle lane)
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

// The lane's CPL map bytes of one row as CPL/4 little-endian words (0 past
// E).  VW = access width: CPL (one load; E % CPL == 0), 8 (E % 8 == 0), 4
// (E % 4 == 0) or 1 (byte loads, any E); a masked access gets the offset
// kOOB and reads 0.
template <int CPL, int VW>
__device__ __forceinline__ void load_map_row(rsrc_t r, uint32_t off, int col0, int E,
                                             uint32_t (&w)[CPL / 4])
{
    constexpr int NW = CPL / 4;
    if constexpr (VW == 16) {
        static_assert(CPL == 16, "one 16-byte load per 16 columns");
        const auto t = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(col0 < E ? off : kOOB), 0,
                                                             kStream);
#pragma unroll
        for (int q = 0; q < 4; q++)
            w[q] = t[q];
    } else if constexpr (VW == 8) {
#pragma unroll
        for (int q = 0; q < NW / 2; q++) {
            const auto t = __builtin_amdgcn_raw_buffer_load_b64(
                r, (int)(col0 + 8 * q < E ? off + 8 * q : kOOB), 0, kStream);
            w[2 * q] = t[0];
            w[2 * q + 1] = t[1];
        }
    } else if constexpr (VW == 4) {
#pragma unroll
        for (int q = 0; q < NW; q++)
            w[q] = __builtin_amdgcn_raw_buffer_load_b32(
                r, (int)(col0 + 4 * q < E ? off + 4 * q : kOOB), 0, kStream);
    } else {
#pragma unroll
        for (int q = 0; q < NW; q++) {
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

// counts[i] = 0: the whole pass when there are no rows.
__global__ __launch_bounds__(kBlock) void zero_counts_kernel(int64_t *counts, int E)
{
    const int i = (int)(blockIdx.x * kBlock + threadIdx.x);
    if (i < E)
        counts[i] = 0;
}

constexpr int kCountThreads = kCountWaves * 64;

// Tokens per expert in one launch.  Block b counts its splits of the rows
// over the columns of its stripe: each lane owns CPL columns and counts its
// rows' bytes two per 32-bit word (SWAR, 16-bit fields), the loads of up to
// 16 rows issued before any is consumed (steps are a power of two: chunks
// of 16, 4 or 1 rows divide them); lanes store their counts to their
// wave's LDS region (lane l at CPL*l, which is row_lane*width + column in
// the stripe) and thread i sums column i over the waves and the rows of a
// wave step.  Column i's 64-bit word in `ws` then takes one device-scope
// atomic add of (1 << 32) + sum from every block of the stripe: the high
// half counts the contributions, the low half the routed tokens.  The add
// that brings the contributions to gsplit (the stripe's block count) is the
// column's last, so its thread writes the total to counts[] and clears the
// word: `ws` is zero again when the kernel ends, with no other ordering
// between blocks than the atomics on each word (one round trip per block;
// a ticket per stripe and a last-block pass cost three, 11.9 us against
// about 7 at T=8192, E=2304).  Integer sums are exact in any order.
template <int CPL, int VW>
__global__ __launch_bounds__(kCountThreads) void count_kernel(const uint8_t *map, ColGeo g,
                                                             int64_t *counts, uint64_t *ws)
{
    constexpr int NW = CPL / 4;
    constexpr int CH = VW == 1 ? 4 : kCountMaxSteps;  // most rows in flight per chunk
    constexpr int kRegion = 64 * CPL;                  // counts one wave holds
    __shared__ uint32_t region[kCountWaves * kRegion];
    const int stripe = (int)(blockIdx.x % (unsigned)g.nstripe);
    const int s0 = (int)(blockIdx.x / (unsigned)g.nstripe);
    const int w = wave_index();
    const LaneCols lc = lane_cols(g, stripe);

    uint32_t c[CPL];
#pragma unroll
    for (int u = 0; u < CPL; u++)
        c[u] = 0;
    for (int64_t sp = s0; sp < g.nsplit; sp += g.gsplit) {
        const rsrc_t r = split_rsrc(map, g, sp, 1);
        // bytes b0 and b2 of each word in `lo`, b1 and b3 in `hi`, one
        // 16-bit field each: at most kCountMaxSteps per field
        uint32_t lo[NW], hi[NW];
#pragma unroll
        for (int q = 0; q < NW; q++)
            lo[q] = hi[q] = 0;
        // rows of a split in chunks of N (a power of two, at most the steps),
        // every load of a chunk issued before any is consumed
        auto rows = [&](auto n) {
            constexpr int N = decltype(n)::value;
            for (int k0 = 0; k0 < g.steps; k0 += N) {
                uint32_t v[N][NW];
#pragma unroll
                for (int k = 0; k < N; k++)
                    load_map_row<CPL, VW>(
                        r,
                        (uint32_t)split_row(g, w, k0 + k, lc.row_lane) * (uint32_t)g.E +
                            (uint32_t)lc.col0,
                        lc.col0, g.E, v[k]);
#pragma unroll
                for (int k = 0; k < N; k++)
#pragma unroll
                    for (int q = 0; q < NW; q++) {
                        const uint32_t t = bytes_nonzero(v[k][q]);
                        lo[q] += t & 0x00010001u;
                        hi[q] += (t >> 8) & 0x00010001u;
                    }
            }
        };
        if (g.steps >= CH)
            rows(std::integral_constant<int, CH>{});
        else if (g.steps >= 4)
            rows(std::integral_constant<int, 4>{});
        else
            rows(std::integral_constant<int, 1>{});
#pragma unroll
        for (int q = 0; q < NW; q++) {
            c[4 * q + 0] += lo[q] & 0xFFFFu;
            c[4 * q + 1] += hi[q] & 0xFFFFu;
            c[4 * q + 2] += lo[q] >> 16;
            c[4 * q + 3] += hi[q] >> 16;
        }
    }
    uint32_t *mine = region + w * kRegion + lane_id() * CPL;
#pragma unroll
    for (int q = 0; q < NW; q++) {
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
        const int col = stripe * width + i;
        if (col >= g.E)
            continue;
        uint32_t a = 0;
        for (int ww = 0; ww < kCountWaves; ww++)
            for (int rl = 0; rl < rpw; rl++)
                a += region[ww * kRegion + rl * width + i];
        const uint64_t add = (1ull << 32) | a;
        const uint64_t old =
            __hip_atomic_fetch_add(ws + col, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((uint32_t)(old >> 32) == (uint32_t)g.gsplit - 1u) {
            counts[col] = (int64_t)((uint32_t)old + a);
            __hip_atomic_store(ws + col, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
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
                        uint64_t *ws, hipStream_t stream)
{
    if (g.gsplit == 0) {
        hipLaunchKernelGGL(zero_counts_kernel, dim3((g.E + kBlock - 1) / kBlock), dim3(kBlock), 0,
                           stream, counts, g.E);
        return hipGetLastError();
    }
    const dim3 grid(grid_of(g)), block(kCountThreads);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, block, 0, stream, map, g, counts, ws);
        return true;
    };
    const bool ok =
        g.cpl_log2 == 4 ? (vec == 16 ? go(count_kernel<16, 16>)
                           : vec == 8 ? go(count_kernel<16, 8>)
                           : vec == 4 ? go(count_kernel<16, 4>)
                                      : go(count_kernel<16, 1>))
        : g.cpl_log2 == 3 ? (vec == 8 ? go(count_kernel<8, 8>)
                             : vec == 4 ? go(count_kernel<8, 4>)
                                        : go(count_kernel<8, 1>))
        : g.cpl_log2 == 2 ? (vec == 4 ? go(count_kernel<4, 4>) : go(count_kernel<4, 1>))
                          : false;
    return ok ? hipGetLastError() : hipErrorInvalidValue;
}

// Device memory the library owns for router_aux_loss_fwd_noalloc: the loss
// kernel's per-block fp64 partial sums, for callers that cannot allocate.
// Every GPU the library runs on holds its own copy until the process ends;
// calls on one GPU share it (their contents need no clearing: every partial
// is written before it is read, in stream order), so calls that overlap on
// one GPU race.  Host code uses the per-device address hipGetSymbolAddress
// returns, never the array's name (a host-side stand-in).
static __device__ __align__(256) unsigned char scratch[kLossScratchBytes];

hipError_t loss_scratch(void **ptr)
{
    constexpr int kMaxDev = 64;
    static std::once_flag once[kMaxDev];
    static void *addr[kMaxDev];
    static hipError_t err[kMaxDev];
    int d = 0;
    const hipError_t e = hipGetDevice(&d);
    if (e != hipSuccess)
        return e;
    if (d < 0 || d >= kMaxDev)
        return hipErrorInvalidDevice;
    // looked up once per device, with that device current
    std::call_once(once[d], [&] { err[d] = hipGetSymbolAddress(&addr[d], HIP_SYMBOL(scratch)); });
    if (err[d] != hipSuccess)
        return err[d];
    *ptr = addr[d];
    return hipSuccess;
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
