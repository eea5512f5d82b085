// router_grid.h -- grid size of a router kernel launch: one block per token
// group (the default), or the occupancy-sized persistent grid: the blocks
// a compute unit keeps resident for that kernel
// (hipOccupancyMaxActiveBlocksPerMultiprocessor) times the compute units,
// with the kernels' grid-stride loops covering the remaining tokens.
// Internal to the library; host code of the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <mutex>

#include "router_params.h"

namespace rker {

// Resident blocks of kernel KERN on the current device for blocks of
// `threads` threads and `smem` bytes of dynamic LDS (times the compute
// units); 0 when the device cannot be queried.  Cached per device, LDS size
// and block size.
template <auto KERN>
unsigned resident_blocks(size_t smem, unsigned threads)
{
    constexpr int kMaxDev = 64, kSlots = 8;
    struct Entry {
        size_t smem;
        unsigned threads;
        unsigned blocks;
    };
    static std::mutex mu;
    static Entry cache[kMaxDev][kSlots];
    static int used[kMaxDev];
    int d = 0;
    if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= kMaxDev)
        return 0;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used[d]; i++)
        if (cache[d][i].smem == smem && cache[d][i].threads == threads)
            return cache[d][i].blocks;
    int occ = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, KERN, (int)threads, smem) !=
            hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, d) != hipSuccess)
        return 0;
    const unsigned blocks = (unsigned)(occ > 0 ? occ : 1) * (unsigned)cus;
    if (used[d] < kSlots)
        cache[d][used[d]++] = Entry{smem, threads, blocks};
    return blocks;
}

// The grid of a launch of KERN: l.grid (one block per token group), or in
// the persistent mode at most the resident blocks.
template <auto KERN>
unsigned launch_grid(const Launch &l)
{
    if (!l.persistent)
        return l.grid;
    const unsigned cap = resident_blocks<KERN>(l.smem, l.threads);
    return cap > 0 && l.grid > cap ? cap : l.grid;
}

}  // namespace rker
