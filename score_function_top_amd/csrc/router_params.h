// router_params.h -- launch parameters shared by the router kernels and
// the host code of the C ABI.  Internal to the library; plain C++ (no
// device code), so host-only translation units can include it.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace rker {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;

enum { SEL_ARGMAX = 0, SEL_PRUNE = 1, SEL_BITS = 2 };
enum { SCORE_SOFTMAX = 0, SCORE_SIGMOID = 1 };
// Group stage of the forward: none, LDS scratch (any group size), or
// registers (groups of 4*L experts, L a power of two up to the lane width,
// so each lane's four elements of a chunk share one group).
enum { GROUP_NONE = 0, GROUP_LDS = 1, GROUP_REG = 2 };

// Register group stage: chunk counts it is built for, and the group slots
// (chunks times groups per chunk) it holds per token: 16 up to two chunks,
// 8 from three on (16 slots there push the prune kernels past 128 VGPRs).
constexpr int kGroupRegMaxNch = 4;

// Whether the pruned selection of a forward kernel takes LPT < K <= 2*LPT
// (the bound from each lane's two largest keys): without groups and with
// fewer than 64 lanes per token.  The host picks the layout accordingly.
constexpr bool prune_top2(int lpt, int gm) { return gm == GROUP_NONE && lpt < 64; }
constexpr int group_reg_slots(int nch) { return nch >= 3 ? 8 : 16; }
// Built (lanes per token LPT, chunks NCH, log2 of lanes per group LG):
// L = 2^LG <= LPT and NCH * LPT / L <= group_reg_slots(NCH).
constexpr bool group_reg_ok(int lpt, int nch, int lg)
{
    return nch <= kGroupRegMaxNch && lg >= 0 && (1 << lg) <= lpt &&
           nch * (lpt >> lg) <= group_reg_slots(nch);
}

struct FwdParams {
    const void *x;        // logits [T,E], TIn
    void *out;            // probs or aux scores [T,E], TIn
    uint8_t *map;         // [T,E]
    float *inter;         // [T,E]
    const float *bias;    // [E] or nullptr
    int64_t T;
    int E;
    int K;
    int sel;              // SEL_*
    int renorm;           // topk: renormalise over the selected experts;
                          // aux sigmoid: normalise over all experts
    int aux;              // 1: aux scores (no bias, no groups)
    int G;                // groups (0 = none)
    int Kg;               // groups kept
    int q;                // K / Kg
    int P;                // E / G (GROUP_REG: 4 * 2^k for 2^k lanes per group)
    float scale;          // scaling factor (topk)
};

struct BwdParams {
    const void *g;        // grad [T,E], TIn
    const float *s;       // intermediate [T,E]
    const uint8_t *m;     // routing map [T,E] or nullptr (aux: all routed)
    void *dx;             // grad_logits [T,E], TIn
    int64_t T;
    int E;
    int K;
    int renorm;
    float scale;
};

// LDS per token group: cand_slots u64 candidate slots; the LDS group stage
// adds group_scratch_floats floats.
constexpr int cand_slots(int lpt) { return 3 * lpt; }
// Workgroup LDS the forward kernels may use: gfx950 gives a workgroup up
// to 160 KB.  With the LDS group stage at 64 lanes per token that bounds
// E + G by 9792 (6144 bytes of candidates plus 16 (E + G + 64)), above
// every shape within the other limits (E <= 4096, G <= 64: 72640 bytes).
constexpr size_t kFwdLdsBytes = 163840;
constexpr int group_scratch_floats(int E, int G, int lpt)
{
    return E + G + lpt;
}

struct Launch {
    unsigned grid;       // one block per token group
    size_t smem;
    hipStream_t stream;
    bool persistent;     // cap the grid at the kernel's resident blocks
    unsigned threads = kBlock;
};

// Waves per block of a forward kernel.  The pruned forwards of 64-lane rows
// of 6..12 chunks (1024 < E <= 3072 on the vector path) run one wave (one
// token) per block: their waves fit only 2 per SIMD, and with single-wave
// blocks the dispatcher refills a slot as soon as its token is done instead
// of when the block's slowest of four is (T=8192: E=2304, K=36 45.5 ->
// 44.3 us; E=1536, K=8 30.0 -> 29.3 us; E=3072, K=8 59.2 -> 56.5 us).  Every
// other forward keeps 4 waves: measured on the same machine, 1-wave blocks
// made the 16- and 32-lane kernels slower (E=256 and E=512 forwards by 6
// and 10%), and the 3- and 16-chunk rows and the argmax path (K=1 at
// E=2304) by 1-3%; 2-wave blocks gave half the gain at E=2304.
constexpr int fwd_waves(int lpt, int nch, int gm, int sel, bool vec)
{
    return lpt == 64 && nch >= 6 && nch <= 12 && gm == GROUP_NONE && sel != SEL_ARGMAX && vec
               ? 1
               : kWaves;
}

// Column-stripe geometry of the aux-loss kernels (tokens per expert, the
// loss and its gradient).  Lane l of a wave owns CPL = 1 << cpl_log2
// consecutive columns, col0 = (stripe*LPR + l % LPR) * CPL, for every row it
// visits, so per-column sums stay in registers; LPR (lanes per row) is the
// smallest power of two with CPL*LPR >= E, at most 64, and a wave step
// covers RPW = 64/LPR rows.  A block of `waves` waves covers one stripe of
// CPL*LPR columns and a split of rows_per_split = waves*steps*RPW rows;
// block b takes stripe b % nstripe and splits b / nstripe,
// b / nstripe + gsplit, ...  gsplit is capped so the per-block partial
// results stay small.  Everything depends on (T, E) only, so the order of
// every sum is fixed.
struct ColGeo {
    int64_t T;
    int E;
    int waves;
    int cpl_log2;
    int lpr_log2;
    int rpw_log2;
    int steps;
    int rows_per_split;
    int nstripe;
    int64_t nsplit;
    int gsplit;
};

inline ColGeo col_geo(int64_t T, int E, int waves, int cpl_log2, int steps, int max_blocks)
{
    ColGeo g{};
    g.T = T;
    g.E = E;
    g.waves = waves;
    g.cpl_log2 = cpl_log2;
    int lpr_log2 = 0;
    while (lpr_log2 < 6 && (1 << (cpl_log2 + lpr_log2)) < E)
        lpr_log2++;
    g.lpr_log2 = lpr_log2;
    g.rpw_log2 = 6 - lpr_log2;
    g.steps = steps;
    g.rows_per_split = waves * steps << g.rpw_log2;
    const int width = 1 << (cpl_log2 + lpr_log2);
    g.nstripe = (E + width - 1) / width;
    g.nsplit = (T + g.rows_per_split - 1) / g.rows_per_split;
    int64_t cap = max_blocks / g.nstripe;
    if (cap < 1)
        cap = 1;
    g.gsplit = (int)(g.nsplit < cap ? g.nsplit : cap);
    return g;
}

// Index maps of the geometry, shared by the kernels and the host-side
// coverage check.  geo_width: columns per stripe; geo_col0: first of the
// columns lane `lane` owns in `stripe`; geo_row_lane: the lane's row within
// a wave step; geo_split_row: row (relative to its split) of step k of wave
// w for that lane.
constexpr int geo_width(const ColGeo &g) { return 1 << (g.cpl_log2 + g.lpr_log2); }
constexpr int geo_col0(const ColGeo &g, int stripe, int lane)
{
    return ((stripe << g.lpr_log2) + (lane & ((1 << g.lpr_log2) - 1))) << g.cpl_log2;
}
constexpr int geo_row_lane(const ColGeo &g, int lane) { return lane >> g.lpr_log2; }
constexpr int geo_split_row(const ColGeo &g, int w, int k, int row_lane)
{
    return ((w + g.waves * k) << g.rpw_log2) + row_lane;
}

// Count kernel: 8 waves; CPL map bytes per lane and row with CPL the
// largest of 16, 8 and 4 whose stripes cover E with at most 5% idle columns
// (else the one that wastes least).  Each column's total takes one atomic
// per row split, and the atomics on one word queue behind each other when
// the blocks finish together (about 20 ns each on MI355X: 512 of them made
// the T=8192, E=512 count 15 us), so at most kCountMaxSplits splits share a
// column; row steps per split are halved from 16 (down to 1) while the grid
// has fewer than kCountMinBlocks blocks and the splits stay within that
// cap, and blocks loop over the splits beyond it.  Loss kernels: 4 waves,
// 4 elements per lane and row.
constexpr int kCountWaves = 8;
constexpr int kCountMaxSteps = 16;    // row steps per wave and split (map)
constexpr int kCountMinBlocks = 512;
constexpr int kCountMaxBlocks = 2048;
constexpr int kCountMaxSplits = 64;   // row splits (atomics) per column
constexpr int kLossWaves = kWaves;
constexpr int kLossCpl = 2;           // log2 of 4 columns per lane
constexpr int kLossSteps = 16;        // row steps per wave and split (scores)
constexpr int kLossMaxBlocks = 4096;

inline int count_cpl_log2(int E)
{
    int best = 4;
    double best_u = -1.0;
    for (int l = 4; l >= 2; l--) {
        const ColGeo g = col_geo(1, E, kCountWaves, l, 1, 1);
        const double u = (double)E / ((double)g.nstripe * geo_width(g));
        if (u >= 0.95)
            return l;
        if (u > best_u) {
            best_u = u;
            best = l;
        }
    }
    return best;
}

inline ColGeo count_geo(int64_t T, int E)
{
    const int cl = count_cpl_log2(E);
    auto geo = [&](int steps) {
        ColGeo g = col_geo(T, E, kCountWaves, cl, steps, kCountMaxBlocks);
        if (g.gsplit > kCountMaxSplits)
            g.gsplit = kCountMaxSplits;
        return g;
    };
    int steps = kCountMaxSteps;
    ColGeo g = geo(steps);
    while (steps > 1 && (int64_t)g.gsplit * g.nstripe < kCountMinBlocks) {
        const ColGeo h = geo(steps / 2);
        if (h.nsplit > kCountMaxSplits)
            break;
        steps /= 2;
        g = h;
    }
    return g;
}

// Workspace of the count kernel: one 64-bit word per stripe column
// (contributions received in the high half, routed tokens in the low half),
// zero before a call and zero again after it (the last contribution to a
// column hands its total out and clears the word).  Depends on E only.
inline size_t count_ws_words(int E)
{
    const ColGeo g = col_geo(1, E, kCountWaves, count_cpl_log2(E), 1, 1);
    return (size_t)g.nstripe * geo_width(g);
}
inline size_t count_ws_bytes(int E)
{
    const size_t n = (count_ws_words(E) * 8 + 255) / 256 * 256;
    return n < 256 ? 256 : n;
}

inline ColGeo loss_geo(int64_t T, int E)
{
    return col_geo(T, E, kLossWaves, kLossCpl, kLossSteps, kLossMaxBlocks);
}

// The loss gradient only writes: fewer rows per wave and more blocks give
// a pure store stream more writers (T=8192, E=2304: 13.9 -> 13.1 us in a
// back-to-back loop, 14.2 -> 13.9 us in the cold benchmark).
constexpr int kLossBwdSteps = 2;
constexpr int kLossBwdMaxBlocks = 32768;

inline ColGeo loss_bwd_geo(int64_t T, int E)
{
    return col_geo(T, E, kLossWaves, kLossCpl, kLossBwdSteps, kLossBwdMaxBlocks);
}

// Workspace of the loss kernel: one fp64 partial per block.
inline size_t loss_ws_bytes(const ColGeo &g) { return (size_t)g.gsplit * g.nstripe * 8; }

// Workspace of the loss for T rows of E experts (>= 256 bytes).
inline size_t aux_ws_bytes(int64_t T, int E)
{
    size_t n = loss_ws_bytes(loss_geo(T, E));
    n = (n + 255) / 256 * 256;
    return n < 256 ? 256 : n;
}

// vec: the widest map load (16, 8 or 4 bytes, at most the bytes a lane owns
// per row) that E and the map's alignment allow, else 1 (byte loads).
hipError_t launch_count(const uint8_t *map, int vec, const ColGeo &g, int64_t *counts,
                        uint64_t *ws, hipStream_t stream);
hipError_t launch_loss(const void *scores, int dtype, bool vec, const ColGeo &g,
                       const int64_t *counts, double C, double *ws, float *loss,
                       hipStream_t stream);
// The library's own loss workspace (per device, kLossScratchBytes): its
// device address on the current device.
constexpr size_t kLossScratchBytes = 32768;
hipError_t loss_scratch(void **ptr);
hipError_t launch_loss_bwd(const float *grad_loss, const int64_t *counts, int dtype, bool vec,
                           const ColGeo &g, double C, void *grad_scores, hipStream_t stream);

// Decode-shape routing with expert maps (one workgroup, one wave per row).
constexpr int kRouteMaxRows = 16;
constexpr int kRouteMaxExperts = 1024;
constexpr int kRouteMaxK = 32;

struct RouteParams {
    const void *x;            // logits [T,E], TIn
    float *weights;           // [T,K]
    int32_t *ids;             // [T,K]
    int32_t *perm_to_unperm;  // [T*K]
    int32_t *unperm_to_perm;  // [T*K]
    int32_t *perm_expert;     // [T*K]
    int64_t *offsets;         // [E+1]
    int T;
    int E;
    int K;
    int score;                // SCORE_*
    int renorm;
};

hipError_t launch_route_maps(const RouteParams &p, int dtype, bool vec, hipStream_t stream);

// Routed top-k with the shared-expert gate (one wave per token).
constexpr int kGateMaxShared = 16;
constexpr int kGateMaxBlocks = 65536;  // the kernel strides over further tokens

struct GateParams {
    const void *x;      // gating logits [M,E]
    const void *hs;     // hidden states [M,H]
    const void *gw;     // gate weights [S,H]
    float *weights;     // [M, ld]
    int32_t *ids;       // [M, ld]
    int64_t M;
    int64_t ld;
    int E;
    int H;
    int K;
    int S;
    int renorm;
    int base;
    float scale;
};

hipError_t launch_shared_gate(const GateParams &p, int dtype, bool vec_g, bool vec_h,
                              hipStream_t stream);

// Chunk counts built per lane-group width (see router_launch.h).
constexpr int kNchLpt16[] = {1, 2, 4};
constexpr int kNchLpt32[] = {1, 2, 4};
constexpr int kNchLpt64[] = {1, 2, 3, 4, 6, 8, 9, 12, 16};
constexpr int kNchScalar[] = {1, 2, 3, 4, 6, 8, 9, 12, 16};

// Group-limited forward for rows of 32-expert groups (router_grouped.h):
// 16- or 32-lane tokens of 1, 2 or 4 chunks (E = nch * 4 * lpt), top lists
// of Q = 2 or 4; false when not built for (lpt, nch, Q).
bool fwd_grouped16(int lpt, int nch, int dtype, int score, int Q, bool bias,
                   const FwdParams &p, const Launch &l, hipError_t *err);
bool fwd_grouped32(int lpt, int nch, int dtype, int score, int Q, bool bias,
                   const FwdParams &p, const Launch &l, hipError_t *err);

// Streaming kernel for the bandwidth ceiling (router_stream.hip).
hipError_t launch_stream(const void *src, int64_t read_bytes, void *dst, int64_t write_bytes,
                         int units, hipStream_t stream);
hipError_t launch_row_stream(const float *x, float *a, float *b, uint8_t *m, int64_t T, int E,
                             hipStream_t stream);

// Each translation unit of kernels defines one pair; they return false when
// the (LPT, NCH, vec) configuration is not built there.
#define ROUTER_DECLARE_PART(NAME)                                                   \
    bool fwd_##NAME(int lpt, int nch, bool vec, int dtype, int score, int gm,       \
                    const FwdParams &p, const Launch &l, hipError_t *err);          \
    bool bwd_##NAME(int lpt, int nch, bool vec, int dtype, int score,               \
                    const BwdParams &p, const Launch &l, hipError_t *err);
ROUTER_DECLARE_PART(lpt16)
ROUTER_DECLARE_PART(lpt32)
ROUTER_DECLARE_PART(lpt64a)
ROUTER_DECLARE_PART(lpt64b)
ROUTER_DECLARE_PART(lpt64c)
ROUTER_DECLARE_PART(scalar)
ROUTER_DECLARE_PART(scalar2)
#undef ROUTER_DECLARE_PART

}  // namespace rker
