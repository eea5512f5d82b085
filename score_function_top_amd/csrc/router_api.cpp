// router_api.cpp -- the C ABI of include/router.h: argument checks, choice
// of kernel configuration and selection path, launch.
//
// Host-side hardening follows the "Hardening" list of "[Common] Optimize
// fused router forward/backward kernels" (NVIDIA TransformerEngine pull
// request 3012): topk in [1, E], topk divisible by group_topk, and an
// element count that cannot overflow the index arithmetic (here 64-bit
// offsets, so the bound is the 64-bit byte count).  The top-k path
// threshold mirrors that page's crossover variable ("Simple kernel path for
// small topk"); by default the crossover follows the row layout.
#include "router.h"

#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cerrno>
#include <cmath>
#include <cstdlib>
#include <mutex>

#include "router_params.h"

using namespace rker;

static_assert(ROUTER_AUX_LOSS_SCRATCH_BYTES == kLossScratchBytes,
              "the header states the library's loss buffer size");
// 64-lane tokens, 4 per workgroup: candidate lists plus the row copy of the
// LDS group stage, (E + G + 64) floats per token
static_assert((kFwdLdsBytes - 4 * cand_slots(64) * 8) / 16 - 64 == ROUTER_GROUP_LDS_MAX_E_PLUS_G,
              "the header states the LDS bound of grouped routing");
static_assert(ROUTER_MAX_GROUPS == 64, "one lane of a 64-lane token per group");
static_assert(ROUTER_MAX_EXPERTS + ROUTER_MAX_GROUPS <= ROUTER_GROUP_LDS_MAX_E_PLUS_G,
              "every grouped shape within the other limits fits the LDS");

namespace {

// ------------------------------------------------------------ threshold

constexpr int kUnread = -2;  // the environment has not been read yet
std::atomic<int> g_threshold{kUnread};
std::once_flag g_threshold_once;

// ROUTER_TOPK_PATH_AUTO or a fixed crossover in [0, ROUTER_MAX_EXPERTS].
int threshold()
{
    std::call_once(g_threshold_once, [] {
        int v = ROUTER_TOPK_PATH_AUTO;
        if (const char *e = std::getenv("ROUTER_TOPK_PATH_THRESHOLD")) {
            char *end = nullptr;
            errno = 0;
            long x = std::strtol(e, &end, 10);
            if (errno == 0 && end != e && *end == '\0' && x >= 0 && x <= ROUTER_MAX_EXPERTS)
                v = (int)x;
        }
        int expect = kUnread;
        g_threshold.compare_exchange_strong(expect, v);
    });
    return g_threshold.load();
}

// Automatic crossover for rows held as `epl` elements per lane: the
// argmax rounds cost about a pass over the lane's elements each, the
// pruned sort a fixed number of cross-lane stages, so the rounds stop
// paying sooner on longer lanes.  Measured on MI355X at T=8192 (graph
// replay, cold): the sort is ahead from K=5 at 4 elements per lane (E=16,
// 64), from K=4 at 8 (E=128, 256: 6.97 -> 6.44 us at E=256, K=4) and from
// K=2 at 16 or more (E=512: 10.25 -> 9.73 us; E=2304: 47.6 -> 44.5 us).
int auto_threshold(int epl) { return epl <= 4 ? 5 : (epl <= 8 ? 4 : 2); }

std::atomic<int> g_group_stage{ROUTER_GROUP_STAGE_AUTO};
std::atomic<int> g_grid_mode{ROUTER_GRID_FULL};

bool persistent() { return g_grid_mode.load() == ROUTER_GRID_PERSISTENT; }

// ------------------------------------------------------------ devices

struct DevInfo {
    int cus = 0;
    size_t lds_per_block = 0;
};

constexpr int kMaxDevices = 64;
DevInfo g_dev[kMaxDevices];
std::once_flag g_dev_once[kMaxDevices];

// Device attributes, read once per device.
hipError_t dev_info(DevInfo *out)
{
    int d = 0;
    hipError_t e = hipGetDevice(&d);
    if (e != hipSuccess)
        return e;
    if (d < 0 || d >= kMaxDevices)
        return hipErrorInvalidDevice;
    hipError_t err = hipSuccess;
    std::call_once(g_dev_once[d], [&] {
        int cus = 0, lds = 0;
        err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, d);
        if (err == hipSuccess)
            err = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, d);
        if (err == hipSuccess) {
            g_dev[d].cus = cus;
            g_dev[d].lds_per_block = (size_t)lds;
        }
    });
    if (err != hipSuccess)
        return err;
    if (g_dev[d].cus <= 0)
        return hipErrorInvalidDevice;
    *out = g_dev[d];
    return hipSuccess;
}

// ------------------------------------------------------------ checks

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t dsize(int dtype) { return dtype == ROUTER_BF16 ? 2 : 4; }

router_status check_common(int dtype, int64_t T, int32_t E, int score_fn)
{
    if (dtype != ROUTER_F32 && dtype != ROUTER_BF16)
        return ROUTER_ERR_INVALID_ARG;
    if (score_fn != ROUTER_SOFTMAX && score_fn != ROUTER_SIGMOID)
        return ROUTER_ERR_INVALID_ARG;
    if (T < 0 || E < 1)
        return ROUTER_ERR_INVALID_ARG;
    if (E > ROUTER_MAX_EXPERTS)
        return ROUTER_ERR_UNSUPPORTED;
    // bytes of the largest [T,E] array (fp32 intermediate) must fit int64
    if (T > INT64_MAX / ((int64_t)E * 4))
        return ROUTER_ERR_OVERFLOW;
    return ROUTER_OK;
}

// ------------------------------------------------------------ configs

struct Cfg {
    int lpt;
    int nch;
    bool vec;
};

template <size_t N>
int pick_nch(const int (&list)[N], int need)
{
    for (size_t i = 0; i < N; i++)
        if (list[i] >= need)
            return list[i];
    return -1;
}

// Lanes per token for rows of E experts: the row in at most 4 chunks of
// 4 elements per lane, except that rows of 129..256 experts take 32 lanes
// (two chunks) when T is small enough that 16-lane tokens leave the SIMDs
// with few waves: T <= 8192, or T <= 16384 with the group stage, whose
// per-token work is larger.  Measured on MI355X (fp32 softmax K=4 at
// T=8192: forward 8.1 -> 7.1 us, backward 7.4 -> 6.4 us; grouped bf16
// sigmoid at T=16384: 18.7 -> 15.8 us; the 16-lane form stays ahead at
// T=65536 and without groups at T=16384).
int lpt_for_rows(int E, int64_t T, bool grouped)
{
    if (E <= 128)
        return 16;
    if (E <= 256)
        return T <= 8192 || (grouped && T <= 16384) ? 32 : 16;
    return E <= 512 ? 32 : 64;
}

// Fills nch for c.lpt / c.vec; false when no built kernel holds E.
bool fill_nch(Cfg &c, int E)
{
    const int need = (E + 4 * c.lpt - 1) / (4 * c.lpt);
    if (!c.vec)
        c.nch = pick_nch(kNchScalar, need);
    else if (c.lpt == 16)
        c.nch = pick_nch(kNchLpt16, need);
    else if (c.lpt == 32)
        c.nch = pick_nch(kNchLpt32, need);
    else
        c.nch = pick_nch(kNchLpt64, need);
    return c.nch > 0;
}

int widen(int lpt, int need) { return need <= lpt ? lpt : (need <= 32 ? 32 : 64); }

// log2 of the lanes per group when the register group stage can take G
// groups of E/G experts in the layout c with q = K/Kg summed per group:
// E/G = 4*L with L a power of two no larger than the lane width, at most
// group_reg_slots(nch) group slots, a vector kernel of at most kGroupRegMaxNch
// chunks, q <= 4.  -1 otherwise.
int group_reg_log(const Cfg &c, int E, int G, int q)
{
    const int P = E / G;
    if (!c.vec || c.nch > kGroupRegMaxNch || q > 4 || P % 4 != 0)
        return -1;
    const int L = P / 4;
    if ((L & (L - 1)) != 0)
        return -1;
    int lg = 0;
    while ((1 << lg) < L)
        lg++;
    return group_reg_ok(c.lpt, c.nch, lg) ? lg : -1;
}

// Lanes per token of the kernel for rows of 32-expert groups
// (router_grouped.h): E = 32 * G with G a power of two in [2, 16],
// q = K / Kg <= 4, a vector layout, and at most one selected expert per
// lane (K <= lanes); 0 when it does not take the shape.  Rows of up to 256
// experts take 16 lanes (one, two or four chunks), 512 experts 32 lanes
// (four chunks).  Measured on MI355X at E=256 in 8 groups, bf16 (full grid,
// interleaved runs): 16 lanes 8.53 us at T=16384 and 28.65 us at T=65536,
// 32 lanes 11.0 and 31.7 us (8.99 us at T=16384 on the persistent grid).
int grouped_lpt(const Cfg &c, int E, int G, int K, int Kg)
{
    if (G < 2 || G > 16 || E != 32 * G || (G & (G - 1)) != 0 || K / Kg > 4 || !c.vec)
        return 0;
    const int lpt = E <= 256 ? 16 : 32;
    return K <= lpt ? lpt : 0;
}

hipError_t launch_fwd(const Cfg &c, int dtype, int score, int gm, const FwdParams &p,
                      const Launch &l)
{
    hipError_t err = hipErrorInvalidValue;
    if (fwd_lpt16(c.lpt, c.nch, c.vec, dtype, score, gm, p, l, &err) ||
        fwd_lpt32(c.lpt, c.nch, c.vec, dtype, score, gm, p, l, &err) ||
        fwd_lpt64a(c.lpt, c.nch, c.vec, dtype, score, gm, p, l, &err) ||
        fwd_lpt64b(c.lpt, c.nch, c.vec, dtype, score, gm, p, l, &err) ||
        fwd_lpt64c(c.lpt, c.nch, c.vec, dtype, score, gm, p, l, &err) ||
        fwd_scalar(c.lpt, c.nch, c.vec, dtype, score, gm, p, l, &err) ||
        fwd_scalar2(c.lpt, c.nch, c.vec, dtype, score, gm, p, l, &err))
        return err;
    return hipErrorInvalidValue;
}

hipError_t launch_bwd(const Cfg &c, int dtype, int score, const BwdParams &p, const Launch &l)
{
    hipError_t err = hipErrorInvalidValue;
    if (bwd_lpt16(c.lpt, c.nch, c.vec, dtype, score, p, l, &err) ||
        bwd_lpt32(c.lpt, c.nch, c.vec, dtype, score, p, l, &err) ||
        bwd_lpt64a(c.lpt, c.nch, c.vec, dtype, score, p, l, &err) ||
        bwd_lpt64b(c.lpt, c.nch, c.vec, dtype, score, p, l, &err) ||
        bwd_lpt64c(c.lpt, c.nch, c.vec, dtype, score, p, l, &err) ||
        bwd_scalar(c.lpt, c.nch, c.vec, dtype, score, p, l, &err) ||
        bwd_scalar2(c.lpt, c.nch, c.vec, dtype, score, p, l, &err))
        return err;
    return hipErrorInvalidValue;
}

unsigned grid_for(int64_t T, int lpt, int waves = kWaves)
{
    const int64_t tpb = (int64_t)waves * (64 / lpt);
    int64_t blocks = (T + tpb - 1) / tpb;
    const int64_t cap = (int64_t)1 << 22;  // the kernels stride over the rest
    return (unsigned)(blocks < cap ? blocks : cap);
}

// Shared forward path of router_topk_fwd and router_aux_scores.
router_status fwd_common(const void *x, int dtype, int64_t T, int32_t E, int32_t K,
                         int score_fn, int renorm, int32_t G, int32_t Kg, float scale,
                         const float *bias, void *out, uint8_t *map, float *inter,
                         void *stream, bool aux)
{
    router_status st = check_common(dtype, T, E, score_fn);
    if (st != ROUTER_OK)
        return st;
    if (K < 1 || K > E || G < 0)
        return ROUTER_ERR_INVALID_ARG;
    if (G > 0 && (E % G != 0 || Kg < 1 || Kg > G || K % Kg != 0 || K / Kg > E / G))
        return ROUTER_ERR_INVALID_ARG;
    if (!std::isfinite(scale))
        return ROUTER_ERR_INVALID_ARG;
    if (bias && score_fn != ROUTER_SIGMOID)
        return ROUTER_ERR_UNSUPPORTED;
    if (G > ROUTER_MAX_GROUPS)
        return ROUTER_ERR_UNSUPPORTED;
    if (T == 0)
        return ROUTER_OK;
    if (!x || !out || !map || !inter)
        return ROUTER_ERR_INVALID_ARG;
    const size_t ds = dsize(dtype);
    if (!aligned(x, ds) || !aligned(out, ds) || !aligned(inter, 4) || (bias && !aligned(bias, 4)))
        return ROUTER_ERR_INVALID_ARG;

    const bool vec = E % 4 == 0 && aligned(x, 16) && aligned(out, 16) && aligned(inter, 16) &&
                     aligned(map, 16) && (!bias || aligned(bias, 16));
    Cfg c{vec ? lpt_for_rows(E, T, G > 0) : 64, 0, vec};
    int thr = threshold();
    if (thr == ROUTER_TOPK_PATH_AUTO) {
        Cfg a = c;
        if (!fill_nch(a, E))
            return ROUTER_ERR_UNSUPPORTED;
        thr = auto_threshold(4 * a.nch);
    }
    int sel = K < thr ? SEL_ARGMAX : SEL_PRUNE;
    // the pruned sort takes K <= 2 * lanes where prune_top2 holds (no
    // groups, fewer than 64 lanes), else K <= lanes
    if (sel == SEL_PRUNE)
        c.lpt = widen(c.lpt, G > 0 ? K : (K + 1) / 2);
    if (G > 0)
        c.lpt = widen(c.lpt, G);
    if (!fill_nch(c, E))
        return ROUTER_ERR_UNSUPPORTED;
    if (sel == SEL_PRUNE && K > (prune_top2(c.lpt, G > 0 ? GROUP_LDS : GROUP_NONE) ? 2 * c.lpt
                                                                                  : c.lpt))
        sel = SEL_BITS;

    // rows of 32-expert groups (E = 64..512) have their own kernel
    if (g_group_stage.load() == ROUTER_GROUP_STAGE_AUTO && G > 0 && vec) {
        const int lg = grouped_lpt(c, E, G, K, Kg);
        if (lg > 0) {
            DevInfo dev;
            if (dev_info(&dev) != hipSuccess)
                return ROUTER_ERR_HIP;
            const int tpb = kWaves * (64 / lg);
            FwdParams p{};
            p.x = x;
            p.out = out;
            p.map = map;
            p.inter = inter;
            p.bias = bias;
            p.T = T;
            p.E = E;
            p.K = K;
            p.sel = SEL_PRUNE;
            p.renorm = renorm ? 1 : 0;
            p.G = G;
            p.Kg = Kg;
            p.q = K / Kg;
            p.P = E / G;
            p.scale = scale;
            // LDS: the candidate lists, and a copy of the expert bias
            const size_t lds = (size_t)tpb * cand_slots(lg) * sizeof(uint64_t) +
                               (bias ? (size_t)E * sizeof(float) : 0);
            const Launch l{grid_for(T, lg), lds, (hipStream_t)stream, persistent()};
            const int nch = E / (4 * lg);
            const int Q = p.q <= 2 ? 2 : 4;
            hipError_t err = hipErrorInvalidValue;
            if (!fwd_grouped16(lg, nch, dtype, score_fn, Q, bias != nullptr, p, l, &err) &&
                !fwd_grouped32(lg, nch, dtype, score_fn, Q, bias != nullptr, p, l, &err))
                return ROUTER_ERR_HIP;
            return err == hipSuccess ? ROUTER_OK : ROUTER_ERR_HIP;
        }
    }

    const bool reg = g_group_stage.load() == ROUTER_GROUP_STAGE_AUTO && G > 0 &&
                     group_reg_log(c, E, G, K / Kg) >= 0;
    const int gm = G == 0 ? GROUP_NONE : (reg ? GROUP_REG : GROUP_LDS);

    // LDS of the launch: the candidate lists, plus the row copy of the LDS
    // group stage; a host-side bound first (the workgroup LDS the kernels
    // are built for), then the device's own limit
    const int waves = fwd_waves(c.lpt, c.nch, gm, sel, c.vec);
    const int tpb = waves * (64 / c.lpt);
    size_t smem = (size_t)tpb * cand_slots(c.lpt) * sizeof(uint64_t);
    if (gm == GROUP_LDS)
        smem += (size_t)tpb * group_scratch_floats(E, G, c.lpt) * sizeof(float);
    if (smem > kFwdLdsBytes)
        return ROUTER_ERR_UNSUPPORTED;
    DevInfo dev;
    if (dev_info(&dev) != hipSuccess)
        return ROUTER_ERR_HIP;
    if (smem > dev.lds_per_block)
        return ROUTER_ERR_UNSUPPORTED;

    FwdParams p{};
    p.x = x;
    p.out = out;
    p.map = map;
    p.inter = inter;
    p.bias = bias;
    p.T = T;
    p.E = E;
    p.K = K;
    p.sel = sel;
    p.renorm = renorm ? 1 : 0;
    p.aux = aux ? 1 : 0;
    p.G = G;
    p.Kg = G > 0 ? Kg : 0;
    p.q = G > 0 ? K / Kg : 0;
    p.P = G > 0 ? E / G : 0;
    p.scale = scale;
    const Launch l{grid_for(T, c.lpt, waves), smem, (hipStream_t)stream, persistent(),
                   (unsigned)(64 * waves)};
    return launch_fwd(c, dtype, score_fn, gm, p, l) == hipSuccess ? ROUTER_OK : ROUTER_ERR_HIP;
}

router_status bwd_common(const void *g, const float *s, const uint8_t *m, int dtype, int64_t T,
                         int32_t E, int32_t K, int score_fn, int renorm, float scale, void *dx,
                         void *stream)
{
    router_status st = check_common(dtype, T, E, score_fn);
    if (st != ROUTER_OK)
        return st;
    if (K < 1 || K > E)
        return ROUTER_ERR_INVALID_ARG;
    if (!std::isfinite(scale))
        return ROUTER_ERR_INVALID_ARG;
    if (T == 0)
        return ROUTER_OK;
    const bool aux = m == nullptr;
    if (!g || !s || !dx)
        return ROUTER_ERR_INVALID_ARG;
    const size_t ds = dsize(dtype);
    if (!aligned(g, ds) || !aligned(dx, ds) || !aligned(s, 4))
        return ROUTER_ERR_INVALID_ARG;
    const bool vec = E % 4 == 0 && aligned(g, 16) && aligned(dx, 16) && aligned(s, 16) &&
                     (aux || aligned(m, 16));
    Cfg c{vec ? lpt_for_rows(E, T, false) : 64, 0, vec};
    if (!fill_nch(c, E))
        return ROUTER_ERR_UNSUPPORTED;
    DevInfo dev;
    if (dev_info(&dev) != hipSuccess)
        return ROUTER_ERR_HIP;
    BwdParams p{};
    p.g = g;
    p.s = s;
    p.m = m;
    p.dx = dx;
    p.T = T;
    p.E = E;
    p.K = K;
    p.renorm = renorm ? 1 : 0;
    p.scale = scale;
    const Launch l{grid_for(T, c.lpt), 0, (hipStream_t)stream, persistent()};
    return launch_bwd(c, dtype, score_fn, p, l) == hipSuccess ? ROUTER_OK : ROUTER_ERR_HIP;
}

// ------------------------------------------------------------ aux loss

router_status check_loss_shape(int64_t T, int32_t E)
{
    if (T < 0 || E < 1)
        return ROUTER_ERR_INVALID_ARG;
    if (E > ROUTER_MAX_EXPERTS)
        return ROUTER_ERR_UNSUPPORTED;
    if (T > INT64_MAX / ((int64_t)E * 4))
        return ROUTER_ERR_OVERFLOW;
    return ROUTER_OK;
}

router_status check_loss_args(int dtype, int64_t N, int32_t K, float coeff)
{
    if (dtype != ROUTER_F32 && dtype != ROUTER_BF16)
        return ROUTER_ERR_INVALID_ARG;
    if (N < 1 || K < 1 || !std::isfinite(coeff))
        return ROUTER_ERR_INVALID_ARG;
    return ROUTER_OK;
}

// C = coeff * E / (N^2 K) in fp64.
double loss_coeff(float coeff, int32_t E, int64_t N, int32_t K)
{
    return (double)coeff * (double)E / ((double)N * (double)N * (double)K);
}

}  // namespace

extern "C" {

router_status router_topk_fwd(const void *logits, int dtype, int64_t T, int32_t E, int32_t K,
                              int score_fn, int renorm, int32_t num_groups, int32_t group_topk,
                              float scaling_factor, const float *expert_bias, void *probs,
                              uint8_t *routing_map, float *intermediate, void *hip_stream)
{
    return fwd_common(logits, dtype, T, E, K, score_fn, renorm, num_groups, group_topk,
                      scaling_factor, expert_bias, probs, routing_map, intermediate, hip_stream,
                      false);
}

router_status router_topk_bwd(const void *grad_probs, const float *intermediate,
                              const uint8_t *routing_map, int dtype, int64_t T, int32_t E,
                              int32_t K, int score_fn, int renorm, float scaling_factor,
                              void *grad_logits, void *hip_stream)
{
    if (T > 0 && !routing_map)
        return ROUTER_ERR_INVALID_ARG;
    return bwd_common(grad_probs, intermediate, routing_map, dtype, T, E, K, score_fn, renorm,
                      scaling_factor, grad_logits, hip_stream);
}

router_status router_aux_scores(const void *logits, int dtype, int64_t T, int32_t E, int32_t K,
                                int score_fn, int renorm, void *scores, uint8_t *routing_map,
                                float *intermediate, void *hip_stream)
{
    return fwd_common(logits, dtype, T, E, K, score_fn, renorm, 0, 0, 1.0f, nullptr, scores,
                      routing_map, intermediate, hip_stream, true);
}

router_status router_aux_scores_bwd(const void *grad_scores, const float *intermediate,
                                    int dtype, int64_t T, int32_t E, int score_fn, int renorm,
                                    void *grad_logits, void *hip_stream)
{
    return bwd_common(grad_scores, intermediate, nullptr, dtype, T, E, E > 0 ? E : 1, score_fn,
                      renorm, 1.0f, grad_logits, hip_stream);
}

size_t router_aux_loss_workspace_bytes(int64_t T, int32_t E)
{
    if (check_loss_shape(T, E) != ROUTER_OK)
        return 0;
    return aux_ws_bytes(T, E);
}

size_t router_tokens_per_expert_workspace_bytes(int64_t T, int32_t E)
{
    if (check_loss_shape(T, E) != ROUTER_OK)
        return 0;
    return count_ws_bytes(E);
}

router_status router_tokens_per_expert(const uint8_t *routing_map, int64_t T, int32_t E,
                                       int64_t *tokens_per_expert, void *workspace,
                                       size_t workspace_bytes, void *hip_stream)
{
    router_status st = check_loss_shape(T, E);
    if (st != ROUTER_OK)
        return st;
    if (T > (int64_t)UINT32_MAX)  // per-column totals are 32-bit
        return ROUTER_ERR_UNSUPPORTED;
    if (!tokens_per_expert || !workspace || (T > 0 && !routing_map))
        return ROUTER_ERR_INVALID_ARG;
    if (!aligned(tokens_per_expert, 8) || !aligned(workspace, 8) ||
        workspace_bytes < count_ws_bytes(E))
        return ROUTER_ERR_INVALID_ARG;
    const ColGeo g = count_geo(T, E);
    const int cpl = 1 << g.cpl_log2;
    const int vec = cpl >= 16 && E % 16 == 0 && aligned(routing_map, 16)  ? 16
                    : cpl >= 8 && E % 8 == 0 && aligned(routing_map, 8) ? 8
                    : E % 4 == 0 && aligned(routing_map, 4)             ? 4
                                                                         : 1;
    const hipError_t e = launch_count(routing_map, vec, g, tokens_per_expert,
                                      (uint64_t *)workspace, (hipStream_t)hip_stream);
    return e == hipSuccess ? ROUTER_OK : ROUTER_ERR_HIP;
}

router_status router_aux_loss_fwd(const void *scores, int dtype, int64_t T, int32_t E,
                                  const int64_t *tokens_per_expert, int64_t total_tokens,
                                  int32_t K, float coeff, float *loss, void *workspace,
                                  size_t workspace_bytes, void *hip_stream)
{
    router_status st = check_loss_shape(T, E);
    if (st == ROUTER_OK)
        st = check_loss_args(dtype, total_tokens, K, coeff);
    if (st != ROUTER_OK)
        return st;
    if (!tokens_per_expert || !loss || !workspace || (T > 0 && !scores))
        return ROUTER_ERR_INVALID_ARG;
    const size_t ds = dsize(dtype);
    if (!aligned(scores, ds) || !aligned(tokens_per_expert, 8) || !aligned(loss, 4) ||
        !aligned(workspace, 8) || workspace_bytes < aux_ws_bytes(T, E))
        return ROUTER_ERR_INVALID_ARG;
    const bool vec = E % 4 == 0 && aligned(scores, 4 * ds);
    const hipError_t e =
        launch_loss(scores, dtype, vec, loss_geo(T, E), tokens_per_expert,
                    loss_coeff(coeff, E, total_tokens, K), (double *)workspace, loss,
                    (hipStream_t)hip_stream);
    return e == hipSuccess ? ROUTER_OK : ROUTER_ERR_HIP;
}

router_status router_aux_loss_fwd_noalloc(const void *scores, int dtype, int64_t T, int32_t E,
                                          const int64_t *tokens_per_expert, int64_t total_tokens,
                                          int32_t K, float coeff, float *loss, void *hip_stream)
{
    router_status st = check_loss_shape(T, E);
    if (st == ROUTER_OK)
        st = check_loss_args(dtype, total_tokens, K, coeff);
    if (st != ROUTER_OK)
        return st;
    if (!tokens_per_expert || !loss || (T > 0 && !scores))
        return ROUTER_ERR_INVALID_ARG;
    const size_t ds = dsize(dtype);
    if (!aligned(scores, ds) || !aligned(tokens_per_expert, 8) || !aligned(loss, 4))
        return ROUTER_ERR_INVALID_ARG;
    if (aux_ws_bytes(T, E) > kLossScratchBytes)
        return ROUTER_ERR_UNSUPPORTED;
    void *ws = nullptr;
    if (loss_scratch(&ws) != hipSuccess)
        return ROUTER_ERR_HIP;
    const bool vec = E % 4 == 0 && aligned(scores, 4 * ds);
    const hipError_t e =
        launch_loss(scores, dtype, vec, loss_geo(T, E), tokens_per_expert,
                    loss_coeff(coeff, E, total_tokens, K), (double *)ws, loss,
                    (hipStream_t)hip_stream);
    return e == hipSuccess ? ROUTER_OK : ROUTER_ERR_HIP;
}

router_status router_aux_loss_bwd(const float *grad_loss, const int64_t *tokens_per_expert,
                                  int dtype, int64_t T, int32_t E, int64_t total_tokens,
                                  int32_t K, float coeff, void *grad_scores, void *hip_stream)
{
    router_status st = check_loss_shape(T, E);
    if (st == ROUTER_OK)
        st = check_loss_args(dtype, total_tokens, K, coeff);
    if (st != ROUTER_OK)
        return st;
    if (T == 0)
        return ROUTER_OK;
    if (!grad_loss || !tokens_per_expert || !grad_scores)
        return ROUTER_ERR_INVALID_ARG;
    const size_t ds = dsize(dtype);
    if (!aligned(grad_loss, 4) || !aligned(tokens_per_expert, 8) || !aligned(grad_scores, ds))
        return ROUTER_ERR_INVALID_ARG;
    const bool vec = E % 4 == 0 && aligned(grad_scores, 4 * ds);
    const hipError_t e = launch_loss_bwd(grad_loss, tokens_per_expert, dtype, vec,
                                         loss_bwd_geo(T, E), loss_coeff(coeff, E, total_tokens, K),
                                         grad_scores, (hipStream_t)hip_stream);
    return e == hipSuccess ? ROUTER_OK : ROUTER_ERR_HIP;
}

router_status router_route_maps(const void *logits, int dtype, int32_t T, int32_t E, int32_t K,
                                int score_fn, int renorm, float *topk_weights,
                                int32_t *topk_ids, int32_t *perm_to_unperm,
                                int32_t *unperm_to_perm, int32_t *perm_expert,
                                int64_t *expert_offsets, void *hip_stream)
{
    if (dtype != ROUTER_F32 && dtype != ROUTER_BF16)
        return ROUTER_ERR_INVALID_ARG;
    if (score_fn != ROUTER_SOFTMAX && score_fn != ROUTER_SIGMOID)
        return ROUTER_ERR_INVALID_ARG;
    if (T < 0 || E < 1 || K < 1 || K > E)
        return ROUTER_ERR_INVALID_ARG;
    if (T > ROUTER_ROUTE_MAX_ROWS || E > ROUTER_ROUTE_MAX_EXPERTS || K > ROUTER_ROUTE_MAX_K)
        return ROUTER_ERR_UNSUPPORTED;
    if (!expert_offsets || !aligned(expert_offsets, 8))
        return ROUTER_ERR_INVALID_ARG;
    if (T > 0 && (!logits || !topk_weights || !topk_ids || !perm_to_unperm || !unperm_to_perm ||
                  !perm_expert))
        return ROUTER_ERR_INVALID_ARG;
    const size_t ds = dsize(dtype);
    if (T > 0 && (!aligned(logits, ds) || !aligned(topk_weights, 4) || !aligned(topk_ids, 4) ||
                  !aligned(perm_to_unperm, 4) || !aligned(unperm_to_perm, 4) ||
                  !aligned(perm_expert, 4)))
        return ROUTER_ERR_INVALID_ARG;
    RouteParams p{};
    p.x = logits;
    p.weights = topk_weights;
    p.ids = topk_ids;
    p.perm_to_unperm = perm_to_unperm;
    p.unperm_to_perm = unperm_to_perm;
    p.perm_expert = perm_expert;
    p.offsets = expert_offsets;
    p.T = T;
    p.E = E;
    p.K = K;
    p.score = score_fn;
    p.renorm = renorm ? 1 : 0;
    const bool vec = E % 4 == 0 && aligned(logits, 4 * ds);
    return launch_route_maps(p, dtype, vec, (hipStream_t)hip_stream) == hipSuccess
               ? ROUTER_OK
               : ROUTER_ERR_HIP;
}

router_status router_topk_shared_gate(const void *gating, const void *hidden,
                                      const void *gate_weight, int dtype, int64_t M, int32_t E,
                                      int32_t H, int32_t K, int32_t S, int renorm,
                                      float shared_scale, int32_t shared_base,
                                      float *topk_weights, int32_t *topk_ids, int64_t ld,
                                      void *hip_stream)
{
    if (dtype != ROUTER_F32 && dtype != ROUTER_BF16)
        return ROUTER_ERR_INVALID_ARG;
    if (M < 0 || E < 1 || H < 1 || K < 1 || K > E || S < 1 || ld < (int64_t)K + S)
        return ROUTER_ERR_INVALID_ARG;
    if (!std::isfinite(shared_scale) || shared_base < 0 || shared_base > INT32_MAX - S)
        return ROUTER_ERR_INVALID_ARG;
    if (E > ROUTER_GATE_MAX_EXPERTS || K > ROUTER_GATE_MAX_K || S > ROUTER_GATE_MAX_SHARED)
        return ROUTER_ERR_UNSUPPORTED;
    const size_t ds = dsize(dtype);
    if ((int64_t)S * H * (int64_t)ds > INT32_MAX || M > INT64_MAX / ((int64_t)H * 4) ||
        M > INT64_MAX / ((int64_t)E * 4) || M > INT64_MAX / (ld * 4))
        return ROUTER_ERR_OVERFLOW;
    if (M == 0)
        return ROUTER_OK;
    if (!gating || !hidden || !gate_weight || !topk_weights || !topk_ids)
        return ROUTER_ERR_INVALID_ARG;
    if (!aligned(gating, ds) || !aligned(hidden, ds) || !aligned(gate_weight, ds) ||
        !aligned(topk_weights, 4) || !aligned(topk_ids, 4))
        return ROUTER_ERR_INVALID_ARG;
    GateParams p{};
    p.x = gating;
    p.hs = hidden;
    p.gw = gate_weight;
    p.weights = topk_weights;
    p.ids = topk_ids;
    p.M = M;
    p.ld = ld;
    p.E = E;
    p.H = H;
    p.K = K;
    p.S = S;
    p.renorm = renorm ? 1 : 0;
    p.base = shared_base;
    p.scale = shared_scale;
    const bool vec_g = E % 4 == 0 && aligned(gating, 4 * ds);
    const int vh = (int)(16 / ds);
    const bool vec_h = H % vh == 0 && aligned(hidden, 16) && aligned(gate_weight, 16);
    return launch_shared_gate(p, dtype, vec_g, vec_h, (hipStream_t)hip_stream) == hipSuccess
               ? ROUTER_OK
               : ROUTER_ERR_HIP;
}

const char *router_status_str(router_status s)
{
    switch (s) {
    case ROUTER_OK:
        return "ROUTER_OK";
    case ROUTER_ERR_INVALID_ARG:
        return "ROUTER_ERR_INVALID_ARG: argument outside the operation's domain";
    case ROUTER_ERR_OVERFLOW:
        return "ROUTER_ERR_OVERFLOW: T*E*element size overflows 64 bits";
    case ROUTER_ERR_UNSUPPORTED:
        return "ROUTER_ERR_UNSUPPORTED: valid arguments this library does not implement";
    case ROUTER_ERR_HIP:
        return "ROUTER_ERR_HIP: a HIP call or kernel launch failed";
    }
    return "unknown router_status";
}

int router_get_topk_path_threshold(void) { return threshold(); }

router_status router_set_topk_path_threshold(int t)
{
    if ((t < 0 && t != ROUTER_TOPK_PATH_AUTO) || t > ROUTER_MAX_EXPERTS)
        return ROUTER_ERR_INVALID_ARG;
    threshold();  // the environment is read first, then overridden
    g_threshold.store(t);
    return ROUTER_OK;
}

router_status router_device_query(int32_t *compute_units, int32_t *clock_khz,
                                  int32_t *memory_clock_khz, int32_t *memory_bus_bits)
{
    int d = 0;
    if (hipGetDevice(&d) != hipSuccess)
        return ROUTER_ERR_HIP;
    const struct {
        int32_t *out;
        hipDeviceAttribute_t attr;
    } q[] = {{compute_units, hipDeviceAttributeMultiprocessorCount},
             {clock_khz, hipDeviceAttributeClockRate},
             {memory_clock_khz, hipDeviceAttributeMemoryClockRate},
             {memory_bus_bits, hipDeviceAttributeMemoryBusWidth}};
    for (const auto &e : q) {
        if (!e.out)
            continue;
        int v = 0;
        if (hipDeviceGetAttribute(&v, e.attr, d) != hipSuccess)
            return ROUTER_ERR_HIP;
        *e.out = (int32_t)v;
    }
    return ROUTER_OK;
}

router_status router_stream_bandwidth(const void *src, int64_t read_bytes, void *dst,
                                      int64_t write_bytes, int32_t units_per_thread,
                                      void *hip_stream)
{
    if (read_bytes < 0 || write_bytes < 0 || read_bytes % 16 != 0 || write_bytes % 16 != 0)
        return ROUTER_ERR_INVALID_ARG;
    if (units_per_thread != 1 && units_per_thread != 2 && units_per_thread != 4 &&
        units_per_thread != 8)
        return ROUTER_ERR_INVALID_ARG;
    if ((read_bytes > 0 && (!src || !aligned(src, 16))) ||
        (write_bytes > 0 && (!dst || !aligned(dst, 16))))
        return ROUTER_ERR_INVALID_ARG;
    return launch_stream(src, read_bytes, dst, write_bytes, units_per_thread,
                         (hipStream_t)hip_stream) == hipSuccess
               ? ROUTER_OK
               : ROUTER_ERR_HIP;
}

router_status router_row_stream_bandwidth(const float *x, float *out_a, float *out_b,
                                          uint8_t *out_map, int64_t T, int64_t E,
                                          void *hip_stream)
{
    if (T < 0 || E < 256 || E > 4096 || E % 256 != 0)
        return ROUTER_ERR_INVALID_ARG;
    if (T > 0 && (!x || !out_a || !out_b || !out_map || !aligned(x, 16) || !aligned(out_a, 16) ||
                  !aligned(out_b, 16) || !aligned(out_map, 4)))
        return ROUTER_ERR_INVALID_ARG;
    return launch_row_stream(x, out_a, out_b, out_map, T, (int)E, (hipStream_t)hip_stream) ==
                   hipSuccess
               ? ROUTER_OK
               : ROUTER_ERR_HIP;
}

int router_get_grid_mode(void) { return g_grid_mode.load(); }

router_status router_set_grid_mode(int mode)
{
    if (mode != ROUTER_GRID_FULL && mode != ROUTER_GRID_PERSISTENT)
        return ROUTER_ERR_INVALID_ARG;
    g_grid_mode.store(mode);
    return ROUTER_OK;
}

int router_get_group_stage(void) { return g_group_stage.load(); }

router_status router_set_group_stage(int stage)
{
    if (stage != ROUTER_GROUP_STAGE_AUTO && stage != ROUTER_GROUP_STAGE_LDS)
        return ROUTER_ERR_INVALID_ARG;
    g_group_stage.store(stage);
    return ROUTER_OK;
}

}  // extern "C"
