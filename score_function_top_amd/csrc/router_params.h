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
    int P;                // E / G
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

// LDS per token group: cand_slots u64 candidate slots; grouped routing adds
// group_scratch_floats floats.
constexpr int cand_slots(int lpt) { return 3 * lpt; }
constexpr int group_scratch_floats(int E, int G, int lpt)
{
    return E + G + lpt;
}

struct Launch {
    unsigned grid;
    size_t smem;
    hipStream_t stream;
};

// Chunk counts built per lane-group width (see router_launch.h).
constexpr int kNchLpt16[] = {1, 2, 4};
constexpr int kNchLpt32[] = {1, 2, 4};
constexpr int kNchLpt64[] = {1, 2, 3, 4, 6, 8, 9, 12, 16};
constexpr int kNchScalar[] = {1, 2, 4, 8, 16};

// Each translation unit of kernels defines one pair; they return false when
// the (LPT, NCH, vec) configuration is not built there.
#define ROUTER_DECLARE_PART(NAME)                                                   \
    bool fwd_##NAME(int lpt, int nch, bool vec, int dtype, int score, bool grouped, \
                    const FwdParams &p, const Launch &l, hipError_t *err);          \
    bool bwd_##NAME(int lpt, int nch, bool vec, int dtype, int score,               \
                    const BwdParams &p, const Launch &l, hipError_t *err);
ROUTER_DECLARE_PART(lpt16)
ROUTER_DECLARE_PART(lpt32)
ROUTER_DECLARE_PART(lpt64a)
ROUTER_DECLARE_PART(lpt64b)
ROUTER_DECLARE_PART(lpt64c)
ROUTER_DECLARE_PART(scalar)
#undef ROUTER_DECLARE_PART

}  // namespace rker
