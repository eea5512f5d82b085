/*
 * router.h -- C ABI of the MI355X (gfx950) fused MoE router library.
 *
 * The library implements the two fused router operations of "[Common]
 * Optimize fused router forward/backward kernels" (NVIDIA TransformerEngine
 * pull request 3012, "Summary"): fused_topk_with_score_function and
 * fused_score_for_moe_aux_loss, each with a forward and a backward, as
 * hand-written HIP kernels; the load-balancing loss that consumes the aux
 * scores (the page's fused_moe_aux_loss, "Files changed"), with the
 * tokens-per-expert counts it needs; decode-shape routing with the
 * (expert, token)-sorted expert maps of "[CUDA] Add fused decode routing,
 * single-pass finalize, and PDL overlap for NVFP4 QMoE" (onnxruntime pull
 * request 33366); and the routed top-k with the shared-expert sigmoid gate
 * of "[HIP] [Perf] Fold shared-expert gate GEMV into topk_softmax kernel"
 * (ROCm aiter pull request 5652).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout.   Every [T,E] array is row-major and contiguous: element (t, j)
 *           sits at offset t*E + j.  T = tokens, E = experts, K = top-k.
 * Memory.   All array arguments are DEVICE pointers, allocated by the
 *           caller.  The library allocates, frees and retains nothing.
 *           Every output element is written, so outputs may be
 *           uninitialised.  Inputs are read only.  Outputs must not alias
 *           inputs.  Each array must be aligned to its element size (else
 *           ROUTER_ERR_INVALID_ARG); when every array is 16-byte aligned
 *           and E is a multiple of 4 the kernels use vector loads and
 *           stores, otherwise element-wise ones (same results).
 *           router_aux_loss_fwd takes a caller-owned device workspace of
 *           router_aux_loss_workspace_bytes(T, E) bytes or more, with any
 *           contents; it is scratch for the duration of the call's kernels
 *           and must not be shared by calls that may run concurrently.
 *           router_tokens_per_expert takes one that starts zero-filled and
 *           is left zero-filled (see there).
 * Dtypes.   `dtype` (router_dtype) is the storage type of logits, probs,
 *           scores and gradients.  intermediate is always fp32 and the
 *           routing map is one byte per element holding 0 or 1 (a torch
 *           bool tensor).  expert_bias is fp32.  Arithmetic is fp32.
 * Ordering. Work is enqueued on `hip_stream` (a hipStream_t; NULL = the
 *           null stream) and is asynchronous: a return of ROUTER_OK means
 *           the kernels were launched.  No host synchronisation and no
 *           host<->device copy happens inside a call.
 * Errors.   All arguments are checked on the host before anything is
 *           launched; on any error nothing is written and the status is
 *           returned.  There is no abort and no device assert.  T == 0 is a
 *           valid no-op.  Finite logits are a precondition.
 * Threads.  Calls are reentrant; the only state is a per-device cache of
 *           device attributes and the top-k path threshold.
 */
#ifndef SCORE_FUNCTION_TOP_AMD_ROUTER_H
#define SCORE_FUNCTION_TOP_AMD_ROUTER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ROUTER_OK = 0,
    ROUTER_ERR_INVALID_ARG = 1, /* argument outside the operation's domain */
    ROUTER_ERR_OVERFLOW = 2,    /* T*E*element size overflows 64 bits      */
    ROUTER_ERR_UNSUPPORTED = 3, /* valid, but not implemented (E > 4096,
                                   expert bias with softmax)             */
    ROUTER_ERR_HIP = 4          /* a HIP call or kernel launch failed      */
} router_status;

typedef enum { ROUTER_F32 = 0, ROUTER_BF16 = 1 } router_dtype;

typedef enum { ROUTER_SOFTMAX = 0, ROUTER_SIGMOID = 1 } router_score_fn;

/* Largest number of experts the kernels handle. */
#define ROUTER_MAX_EXPERTS 4096

/*
 * router_topk_fwd -- fused_topk_with_score_function forward.
 * Passage: the fused-router page, "Performance" paragraph (the forward
 * reads logits [T,E] and writes probs [T,E] in the logits dtype, a one-byte
 * routing_map [T,E] and a four-byte intermediate [T,E]) and "Hardening"
 * (1 <= topk <= E; topk divisible by group_topk).
 *
 * Per token (row of E logits x):
 *   s      = softmax(x) over all E, or sigmoid(x) element-wise (score_fn).
 *   key    = x without expert_bias; fp32(s + expert_bias) with it.
 *   groups = if num_groups > 0: the E experts form num_groups groups of
 *            E/num_groups consecutive experts; a group scores the fp32 sum
 *            of its K/group_topk largest fp32 values s + bias (bias 0 when
 *            absent); only the group_topk best groups (ties: lower group)
 *            compete.
 *   select = the K competing experts with the largest key; ties go to the
 *            lower expert index.  Exact: the map is fully determined.
 *   p      = s, or with renorm s / (sum of s over the selected experts)
 *            (sigmoid with K == 1 keeps p = s).
 *   probs  = scaling_factor * p on the selected experts, exactly 0 elsewhere.
 *   routing_map  = 1 on the selected experts, 0 elsewhere.
 *   intermediate = s for every expert (fp32).
 * expert_bias ([E] fp32, or NULL) affects the selection only, and is only
 * accepted with the sigmoid (else ROUTER_ERR_UNSUPPORTED).
 * Checks (INVALID_ARG): T >= 0; E >= 1; 1 <= K <= E; num_groups >= 0;
 * with num_groups > 0: E % num_groups == 0, 1 <= group_topk <= num_groups,
 * K % group_topk == 0 and K / group_topk <= E / num_groups; scaling_factor
 * finite; known dtype and score_fn; non-NULL arrays when T > 0.
 * Not implemented (UNSUPPORTED), all decided on the host before any
 * launch: E > ROUTER_MAX_EXPERTS; expert_bias with the softmax;
 * num_groups > ROUTER_MAX_GROUPS (one lane of a 64-lane token scores each
 * group); with num_groups > 0, E + num_groups >
 * ROUTER_GROUP_LDS_MAX_E_PLUS_G, where the group stage's LDS copy of the
 * row (used for groups that are not 4*2^k experts, K / group_topk > 4,
 * rows of more than 1024 experts, unaligned arrays, or
 * router_set_group_stage(ROUTER_GROUP_STAGE_LDS)) and the candidate lists
 * would exceed the 160 KB of LDS a gfx950 workgroup gets -- a bound above
 * ROUTER_MAX_EXPERTS + ROUTER_MAX_GROUPS, so every grouped shape within
 * the other limits is supported.  On a device that gives a workgroup less
 * LDS (not a target of this library), the device query decides, after the
 * host checks.  The bounds follow the fused-router page, "Hardening"
 * (host-side checks, and the device's shared-memory limit in the
 * buffer decision).
 */
#define ROUTER_MAX_GROUPS 64
#define ROUTER_GROUP_LDS_MAX_E_PLUS_G 9792
router_status router_topk_fwd(const void *logits, int dtype, int64_t T,
                              int32_t E, int32_t K, int score_fn, int renorm,
                              int32_t num_groups, int32_t group_topk,
                              float scaling_factor, const float *expert_bias,
                              void *probs, uint8_t *routing_map,
                              float *intermediate, void *hip_stream);

/*
 * router_topk_bwd -- fused_topk_with_score_function backward.
 * Passage: the fused-router page, "Backward kernels" (pass 1 reduces
 * per-token sums of grad * mask * score; pass 2 writes one gradient per
 * element; inputs are the gradient, the forward's intermediate and its
 * routing map).
 *
 * Given g = grad_probs, s = intermediate and m = routing_map of one token,
 * with A = sum m s and B = sum g m s and c = scaling_factor:
 *   softmax, no renorm:    dx = c s (m g - B)
 *   softmax, renorm:       dx = c m (s / A) (g - B / A)
 *   sigmoid, no renorm or K == 1: dx = c m g s (1 - s)
 *   sigmoid, renorm, K > 1: dx = c m s (1 - s) (g - B / A) / A
 * grad_logits is written in `dtype`.  Checks as router_topk_fwd (T, E, K,
 * dtype, score_fn, scaling_factor, non-NULL arrays).
 */
router_status router_topk_bwd(const void *grad_probs,
                              const float *intermediate,
                              const uint8_t *routing_map, int dtype,
                              int64_t T, int32_t E, int32_t K, int score_fn,
                              int renorm, float scaling_factor,
                              void *grad_logits, void *hip_stream);

/*
 * router_aux_scores -- fused_score_for_moe_aux_loss forward.
 * Passage: the fused-router page, "Summary" (the aux-loss score operation)
 * and the benchmark rows "aux_loss fprop".
 *
 * Per token: s = softmax(x) or sigmoid(x).  scores = s for softmax; for the
 * sigmoid scores = s / (sum of s over all E) when renorm, else s.
 * routing_map = the K largest logits (ties: lower index).  intermediate = s.
 * scores are written in `dtype`.  Checks as router_topk_fwd (no groups,
 * no bias).
 */
router_status router_aux_scores(const void *logits, int dtype, int64_t T,
                                int32_t E, int32_t K, int score_fn,
                                int renorm, void *scores,
                                uint8_t *routing_map, float *intermediate,
                                void *hip_stream);

/*
 * router_aux_scores_bwd -- fused_score_for_moe_aux_loss backward.
 * Passage: the fused-router page, "Backward kernels" and the benchmark rows
 * "aux_loss bprop".
 *
 * The topk backward with every expert routed and no scaling factor: with
 * A = sum s and B = sum g s,
 *   softmax:                dx = s (g - B)
 *   sigmoid, renorm:        dx = s (1 - s) (g - B / A) / A
 *   sigmoid, no renorm:     dx = g s (1 - s)
 */
router_status router_aux_scores_bwd(const void *grad_scores,
                                    const float *intermediate, int dtype,
                                    int64_t T, int32_t E, int score_fn,
                                    int renorm, void *grad_logits,
                                    void *hip_stream);

/*
 * Load-balancing aux loss.  Passage: the fused-router page, "Files
 * changed": fused_moe_aux_loss, the kernel that consumes the aux scores.
 * The page does not state the loss; the one implemented is the
 * Switch-Transformer balancing loss extended to top-K routing,
 *   L = coeff * E / (N^2 K) * sum_i n_i * sum_t scores[t,i],
 * where n_i = tokens_per_expert[i] is the number of tokens routed to expert
 * i among N = total_tokens tokens (n and N may cover more tokens than the
 * T local rows of `scores`, e.g. after summing the counts over ranks).
 * Its gradient is dL/dscores[t,i] = coeff * E * n_i / (N^2 K).
 *
 * The loss is summed in fp64 in an order fixed by (T, E) alone, so it is
 * reproducible bit for bit, and rounded to fp32 once.
 */

/* Bytes of workspace router_aux_loss_fwd needs for T rows of E experts (at
 * least 256); 0 when T or E is out of range. */
size_t router_aux_loss_workspace_bytes(int64_t T, int32_t E);

/* Bytes of workspace router_tokens_per_expert needs for T rows of E
 * experts (at least 256; depends on E only, at most 65536 for E <= 4096);
 * 0 when T or E is out of range. */
size_t router_tokens_per_expert_workspace_bytes(int64_t T, int32_t E);

/*
 * router_tokens_per_expert -- tokens_per_expert[i] = number of rows t of
 * routing_map [T,E] (uint8) with a nonzero byte at (t, i); int64 [E] out.
 * Exact (integer atomics), one kernel launch.  The workspace (device
 * memory, router_tokens_per_expert_workspace_bytes(T, E) bytes or more,
 * 8-byte aligned) holds a per-expert accumulator that also counts the
 * contributions it received: it
 * must be zero-filled before its first use (e.g. allocated with zeros), and
 * every call leaves it zero-filled again, so later calls ordered after this
 * one (same stream) can reuse it; calls that may run concurrently need
 * separate workspaces.  T == 0 writes zeros.  Errors: E < 1 or T < 0
 * INVALID_ARG, E > ROUTER_MAX_EXPERTS or T > 2^32 - 1 UNSUPPORTED, T*E
 * bytes overflowing OVERFLOW; null pointers, counts or workspace not
 * 8-byte aligned, a workspace smaller than the query INVALID_ARG.
 */
router_status router_tokens_per_expert(const uint8_t *routing_map,
                                       int64_t T, int32_t E,
                                       int64_t *tokens_per_expert,
                                       void *workspace, size_t workspace_bytes,
                                       void *hip_stream);

/*
 * router_aux_loss_fwd -- loss (one fp32 on the device) of scores [T,E]
 * (`dtype`) with tokens_per_expert int64 [E] (device), total_tokens = N,
 * K = topk and coeff.  T == 0 writes 0.  Errors (INVALID_ARG): N < 1,
 * K < 1, coeff not finite, null pointers, misaligned arrays, a workspace
 * smaller than router_aux_loss_workspace_bytes(T, E) or not 8-byte
 * aligned; E > ROUTER_MAX_EXPERTS UNSUPPORTED.
 */
router_status router_aux_loss_fwd(const void *scores, int dtype, int64_t T,
                                  int32_t E, const int64_t *tokens_per_expert,
                                  int64_t total_tokens, int32_t K,
                                  float coeff, float *loss, void *workspace,
                                  size_t workspace_bytes, void *hip_stream);

/*
 * router_aux_loss_fwd_noalloc -- router_aux_loss_fwd without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 * The same kernels and the same result, bit for bit; the per-block partial
 * sums go to a buffer of ROUTER_AUX_LOSS_SCRATCH_BYTES that the library
 * holds in device memory on every GPU it runs on (until the process ends).
 * The call allocates nothing.  Calls on one GPU share that buffer, so calls
 * that may overlap on one GPU (other streams, other threads) race and must
 * not be issued; stream-ordered calls are fine.  Errors as
 * router_aux_loss_fwd; shapes whose partials exceed the buffer return
 * ROUTER_ERR_UNSUPPORTED (none with E <= ROUTER_MAX_EXPERTS: the partials
 * take at most 32768 bytes); ROUTER_ERR_HIP if the buffer's device address
 * cannot be found.
 */
#define ROUTER_AUX_LOSS_SCRATCH_BYTES 32768
router_status router_aux_loss_fwd_noalloc(const void *scores, int dtype,
                                          int64_t T, int32_t E,
                                          const int64_t *tokens_per_expert,
                                          int64_t total_tokens, int32_t K,
                                          float coeff, float *loss,
                                          void *hip_stream);

/*
 * router_aux_loss_bwd -- grad_scores [T,E] (`dtype`) =
 * grad_loss[0] * coeff * E * n_i / (N^2 K), with grad_loss one fp32 on the
 * device (the upstream gradient of the loss).  Arguments and errors as
 * router_aux_loss_fwd; needs no workspace.  T == 0 is a no-op.
 */
router_status router_aux_loss_bwd(const float *grad_loss,
                                  const int64_t *tokens_per_expert, int dtype,
                                  int64_t T, int32_t E, int64_t total_tokens,
                                  int32_t K, float coeff, void *grad_scores,
                                  void *hip_stream);

/*
 * router_route_maps -- decode-shape routing with expert maps.  Passage: the
 * onnxruntime decode-routing page, Description item 1 (one launch does the
 * softmax, the top-k and the (expert, token)-sorted expert maps for up to
 * 4 rows, 512 experts, k in {1, 2, 4, 6, 8, 10}); the map layout follows
 * the permutation maps of the TensorRT-LLM fused gather/finalize page
 * (permuted row of unpermuted index token + k * num_rows, expert of each
 * permuted row, first permuted row of each expert).
 *
 * Per token t (logits row [E] in `dtype`): s = softmax(x) or sigmoid(x);
 * slots k = 0..K-1 hold the K largest logits in descending order (ties:
 * lower expert index); topk_ids [T,K] int32 = their experts; topk_weights
 * [T,K] fp32 = s, divided by the sum of the K selected s when renorm (not
 * for sigmoid with K == 1).  The T*K pairs (t, k), unpermuted index
 * u = t + k*T, sorted by (expert, token) give the permuted order p:
 *   perm_to_unperm [T*K] int32:  u of permuted row p
 *   unperm_to_perm [T*K] int32:  p of unpermuted index u
 *   perm_expert    [T*K] int32:  expert of permuted row p
 *   expert_offsets [E+1] int64:  first permuted row of each expert;
 *                                expert_offsets[E] = T*K
 * All integer outputs are exact.  One workgroup, one wave per row.
 * Limits: 0 <= T <= ROUTER_ROUTE_MAX_ROWS, 1 <= K <= min(E,
 * ROUTER_ROUTE_MAX_K), E <= ROUTER_ROUTE_MAX_EXPERTS (beyond:
 * UNSUPPORTED).  T == 0 writes expert_offsets as zeros.  Errors
 * (INVALID_ARG): dtype, score_fn, K outside [1, E], null or misaligned
 * pointers (expert_offsets 8-byte aligned).
 */
#define ROUTER_ROUTE_MAX_ROWS 16
#define ROUTER_ROUTE_MAX_EXPERTS 1024
#define ROUTER_ROUTE_MAX_K 32
router_status router_route_maps(const void *logits, int dtype, int32_t T,
                                int32_t E, int32_t K, int score_fn, int renorm,
                                float *topk_weights, int32_t *topk_ids,
                                int32_t *perm_to_unperm,
                                int32_t *unperm_to_perm, int32_t *perm_expert,
                                int64_t *expert_offsets, void *hip_stream);

/*
 * router_topk_shared_gate -- routed softmax top-k with the shared-expert
 * sigmoid gate in the same kernel.  Passage: the aiter fused-gate page
 * (the op topk_softmax_fused_shared_gate: hidden_states, gate_weight,
 * shared_expert_scale, shared_expert_base; the unfused baseline of its
 * review: topk_softmax, then sigmoid(hidden_states @ gate_weight^T) *
 * scale into the columns after top_k, shared ids base + s).
 *
 * Per token m: slots k < K hold the K largest gating logits in descending
 * order (ties: lower expert): topk_ids[m*ld + k] = expert,
 * topk_weights[m*ld + k] = softmax score, divided by the sum of the K
 * selected scores when renorm.  Slots K + s, s < S:
 *   topk_weights[m*ld + K + s] = shared_scale * sigmoid(sum_h
 *       hidden[m,h] * gate_weight[s,h]),  topk_ids = shared_base + s.
 * gating [M,E], hidden [M,H] and gate_weight [S,H] are row-major in
 * `dtype`; the dot products accumulate in fp32.  Output rows have stride
 * ld >= K + S (elements); columns past K + S are not touched.
 * Limits: E <= ROUTER_GATE_MAX_EXPERTS, K <= ROUTER_GATE_MAX_K,
 * S <= ROUTER_GATE_MAX_SHARED (else UNSUPPORTED); any H >= 1 (16-byte
 * aligned rows with H a multiple of 8 bf16 / 4 fp32 elements take vector
 * loads).  M == 0 is a no-op.  Errors (INVALID_ARG): dtype, E, H, K
 * outside [1, E], S < 1, ld < K + S, non-finite scale, shared_base < 0 or
 * shared_base + S past INT32_MAX, null or misaligned pointers; OVERFLOW
 * when S*H elements or M rows overflow the offsets.
 */
#define ROUTER_GATE_MAX_EXPERTS 1024
#define ROUTER_GATE_MAX_K 32
#define ROUTER_GATE_MAX_SHARED 16
router_status router_topk_shared_gate(const void *gating, const void *hidden,
                                      const void *gate_weight, int dtype,
                                      int64_t M, int32_t E, int32_t H, int32_t K,
                                      int32_t S, int renorm, float shared_scale,
                                      int32_t shared_base, float *topk_weights,
                                      int32_t *topk_ids, int64_t ld,
                                      void *hip_stream);

/* Static, human-readable name of a status code. */
const char *router_status_str(router_status s);

/*
 * Top-k path threshold.  Passage: the fused-router page, "Simple kernel
 * path for small topk" and its tunable crossover variable.
 * K below the threshold selects by K rounds of a lane-group argmax; K at or
 * above it selects through a pruned candidate sort (an exact bit-wise
 * search when K exceeds the lanes per token or the pruning leaves too many
 * candidates).  Every path returns the same map.
 * ROUTER_TOPK_PATH_AUTO (the default) picks the crossover from the row
 * layout: with e elements of a row per lane, the argmax rounds run for
 * K < 5 when e <= 4, K < 4 when e <= 8 and K < 2 otherwise (where the
 * rounds measured slower than the pruned sort on MI355X).  A value in
 * [0, 4096] fixes the crossover for every shape.  The setting is read once
 * from the environment variable ROUTER_TOPK_PATH_THRESHOLD (an integer in
 * [0, 4096]; anything else, or no variable, means auto) and can be
 * overridden with router_set_topk_path_threshold, which takes
 * ROUTER_TOPK_PATH_AUTO or [0, 4096] and rejects other values with
 * ROUTER_ERR_INVALID_ARG.  router_get_topk_path_threshold returns the
 * setting (ROUTER_TOPK_PATH_AUTO in auto mode).
 */
#define ROUTER_TOPK_PATH_AUTO (-1)
int router_get_topk_path_threshold(void);
router_status router_set_topk_path_threshold(int threshold);

/*
 * Attributes of the current HIP device, for reports next to measured
 * bandwidth (no passage: bookkeeping of the measurement).  Writes the
 * compute-unit count, the peak engine clock and the peak memory clock (kHz)
 * and the memory bus width (bits) through the non-null pointers.
 * ROUTER_ERR_HIP when no device is usable.
 */
router_status router_device_query(int32_t *compute_units, int32_t *clock_khz,
                                  int32_t *memory_clock_khz, int32_t *memory_bus_bits);

/*
 * Bandwidth reference for the measurement (no passage: bookkeeping of the
 * measurement, like router_device_query).  Reads read_bytes from src and
 * writes write_bytes to dst (device pointers, 16-byte aligned, sizes
 * multiples of 16) with the router kernels' access style and no other
 * work, each thread moving units_per_thread 16-byte units (1, 2, 4 or 8)
 * with every load issued before its stores; the fastest of these at a
 * kernel's read:write mix gives the bandwidth this device reaches for that
 * mix.  The first min(read_bytes, write_bytes) bytes of dst receive src;
 * the rest arbitrary contents.  Errors: negative or unaligned sizes, null
 * or misaligned pointers, another units_per_thread INVALID_ARG.
 */
router_status router_stream_bandwidth(const void *src, int64_t read_bytes,
                                      void *dst, int64_t write_bytes,
                                      int32_t units_per_thread, void *hip_stream);

/*
 * Bandwidth reference in the forward's own access pattern (no passage:
 * bookkeeping of the measurement).  One 64-lane wave per row of E fp32
 * values (E a multiple of 256, 256..4096): the row is read whole (16 bytes
 * per lane and chunk), then written to out_a and out_b (E floats per row)
 * and one byte per element to out_map (the value's sign bit), with no
 * other work.  x, out_a, out_b: [T, E] fp32, 16-byte aligned; out_map:
 * [T, E] bytes, 4-byte aligned; device pointers.  Timing it gives the
 * bandwidth a one-row-per-wave forward reaches at best.  Errors: T < 0, E
 * out of range or not a multiple of 256, null or misaligned pointers
 * (T > 0) INVALID_ARG.
 */
router_status router_row_stream_bandwidth(const float *x, float *out_a, float *out_b,
                                          uint8_t *out_map, int64_t T, int64_t E,
                                          void *hip_stream);

/*
 * Group stage of the group-limited forward.  Passage: the fused-router
 * page, "Hardening" (group-limited routing: topk divisible by group_topk,
 * and the shared-memory limit that decides how a kernel buffers its data).
 * ROUTER_GROUP_STAGE_AUTO (default) scores the groups in registers when
 * each group of E/num_groups experts is 4*L experts with L a power of two
 * that fits the kernel's lane layout, and through an LDS scratch copy of
 * the row otherwise; ROUTER_GROUP_STAGE_LDS always takes the LDS copy
 * (and with it the bound E + num_groups <= ROUTER_GROUP_LDS_MAX_E_PLUS_G).
 * Both give the same scores, maps and outputs.  A process-wide setting;
 * other values return ROUTER_ERR_INVALID_ARG.
 */
#define ROUTER_GROUP_STAGE_AUTO 0
#define ROUTER_GROUP_STAGE_LDS 1
int router_get_group_stage(void);
router_status router_set_group_stage(int stage);

/*
 * Grid of the router's token kernels (forward, backward, aux scores, the
 * grouped forward).  Passage: the fused-router page, "Forward kernels"
 * (an occupancy-aware persistent grid, compute_persistent_grid).
 * ROUTER_GRID_FULL (the default) launches one block per group of tokens a
 * block holds; ROUTER_GRID_PERSISTENT launches at most the blocks the
 * device keeps resident for that kernel (its occupancy, from
 * hipOccupancyMaxActiveBlocksPerMultiprocessor, times the compute units,
 * read once per device and kernel), and each wave loops over further
 * token groups (the grouped forward requests the next group's logits
 * before working on the current one).  The default is the faster on
 * MI355X for the shapes measured (see the benchmark's grid study); the
 * results are the same bit for bit.  A process-wide setting; other values
 * return ROUTER_ERR_INVALID_ARG.
 */
#define ROUTER_GRID_FULL 0
#define ROUTER_GRID_PERSISTENT 1
int router_get_grid_mode(void);
router_status router_set_grid_mode(int mode);

#ifdef __cplusplus
}
#endif

#endif /* SCORE_FUNCTION_TOP_AMD_ROUTER_H */
