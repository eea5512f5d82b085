/*
 * router_oracle.c -- plain, slow fp64 CPU oracle of the fused MoE router.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file.  Its only users are the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark.  It shares no code with
 * the HIP library.
 *
 * What it computes follows "[Common] Optimize fused router forward/backward
 * kernels" (NVIDIA TransformerEngine pull request 3012):
 *   - "Summary": two operations, fused_topk_with_score_function and
 *     fused_score_for_moe_aux_loss, each with a forward and a backward.
 *   - "Performance" paragraph: the forward reads logits [T,E] and writes
 *     probs [T,E] (logits dtype), routing_map [T,E] (1 byte) and
 *     intermediate_output [T,E] (4 bytes).
 *   - "Hardening": 1 <= topk <= E, and topk divisible by group_topk.
 *   - "Backward kernels": pass 1 forms per-token sums of grad*mask*score,
 *     pass 2 writes one gradient per element.
 *   - greptile "Confidence Score": several score functions, each with and
 *     without pre-softmax.
 *   - "Files changed", fused_moe_aux_loss.cu: the load-balancing loss that
 *     consumes the aux scores (the page names the kernel, not its formula).
 * The pages give no formula.  Readings used where they are silent:
 *   softmax = exp(x - max) / sum; sigmoid = 1 / (1 + exp(-x)); expert bias
 *   and groups influence selection only; group score = sum of the q = K/Kg
 *   largest biased scores of the group; ties go to the lower index (expert
 *   or group); renormalisation divides by the sum of the selected scores
 *   (skipped for sigmoid with K == 1); the scaling factor multiplies last;
 *   intermediate = the full-row score for every mode; the aux loss is the
 *   Switch-Transformer balancing loss extended to top-K,
 *   coeff * E / (N^2 K) * sum_i n_i * sum_t scores[t,i], n_i the tokens
 *   routed to expert i, N the tokens those counts cover.
 *
 * Precision: every value is fp64, except where floating point decides an
 * integer.  With an expert bias the selection key is r = s + b evaluated in
 * fp32 (s rounded to fp32 first).  Group scores are fp32 sums of the q
 * largest fp32 values s + b (b = 0 without a bias).  So the oracle takes the
 * selection decisions in the same precision as the GPU kernels.  Without a
 * bias the expert-stage key is the raw logit, which is exact and strictly
 * monotone in the score.
 *
 * All loops go one token at a time.  The caller may split tokens over
 * threads; this file is single threaded.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_SOFTMAX 0
#define ORACLE_SIGMOID 1

/* ---------------------------------------------------------------- scores */

/* Full-row score of one token: softmax over all E logits, or the logistic
 * sigmoid of each logit. */
static void score_row(const double *x, int E, int score_fn, double *s)
{
    int j;
    if (score_fn == ORACLE_SOFTMAX) {
        double mx = x[0];
        double z = 0.0;
        for (j = 1; j < E; j++)
            if (x[j] > mx)
                mx = x[j];
        for (j = 0; j < E; j++) {
            s[j] = exp(x[j] - mx);
            z += s[j];
        }
        for (j = 0; j < E; j++)
            s[j] = s[j] / z;
    } else {
        for (j = 0; j < E; j++)
            s[j] = 1.0 / (1.0 + exp(-x[j]));
    }
}

/* ------------------------------------------------------------- selection */

/* Sort order used for every selection: larger key first, lower index first
 * among equal keys. */
typedef struct {
    double key;
    int idx;
} keyed;

static int keyed_cmp(const void *pa, const void *pb)
{
    const keyed *a = (const keyed *)pa;
    const keyed *b = (const keyed *)pb;
    if (a->key > b->key)
        return -1;
    if (a->key < b->key)
        return 1;
    if (a->idx < b->idx)
        return -1;
    if (a->idx > b->idx)
        return 1;
    return 0;
}

/*
 * Selects K experts of one token.  key[j] is the expert-stage selection key
 * of expert j.  With G > 0 groups, each group of E/G consecutive experts is
 * scored by the fp32 sum of its q = K/Kg largest group values gval[j]
 * (largest first), the Kg best groups are kept (ties to the lower group) and
 * only their experts compete.  Writes sel[j] = 1 for the chosen experts.
 * *margin receives the smallest gap between the last kept and the first
 * dropped candidate over the group stage and the expert stage (INFINITY when
 * nothing was dropped).  work needs E entries.
 */
static void select_row(const double *key, const double *gval, int E, int K,
                       int G, int Kg, uint8_t *sel, keyed *work,
                       double *margin)
{
    int j, g, n = 0;
    double gap = INFINITY;
    uint8_t allowed_group[4096];

    memset(sel, 0, (size_t)E);
    if (G > 0) {
        int per = E / G;
        int q = K / Kg;
        keyed gs[4096];
        for (g = 0; g < G; g++) {
            float h = 0.0f;
            int t;
            for (j = 0; j < per; j++) {
                work[j].key = gval[g * per + j];
                work[j].idx = g * per + j;
            }
            qsort(work, (size_t)per, sizeof(keyed), keyed_cmp);
            for (t = 0; t < q; t++)
                h = h + (float)work[t].key;
            gs[g].key = (double)h;
            gs[g].idx = g;
        }
        qsort(gs, (size_t)G, sizeof(keyed), keyed_cmp);
        for (g = 0; g < G; g++)
            allowed_group[gs[g].idx] = (uint8_t)(g < Kg);
        if (Kg < G && gs[Kg - 1].key - gs[Kg].key < gap)
            gap = gs[Kg - 1].key - gs[Kg].key;
        for (j = 0; j < E; j++) {
            if (allowed_group[j / per]) {
                work[n].key = key[j];
                work[n].idx = j;
                n++;
            }
        }
    } else {
        for (j = 0; j < E; j++) {
            work[n].key = key[j];
            work[n].idx = j;
            n++;
        }
    }
    qsort(work, (size_t)n, sizeof(keyed), keyed_cmp);
    for (j = 0; j < K; j++)
        sel[work[j].idx] = 1;
    if (K < n && work[K - 1].key - work[K].key < gap)
        gap = work[K - 1].key - work[K].key;
    if (margin)
        *margin = gap;
}

/* ------------------------------------------------------------- topk fwd */

/*
 * fused_topk_with_score_function forward.
 *   x [T,E]        logits (fp64 promotion of the fp32/bf16 input)
 *   bias [E]       expert bias or NULL (sigmoid only); selection only
 *   probs [T,E]    c * p_j on the selected experts, exactly 0 elsewhere
 *   map [T,E]      1 on the selected experts, else 0
 *   inter [T,E]    the full-row score s
 *   margin [T]     optional, see select_row
 * p_j = s_j, or s_j / sum_{k selected} s_k when renorm is set (for sigmoid
 * only when K > 1).
 * Returns 0, or -1 for arguments outside the operation's domain.
 */
int oracle_topk_fwd(const double *x, int64_t T, int E, int K, int score_fn,
                    int renorm, int G, int Kg, double c, const double *bias,
                    double *probs, uint8_t *map, double *inter, double *margin)
{
    int64_t t;
    int j;
    double *s, *key, *gval;
    keyed *work;

    if (T < 0 || E < 1 || K < 1 || K > E || E > 1 << 20)
        return -1;
    if (G > 0 && (E % G != 0 || Kg < 1 || Kg > G || K % Kg != 0 ||
                  K / Kg > E / G || G > 4096))
        return -1;
    if (bias && score_fn != ORACLE_SIGMOID)
        return -1;
    s = (double *)malloc(sizeof(double) * (size_t)E);
    key = (double *)malloc(sizeof(double) * (size_t)E);
    gval = (double *)malloc(sizeof(double) * (size_t)E);
    work = (keyed *)malloc(sizeof(keyed) * (size_t)E);
    if (!s || !key || !gval || !work) {
        free(s);
        free(key);
        free(gval);
        free(work);
        return -1;
    }
    for (t = 0; t < T; t++) {
        const double *xr = x + t * E;
        double *pr = probs + t * E;
        uint8_t *mr = map + t * E;
        double denom = 1.0;

        score_row(xr, E, score_fn, s);
        for (j = 0; j < E; j++) {
            float b = bias ? (float)bias[j] : 0.0f;
            gval[j] = (double)((float)s[j] + b);
            key[j] = bias ? gval[j] : xr[j];
        }
        select_row(key, gval, E, K, G, Kg, mr, work,
                   margin ? margin + t : NULL);
        if (renorm && (score_fn == ORACLE_SOFTMAX || K > 1)) {
            denom = 0.0;
            for (j = 0; j < E; j++)
                if (mr[j])
                    denom += s[j];
        }
        for (j = 0; j < E; j++) {
            pr[j] = mr[j] ? c * (s[j] / denom) : 0.0;
            inter[t * E + j] = s[j];
        }
    }
    free(s);
    free(key);
    free(gval);
    free(work);
    return 0;
}

/*
 * The selection step alone, for keys and group values given per token:
 *   key [T,E]    expert-stage selection keys
 *   gval [T,E]   group values (fp32 values promoted to fp64); read only
 *                when G > 0
 *   map [T,E]    1 on the selected experts, else 0
 *   margin [T]   optional, as in select_row
 * The same rule as the forward (group score = fp32 sum of the q = K/Kg
 * largest group values, largest first; Kg best groups, ties to the lower
 * group; then the K largest keys among their experts, ties to the lower
 * expert).  Lets a caller decide a selection from keys computed elsewhere,
 * e.g. from another implementation's fp32 scores.
 * Returns 0, or -1 for arguments outside the operation's domain.
 */
int oracle_select(const double *key, const double *gval, int64_t T, int E,
                  int K, int G, int Kg, uint8_t *map, double *margin)
{
    int64_t t;
    keyed *work;

    if (T < 0 || E < 1 || K < 1 || K > E || E > 1 << 20)
        return -1;
    if (G > 0 && (E % G != 0 || Kg < 1 || Kg > G || K % Kg != 0 ||
                  K / Kg > E / G || G > 4096 || !gval))
        return -1;
    work = (keyed *)malloc(sizeof(keyed) * (size_t)E);
    if (!work)
        return -1;
    for (t = 0; t < T; t++)
        select_row(key + t * E, G > 0 ? gval + t * E : NULL, E, K, G, Kg,
                   map + t * E, work, margin ? margin + t : NULL);
    free(work);
    return 0;
}

/* ------------------------------------------------------------- topk bwd */

/*
 * fused_topk_with_score_function backward: gradient of sum_j g_j probs_j
 * with respect to the logits, from the forward's intermediate s and map m.
 * Pass 1 forms A = sum_j m_j s_j and B = sum_j g_j m_j s_j; pass 2 writes:
 *   softmax, no renorm:   dx_i = c s_i (m_i g_i - B)
 *   softmax, renorm:      dx_i = c m_i (s_i / A) (g_i - B / A)
 *   sigmoid, no renorm:   dx_i = c m_i g_i s_i (1 - s_i)
 *   sigmoid, renorm, K>1: dx_i = c m_i s_i (1 - s_i) (g_i - B / A) / A
 */
int oracle_topk_bwd(const double *g, const double *s, const uint8_t *m,
                    int64_t T, int E, int K, int score_fn, int renorm,
                    double c, double *dx)
{
    int64_t t;
    int i;

    if (T < 0 || E < 1 || K < 1 || K > E)
        return -1;
    for (t = 0; t < T; t++) {
        const double *gr = g + t * E;
        const double *sr = s + t * E;
        const uint8_t *mr = m + t * E;
        double *dr = dx + t * E;
        double A = 0.0, B = 0.0;

        for (i = 0; i < E; i++) {
            if (mr[i]) {
                A += sr[i];
                B += gr[i] * sr[i];
            }
        }
        for (i = 0; i < E; i++) {
            double mi = mr[i] ? 1.0 : 0.0;
            if (score_fn == ORACLE_SOFTMAX && !renorm)
                dr[i] = c * sr[i] * (mi * gr[i] - B);
            else if (score_fn == ORACLE_SOFTMAX)
                dr[i] = c * mi * (sr[i] / A) * (gr[i] - B / A);
            else if (!renorm || K == 1)
                dr[i] = c * mi * gr[i] * sr[i] * (1.0 - sr[i]);
            else
                dr[i] = c * mi * sr[i] * (1.0 - sr[i]) * (gr[i] - B / A) / A;
        }
    }
    return 0;
}

/* -------------------------------------------------------------- aux fwd */

/*
 * fused_score_for_moe_aux_loss forward: full-row scores for the aux loss.
 *   scores [T,E]  softmax s, or for sigmoid s / sum_j s_j (renorm set) or s
 *   map [T,E]     top-K experts by raw logit, ties to the lower index
 *   inter [T,E]   the full-row score s (softmax, or the raw sigmoid)
 */
int oracle_aux_fwd(const double *x, int64_t T, int E, int K, int score_fn,
                   int renorm, double *scores, uint8_t *map, double *inter)
{
    int64_t t;
    int j;
    double *s;
    keyed *work;

    if (T < 0 || E < 1 || K < 1 || K > E)
        return -1;
    s = (double *)malloc(sizeof(double) * (size_t)E);
    work = (keyed *)malloc(sizeof(keyed) * (size_t)E);
    if (!s || !work) {
        free(s);
        free(work);
        return -1;
    }
    for (t = 0; t < T; t++) {
        const double *xr = x + t * E;
        double z = 1.0;

        score_row(xr, E, score_fn, s);
        select_row(xr, xr, E, K, 0, 0, map + t * E, work, NULL);
        if (score_fn == ORACLE_SIGMOID && renorm) {
            z = 0.0;
            for (j = 0; j < E; j++)
                z += s[j];
        }
        for (j = 0; j < E; j++) {
            scores[t * E + j] = s[j] / z;
            inter[t * E + j] = s[j];
        }
    }
    free(s);
    free(work);
    return 0;
}

/* -------------------------------------------------------------- aux bwd */

/*
 * fused_score_for_moe_aux_loss backward: the topk backward with every
 * expert routed and no scaling factor.
 *   softmax:              dx_i = s_i (g_i - B)
 *   sigmoid, normalised:  dx_i = s_i (1 - s_i) (g_i - B / A) / A
 *   sigmoid, raw:         dx_i = g_i s_i (1 - s_i)
 * with A = sum_j s_j and B = sum_j g_j s_j.
 */
int oracle_aux_bwd(const double *g, const double *s, int64_t T, int E,
                   int score_fn, int renorm, double *dx)
{
    int64_t t;
    int i;

    if (T < 0 || E < 1)
        return -1;
    for (t = 0; t < T; t++) {
        const double *gr = g + t * E;
        const double *sr = s + t * E;
        double *dr = dx + t * E;
        double A = 0.0, B = 0.0;

        for (i = 0; i < E; i++) {
            A += sr[i];
            B += gr[i] * sr[i];
        }
        for (i = 0; i < E; i++) {
            if (score_fn == ORACLE_SOFTMAX)
                dr[i] = sr[i] * (gr[i] - B);
            else if (renorm)
                dr[i] = sr[i] * (1.0 - sr[i]) * (gr[i] - B / A) / A;
            else
                dr[i] = gr[i] * sr[i] * (1.0 - sr[i]);
        }
    }
    return 0;
}

/* ------------------------------------------------------- aux loss scalar */

/*
 * Tokens routed to each expert: counts[i] = sum over tokens of map[t,i].
 */
int oracle_tokens_per_expert(const uint8_t *map, int64_t T, int E,
                             int64_t *counts)
{
    int64_t t;
    int i;

    if (T < 0 || E < 1)
        return -1;
    for (i = 0; i < E; i++)
        counts[i] = 0;
    for (t = 0; t < T; t++)
        for (i = 0; i < E; i++)
            counts[i] += map[t * E + i] ? 1 : 0;
    return 0;
}

/*
 * Load-balancing loss over the aux scores (the router page names the
 * fused_moe_aux_loss kernel but not its formula; reading: the Switch
 * Transformer balancing loss extended to top-K routing):
 *   L = coeff * E / (N^2 K) * sum_i counts[i] * sum_t scores[t,i]
 * i.e. coeff * E * sum_i f_i P_i with f_i = counts[i] / (N K) and
 * P_i = sum_t scores[t,i] / N.  N = total_tokens (the tokens the counts and
 * the normalisation refer to).  *loss receives L.
 */
int oracle_aux_loss(const double *scores, const int64_t *counts, int64_t T,
                    int E, int64_t N, int K, double coeff, double *loss)
{
    int64_t t;
    int i;
    double acc = 0.0;
    double *col;

    if (T < 0 || E < 1 || N < 1 || K < 1)
        return -1;
    col = calloc((size_t)E, sizeof(double));
    if (!col)
        return -1;
    /* column sums, each over the tokens in order (row-major walk) */
    for (t = 0; t < T; t++)
        for (i = 0; i < E; i++)
            col[i] += scores[t * E + i];
    for (i = 0; i < E; i++)
        acc += (double)counts[i] * col[i];
    free(col);
    *loss = coeff * (double)E / ((double)N * (double)N * (double)K) * acc;
    return 0;
}

/*
 * Gradient of the loss above with respect to the scores, times grad_loss:
 *   grad_scores[t,i] = grad_loss * coeff * E * counts[i] / (N^2 K)
 * (the counts are integers and carry no gradient).
 */
int oracle_aux_loss_bwd(double grad_loss, const int64_t *counts, int64_t T,
                        int E, int64_t N, int K, double coeff,
                        double *grad_scores)
{
    int64_t t;
    int i;

    if (T < 0 || E < 1 || N < 1 || K < 1)
        return -1;
    for (t = 0; t < T; t++)
        for (i = 0; i < E; i++)
            grad_scores[t * E + i] = grad_loss * coeff * (double)E *
                                     (double)counts[i] /
                                     ((double)N * (double)N * (double)K);
    return 0;
}

/* ------------------------------------------- decode routing + expert maps */

typedef struct {
    int expert;
    int token;
    int unpermuted; /* token + k * T */
} pair_rec;

static int pair_cmp(const void *pa, const void *pb)
{
    const pair_rec *a = (const pair_rec *)pa, *b = (const pair_rec *)pb;
    if (a->expert != b->expert)
        return a->expert < b->expert ? -1 : 1;
    if (a->token != b->token)
        return a->token < b->token ? -1 : 1;
    return 0;
}

/*
 * Decode-shape routing with expert maps (the onnxruntime page's fused
 * softmax + top-k + expert-map kernel; the map layout of the TensorRT-LLM
 * page's permutation maps).  Per token t: scores s = score_fn(x), the K
 * experts with the largest logits in descending order (ties: lower index),
 * ids[t*K + k] and weights[t*K + k] = s / (sum of the K selected scores)
 * when renorm (skipped for sigmoid with K == 1), else s.  The T*K
 * (token, slot) pairs, unpermuted index u = t + k*T, sorted by (expert,
 * token) give the permuted order p: perm_to_unperm[p] = u,
 * unperm_to_perm[u] = p, perm_expert[p] = expert, and expert_offsets[e] =
 * number of pairs routed to experts below e (e = 0..E, last = T*K).
 */
int oracle_route_maps(const double *x, int T, int E, int K, int score_fn,
                      int renorm, double *weights, int32_t *ids,
                      int32_t *perm_to_unperm, int32_t *unperm_to_perm,
                      int32_t *perm_expert, int64_t *expert_offsets)
{
    int t, k, j, p, n;
    double *s;
    keyed *work;
    pair_rec *pairs;

    if (T < 0 || E < 1 || K < 1 || K > E)
        return -1;
    n = T * K;
    s = (double *)malloc(sizeof(double) * (size_t)E);
    work = (keyed *)malloc(sizeof(keyed) * (size_t)E);
    pairs = (pair_rec *)malloc(sizeof(pair_rec) * (size_t)(n > 0 ? n : 1));
    if (!s || !work || !pairs) {
        free(s);
        free(work);
        free(pairs);
        return -1;
    }
    for (t = 0; t < T; t++) {
        const double *xr = x + (int64_t)t * E;
        double denom = 1.0;

        score_row(xr, E, score_fn, s);
        for (j = 0; j < E; j++) {
            work[j].key = xr[j];
            work[j].idx = j;
        }
        qsort(work, (size_t)E, sizeof(keyed), keyed_cmp);
        if (renorm && (score_fn == ORACLE_SOFTMAX || K > 1)) {
            denom = 0.0;
            for (k = 0; k < K; k++)
                denom += s[work[k].idx];
        }
        for (k = 0; k < K; k++) {
            ids[t * K + k] = work[k].idx;
            weights[t * K + k] = s[work[k].idx] / denom;
            pairs[t + k * T].expert = work[k].idx;
            pairs[t + k * T].token = t;
            pairs[t + k * T].unpermuted = t + k * T;
        }
    }
    qsort(pairs, (size_t)n, sizeof(pair_rec), pair_cmp);
    for (p = 0; p < n; p++) {
        perm_to_unperm[p] = pairs[p].unpermuted;
        unperm_to_perm[pairs[p].unpermuted] = p;
        perm_expert[p] = pairs[p].expert;
    }
    for (j = 0, p = 0; j <= E; j++) {
        while (p < n && pairs[p].expert < j)
            p++;
        expert_offsets[j] = p;
    }
    free(s);
    free(work);
    free(pairs);
    return 0;
}

/* --------------------------------------- routed top-k + shared-expert gate */

/*
 * Routed softmax top-k with the shared-expert sigmoid gate folded in (the
 * aiter page "[HIP] [Perf] Fold shared-expert gate GEMV into topk_softmax
 * kernel": routed top-k weights and ids, then for each shared expert s the
 * gate scale * sigmoid(hidden_states[m,:] . gate_weight[s,:]) with id
 * shared_base + s, in the columns after the K routed ones).  Per token m:
 *   slots k < K: the K largest gating logits in descending order (ties:
 *   lower expert), weight = softmax score, divided by the sum of the K
 *   selected scores when renorm;
 *   slots K + s: weight = scale / (1 + exp(-sum_h hs[m,h] * gw[s,h])),
 *   id = shared_base + s.
 * weights/ids rows have stride ld >= K + S.
 */
int oracle_topk_shared_gate(const double *x, const double *hs, const double *gw,
                            int64_t M, int E, int H, int K, int S, int renorm,
                            double scale, int shared_base, int64_t ld,
                            double *weights, int32_t *ids)
{
    int64_t m;
    int j, k, s, h;
    double *sc;
    keyed *work;

    if (M < 0 || E < 1 || H < 1 || K < 1 || K > E || S < 1 || ld < K + S)
        return -1;
    sc = (double *)malloc(sizeof(double) * (size_t)E);
    work = (keyed *)malloc(sizeof(keyed) * (size_t)E);
    if (!sc || !work) {
        free(sc);
        free(work);
        return -1;
    }
    for (m = 0; m < M; m++) {
        const double *xr = x + m * E;
        double denom = 1.0;

        score_row(xr, E, ORACLE_SOFTMAX, sc);
        for (j = 0; j < E; j++) {
            work[j].key = xr[j];
            work[j].idx = j;
        }
        qsort(work, (size_t)E, sizeof(keyed), keyed_cmp);
        if (renorm) {
            denom = 0.0;
            for (k = 0; k < K; k++)
                denom += sc[work[k].idx];
        }
        for (k = 0; k < K; k++) {
            weights[m * ld + k] = sc[work[k].idx] / denom;
            ids[m * ld + k] = work[k].idx;
        }
        for (s = 0; s < S; s++) {
            double dot = 0.0;
            for (h = 0; h < H; h++)
                dot += hs[m * H + h] * gw[(int64_t)s * H + h];
            weights[m * ld + K + s] = scale / (1.0 + exp(-dot));
            ids[m * ld + K + s] = shared_base + s;
        }
    }
    free(sc);
    free(work);
    return 0;
}
