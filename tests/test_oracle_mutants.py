"""Plants plausible mistakes in copies of the oracle source (on the CPU) and
checks that at least one pin catches each one.  A mutant that survives
every pin means the pins do not cover that part of the oracle."""
import os

import pytest

import oracle
from oracle import build as obuild
from oracle_pins import PINS

# (name, text in router_oracle.c, replacement, which occurrence)
MUTANTS = [
    ("no_max_subtraction", "s[j] = exp(x[j] - mx);", "s[j] = exp(x[j]);", 0),
    ("softmax_not_normalised", "s[j] = s[j] / z;", "s[j] = s[j] / (z + 1e-3);", 0),
    ("sigmoid_sign", "s[j] = 1.0 / (1.0 + exp(-x[j]));",
     "s[j] = 1.0 / (1.0 + exp(x[j]));", 0),
    ("ties_to_higher_index",
     "if (a->idx < b->idx)\n        return -1;\n    if (a->idx > b->idx)\n        return 1;",
     "if (a->idx > b->idx)\n        return -1;\n    if (a->idx < b->idx)\n        return 1;", 0),
    ("select_smallest", "if (a->key > b->key)\n        return -1;\n    if (a->key < b->key)\n        return 1;",
     "if (a->key < b->key)\n        return -1;\n    if (a->key > b->key)\n        return 1;", 0),
    ("group_keeps_last_not_sum", "h = h + (float)work[t].key;",
     "h = (float)work[t].key;", 0),
    ("group_keeps_one_more", "(uint8_t)(g < Kg)", "(uint8_t)(g <= Kg)", 0),
    ("group_scored_on_logits", "work[j].key = gval[g * per + j];",
     "work[j].key = key[g * per + j];", 0),
    ("group_q_is_one", "int q = K / Kg;", "int q = 1;", 0),
    ("bias_subtracted", "gval[j] = (double)((float)s[j] + b);",
     "gval[j] = (double)((float)s[j] - b);", 0),
    ("bias_in_probs", "pr[j] = mr[j] ? c * (s[j] / denom) : 0.0;",
     "pr[j] = mr[j] ? c * ((s[j] + (bias ? bias[j] : 0.0)) / denom) : 0.0;", 0),
    ("renorm_over_all", "if (mr[j])\n                    denom += s[j];",
     "denom += s[j];", 0),
    ("sigmoid_k1_renorm", "(score_fn == ORACLE_SOFTMAX || K > 1)",
     "(score_fn == ORACLE_SOFTMAX || K > 0)", 0),
    ("no_scale_in_probs", "pr[j] = mr[j] ? c * (s[j] / denom) : 0.0;",
     "pr[j] = mr[j] ? (s[j] / denom) : 0.0;", 0),
    ("inter_holds_probs", "inter[t * E + j] = s[j];\n        }\n    }\n    free(s);\n    free(key);",
     "inter[t * E + j] = pr[j];\n        }\n    }\n    free(s);\n    free(key);", 0),
    ("row_offset_dropped", "const double *xr = x + t * E;", "const double *xr = x;", 0),
    ("bwd_softmax_mask_dropped", "c * sr[i] * (mi * gr[i] - B)", "c * sr[i] * (gr[i] - B)", 0),
    ("bwd_softmax_sign", "c * sr[i] * (mi * gr[i] - B)", "c * sr[i] * (mi * gr[i] + B)", 0),
    ("bwd_softmax_renorm_B", "c * mi * (sr[i] / A) * (gr[i] - B / A)",
     "c * mi * (sr[i] / A) * (gr[i] - B)", 0),
    ("bwd_softmax_renorm_A", "c * mi * (sr[i] / A) * (gr[i] - B / A)",
     "c * mi * sr[i] * (gr[i] - B / A)", 0),
    ("bwd_sigmoid_derivative", "c * mi * gr[i] * sr[i] * (1.0 - sr[i])",
     "c * mi * gr[i] * sr[i]", 0),
    ("bwd_sigmoid_no_scale", "c * mi * gr[i] * sr[i] * (1.0 - sr[i])",
     "mi * gr[i] * sr[i] * (1.0 - sr[i])", 0),
    ("bwd_sigmoid_renorm_B", "c * mi * sr[i] * (1.0 - sr[i]) * (gr[i] - B / A) / A",
     "c * mi * sr[i] * (1.0 - sr[i]) * (gr[i] - B) / A", 0),
    ("bwd_sigmoid_renorm_A", "c * mi * sr[i] * (1.0 - sr[i]) * (gr[i] - B / A) / A",
     "c * mi * sr[i] * (1.0 - sr[i]) * (gr[i] - B / A)", 0),
    ("bwd_B_unweighted", "B += gr[i] * sr[i];", "B += gr[i];", 0),
    ("bwd_A_unmasked", "if (mr[i]) {\n                A += sr[i];",
     "A += sr[i];\n            if (mr[i]) {", 0),
    ("bwd_sigmoid_k1_rule", "else if (!renorm || K == 1)", "else if (!renorm)", 0),
    ("aux_not_normalised", "z += s[j];", "z += 0.0;", 0),
    ("aux_map_wrong_k", "select_row(xr, xr, E, K, 0, 0, map + t * E, work, NULL);",
     "select_row(xr, xr, E, K > 1 ? K - 1 : K, 0, 0, map + t * E, work, NULL);", 0),
    ("aux_bwd_softmax_B", "dr[i] = sr[i] * (gr[i] - B);", "dr[i] = sr[i] * gr[i];", 0),
    ("aux_bwd_sigmoid_derivative", "dr[i] = sr[i] * (1.0 - sr[i]) * (gr[i] - B / A) / A;",
     "dr[i] = sr[i] * (gr[i] - B / A) / A;", 0),
    ("aux_bwd_B_unweighted", "B += gr[i] * sr[i];", "B += sr[i];", 1),
    ("aux_bwd_raw_sigmoid", "dr[i] = gr[i] * sr[i] * (1.0 - sr[i]);",
     "dr[i] = gr[i] * sr[i];", 0),
    ("tokens_row_offset", "counts[i] += map[t * E + i] ? 1 : 0;",
     "counts[i] += map[i] ? 1 : 0;", 0),
    ("tokens_not_reset", "counts[i] = 0;", "counts[i] = counts[i];", 0),
    ("loss_no_E", "*loss = coeff * (double)E /", "*loss = coeff * 1.0 /", 0),
    ("loss_N_not_squared", "/ ((double)N * (double)N * (double)K) * acc;",
     "/ ((double)N * (double)K) * acc;", 0),
    ("loss_no_K", "/ ((double)N * (double)N * (double)K) * acc;",
     "/ ((double)N * (double)N) * acc;", 0),
    ("loss_counts_ignored", "acc += (double)counts[i] * col[i];", "acc += col[i];", 0),
    ("loss_col_row_offset", "col[i] += scores[t * E + i];", "col[i] += scores[i];", 0),
    ("loss_bwd_counts_ignored", "(double)counts[i] /\n", "1.0 /\n", 0),
    ("loss_bwd_grad_dropped", "grad_scores[t * E + i] = grad_loss * coeff",
     "grad_scores[t * E + i] = coeff", 0),
    ("maps_sort_token_first", "if (a->expert != b->expert)\n        return a->expert < b->expert ? -1 : 1;\n    if (a->token != b->token)\n        return a->token < b->token ? -1 : 1;",
     "if (a->token != b->token)\n        return a->token < b->token ? -1 : 1;\n    if (a->expert != b->expert)\n        return a->expert < b->expert ? -1 : 1;", 0),
    ("maps_unpermuted_token_major", "pairs[t + k * T].unpermuted = t + k * T;",
     "pairs[t + k * T].unpermuted = t * K + k;", 0),
    ("maps_offsets_inclusive", "while (p < n && pairs[p].expert < j)",
     "while (p < n && pairs[p].expert <= j)", 0),
    ("maps_weights_first_only", "denom += s[work[k].idx];", "denom += s[work[0].idx];", 0),
    ("maps_inverse_swapped", "unperm_to_perm[pairs[p].unpermuted] = p;",
     "unperm_to_perm[p] = pairs[p].unpermuted;", 0),
    ("maps_ids_unsorted_slot", "ids[t * K + k] = work[k].idx;",
     "ids[t * K + k] = work[K - 1 - k].idx;", 0),
    ("gate_sign", "weights[m * ld + K + s] = scale / (1.0 + exp(-dot));",
     "weights[m * ld + K + s] = scale / (1.0 + exp(dot));", 0),
    ("gate_scale_dropped", "weights[m * ld + K + s] = scale / (1.0 + exp(-dot));",
     "weights[m * ld + K + s] = 1.0 / (1.0 + exp(-dot));", 0),
    ("gate_weight_row", "dot += hs[m * H + h] * gw[(int64_t)s * H + h];",
     "dot += hs[m * H + h] * gw[h];", 0),
    ("gate_hidden_row", "dot += hs[m * H + h] * gw[(int64_t)s * H + h];",
     "dot += hs[h] * gw[(int64_t)s * H + h];", 0),
    ("gate_id_base", "ids[m * ld + K + s] = shared_base + s;",
     "ids[m * ld + K + s] = shared_base + s + 1;", 0),
    ("gate_routed_not_renormed", "denom += sc[work[k].idx];", "denom += sc[work[0].idx];", 0),
    ("margin_sign", "gap = work[K - 1].key - work[K].key;",
     "gap = work[K].key - work[K - 1].key;", 0),
]


def _mutate(src, old, new, occ):
    at = -1
    for _ in range(occ + 1):
        at = src.index(old, at + 1)
    return src[:at] + new + src[at + len(old):]


def test_mutation_sites_exist():
    src = open(obuild.SRC).read()
    for name, old, _, occ in MUTANTS:
        assert src.count(old) > occ, name


@pytest.mark.parametrize("name,old,new,occ", MUTANTS,
                         ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, occ, tmp_path):
    src = open(obuild.SRC).read()
    path = tmp_path / f"mut_{name}.c"
    path.write_text(_mutate(src, old, new, occ))
    lib = oracle._load(obuild.build(str(path), str(tmp_path / f"lib_{name}.so")))
    caught = []
    for pin in PINS:
        try:
            pin(lib)
        except Exception as e:  # noqa: BLE001 - any failure catches it
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"mutant {name} survived every pin"
