"""The GPU parity tests' comparison rules, exercised on the CPU: a simulated
correct GPU (fp32 scores a few ulp off the oracle's, its map decided on its
own keys) passes them, and planted mistakes in its outputs fail them.  The
"GPU" arrays here come from the oracle plus seeded perturbations; no GPU
and no HIP library are involved."""
import numpy as np
import pytest

import oracle
from gpu_support import (MAX_DIFFER_ROWS, check_forward, check_near_tie, decision_inputs,
                         group_scores32)
from score_function_top_amd import synth


def _case(T, E, K, G, Kg, sf, bias, dtype=synth.F32, seed=3):
    return synth.Workload(name=f"rules_{E}x{K}_g{G}", T=T, E=E, K=K, score_fn=sf, renorm=True,
                          num_groups=G, group_topk=Kg, scaling_factor=2.5, dtype=dtype,
                          bias_range=bias, seed_logits=seed, seed_grad=seed + 1,
                          seed_bias=seed + 2, seed_aux_grad=seed + 3)


def _oracle(wl):
    _, x64 = wl.logits()
    bias = wl.bias()
    P, M, S, margin = oracle.topk_fwd(x64, wl.K, wl.score_fn, wl.renorm, wl.num_groups,
                                      wl.group_topk, wl.scaling_factor,
                                      None if bias is None else bias.astype(np.float64),
                                      threads=4)
    return x64, bias, P, M, S, margin


def _simulated_gpu(wl, x64, bias, S, ulps, seed=0):
    """fp32 scores off by up to `ulps` ulp, the selection decided on them,
    probs consistent with that selection."""
    rng = np.random.default_rng(seed)
    s32 = S.astype(np.float32)
    step = rng.integers(-ulps, ulps + 1, s32.shape).astype(np.int32)
    gi = (s32.view(np.int32) + step).view(np.float32).astype(np.float64)
    key, gv = decision_inputs(gi, x64, bias)
    gm, _ = oracle.select(key, wl.K, wl.num_groups, wl.group_topk, gv, threads=4)
    m = gm.astype(bool)
    denom = np.where(m, gi, 0.0).sum(1, keepdims=True)
    gp = np.where(m, wl.scaling_factor * gi / denom, 0.0)
    return gp, gm.astype(np.float64), gi


CASES = [(700, 256, 8, 8, 4, synth.SIGMOID, 0.05), (500, 512, 22, 0, 0, synth.SIGMOID, 0.1),
         (400, 1024, 8, 8, 4, synth.SOFTMAX, 0.0), (300, 96, 12, 12, 4, synth.SIGMOID, 0.0)]


@pytest.mark.parametrize("T,E,K,G,Kg,sf,b", CASES)
def test_correct_selection_passes(T, E, K, G, Kg, sf, b):
    wl = _case(T, E, K, G, Kg, sf, b)
    x64, bias, P, M, S, margin = _oracle(wl)
    gp, gm, gi = _simulated_gpu(wl, x64, bias, S, ulps=3)
    near, differ = check_forward(wl, x64, bias, gp, gm, gi, P, M, S, margin)
    assert set(differ) <= set(near)


def test_band_is_scale_aware():
    """Softmax group scores near q/E: the measured band is a few ulp of
    them, far below the old absolute 2e-6."""
    wl = _case(400, 1024, 8, 8, 4, synth.SOFTMAX, 0.0)
    x64, bias, P, M, S, margin = _oracle(wl)
    gp, gm, gi = _simulated_gpu(wl, x64, bias, S, ulps=3)
    key_g, gv_g = decision_inputs(gi, x64, bias)
    key_o, gv_o = decision_inputs(S, x64, bias)
    h_o = group_scores32(gv_o.astype(np.float32), 8, 2)
    e = np.abs(group_scores32(gv_g.astype(np.float32), 8, 2) - h_o).max(1)
    assert (e <= 2.0 ** -19 * h_o.max(1)).all() and e.max() < 2e-8
    near, _ = check_forward(wl, x64, bias, gp, gm, gi, P, M, S, margin)
    assert near.size <= 2


def test_planted_tie_rule_reversed_fails():
    """A map that breaks an exact tie toward the higher index fails decision
    parity (integer logits make groups and experts tie)."""
    wl = _case(64, 64, 6, 4, 2, synth.SIGMOID, 0.0)
    x64 = np.random.default_rng(5).integers(0, 3, (64, 64)).astype(np.float64)
    P, M, S, margin = oracle.topk_fwd(x64, 6, synth.SIGMOID, True, 4, 2, 2.5, threads=4)
    bad = M.copy().astype(np.float64)
    # row with an exact tie at the K-th key inside a kept group: swap the
    # lower-index winner for the higher-index loser
    swapped = False
    for t in range(64):
        kept = M[t].reshape(4, 16).any(1).repeat(16)
        sel = np.nonzero(M[t])[0]
        kth = x64[t, sel].min()
        losers = [j for j in range(64) if kept[j] and not M[t, j] and x64[t, j] == kth]
        winners = [j for j in sel if x64[t, j] == kth]
        if losers and winners:
            bad[t, winners[-1]], bad[t, losers[0]] = 0, 1
            swapped = True
            break
    assert swapped
    with pytest.raises(AssertionError, match="own keys"):
        check_forward(wl, x64, None, P, bad, S, P, M, S, margin)


def test_planted_large_score_error_fails():
    wl = _case(300, 256, 8, 8, 4, synth.SIGMOID, 0.05)
    x64, bias, P, M, S, margin = _oracle(wl)
    gp, gm, gi = _simulated_gpu(wl, x64, bias, S, ulps=3)
    gi = gi.copy()
    gi[7] *= 1.0 + 1e-5          # one row 10 ppm off: keys outside the relative bound
    key, gv = decision_inputs(gi, x64, bias)
    gm, _ = oracle.select(key, wl.K, 8, 4, gv, threads=4)
    with pytest.raises(AssertionError):
        check_forward(wl, x64, bias, gp, gm.astype(np.float64), gi, P, M, S, margin)


def test_planted_dropped_must_keep_group_fails():
    """A selection that skips the best group (well clear of the band) for
    the (Kg+1)-th fails the near-tie validity check."""
    wl = _case(50, 256, 8, 8, 4, synth.SIGMOID, 0.05)
    x64, bias, P, M, S, margin = _oracle(wl)
    key_o, gv_o = decision_inputs(S, x64, bias)
    h = group_scores32(gv_o.astype(np.float32), 8, 2)
    t = 0
    order = np.argsort(-h[t], kind="stable")
    groups = order[1:5]                        # ranks 2..Kg+1, the best one dropped
    allowed = np.zeros(256, bool)
    for g in groups:
        allowed[g * 32:(g + 1) * 32] = True
    sel = np.argsort(-np.where(allowed, key_o[t], -np.inf), kind="stable")[:8]
    bad = M.astype(np.float64).copy()
    bad[t] = 0
    bad[t, sel] = 1
    band = np.full(50, 1e-7)
    with pytest.raises(AssertionError, match="more than Kg groups"):
        check_near_tie(np.array([t]), band, bad, P, S, key_o, gv_o, wl)


def test_planted_order_violation_fails():
    """Inside the kept groups, replacing a selected expert by a clearly
    worse one fails the order check."""
    wl = _case(50, 512, 22, 0, 0, synth.SIGMOID, 0.1)
    x64, bias, P, M, S, margin = _oracle(wl)
    key_o, gv_o = decision_inputs(S, x64, bias)
    t = 3
    sel = np.nonzero(M[t])[0]
    worst_out = np.argsort(np.where(M[t] == 0, key_o[t], np.inf))[0]
    bad = M.astype(np.float64).copy()
    bad[t, sel[np.argmax(key_o[t, sel])]] = 0
    bad[t, worst_out] = 1
    with pytest.raises(AssertionError, match="order"):
        check_near_tie(np.array([t]), np.full(50, 1e-7), bad, P, S, key_o, gv_o, wl)


def _tied_rows(n_tied):
    """Sigmoid rows with a zero bias whose 2nd and 3rd largest logits tie
    exactly on the first n_tied rows; a simulated GPU scores the 3rd one
    an ulp higher there, so it legitimately picks it (K = 2)."""
    T, E, K = 12, 16, 2
    wl = _case(T, E, K, 0, 0, synth.SIGMOID, 0.0)
    rng = np.random.default_rng(9)
    x = np.stack([rng.permutation(np.linspace(-2.0, 1.5, E)) for _ in range(T)])
    x = x.astype(np.float32).astype(np.float64)
    for t in range(n_tied):
        o = np.argsort(-x[t], kind="stable")
        x[t, o[2]] = x[t, o[1]]
    bias = np.zeros(E, np.float32)
    P, M, S, margin = oracle.topk_fwd(x, K, synth.SIGMOID, True, 0, 0, 2.5,
                                      bias.astype(np.float64), threads=4)
    s32 = S.astype(np.float32)
    for t in range(n_tied):
        tied = np.nonzero((x[t] == np.sort(x[t])[-2]))[0]
        hi = tied.max()
        s32[t, hi] = np.nextafter(s32[t, hi], np.float32(2))
    gi = s32.astype(np.float64)
    key, _ = decision_inputs(gi, x, bias)
    gm, _ = oracle.select(key, K, threads=4)
    m = gm.astype(bool)
    gp = np.where(m, 2.5 * gi / np.where(m, gi, 0.0).sum(1, keepdims=True), 0.0)
    return wl, x, bias, gp, gm.astype(np.float64), gi, P, M, S, margin


def test_legitimate_flips_counted():
    """Rows whose oracle keys tie exactly and whose GPU keys differ by an
    ulp may differ; they are near-tie rows."""
    wl, x, bias, gp, gm, gi, P, M, S, margin = _tied_rows(MAX_DIFFER_ROWS)
    near, differ = check_forward(wl, x, bias, gp, gm, gi, P, M, S, margin)
    assert list(differ) == list(range(MAX_DIFFER_ROWS)) and set(differ) <= set(near)


def test_too_many_differing_rows_fail():
    """More differing rows than MAX_DIFFER_ROWS fail even when each one is
    individually valid."""
    with pytest.raises(AssertionError, match="rows differ"):
        check_forward(*_tied_rows(MAX_DIFFER_ROWS + 1))
