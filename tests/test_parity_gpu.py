"""GPU parity: the HIP router library (through its C ABI) against the fp64
oracle on the same seeded inputs.  Needs an MI355X and a built
librouter.so; every case prints its name before touching the GPU."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from gpu_support import (DEV, MAX_DIFFER_ROWS, SCORE_NAME, assert_close, chain_tol, f64,
                         run_aux_fwd, run_fwd, say, threads, to_dev)
from score_function_top_amd import router, synth

pytestmark = pytest.mark.gpu

WL = synth.WORKLOADS


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    router.load()
    yield
    router.set_topk_path_threshold(router.TOPK_PATH_AUTO)


def wl_variant(base, **kw):
    return dataclasses.replace(base, **kw)


def grads(wl, T, aux=False):
    st, g64 = wl.aux_grad() if aux else wl.grad()
    return st[:T], g64[:T]


# ------------------------------------------------------------ workloads

@pytest.mark.parametrize("name", list(WL))
def test_workload_forward(name):
    run_fwd(WL[name])


@pytest.mark.parametrize("name", list(WL))
def test_workload_backward_isolated(name):
    """GPU and oracle backward on identical inputs: the oracle's forward
    intermediate (rounded to fp32) and map, and seeded gradients."""
    wl = WL[name]
    _, x64 = wl.logits()
    bias = wl.bias()
    say(f"[bwd isolated] {name}")
    _, M, S, _ = oracle.topk_fwd(x64, wl.K, wl.score_fn, wl.renorm, wl.num_groups,
                                 wl.group_topk, wl.scaling_factor,
                                 None if bias is None else bias.astype(np.float64),
                                 threads=threads())
    g_st, g64 = grads(wl, wl.T)
    if wl.grad_on_map:
        g64 = g64 * M
        if wl.dtype == synth.F32:
            g_st = (g_st * M).astype(np.float32)
        else:
            g_st = np.where(M.astype(bool), g_st, np.uint16(0)).astype(np.uint16)
    s32 = S.astype(np.float32)
    dx = router.router_topk_bwd(to_dev(g_st, wl.dtype), torch.from_numpy(s32).to(DEV),
                                torch.from_numpy(M.astype(bool)).to(DEV), wl.K,
                                SCORE_NAME[wl.score_fn], wl.renorm, wl.scaling_factor)
    torch.cuda.synchronize()
    ref = oracle.topk_bwd(g64, s32.astype(np.float64), M, wl.K, wl.score_fn, wl.renorm,
                          wl.scaling_factor, threads=threads())
    assert_close(f64(dx), ref, wl.dtype, f"{name} grad_logits")


@pytest.mark.parametrize("name", list(WL))
def test_workload_backward_chained(name):
    """x -> fwd -> bwd on each side; rows whose maps agree are compared."""
    wl = WL[name]
    r = run_fwd(wl, check=False)
    g_st, g64 = grads(wl, wl.T)
    say(f"[bwd chained] {name}")
    dx = router.router_topk_bwd(to_dev(g_st, wl.dtype), r["inter"], r["map"], wl.K,
                                SCORE_NAME[wl.score_fn], wl.renorm, wl.scaling_factor)
    torch.cuda.synchronize()
    ref = oracle.topk_bwd(g64, r["S"], r["M"], wl.K, wl.score_fn, wl.renorm,
                          wl.scaling_factor, threads=threads())
    same = np.nonzero((f64(r["map"]) == r["M"]).all(1))[0]
    assert same.size >= wl.T - MAX_DIFFER_ROWS
    ext = chain_tol(g64, r["S"], r["M"], wl.K, wl.score_fn, wl.renorm, wl.scaling_factor)
    assert_close(f64(dx), ref, wl.dtype, f"{name} chained grad", rows=same, extra=ext)


@pytest.mark.parametrize("name", [n for n in WL if WL[n].aux])
def test_workload_aux(name):
    wl = WL[name]
    r = run_aux_fwd(wl)
    g_st, g64 = grads(wl, wl.T, aux=True)
    say(f"[aux bwd] {name}")
    s32 = r["S"].astype(np.float32)
    dx = router.router_aux_scores_bwd(to_dev(g_st, wl.dtype), torch.from_numpy(s32).to(DEV),
                                      SCORE_NAME[wl.score_fn], wl.aux_renorm)
    dxc = router.router_aux_scores_bwd(to_dev(g_st, wl.dtype), r["inter"],
                                       SCORE_NAME[wl.score_fn], wl.aux_renorm)
    torch.cuda.synchronize()
    ref = oracle.aux_bwd(g64, s32.astype(np.float64), wl.score_fn, wl.aux_renorm,
                         threads=threads())
    assert_close(f64(dx), ref, wl.dtype, f"{name} aux grad")
    refc = oracle.aux_bwd(g64, r["S"], wl.score_fn, wl.aux_renorm, threads=threads())
    ext = chain_tol(g64, r["S"], None, wl.K, wl.score_fn, wl.aux_renorm, 1.0, aux=True)
    assert_close(f64(dxc), refc, wl.dtype, f"{name} aux chained grad", extra=ext)


# ------------------------------------------------------------ E/K sweep

SWEEP = [(E, K, sf) for E in (256, 512, 2304) for K in (4, 8, 22, 36) if K <= E
         for sf in (synth.SOFTMAX, synth.SIGMOID)]


@pytest.mark.parametrize("E,K,sf", SWEEP)
def test_sweep(E, K, sf):
    """T=8192 E/K grid at a ragged T=1031 slice: fwd, bwd, aux fwd/bwd."""
    wl = synth.sweep_workload(E, K, sf)
    T = 1031
    r = run_fwd(wl, T=T)
    g_st, g64 = grads(wl, T)
    dx = router.router_topk_bwd(to_dev(g_st, wl.dtype), r["inter"], r["map"], K,
                                SCORE_NAME[sf], wl.renorm, wl.scaling_factor)
    torch.cuda.synchronize()
    ref = oracle.topk_bwd(g64, r["S"], r["M"], K, sf, wl.renorm, wl.scaling_factor,
                          threads=threads())
    ext = chain_tol(g64, r["S"], r["M"], K, sf, wl.renorm, wl.scaling_factor)
    assert_close(f64(dx), ref, wl.dtype, f"{wl.name} grad", extra=ext)
    a = run_aux_fwd(wl, T=T)
    dxa = router.router_aux_scores_bwd(to_dev(g_st, wl.dtype), a["inter"], SCORE_NAME[sf],
                                       wl.aux_renorm)
    torch.cuda.synchronize()
    refa = oracle.aux_bwd(g64, a["S"], sf, wl.aux_renorm, threads=threads())
    ext = chain_tol(g64, a["S"], None, K, sf, wl.aux_renorm, 1.0, aux=True)
    assert_close(f64(dxa), refa, wl.dtype, f"{wl.name} aux grad", extra=ext)


# ------------------------------------------------------------ edge shapes

def edge_wl(T, E, K, sf, renorm=False, bias=0.0, G=0, Kg=0, dtype=synth.F32, c=1.0,
            seed=7):
    return synth.Workload(name=f"edge_T{T}_E{E}_K{K}_{SCORE_NAME[sf]}_r{int(renorm)}"
                          f"_b{bias}_G{G}_{'bf16' if dtype else 'f32'}",
                          T=T, E=E, K=K, score_fn=sf, renorm=renorm, num_groups=G,
                          group_topk=Kg, scaling_factor=c, dtype=dtype, bias_range=bias,
                          seed_logits=seed, seed_grad=seed + 1, seed_bias=seed + 2,
                          seed_aux_grad=seed + 3)


EDGE = [
    (1, 16, 2, synth.SOFTMAX), (65, 16, 16, synth.SOFTMAX), (8193, 64, 8, synth.SIGMOID),
    (33, 1, 1, synth.SOFTMAX), (33, 1, 1, synth.SIGMOID), (70, 3, 2, synth.SOFTMAX),
    (70, 3, 3, synth.SIGMOID), (129, 100, 7, synth.SOFTMAX), (129, 100, 100, synth.SIGMOID),
    (77, 257, 9, synth.SOFTMAX), (77, 257, 40, synth.SIGMOID), (50, 4096, 36, synth.SOFTMAX),
    (50, 4096, 1, synth.SIGMOID), (40, 4096, 100, synth.SOFTMAX), (31, 2304, 64, synth.SOFTMAX),
    (31, 2304, 65, synth.SOFTMAX), (19, 2000, 2000, synth.SOFTMAX), (300, 512, 33, synth.SIGMOID),
    (300, 256, 17, synth.SOFTMAX), (300, 128, 64, synth.SOFTMAX),
    # one-wave blocks: 6- and 12-chunk rows, with a partial last row batch
    (1029, 1536, 8, synth.SOFTMAX), (517, 3072, 20, synth.SIGMOID),
]


@pytest.mark.parametrize("T,E,K,sf", EDGE)
@pytest.mark.parametrize("renorm", [False, True])
def test_edge_shapes(T, E, K, sf, renorm):
    wl = edge_wl(T, E, K, sf, renorm, c=1.5)
    r = run_fwd(wl)
    g_st, g64 = grads(wl, T)
    dx = router.router_topk_bwd(to_dev(g_st, wl.dtype), r["inter"], r["map"], K,
                                SCORE_NAME[sf], renorm, 1.5)
    torch.cuda.synchronize()
    ref = oracle.topk_bwd(g64, r["S"], r["M"], K, sf, renorm, 1.5, threads=threads())
    ext = chain_tol(g64, r["S"], r["M"], K, sf, renorm, 1.5)
    assert_close(f64(dx), ref, synth.F32, f"{wl.name} grad", extra=ext)


@pytest.mark.parametrize("T,E,K,G,Kg,dtype", [
    (500, 256, 8, 8, 4, synth.BF16), (300, 256, 8, 8, 4, synth.F32), (200, 64, 6, 4, 2, synth.F32),
    (129, 512, 22, 16, 11, synth.F32), (64, 2304, 36, 36, 6, synth.F32),
    (90, 96, 12, 12, 4, synth.F32), (70, 160, 9, 10, 3, synth.F32), (50, 256, 8, 64, 8, synth.F32),
    # q = 4 with groups of 64, 32 and 8 lanes; a group size that is no power-of-two
    # number of lane quads (24 experts)
    (100, 2048, 16, 8, 4, synth.F32), (100, 512, 16, 4, 4, synth.F32),
    (257, 256, 16, 8, 4, synth.BF16), (60, 192, 8, 8, 4, synth.F32),
])
@pytest.mark.parametrize("biased", [False, True])
def test_groups(T, E, K, G, Kg, dtype, biased):
    """Group-limited routing; shapes cover both group stages (registers:
    group = 4 values of a power-of-two number of lanes and q <= 4; LDS:
    otherwise)."""
    wl = edge_wl(T, E, K, synth.SIGMOID, True, bias=0.05 if biased else 0.0, G=G, Kg=Kg,
                 dtype=dtype, c=2.5, seed=11)
    run_fwd(wl)


@pytest.mark.parametrize("E,G,Kg,K,b", [(4096, 64, 4, 8, 0.05), (4096, 2, 1, 4, 0.0),
                                        (4092, 62, 8, 16, 0.05)])
def test_group_largest_rows(E, G, Kg, K, b):
    """The largest grouped rows (LDS group stage, up to 72 KB of LDS per
    workgroup) run and match the oracle; more than 64 groups is rejected
    on the host."""
    wl = edge_wl(70, E, K, synth.SIGMOID, True, bias=b, G=G, Kg=Kg, c=2.5, seed=31)
    run_fwd(wl)
    x = torch.zeros((4, 130), device=DEV)
    with pytest.raises(router.RouterError) as e:
        router.router_topk_fwd(x, 2, "sigmoid", True, 65, 1)
    assert e.value.status == router.ERR_UNSUPPORTED


@pytest.mark.parametrize("sf,b,dtype,E,G", [(synth.SIGMOID, 0.05, synth.BF16, 256, 8),
                                            (synth.SOFTMAX, 0.0, synth.F32, 256, 8),
                                            (synth.SIGMOID, 0.0, synth.F32, 512, 16),
                                            (synth.SIGMOID, 0.05, synth.F32, 64, 2)])
def test_grouped_persistent_rows(sf, b, dtype, E, G):
    """Rows of 32-expert groups on the occupancy-sized grid: with 50001
    tokens every wave loops over several token groups (the next group's
    logits in flight) and the last group is ragged."""
    wl = edge_wl(50001, E, 8, sf, True, bias=b, G=G, Kg=min(4, G), dtype=dtype, c=2.5,
                 seed=37)
    run_fwd(wl)


def _random_cases(n=48, seed=2024):
    """Seeded random router configurations around the size boundaries of
    the launch plans (lanes per token, chunk counts, selection paths, both
    group stages)."""
    rng = np.random.default_rng(seed)
    edges = [(1, 16), (60, 70), (125, 135), (250, 260), (500, 520), (1000, 1030),
             (2300, 2310), (4090, 4096)]
    out = []
    while len(out) < n:
        lo, hi = edges[rng.integers(len(edges))]
        E = int(rng.integers(lo, hi + 1))
        T = int(rng.choice([1, 3, 17, 64, 129, 300, 513, 700, 8193]))
        sf = int(rng.integers(2))
        G = Kg = 0
        divs = [d for d in range(2, 65) if E % d == 0]
        if divs and rng.random() < 0.4:
            G = int(rng.choice(divs))
            Kg = int(rng.integers(1, G + 1))
            q = int(rng.integers(1, min(6, E // G) + 1))
            K = Kg * q
        else:
            K = int(rng.integers(1, min(E, 80) + 1))
        bias = 0.05 if sf == synth.SIGMOID and rng.random() < 0.5 else 0.0
        dtype = synth.BF16 if rng.random() < 0.3 else synth.F32
        renorm = bool(rng.integers(2))
        out.append((T, E, K, sf, renorm, bias, G, Kg, dtype, int(rng.integers(1 << 20))))
    return out


@pytest.mark.parametrize("T,E,K,sf,renorm,b,G,Kg,dtype,seed",
                         _random_cases() + _random_cases(48, 2025) + _random_cases(150, 7001) +
                         _random_cases(150, 7002) + _random_cases(150, 7003))
def test_random_configs(T, E, K, sf, renorm, b, G, Kg, dtype, seed):
    """Forward and backward against the oracle on seeded random shapes.  The
    backward reference uses the GPU's map: it equals the oracle's except on
    near-tie rows, where run_fwd has checked it is a valid selection (the
    selection there is decided on fp32 keys or group sums)."""
    wl = edge_wl(T, E, K, sf, renorm, bias=b, G=G, Kg=Kg, dtype=dtype, c=1.25, seed=seed)
    r = run_fwd(wl)
    g_st, g64 = grads(wl, T)
    dx = router.router_topk_bwd(to_dev(g_st, dtype), r["inter"], r["map"], K,
                                SCORE_NAME[sf], renorm, 1.25)
    torch.cuda.synchronize()
    m_gpu = f64(r["map"])
    ref = oracle.topk_bwd(g64, r["S"], m_gpu, K, sf, renorm, 1.25, threads=threads())
    ext = chain_tol(g64, r["S"], m_gpu, K, sf, renorm, 1.25)
    assert_close(f64(dx), ref, dtype, f"{wl.name} grad", extra=ext)


@pytest.mark.parametrize("E,K,sf,b,dtype", [
    (4090, 6, synth.SIGMOID, 0.05, synth.F32), (4090, 8, synth.SIGMOID, 0.05, synth.F32),
    (4094, 12, synth.SIGMOID, 0.0, synth.F32), (4090, 6, synth.SIGMOID, 0.05, synth.BF16),
    (4090, 6, synth.SOFTMAX, 0.0, synth.F32), (2302, 6, synth.SIGMOID, 0.05, synth.F32)])
def test_elementwise_padding_lanes(E, K, sf, b, dtype):
    """Element-wise rows (E not a multiple of 4) whose last chunk is padding
    on some lanes only, with the LDS group stage and the pruned select: the
    intermediate, probs and map of every lane match the oracle.  (A
    lane-divergent branch around the padding test once let the lanes with
    padding store another element's raw logit as the intermediate.)"""
    for thr in (router.TOPK_PATH_AUTO, 0, 4096):
        router.set_topk_path_threshold(thr)
        try:
            run_fwd(edge_wl(3, E, K, sf, True, bias=b, G=2, Kg=2, dtype=dtype, c=1.25,
                            seed=646769))
            run_fwd(edge_wl(67, E, K, sf, False, bias=b, dtype=dtype, seed=5))
        finally:
            router.set_topk_path_threshold(router.TOPK_PATH_AUTO)


def _random_aux_cases(n=24, seed=2026):
    """Aux-score shapes drawn like _random_cases (no bias or groups: the aux
    map is the plain top-K of the logits)."""
    return [(T, E, K, sf, renorm, dtype, sd)
            for T, E, K, sf, renorm, _b, _G, _Kg, dtype, sd in _random_cases(n, seed)]


@pytest.mark.parametrize("T,E,K,sf,renorm,dtype,seed", _random_aux_cases())
def test_random_aux(T, E, K, sf, renorm, dtype, seed):
    """Aux scores forward (map exact, scores and intermediate within
    tolerance) and backward, isolated and chained, on seeded random shapes."""
    wl = dataclasses.replace(edge_wl(T, E, K, sf, dtype=dtype, seed=seed), aux_renorm=renorm)
    r = run_aux_fwd(wl)
    g_st, g64 = grads(wl, T, aux=True)
    s32 = r["S"].astype(np.float32)
    dx = router.router_aux_scores_bwd(to_dev(g_st, dtype), torch.from_numpy(s32).to(DEV),
                                      SCORE_NAME[sf], renorm)
    dxc = router.router_aux_scores_bwd(to_dev(g_st, dtype), r["inter"], SCORE_NAME[sf], renorm)
    torch.cuda.synchronize()
    ref = oracle.aux_bwd(g64, s32.astype(np.float64), sf, renorm, threads=threads())
    assert_close(f64(dx), ref, dtype, f"{wl.name} aux grad")
    refc = oracle.aux_bwd(g64, r["S"], sf, renorm, threads=threads())
    ext = chain_tol(g64, r["S"], None, K, sf, renorm, 1.0, aux=True)
    assert_close(f64(dxc), refc, dtype, f"{wl.name} aux chained grad", extra=ext)


def test_grouped_softmax():
    run_fwd(edge_wl(300, 256, 8, synth.SOFTMAX, True, G=8, Kg=4, seed=13))


# Shapes the register group stage takes (4*L experts per group, L a power of
# two up to the lanes per token, at most 16 group slots (8 from three chunks
# on), q <= 4).
GROUP_STAGE_CASES = [
    (500, 256, 8, 8, 4, synth.BF16, synth.SIGMOID, 0.05),   # 8 lanes per group, q = 2
    (257, 256, 16, 8, 4, synth.BF16, synth.SIGMOID, 0.0),   # q = 4
    (200, 64, 6, 4, 2, synth.F32, synth.SIGMOID, 0.05),     # 4 lanes, one chunk
    (90, 96, 12, 12, 4, synth.F32, synth.SIGMOID, 0.0),     # 2 lanes, q = 3, 16 slots
    (70, 192, 6, 6, 3, synth.F32, synth.SOFTMAX, 0.0),      # slots past E
    (70, 160, 9, 10, 3, synth.F32, synth.SOFTMAX, 0.0),     # 16 slots at 4 chunks: LDS
    (129, 512, 12, 8, 4, synth.F32, synth.SIGMOID, 0.05),   # 32-lane tokens, q = 3
    (100, 512, 16, 4, 4, synth.F32, synth.SIGMOID, 0.0),    # a group fills a chunk
    (64, 1024, 8, 8, 4, synth.F32, synth.SIGMOID, 0.05),    # 64-lane tokens
    (65, 768, 12, 6, 3, synth.BF16, synth.SOFTMAX, 0.0),    # three chunks
    (100, 64, 8, 16, 8, synth.F32, synth.SIGMOID, 0.05),    # 1 lane per group, 16 slots, q = 1
    (80, 1024, 4, 4, 2, synth.BF16, synth.SOFTMAX, 0.0),    # 64 lanes per group
    # bias with q = 3 and 4 in two-chunk kernels: the group stage's pruning bound
    (300, 256, 16, 8, 4, synth.BF16, synth.SIGMOID, 0.05),  # 32 lanes, q = 4
    (150, 128, 12, 4, 4, synth.F32, synth.SIGMOID, 0.05),   # 16 lanes, q = 3
]


def _group_stage_outputs(wl, x_st, stage):
    router.set_group_stage(stage)
    try:
        bias = wl.bias()
        bt = None if bias is None else torch.from_numpy(bias).to(DEV)
        out = router.router_topk_fwd(to_dev(x_st, wl.dtype), wl.K, SCORE_NAME[wl.score_fn],
                                     wl.renorm, wl.num_groups, wl.group_topk,
                                     wl.scaling_factor, bt)
        torch.cuda.synchronize()
    finally:
        router.set_group_stage(router.GROUP_STAGE_AUTO)
    return out


@pytest.mark.parametrize("T,E,K,G,Kg,dtype,sf,b", GROUP_STAGE_CASES)
def test_group_stage_parity(T, E, K, G, Kg, dtype, sf, b):
    """The register (or 32-expert-group) and the LDS group stages agree: the
    same group scores, so the same maps and intermediates bit for bit (the
    probs to the last bits of their renormalisation sums), on random logits
    and on integer logits whose groups tie; the register stage matches the
    oracle on both, exactly on the map where groups tie."""
    wl = edge_wl(T, E, K, sf, True, bias=b, G=G, Kg=Kg, dtype=dtype, c=2.5, seed=29)
    run_fwd(wl)

    def cast(x):
        return (x.astype(np.float32) if dtype == synth.F32 else
                synth.f32_to_bf16_bits(x.astype(np.float32)))

    rng = np.random.default_rng(T + E)
    xi = rng.integers(-2, 3, (T, E)).astype(np.float64)
    xi[1] = 1.0                       # every group ties
    x_st, _ = wl.logits()
    for name, xs in (("random", x_st), ("integer", cast(xi))):
        say(f"[group stage] {wl.name} {name}")
        reg = _group_stage_outputs(wl, xs, router.GROUP_STAGE_AUTO)
        lds = _group_stage_outputs(wl, xs, router.GROUP_STAGE_LDS)
        # same group scores: the same maps and intermediates bit for bit; the
        # probs' renormalisation sums may take another lane layout (rows of
        # 32-expert groups have their own kernel), so their last bits may differ
        assert torch.equal(reg[1], lds[1]), f"{wl.name} {name}: maps differ"
        assert torch.equal(reg[2], lds[2]), f"{wl.name} {name}: intermediates differ"
        if dtype == synth.F32:
            assert_close(f64(reg[0]), f64(lds[0]), dtype, f"{wl.name} {name} probs",
                         rtol=1e-6, atol=0)
        else:
            assert_close(f64(reg[0]), f64(lds[0]), dtype, f"{wl.name} {name} probs")

    # Logits in {0, 1, 2} and no bias: groups tie exactly when their top-q
    # multisets are equal (the lower group wins), and otherwise differ by far
    # more than rounding, so the map is exact.
    nob = dataclasses.replace(wl, bias_range=0.0, name=wl.name + "_ties")
    xo = rng.integers(0, 3, (T, E)).astype(np.float64)
    xo[1] = 1.0
    xo_st = cast(xo)
    x64 = xo if dtype == synth.F32 else synth.bf16_bits_to_f32(xo_st).astype(np.float64)
    P, M, _, _ = oracle.topk_fwd(x64, K, sf, True, G, Kg, 2.5, threads=threads())
    say(f"[group stage] {nob.name} against the oracle")
    reg = _group_stage_outputs(nob, xo_st, router.GROUP_STAGE_AUTO)
    assert (f64(reg[1]) == M).all(), f"{nob.name}: map differs from the oracle"
    assert_close(f64(reg[0]), P, dtype, f"{nob.name} probs")


def test_bf16_paths():
    for sf in (synth.SOFTMAX, synth.SIGMOID):
        for E, K in ((256, 4), (512, 22), (2304, 36), (100, 5)):
            wl = edge_wl(257, E, K, sf, sf == synth.SIGMOID, dtype=synth.BF16, seed=17)
            r = run_fwd(wl)
            g_st, g64 = grads(wl, 257)
            dx = router.router_topk_bwd(to_dev(g_st, wl.dtype), r["inter"], r["map"], K,
                                        SCORE_NAME[sf], wl.renorm, 1.0)
            torch.cuda.synchronize()
            ref = oracle.topk_bwd(g64, r["S"], r["M"], K, sf, wl.renorm, 1.0,
                                  threads=threads())
            assert_close(f64(dx), ref, synth.BF16, f"{wl.name} grad")
            run_aux_fwd(wl, T=257)


# ------------------------------------------------------------ ties

def _tie_case(x64, K, sf, renorm, dtype=synth.F32):
    if dtype == synth.F32:
        st = x64.astype(np.float32)
    else:
        st = synth.f32_to_bf16_bits(x64.astype(np.float32))
        x64 = synth.bf16_bits_to_f32(st).astype(np.float64)
    xt = to_dev(st, dtype)
    p, m, i = router.router_topk_fwd(xt, K, SCORE_NAME[sf], renorm)
    a, am, ai = router.router_aux_scores(xt, K, SCORE_NAME[sf], renorm)
    torch.cuda.synchronize()
    P, M, S, _ = oracle.topk_fwd(x64, K, sf, renorm, threads=threads())
    A, AM, AS = oracle.aux_fwd(x64, K, sf, renorm, threads=threads())
    assert (f64(m) == M).all() and (f64(am) == AM).all()
    assert_close(f64(p), P, dtype, "tie probs")
    assert_close(f64(a), A, dtype, "tie aux scores")


@pytest.mark.parametrize("E,K", [(16, 2), (256, 4), (256, 8), (512, 22), (2304, 36),
                                 (2304, 4), (100, 50)])
def test_ties(E, K):
    say(f"[ties] E={E} K={K}")
    rng = np.random.default_rng(E + K)
    T = 300
    x = np.zeros((T, E))
    x[1] = 1.5                                         # all equal
    x[2:100] = rng.integers(-3, 4, (98, E))            # heavy ties everywhere
    x[100:200] = rng.integers(0, 2, (100, E)) * 0.5    # two values only
    x[200:] = np.round(rng.normal(0, 1, (T - 200, E)), 1)
    x[3, :] = -0.0                                      # signed zeros tie
    x[3, 1::2] = 0.0
    for sf in (synth.SOFTMAX, synth.SIGMOID):
        for renorm in (False, True):
            _tie_case(x, K, sf, renorm)
            _tie_case(x, K, sf, renorm, synth.BF16)


# ------------------------------------------------------------ paths

PATH_CASES = [(512, 2304, 36, synth.SOFTMAX, 0.0, 0), (700, 256, 4, synth.SOFTMAX, 0.0, 0),
              (700, 512, 22, synth.SIGMOID, 0.1, 0), (300, 256, 8, synth.SIGMOID, 0.05, 8),
              (300, 100, 30, synth.SOFTMAX, 0.0, 0), (90, 2304, 8, synth.SIGMOID, 0.0, 0),
              # around the automatic crossovers (4, 8 and 16+ elements per lane)
              (333, 64, 5, synth.SOFTMAX, 0.0, 0), (333, 64, 4, synth.SIGMOID, 0.0, 0),
              (257, 128, 4, synth.SOFTMAX, 0.0, 0), (257, 512, 2, synth.SIGMOID, 0.1, 0),
              (129, 2304, 3, synth.SOFTMAX, 0.0, 0), (129, 1000, 2, synth.SOFTMAX, 0.0, 0),
              # lanes < K <= 2 * lanes: the bound from the lanes' two largest keys
              (300, 256, 36, synth.SOFTMAX, 0.0, 0), (129, 512, 36, synth.SIGMOID, 0.1, 0),
              (65, 64, 30, synth.SOFTMAX, 0.0, 0), (33, 128, 64, synth.SIGMOID, 0.0, 0),
              (300, 256, 36, synth.SIGMOID, 0.05, 8), (77, 2304, 100, synth.SOFTMAX, 0.0, 0),
              (300, 128, 12, synth.SOFTMAX, 0.0, 0), (129, 64, 9, synth.SIGMOID, 0.1, 0)]


@pytest.mark.parametrize("T,E,K,sf,b,G", PATH_CASES)
def test_path_parity(T, E, K, sf, b, G):
    """Every selection path gives the same map and the same weights."""
    wl = edge_wl(T, E, K, sf, True, bias=b, G=G, Kg=4 if G else 0, c=2.0, seed=23)
    outs = []
    try:
        for thr in (router.TOPK_PATH_AUTO, 0, 8, 4096):
            router.set_topk_path_threshold(thr)
            r = run_fwd(wl, check=(thr == router.TOPK_PATH_AUTO))
            outs.append((f64(r["probs"]), f64(r["map"]), f64(r["inter"])))
    finally:
        router.set_topk_path_threshold(router.TOPK_PATH_AUTO)
    # maps are identical; weights may differ in the last bits where the
    # paths use different lane-group widths (different reduction trees)
    for o in outs[1:]:
        assert (o[1] == outs[0][1]).all(), "maps differ between paths"
        assert_close(o[0], outs[0][0], synth.F32, "probs across paths", rtol=1e-6, atol=0)
        assert_close(o[2], outs[0][2], synth.F32, "intermediate across paths", rtol=1e-6, atol=0)


# (workload, token rows): the full C4 batch (4 rows per persistent block),
# ragged row counts, and 6- and 8-chunk rows (E=1536, E=2048 bf16)
GRID_CASES = [("c4_softmax_2304x36", None), ("c4_softmax_2304x36", 6001),
              ("c5_group_sigmoid_256x8_bf16", None),
              ("c2_softmax_256x4", None), ("c3_sigmoid_512x22", 4097),
              ("sweep_softmax_1536x8", 5003), ("sweep_sigmoid_2048x22_bf16", 4099),
              ("sweep_softmax_3072x8", 3001)]


def grid_workload(name):
    if name in WL:
        return WL[name]
    _, score, shape, *dt = name.split("_")
    E, K = (int(v) for v in shape.split("x"))
    wl = synth.sweep_workload(E, K, synth.SOFTMAX if score == "softmax" else synth.SIGMOID)
    return dataclasses.replace(wl, dtype=synth.BF16) if dt else wl


@pytest.mark.parametrize("name,T", GRID_CASES)
def test_grid_modes_identical(name, T):
    """The occupancy-sized persistent grid (waves loop over token groups;
    the grouped forward prefetches the next group) gives the same bits as
    one block per token group: forward, backward, aux scores."""
    wl = grid_workload(name)
    x_st, _ = wl.logits()
    g_st, _ = wl.grad()
    if T is not None:
        x_st, g_st = x_st[:T], g_st[:T]
    bias = wl.bias()
    bt = None if bias is None else torch.from_numpy(bias).to(DEV)
    xt, gt = to_dev(x_st, wl.dtype), to_dev(g_st, wl.dtype)
    sf = SCORE_NAME[wl.score_fn]
    outs = []
    try:
        for mode in (router.GRID_FULL, router.GRID_PERSISTENT):
            say(f"[grid] {name} mode {mode}")
            router.set_grid_mode(mode)
            p, m, i = router.router_topk_fwd(xt, wl.K, sf, wl.renorm, wl.num_groups,
                                             wl.group_topk, wl.scaling_factor, bt)
            dx = router.router_topk_bwd(gt, i, m, wl.K, sf, wl.renorm, wl.scaling_factor)
            a = router.router_aux_scores(xt, wl.K, sf, wl.aux_renorm)
            adx = router.router_aux_scores_bwd(gt, a[2], sf, wl.aux_renorm)
            torch.cuda.synchronize()
            outs.append((p, m, i, dx, *a, adx))
    finally:
        router.set_grid_mode(router.GRID_FULL)
    for u, v in zip(*outs):
        assert torch.equal(u, v), f"{name}: grid modes differ"


def test_deterministic():
    wl = WL["c4_softmax_2304x36"]
    x_st, _ = wl.logits()
    xt = to_dev(x_st[:2048], wl.dtype)
    say("[determinism] c4 slice")
    a = router.router_topk_fwd(xt, wl.K)
    b = router.router_topk_fwd(xt, wl.K)
    g = torch.randn(xt.shape, device=DEV, generator=torch.Generator(DEV).manual_seed(5))
    da = router.router_topk_bwd(g, a[2], a[1], wl.K)
    db = router.router_topk_bwd(g, b[2], b[1], wl.K)
    torch.cuda.synchronize()
    for u, v in zip((*a, da), (*b, db)):
        assert torch.equal(u, v)


# ------------------------------------------------------------ layouts

@pytest.mark.parametrize("E,K,sf", [(256, 4, synth.SOFTMAX), (2304, 36, synth.SOFTMAX),
                                    (512, 22, synth.SIGMOID)])
def test_unaligned_views(E, K, sf):
    """Arrays offset by one element take the element-wise kernels."""
    wl = edge_wl(133, E, K, sf, sf == synth.SIGMOID, c=1.25, seed=29)
    x_st, x64 = wl.logits()
    say(f"[unaligned] {wl.name}")
    n = x64.size
    buf = torch.empty(n + 1, dtype=torch.float32, device=DEV)
    buf[1:] = torch.from_numpy(x_st.reshape(-1)).to(DEV)
    xt = buf[1:].view(133, E)
    outs = [torch.empty(n + 1, dtype=dt, device=DEV)[1:].view(133, E)
            for dt in (torch.float32, torch.bool, torch.float32)]
    p, m, i = router.router_topk_fwd(xt, K, SCORE_NAME[sf], wl.renorm, scaling_factor=1.25,
                                     out=outs)
    g = torch.empty(n + 1, dtype=torch.float32, device=DEV)[1:].view(133, E)
    g_st, g64 = wl.grad()
    g.copy_(torch.from_numpy(g_st))
    dx = router.router_topk_bwd(g, i, m, K, SCORE_NAME[sf], wl.renorm, 1.25,
                                out=torch.empty(n + 1, device=DEV)[1:].view(133, E))
    torch.cuda.synchronize()
    P, M, S, _ = oracle.topk_fwd(x64, K, sf, wl.renorm, scaling_factor=1.25, threads=threads())
    assert (f64(m) == M).all()
    assert_close(f64(p), P, synth.F32, "unaligned probs")
    assert_close(f64(i), S, synth.F32, "unaligned intermediate")
    ref = oracle.topk_bwd(g64, S, M, K, sf, wl.renorm, 1.25, threads=threads())
    ext = chain_tol(g64, S, M, K, sf, wl.renorm, 1.25)
    assert_close(f64(dx), ref, synth.F32, "unaligned grad", extra=ext)


def test_zero_tokens():
    x = torch.empty(0, 64, device=DEV)
    p, m, i = router.router_topk_fwd(x, 4)
    dx = router.router_topk_bwd(x, i, m, 4)
    a = router.router_aux_scores(x, 4)
    da = router.router_aux_scores_bwd(x, i)
    torch.cuda.synchronize()
    assert p.shape == (0, 64) and dx.shape == (0, 64) and a[0].shape == (0, 64)
    assert da.shape == (0, 64)


def test_device_query():
    q = router.device_query()
    props = torch.cuda.get_device_properties(0)
    assert q["compute_units"] == props.multi_processor_count
    assert q["clock_khz"] > 0 and q["memory_clock_khz"] > 0 and q["memory_bus_bits"] > 0


def test_side_stream():
    wl = WL["c2_softmax_256x4"]
    x_st, x64 = wl.logits()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        xt = to_dev(x_st[:1000], wl.dtype)
        p, m, i = router.router_topk_fwd(xt, wl.K)
    s.synchronize()
    P, M, S, _ = oracle.topk_fwd(x64[:1000], wl.K, threads=threads())
    assert (f64(m) == M).all()
    assert_close(f64(p), P, synth.F32, "side-stream probs")


def test_beyond_32bit_elements():
    """T*E > 2^31 elements: sampled rows against the oracle."""
    E, K = 256, 8
    T = (1 << 31) // E + 4099
    say(f"[large] T={T} E={E}")
    gen = torch.Generator(DEV).manual_seed(31)
    x = torch.randn(T, E, device=DEV, generator=gen)
    p, m, i = router.router_topk_fwd(x, K, "sigmoid", True, scaling_factor=2.0)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(8), np.arange(T - 8, T),
                                     np.random.default_rng(3).integers(0, T, 200)]))
    rt = torch.from_numpy(rows).to(DEV)
    x64 = f64(x[rt])
    P, M, S, _ = oracle.topk_fwd(x64, K, synth.SIGMOID, True, scaling_factor=2.0)
    assert (f64(m[rt]) == M).all()
    assert_close(f64(p[rt]), P, synth.F32, "large probs")
    assert_close(f64(i[rt]), S, synth.F32, "large intermediate")
    g = torch.randn(T, E, device=DEV, generator=gen)
    del x
    dx = router.router_topk_bwd(g, i, m, K, "sigmoid", True, 2.0)
    torch.cuda.synchronize()
    ref = oracle.topk_bwd(f64(g[rt]), S, M, K, synth.SIGMOID, True, 2.0)
    ext = chain_tol(f64(g[rt]), S, M, K, synth.SIGMOID, True, 2.0)
    assert_close(f64(dx[rt]), ref, synth.F32, "large grad", extra=ext)


def test_graph_replay_matches_eager():
    """The four passes captured in one HIP graph: every replay, with eager
    work and synchronisation between replays, equals the eager results bit
    for bit (no memset nodes: the library writes every output element)."""
    wl = WL["c3_sigmoid_512x22"]
    x_st, _ = wl.logits()
    g_st, _ = wl.grad()
    T = 2048
    x = to_dev(x_st[:T], wl.dtype)
    g = to_dev(g_st[:T], wl.dtype)
    b = torch.from_numpy(wl.bias()).to(DEV)
    say("[graph] c3 slice")

    def passes(o):
        router.router_topk_fwd(x, wl.K, "sigmoid", True, 0, 0, 2.5, b,
                               out=(o["p"], o["m"], o["i"]))
        router.router_topk_bwd(g, o["i"], o["m"], wl.K, "sigmoid", True, 2.5, out=o["dx"])
        router.router_aux_scores(x, wl.K, "sigmoid", True, out=(o["a"], o["am"], o["ai"]))
        router.router_aux_scores_bwd(g, o["ai"], "sigmoid", True, out=o["adx"])

    def bufs():
        o = {k: torch.empty(T, wl.E, device=DEV) for k in ("p", "i", "dx", "a", "ai", "adx")}
        o.update({k: torch.empty(T, wl.E, dtype=torch.bool, device=DEV) for k in ("m", "am")})
        return o

    eager, cap = bufs(), bufs()
    passes(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        passes(cap)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        passes(cap)
    other = bufs()
    for rep in range(3):
        for t in cap.values():
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        passes(other)                 # eager work between replays
        torch.cuda.synchronize()
        for k in eager:
            assert torch.equal(cap[k], eager[k]), (rep, k)
            assert torch.equal(other[k], eager[k]), (rep, k)
