"""GPU parity of the load-balancing aux loss (tokens per expert, the loss and
its gradient) against the fp64 oracle, through the C ABI.

Bars: counts bit-exact (integer work); loss and gradient within the fp32
tolerance (rtol 2e-6, atol 1e-7; bf16 gradients rtol 1e-2).  With fp32 or
bf16 scores fed to both sides unchanged, the GPU sums in fp64 and rounds
once, so the isolated loss must also sit within one fp32 ulp of the
oracle's value, which the tests check as well.
"""
import numpy as np
import pytest
import torch

from gpu_support import (DEV, F32_ATOL, F32_RTOL, SCORE_NAME, assert_close, chain_tol, f64,
                         say, threads, to_dev)
import oracle
from score_function_top_amd import router, synth

pytestmark = pytest.mark.gpu
COEFF = synth.AUX_LOSS_COEFF


def ulp32(x):
    return float(np.spacing(np.float32(abs(x))))


def gpu_counts(m_np, **kw):
    t = torch.from_numpy(np.ascontiguousarray(m_np)).to(DEV)
    c = router.router_tokens_per_expert(t, **kw)
    torch.cuda.synchronize()
    return c.cpu().numpy()


def check_loss(gpu, ref, what):
    gpu = float(gpu)
    assert abs(gpu - ref) <= F32_ATOL + F32_RTOL * abs(ref), (what, gpu, ref)
    assert abs(gpu - ref) <= ulp32(ref), (what, "more than one fp32 ulp", gpu, ref)


def run_loss(T, E, K, seed, dtype=synth.F32, N=None, coeff=COEFF, counts=None, view=False):
    """Isolated loss forward and backward on seeded inputs; returns the GPU
    loss for further checks."""
    N = T if N is None else N
    say(f"[aux loss] T={T} E={E} K={K} N={N} dtype={dtype} view={view}")
    st, s64 = synth.prob_like(seed, T, E, dtype)
    if counts is None:
        counts = oracle.tokens_per_expert(synth.random_map(seed + 1, T, E, min(K, E)))
    if view:
        # an unaligned view: one element in, so only element-wise access fits
        big = np.zeros((T * E + 1,), st.dtype)
        big[1:] = st.ravel()
        dev = to_dev(big, dtype)[1:].view(T, E)
    else:
        dev = to_dev(st, dtype)
    ct = torch.from_numpy(np.ascontiguousarray(counts, np.int64)).to(DEV)
    loss = router.router_aux_loss_fwd(dev, ct, N, K, coeff)
    g = torch.tensor([-0.75], dtype=torch.float32, device=DEV)
    tdt = torch.float32 if dtype == synth.F32 else torch.bfloat16
    dx = router.router_aux_loss_bwd(g, ct, T, N, K, coeff, dtype=tdt)
    torch.cuda.synchronize()
    ref = oracle.aux_loss(s64, counts, K, coeff, N)
    check_loss(loss.item(), ref, f"loss T={T} E={E}")
    dref = oracle.aux_loss_bwd(-0.75, counts, T, K, coeff, N)
    assert_close(f64(dx), dref, dtype, f"aux loss grad T={T} E={E}")
    return loss.item()


# ------------------------------------------------------------------ counts

# Shapes cover every lane width and load width of the count kernel: 16
# map bytes per lane with 16-, 8-, 4- and 1-byte loads (E = 4096, 1000,
# 100, 999), 8 (E = 1536 with 8-byte loads, 1532 with 4-byte, 5 with byte
# loads), 4 (E = 2304, 1540 with 4-byte loads; 1537 and 1 with byte loads),
# and grids from 1 to 2048 blocks (the cap makes blocks loop over several
# row splits at T = 300000 and 70000).
@pytest.mark.parametrize("T,E,K", [(64, 16, 2), (8192, 256, 4), (8192, 512, 22),
                                   (8192, 2304, 36), (1031, 999, 7), (129, 5, 2),
                                   (1, 1, 1), (3, 4096, 100), (40000, 2304, 36),
                                   (300000, 64, 6), (8192, 4096, 16), (4099, 1000, 9),
                                   (2000, 100, 3), (3001, 1536, 12), (3001, 1532, 12),
                                   (2500, 1540, 8), (2500, 1537, 8), (16384, 256, 8),
                                   (70000, 2304, 36)])
def test_tokens_per_expert(T, E, K):
    say(f"[counts] T={T} E={E} K={K}")
    m = synth.random_map(7000 + E + K, T, E, K)
    assert (gpu_counts(m) == oracle.tokens_per_expert(m)).all()


def test_tokens_per_expert_nonbinary_bytes_and_dense():
    """Any nonzero byte counts as routed; an all-ones map counts T."""
    rng = np.random.default_rng(71)
    m = rng.integers(0, 256, (777, 130)).astype(np.uint8)
    m[rng.random(m.shape) < 0.6] = 0
    assert (gpu_counts(m) == oracle.tokens_per_expert(m)).all()
    ones = np.ones((513, 260), np.uint8)
    assert (gpu_counts(ones) == 513).all()


def test_tokens_per_expert_zero_rows_and_stale_output():
    """T = 0 writes zeros; a preallocated output holding old values is
    overwritten, not added to."""
    z = torch.zeros((0, 37), dtype=torch.bool, device=DEV)
    out = torch.full((37,), 5, dtype=torch.int64, device=DEV)
    router.router_tokens_per_expert(z, out=out)
    torch.cuda.synchronize()
    assert (out.cpu() == 0).all()
    m = synth.random_map(72, 4099, 300, 9)
    out = torch.full((300,), 123456, dtype=torch.int64, device=DEV)
    assert (gpu_counts(m, out=out) == oracle.tokens_per_expert(m)).all()


def test_tokens_per_expert_workspace_reuse():
    """One zero-filled workspace serves a run of calls of different shapes
    (stream-ordered); each call leaves it zero-filled again."""
    ws = torch.zeros((router.router_tokens_per_expert_workspace_bytes(1, 4096),),
                     dtype=torch.uint8, device=DEV)
    for i, (T, E, K) in enumerate([(8192, 2304, 36), (513, 64, 5), (8192, 2304, 36),
                                   (4099, 4096, 30), (1, 7, 1), (16384, 256, 8)]):
        say(f"[counts reuse] T={T} E={E}")
        m = synth.random_map(7400 + i, T, E, K)
        t = torch.from_numpy(m).to(DEV)
        c = router.router_tokens_per_expert(t, workspace=ws)
        c2 = router.router_tokens_per_expert(t, workspace=ws)
        torch.cuda.synchronize()
        want = oracle.tokens_per_expert(m)
        assert (c.cpu().numpy() == want).all() and (c2.cpu().numpy() == want).all(), (T, E)
        assert int(ws.count_nonzero()) == 0, "workspace not returned zero-filled"


def test_tokens_per_expert_unaligned_view():
    m = synth.random_map(73, 301, 64, 5)
    big = torch.zeros(301 * 64 + 1, dtype=torch.uint8, device=DEV)
    big[1:] = torch.from_numpy(m.ravel()).to(DEV)
    c = router.router_tokens_per_expert(big[1:].view(301, 64))
    torch.cuda.synchronize()
    assert (c.cpu().numpy() == oracle.tokens_per_expert(m)).all()


# -------------------------------------------------------------------- loss

@pytest.mark.parametrize("T,E,K", [(64, 16, 2), (8192, 256, 4), (8192, 512, 22),
                                   (8192, 2304, 36), (1031, 999, 7), (129, 5, 2),
                                   (1, 1, 1), (3, 4096, 100), (40000, 2304, 36),
                                   (100000, 8, 2)])
def test_aux_loss_fp32(T, E, K):
    run_loss(T, E, K, 7100 + E + K)


@pytest.mark.parametrize("T,E,K", [(8192, 256, 8), (1031, 999, 7), (16384, 256, 8)])
def test_aux_loss_bf16(T, E, K):
    run_loss(T, E, K, 7200 + E + K, dtype=synth.BF16)


@pytest.mark.parametrize("T,E,dtype", [(301, 64, synth.F32), (129, 260, synth.BF16)])
def test_aux_loss_unaligned_view(T, E, dtype):
    run_loss(T, E, 4, 7300 + E, dtype=dtype, view=True)


def test_aux_loss_global_counts_and_coefficients():
    """Counts gathered over more tokens than the local rows (N > T)."""
    T, E, K = 1000, 128, 4
    counts = oracle.tokens_per_expert(synth.random_map(7401, 4 * T, E, K))
    run_loss(T, E, K, 7400, N=4 * T, counts=counts)
    run_loss(T, E, K, 7402, coeff=1.0)
    run_loss(T, E, 1, 7403, coeff=3e-4)


def test_aux_loss_closed_forms_on_gpu():
    """Balanced routing gives coeff; full collapse gives coeff * E."""
    T, E, K = 4096, 64, 4
    s = torch.full((T, E), 1.0 / E, device=DEV)
    c = torch.full((E,), T * K // E, dtype=torch.int64, device=DEV)
    got = router.router_aux_loss_fwd(s, c, T, K, 0.5).item()
    assert abs(got - 0.5) <= 2e-6 * 0.5
    s = torch.zeros((T, E), device=DEV)
    s[:, 3] = 1.0
    c = torch.zeros((E,), dtype=torch.int64, device=DEV)
    c[3] = T
    got = router.router_aux_loss_fwd(s, c, T, 1, 0.5).item()
    assert abs(got - 0.5 * E) <= 2e-6 * 0.5 * E


def test_aux_loss_zero_rows():
    s = torch.zeros((0, 16), device=DEV)
    c = torch.zeros((16,), dtype=torch.int64, device=DEV)
    loss = torch.full((), 7.0, device=DEV)
    router.router_aux_loss_fwd(s, c, 10, 2, COEFF, out=loss)
    dx = router.router_aux_loss_bwd(torch.ones(1, device=DEV), c, 0, 10, 2, COEFF)
    torch.cuda.synchronize()
    assert loss.item() == 0.0 and dx.shape == (0, 16)


def test_aux_loss_deterministic_and_workspace_contents_ignored():
    T, E, K = 8192, 2304, 36
    st, _ = synth.prob_like(7500, T, E)
    s = to_dev(st, synth.F32)
    c = torch.from_numpy(oracle.tokens_per_expert(synth.random_map(7501, T, E, K))).to(DEV)
    ws = torch.empty((router.router_aux_loss_workspace_bytes(T, E),), dtype=torch.uint8,
                     device=DEV)
    vals = []
    for fill in (0, 0xFF, 0x7F):
        ws.fill_(fill)
        vals.append(router.router_aux_loss_fwd(s, c, T, K, COEFF, workspace=ws).item())
    assert vals[0] == vals[1] == vals[2]


def test_aux_loss_chain_from_logits():
    """GPU chain (aux scores -> map -> counts -> loss -> its gradient ->
    aux-score backward) against the oracle chain, on the two aux workloads.
    Counts are exact (the aux map is decided on the logits); the loss is a
    positive combination of scores each within the fp32 tolerance, so it
    keeps that tolerance."""
    for name in ("c3_sigmoid_512x22", "c4_softmax_2304x36"):
        wl = synth.WORKLOADS[name]
        say(f"[aux loss chain] {name}")
        x_st, x64 = wl.logits()
        xt = to_dev(x_st, wl.dtype)
        sc, rmap, inter = router.router_aux_scores(xt, wl.K, SCORE_NAME[wl.score_fn],
                                                   wl.aux_renorm)
        cnt = router.router_tokens_per_expert(rmap)
        loss = router.router_aux_loss_fwd(sc, cnt, wl.T, wl.K, COEFF)
        # grad_loss 2^20 (exact scaling) lifts the gradients well above atol
        g = torch.full((1,), 2.0 ** 20, device=DEV)
        dsc = router.router_aux_loss_bwd(g, cnt, wl.T, wl.T, wl.K, COEFF)
        dx = router.router_aux_scores_bwd(dsc, inter, SCORE_NAME[wl.score_fn], wl.aux_renorm)
        torch.cuda.synchronize()
        A, M, S = oracle.aux_fwd(x64, wl.K, wl.score_fn, wl.aux_renorm, threads=threads())
        n = oracle.tokens_per_expert(M)
        assert (cnt.cpu().numpy() == n).all(), name
        ref = oracle.aux_loss(A, n, wl.K, COEFF)
        got = loss.item()
        assert abs(got - ref) <= F32_ATOL + F32_RTOL * abs(ref), (name, got, ref)
        dref = oracle.aux_loss_bwd(2.0 ** 20, n, wl.T, wl.K, COEFF)
        assert_close(f64(dsc), dref, synth.F32, f"{name} loss grad")
        dxr = oracle.aux_bwd(dref, S, wl.score_fn, wl.aux_renorm, threads=threads())
        # the aux-score backward sees the exact same gradient on both sides;
        # only its intermediate differs (GPU scores within the fp32 tolerance)
        extra = chain_tol(dref, S, None, wl.K, wl.score_fn, wl.aux_renorm, 1.0, aux=True)
        assert_close(f64(dx), dxr, synth.F32, f"{name} chained aux bwd", extra=extra)


def test_aux_loss_graph_replay():
    """Counts and loss captured in a HIP graph and replayed several times,
    with eager work between replays (the outputs cleared and the loss
    workspace refilled), match the eager results each time; the count
    workspace is zero-filled after every replay."""
    T, E, K = 4096, 512, 8
    st, _ = synth.prob_like(7600, T, E)
    s = to_dev(st, synth.F32)
    m = torch.from_numpy(synth.random_map(7601, T, E, K)).to(DEV)
    ws = torch.empty((router.router_aux_loss_workspace_bytes(T, E),), dtype=torch.uint8,
                     device=DEV)
    cws = torch.zeros((router.router_tokens_per_expert_workspace_bytes(T, E),),
                      dtype=torch.uint8, device=DEV)
    cnt = torch.empty((E,), dtype=torch.int64, device=DEV)
    loss = torch.empty((), dtype=torch.float32, device=DEV)
    router.router_tokens_per_expert(m, out=cnt, workspace=cws)
    router.router_aux_loss_fwd(s, cnt, T, K, COEFF, out=loss, workspace=ws)
    torch.cuda.synchronize()
    want_c, want_l = cnt.clone(), loss.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            router.router_tokens_per_expert(m, out=cnt, workspace=cws)
            router.router_aux_loss_fwd(s, cnt, T, K, COEFF, out=loss, workspace=ws)
    torch.cuda.synchronize()
    for i in range(4):
        cnt.zero_()
        loss.zero_()
        ws.fill_(i * 37)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(cnt, want_c) and torch.equal(loss, want_l), i
        assert int(cws.count_nonzero()) == 0, i
