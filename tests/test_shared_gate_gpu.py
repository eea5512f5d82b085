"""GPU parity of the routed top-k with the shared-expert sigmoid gate against
the fp64 oracle, through the C ABI.

Bars: routed ids and shared ids bit-exact (the selection is decided on the
gating logits themselves); routed weights within the fp32 tolerance (rtol
2e-6, atol 1e-7); gates within that tolerance plus the accumulation bound
of their dot products: each lane sums H/64 products in fp32 (bf16 products
are exact in fp32) and a 6-level wave tree adds the lanes, so the logit is
off by at most (H/64 + 6) * 2^-24 * sum_h |hs_h * w_h| (taken twice, for
margin), and the sigmoid's slope is at most 1/4.
"""
import numpy as np
import pytest
import torch

from gpu_support import DEV, assert_close, say, threads, to_dev
import oracle
from score_function_top_amd import router, synth

pytestmark = pytest.mark.gpu


def inputs(seed, M, E, H, S, dtype, views=False, ties=False):
    x_st, x64 = synth.storage(synth.normal(seed, (M, E), 1.0), dtype)
    if ties:   # small integers: many keys tie at the pruning bound
        x_st, x64 = synth.storage(np.round(synth.normal(seed, (M, E), 1.0)), dtype)
    h_st, h64 = synth.storage(synth.normal(seed + 1, (M, H), 1.0), dtype)
    g_st, g64 = synth.storage(synth.normal(seed + 2, (S, H), 0.05), dtype)
    if views:
        devs = []
        for a in (x_st, h_st, g_st):
            big = np.zeros((a.size + 1,), a.dtype)
            big[1:] = a.ravel()
            devs.append(to_dev(big, dtype)[1:].view(a.shape))
        return devs, (x64, h64, g64)
    return [to_dev(a, dtype) for a in (x_st, h_st, g_st)], (x64, h64, g64)


def run(M, E, H, K, S, dtype=synth.BF16, renorm=True, scale=1.0, base=None, ld_extra=0,
        views=False, seed=None, ties=False):
    seed = seed if seed is not None else 9500 + M + E + H + K + S
    say(f"[shared gate] M={M} E={E} H={H} K={K} S={S} dtype={dtype} renorm={renorm} "
        f"scale={scale} ld+{ld_extra} views={views}")
    (xt, ht, gt), (x64, h64, g64) = inputs(seed, M, E, H, S, dtype, views, ties)
    out = None
    if ld_extra:
        wbig = torch.full((M, K + S + ld_extra), -7.0, dtype=torch.float32, device=DEV)
        ibig = torch.full((M, K + S + ld_extra), -7, dtype=torch.int32, device=DEV)
        out = (wbig[:, :K + S], ibig[:, :K + S])
    w, ids = router.router_topk_shared_gate(xt, ht, gt, K, renorm, scale, base, out=out)
    torch.cuda.synchronize()
    b = E if base is None else base
    W, I = oracle.topk_shared_gate(x64, h64, g64, K, renorm, scale, b, threads=threads())
    gi, gw_ = ids.cpu().numpy(), w.cpu().numpy().astype(np.float64)
    assert (gi == I).all(), ("ids", np.argwhere(gi != I)[:5].tolist())
    assert_close(gw_[:, :K], W[:, :K], synth.F32, "routed weights")
    terms = np.abs(h64) @ np.abs(g64).T                      # sum_h |hs_h w_h| per (m, s)
    extra = abs(scale) * 0.25 * 2.0 * (H / 64 + 6) * 2.0 ** -24 * terms
    assert_close(gw_[:, K:], W[:, K:], synth.F32, "gates", extra=extra)
    if ld_extra:
        assert (wbig[:, K + S:].cpu() == -7.0).all() and (ibig[:, K + S:].cpu() == -7).all()
    return w, ids


@pytest.mark.parametrize("M", [1, 4, 16, 64, 256, 1024, 4096, 16384])
def test_page_shape(M):
    """Qwen3-Next routing: 512 experts, hidden 4096, top-10, one shared
    expert, bf16 (the page's sweep over tokens)."""
    run(M, 512, 4096, 10, 1)


@pytest.mark.parametrize("kw", [
    dict(S=2), dict(S=8), dict(dtype=synth.F32), dict(renorm=False), dict(scale=0.5),
    dict(E=256), dict(M=65), dict(M=1, S=8, dtype=synth.F32), dict(base=0),
    dict(E=160, K=7), dict(E=1000, K=32, S=16), dict(E=1, K=1), dict(H=4100),
    dict(H=33, dtype=synth.F32), dict(H=7168), dict(ld_extra=5), dict(views=True),
    dict(views=True, dtype=synth.F32, H=100), dict(ties=True), dict(ties=True, K=32),
    dict(K=3), dict(K=4),
])
def test_page_axes_and_edges(kw):
    """The page's test axes (S = 2 and 8, fp32 inputs, no renorm, scale 0.5,
    E = 256, M = 1 and 65) and edges: non-power-of-two E, a hidden size that
    is no multiple of the vector width, wide rows, unaligned views, wider
    output rows whose extra columns must stay untouched."""
    a = dict(M=64, E=512, H=4096, K=10, S=1)
    a.update(kw)
    run(**a)


# The library takes one wave per half of a token up to 1024 tokens, one
# wave per token above, and from 8192 tokens on (rows that fit the
# prefetch) one wave per token with the routed half last; the edges again
# on the last two.
_LATE_EDGES = [dict(), dict(S=8), dict(dtype=synth.F32), dict(renorm=False, scale=0.5),
               dict(E=1000, K=32, S=16), dict(ld_extra=5), dict(ties=True, K=32), dict(K=3)]


@pytest.mark.parametrize("kw", _LATE_EDGES)
def test_page_axes_and_edges_routed_half_last(kw):
    a = dict(M=8200, E=512, H=4096, K=10, S=1)
    a.update(kw)
    run(**a)


@pytest.mark.parametrize("kw", [
    dict(), dict(S=8), dict(dtype=synth.F32), dict(renorm=False, scale=0.5),
    dict(E=1000, K=32, S=16), dict(H=4100), dict(H=33, dtype=synth.F32), dict(H=7168),
    dict(ld_extra=5), dict(views=True), dict(ties=True, K=32), dict(K=3),
])
def test_page_axes_and_edges_many_tokens(kw):
    a = dict(M=1100, E=512, H=4096, K=10, S=1)
    a.update(kw)
    run(**a)


@pytest.mark.parametrize("m_big,m_small", [(1100, 1024), (8200, 8000)])
@pytest.mark.parametrize("kw", [dict(), dict(E=1000, K=32, S=16, dtype=synth.F32),
                                dict(E=1000, K=32, S=16, H=4100, dtype=synth.F32),
                                dict(ties=True, K=32), dict(H=7168, S=2)])
def test_gate_kernels_agree(kw, m_big, m_small):
    """The first rows of a longer call equal, bit for bit, the call on those
    rows alone: 1100 tokens (one wave per token) against 1024 (one wave per
    half), 8200 (routed half last) against 8000 (routed half first)."""
    a = dict(E=512, H=4096, K=10, S=1, dtype=synth.BF16, ties=False)
    a.update(kw)
    say(f"[shared gate] {m_big} against {m_small} tokens {a}")
    (xt, ht, gt), _ = inputs(9650, m_big, a["E"], a["H"], a["S"], a["dtype"], ties=a["ties"])
    w1, i1 = router.router_topk_shared_gate(xt, ht, gt, a["K"])
    w0, i0 = router.router_topk_shared_gate(xt[:m_small], ht[:m_small], gt, a["K"])
    torch.cuda.synchronize()
    assert torch.equal(i0, i1[:m_small])
    assert torch.equal(w0.view(torch.int32), w1[:m_small].view(torch.int32))


def test_zero_tokens_noop():
    x = torch.zeros((0, 512), dtype=torch.bfloat16, device=DEV)
    h = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    g = torch.zeros((1, 64), dtype=torch.bfloat16, device=DEV)
    w, ids = router.router_topk_shared_gate(x, h, g, 4)
    assert w.shape == (0, 5) and ids.shape == (0, 5)


def test_graph_replay():
    (xt, ht, gt), _ = inputs(9601, 256, 512, 4096, 1, synth.BF16)
    w, ids = router.router_topk_shared_gate(xt, ht, gt, 10)
    torch.cuda.synchronize()
    keep = (w.clone(), ids.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            router.router_topk_shared_gate(xt, ht, gt, 10, out=(w, ids))
    torch.cuda.synchronize()
    for i in range(4):
        w.zero_()
        ids.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(w, keep[0]) and torch.equal(ids, keep[1]), i
