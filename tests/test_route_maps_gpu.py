"""GPU parity of decode-shape routing with expert maps against the fp64
oracle, through the C ABI.

Bars: top-k ids and all four maps bit-exact (integer work; the selection is
decided on the logits themselves, the same fp32 or bf16 values on both
sides, so there is no near-tie band); weights within the fp32 tolerance
(rtol 2e-6, atol 1e-7), for fp32 and bf16 logits alike (weights are fp32).
"""
import numpy as np
import pytest
import torch

from gpu_support import DEV, assert_close, say, to_dev
import oracle
from score_function_top_amd import router, synth

pytestmark = pytest.mark.gpu
SF = {"softmax": synth.SOFTMAX, "sigmoid": synth.SIGMOID}
MAPS = ("topk_ids", "perm_to_unperm", "unperm_to_perm", "perm_expert", "expert_offsets")
ORACLE_KEY = {"topk_ids": "ids", "perm_to_unperm": "perm_to_unperm",
              "unperm_to_perm": "unperm_to_perm", "perm_expert": "perm_expert",
              "expert_offsets": "expert_offsets"}


def check(x_st, x64, dtype, K, sf="softmax", renorm=False, view=False, what=""):
    T, E = x64.shape
    say(f"[route maps] {what} T={T} E={E} K={K} {sf} renorm={renorm} dtype={dtype}")
    if view:
        big = np.zeros((T * E + 1,), x_st.dtype)
        big[1:] = x_st.ravel()
        xt = to_dev(big, dtype)[1:].view(T, E)
    else:
        xt = to_dev(x_st, dtype)
    r = router.router_route_maps(xt, K, sf, renorm)
    torch.cuda.synchronize()
    ref = oracle.route_maps(x64, K, SF[sf], renorm)
    for f in MAPS:
        got = r[f].cpu().numpy()
        want = ref[ORACLE_KEY[f]].reshape(got.shape)
        assert (got == want).all(), (what, f, got.tolist()[:16], want.tolist()[:16])
    assert_close(r["topk_weights"].cpu().numpy(), ref["weights"], synth.F32,
                 f"{what} weights")
    return r


def normal_logits(seed, T, E, dtype, std=1.0):
    return synth.storage(synth.normal(seed, (T, E), std), dtype)


@pytest.mark.parametrize("T", [1, 2, 3, 4])
@pytest.mark.parametrize("K", [1, 2, 4, 6, 8, 10])
@pytest.mark.parametrize("renorm", [False, True])
def test_decode_shapes(T, K, renorm):
    """The page's shapes: up to 4 rows, 512 experts, k in {1,2,4,6,8,10}."""
    for dtype in (synth.F32, synth.BF16):
        st, x64 = normal_logits(8000 + 10 * T + K, T, 512, dtype)
        check(st, x64, dtype, K, "softmax", renorm, what="decode")


@pytest.mark.parametrize("T,E,K,sf,renorm", [
    (16, 512, 10, "softmax", True), (16, 1024, 32, "softmax", False), (5, 1, 1, "softmax", True),
    (7, 7, 3, "sigmoid", True), (4, 255, 8, "sigmoid", False), (9, 1000, 17, "softmax", True),
    (3, 64, 32, "softmax", True), (3, 32, 32, "sigmoid", False), (2, 33, 1, "sigmoid", True), (11, 257, 32, "sigmoid", True),
])
def test_edge_shapes(T, E, K, sf, renorm):
    st, x64 = normal_logits(8100 + T + E + K, T, E, synth.F32, std=2.0)
    check(st, x64, synth.F32, K, sf, renorm, what="edge")


def test_tied_logits():
    """Integer logits (heavy ties) and bf16 duplicates: slots and maps
    follow the lower expert index on ties."""
    rng = np.random.default_rng(81)
    x = rng.integers(-2, 3, (4, 512)).astype(np.float32)
    check(x, x.astype(np.float64), synth.F32, 10, "softmax", True, what="integer ties")
    x = np.zeros((3, 512), np.float32)
    check(x, x.astype(np.float64), synth.F32, 8, "softmax", False, what="all equal")
    st, x64 = normal_logits(82, 4, 512, synth.BF16, std=0.05)   # many bf16 duplicates
    check(st, x64, synth.BF16, 6, "softmax", True, what="bf16 duplicates")
    x = np.array([[0.0, -0.0, 0.0, -0.0, 1.0, 1.0]], np.float32)
    check(x, x.astype(np.float64), synth.F32, 4, "softmax", False, what="signed zeros")


def test_unaligned_views():
    st, x64 = normal_logits(83, 4, 512, synth.F32)
    check(st, x64, synth.F32, 8, "softmax", True, view=True, what="unaligned f32")
    st, x64 = normal_logits(84, 3, 512, synth.BF16)
    check(st, x64, synth.BF16, 6, "softmax", False, view=True, what="unaligned bf16")


def test_zero_rows_write_zero_offsets():
    x = torch.zeros((0, 512), device=DEV)
    out = {"expert_offsets": torch.full((513,), 9, dtype=torch.int64, device=DEV)}
    r = router.router_route_maps(x, 4, out=out)
    torch.cuda.synchronize()
    assert (r["expert_offsets"].cpu() == 0).all()


def test_deterministic_and_graph_replay():
    st, x64 = normal_logits(85, 4, 512, synth.F32)
    xt = to_dev(st, synth.F32)
    first = router.router_route_maps(xt, 10, "softmax", True)
    torch.cuda.synchronize()
    keep = {k: v.clone() for k, v in first.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            router.router_route_maps(xt, 10, "softmax", True, out=first)
    torch.cuda.synchronize()
    for i in range(4):
        for v in first.values():
            v.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in keep.items():
            assert torch.equal(first[k], v), (i, k)
