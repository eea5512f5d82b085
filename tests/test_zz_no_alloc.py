"""The aux-loss forward that allocates nothing (router_aux_loss_fwd_noalloc)
against the workspace entry point (router_aux_loss_fwd), through the C ABI:
the same kernels in the same order, so the loss must be the same bits; the
oracle's loss brackets both.  Two calls in a row, the second on a smaller
input (the library's buffer keeps the first call's partials, which the
second must not read), then once more on the first shape."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from gpu_support import DEV, F32_ATOL, F32_RTOL, say, to_dev
from score_function_top_amd import router, synth

pytestmark = pytest.mark.gpu
COEFF = synth.AUX_LOSS_COEFF


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    router.load()


def _inputs(T, E, K, seed, dtype):
    st, s64 = synth.prob_like(seed, T, E, dtype)
    counts = oracle.tokens_per_expert(synth.random_map(seed + 1, T, E, K))
    return to_dev(st, dtype), s64, torch.from_numpy(counts).to(DEV), counts


def _noalloc(lib, scores, counts, N, K, loss):
    T, E = scores.shape
    dt = router.F32 if scores.dtype == torch.float32 else router.BF16
    stream = ctypes.c_void_p(torch.cuda.current_stream(scores.device).cuda_stream)
    return lib.router_aux_loss_fwd_noalloc(
        ctypes.c_void_p(scores.data_ptr()), dt, T, E, ctypes.c_void_p(counts.data_ptr()), N, K,
        ctypes.c_float(COEFF), ctypes.c_void_p(loss.data_ptr()), stream)


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_noalloc_matches_workspace_entry(dtype):
    lib = router.load()
    shapes = [(8192, 2304, 36), (1031, 256, 8), (8192, 2304, 36)]   # then smaller, then again
    for i, (T, E, K) in enumerate(shapes):
        say(f"[noalloc] call {i}: T={T} E={E} K={K} dtype={dtype}")
        s, s64, c, c_np = _inputs(T, E, K, 7700 + i, dtype)
        want = router.router_aux_loss_fwd(s, c, T, K, COEFF)
        got = torch.full((), float("nan"), dtype=torch.float32, device=DEV)
        assert _noalloc(lib, s, c, T, K, got) == router.OK
        torch.cuda.synchronize()
        assert got.view(torch.int32).item() == want.view(torch.int32).item(), \
            (i, got.item(), want.item())
        ref = oracle.aux_loss(s64, c_np, K, COEFF)
        assert abs(got.item() - ref) <= F32_ATOL + F32_RTOL * abs(ref), (i, got.item(), ref)


def test_noalloc_zero_rows_and_errors():
    lib = router.load()
    E = 64
    s = torch.empty((0, E), dtype=torch.float32, device=DEV)
    c = torch.zeros(E, dtype=torch.int64, device=DEV)
    out = torch.full((), 7.0, dtype=torch.float32, device=DEV)
    assert _noalloc(lib, s, c, 5, 2, out) == router.OK
    torch.cuda.synchronize()
    assert out.item() == 0.0
    # invalid arguments are rejected before any launch and write nothing
    s2 = torch.rand((16, E), device=DEV)
    assert _noalloc(lib, s2, c, 0, 2, out) == router.ERR_INVALID_ARG      # N = 0
    torch.cuda.synchronize()
    assert out.item() == 0.0
