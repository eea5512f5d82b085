"""The data-movement kernels that bench.py times as bandwidth references
move what they document (they do no routing work, so there is no oracle:
the expected outputs are copies of the input and its sign bits)."""
import pytest
import torch

from gpu_support import DEV, say
from score_function_top_amd import router

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("units", [1, 2, 4, 8])
@pytest.mark.parametrize("rb,wb", [(4096, 8192), (8192, 4096), (65536 + 48, 16 * 40000),
                                   (0, 4096), (4096, 0)])
def test_stream_copies_the_read_part(units, rb, wb):
    g = torch.Generator(DEV).manual_seed(11 + units)
    src = torch.randint(0, 256, (max(rb, 16),), dtype=torch.uint8, device=DEV, generator=g)
    dst = torch.zeros(max(wb, 16), dtype=torch.uint8, device=DEV)
    say(f"[bandwidth refs] stream {rb} read, {wb} written, {units} units per thread")
    router.stream_bandwidth(src, rb, dst, wb, units)
    torch.cuda.synchronize()
    n = min(rb, wb)
    assert torch.equal(dst[:n], src[:n])


@pytest.mark.parametrize("T,E", [(37, 256), (37, 2304), (5, 4096), (0, 512)])
def test_row_stream_writes_rows_and_sign_bytes(T, E):
    g = torch.Generator(DEV).manual_seed(T + E)
    x = torch.randn(T, E, device=DEV, generator=g)
    a = torch.zeros_like(x)
    b = torch.zeros_like(x)
    m = torch.full((T, E), 7, dtype=torch.uint8, device=DEV)
    say(f"[bandwidth refs] row stream T={T} E={E}")
    router.row_stream_bandwidth(x, a, b, m)
    torch.cuda.synchronize()
    assert torch.equal(a, x) and torch.equal(b, x)
    assert torch.equal(m, (torch.signbit(x)).to(torch.uint8))
