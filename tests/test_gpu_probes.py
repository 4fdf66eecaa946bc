"""The measurement probes of include/swa_probe.h on the GPU: the streaming read
sums exactly what it reads, and the MFMA loop gives finite, repeatable output."""

import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("grid", [1, 7, 64])
def test_probe_read_sums_every_element_once(grid):
    from sliding_window_attention_swa_amd import swa
    n = 4 * 1000 + 4 * 3  # floats, a multiple of 4 (16-byte loads) that no grid divides evenly
    buf = torch.arange(n, dtype=torch.float32, device="cuda") % 7
    out = torch.full((grid * 256,), float("nan"), dtype=torch.float32, device="cuda")
    swa.swa_probe_read(buf, out, grid)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()  # every thread wrote its sum
    assert out.double().sum().item() == buf.double().sum().item()  # small integers: exact in f32


def test_probe_mfma_repeatable():
    from sliding_window_attention_swa_amd import swa
    grid, iters = 16, 64
    a = torch.full((grid * 256,), float("nan"), dtype=torch.float32, device="cuda")
    b = torch.full_like(a, float("nan"))
    swa.swa_probe_mfma(a, grid, iters)
    swa.swa_probe_mfma(b, grid, iters)
    torch.cuda.synchronize()
    assert torch.isfinite(a).all() and (a > 0).all()
    assert torch.equal(a, b)


@pytest.mark.parametrize("grid", [1, 5, 64])
def test_probe_copy_copies_every_byte(grid):
    from sliding_window_attention_swa_amd import swa
    src = torch.randint(0, 256, (16 * 1003,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros(16 * 1003 + 64, dtype=torch.uint8, device="cuda")
    swa.swa_probe_copy(src, dst[:src.numel()], grid)
    torch.cuda.synchronize()
    assert torch.equal(dst[:src.numel()], src)
    assert int(dst[src.numel():].count_nonzero()) == 0  # nothing written past the end
