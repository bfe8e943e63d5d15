"""txl_probe_mfma on the GPU: every workgroup reports the shader-clock cycles and
100 MHz reference ticks of its first wave's product loop; the cycles cover at
least the matrix-core time of that wave's products (32 cycles per 32x32x16 bf16
product; the wave may finish before the other wave of its SIMD), and the clock
they imply is a plausible one."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def txl():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import transformer_xl_relative_attn_amd as mod
    return mod


def test_probe_reports_cycles_and_clock(txl):
    import torch
    n_wg, iters = 8, 64
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    ops = torch.randn(n_wg * 512 * 24 * 8, generator=gen, device="cuda").to(torch.bfloat16)
    clocks = torch.full((2 * n_wg + 1,), -1, dtype=torch.int64, device="cuda")
    txl.txl_probe_mfma(ops, n_wg, iters, clocks)
    torch.cuda.synchronize()
    c = clocks[:2 * n_wg].view(n_wg, 2).cpu().numpy()
    cycles, ticks = c[:, 0].astype(np.float64), c[:, 1].astype(np.float64)
    assert (ticks > 0).all()
    # 16 products per round, 32 cycles each
    assert (cycles >= 0.9 * iters * 16 * 32).all(), cycles
    ghz = cycles / ticks * 0.1
    assert ((ghz > 0.3) & (ghz < 3.5)).all(), ghz
    with pytest.raises(txl.TxlError):
        txl.txl_probe_mfma(ops, n_wg, 3, clocks)
