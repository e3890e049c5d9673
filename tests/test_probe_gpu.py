"""The MFMA-only probe (include/gemm_epilog_probe.h) on the GPU: it runs, writes every
output, and its sums follow from the operands (zero operands give zero; the rest are
finite); its argument errors come back before any launch."""
import pytest
import torch

from gemm_epilogues_epilog_amd import probe as gprobe

pytestmark = pytest.mark.gpu


def test_mfma_probe_runs_and_writes_every_output(gpu):
    wgs, iters = 8, 16
    out = torch.full((wgs * 256,), float("nan"), dtype=torch.float32, device="cuda")
    zeros = torch.zeros(4096, dtype=torch.float16, device="cuda")
    gprobe.gemm_epilog_mfma_probe(zeros, "f16", iters, wgs, out)
    torch.cuda.synchronize()
    assert bool((out == 0).all())
    g = torch.Generator(device="cuda").manual_seed(0)
    vals = (torch.randn(4096, device="cuda", generator=g) / 64).to(torch.bfloat16)
    out.fill_(float("nan"))
    gprobe.gemm_epilog_mfma_probe(vals, "bf16", iters, wgs, out)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()) and bool((out != 0).any())
    assert gprobe.gemm_epilog_mfma_probe(vals, "f32", iters, wgs, out, check=False) == 2


def test_device_info_matches_torch(gpu):
    cus, mhz = gprobe.gemm_epilog_device_info()
    assert cus == torch.cuda.get_device_properties(0).multi_processor_count
    assert 500.0 <= mhz <= 5000.0
