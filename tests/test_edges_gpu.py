"""The size limits of the C ABI on the GPU, against the CPU oracle: n = 2^20 and m just
past 2^21 (integer-valued, bit for bit, with the mask and the backward), k = 2^20 (a
single tile whose k loop is split across workgroups; random inputs, tolerance), and
m = 2^20 with A transposed, n = 2^20 with B transposed (the largest rows those layouts
accept)."""
import numpy as np
import pytest
import torch

import oracle
from gemm_epilogues_epilog_amd import inputs
from tests import gpu_runner as R
from tests.helpers import assert_close, tight_ratio, to_np

pytestmark = pytest.mark.gpu

BIG = 1 << 20


def _same(x, y):
    return np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8))


def _integer_round_trip(gpu, dt, m, n, k, ta=False, tb=False):
    A, B, bias, A2, B2 = inputs.integer_case(m, n, k, dt)
    As = A.t().contiguous() if ta else A
    Bs = B.t().contiguous() if tb else B
    kw = dict(trans_a=ta, trans_b=tb)
    g = R.run(gpu, "RELU_AUX_BIAS", dt, As, Bs, bias, **kw)
    o = oracle.gemm_epilog(to_np(As), to_np(Bs), "RELU_AUX_BIAS", bias=to_np(bias), ab=dt, **kw)
    assert _same(g["D"], o["D"]) and _same(g["mask"], o["mask"]), g["desc"]
    mask = torch.from_numpy(o["mask"].view(np.int32).copy())
    A2s = A2.t().contiguous() if ta else A2
    B2s = B2.t().contiguous() if tb else B2
    gb = R.run(gpu, "DRELU_BGRAD", dt, A2s, B2s, mask=mask, **kw)
    ob = oracle.gemm_epilog(to_np(A2s), to_np(B2s), "DRELU_BGRAD", mask=o["mask"], ab=dt, **kw)
    assert _same(gb["D"], ob["D"]) and _same(gb["bgrad"], ob["bgrad"]), gb["desc"]
    return g["desc"], gb["desc"]


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_widest_n(gpu, dt):
    print(f"[case] edge n=2^20 {dt}", flush=True)
    _integer_round_trip(gpu, dt, 8, BIG, 8)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_tallest_m(gpu, dt):
    m = (1 << 21) + 5
    print(f"[case] edge m={m} {dt}", flush=True)
    _integer_round_trip(gpu, dt, m, 8, 8)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_transposed_operands_at_their_limits(gpu, dt):
    print(f"[case] edge m=2^20 with A transposed, n=2^20 with B transposed {dt}", flush=True)
    d1, _ = _integer_round_trip(gpu, dt, BIG, 8, 8, ta=True)
    d2, _ = _integer_round_trip(gpu, dt, 8, BIG, 8, tb=True)
    assert "op_a T" in d1 and "op_b T" in d2


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_deepest_k(gpu, dt):
    m, n, k = 40, 8, BIG
    print(f"[case] edge k=2^20 {dt}", flush=True)
    A, B, bias, _, _ = inputs.small_case(m, n, k, dt, std=k ** -0.25, std_bias=0.5)
    g = R.run(gpu, "RELU_BIAS", dt, A, B, bias)
    o = oracle.gemm_epilog(to_np(A), to_np(B), "RELU_BIAS", bias=to_np(bias), ab=dt)
    assert_close(g["D"], o["D"], dt, g["desc"])
    r = tight_ratio(g["D"], o["D"], dt, oracle.to_f32(to_np(A), dt), oracle.to_f32(to_np(B), dt))
    assert r <= 4.0, f"{g['desc']}: rounding-model ratio {r}"
