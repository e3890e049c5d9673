"""Special values through the HIP path against the oracle: infinities and NaN in the
operands (their products and sums follow IEEE arithmetic: +inf rows, -inf rows, +inf
with -inf in one row giving NaN, NaN rows, inf x 0 giving NaN in one column) and fp16
outputs that overflow (RNE: 65519 -> 65504, the tie 65520 -> +inf). Every epilogue but
GELU, every tile configuration; NaN positions must agree and every other element, mask
word and bias gradient must agree bit for bit. GELU: the same NaN and infinity positions,
its finite elements within the path's tolerance. The finite values are small integers, so
no summation order changes them."""
import numpy as np
import pytest
import torch

import oracle
from tests import gpu_runner as R
from tests.helpers import to_np

pytestmark = pytest.mark.gpu

TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
TILES = {"f32": [None, "S", "M"], "f16": [None, "L", "LH", "LM", "LM4", "LMD"], "bf16": [None, "L", "LM", "LMD"]}


def special_operands(m, n, k, dt):
    """A in {-1, 0, 1} and B in {1..4} with the special entries placed in several row
    groups and k-tiles; returns torch tensors in dt."""
    i, kk = np.meshgrid(np.arange(m), np.arange(k), indexing="ij")
    A = ((i * 7 + kk * 3) % 3 - 1).astype(np.float64)
    B = (np.arange(k * n).reshape(k, n) % 4 + 1).astype(np.float64)
    A[0, 5] = np.inf                             # +inf row
    A[1, 40 % k] = -np.inf                       # -inf row
    A[2, 3], A[2, k - 2] = np.inf, -np.inf       # inf - inf: NaN row
    A[3, k // 2] = np.nan                        # NaN row
    A[35 % m, k - 1] = np.inf                    # +inf row, but
    B[k - 1, 7 % n] = 0.0                        # inf x 0: NaN in one column
    A[33 % m, 9], A[33 % m, 10] = -np.inf, -np.inf
    t = TORCH[dt]
    return torch.from_numpy(A).to(t), torch.from_numpy(B).to(t)


def same(got, ref, dt):
    g, r = oracle.to_f32(got, dt), oracle.to_f32(ref, dt)
    gn, rn = np.isnan(g), np.isnan(r)
    assert np.array_equal(gn, rn), f"NaN positions differ: {np.argwhere(gn != rn)[:5]}"
    gb, rb = np.asarray(got).view(np.uint8), np.asarray(ref).view(np.uint8)
    es = g.dtype.itemsize if dt == "f32" else 2
    keep = np.repeat(~gn.reshape(-1), es)
    assert np.array_equal(gb.reshape(-1)[keep], rb.reshape(-1)[keep])


def cases():
    for dt, tiles in TILES.items():
        for tile in tiles:
            for shape in ((40, 136, 72), (300, 264, 256)):
                yield dt, tile, shape


@pytest.mark.parametrize("dt,tile,shape", list(cases()))
def test_special_values_match_oracle(gpu, dt, tile, shape):
    m, n, k = shape
    print(f"[case] special values {dt} tile {tile} m={m} n={n} k={k}", flush=True)
    A, B = special_operands(m, n, k, dt)
    bias = torch.from_numpy((np.arange(m) % 5 - 2).astype(np.float64)).to(TORCH[dt])
    bias[4] = float("nan") if m > 4 else bias[4]
    a, b, c = to_np(A), to_np(B), to_np(bias)
    for ep in ("NONE", "BIAS", "RELU_BIAS"):
        g = R.run(gpu, ep, dt, A, B, bias, tile=tile)
        o = oracle.gemm_epilog(a, b, ep, bias=c, ab=dt)
        same(g["D"], o["D"], dt)
    g = R.run(gpu, "RELU_AUX_BIAS", dt, A, B, bias, tile=tile)
    o = oracle.gemm_epilog(a, b, "RELU_AUX_BIAS", bias=c, ab=dt)
    same(g["D"], o["D"], dt)
    assert np.array_equal(g["mask"].view(np.uint32), o["mask"]), g["desc"]
    # the backward on the same product, with the forward's mask (bits cleared where the
    # product is NaN stay +0; set ones carry the NaN)
    mask = torch.from_numpy(o["mask"].view(np.int32).copy())
    gb = R.run(gpu, "DRELU_BGRAD", dt, A, B, mask=mask, tile=tile, vec="f32")
    ob = oracle.gemm_epilog(a, b, "DRELU_BGRAD", mask=o["mask"], ab=dt, vec="f32")
    same(gb["D"], ob["D"], dt)
    same(gb["bgrad"], ob["bgrad"], "f32")


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_gelu_special_values(gpu, dt):
    # GELU's pre-activations at +inf, -inf and NaN give +inf, NaN and NaN on both sides;
    # the finite elements keep the path's tolerance
    from tests.helpers import assert_close
    m, n, k = 40, 136, 72
    A, B = special_operands(m, n, k, dt)
    bias = torch.zeros(m, dtype=TORCH[dt])
    g = R.run(gpu, "GELU_BIAS", dt, A, B, bias)
    o = oracle.gemm_epilog(to_np(A), to_np(B), "GELU_BIAS", bias=to_np(bias), ab=dt)
    gf, of = oracle.to_f32(g["D"], dt), oracle.to_f32(o["D"], dt)
    assert np.array_equal(np.isnan(gf), np.isnan(of))
    assert np.array_equal(np.isposinf(gf), np.isposinf(of)) and np.array_equal(np.isneginf(gf), np.isneginf(of))
    assert np.isposinf(of).any() and np.isnan(of).any()
    fin = np.isfinite(of)
    assert_close(np.where(fin, g["D"], 0), np.where(fin, o["D"], 0), dt, "GELU finite elements")


@pytest.mark.parametrize("tile", [None, "L", "LH", "LM", "LMD"])
def test_f16_output_overflow(gpu, tile):
    # sums of fp16 integers around the top of fp16's range; k = 8 (five of them zero)
    rows = [[32768, 32736, 0], [32768, 32736, 15], [32768, 32752, 0], [32768, 32768, 0],
            [-32768, -32768, 0], [32768, 32752, -16], [1, 2, 3], [0, 0, 0]]
    m, n, k = 296, 136, 8
    A = np.zeros((m, k))
    for i in range(m):
        A[i, :3] = rows[i % 8]
    A = torch.from_numpy(A).half()
    B = torch.ones(k, n, dtype=torch.float16)
    bias = torch.zeros(m, dtype=torch.float16)
    a, b, c = to_np(A), to_np(B), to_np(bias)
    for ep in ("BIAS", "RELU_BIAS", "NONE"):
        g = R.run(gpu, ep, "f16", A, B, bias, tile=tile)
        o = oracle.gemm_epilog(a, b, ep, bias=c)
        assert np.array_equal(g["D"].view(np.uint16), o["D"].view(np.uint16)), f"{ep} {g['desc']}"
    assert np.isinf(o["D"].astype(np.float32)).any()
