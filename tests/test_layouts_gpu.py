"""GPU parity of the transposed-operand plans (gemm_epilog_plan_ex) against the CPU
oracle, through the C ABI: A handed over as its (k, m) transpose (the backward's
dX = W^T . dY with W as stored), B as its (n, k) transpose (the weight gradient
dW = dZ . X^T with X as stored), or both.

* integer-valued inputs: D, the mask and bgrad equal the oracle bit for bit, for every
  epilogue but GELU, both 16-bit types, the tiles with layouts (256 x 256 "LH", 128 x 128
  "LM" and "LMD", the same tile with a 3-stage ring), ragged n, several k-tiles and a
  ragged k tail (and a ragged m where A is not transposed);
* random normal inputs: the fused-epilogue tolerances and the rounding-model ratio;
* the same tile on the same data gives the same bits whatever the operands' order.
"""
import numpy as np
import pytest
import torch

import oracle
from gemm_epilogues_epilog_amd import inputs
from tests import gpu_runner as R
from tests.helpers import assert_bgrad, assert_close, assert_mask, tight_ratio, to_np

pytestmark = pytest.mark.gpu

LAYOUTS = {"TN": (True, False), "NT": (False, True), "TT": (True, True)}
TILES = [None, "L", "LH", "LM", "LMD"]
# the last two run the persistent kernel under "L" (k a multiple of 64 over an even number
# of at least 4 k-tiles); the others fall back to one workgroup per tile
INT_SHAPES = [(8, 8, 8), (40, 136, 72), (200, 264, 200), (304, 520, 136), (512, 520, 256), (264, 392, 512)]
RAGGED_M = [(33, 136, 72), (300, 520, 256)]   # A not transposed: m need not be a multiple of 8


def stored(t: torch.Tensor, trans: bool) -> torch.Tensor:
    """The operand in the storage order the plan expects."""
    return t.t().contiguous() if trans else t


def cases_int():
    for dt in ("f16", "bf16"):
        for lay, (ta, tb) in LAYOUTS.items():
            for tile in TILES:
                for shape in INT_SHAPES + (RAGGED_M if not ta else []):
                    yield dt, lay, tile, shape


@pytest.mark.parametrize("dt,lay,tile,shape", list(cases_int()))
def test_integer_exact_layouts(gpu, dt, lay, tile, shape):
    ta, tb = LAYOUTS[lay]
    m, n, k = shape
    print(f"[case] integer {dt} {lay} tile {tile} m={m} n={n} k={k}", flush=True)
    A, B, bias, A2, B2 = inputs.integer_case(m, n, k, dt)
    As, Bs = stored(A, ta), stored(B, tb)
    a, b, c = to_np(As), to_np(Bs), to_np(bias)
    kw = dict(trans_a=ta, trans_b=tb)
    for ep in ("NONE", "BIAS", "RELU_BIAS", "RELU_BIAS_UNFUSED"):
        g = R.run(gpu, ep, dt, As, Bs, bias, tile=tile, **kw)
        o = oracle.gemm_epilog(a, b, ep, bias=c, ab=dt, **kw)
        assert np.array_equal(g["D"].view(np.uint8), o["D"].view(np.uint8)), f"{ep} {g['desc']}"
    g = R.run(gpu, "RELU_AUX_BIAS", dt, As, Bs, bias, tile=tile, **kw)
    o = oracle.gemm_epilog(a, b, "RELU_AUX_BIAS", bias=c, ab=dt, **kw)
    assert np.array_equal(g["D"].view(np.uint8), o["D"].view(np.uint8)), g["desc"]
    assert np.array_equal(g["mask"].view(np.uint32), o["mask"]), g["desc"]
    mask = torch.from_numpy(o["mask"].view(np.int32).copy())
    A2s, B2s = stored(A2, ta), stored(B2, tb)
    gb = R.run(gpu, "DRELU_BGRAD", dt, A2s, B2s, mask=mask, tile=tile, **kw)
    ob = oracle.gemm_epilog(to_np(A2s), to_np(B2s), "DRELU_BGRAD", mask=o["mask"], ab=dt, **kw)
    assert np.array_equal(gb["D"].view(np.uint8), ob["D"].view(np.uint8)), gb["desc"]
    assert np.array_equal(gb["bgrad"].view(np.uint8), ob["bgrad"].view(np.uint8)), gb["desc"]
    gu = R.run(gpu, "DRELU_BGRAD_UNFUSED", dt, A2s, B2s, act=g["D_dev"], tile=tile, **kw)
    ou = oracle.gemm_epilog(to_np(A2s), to_np(B2s), "DRELU_BGRAD_UNFUSED", act=g["D"], ab=dt, **kw)
    assert np.array_equal(gu["D"].view(np.uint8), ou["D"].view(np.uint8)), gu["desc"]
    assert np.array_equal(gu["bgrad"].view(np.uint8), ou["bgrad"].view(np.uint8)), gu["desc"]


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("lay", list(LAYOUTS))
@pytest.mark.parametrize("shape", [(64, 48, 32), (136, 200, 264), (256, 392, 520), (1024, 512, 2048)])
def test_random_parity_layouts(gpu, dt, lay, shape):
    ta, tb = LAYOUTS[lay]
    m, n, k = shape
    print(f"[case] random {dt} {lay} m={m} n={n} k={k}", flush=True)
    A, B, bias, A2, B2 = inputs.small_case(m, n, k, dt, std=1.0, std_bias=1.0)
    As, Bs = stored(A, ta), stored(B, tb)
    a, b, c = to_np(As), to_np(Bs), to_np(bias)
    wa, wb = oracle.to_f32(to_np(A), dt), oracle.to_f32(to_np(B), dt)
    kw = dict(trans_a=ta, trans_b=tb)
    for ep in ("RELU_BIAS", "GELU_BIAS", "BIAS"):
        g = R.run(gpu, ep, dt, As, Bs, bias, **kw)
        o = oracle.gemm_epilog(a, b, ep, bias=c, ab=dt, **kw)
        assert_close(g["D"], o["D"], dt, f"{ep} {g['desc']}")
        r = tight_ratio(g["D"], o["D"], dt, wa, wb, 1.13 if ep == "GELU_BIAS" else 1.0)
        assert r <= 4.0, f"{ep} {g['desc']}: rounding-model ratio {r}"
    g = R.run(gpu, "RELU_AUX_BIAS", dt, As, Bs, bias, **kw)
    o = oracle.gemm_epilog(a, b, "RELU_AUX_BIAS", bias=c, ab=dt, want_pre=True, **kw)
    assert_close(g["D"], o["D"], dt, g["desc"])
    assert_mask(g["mask"], o["mask"], o["pre"], m)
    mask = torch.from_numpy(g["mask"].view(np.int32).copy())   # the GPU forward's mask
    A2s, B2s = stored(A2, ta), stored(B2, tb)
    gb = R.run(gpu, "DRELU_BGRAD", dt, A2s, B2s, mask=mask, **kw)
    ob = oracle.gemm_epilog(to_np(A2s), to_np(B2s), "DRELU_BGRAD", mask=g["mask"].view(np.uint32), ab=dt, **kw)
    assert_close(gb["D"], ob["D"], dt, gb["desc"])
    assert_bgrad(gb["bgrad"], ob["bgrad"], ob["absum"], dt)
    gu = R.run(gpu, "DRELU_BGRAD_UNFUSED", dt, A2s, B2s, act=g["D_dev"], **kw)
    ou = oracle.gemm_epilog(to_np(A2s), to_np(B2s), "DRELU_BGRAD_UNFUSED", act=g["D"], ab=dt, **kw)
    assert_close(gu["D"], ou["D"], dt, gu["desc"])
    assert_bgrad(gu["bgrad"], ou["bgrad"], ou["absum"], dt)


@pytest.mark.parametrize("tile", ["L", "LH", "LM", "LMD"])
def test_layout_does_not_change_bits(gpu, tile):
    # one tile configuration, one k order: the storage order of the operands only changes
    # how they reach LDS, so the random-input results agree bit for bit (the reference
    # keeps whole tiles, as the transposed plans always do: a split k loop adds its
    # partial sums in another order)
    m, n, k = 512, 520, 1024
    A, B, bias, A2, B2 = inputs.small_case(m, n, k, "bf16")
    ref = R.run(gpu, "RELU_AUX_BIAS", "bf16", A, B, bias, tile=tile + "-nosk")
    if tile == "L":
        assert "persistent workgroups" in ref["desc"], ref["desc"]
    for lay, (ta, tb) in LAYOUTS.items():
        g = R.run(gpu, "RELU_AUX_BIAS", "bf16", stored(A, ta), stored(B, tb), bias, tile=tile,
                  trans_a=ta, trans_b=tb)
        assert np.array_equal(g["D"], ref["D"]) and np.array_equal(g["mask"], ref["mask"]), f"{lay} {g['desc']}"


def test_plan_describes_layout(gpu):
    ge = gpu
    h = ge.gemm_epilog_plan_ex(4096, 4096, 512, ("bf16", "bf16", "bf16"), "DRELU_BGRAD", 1, 0)
    try:
        d = ge.gemm_epilog_describe(h)
        assert "op_a T op_b N" in d and "tile 256x256" in d and "persistent workgroups" in d, d
    finally:
        ge.gemm_epilog_free(h)
    h = ge.gemm_epilog_plan_ex(256, 256, 512, ("f16", "f16", "f16"), "NONE", 0, 1)
    try:
        d = ge.gemm_epilog_describe(h)
        assert "op_a N op_b T" in d and "tile 128x128" in d, d
    finally:
        ge.gemm_epilog_free(h)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("lay", list(LAYOUTS))
@pytest.mark.parametrize("tile", [None, "L"])
def test_integer_exact_fp32_vectors_layouts(gpu, dt, lay, tile):
    # fp32 bias and bgrad with 16-bit matrices handed over transposed
    ta, tb = LAYOUTS[lay]
    m, n, k = 264, 392, 512
    A, B, bias, A2, B2 = inputs.integer_case(m, n, k, dt, vec="f32")
    As, Bs, A2s, B2s = stored(A, ta), stored(B, tb), stored(A2, ta), stored(B2, tb)
    kw = dict(trans_a=ta, trans_b=tb)
    o = oracle.gemm_epilog(to_np(As), to_np(Bs), "RELU_AUX_BIAS", bias=to_np(bias), ab=dt, vec="f32", **kw)
    g = R.run(gpu, "RELU_AUX_BIAS", dt, As, Bs, bias, vec="f32", tile=tile, **kw)
    assert np.array_equal(g["D"].view(np.uint8), o["D"].view(np.uint8)), g["desc"]
    assert np.array_equal(g["mask"].view(np.uint32), o["mask"]), g["desc"]
    mask = torch.from_numpy(o["mask"].view(np.int32).copy())
    gb = R.run(gpu, "DRELU_BGRAD", dt, A2s, B2s, mask=mask, vec="f32", tile=tile, **kw)
    ob = oracle.gemm_epilog(to_np(A2s), to_np(B2s), "DRELU_BGRAD", mask=o["mask"], ab=dt, vec="f32", **kw)
    assert np.array_equal(gb["D"].view(np.uint8), ob["D"].view(np.uint8)), gb["desc"]
    assert np.array_equal(gb["bgrad"], ob["bgrad"]), gb["desc"]


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("lay", list(LAYOUTS))
def test_random_parity_layouts_persistent(gpu, dt, lay):
    # the persistent kernel with transposed operands on normal inputs: GELU (not exact
    # on integers) and the ReLU mask within the tolerances
    ta, tb = LAYOUTS[lay]
    m, n, k = 520, 776, 1024
    A, B, bias, _, _ = inputs.small_case(m, n, k, dt, std=1.0, std_bias=1.0)
    As, Bs = stored(A, ta), stored(B, tb)
    a, b, c = to_np(As), to_np(Bs), to_np(bias)
    wa, wb = oracle.to_f32(to_np(A), dt), oracle.to_f32(to_np(B), dt)
    kw = dict(trans_a=ta, trans_b=tb)
    g = R.run(gpu, "GELU_BIAS", dt, As, Bs, bias, tile="L", **kw)
    assert "persistent workgroups" in g["desc"], g["desc"]
    o = oracle.gemm_epilog(a, b, "GELU_BIAS", bias=c, ab=dt, **kw)
    assert_close(g["D"], o["D"], dt, g["desc"])
    assert tight_ratio(g["D"], o["D"], dt, wa, wb, 1.13) <= 4.0
    g = R.run(gpu, "RELU_AUX_BIAS", dt, As, Bs, bias, tile="L", **kw)
    o = oracle.gemm_epilog(a, b, "RELU_AUX_BIAS", bias=c, ab=dt, want_pre=True, **kw)
    assert_close(g["D"], o["D"], dt, g["desc"])
    assert_mask(g["mask"], o["mask"], o["pre"], m)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("lay", list(LAYOUTS))
def test_persistent_transposed_many_tiles_integer_exact(gpu, dt, lay):
    """The persistent kernel with operands stored transposed walks several tiles per
    workgroup: 528 tiles of a ragged 4000 x 8200 output on 256 workgroups, so every tile
    after a workgroup's first starts from operands its copy plan fetched during the
    previous tile (the retargeted k-major and mn-major copies, with their row and column
    limits on the ragged tiles). Integer inputs make every epilogue bit-exact."""
    ta, tb = LAYOUTS[lay]
    m, n, k = 4000, 8200, 256
    print(f"[case] persistent transposed integer {dt} {lay} m={m} n={n} k={k}", flush=True)
    A, B, bias, A2, B2 = inputs.integer_case(m, n, k, dt)
    As, Bs = stored(A, ta), stored(B, tb)
    a, b, c = to_np(A), to_np(B), to_np(bias)   # the oracle on the product's own orientation
    kw = dict(trans_a=ta, trans_b=tb)
    for ep in ("NONE", "BIAS", "RELU_BIAS"):
        g = R.run(gpu, ep, dt, As, Bs, bias, tile="L", **kw)
        assert "persistent workgroups" in g["desc"] and "grid 528" in g["desc"], g["desc"]
        o = oracle.gemm_epilog(a, b, ep, bias=c, ab=dt)
        assert np.array_equal(g["D"].view(np.uint8), o["D"].view(np.uint8)), f"{ep} {g['desc']}"
    g = R.run(gpu, "RELU_AUX_BIAS", dt, As, Bs, bias, tile="L", **kw)
    o = oracle.gemm_epilog(a, b, "RELU_AUX_BIAS", bias=c, ab=dt)
    assert np.array_equal(g["D"].view(np.uint8), o["D"].view(np.uint8)), g["desc"]
    assert np.array_equal(g["mask"].view(np.uint32), o["mask"]), g["desc"]
    mask = torch.from_numpy(o["mask"].view(np.int32).copy())
    gb = R.run(gpu, "DRELU_BGRAD", dt, stored(A2, ta), stored(B2, tb), mask=mask, tile="L", **kw)
    assert "persistent workgroups" in gb["desc"], gb["desc"]
    ob = oracle.gemm_epilog(to_np(A2), to_np(B2), "DRELU_BGRAD", mask=o["mask"], ab=dt)
    assert np.array_equal(gb["D"].view(np.uint8), ob["D"].view(np.uint8)), gb["desc"]
    assert np.array_equal(gb["bgrad"].view(np.uint8), ob["bgrad"].view(np.uint8)), gb["desc"]
