"""The plan's own configuration at the shapes its tile rule was measured on.

Each shape runs the configuration the plan picks for it: the persistent 256 x 256 tile,
its split tail, the persistent 192 x 256 and 128 x 256 tiles, the 128 x 128 tiles with
two and three stages, split and whole, four waves, and transposed operands, each at its
real grid size. A and B hold integers in [-2, 2] and the bias half-integers, so the fp32
sums are exact and any correct kernel gives the oracle's bits. The oracle recomputes
sampled 32-row groups (the first, the last and random ones): D and the mask words of the
forward (RELU_AUX_BIAS), and D and the bias gradient of the backward (DRELU_BGRAD on the
GPU's own mask), bit for bit; D must also be finite everywhere (it is NaN-filled before
each run, so an element no kernel wrote fails)."""
import numpy as np
import pytest
import torch

import oracle
from gemm_epilogues_epilog_amd import inputs
from tests import gpu_runner as R
from tests.helpers import assert_all_finite, to_np

pytestmark = pytest.mark.gpu

# (m, n, k), operand order, type, the tile (tile_m, tile_n) the plan picks
SHAPES = [
    ((4096, 2752, 4096), "NN", "f16", (192, 256)),    # 242 tiles of 192 x 256: one round
    ((8448, 4096, 4096), "NN", "bf16", (192, 256)),   # 704 tiles: 2.75 rounds
    ((4000, 2744, 4096), "NN", "f16", None),          # ragged m and n near the first
    ((4352, 4096, 4096), "NN", "bf16", (256, 256)),   # 272 tiles, a split last round of 16
    ((4096, 3200, 4096), "NN", "f16", (256, 256)),    # persistent, 208 tiles
    ((2048, 1024, 16384), "NN", "bf16", (256, 256)),  # split k loop, 256 k-tiles
    ((2048, 1024, 8192), "NN", "f16", (128, 128)),    # three stages, split runs of 64 k-tiles
    ((1024, 1024, 4096), "NN", "bf16", (128, 128)),   # three stages, split runs of 16 k-tiles
    ((4096, 1376, 4096), "NN", "f16", (128, 128)),    # four waves of 64 x 64, two workgroups per CU
    ((3072, 2560, 4096), "NN", "bf16", (128, 256)),   # persistent 128 x 256, one round
    ((3000, 2552, 4096), "NN", "f16", None),          # ragged m and n near the last
    ((2048, 2048, 1024), "NN", "bf16", (128, 128)),   # two stages, whole
    ((8192, 1024, 8192), "TN", "bf16", (128, 128)),   # A transposed: never split
    ((4096, 2752, 4096), "NT", "f16", (256, 256)),    # B transposed: the persistent 256 x 256 tile
    ((4096, 2752, 4040), "NN", "bf16", (192, 256)),   # a ragged last k-tile: one workgroup per tile
    ((4000, 11000, 1000), "NN", "f16", (256, 256)),   # ragged m, n and k on the 256 x 256 tile
]


def groups_of(m, count=5, seed=7):
    g = (m + 31) // 32
    rng = np.random.default_rng(seed + m)
    mid = sorted(set(rng.choice(np.arange(1, g - 1), size=min(count, g - 2), replace=False).tolist()))
    return [0] + mid + [g - 1]   # the ragged last group, if any, comes last


@pytest.mark.parametrize("shape,lay,dt,tile", SHAPES)
def test_plan_choice_integer_exact(gpu, shape, lay, dt, tile):
    m, n, k = shape
    print(f"[case] plan shape {dt} {lay} m={m} n={n} k={k}", flush=True)
    A, B, bias, _, _ = inputs.integer_case(m, n, k, dt, second=False)
    ta, tb = lay[0] == "T", lay[1] == "T"
    Ad = A.t().contiguous() if ta else A
    Bd = B.t().contiguous() if tb else B
    info = gpu.gemm_epilog_plan_info(m, n, k, (dt, dt, dt), "RELU_AUX_BIAS", op_a=int(ta), op_b=int(tb))
    if tile is not None:
        assert (info["tile_m"], info["tile_n"]) == tile, info

    g = R.run(gpu, "RELU_AUX_BIAS", dt, Ad, Bd, bias, trans_a=ta, trans_b=tb)
    assert_all_finite(g["D_dev"], f"{shape} {lay} D")
    groups = groups_of(m)
    rows = np.concatenate([np.arange(32 * q, min(m, 32 * q + 32)) for q in groups])
    a, b, c = to_np(A)[rows], to_np(B), to_np(bias)[rows]
    o = oracle.gemm_epilog(a, b, "RELU_AUX_BIAS", bias=c, ab=dt)
    assert np.array_equal(g["D"][rows].view(np.uint8), o["D"].view(np.uint8)), g["desc"]
    assert np.array_equal(g["mask"].view(np.uint32)[groups], o["mask"]), g["desc"]

    gb = R.run(gpu, "DRELU_BGRAD", dt, Ad, Bd, mask=g["mask_dev"], trans_a=ta, trans_b=tb)
    assert_all_finite(gb["D_dev"], f"{shape} {lay} backward D")
    ob = oracle.gemm_epilog(a, b, "DRELU_BGRAD", mask=o["mask"], ab=dt)
    assert np.array_equal(gb["D"][rows].view(np.uint8), ob["D"].view(np.uint8)), gb["desc"]
    assert np.array_equal(gb["bgrad"][rows].view(np.uint8), ob["bgrad"].view(np.uint8)), gb["desc"]
