"""The plan's decisions on the host, through gemm_epilog_plan_info (no HIP call): the
measured tile rule, where the persistent kernel and the split tail apply, the tile order
groups, and the workspace. CPU tests; one GPU test checks that a real plan agrees."""
import pytest

import gemm_epilogues_epilog_amd as ge

F16 = ("f16", "f16", "f16")


def info(m, n, k, lay="NN", ep="RELU_BIAS", dts=F16, cus=256):
    return ge.gemm_epilog_plan_info(m, n, k, dts, ep, int(lay[0] == "T"), int(lay[1] == "T"), compute_units=cus)


@pytest.mark.parametrize("shape,lay,tile,waves,stages,split", [  # tile: (tile_m, tile_n)
    ((4096, 11008, 4096), "NN", (256, 256), 8, 2, False),   # the 7B FFN layer: 688 tiles, last round 69% full, not split
    ((4096, 2752, 4096), "NN", (192, 256), 8, 2, False),    # 176 tiles of 256 x 256 in one round; 242 of 192 x 256
    ((3072, 4096, 4096), "NN", (192, 256), 8, 2, False),    # 192 tiles of 256 x 256; 256 of 192 x 256: a full round
    ((6144, 4096, 4096), "NN", (192, 256), 8, 2, False),    # 384 (1.5 rounds) against 512 (2)
    ((8448, 4096, 4096), "NN", (192, 256), 8, 2, False),    # 528 (2 rounds and a split tail) against 704 (2.75)
    ((4352, 4096, 4096), "NN", (256, 256), 8, 2, True),     # 368 of 192 x 256 would split a 112-tile last round
    ((4096, 2752, 4096), "TN", (256, 256), 8, 2, False),    # no 192 x 256 tile for transposed operands
    ((4096, 3200, 4096), "NN", (256, 256), 8, 2, False),    # 208 tiles; 286 of 192 x 256 would take 2 rounds
    ((4096, 4096, 4096), "NN", (256, 256), 8, 2, False),
    ((4096, 2048, 8192), "NN", (256, 256), 8, 2, True),     # half a round: the 256 x 256 split already fills the CUs
    ((8192, 1024, 8192), "NN", (256, 256), 8, 2, True),     # 128 tiles, 128 k-tiles: split k loop
    ((2048, 2048, 8192), "NN", (256, 256), 8, 2, True),     # 256 tiles of 128 x 128 would fill the CUs unsplit
    ((2048, 1024, 16384), "NN", (256, 256), 8, 2, True),    # its 128 x 128 split would run 128 k-tiles per run
    ((2048, 1024, 8192), "NN", (128, 128), 8, 3, True),     # 128 tiles of 128 x 128, runs of 64 k-tiles
    ((1024, 1024, 8192), "NN", (128, 128), 8, 3, True),
    ((512, 512, 8192), "NN", (128, 128), 8, 3, True),
    ((4096, 1376, 4096), "NN", (128, 128), 4, 2, False),    # 352 tiles of 128 x 128: one round at two per CU (n pads to 1536)
    ((3072, 2560, 4096), "NN", (128, 256), 8, 2, False),    # 240 tiles of 128 x 256 in one round
    ((2048, 4096, 4096), "NN", (128, 256), 8, 2, False),
    ((2048, 4096, 8192), "NN", (256, 256), 8, 2, True),     # 128 k-tiles: the 256 x 256 split
    ((1024, 512, 2048), "NN", (128, 128), 8, 2, True),      # split runs of 8 k-tiles: the 2-stage ring
    ((1024, 1024, 4096), "NN", (128, 128), 8, 3, True),     # split runs of 16 k-tiles: the 3-stage ring
    ((2048, 2048, 1024), "NN", (128, 128), 8, 2, False),    # 16 k-tiles: the 2-stage ring
    ((2048, 2048, 2048), "NN", (128, 128), 8, 3, False),    # 32 k-tiles, one workgroup per CU: the 3-stage ring
    ((2048, 2048, 4096), "NN", (128, 128), 8, 3, False),
    ((4096, 2048, 2048), "NN", (128, 256), 8, 2, False),    # 256 tiles of 128 x 256 in one round
    ((1536, 2048, 4096), "NN", (128, 128), 8, 3, False),    # 192 tiles, fewer than the CUs
    ((8192, 1024, 8192), "TN", (128, 128), 8, 2, False),    # transposed operands never split
    ((2048, 2048, 2048), "TN", (128, 128), 8, 3, False),
    ((4096, 2752, 4096), "TN", (256, 256), 8, 2, False),
])
def test_tile_rule(shape, lay, tile, waves, stages, split):
    r = info(*shape, lay=lay)
    assert ((r["tile_m"], r["tile_n"]), r["waves"], r["stages"]) == (tile, waves, stages), r
    assert (r["split_workgroups"] > 0) == split, r


@pytest.mark.parametrize("shape,persistent", [
    ((4096, 11008, 4096), 256), ((4096, 11008, 4160), 0), ((4096, 11008, 4040), 0),
    ((4096, 11008, 128), 0), ((4352, 4096, 1024), 0), ((4096, 4096, 256), 256),
])
def test_persistent_conditions(shape, persistent, monkeypatch):
    # the persistent kernel runs only when k is a multiple of 64 spanning an even number
    # (at least 4) of k-tiles and the tile grid is not split
    monkeypatch.setenv("GE_TILE", "L")
    assert info(*shape)["persistent_workgroups"] == persistent


def test_group_of_m_tiles_follows_the_size_of_A():
    assert info(4096, 11008, 4096)["group_m"] == 8
    assert info(65536, 8192, 16384)["group_m"] == 4   # A of 2 GiB outgrows the 256 MB MALL


def test_split_plans_take_groups_of_4():
    # split runs of one XCD cover fewer tiles: groups of 4 m-tiles share more panels
    for shape in ((1024, 512, 2048), (1024, 1024, 4096), (2048, 2048, 8192), (8192, 1024, 8192)):
        r = info(*shape)
        assert r["split_workgroups"] > 0 and r["group_m"] == 4, (shape, r)


def test_workspace():
    assert info(4096, 11008, 4096)["workspace_bytes"] == 0
    # DRELU_BGRAD: one fp32 row sum per row and 64-column wave tile
    assert info(8192, 8192, 8192, ep="DRELU_BGRAD", dts=("bf16", "bf16", "bf16"))["workspace_bytes"] == 128 * 8192 * 4
    # the unfused chain: T1 and T2 in D's type
    assert info(4096, 11008, 4096, ep="RELU_BIAS_UNFUSED")["workspace_bytes"] == 2 * 4096 * 11008 * 2
    # the split tail: the flag region, then one fp32 256 x 256 tile per split workgroup
    r = info(4352, 4096, 1024)
    assert r["split_workgroups"] == 64 and r["workspace_bytes"] == 4096 + 64 * 256 * 256 * 4


def test_errors_and_device_size():
    st, _ = ge.gemm_epilog_plan_info(8, 12, 8, F16, "RELU_BIAS", check=False)
    assert st == 2
    st, _ = ge.gemm_epilog_plan_info(8, 8, 8, F16, "RELU_BIAS", compute_units=0, check=False)
    assert st == 1
    # a smaller device: the 7B FFN grid is several full rounds on 80 compute units
    r = info(4096, 11008, 4096, cus=80)
    assert r["persistent_workgroups"] == 80 and r["split_workgroups"] == 0


@pytest.mark.gpu
@pytest.mark.parametrize("shape,lay,ep", [
    ((4096, 11008, 4096), "NN", "RELU_BIAS"), ((1024, 512, 2048), "NN", "RELU_BIAS"),
    ((8192, 1024, 8192), "NN", "DRELU_BGRAD"), ((4096, 1376, 4096), "NN", "RELU_AUX_BIAS"),
    ((8192, 1024, 8192), "TN", "DRELU_BGRAD"), ((4096, 11008, 4096), "NN", "RELU_BIAS_UNFUSED"),
])
def test_plan_agrees_with_plan_info(gpu, shape, lay, ep):
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    r = info(*shape, lay=lay, ep=ep, cus=cus)
    h = gpu.gemm_epilog_plan_ex(*shape, F16, ep, int(lay[0] == "T"), int(lay[1] == "T"))
    try:
        d = gpu.gemm_epilog_describe(h)
        assert f"tile {r['tile_m']}x{r['tile_n']}" in d and f"grid {r['tiles']}" in d, (d, r)
        assert ("persistent workgroups" in d) == (r["persistent_workgroups"] > 0), (d, r)
        assert ("split over" in d) == (r["split_workgroups"] > 0), (d, r)
        assert gpu.gemm_epilog_workspace_bytes(h) == r["workspace_bytes"]
    finally:
        gpu.gemm_epilog_free(h)
