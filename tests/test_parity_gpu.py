"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

* integer-valued inputs: every product and sum is exact, so D, the mask and bgrad
  must equal the oracle bit for bit (all epilogues but GELU, all dtypes, all tile
  configurations, ragged m, several k-tiles and a ragged k tail);
* random normal inputs: the tolerances of the fused-epilogue path, plus a tighter
  rounding-model ratio;
* guard zones around every output, run-to-run bitwise determinism, host-side errors.
"""
import numpy as np
import pytest
import torch

import oracle
from gemm_epilogues_epilog_amd import inputs
from tests import gpu_runner as R
from tests.helpers import assert_bgrad, assert_close, assert_mask, tight_ratio, to_np

pytestmark = pytest.mark.gpu

DTS = ["f32", "f16", "bf16"]
# split tails: "L", "LM" and "LMD" split k loops into runs that divide a tile's k-tiles (each run
# finishes a part of the tile); "-run3" forces runs of 3 k-tiles, which do not divide the
# 4 k-tiles of k = 200 or 256 (an owner run adds its partners' partials)
TILES16 = ["S", "M", "L", "L-nosk", "L-run3", "LH", "LM", "LM-nosk", "LM-run3", "LM4", "LMD", "LMD-nosk", "LMD-run3",
           "L3", "L3-nosk", "L3-run3", "LW", "LW-nosk", "LW-run3"]
TILES = {"f32": ["S", "M"], "f16": TILES16, "bf16": TILES16}
# the last shape (k a multiple of 64 over 4 k-tiles) runs the persistent kernel in "L"
INT_SHAPES = [(1, 8, 8), (33, 136, 72), (200, 264, 200), (300, 520, 136), (300, 520, 256)]


def cases_int():
    for dt in DTS:
        for tile in TILES[dt]:
            for shape in INT_SHAPES:
                yield dt, tile, shape


@pytest.mark.parametrize("dt,tile,shape", list(cases_int()))
def test_integer_exact_all_epilogues(gpu, dt, tile, shape):
    m, n, k = shape
    print(f"[case] integer {dt} tile {tile} m={m} n={n} k={k}", flush=True)
    A, B, bias, A2, B2 = inputs.integer_case(m, n, k, dt)
    a, b, c = to_np(A), to_np(B), to_np(bias)
    for ep in ("NONE", "BIAS", "RELU_BIAS", "RELU_BIAS_UNFUSED"):
        g = R.run(gpu, ep, dt, A, B, bias, tile=tile)
        o = oracle.gemm_epilog(a, b, ep, bias=c, ab=dt)
        assert np.array_equal(g["D"].view(np.uint8), o["D"].view(np.uint8)), f"{ep} {g['desc']}"
    g = R.run(gpu, "RELU_AUX_BIAS", dt, A, B, bias, tile=tile)
    o = oracle.gemm_epilog(a, b, "RELU_AUX_BIAS", bias=c, ab=dt)
    assert np.array_equal(g["D"].view(np.uint8), o["D"].view(np.uint8)), g["desc"]
    assert np.array_equal(g["mask"].view(np.uint32), o["mask"]), g["desc"]
    mask = torch.from_numpy(o["mask"].view(np.int32).copy())
    gb = R.run(gpu, "DRELU_BGRAD", dt, A2, B2, mask=mask, tile=tile)
    ob = oracle.gemm_epilog(to_np(A2), to_np(B2), "DRELU_BGRAD", mask=o["mask"], ab=dt)
    assert np.array_equal(gb["D"].view(np.uint8), ob["D"].view(np.uint8)), gb["desc"]
    assert np.array_equal(gb["bgrad"].view(np.uint8), ob["bgrad"].view(np.uint8)), gb["desc"]
    # the unfused backward against the forward's activation (ReLU output: zeros and
    # positive half-integers)
    act = g["D_dev"]
    gu = R.run(gpu, "DRELU_BGRAD_UNFUSED", dt, A2, B2, act=act, tile=tile)
    ou = oracle.gemm_epilog(to_np(A2), to_np(B2), "DRELU_BGRAD_UNFUSED", act=g["D"], ab=dt)
    assert np.array_equal(gu["D"].view(np.uint8), ou["D"].view(np.uint8)), gu["desc"]
    assert np.array_equal(gu["bgrad"].view(np.uint8), ou["bgrad"].view(np.uint8)), gu["desc"]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("shape", [(96, 72, 40), (300, 264, 256)])
def test_integer_exact_fp32_vectors(gpu, dt, shape):
    # bias and bgrad in fp32 with 16-bit matrices (and fp32 with fp32)
    m, n, k = shape
    A, B, bias, A2, B2 = inputs.integer_case(m, n, k, dt, vec="f32")
    o = oracle.gemm_epilog(to_np(A), to_np(B), "RELU_AUX_BIAS", bias=to_np(bias), ab=dt, vec="f32")
    g = R.run(gpu, "RELU_AUX_BIAS", dt, A, B, bias, vec="f32")
    assert np.array_equal(g["D"].view(np.uint8), o["D"].view(np.uint8))
    assert np.array_equal(g["mask"].view(np.uint32), o["mask"])
    mask = torch.from_numpy(o["mask"].view(np.int32).copy())
    gb = R.run(gpu, "DRELU_BGRAD", dt, A2, B2, mask=mask, vec="f32")
    ob = oracle.gemm_epilog(to_np(A2), to_np(B2), "DRELU_BGRAD", mask=o["mask"], ab=dt, vec="f32")
    assert np.array_equal(gb["bgrad"], ob["bgrad"])
    gu = R.run(gpu, "DRELU_BGRAD_UNFUSED", dt, A2, B2, act=g["D_dev"], vec="f32")
    ou = oracle.gemm_epilog(to_np(A2), to_np(B2), "DRELU_BGRAD_UNFUSED", act=g["D"], ab=dt, vec="f32")
    assert np.array_equal(gu["D"].view(np.uint8), ou["D"].view(np.uint8))
    assert np.array_equal(gu["bgrad"], ou["bgrad"])


RAND_SHAPES = [(64, 48, 32), (130, 200, 264), (257, 392, 520), (512, 256, 1024)]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("shape", RAND_SHAPES)
def test_random_parity(gpu, dt, shape):
    m, n, k = shape
    print(f"[case] random {dt} m={m} n={n} k={k}", flush=True)
    A, B, bias, A2, B2 = inputs.small_case(m, n, k, dt, std=1.0, std_bias=1.0)
    a, b, c = to_np(A), to_np(B), to_np(bias)
    wa, wb = oracle.to_f32(a, dt), oracle.to_f32(b, dt)
    for tile in TILES[dt]:
        for ep in ("RELU_BIAS", "GELU_BIAS", "BIAS"):
            g = R.run(gpu, ep, dt, A, B, bias, tile=tile)
            o = oracle.gemm_epilog(a, b, ep, bias=c, ab=dt, want_pre=True)
            assert_close(g["D"], o["D"], dt, f"{ep} {g['desc']}")
            gelu = ep == "GELU_BIAS"
            r = tight_ratio(g["D"], o["D"], dt, wa, wb, 1.13 if gelu else 1.0, gelu_pre=o["pre"] if gelu else None)
            assert r <= 4.0, f"{ep} {g['desc']}: rounding-model ratio {r}"
        g = R.run(gpu, "RELU_AUX_BIAS", dt, A, B, bias, tile=tile)
        o = oracle.gemm_epilog(a, b, "RELU_AUX_BIAS", bias=c, ab=dt, want_pre=True)
        assert_close(g["D"], o["D"], dt, g["desc"])
        assert_mask(g["mask"], o["mask"], o["pre"], m)
        mask = torch.from_numpy(g["mask"].view(np.int32).copy())   # the GPU forward's mask
        gb = R.run(gpu, "DRELU_BGRAD", dt, A2, B2, mask=mask, tile=tile)
        ob = oracle.gemm_epilog(to_np(A2), to_np(B2), "DRELU_BGRAD", mask=g["mask"].view(np.uint32), ab=dt)
        assert_close(gb["D"], ob["D"], dt, gb["desc"])
        assert_bgrad(gb["bgrad"], ob["bgrad"], ob["absum"], dt)
        gu = R.run(gpu, "DRELU_BGRAD_UNFUSED", dt, A2, B2, act=g["D_dev"], tile=tile)
        ou = oracle.gemm_epilog(to_np(A2), to_np(B2), "DRELU_BGRAD_UNFUSED", act=g["D"], ab=dt)
        assert_close(gu["D"], ou["D"], dt, gu["desc"])
        assert_bgrad(gu["bgrad"], ou["bgrad"], ou["absum"], dt)


def test_zero_A_closed_form(gpu):
    m, n, k = 300, 264, 136
    _, B, bias, _, _ = inputs.small_case(m, n, k, "f16")
    A = torch.zeros(m, k, dtype=torch.float16)
    g = R.run(gpu, "RELU_AUX_BIAS", "f16", A, B, bias)
    bv = bias.float().numpy()
    assert np.array_equal(g["D"].astype(np.float32), np.repeat(np.maximum(bv, 0)[:, None], n, 1))
    from tests.helpers import unpack_mask
    assert np.array_equal(unpack_mask(g["mask"], m), np.repeat((bv > 0)[:, None], n, 1))
    gb = R.run(gpu, "DRELU_BGRAD", "f16", A, B, mask=torch.from_numpy(g["mask"].view(np.int32).copy()))
    assert not gb["D"].astype(np.float32).any() and not gb["bgrad"].astype(np.float32).any()


def test_deterministic_and_repeatable(gpu):
    m, n, k = 512, 520, 1032
    A, B, bias, A2, B2 = inputs.small_case(m, n, k, "bf16")
    g1 = R.run(gpu, "RELU_AUX_BIAS", "bf16", A, B, bias)
    g2 = R.run(gpu, "RELU_AUX_BIAS", "bf16", A, B, bias, repeat=3)
    assert np.array_equal(g1["D"], g2["D"]) and np.array_equal(g1["mask"], g2["mask"])
    mask = torch.from_numpy(g1["mask"].view(np.int32).copy())
    b1 = R.run(gpu, "DRELU_BGRAD", "bf16", A2, B2, mask=mask)
    b2 = R.run(gpu, "DRELU_BGRAD", "bf16", A2, B2, mask=mask, repeat=2)
    assert np.array_equal(b1["D"], b2["D"]) and np.array_equal(b1["bgrad"], b2["bgrad"])


def test_execute_rejects_bad_pointers_on_host(gpu):
    ge = gpu
    h = ge.gemm_epilog_plan(64, 64, 64, ("f16", "f16", "f16"), "RELU_AUX_BIAS")
    try:
        A = torch.zeros(64 * 64 + 8, dtype=torch.float16, device="cuda")
        D = torch.zeros(64, 64, dtype=torch.float16, device="cuda")
        bias = torch.zeros(64, dtype=torch.float16, device="cuda")
        aux = torch.zeros(2, 64, dtype=torch.int32, device="cuda")
        mis = A.data_ptr() + 2
        assert ge.gemm_epilog_execute(h, mis, A, bias, D, aux, None, check=False) == 4
        assert ge.gemm_epilog_execute(h, A, A, None, D, aux, None, check=False) == 3
        assert ge.gemm_epilog_execute(h, A, A, bias, D, None, None, check=False) == 3
        assert ge.gemm_epilog_execute(h, A, A, bias.data_ptr() + 1, D, aux, None, check=False) == 4
        assert ge.gemm_epilog_execute(h, A, A, bias, D, aux.data_ptr() + 4, None, check=False) == 4
        assert ge.gemm_epilog_execute(h, A, A, bias, None, aux, None, check=False) == 3
        torch.cuda.synchronize()
    finally:
        ge.gemm_epilog_free(h)


def test_matmul_wrapper_round_trip(gpu):
    m, n, k = 64, 48, 32
    A, B, bias, A2, B2 = inputs.small_case(m, n, k, "f32", std_bias=0.1)
    with gpu.Matmul(m, n, k, "f32", "RELU_AUX_BIAS") as mm:
        D, aux = mm.execute(A.cuda(), B.cuda(), bias.cuda())
        assert "relu_aux" in aux and aux["relu_aux"].shape == ((m + 31) // 32, n)
        assert gpu.gemm_epilog_workspace_bytes(mm.handle) == 0
    with gpu.Matmul(m, n, k, "f32", "DRELU_BGRAD") as mm:
        dZ, g = mm.execute(A2.cuda(), B2.cuda(), relu_aux=aux["relu_aux"])
        assert gpu.gemm_epilog_workspace_bytes(mm.handle) > 0
    torch.cuda.synchronize()
    ref = oracle.gemm_epilog(A2.numpy(), B2.numpy(), "DRELU_BGRAD", mask=to_np(aux["relu_aux"]), ab="f32")
    assert_close(to_np(dZ), ref["D"], "f32")
    assert_bgrad(to_np(g["drelu_bgrad"]), ref["bgrad"], ref["absum"], "f32")


def test_stream_argument(gpu):
    m, n, k = 128, 128, 128
    A, B, bias, _, _ = inputs.small_case(m, n, k, "f16")
    s = torch.cuda.Stream()
    g = R.run(gpu, "RELU_BIAS", "f16", A, B, bias, stream=s)
    o = oracle.gemm_epilog(to_np(A), to_np(B), "RELU_BIAS", bias=to_np(bias))
    assert_close(g["D"], o["D"], "f16")


def test_split_tail_plan_and_determinism(gpu):
    """4352 x 4096 (272 tiles on 256 compute units) splits its last round of 16 tiles;
    the split result matches the unsplit one within rounding and repeats bit for bit,
    and the 7B-FFN shape (its last pass over the CUs 69% full) is not split."""
    ge = gpu
    h = ge.gemm_epilog_plan(4096, 11008, 4096, ("f16", "f16", "f16"), "RELU_BIAS")
    try:
        assert "split" not in ge.gemm_epilog_describe(h)
    finally:
        ge.gemm_epilog_free(h)
    m, n, k = 4352, 4096, 1024
    A, B, bias, _, _ = inputs.small_case(m, n, k, "f16", std=k ** -0.5, std_bias=0.02)
    g1 = R.run(gpu, "RELU_AUX_BIAS", "f16", A, B, bias, repeat=2)
    assert "split" in g1["desc"]
    g2 = R.run(gpu, "RELU_AUX_BIAS", "f16", A, B, bias)
    assert torch.equal(g1["D_dev"], g2["D_dev"]) and torch.equal(g1["mask_dev"], g2["mask_dev"])
    g0 = R.run(gpu, "RELU_AUX_BIAS", "f16", A, B, bias, tile="LH-nosk")
    assert "split" not in g0["desc"]
    assert_close(g1["D"], g0["D"], "f16", "split vs unsplit")
    rows = np.r_[0:32, 4096:4352]   # the first row group and the split tiles' rows
    o = oracle.gemm_epilog(to_np(A)[rows], to_np(B), "RELU_AUX_BIAS", bias=to_np(bias)[rows], want_pre=True)
    assert_close(g1["D"][rows], o["D"], "f16", "split vs oracle")



@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_persistent_tiles_integer_exact(gpu, dt):
    """The persistent kernel (one workgroup per compute unit walking the tile order,
    k loop running on from one tile into the next): 528 tiles of a ragged 4000 x 8200
    output on 256 workgroups, so most workgroups finish three tiles and every tile
    after a workgroup's first starts from operands fetched during the previous one.
    Integer inputs make every epilogue bit-exact against the oracle."""
    m, n, k = 4000, 8200, 256
    print(f"[case] persistent integer {dt} m={m} n={n} k={k}", flush=True)
    A, B, bias, A2, B2 = inputs.integer_case(m, n, k, dt)
    a, b, c = to_np(A), to_np(B), to_np(bias)
    for ep in ("NONE", "BIAS", "RELU_BIAS"):
        g = R.run(gpu, ep, dt, A, B, bias, tile="L-nosk")
        assert "persistent workgroups" in g["desc"], g["desc"]
        o = oracle.gemm_epilog(a, b, ep, bias=c, ab=dt)
        assert np.array_equal(g["D"].view(np.uint8), o["D"].view(np.uint8)), f"{ep} {g['desc']}"
    g = R.run(gpu, "RELU_AUX_BIAS", dt, A, B, bias, tile="L-nosk")
    o = oracle.gemm_epilog(a, b, "RELU_AUX_BIAS", bias=c, ab=dt)
    assert np.array_equal(g["D"].view(np.uint8), o["D"].view(np.uint8)), g["desc"]
    assert np.array_equal(g["mask"].view(np.uint32), o["mask"]), g["desc"]
    mask = torch.from_numpy(o["mask"].view(np.int32).copy())
    gb = R.run(gpu, "DRELU_BGRAD", dt, A2, B2, mask=mask, tile="L-nosk")
    assert "persistent workgroups" in gb["desc"], gb["desc"]
    ob = oracle.gemm_epilog(to_np(A2), to_np(B2), "DRELU_BGRAD", mask=o["mask"], ab=dt)
    assert np.array_equal(gb["D"].view(np.uint8), ob["D"].view(np.uint8)), gb["desc"]
    assert np.array_equal(gb["bgrad"].view(np.uint8), ob["bgrad"].view(np.uint8)), gb["desc"]


def test_persistent_random_matches_one_tile_per_workgroup(gpu):
    """Normal inputs at 2048 x 11008 x 512 (344 tiles): the persistent kernel and the
    one-workgroup-per-tile kernel of the same loop agree bit for bit (same k order per
    tile), repeat bit for bit, and match the oracle on sampled rows."""
    m, n, k = 2048, 11008, 512
    A, B, bias, _, _ = inputs.small_case(m, n, k, "f16", std=k ** -0.5, std_bias=0.02)
    gp = R.run(gpu, "RELU_AUX_BIAS", "f16", A, B, bias, tile="L-nosk", repeat=2)
    assert "persistent workgroups" in gp["desc"], gp["desc"]
    gq = R.run(gpu, "RELU_AUX_BIAS", "f16", A, B, bias, tile="L-nosk")
    assert torch.equal(gp["D_dev"], gq["D_dev"]) and torch.equal(gp["mask_dev"], gq["mask_dev"])
    with R.env({"GE_PERSIST": "0"}):
        g1 = R.run(gpu, "RELU_AUX_BIAS", "f16", A, B, bias, tile="L-nosk")
    assert "persistent workgroups" not in g1["desc"], g1["desc"]
    assert torch.equal(gp["D_dev"], g1["D_dev"]) and torch.equal(gp["mask_dev"], g1["mask_dev"])
    rows = np.r_[0:32, 992:1056, 2016:2048]
    o = oracle.gemm_epilog(to_np(A)[rows], to_np(B), "RELU_AUX_BIAS", bias=to_np(bias)[rows], want_pre=True)
    assert_close(gp["D"][rows], o["D"], "f16", "persistent vs oracle")


def test_plan_log(gpu, capfd):
    ge = gpu
    with R.env({"GE_LOG": "1"}):
        h = ge.gemm_epilog_plan(1024, 512, 2048, ("f16", "f16", "f16"), "RELU_BIAS")
    try:
        err = capfd.readouterr().err
        assert "gemm_epilog_plan: m=1024 n=512 k=2048 -> " + ge.gemm_epilog_describe(h) in err, err
    finally:
        ge.gemm_epilog_free(h)
    with R.env({"GE_LOG": "0"}):
        h = ge.gemm_epilog_plan(1024, 512, 2048, ("f16", "f16", "f16"), "RELU_BIAS")
    ge.gemm_epilog_free(h)
    assert "gemm_epilog_plan" not in capfd.readouterr().err
