"""The benchmark workloads at their full sizes, in the configuration the benchmark times.

Small workloads are compared with the oracle in full. For the large ones the oracle
recomputes whole 32-row groups chosen at random (whole mask words, whole bias-gradient
rows), and properties that hold at any size are checked on the full GPU outputs:
ReLU outputs are >= 0, a set mask bit <=> a positive output, bgrad equals the row sum
of the GPU's own backward output, and about half of the mask bits are set."""
import numpy as np
import pytest
import torch

import oracle
from gemm_epilogues_epilog_amd import inputs
from tests import gpu_runner as R
from tests.helpers import assert_all_finite, assert_bgrad, assert_close, assert_mask, tight_ratio, to_np

pytestmark = pytest.mark.gpu


def sample_groups(m, count=8, seed=1234):
    g = (m + 31) // 32
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(g, size=min(count, g), replace=False).tolist()) | {0, g - 1}
    return sorted(pick)


def check_rows(gD, W, A, B, bias, groups, epilog, dt, want_mask=None):
    """Oracle on each sampled 32-row group; gD: device D, which must also be finite
    everywhere (it is NaN-filled before the run, so an unwritten element fails)."""
    assert_all_finite(gD, f"{W.name} {epilog} D")
    a_all, b, c_all = to_np(A), to_np(B), to_np(bias)
    wb = oracle.to_f32(b, dt)
    worst = 0.0
    for g in groups:
        r0, r1 = 32 * g, min(W.m, 32 * g + 32)
        o = oracle.gemm_epilog(a_all[r0:r1], b, epilog, bias=c_all[r0:r1], ab=dt, want_pre=True)
        d = to_np(gD[r0:r1])
        assert_close(d, o["D"], dt, f"{W.name} rows {r0}:{r1}")
        slope = 1.13 if epilog == "GELU_BIAS" else 1.0
        worst = max(worst, tight_ratio(d, o["D"], dt, oracle.to_f32(a_all[r0:r1], dt), wb, slope))
        if want_mask is not None:
            assert_mask(to_np(want_mask[g:g + 1]), o["mask"], o["pre"], r1 - r0)
    assert worst <= 4.0, f"rounding-model ratio {worst}"


def relu_mask_invariants(D, mask, m):
    assert not torch.isnan(D).any()
    assert bool((D >= 0).all())
    G, n = mask.shape
    shifts = torch.arange(32, device=mask.device, dtype=torch.int32).view(1, 32, 1)
    bits = ((mask.view(G, 1, n) >> shifts) & 1).view(G * 32, n)
    pad = bits[m:]
    assert not bool(pad.any()), "pad bits set"
    bits = bits[:m].bool()
    pos = D > 0
    assert not bool((pos & ~bits).any()), "positive output with a zero mask bit"
    assert not bool((~bits & (D != 0)).any()), "zero mask bit with a nonzero output"
    frac = bits.float().mean().item()
    assert 0.3 < frac < 0.7, f"set-bit fraction {frac}"


def test_mlp_tiny_f32_forward_backward(gpu):
    W = inputs.WORKLOADS["mlp_tiny_f32_64x48x32"]
    A, B, bias, A2, B2 = W.a(), W.b(), W.bias(), W.a2(), W.b2()
    g = R.run(gpu, "RELU_AUX_BIAS", "f32", A, B, bias)
    o = oracle.gemm_epilog(to_np(A), to_np(B), "RELU_AUX_BIAS", bias=to_np(bias), ab="f32", want_pre=True)
    assert_close(g["D"], o["D"], "f32")
    assert_mask(g["mask"], o["mask"], o["pre"], W.m)
    mask = torch.from_numpy(g["mask"].view(np.int32).copy())
    gb = R.run(gpu, "DRELU_BGRAD", "f32", A2, B2, mask=mask)
    ob = oracle.gemm_epilog(to_np(A2), to_np(B2), "DRELU_BGRAD", mask=g["mask"].view(np.uint32), ab="f32")
    assert_close(gb["D"], ob["D"], "f32")
    assert_bgrad(gb["bgrad"], ob["bgrad"], ob["absum"], "f32")


def test_relu_bias_f16_1024x512x2048(gpu):
    W = inputs.WORKLOADS["relu_bias_f16_1024x512x2048"]
    A, B, bias = W.a(), W.b(), W.bias()
    g = R.run(gpu, "RELU_BIAS", "f16", A, B, bias)
    o = oracle.gemm_epilog(to_np(A), to_np(B), "RELU_BIAS", bias=to_np(bias))
    assert_close(g["D"], o["D"], "f16")
    r = tight_ratio(g["D"], o["D"], "f16", oracle.to_f32(to_np(A), "f16"), oracle.to_f32(to_np(B), "f16"))
    assert r <= 4.0


@pytest.fixture(scope="module")
def ffn():
    W = inputs.WORKLOADS["ffn_f16_4096x11008x4096"]
    return W, W.a(), W.b(), W.bias()


def test_ffn_f16_fused_relu_bias(gpu, ffn):
    W, A, B, bias = ffn
    print(f"[case] {W.name} RELU_BIAS", flush=True)
    g = R.run(gpu, "RELU_BIAS", "f16", A, B, bias)
    D = g["D_dev"]
    check_rows(D, W, A, B, bias, sample_groups(W.m), "RELU_BIAS", "f16")
    assert bool((D >= 0).all()) and not bool(torch.isnan(D).any())


def test_ffn_f16_unfused_matches_fused(gpu, ffn):
    W, A, B, bias = ffn
    gf = R.run(gpu, "RELU_BIAS", "f16", A, B, bias)
    gu = R.run(gpu, "RELU_BIAS_UNFUSED", "f16", A, B, bias)
    assert_all_finite(gu["D_dev"], "unfused D")
    assert_close(gu["D"], gf["D"], "f16", "unfused vs fused")
    groups = sample_groups(W.m)[:4]
    a, b, c = to_np(A), to_np(B), to_np(bias)
    for grp in groups:
        r0, r1 = 32 * grp, 32 * grp + 32
        o = oracle.gemm_epilog(a[r0:r1], b, "RELU_BIAS_UNFUSED", bias=c[r0:r1])
        assert_close(gu["D"][r0:r1], o["D"], "f16", "unfused vs oracle chain")


def test_ffn_f16_aux_bias_none(gpu, ffn):
    # the other epilogues the benchmark times on the headline inputs
    W, A, B, bias = ffn
    groups = sample_groups(W.m, count=4)
    print(f"[case] {W.name} RELU_AUX_BIAS", flush=True)
    g = R.run(gpu, "RELU_AUX_BIAS", "f16", A, B, bias)
    assert "persistent" in g["desc"]
    check_rows(g["D_dev"], W, A, B, bias, groups, "RELU_AUX_BIAS", "f16", want_mask=g["mask_dev"])
    relu_mask_invariants(g["D_dev"], g["mask_dev"], W.m)
    del g
    for ep in ("BIAS", "NONE"):
        print(f"[case] {W.name} {ep}", flush=True)
        g = R.run(gpu, ep, "f16", A, B, bias)
        check_rows(g["D_dev"], W, A, B, bias, groups, ep, "f16")
        del g


def test_ffn_bf16_gelu_bias(gpu):
    W = inputs.WORKLOADS["ffn_gelu_bf16_4096x11008x4096"]
    A, B, bias = W.a(), W.b(), W.bias()
    g = R.run(gpu, "GELU_BIAS", "bf16", A, B, bias)
    check_rows(g["D_dev"], W, A, B, bias, sample_groups(W.m), "GELU_BIAS", "bf16")


def test_mlp_bf16_8192_forward_backward(gpu):
    W = inputs.WORKLOADS["mlp_bf16_8192"]
    A, B, bias = W.a(), W.b(), W.bias()
    print(f"[case] {W.name} forward", flush=True)
    g = R.run(gpu, "RELU_AUX_BIAS", "bf16", A, B, bias)
    groups = sample_groups(W.m)
    check_rows(g["D_dev"], W, A, B, bias, groups, "RELU_AUX_BIAS", "bf16", want_mask=g["mask_dev"])
    relu_mask_invariants(g["D_dev"], g["mask_dev"], W.m)
    mask_dev = g["mask_dev"]
    del g
    print(f"[case] {W.name} backward", flush=True)
    A2, B2 = W.a2(), W.b2()
    gb = R.run(gpu, "DRELU_BGRAD", "bf16", A2, B2, mask=mask_dev)
    assert_all_finite(gb["D_dev"], "backward D")
    assert np.isfinite(oracle.to_f32(gb["bgrad"], "bf16")).all(), "bgrad"
    a2, b2 = to_np(A2), to_np(B2)
    mask_np = to_np(mask_dev)
    for grp in groups:
        r0, r1 = 32 * grp, 32 * grp + 32
        ob = oracle.gemm_epilog(a2[r0:r1], b2, "DRELU_BGRAD", mask=mask_np[grp:grp + 1], ab="bf16")
        assert_close(to_np(gb["D_dev"][r0:r1]), ob["D"], "bf16", f"dz rows {r0}:{r1}")
        assert_bgrad(gb["bgrad"][r0:r1], ob["bgrad"], ob["absum"], "bf16")
    # bgrad equals the row sums of the GPU's own masked output (full size)
    Dd = gb["D_dev"].float()
    rows = Dd.sum(dim=1).double().cpu().numpy()
    absrow = Dd.abs().sum(dim=1).double().cpu().numpy()
    bg = oracle.to_f32(gb["bgrad"], "bf16").astype(np.float64)
    assert (np.abs(bg - rows) <= (1e-3 + 2.0 ** -8) * absrow + 2.0 ** -8 * np.abs(rows)).all()


def test_large_f16_relu_bias_and_aux(gpu):
    W = inputs.WORKLOADS["large_f16_65536x8192x16384"]
    print(f"[case] {W.name} generating inputs", flush=True)
    A, B, bias = W.a(), W.b(), W.bias()
    groups = sample_groups(W.m, count=6)
    print(f"[case] {W.name} RELU_BIAS", flush=True)
    g = R.run(gpu, "RELU_BIAS", "f16", A, B, bias)
    check_rows(g["D_dev"], W, A, B, bias, groups, "RELU_BIAS", "f16")
    D1 = g["D_dev"].clone()
    del g
    print(f"[case] {W.name} RELU_AUX_BIAS", flush=True)
    g = R.run(gpu, "RELU_AUX_BIAS", "f16", A, B, bias)
    assert torch.equal(g["D_dev"], D1), "RELU_AUX_BIAS changed D"
    check_rows(g["D_dev"], W, A, B, bias, groups[:3], "RELU_AUX_BIAS", "f16", want_mask=g["mask_dev"])
    relu_mask_invariants(g["D_dev"], g["mask_dev"], W.m)


def test_mlp_bf16_8192_backward_with_weights_as_stored(gpu):
    # the rest of the 8192 layer's backward as the benchmark times it: dX = W^T dY with
    # W handed over as stored (A as its (k, m) transpose, DRELU_BGRAD), and the weight
    # gradient dW = dZ X^T with X as stored (B as its (n, k) transpose, NONE)
    W = inputs.WORKLOADS["mlp_bf16_8192"]
    A, B, bias = W.a(), W.b(), W.bias()
    g = R.run(gpu, "RELU_AUX_BIAS", "bf16", A, B, bias)
    mask_dev = g["mask_dev"]
    del g, A, B
    A2, B2 = W.a2(), W.b2()
    groups = sample_groups(W.m)
    a2, b2 = to_np(A2), to_np(B2)
    mask_np = to_np(mask_dev)
    print(f"[case] {W.name} DRELU_BGRAD, A as its transpose", flush=True)
    gb = R.run(gpu, "DRELU_BGRAD", "bf16", A2.t().contiguous(), B2, mask=mask_dev, trans_a=True)
    assert "op_a T" in gb["desc"]
    assert_all_finite(gb["D_dev"], "dX D")
    assert np.isfinite(oracle.to_f32(gb["bgrad"], "bf16")).all(), "dX bgrad"
    for grp in groups:
        r0, r1 = 32 * grp, 32 * grp + 32
        ob = oracle.gemm_epilog(a2[r0:r1], b2, "DRELU_BGRAD", mask=mask_np[grp:grp + 1], ab="bf16")
        assert_close(to_np(gb["D_dev"][r0:r1]), ob["D"], "bf16", f"dz rows {r0}:{r1}")
        assert_bgrad(gb["bgrad"][r0:r1], ob["bgrad"], ob["absum"], "bf16")
    del gb
    print(f"[case] {W.name} NONE, B as its transpose", flush=True)
    g = R.run(gpu, "NONE", "bf16", A2, B2.t().contiguous(), trans_b=True)
    assert "op_b T" in g["desc"]
    assert_all_finite(g["D_dev"], "dW D")
    for grp in groups[:4]:
        r0, r1 = 32 * grp, 32 * grp + 32
        o = oracle.gemm_epilog(a2[r0:r1], b2, "NONE", ab="bf16")
        assert_close(to_np(g["D_dev"][r0:r1]), o["D"], "bf16", f"dW rows {r0}:{r1}")


def test_square_f16_4096_fused_and_unfused(gpu):
    W = inputs.WORKLOADS["square_f16_4096"]
    A, B, bias = W.a(), W.b(), W.bias()
    print(f"[case] {W.name} RELU_BIAS and RELU_BIAS_UNFUSED", flush=True)
    gf = R.run(gpu, "RELU_BIAS", "f16", A, B, bias)
    assert "persistent" in gf["desc"]
    check_rows(gf["D_dev"], W, A, B, bias, sample_groups(W.m), "RELU_BIAS", "f16")
    gu = R.run(gpu, "RELU_BIAS_UNFUSED", "f16", A, B, bias)
    assert_all_finite(gu["D_dev"], "square unfused D")
    assert_close(gu["D"], gf["D"], "f16", "unfused vs fused")


def test_shard4_ffn_on_the_192x256_tile(gpu):
    # one GPU's share of a 4-way split of the FFN layer, which the plan gives the
    # 192 x 256 tile (242 tiles in one round instead of 176 of 256 x 256)
    W = inputs.WORKLOADS["ffn_shard4_f16_4096x2752x4096"]
    A, B, bias = W.a(), W.b(), W.bias()
    print(f"[case] {W.name} RELU_BIAS", flush=True)
    g = R.run(gpu, "RELU_BIAS", "f16", A, B, bias)
    assert "tile 192x256" in g["desc"] and "persistent" in g["desc"], g["desc"]
    assert_all_finite(g["D_dev"], "4-way shard D")
    check_rows(g["D_dev"], W, A, B, bias, sample_groups(W.m, count=4), "RELU_BIAS", "f16")   # the last group lies in the ragged last tile


def test_shard8_shapes(gpu):
    # one GPU's share of an 8-way split along n, as the benchmark times it
    W = inputs.WORKLOADS["ffn_shard8_f16_4096x1376x4096"]
    A, B, bias = W.a(), W.b(), W.bias()
    print(f"[case] {W.name} RELU_BIAS", flush=True)
    g = R.run(gpu, "RELU_BIAS", "f16", A, B, bias)
    check_rows(g["D_dev"], W, A, B, bias, sample_groups(W.m, count=4), "RELU_BIAS", "f16")
    del g
    W = inputs.WORKLOADS["mlp_shard8_bf16_8192x1024x8192"]
    A, B, bias = W.a(), W.b(), W.bias()
    print(f"[case] {W.name} forward and backward", flush=True)
    g = R.run(gpu, "RELU_AUX_BIAS", "bf16", A, B, bias)
    groups = sample_groups(W.m, count=4)
    check_rows(g["D_dev"], W, A, B, bias, groups, "RELU_AUX_BIAS", "bf16", want_mask=g["mask_dev"])
    mask_dev = g["mask_dev"]
    del g
    A2, B2 = W.a2(), W.b2()
    gb = R.run(gpu, "DRELU_BGRAD", "bf16", A2, B2, mask=mask_dev)
    assert_all_finite(gb["D_dev"], "shard backward D")
    assert np.isfinite(oracle.to_f32(gb["bgrad"], "bf16")).all(), "shard bgrad"
    a2, b2, mask_np = to_np(A2), to_np(B2), to_np(mask_dev)
    for grp in groups:
        r0, r1 = 32 * grp, 32 * grp + 32
        ob = oracle.gemm_epilog(a2[r0:r1], b2, "DRELU_BGRAD", mask=mask_np[grp:grp + 1], ab="bf16")
        assert_close(to_np(gb["D_dev"][r0:r1]), ob["D"], "bf16", f"dz rows {r0}:{r1}")
        assert_bgrad(gb["bgrad"][r0:r1], ob["bgrad"], ob["absum"], "bf16")
