"""GPU parity of the two-layer perceptron training step (gemm_epilogues_epilog_amd.mlp),
stage by stage against the CPU oracle: each of the five products is compared with the
oracle on the inputs that stage received on the GPU (the forward's mask as the GPU
wrote it), so the test checks both the wiring of the step (operands, storage orders,
mask hand-over) and each product's numerics, within the fused-epilogue tolerances."""
import numpy as np
import pytest
import torch

import oracle
from gemm_epilogues_epilog_amd import inputs
from tests.helpers import assert_all_finite, assert_bgrad, assert_close, assert_mask, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("dims", [(72, 136, 40, 264), (520, 264, 136, 1032), (1024, 2048, 512, 1024)])
def test_mlp_step_stage_parity(gpu, dt, dims):
    from gemm_epilogues_epilog_amd.mlp import MLP2Step
    d, h, o, b = dims
    print(f"[case] mlp step {dt} d={d} h={h} o={o} batch={b}", flush=True)
    X, W1, b1, W2, dY = inputs.mlp_case(d, h, o, b, dt)
    Xd, W1d, b1d, W2d, dYd = (t.cuda() for t in (X, W1, b1, W2, dY))
    with MLP2Step(d, h, o, b, dt) as st:
        assert "op_a T" in st.dz1.describe() and "op_b T" in st.dw1.describe()
        g = st.step(Xd, W1d, b1d, W2d, dYd)
        torch.cuda.synchronize()
        H, mask, Y = to_np(st.H), to_np(st.mask), to_np(st.Y)
        dW2, dZ1, db1, dW1 = to_np(g["dW2"]), to_np(g["dZ1"]), to_np(g["db1"]), to_np(g["dW1"])
    x, w1, bb1, w2, dy = (to_np(t) for t in (X, W1, b1, W2, dY))
    o1 = oracle.gemm_epilog(w1, x, "RELU_AUX_BIAS", bias=bb1, ab=dt, want_pre=True)
    assert_close(H, o1["D"], dt, "H")
    assert_mask(mask, o1["mask"], o1["pre"], h)
    assert_close(Y, oracle.gemm_epilog(w2, H, "NONE", ab=dt)["D"], dt, "Y")
    assert_close(dW2, oracle.gemm_epilog(dy, H, "NONE", ab=dt, trans_b=True)["D"], dt, "dW2")
    ob = oracle.gemm_epilog(w2, dy, "DRELU_BGRAD", mask=mask.view(np.uint32), ab=dt, trans_a=True)
    assert_close(dZ1, ob["D"], dt, "dZ1")
    assert_bgrad(db1, ob["bgrad"], ob["absum"], dt)
    assert_close(dW1, oracle.gemm_epilog(dZ1, x, "NONE", ab=dt, trans_b=True)["D"], dt, "dW1")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("dims", [(72, 136, 40, 264), (520, 264, 136, 1032)])
def test_mlp_step_unfused_stage_parity(gpu, dt, dims):
    # the baseline step: the forward's unfused chain keeps H and no mask, the backward's
    # unfused chain reads H; every stage against the oracle on the inputs it received
    from gemm_epilogues_epilog_amd.mlp import MLP2Step
    d, h, o, b = dims
    print(f"[case] unfused mlp step {dt} d={d} h={h} o={o} batch={b}", flush=True)
    X, W1, b1, W2, dY = inputs.mlp_case(d, h, o, b, dt)
    Xd, W1d, b1d, W2d, dYd = (t.cuda() for t in (X, W1, b1, W2, dY))
    with MLP2Step(d, h, o, b, dt, fused=False) as st:
        assert st.mask is None
        assert "RELU_BIAS_UNFUSED" in st.fwd1.describe() and "DRELU_BGRAD_UNFUSED" in st.dz1.describe()
        g = st.step(Xd, W1d, b1d, W2d, dYd)
        torch.cuda.synchronize()
        H, Y = to_np(st.H), to_np(st.Y)
        dW2, dZ1, db1, dW1 = to_np(g["dW2"]), to_np(g["dZ1"]), to_np(g["db1"]), to_np(g["dW1"])
    x, w1, bb1, w2, dy = (to_np(t) for t in (X, W1, b1, W2, dY))
    assert_close(H, oracle.gemm_epilog(w1, x, "RELU_BIAS_UNFUSED", bias=bb1, ab=dt)["D"], dt, "H")
    assert_close(Y, oracle.gemm_epilog(w2, H, "NONE", ab=dt)["D"], dt, "Y")
    assert_close(dW2, oracle.gemm_epilog(dy, H, "NONE", ab=dt, trans_b=True)["D"], dt, "dW2")
    ob = oracle.gemm_epilog(w2, dy, "DRELU_BGRAD_UNFUSED", act=H, ab=dt, trans_a=True)
    assert_close(dZ1, ob["D"], dt, "dZ1")
    assert_bgrad(db1, ob["bgrad"], ob["absum"], dt)
    assert_close(dW1, oracle.gemm_epilog(dZ1, x, "NONE", ab=dt, trans_b=True)["D"], dt, "dW1")


def test_mlp_step_rejects_bad_sizes(gpu):
    from gemm_epilogues_epilog_amd.mlp import MLP2Step
    with pytest.raises(ValueError):
        MLP2Step(72, 130, 40, 264, "bf16")
    with pytest.raises(ValueError):
        MLP2Step(72, 136, 40, 264, "f32")


def test_mlp_step_8192_sampled_rows(gpu):
    # the step as the benchmark times it (all sizes 8192, bf16): every stage's output on
    # sampled 32-row groups against the oracle on that stage's GPU inputs
    from gemm_epilogues_epilog_amd.mlp import MLP2Step
    n = 8192
    print("[case] mlp step 8192 bf16: generating inputs", flush=True)
    X, W1, b1, W2, dY = inputs.mlp_case(n, n, n, n, "bf16")
    with MLP2Step(n, n, n, n, "bf16") as st:
        print("[case] mlp step 8192 bf16: step", flush=True)
        g = st.step(X.cuda(), W1.cuda(), b1.cuda(), W2.cuda(), dY.cuda())
        torch.cuda.synchronize()
        for name, t in (("H", st.H), ("Y", st.Y), ("dW2", g["dW2"]), ("dZ1", g["dZ1"]), ("db1", g["db1"]),
                        ("dW1", g["dW1"])):
            assert_all_finite(t, name)
        H, mask, Y = to_np(st.H), to_np(st.mask), to_np(st.Y)
        dW2, dZ1, db1, dW1 = to_np(g["dW2"]), to_np(g["dZ1"]), to_np(g["db1"]), to_np(g["dW1"])
    x, w1, bb1, w2, dy = (to_np(t) for t in (X, W1, b1, W2, dY))
    rng = np.random.default_rng(7)
    groups = sorted(set(rng.choice(n // 32, size=3, replace=False).tolist()) | {0, n // 32 - 1})
    w2t = np.ascontiguousarray(w2.T)        # rows of W2^T, the DRELU_BGRAD operand
    Ht = np.ascontiguousarray(H.T)          # H^T (batch, hidden), the dW2 operand
    xt = np.ascontiguousarray(x.T)          # X^T, the dW1 operand
    for grp in groups:
        r = slice(32 * grp, 32 * grp + 32)
        print(f"[case] mlp step 8192 rows {r.start}:{r.stop}", flush=True)
        o1 = oracle.gemm_epilog(w1[r], x, "RELU_AUX_BIAS", bias=bb1[r], ab="bf16", want_pre=True)
        assert_close(H[r], o1["D"], "bf16", "H")
        assert_mask(mask[grp:grp + 1], o1["mask"], o1["pre"], 32)
        assert_close(Y[r], oracle.gemm_epilog(w2[r], H, "NONE", ab="bf16")["D"], "bf16", "Y")
        assert_close(dW2[r], oracle.gemm_epilog(dy[r], Ht, "NONE", ab="bf16")["D"], "bf16", "dW2")
        ob = oracle.gemm_epilog(w2t[r], dy, "DRELU_BGRAD", mask=mask[grp:grp + 1].view(np.uint32), ab="bf16")
        assert_close(dZ1[r], ob["D"], "bf16", "dZ1")
        assert_bgrad(db1[r], ob["bgrad"], ob["absum"], "bf16")
        assert_close(dW1[r], oracle.gemm_epilog(dZ1[r], xt, "NONE", ab="bf16")["D"], "bf16", "dW1")
