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
from tests.helpers import assert_bgrad, assert_close, assert_mask, to_np

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


def test_mlp_step_rejects_bad_sizes(gpu):
    from gemm_epilogues_epilog_amd.mlp import MLP2Step
    with pytest.raises(ValueError):
        MLP2Step(72, 130, 40, 264, "bf16")
    with pytest.raises(ValueError):
        MLP2Step(72, 136, 40, 264, "f32")
