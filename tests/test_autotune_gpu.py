"""gemm_epilog_autotune on the GPU: after the search the plan still computes what the
oracle computes (bit for bit on integer-valued inputs, for a forward with the mask, the
backward with bgrad, transposed operands and fp32), the outputs the call leaves behind
are those of an execute, and its argument errors come back before any timing."""
import numpy as np
import pytest
import torch

import oracle
from gemm_epilogues_epilog_amd import inputs
from tests.helpers import to_np

pytestmark = pytest.mark.gpu

TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _same(x, y):
    return np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8))


@pytest.mark.parametrize("dt,shape,lay", [
    ("f16", (300, 520, 256), "NN"),      # candidates: persistent, split tail, LH, LM
    ("bf16", (1024, 512, 200), "NN"),    # ragged k tail, split tails
    ("bf16", (304, 520, 136), "TN"),
    ("f16", (200, 264, 200), "NT"),
    ("f32", (96, 72, 40), "NN"),
])
def test_autotuned_plan_matches_oracle(gpu, dt, shape, lay):
    ge = gpu
    m, n, k = shape
    ta, tb = lay[0] == "T", lay[1] == "T"
    print(f"[case] autotune {dt} {lay} m={m} n={n} k={k}", flush=True)
    A, B, bias, A2, B2 = inputs.integer_case(m, n, k, dt)
    st = (lambda t, tr: t.t().contiguous() if tr else t)
    As, Bs, A2s, B2s = st(A, ta), st(B, tb), st(A2, ta), st(B2, tb)
    kw = dict(trans_a=ta, trans_b=tb)
    o = oracle.gemm_epilog(to_np(As), to_np(Bs), "RELU_AUX_BIAS", bias=to_np(bias), ab=dt, **kw)
    with ge.Matmul(m, n, k, dt, "RELU_AUX_BIAS", **kw) as mm:
        before = mm.describe()
        ms, (D, aux) = mm.autotune(As.cuda(), Bs.cuda(), bias.cuda(), repeats=3)
        torch.cuda.synchronize()
        print(f"  forward: {before} -> {mm.describe()}, {ms:.4f} ms", flush=True)
        assert ms > 0.0
        assert _same(to_np(D), o["D"]) and _same(to_np(aux["relu_aux"]), o["mask"]), mm.describe()
        D2, aux2 = mm.execute(As.cuda(), Bs.cuda(), bias.cuda())
        torch.cuda.synchronize()
        assert _same(to_np(D2), o["D"]) and _same(to_np(aux2["relu_aux"]), o["mask"]), mm.describe()
    mask = torch.from_numpy(o["mask"].view(np.int32).copy()).cuda()
    ob = oracle.gemm_epilog(to_np(A2s), to_np(B2s), "DRELU_BGRAD", mask=o["mask"], ab=dt, **kw)
    with ge.Matmul(m, n, k, dt, "DRELU_BGRAD", **kw) as mm:
        ms, (dZ, g) = mm.autotune(A2s.cuda(), B2s.cuda(), relu_aux=mask, repeats=3)
        torch.cuda.synchronize()
        print(f"  backward: {mm.describe()}, {ms:.4f} ms", flush=True)
        assert _same(to_np(dZ), ob["D"]) and _same(to_np(g["drelu_bgrad"]), ob["bgrad"]), mm.describe()
        dZ2, g2 = mm.execute(A2s.cuda(), B2s.cuda(), relu_aux=mask)
        torch.cuda.synchronize()
        assert _same(to_np(dZ2), ob["D"]) and _same(to_np(g2["drelu_bgrad"]), ob["bgrad"]), mm.describe()


def test_autotune_argument_errors(gpu):
    ge = gpu
    h = ge.gemm_epilog_plan(64, 64, 64, ("f16", "f16", "f16"), "RELU_BIAS")
    try:
        A = torch.zeros(64, 64, dtype=torch.float16, device="cuda")
        bias = torch.zeros(64, dtype=torch.float16, device="cuda")
        D = torch.empty(64, 64, dtype=torch.float16, device="cuda")
        desc = ge.gemm_epilog_describe(h)
        assert ge.gemm_epilog_autotune(h, A, A, bias, D, repeats=0, check=False)[0] == 1
        assert ge.gemm_epilog_autotune(h, A, A, bias, D, repeats=1001, check=False)[0] == 1
        assert ge.gemm_epilog_autotune(h, A, A, None, D, repeats=2, check=False)[0] == 3
        assert ge.gemm_epilog_autotune(h, A.data_ptr() + 2, A, bias, D, repeats=2, check=False)[0] == 4
        assert ge.gemm_epilog_describe(h) == desc
        st, ms = ge.gemm_epilog_autotune(h, A, A, bias, D, repeats=2, check=False)
        torch.cuda.synchronize()
        assert st == 0 and ms > 0.0
        assert not D.float().any()
    finally:
        ge.gemm_epilog_free(h)
