"""The ReLU tie on the GPU: integer operands with an integer bias, so that a share of
the pre-activations is exactly 0. The reading of the pages taken for the tie (ReLU of
0 is +0, its mask bit is 0, and the masked gradient there is +0; "Fusing bias addition
via the nvmath-python epilog mechanism", paragraph 3: RELU_BIAS and the RELU_AUX_BIAS
mask; "Fusing epilogs with matrix multiplication using nvmath-python", section on the
DRELU_BGRAD path) must hold bit for bit: every output equals the oracle's, every tie
gives the +0 bit pattern, and every tie's mask bit is 0. Products and sums are exact
integers, so any summation order gives the same bits."""
import numpy as np
import pytest
import torch

import oracle
from gemm_epilogues_epilog_amd import inputs
from tests import gpu_runner as R
from tests.helpers import to_np, unpack_mask

pytestmark = pytest.mark.gpu

# (300, 520, 256): k over 4 k-tiles of 64, so the 256 x 256 tile runs the persistent
# kernel; (257, 392, 72): ragged m and a ragged k tail
CASES = [(dt, tile, shape) for dt, tiles in (("f32", [None, "S", "M"]), ("f16", [None, "L", "LH", "LM", "LM4", "LMD", "L3", "LW"]),
                                             ("bf16", [None, "L", "LH", "LM", "LM4", "LMD", "L3", "LW"]))
         for tile in tiles for shape in ((300, 520, 256), (257, 392, 72))]


def bits(a):
    return np.asarray(a).view(np.uint32 if a.dtype.itemsize == 4 else np.uint16)


@pytest.mark.parametrize("dt,tile,shape", CASES)
def test_relu_tie_bit_exact(gpu, dt, tile, shape):
    m, n, k = shape
    print(f"[case] tie {dt} tile {tile} m={m} n={n} k={k}", flush=True)
    A, B, bias, A2, B2 = inputs.integer_tie_case(m, n, k, dt)
    a, b, c = to_np(A), to_np(B), to_np(bias)
    pre = A.double().numpy() @ B.double().numpy() + bias.double().numpy()[:, None]
    ties = pre == 0
    assert ties.sum() > 50, "the case must hold ties"
    for ep in ("RELU_BIAS", "RELU_AUX_BIAS"):
        g = R.run(gpu, ep, dt, A, B, bias, tile=tile)
        o = oracle.gemm_epilog(a, b, ep, bias=c, ab=dt)
        assert np.array_equal(bits(g["D"]), bits(o["D"])), f"{ep} {g['desc']}"
        assert not bits(g["D"])[ties].any(), f"{ep}: a tie gave a nonzero bit pattern (-0?) {g['desc']}"
        if ep == "RELU_AUX_BIAS":
            assert np.array_equal(g["mask"].view(np.uint32), o["mask"]), g["desc"]
            mbits = unpack_mask(g["mask"], m)
            assert not mbits[ties].any(), "a tie has its mask bit set"
            assert np.array_equal(mbits, pre > 0)
            fwd_mask = g["mask"]
    mask = torch.from_numpy(fwd_mask.view(np.int32).copy())
    gb = R.run(gpu, "DRELU_BGRAD", dt, A2, B2, mask=mask, tile=tile)
    ob = oracle.gemm_epilog(to_np(A2), to_np(B2), "DRELU_BGRAD", mask=fwd_mask.view(np.uint32), ab=dt)
    assert np.array_equal(bits(gb["D"]), bits(ob["D"])), gb["desc"]
    assert not bits(gb["D"])[ties].any(), "a tie's masked gradient is not +0"
    assert np.array_equal(bits(gb["bgrad"]), bits(ob["bgrad"])), gb["desc"]


LAYOUT_CASES = [(dt, lay, tile) for dt in ("f16", "bf16") for lay in ("TN", "NT", "TT")
                for tile in (None, "L", "LH", "LM", "LMD")]


@pytest.mark.parametrize("dt,lay,tile", LAYOUT_CASES)
def test_relu_tie_bit_exact_transposed(gpu, dt, lay, tile):
    # the same reading with A given as its (k, m) transpose and/or B as its (n, k) one
    ta, tb = lay[0] == "T", lay[1] == "T"
    m, n, k = 304, 392, 256
    print(f"[case] tie {dt} {lay} tile {tile} m={m} n={n} k={k}", flush=True)
    A, B, bias, A2, B2 = inputs.integer_tie_case(m, n, k, dt)
    pre = A.double().numpy() @ B.double().numpy() + bias.double().numpy()[:, None]
    ties = pre == 0
    assert ties.sum() > 50, "the case must hold ties"
    st = lambda t, tr: t.t().contiguous() if tr else t
    As, Bs, A2s, B2s = st(A, ta), st(B, tb), st(A2, ta), st(B2, tb)
    kw = dict(trans_a=ta, trans_b=tb)
    g = R.run(gpu, "RELU_AUX_BIAS", dt, As, Bs, bias, tile=tile, **kw)
    o = oracle.gemm_epilog(to_np(As), to_np(Bs), "RELU_AUX_BIAS", bias=to_np(bias), ab=dt, **kw)
    assert np.array_equal(bits(g["D"]), bits(o["D"])), g["desc"]
    assert not bits(g["D"])[ties].any(), f"a tie gave a nonzero bit pattern (-0?) {g['desc']}"
    assert np.array_equal(g["mask"].view(np.uint32), o["mask"]), g["desc"]
    assert not unpack_mask(g["mask"], m)[ties].any(), "a tie has its mask bit set"
    mask = torch.from_numpy(g["mask"].view(np.int32).copy())
    gb = R.run(gpu, "DRELU_BGRAD", dt, A2s, B2s, mask=mask, tile=tile, **kw)
    ob = oracle.gemm_epilog(to_np(A2s), to_np(B2s), "DRELU_BGRAD", mask=g["mask"].view(np.uint32), ab=dt, **kw)
    assert np.array_equal(bits(gb["D"]), bits(ob["D"])), gb["desc"]
    assert not bits(gb["D"])[ties].any(), "a tie's masked gradient is not +0"
    assert np.array_equal(bits(gb["bgrad"]), bits(ob["bgrad"])), gb["desc"]
