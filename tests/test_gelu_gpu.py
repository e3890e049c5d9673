"""The device GELU's own error, isolated: with A the identity (k = m) every accumulator
is exactly an element of B, so D = gelu(B + bias) computed on the GPU is compared with
the oracle's gelu (evaluated in double, then rounded) with no summation error in
between. The device evaluates 0.5 x (1 + tanh(u)) as x / (1 + 2^(-2 log2(e) u)) with
the hardware exp2 and reciprocal; its error bound, stated in units of 2^-24, is

    |y - y_ref| <= C (|y_ref| + |x| e/(1+e)^2 |t|) 2^-24 + 2^-126,   t = 2 log2(e) u,

where the second term is the argument's rounding carried through exp2 (relative error
of about ln 2 |t| ulps in e, scaled by the sigmoid's slope). C is measured here over
x in [-12, 12]; the fp32 tolerance of the fused path (1e-4 max(1, |y|)) holds with a
wide margin.

The oracle evaluates the pages' tanh form literally, in double: for x far below 0,
1 + tanh(u) cancels (tanh(u) is -1 to within 2^-53), so its value there is only good to
about |x| 2^-53 absolutely (it returns -0 where the true value is about -2e-16 at
x = -7.2). That term is part of the comparison's scale."""
import numpy as np
import pytest
import torch

import oracle
from tests import gpu_runner as R

pytestmark = pytest.mark.gpu

from tests.helpers import GELU_DEVICE_UNITS as C_BOUND   # units of 2^-24 (measured: at most 3.1)


def gelu_error_units(x, y, y_ref):
    x, y, y_ref = (np.asarray(v, np.float64) for v in (x, y, y_ref))
    u = 0.7978845608028654 * (x + 0.044715 * x ** 3)
    t = 2.0 * np.log2(np.e) * u
    e = np.exp2(np.clip(-t, -200, 200))
    slope = e / (1.0 + e) ** 2
    scale = (np.abs(y_ref) + np.abs(x) * slope * np.abs(t)) * 2.0 ** -24 + np.abs(x) * 2.0 ** -53 + 2.0 ** -126
    return np.abs(y - y_ref) / scale


@pytest.mark.parametrize("tile", ["S", "M"])
def test_device_gelu_error_bound_fp32(gpu, tile):
    m = k = 128
    n = 4096
    g = torch.Generator().manual_seed(5)
    B = (torch.rand(k, n, generator=g, dtype=torch.float64) * 24 - 12).float()
    B[:, :64] = torch.linspace(-3, 3, 64).float()   # a fine sweep through the bend
    A = torch.eye(m, dtype=torch.float32)
    bias = torch.zeros(m, dtype=torch.float32)
    out = R.run(gpu, "GELU_BIAS", "f32", A, B, bias, tile=tile)
    ref = oracle.gemm_epilog(A.numpy(), B.numpy(), "GELU_BIAS", bias=bias.numpy(), ab="f32")
    x = B.numpy()
    units = gelu_error_units(x, out["D"], ref["D"])
    worst = float(units.max())
    i = np.unravel_index(int(units.argmax()), units.shape)
    for j in np.argsort(units, axis=None)[-5:]:
        jj = np.unravel_index(int(j), units.shape)
        print(f"[gelu]   x = {x[jj]!r}: y = {out['D'][jj]!r}, y_ref = {ref['D'][jj]!r}, {units[jj]:.3f} units",
              flush=True)
    # plain relative error in units of 2^-24 where the output is at least 1e-3 in size (below that the
    # tail's tiny outputs make relative units meaningless; the bound above covers them)
    big = np.abs(ref["D"]) >= 1e-3
    rel = float((np.abs(out["D"] - ref["D"])[big] / (np.abs(ref["D"])[big] * 2.0 ** -24)).max())
    print(f"[gelu] tile {tile}: max error {worst:.3f} units of the bound's scale at x = {x[i]!r}, "
          f"y = {out['D'][i]!r}, y_ref = {ref['D'][i]!r}; relative error where |y_ref| >= 1e-3: "
          f"{rel:.1f} units of 2^-24", flush=True)
    assert np.isfinite(out["D"]).all()
    assert worst <= C_BOUND, f"device GELU error {worst} > {C_BOUND} units at x = {x[i]}"
    # the fused path's fp32 tolerance, for scale
    assert (np.abs(out["D"] - ref["D"]) <= 1e-4 * np.maximum(1.0, np.abs(ref["D"]))).all()
