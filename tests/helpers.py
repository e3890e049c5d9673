"""Comparison helpers for the parity tests (tolerances of the fused-epilogue path).

Float outputs: |y - y_ref| <= tol * max(1, |y_ref|), tol = 2e-2 for fp16/bf16 and 1e-4
for fp32. Mask bits: exact except where the oracle's |pre-activation| < 1e-3. Bias
gradient: |g - g_ref| <= 1e-3 * sum_j |dz[i, j]|.
"""
import numpy as np
import torch

import oracle

TOL = {"f16": 2e-2, "bf16": 2e-2, "f32": 1e-4}
MASK_EXEMPT = 1e-3
BGRAD_TOL = 1e-3


def to_np(t: torch.Tensor) -> np.ndarray:
    """CPU copy in the oracle's representation (bf16 as uint16 bit patterns)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.int32:
        return t.numpy().view(np.uint32)
    return t.numpy()


def widen(a: np.ndarray, dt: str) -> np.ndarray:
    return oracle.to_f32(a, dt).astype(np.float64)


def assert_close(y: np.ndarray, y_ref: np.ndarray, dt: str, what: str = "D"):
    y = widen(y, dt)
    y_ref = widen(y_ref, dt)
    err = np.abs(y - y_ref)
    bound = TOL[dt] * np.maximum(1.0, np.abs(y_ref))
    # "not within" rather than "beyond": a NaN error (an element never written, or a
    # NaN where the reference is finite) fails too
    bad = ~(err <= bound) | (~np.isfinite(y) & np.isfinite(y_ref))
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements outside tolerance, e.g. "
                             + ", ".join(f"{tuple(i)}: {y[tuple(i)]} vs {y_ref[tuple(i)]}" for i in idx))
    return float((err / np.maximum(1.0, np.abs(y_ref))).max()) if err.size else 0.0


def unpack_mask(words: np.ndarray, m: int) -> np.ndarray:
    """(ceil(m/32), n) uint32 words -> (m, n) bool, bit i%32 of word (i/32, j)."""
    words = np.asarray(words).view(np.uint32)
    g, n = words.shape
    bits = (words[:, None, :] >> np.arange(32, dtype=np.uint32)[None, :, None]) & 1
    return bits.reshape(g * 32, n)[:m].astype(bool)


def assert_mask(mask: np.ndarray, mask_ref: np.ndarray, pre_ref: np.ndarray, m: int):
    mask = np.asarray(mask).view(np.uint32)
    mask_ref = np.asarray(mask_ref).view(np.uint32)
    assert mask.shape == mask_ref.shape
    # pad bits (rows >= m) must be zero
    g = mask.shape[0]
    if g * 32 > m:
        pad = np.uint32(((1 << 32) - 1) ^ ((1 << (m % 32)) - 1)) if m % 32 else np.uint32(0)
        assert not (mask[-1] & pad).any(), "pad bits of the last mask group are not zero"
    a, b = unpack_mask(mask, m), unpack_mask(mask_ref, m)
    diff = (a != b) & (np.abs(pre_ref) >= MASK_EXEMPT)
    assert not diff.any(), f"{int(diff.sum())} mask bits differ outside the |pre| < 1e-3 band"
    return int(((a != b)).sum())


def assert_bgrad(bg: np.ndarray, bg_ref: np.ndarray, absum: np.ndarray, dt: str):
    g = widen(bg, dt)
    r = widen(bg_ref, dt)
    # the reference is rounded to dt too: allow the output rounding on top of 1e-3
    rnd = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8, "f32": 2.0 ** -24}[dt]
    bound = BGRAD_TOL * absum + rnd * np.abs(r) + 1e-30
    bad = ~(np.abs(g - r) <= bound) | (~np.isfinite(g) & np.isfinite(r))
    assert not bad.any(), f"bgrad: {int(bad.sum())} of {bad.size} outside 1e-3 * sum|dz|"


GELU_DEVICE_UNITS = 4.0   # the device GELU's error bound in units of 2^-24 (tests/test_gelu_gpu.py)


def gelu_device_term(x: np.ndarray, y_ref: np.ndarray) -> np.ndarray:
    """Bound on the device GELU's own error beyond the output rounding, for
    pre-activations x (float64): GELU_DEVICE_UNITS 2^-24 (|y_ref| + |x| s |t|), with
    t = 2 log2(e) u the exp2 argument and s = e/(1+e)^2 the sigmoid's slope (the
    argument's rounding carried through exp2), plus |x| 2^-53 for the oracle's own
    cancellation of 1 + tanh(u) in double where x is far below 0."""
    u = 0.7978845608028654 * (x + 0.044715 * x ** 3)
    t = 2.0 * np.log2(np.e) * u
    e = np.exp2(np.clip(-t, -200.0, 200.0))
    s = e / (1.0 + e) ** 2
    return GELU_DEVICE_UNITS * 2.0 ** -24 * (np.abs(y_ref) + np.abs(x) * s * np.abs(t)) + np.abs(x) * 2.0 ** -53


def tight_ratio(y: np.ndarray, y_ref: np.ndarray, dt: str, A: np.ndarray, B: np.ndarray, act_slope: float = 1.0,
                gelu_pre: np.ndarray = None):
    """Error relative to a rounding-error model: output rounding 2^-p |y_ref| plus
    fp32 accumulation k 2^-24 sum_kk |a b| (times the activation's slope), plus, for
    GELU (gelu_pre: the oracle's pre-activations), the device GELU's own error bound.
    Returns max ratio (should be O(1))."""
    p = {"f16": 11, "bf16": 8, "f32": 24}[dt]
    y = widen(y, dt)
    y_ref = widen(y_ref, dt)
    k = A.shape[1]
    absprod = np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64))
    scale = 2.0 ** -p * np.abs(y_ref) + act_slope * k * 2.0 ** -24 * absprod + 1e-7
    if gelu_pre is not None:
        scale = scale + gelu_device_term(np.asarray(gelu_pre, np.float64), y_ref)
    ratio = np.abs(y - y_ref) / scale
    # NaN anywhere (an unwritten element) counts as an unbounded error
    return float("inf") if np.isnan(ratio).any() else float(ratio.max())


def assert_all_finite(t, what: str):
    """Every element of a full-size device output is finite (outputs are filled with NaN
    before each run, so this also shows that every element was written)."""
    import torch
    bad = int((~torch.isfinite(t)).sum().item())
    assert bad == 0, f"{what}: {bad} non-finite elements (unwritten or NaN)"
