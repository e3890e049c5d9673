"""The parity helpers reject NaN outputs (CPU only): an element the kernel never writes
keeps the NaN fill of its output buffer, so every comparison must fail on it."""
import numpy as np
import pytest
import torch

from tests.helpers import assert_all_finite, assert_bgrad, assert_close, tight_ratio


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_assert_close_fails_on_nan(dt):
    npt = np.float32 if dt == "f32" else np.float16
    ref = np.ones((4, 4), npt)
    y = ref.copy()
    assert_close(y, ref, dt)   # equal: passes
    y[2, 3] = np.nan
    with pytest.raises(AssertionError):
        assert_close(y, ref, dt)
    y[2, 3] = np.inf
    with pytest.raises(AssertionError):
        assert_close(y, ref, dt)


def test_assert_close_fails_on_nan_bf16():
    ref = np.full((3, 5), 0x3F80, np.uint16)   # 1.0 in bf16
    y = ref.copy()
    assert_close(y, ref, "bf16")
    y[1, 1] = 0x7FC0                           # quiet NaN in bf16
    with pytest.raises(AssertionError):
        assert_close(y, ref, "bf16")


def test_assert_bgrad_fails_on_nan():
    r = np.array([1.0, 2.0, -3.0], np.float32)
    absum = np.array([1.0, 2.0, 3.0])
    assert_bgrad(r.copy(), r, absum, "f32")
    g = r.copy()
    g[1] = np.nan
    with pytest.raises(AssertionError):
        assert_bgrad(g, r, absum, "f32")


def test_tight_ratio_is_inf_on_nan():
    A = np.ones((2, 3), np.float32)
    B = np.ones((3, 2), np.float32)
    ref = (A @ B).astype(np.float32)
    assert tight_ratio(ref.copy(), ref, "f32", A, B) == 0.0
    y = ref.copy()
    y[0, 1] = np.nan
    assert tight_ratio(y, ref, "f32", A, B) == float("inf")
    assert max(0.5, tight_ratio(y, ref, "f32", A, B)) == float("inf")


def test_assert_all_finite():
    assert_all_finite(torch.ones(8, dtype=torch.float16), "ok")
    t = torch.ones(8, dtype=torch.bfloat16)
    t[3] = float("nan")
    with pytest.raises(AssertionError):
        assert_all_finite(t, "nan")
