"""Python view of the CPU oracle (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this
package. It loads oracle/liboracle.so (built by oracle/build.py with g++) and never
touches the HIP library.

Arrays are numpy: float32 for fp32, numpy.float16 for fp16 and uint16 bit patterns
for bf16 (numpy has no bfloat16). dtype names: "f32", "f16", "bf16".
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

DT = {"f32": 0, "f16": 1, "bf16": 2}
EPILOG = {"NONE": 0, "RELU_BIAS": 1, "GELU_BIAS": 2, "RELU_AUX_BIAS": 3, "DRELU_BGRAD": 4,
          "BIAS": 5, "RELU_BIAS_UNFUSED": 100, "DRELU_BGRAD_UNFUSED": 101}
_NP = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            _build.build()
        L = ctypes.CDLL(_LIB_PATH)
        i64, c_int, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.oracle_gemm_epilog.argtypes = [i64, i64, i64, c_int, c_int, c_int, c_int,
                                         vp, vp, vp, vp, vp, vp, vp, vp, c_int]
        L.oracle_gemm_epilog.restype = c_int
        L.oracle_gemm_epilog_t.argtypes = [i64, i64, i64, c_int, c_int, c_int, c_int, c_int, c_int,
                                           vp, vp, vp, vp, vp, vp, vp, vp, c_int]
        L.oracle_gemm_epilog_t.restype = c_int
        L.oracle_gemm_epilog_act_t.argtypes = [i64, i64, i64, c_int, c_int, c_int, c_int, c_int, c_int,
                                               vp, vp, vp, vp, vp, vp, vp, vp, vp, c_int]
        L.oracle_gemm_epilog_act_t.restype = c_int
        L.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f32.restype = ctypes.c_float
        L.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_f16.restype = ctypes.c_uint16
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_gelu_tanh.argtypes = [ctypes.c_double]
        L.oracle_gelu_tanh.restype = ctypes.c_double
        L.oracle_default_threads.restype = c_int
        for name in ("oracle_f32_to_f16_n", "oracle_f16_to_f32_n",
                     "oracle_f32_to_bf16_n", "oracle_bf16_to_f32_n"):
            getattr(L, name).argtypes = [vp, vp, i64]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def default_threads() -> int:
    return int(lib().oracle_default_threads())


def f32_to_f16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, np.uint16)
    lib().oracle_f32_to_f16_n(_ptr(x), _ptr(y), x.size)
    return y


def f16_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h).view(np.uint16)
    y = np.empty(h.shape, np.float32)
    lib().oracle_f16_to_f32_n(_ptr(h), _ptr(y), h.size)
    return y


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, np.uint16)
    lib().oracle_f32_to_bf16_n(_ptr(x), _ptr(y), x.size)
    return y


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h).view(np.uint16)
    y = np.empty(h.shape, np.float32)
    lib().oracle_bf16_to_f32_n(_ptr(h), _ptr(y), h.size)
    return y


def gelu_tanh(x: float) -> float:
    return float(lib().oracle_gelu_tanh(float(x)))


def to_f32(a: np.ndarray, dt: str) -> np.ndarray:
    """Exact widening of an array stored in dtype dt (bit patterns for bf16)."""
    if dt == "f32":
        return np.asarray(a, np.float32)
    if dt == "f16":
        return f16_to_f32(np.asarray(a).view(np.uint16))
    return bf16_to_f32(np.asarray(a).view(np.uint16))


def gemm_epilog(A, B, epilog, bias=None, mask=None, ab="f16", d=None, vec=None,
                want_pre=False, nthreads=0, trans_a=False, trans_b=False, act=None):
    """Compute one epilogue on the CPU.

    A: (m,k), B: (k,n) arrays in dtype `ab` (A given as its (k,m) transpose with
    trans_a, B as its (n,k) transpose with trans_b); bias: (m,) in `vec` (forward
    epilogs); mask: uint32 (ceil(m/32), n) words, read by DRELU_BGRAD; act: the
    (m,n) forward activation in `d`, read by DRELU_BGRAD_UNFUSED.
    Returns a dict with "D" (m,n) in `d`, and as applicable "mask", "bgrad",
    "pre" (fp32 pre-activation, or dz for the backward) and "absum" (sum_j |dz|).
    """
    d = d or ab
    vec = vec or d
    ep = EPILOG[epilog]
    A = np.ascontiguousarray(A, dtype=_NP[ab])
    B = np.ascontiguousarray(B, dtype=_NP[ab])
    m, k = A.shape[::-1] if trans_a else A.shape
    k2, n = B.shape[::-1] if trans_b else B.shape
    assert k == k2, "inner dimensions differ"
    D = np.empty((m, n), _NP[d])
    out = {"D": D}
    uses_bias = epilog in ("BIAS", "RELU_BIAS", "GELU_BIAS", "RELU_AUX_BIAS", "RELU_BIAS_UNFUSED")
    if uses_bias and bias is not None:
        bias = np.ascontiguousarray(np.asarray(bias).reshape(m), dtype=_NP[vec])
    else:
        bias = None
    aux = None
    if epilog == "RELU_AUX_BIAS":
        aux = np.zeros(((m + 31) // 32, n), np.uint32)
        out["mask"] = aux
    elif epilog == "DRELU_BGRAD":
        aux = np.ascontiguousarray(mask, dtype=np.uint32)
        assert aux.shape == ((m + 31) // 32, n), "mask shape must be (ceil(m/32), n)"
    if epilog == "DRELU_BGRAD_UNFUSED":
        act = np.ascontiguousarray(act, dtype=_NP[d])
        assert act.shape == (m, n), "the activation must be (m, n)"
    else:
        act = None
    bgrad = None
    absum = None
    if epilog in ("DRELU_BGRAD", "DRELU_BGRAD_UNFUSED"):
        bgrad = np.empty(m, _NP[vec])
        absum = np.empty(m, np.float64)
        out["bgrad"] = bgrad
        out["absum"] = absum
    pre = np.empty((m, n), np.float32) if want_pre else None
    if want_pre:
        out["pre"] = pre
    rc = lib().oracle_gemm_epilog_act_t(m, n, k, DT[ab], DT[d], DT[vec], ep, int(bool(trans_a)),
                                        int(bool(trans_b)), _ptr(A), _ptr(B), _ptr(bias), _ptr(act), _ptr(D),
                                        _ptr(aux), _ptr(bgrad), _ptr(pre), _ptr(absum), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out
