"""Binding of the MFMA-rate probe (include/gemm_epilog_probe.h), a measurement aid that
lives in its own library, libgemm_epilog_probe.so, apart from the epilogue library.

The probe issues nothing but v_mfma_f32_32x32x16 on the operand values it is given, so
its rate on a workload's value distribution is the ceiling of any kernel on those values
under the chip's power limit; the benchmark reads the fused kernel's rate against it.
"""
import ctypes
import os

from . import GemmEpilogError, _dt, _ptr

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgemm_epilog_probe.so")
EXPORTS = ("gemm_epilog_mfma_probe", "gemm_epilog_device_info")

_lib = None


def load() -> ctypes.CDLL:
    """Load libgemm_epilog_probe.so; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with gemm_epilogues_epilog_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    vp, c_int = ctypes.c_void_p, ctypes.c_int
    L.gemm_epilog_mfma_probe.argtypes = [vp, ctypes.c_size_t, c_int, c_int, c_int, vp, vp]
    L.gemm_epilog_mfma_probe.restype = c_int
    L.gemm_epilog_device_info.argtypes = [ctypes.POINTER(c_int), ctypes.POINTER(c_int)]
    L.gemm_epilog_device_info.restype = c_int
    _lib = L
    return L


def gemm_epilog_mfma_probe(operands, dtype, iters: int, workgroups: int, out, stream=None, check: bool = True):
    """Enqueue the probe on fp16/bf16 operand values: `operands` a device tensor (its
    bytes are used), `out` a float32 device tensor of workgroups * 256 elements.
    Flop: workgroups * 16 * iters * 32768."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    nbytes = operands.numel() * operands.element_size()
    st = load().gemm_epilog_mfma_probe(_ptr(operands), nbytes, _dt(dtype), int(iters), int(workgroups), _ptr(out),
                                       stream)
    if check and st != 0:
        raise GemmEpilogError(st, "gemm_epilog_mfma_probe")
    return st


def gemm_epilog_device_info():
    """(compute units, peak shader clock in MHz) of the current device."""
    cus, khz = ctypes.c_int(0), ctypes.c_int(0)
    st = load().gemm_epilog_device_info(ctypes.byref(cus), ctypes.byref(khz))
    if st != 0:
        raise GemmEpilogError(st, "gemm_epilog_device_info")
    return cus.value, khz.value / 1000.0
