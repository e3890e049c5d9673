"""Python binding of the fused GEMM + epilogue library for MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP kernels of
libgemm_epilog.so (built by gemm_epilogues_epilog_amd/build.py). There is no CPU
fallback; if the library is missing every call raises.

Low-level functions carry the names of the C ABI in include/gemm_epilog.h:
gemm_epilog_plan, gemm_epilog_plan_ex, gemm_epilog_plan_info, gemm_epilog_execute,
gemm_epilog_execute_noalloc, gemm_epilog_autotune, gemm_epilog_lost_waits,
gemm_epilog_free, gemm_epilog_aux_bytes, gemm_epilog_workspace_bytes,
gemm_epilog_describe, gemm_epilog_status_string.
Pointers may be given as torch tensors (device memory), integers or None.

`Matmul` wraps them in the stateful plan / execute / free object with a context
manager that the nvmath-python pages describe ("Fusing bias addition via the
nvmath-python epilog mechanism", paragraph 4, lifecycle item; "Dissecting
nvmath-python", paragraph on the plan-execute-free lifecycle). Its execute returns
D, (D, {"relu_aux": mask}) for RELU_AUX_BIAS, or (D, {"drelu_bgrad": bgrad}) for
DRELU_BGRAD (and its unfused baseline, which takes the forward activation as `act`),
as the pages' auxiliary outputs ("Fusing epilogs with matrix
multiplication using nvmath-python", sections on the forward epilogs and on the
DRELU_BGRAD path).
"""
import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgemm_epilog.so")

F32, F16, BF16 = 0, 1, 2
DTYPES = {"f32": F32, "f16": F16, "bf16": BF16}
EPILOG = {"NONE": 0, "RELU_BIAS": 1, "GELU_BIAS": 2, "RELU_AUX_BIAS": 3, "DRELU_BGRAD": 4, "BIAS": 5,
          "RELU_BIAS_UNFUSED": 100, "DRELU_BGRAD_UNFUSED": 101}
STATUS = {0: "GE_OK", 1: "GE_ERR_INVALID_VALUE", 2: "GE_ERR_NOT_SUPPORTED", 3: "GE_ERR_NULL_POINTER",
          4: "GE_ERR_MISALIGNED", 5: "GE_ERR_ALLOC", 6: "GE_ERR_HIP", 7: "GE_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 64 << 20
EXPORTS = ("gemm_epilog_plan", "gemm_epilog_plan_ex", "gemm_epilog_plan_info", "gemm_epilog_execute",
           "gemm_epilog_execute_noalloc",
           "gemm_epilog_autotune", "gemm_epilog_lost_waits", "gemm_epilog_free",
           "gemm_epilog_aux_bytes", "gemm_epilog_workspace_bytes", "gemm_epilog_describe",
           "gemm_epilog_status_string")
OP_N, OP_T = 0, 1


class ge_dtypes_t(ctypes.Structure):
    _fields_ = [("ab", ctypes.c_int), ("d", ctypes.c_int), ("vec", ctypes.c_int)]


class ge_plan_info_t(ctypes.Structure):
    _fields_ = [("tile_m", ctypes.c_int), ("tile_n", ctypes.c_int), ("tile_k", ctypes.c_int), ("waves", ctypes.c_int),
                ("tiles", ctypes.c_int64), ("persistent_workgroups", ctypes.c_int), ("whole_tiles", ctypes.c_int),
                ("split_workgroups", ctypes.c_int), ("split_run_ktiles", ctypes.c_int), ("group_m", ctypes.c_int),
                ("workspace_bytes", ctypes.c_size_t), ("stages", ctypes.c_int)]


class GemmEpilogError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {gemm_epilog_status_string(status)}")


_lib = None


def load() -> ctypes.CDLL:
    """Load libgemm_epilog.so; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with gemm_epilogues_epilog_amd/build.py "
                           "(or __graft_entry__.build()); there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, c_int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.gemm_epilog_plan.argtypes = [i64, i64, i64, ge_dtypes_t, c_int, ctypes.POINTER(vp)]
    L.gemm_epilog_plan.restype = c_int
    L.gemm_epilog_plan_ex.argtypes = [i64, i64, i64, ge_dtypes_t, c_int, c_int, c_int, ctypes.POINTER(vp)]
    L.gemm_epilog_plan_ex.restype = c_int
    L.gemm_epilog_plan_info.argtypes = [i64, i64, i64, ge_dtypes_t, c_int, c_int, c_int, c_int,
                                        ctypes.POINTER(ge_plan_info_t)]
    L.gemm_epilog_plan_info.restype = c_int
    L.gemm_epilog_execute.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp]
    L.gemm_epilog_execute.restype = c_int
    L.gemm_epilog_execute_noalloc.argtypes = [i64, i64, i64, ge_dtypes_t, c_int, c_int, c_int,
                                              vp, vp, vp, vp, vp, vp, vp]
    L.gemm_epilog_execute_noalloc.restype = c_int
    L.gemm_epilog_autotune.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, c_int, ctypes.POINTER(ctypes.c_float)]
    L.gemm_epilog_autotune.restype = c_int
    L.gemm_epilog_lost_waits.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_uint32)]
    L.gemm_epilog_lost_waits.restype = c_int
    L.gemm_epilog_free.argtypes = [vp]
    L.gemm_epilog_free.restype = c_int
    L.gemm_epilog_aux_bytes.argtypes = [i64, i64]
    L.gemm_epilog_aux_bytes.restype = ctypes.c_size_t
    L.gemm_epilog_workspace_bytes.argtypes = [vp]
    L.gemm_epilog_workspace_bytes.restype = ctypes.c_size_t
    L.gemm_epilog_describe.argtypes = [vp]
    L.gemm_epilog_describe.restype = ctypes.c_char_p
    L.gemm_epilog_status_string.argtypes = [c_int]
    L.gemm_epilog_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def _dt(x) -> int:
    return DTYPES[x] if isinstance(x, str) else int(x)


def _ep(x) -> int:
    return EPILOG[x] if isinstance(x, str) else int(x)


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def gemm_epilog_status_string(status: int) -> str:
    return load().gemm_epilog_status_string(int(status)).decode()


def gemm_epilog_aux_bytes(m: int, n: int) -> int:
    return int(load().gemm_epilog_aux_bytes(m, n))


def gemm_epilog_plan(m: int, n: int, k: int, dtypes, epilog, check: bool = True):
    """dtypes: (ab, d, vec) names or codes. Returns the handle (int), or
    (status, handle) when check=False."""
    ab, d, vec = (_dt(x) for x in dtypes)
    h = ctypes.c_void_p()
    st = load().gemm_epilog_plan(int(m), int(n), int(k), ge_dtypes_t(ab, d, vec), _ep(epilog), ctypes.byref(h))
    if not check:
        return st, h.value
    if st != 0:
        raise GemmEpilogError(st, "gemm_epilog_plan")
    return h.value


def gemm_epilog_plan_ex(m: int, n: int, k: int, dtypes, epilog, op_a: int = OP_N, op_b: int = OP_N,
                        check: bool = True):
    """gemm_epilog_plan with operand storage orders: op_a = OP_T takes A as its (k, m)
    transpose, op_b = OP_T takes B as its (n, k) transpose."""
    ab, d, vec = (_dt(x) for x in dtypes)
    h = ctypes.c_void_p()
    st = load().gemm_epilog_plan_ex(int(m), int(n), int(k), ge_dtypes_t(ab, d, vec), _ep(epilog), int(op_a),
                                    int(op_b), ctypes.byref(h))
    if not check:
        return st, h.value
    if st != 0:
        raise GemmEpilogError(st, "gemm_epilog_plan_ex")
    return h.value


def gemm_epilog_plan_info(m: int, n: int, k: int, dtypes, epilog, op_a: int = OP_N, op_b: int = OP_N,
                          compute_units: int = 256, check: bool = True):
    """The configuration a plan would take on a device with `compute_units` compute
    units, computed on the host without any HIP call: a dict of ge_plan_info_t's
    fields (or (status, dict) with check=False)."""
    ab, d, vec = (_dt(x) for x in dtypes)
    info = ge_plan_info_t()
    st = load().gemm_epilog_plan_info(int(m), int(n), int(k), ge_dtypes_t(ab, d, vec), _ep(epilog), int(op_a),
                                      int(op_b), int(compute_units), ctypes.byref(info))
    out = {name: getattr(info, name) for name, _ in ge_plan_info_t._fields_}
    if not check:
        return st, out
    if st != 0:
        raise GemmEpilogError(st, "gemm_epilog_plan_info")
    return out


def gemm_epilog_execute(handle, A, B, bias=None, D=None, aux=None, bgrad=None, stream=None, check: bool = True):
    """Enqueue one execute. stream: hipStream_t as int, a torch stream, or None for
    torch's current stream on the current device."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    st = load().gemm_epilog_execute(handle, _ptr(A), _ptr(B), _ptr(bias), _ptr(D), _ptr(aux), _ptr(bgrad), stream)
    if check and st != 0:
        raise GemmEpilogError(st, "gemm_epilog_execute")
    return st


def gemm_epilog_execute_noalloc(m: int, n: int, k: int, dtypes, epilog, A, B, bias=None, D=None, aux=None,
                                bgrad=None, op_a: int = OP_N, op_b: int = OP_N, stream=None, check: bool = True):
    """Plan and enqueue in one call that allocates nothing: the workspace is the library's
    static per-device scratch (NOALLOC_SCRATCH_BYTES). Calls that overlap on one device
    race. Returns the status (raises unless check=False)."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    ab, d, vec = (_dt(x) for x in dtypes)
    st = load().gemm_epilog_execute_noalloc(int(m), int(n), int(k), ge_dtypes_t(ab, d, vec), _ep(epilog), int(op_a),
                                            int(op_b), _ptr(A), _ptr(B), _ptr(bias), _ptr(D), _ptr(aux), _ptr(bgrad),
                                            stream)
    if check and st != 0:
        raise GemmEpilogError(st, "gemm_epilog_execute_noalloc")
    return st


def gemm_epilog_autotune(handle, A, B, bias=None, D=None, aux=None, bgrad=None, stream=None, repeats: int = 10,
                         check: bool = True):
    """Time the plan's candidate configurations on these operands and keep the fastest.
    Returns the chosen configuration's mean ms per execute (or (status, ms) with
    check=False). Synchronises the stream."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    ms = ctypes.c_float(0.0)
    st = load().gemm_epilog_autotune(handle, _ptr(A), _ptr(B), _ptr(bias), _ptr(D), _ptr(aux), _ptr(bgrad), stream,
                                     int(repeats), ctypes.byref(ms))
    if not check:
        return st, ms.value
    if st != 0:
        raise GemmEpilogError(st, "gemm_epilog_autotune")
    return ms.value


def gemm_epilog_lost_waits(handle, stream=None) -> int:
    """Synchronise the stream and return (and reset) the count of split-tail waits of
    this plan that ran out (their tiles hold NaN)."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    n = ctypes.c_uint32(0)
    st = load().gemm_epilog_lost_waits(handle, stream, ctypes.byref(n))
    if st != 0:
        raise GemmEpilogError(st, "gemm_epilog_lost_waits")
    return int(n.value)


def gemm_epilog_free(handle) -> int:
    return int(load().gemm_epilog_free(handle))


def gemm_epilog_workspace_bytes(handle) -> int:
    return int(load().gemm_epilog_workspace_bytes(handle))


def gemm_epilog_describe(handle) -> str:
    return load().gemm_epilog_describe(handle).decode()


_TORCH_NAME = {"torch.float32": "f32", "torch.float16": "f16", "torch.bfloat16": "bf16"}
_BIAS_EPILOGS = ("RELU_BIAS", "GELU_BIAS", "RELU_AUX_BIAS", "BIAS", "RELU_BIAS_UNFUSED")


def _require(t, name: str, dtype_name: str, numel: int, device) -> None:
    """A caller-supplied tensor that the kernels will read or write through its data
    pointer: a contiguous device tensor on `device`, of element type `dtype_name`
    ("f32", "f16", "bf16" or "i32") and exactly `numel` elements. Raises ValueError,
    before any pointer reaches the library, when it is not."""
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a device tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the operands on {device}")
    got = "i32" if str(t.dtype) == "torch.int32" else _TORCH_NAME.get(str(t.dtype))
    if got != dtype_name:
        raise ValueError(f"{name} must hold {dtype_name} elements, not {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, not {t.numel()}")


class Matmul:
    """Stateful fused matmul over torch device tensors: plan once, execute many times.

    mm = Matmul(m, n, k, "f16", "RELU_BIAS"); mm.plan(); D = mm.execute(A, B, bias); mm.free()
    or `with Matmul(...) as mm:` which plans on entry and frees on exit.
    trans_a=True takes A as its (k, m) transpose, trans_b=True B as its (n, k) transpose.
    DRELU_BGRAD_UNFUSED takes the forward pass's (m, n) activation as `act`.
    """

    def __init__(self, m: int, n: int, k: int, dtype: str, epilog: str, vec_dtype: Optional[str] = None,
                 trans_a: bool = False, trans_b: bool = False):
        self.m, self.n, self.k = int(m), int(n), int(k)
        self.dtype, self.epilog = dtype, epilog
        self.vec_dtype = vec_dtype or dtype
        self.trans_a, self.trans_b = bool(trans_a), bool(trans_b)
        self.handle = None

    def plan(self):
        if self.handle is None:
            dts = (self.dtype, self.dtype, self.vec_dtype)
            if self.trans_a or self.trans_b:
                self.handle = gemm_epilog_plan_ex(self.m, self.n, self.k, dts, self.epilog,
                                                  OP_T if self.trans_a else OP_N, OP_T if self.trans_b else OP_N)
            else:
                self.handle = gemm_epilog_plan(self.m, self.n, self.k, dts, self.epilog)
        return self

    def describe(self) -> str:
        return gemm_epilog_describe(self.handle) if self.handle is not None else ""

    def _outputs(self, A, B, bias, relu_aux, out, bgrad, act=None):
        """Check the operands and every tensor given against the plan, then plan (once)
        and allocate the outputs not given."""
        import torch
        for name, t in (("A", A), ("B", B)):
            if not (getattr(t, "is_cuda", False) and t.is_contiguous() and _TORCH_NAME.get(str(t.dtype)) == self.dtype):
                raise ValueError(f"{name} must be a contiguous {self.dtype} device tensor")
        if B.device != A.device:
            raise ValueError("A and B must be on the same device")
        a_shape = (self.k, self.m) if self.trans_a else (self.m, self.k)
        b_shape = (self.n, self.k) if self.trans_b else (self.k, self.n)
        if tuple(A.shape) != a_shape or tuple(B.shape) != b_shape:
            raise ValueError("operand shapes do not match the plan")
        dev = A.device
        aux_words = (self.m + 31) // 32
        if self.epilog in _BIAS_EPILOGS:
            if bias is None:
                raise ValueError(f"{self.epilog} needs a bias of m = {self.m} values")
            _require(bias, "bias", self.vec_dtype, self.m, dev)
        if out is not None:
            _require(out, "out", self.dtype, self.m * self.n, dev)
        if relu_aux is not None:
            _require(relu_aux, "relu_aux", "i32", aux_words * self.n, dev)
        if bgrad is not None:
            _require(bgrad, "bgrad", self.vec_dtype, self.m, dev)
        if self.epilog == "DRELU_BGRAD" and relu_aux is None:
            raise ValueError("DRELU_BGRAD needs the relu_aux mask of the forward pass")
        if self.epilog == "DRELU_BGRAD_UNFUSED":
            if act is None:
                raise ValueError("DRELU_BGRAD_UNFUSED needs the forward activation as act")
            _require(act, "act", self.dtype, self.m * self.n, dev)
        if self.handle is None:
            self.plan()
        if out is None:
            out = torch.empty((self.m, self.n), dtype=A.dtype, device=dev)
        if self.epilog == "RELU_AUX_BIAS" and relu_aux is None:
            relu_aux = torch.empty((aux_words, self.n), dtype=torch.int32, device=dev)
        if self.epilog in ("DRELU_BGRAD", "DRELU_BGRAD_UNFUSED") and bgrad is None:
            vt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[self.vec_dtype]
            bgrad = torch.empty(self.m, dtype=vt, device=dev)
        return relu_aux, out, bgrad

    def _result(self, out, relu_aux, bgrad):
        if self.epilog == "RELU_AUX_BIAS":
            return out, {"relu_aux": relu_aux}
        if self.epilog in ("DRELU_BGRAD", "DRELU_BGRAD_UNFUSED"):
            return out, {"drelu_bgrad": bgrad}
        return out

    def execute(self, A, B, bias=None, relu_aux=None, out=None, bgrad=None, stream=None, act=None):
        relu_aux, out, bgrad = self._outputs(A, B, bias, relu_aux, out, bgrad, act)
        aux = act if self.epilog == "DRELU_BGRAD_UNFUSED" else relu_aux
        gemm_epilog_execute(self.handle, A, B, bias, out, aux, bgrad, stream)
        return self._result(out, relu_aux, bgrad)

    def autotune(self, A, B, bias=None, relu_aux=None, out=None, bgrad=None, stream=None, repeats: int = 10,
                 act=None):
        """Time the candidate configurations on these operands and keep the fastest in
        the plan (gemm_epilog_autotune). Returns (ms per execute, the result as
        execute returns it)."""
        relu_aux, out, bgrad = self._outputs(A, B, bias, relu_aux, out, bgrad, act)
        aux = act if self.epilog == "DRELU_BGRAD_UNFUSED" else relu_aux
        ms = gemm_epilog_autotune(self.handle, A, B, bias, out, aux, bgrad, stream, repeats)
        return ms, self._result(out, relu_aux, bgrad)

    def free(self):
        if self.handle is not None:
            gemm_epilog_free(self.handle)
            self.handle = None

    def __enter__(self):
        return self.plan()

    def __exit__(self, *exc):
        self.free()
        return False

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass
