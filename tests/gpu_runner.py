"""Run one planned epilogue on cuda:0 through the C ABI, with guard zones around every
output so writes outside the stated extents are caught."""
import os
from contextlib import contextmanager

import numpy as np
import torch

from tests.helpers import to_np

TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
GUARD = 256   # guard elements (multiple of 16 bytes for every dtype)


@contextmanager
def tile_env(tile):
    """Force a tile configuration for the plans made inside. A "-nosk" suffix also turns
    off the split tail (GE_STREAMK=0); "-runN" forces split runs of N k-tiles
    (GE_SK_RUN), so runs that do not divide a tile's k loop take the owner-adds-partials
    protocol."""
    saved = {k: os.environ.get(k) for k in ("GE_TILE", "GE_STREAMK", "GE_SK_RUN")}
    if tile:
        name, _, opt = tile.partition("-")
        os.environ["GE_TILE"] = name
        if opt == "nosk":
            os.environ["GE_STREAMK"] = "0"
        elif opt.startswith("run"):
            os.environ["GE_SK_RUN"] = opt[3:]
    try:
        yield
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


@contextmanager
def env(values):
    """Set environment variables for the plans made inside."""
    saved = {k: os.environ.get(k) for k in values}
    os.environ.update(values)
    try:
        yield
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def guarded(numel, dtype, fill):
    buf = torch.full((numel + 2 * GUARD,), fill, dtype=dtype, device="cuda")
    return buf, buf[GUARD:GUARD + numel]


def check_guard(buf, fill, what):
    b = buf.detach()
    head, tail = b[:GUARD], b[-GUARD:]
    f = torch.tensor(fill, dtype=b.dtype, device=b.device)
    ok = bool(((head == f) | (head != head)).all() and ((tail == f) | (tail != tail)).all()) \
        if b.dtype.is_floating_point else bool((head == f).all() and (tail == f).all())
    assert ok, f"{what}: a write landed outside the output extent"


def run(ge, epilog, dt, A, B, bias=None, mask=None, vec=None, tile=None, stream=None, repeat=1,
        trans_a=False, trans_b=False, act=None):
    """A, B, bias, mask, act: CPU or device tensors; A is (k, m) with trans_a and B is
    (n, k) with trans_b; act is the (m, n) forward activation DRELU_BGRAD_UNFUSED reads.
    Returns numpy outputs + plan description."""
    vec = vec or dt
    m, k = A.shape[::-1] if trans_a else A.shape
    n = B.shape[0] if trans_b else B.shape[1]
    with tile_env(tile):
        if trans_a or trans_b:
            h = ge.gemm_epilog_plan_ex(m, n, k, (dt, dt, vec), epilog, int(trans_a), int(trans_b))
        else:
            h = ge.gemm_epilog_plan(m, n, k, (dt, dt, vec), epilog)
    try:
        Ad = A.to("cuda").contiguous()
        Bd = B.to("cuda").contiguous()
        bd = bias.to("cuda").contiguous() if bias is not None else None
        dbuf, D = guarded(m * n, TORCH[dt], float("nan"))
        D = D.view(m, n)
        groups = (m + 31) // 32
        abuf = aux = None
        if epilog == "RELU_AUX_BIAS":
            abuf, aux = guarded(groups * n, torch.int32, 0x5A5A5A5A)
            aux = aux.view(groups, n)
        elif epilog == "DRELU_BGRAD":
            aux = mask.to("cuda").contiguous()
        elif epilog == "DRELU_BGRAD_UNFUSED":
            aux = act.to("cuda").contiguous()
        gbuf = bg = None
        if epilog in ("DRELU_BGRAD", "DRELU_BGRAD_UNFUSED"):
            gbuf, bg = guarded(m, TORCH[vec], float("nan"))
        if stream is not None:
            stream.wait_stream(torch.cuda.current_stream())
        for _ in range(repeat):
            ge.gemm_epilog_execute(h, Ad, Bd, bd, D, aux, bg, stream)
        torch.cuda.synchronize()
        check_guard(dbuf, float("nan"), "D")
        out = {"D": to_np(D) if m * n <= (1 << 26) else None, "desc": ge.gemm_epilog_describe(h), "D_dev": D}
        if abuf is not None:
            check_guard(abuf, 0x5A5A5A5A, "mask")
            out["mask"] = to_np(aux)
            out["mask_dev"] = aux
        if gbuf is not None:
            check_guard(gbuf, float("nan"), "bgrad")
            out["bgrad"] = to_np(bg)
        return out
    finally:
        ge.gemm_epilog_free(h)


def np_in(t: torch.Tensor) -> np.ndarray:
    return to_np(t)
