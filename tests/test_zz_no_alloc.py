"""gemm_epilog_execute_noalloc (the entry point that allocates nothing, working in the
library's static per-device scratch) against plan + execute, the entry point whose
kernels it shares: the same plan on the same operands must give the same bits. Two and
more calls in a row share the scratch, the later ones on smaller problems, so what an
earlier call left there must not leak into a later one: the split tail's flags, the
bias-gradient partial sums and the unfused chains' intermediates. A problem whose
workspace exceeds the scratch is refused on the host."""
import numpy as np
import pytest
import torch

import oracle
from gemm_epilogues_epilog_amd import inputs
from tests.helpers import to_np

pytestmark = pytest.mark.gpu

T = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def outputs(m, n, dt, ep):
    D = torch.full((m, n), float("nan"), dtype=T[dt], device="cuda")
    aux = torch.full(((m + 31) // 32, n), 0x5A5A5A5A, dtype=torch.int32, device="cuda") \
        if ep == "RELU_AUX_BIAS" else None
    bg = torch.full((m,), float("nan"), dtype=T[dt], device="cuda") \
        if ep in ("DRELU_BGRAD", "DRELU_BGRAD_UNFUSED") else None
    return D, aux, bg


def both(ge, m, n, k, dt, ep, A, B, bias=None, mask=None, ta=False, tb=False, act=None):
    """(noalloc outputs, plan + execute outputs), each a list of device tensors."""
    res = []
    for noalloc in (True, False):
        D, aux, bg = outputs(m, n, dt, ep)
        if ep == "DRELU_BGRAD":
            aux = mask
        elif ep == "DRELU_BGRAD_UNFUSED":
            aux = act
        if noalloc:
            ge.gemm_epilog_execute_noalloc(m, n, k, (dt, dt, dt), ep, A, B, bias, D, aux, bg, int(ta), int(tb))
        else:
            h = ge.gemm_epilog_plan_ex(m, n, k, (dt, dt, dt), ep, int(ta), int(tb))
            try:
                ge.gemm_epilog_execute(h, A, B, bias, D, aux, bg)
                torch.cuda.synchronize()
            finally:
                ge.gemm_epilog_free(h)
        torch.cuda.synchronize()
        res.append([t for t in (D, aux if ep == "RELU_AUX_BIAS" else None, bg) if t is not None])
    return res


def same_bits(a, b):
    return all(torch.equal(x.view(torch.uint8) if x.dtype != torch.int32 else x,
                           y.view(torch.uint8) if y.dtype != torch.int32 else y) for x, y in zip(a, b))


def test_noalloc_matches_plan_and_execute(gpu):
    ge = gpu
    # 1. split tail (128 x 128 tiles, 32 tiles split over 128 workgroups): flags and partials
    m, n, k = 1024, 512, 2048
    print(f"[case] noalloc split RELU_AUX_BIAS f16 {m}x{n}x{k}", flush=True)
    info = ge.gemm_epilog_plan_info(m, n, k, ("f16",) * 3, "RELU_AUX_BIAS")
    assert info["split_workgroups"] > 0 and info["workspace_bytes"] <= ge.NOALLOC_SCRATCH_BYTES
    A, B, bias, A2, B2 = inputs.small_case(m, n, k, "f16", std=k ** -0.5, std_bias=0.5)
    na, pe = both(ge, m, n, k, "f16", "RELU_AUX_BIAS", A.cuda(), B.cuda(), bias.cuda())
    assert same_bits(na, pe)
    assert torch.isfinite(na[0]).all()
    # 2. a smaller problem right after, in the same scratch: DRELU_BGRAD (its partial
    #    sums) with a split tail of its own (fewer, shorter runs)
    m2, n2, k2 = 512, 264, 1024
    print(f"[case] noalloc DRELU_BGRAD bf16 {m2}x{n2}x{k2}", flush=True)
    A, B, bias, A2, B2 = inputs.small_case(m2, n2, k2, "bf16", std=k2 ** -0.5, std_bias=0.5)
    mask = torch.randint(-2 ** 31, 2 ** 31 - 1, ((m2 + 31) // 32, n2), dtype=torch.int32).cuda()
    na, pe = both(ge, m2, n2, k2, "bf16", "DRELU_BGRAD", A2.cuda(), B2.cuda(), mask=mask)
    assert same_bits(na, pe)
    # 3. smaller still: the unfused chain (T1, T2 in the scratch) and RELU_BIAS with A
    #    stored transposed
    m3, n3, k3 = 200, 264, 136
    A, B, bias, _, _ = inputs.integer_case(m3, n3, k3, "f16")
    print(f"[case] noalloc unfused f16 {m3}x{n3}x{k3}", flush=True)
    na, pe = both(ge, m3, n3, k3, "f16", "RELU_BIAS_UNFUSED", A.cuda(), B.cuda(), bias.cuda())
    assert same_bits(na, pe)
    o = oracle.gemm_epilog(to_np(A), to_np(B), "RELU_BIAS_UNFUSED", bias=to_np(bias))
    assert np.array_equal(to_np(na[0]).view(np.uint16), o["D"].view(np.uint16))
    #    the unfused backward (T1 in the scratch) on that forward's activation
    _, _, _, A2, B2 = inputs.integer_case(m3, n3, k3, "f16")
    act = na[0]
    print(f"[case] noalloc unfused backward f16 {m3}x{n3}x{k3}", flush=True)
    na, pe = both(ge, m3, n3, k3, "f16", "DRELU_BGRAD_UNFUSED", A2.cuda(), B2.cuda(), act=act)
    assert same_bits(na, pe)
    o = oracle.gemm_epilog(to_np(A2), to_np(B2), "DRELU_BGRAD_UNFUSED", act=to_np(act))
    assert np.array_equal(to_np(na[0]).view(np.uint16), o["D"].view(np.uint16))
    assert np.array_equal(to_np(na[1]).view(np.uint16), o["bgrad"].view(np.uint16))
    m4, n4, k4 = 128, 136, 72
    A, B, bias, _, _ = inputs.integer_case(m4, n4, k4, "bf16")
    print(f"[case] noalloc A transposed bf16 {m4}x{n4}x{k4}", flush=True)
    na, pe = both(ge, m4, n4, k4, "bf16", "RELU_BIAS", A.t().contiguous().cuda(), B.cuda(), bias.cuda(), ta=True)
    assert same_bits(na, pe)
    # 4. the 3-stage 128 x 128 ring with its split tail (runs of 16 k-tiles)
    m5, n5, k5 = 1024, 1024, 4096
    print(f"[case] noalloc 3-stage split RELU_AUX_BIAS f16 {m5}x{n5}x{k5}", flush=True)
    info = ge.gemm_epilog_plan_info(m5, n5, k5, ("f16",) * 3, "RELU_AUX_BIAS")
    assert info["stages"] == 3 and info["split_workgroups"] > 0, info
    A, B, bias, _, _ = inputs.small_case(m5, n5, k5, "f16", std=k5 ** -0.5, std_bias=0.5, seed=5)
    na, pe = both(ge, m5, n5, k5, "f16", "RELU_AUX_BIAS", A.cuda(), B.cuda(), bias.cuda())
    assert same_bits(na, pe)
    # 5. the first shape again (flags left by the earlier calls must be idle)
    A, B, bias, _, _ = inputs.small_case(m, n, k, "f16", std=k ** -0.5, std_bias=0.5, seed=3)
    na, pe = both(ge, m, n, k, "f16", "RELU_AUX_BIAS", A.cuda(), B.cuda(), bias.cuda())
    assert same_bits(na, pe)


def test_noalloc_refuses_what_does_not_fit(gpu):
    ge = gpu
    # the unfused chain at 4096 x 11008 needs 180 MB of T1 and T2
    m, n, k = 4096, 11008, 64
    info = ge.gemm_epilog_plan_info(m, n, k, ("f16",) * 3, "RELU_BIAS_UNFUSED")
    assert info["workspace_bytes"] > ge.NOALLOC_SCRATCH_BYTES
    A = torch.zeros(m, k, dtype=torch.float16, device="cuda")
    B = torch.zeros(k, n, dtype=torch.float16, device="cuda")
    bias = torch.zeros(m, dtype=torch.float16, device="cuda")
    D = torch.full((m, n), 7.0, dtype=torch.float16, device="cuda")
    st = ge.gemm_epilog_execute_noalloc(m, n, k, ("f16",) * 3, "RELU_BIAS_UNFUSED", A, B, bias, D, check=False)
    torch.cuda.synchronize()
    assert st == 7 and "static scratch" in ge.gemm_epilog_status_string(st)
    assert bool((D == 7.0).all()), "a refused call must launch nothing"
    # host-side argument errors come first, as for plan and execute
    assert ge.gemm_epilog_execute_noalloc(8, 12, 8, ("f16",) * 3, "RELU_BIAS", A, B, bias, D, check=False) == 2
    assert ge.gemm_epilog_execute_noalloc(64, 64, 64, ("f16",) * 3, "RELU_BIAS", A, B, None, D, check=False) == 3
