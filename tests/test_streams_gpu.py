"""Plans on several streams at once.

Each plan owns its workspace (split-tail flags and partial slots, bias-gradient
partials), so executes of different plans may run concurrently on different streams.
Three plans, a split tail of 128 x 128 runs (1024 x 512 x 2048), the persistent
256 x 256 kernel (4000 x 8200 x 256, ragged) and a DRELU_BGRAD with its second pass
(2048 x 1024 x 512), are launched in turn on three side streams, 12 rounds, and each
one's last output must equal the oracle's bits on integer inputs, with no split-tail
wait run out."""
import numpy as np
import pytest
import torch

import oracle
from gemm_epilogues_epilog_amd import inputs
from tests.helpers import to_np

pytestmark = pytest.mark.gpu


def test_three_plans_on_three_streams(gpu):
    ge = gpu
    cases = [((1024, 512, 2048), "f16", "RELU_AUX_BIAS"), ((4000, 8200, 256), "bf16", "RELU_BIAS"),
             ((2048, 1024, 512), "bf16", "DRELU_BGRAD")]
    print("[case] three plans on three streams", flush=True)
    runs = []
    for (m, n, k), dt, ep in cases:
        A, B, bias, _, _ = inputs.integer_case(m, n, k, dt, second=False)
        a, b, c = to_np(A), to_np(B), to_np(bias)
        tdt = A.dtype
        mask = None
        if ep == "DRELU_BGRAD":
            fwd = oracle.gemm_epilog(a, b, "RELU_AUX_BIAS", bias=c, ab=dt)
            mask = torch.from_numpy(fwd["mask"].view(np.int32).copy()).cuda()
            ref = oracle.gemm_epilog(a, b, ep, mask=fwd["mask"], ab=dt)
        else:
            ref = oracle.gemm_epilog(a, b, ep, bias=c, ab=dt)
        h = ge.gemm_epilog_plan(m, n, k, (dt, dt, dt), ep)
        run = {"h": h, "A": A.cuda(), "B": B.cuda(), "bias": bias.cuda() if ep != "DRELU_BGRAD" else None,
               "D": torch.full((m, n), float("nan"), dtype=tdt, device="cuda"), "ref": ref, "ep": ep,
               "desc": ge.gemm_epilog_describe(h), "stream": torch.cuda.Stream()}
        run["aux"] = (torch.zeros((m + 31) // 32, n, dtype=torch.int32, device="cuda") if ep == "RELU_AUX_BIAS"
                      else mask)
        run["bgrad"] = torch.full((m,), float("nan"), dtype=tdt, device="cuda") if ep == "DRELU_BGRAD" else None
        runs.append(run)
    assert "split" in runs[0]["desc"] and "persistent workgroups" in runs[1]["desc"], [r["desc"] for r in runs]
    try:
        torch.cuda.synchronize()
        for _ in range(12):
            for r in runs:
                ge.gemm_epilog_execute(r["h"], r["A"], r["B"], r["bias"], r["D"], r["aux"], r["bgrad"],
                                       stream=r["stream"].cuda_stream)
        torch.cuda.synchronize()
        for r in runs:
            assert np.array_equal(to_np(r["D"]).view(np.uint8), r["ref"]["D"].view(np.uint8)), r["desc"]
            if r["ep"] == "RELU_AUX_BIAS":
                assert np.array_equal(to_np(r["aux"]).view(np.uint32), r["ref"]["mask"]), r["desc"]
            if r["ep"] == "DRELU_BGRAD":
                assert np.array_equal(to_np(r["bgrad"]).view(np.uint8), r["ref"]["bgrad"].view(np.uint8)), r["desc"]
            assert ge.gemm_epilog_lost_waits(r["h"], r["stream"].cuda_stream) == 0, r["desc"]
    finally:
        torch.cuda.synchronize()
        for r in runs:
            ge.gemm_epilog_free(r["h"])
