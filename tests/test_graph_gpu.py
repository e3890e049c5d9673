"""Executes captured into a HIP graph (torch.cuda.graph) and replayed: each replay runs on
new operand values written into the captured buffers, with eager work in between, and
must give the bits of an eager execute of the same plan on the same values. Covers the
split tail (whose flags carry the frozen epoch of the capture), the persistent kernel,
DRELU_BGRAD with its second pass, the three-kernel unfused chains (forward and
backward), transposed operands (one workgroup per tile and persistent), the four-wave
128 x 128 tile, the 3-stage ring of the eight-wave one and the persistent 192 x 256 and 128 x 256 tiles."""
import numpy as np
import pytest
import torch

from gemm_epilogues_epilog_amd import inputs

pytestmark = pytest.mark.gpu

CASES = [
    # (name, m, n, k, dtype, epilog, trans_a, trans_b, substring of the plan description)
    ("split tail", 1024, 512, 2048, "f16", "RELU_AUX_BIAS", False, False, "split"),
    ("persistent", 4096, 4096, 256, "bf16", "RELU_BIAS", False, False, "persistent"),
    ("bgrad", 1024, 1032, 512, "bf16", "DRELU_BGRAD", False, False, ""),
    ("bgrad split tail", 1024, 512, 2048, "f16", "DRELU_BGRAD", False, False, "split"),
    ("unfused", 512, 520, 256, "f16", "RELU_BIAS_UNFUSED", False, False, ""),
    ("unfused backward, A transposed", 512, 520, 264, "bf16", "DRELU_BGRAD_UNFUSED", True, False, "op_a T"),
    ("A transposed", 512, 520, 264, "bf16", "RELU_AUX_BIAS", True, False, "op_a T"),
    ("A transposed, persistent", 4096, 4096, 256, "bf16", "RELU_AUX_BIAS", True, False, "persistent"),
    ("B transposed, persistent", 4096, 4096, 256, "f16", "DRELU_BGRAD", False, True, "persistent"),
    ("four-wave 128x128", 4096, 1376, 4096, "f16", "RELU_BIAS", False, False, "waves 2x2"),
    ("three-stage 128x128, split tail", 1024, 1024, 4096, "f16", "RELU_AUX_BIAS", False, False, "stages 3"),
    ("192x256 persistent", 4096, 2752, 256, "bf16", "DRELU_BGRAD", False, False, "tile 192x256"),
    ("128x256 persistent", 2048, 4096, 256, "f16", "RELU_AUX_BIAS", False, False, "tile 128x256"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(gpu, case):
    ge = gpu
    name, m, n, k, dt, ep, ta, tb, want = case
    print(f"[case] graph {name}: {dt} {ep} m={m} n={n} k={k}", flush=True)
    t = inputs.TORCH_DT[dt]
    A, B, bias, A2, B2 = inputs.small_case(m, n, k, dt, std=k ** -0.5, std_bias=0.5)
    a_shape = (k, m) if ta else (m, k)
    Ad = torch.empty(a_shape, dtype=t, device="cuda")
    Bkn = B.cuda()                                   # (k, n), for the mask's forward pass
    Bd = B.t().contiguous().cuda() if tb else Bkn    # in the storage order the plan takes
    bd = bias.cuda()
    D = torch.empty(m, n, dtype=t, device="cuda")
    groups = (m + 31) // 32
    aux = torch.zeros(groups, n, dtype=torch.int32, device="cuda")
    backward = ep in ("DRELU_BGRAD", "DRELU_BGRAD_UNFUSED")
    bg = torch.empty(m, dtype=t, device="cuda") if backward else None
    if ep == "DRELU_BGRAD":
        # a mask from a forward of other operands, fixed for every replay
        hf = ge.gemm_epilog_plan(m, n, k, (dt, dt, dt), "RELU_AUX_BIAS")
        ge.gemm_epilog_execute(hf, A.cuda(), Bkn, bd, D, aux, None)
        torch.cuda.synchronize()
        ge.gemm_epilog_free(hf)
    if ep == "DRELU_BGRAD_UNFUSED":
        # the activation of an unfused forward of other operands, fixed for every replay
        aux = torch.empty(m, n, dtype=t, device="cuda")
        hf = ge.gemm_epilog_plan(m, n, k, (dt, dt, dt), "RELU_BIAS_UNFUSED")
        ge.gemm_epilog_execute(hf, A.cuda(), Bkn, bd, aux, None, None)
        torch.cuda.synchronize()
        ge.gemm_epilog_free(hf)
    h = ge.gemm_epilog_plan_ex(m, n, k, (dt, dt, dt), ep, int(ta), int(tb))
    try:
        assert want in ge.gemm_epilog_describe(h), ge.gemm_epilog_describe(h)
        use_bias = None if backward else bd

        def operands(i):
            # new values for replay i, written into the captured buffer
            Ai = inputs.normal(m, k, k ** -0.5, dt, seed=100 + i, tag=1)
            Ad.copy_(Ai.t().contiguous() if ta else Ai)

        def run():
            ge.gemm_epilog_execute(h, Ad, Bd, use_bias, D, aux, bg)

        def snapshot():
            out = [D.clone()]
            if ep == "RELU_AUX_BIAS":
                out.append(aux.clone())
            if bg is not None:
                out.append(bg.clone())
            return out

        operands(0)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run()   # warm-up outside the capture
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run()
        torch.cuda.synchronize()
        for i in range(1, 5):
            operands(i)
            run()   # eager, same plan
            torch.cuda.synchronize()
            ref = snapshot()
            D.fill_(float("nan"))   # eager work between replays
            if ep == "RELU_AUX_BIAS":
                aux.fill_(0x5A5A5A5A)
            if bg is not None:
                bg.fill_(float("nan"))
            graph.replay()
            torch.cuda.synchronize()
            got = snapshot()
            for r, g in zip(ref, got):
                assert torch.equal(r.view(torch.uint8) if r.dtype != torch.int32 else r,
                                   g.view(torch.uint8) if g.dtype != torch.int32 else g), f"replay {i}"
        del graph
    finally:
        ge.gemm_epilog_free(h)
