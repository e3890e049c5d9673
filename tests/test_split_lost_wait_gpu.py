"""The split tail's bounded wait, forced to run out from the host: a plan made with
GE_SK_SPIN=0 lets each waiting workgroup poll zero times before it gives up, so whether
a partial is taken depends on the race with its publisher. Every kernel still ends
normally. Two protocols are covered: runs that cover whole tiles (each run finishes the
sub-tiles of some of its waves, counting publications per tile) and runs of any other
length (forced with GE_SK_RUN: an owner run adds its partners' partials, one flag per
partial). Each wave sub-tile of D must then be either exactly the result of a normal
plan or all NaN (a lost wait), never a wrong finite value; gemm_epilog_lost_waits counts
the lost waits, each of which accounts for at most one workgroup's eight sub-tiles.
Replays of a captured graph repeat the epoch of the capture, so a flag or counter left
set would hand a later replay the previous replay's partial: the replays below run on
new operand values each time and would show that as a wrong finite sub-tile."""
import os

import numpy as np
import pytest
import torch

from gemm_epilogues_epilog_amd import inputs
from tests import gpu_runner as R

pytestmark = pytest.mark.gpu


def tile_states(D, ref, bm, bn):
    """Per bm x bn block of D: 'ok' (bits equal to ref), 'nan' (all NaN) or 'bad'."""
    m, n = D.shape
    out = []
    for i in range(0, m, bm):
        for j in range(0, n, bn):
            d, r = D[i:i + bm, j:j + bn], ref[i:i + bm, j:j + bn]
            if torch.equal(d.view(torch.uint8), r.view(torch.uint8)):
                out.append("ok")
            elif bool(torch.isnan(d).all()):
                out.append("nan")
            else:
                out.append("bad")
    return out


# (shape, wave sub-tile, forced run length, whether the runs cover whole tiles)
CASES = [((1024, 512, 2048), (32, 64), None, True),      # 128 x 128 tiles, 4 parts per tile
         ((4352, 4096, 1024), (128, 64), None, True),    # 256 x 256 tiles, 4 parts per tile
         ((1024, 512, 2048), (32, 64), "12", False),     # runs of 12 of a tile's 32 k-tiles
         ((1024, 1024, 4096), (32, 64), None, True)]     # the 3-stage 128 x 128 ring, 4 parts per tile


@pytest.mark.parametrize("shape,sub,run_len,parts", CASES)
def test_lost_waits_leave_clean_flags(gpu, shape, sub, run_len, parts):
    ge = gpu
    m, n, k = shape
    dt = "f16"
    print(f"[case] lost waits m={m} n={n} k={k} run={run_len}", flush=True)
    A, B, bias, _, _ = inputs.small_case(m, n, k, dt, std=k ** -0.5, std_bias=0.5)
    Ad, Bd, bd = A.cuda(), B.cuda(), bias.cuda()
    D = torch.empty(m, n, dtype=torch.float16, device="cuda")
    ref = torch.empty_like(D)
    env = {"GE_SK_RUN": run_len} if run_len else {}
    with R.env(env):
        h0 = ge.gemm_epilog_plan(m, n, k, (dt, dt, dt), "RELU_BIAS")
    with R.env({**env, "GE_SK_SPIN": "0"}):
        h1 = ge.gemm_epilog_plan(m, n, k, (dt, dt, dt), "RELU_BIAS")
    try:
        desc = ge.gemm_epilog_describe(h1)
        assert "split" in desc and ("parts per tile" in desc) == parts, desc
        assert ge.gemm_epilog_describe(h0) == desc
        run = lambda: ge.gemm_epilog_execute(h1, Ad, Bd, bd, D)
        run()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run()
        torch.cuda.synchronize()
        lost_before = ge.gemm_epilog_lost_waits(h1)
        nan_tiles = 0
        for i in range(1, 7):
            Ad.copy_(inputs.normal(m, k, k ** -0.5, dt, seed=200 + i, tag=1))
            ge.gemm_epilog_execute(h0, Ad, Bd, bd, ref)          # the normal plan, eager
            torch.cuda.synchronize()
            D.fill_(float("nan"))
            if i % 2:
                graph.replay()                                   # frozen epoch
            else:
                run()                                            # eager, new epoch
            torch.cuda.synchronize()
            st = tile_states(D, ref, *sub)
            assert "bad" not in st, f"round {i}: a sub-tile holds wrong finite values"
            nan_tiles += st.count("nan")
        lost = ge.gemm_epilog_lost_waits(h1)
        print(f"[case] lost waits: {lost} (+{lost_before} at capture), NaN sub-tiles {nan_tiles}", flush=True)
        assert 8 * lost >= nan_tiles
        assert ge.gemm_epilog_lost_waits(h1) == 0            # the count was reset
        assert ge.gemm_epilog_lost_waits(h0) == 0            # the normal plan never lost a wait
        del graph
    finally:
        ge.gemm_epilog_free(h0)
        ge.gemm_epilog_free(h1)
