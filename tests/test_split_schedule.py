"""Model of the split-tail schedule of the direct-to-LDS kernels (CPU only).

The plan gives the last, partly empty round of T tiles on P compute units
(T % P tiles) to runs of sk_units k-tiles, one workgroup per run, which computes its
partial piece (if any) before its owner piece (if any). The plan's numbers (whole
tiles, run length, split workgroups) come from the library's own host plan unit
through gemm_epilog_plan_info (no HIP call). This file models the kernel's piece
arithmetic independently and checks the invariants the kernel relies on: every
(tile, k-tile) is computed exactly once, each tile has exactly one owner piece
starting at k = 0, each run publishes at most one partial (which never starts at
k = 0), and the runs an owner waits for are exactly the runs that hold the rest of
its tile, each of which publishes before it waits for anything. Every published flag
has exactly one owner that waits for it, which is what lets that owner clear it
afterwards. The run length may also be forced (GE_SK_RUN), never below one run per
compute unit, so every split workgroup is resident at once. The kernel's own run
arithmetic (gek::sk_run) is checked against the same invariants under the sanitizers
(tests/test_plan_sanitize.py)."""
import os

import pytest

import gemm_epilogues_epilog_amd as ge


def plan(tiles, kt, cus=256, run=None, slots=None):
    """The library's split of `tiles` output tiles of k-tiles `kt`: (whole tiles, run
    length, split workgroups), or None when the plan does not split. slots = 2 cus
    asks for the 128 x 128 tile (two workgroups per CU), else the 256 x 256 tile."""
    lm = slots is not None and slots == 2 * cus
    bm = 128 if lm else 256
    saved = {k: os.environ.get(k) for k in ("GE_TILE", "GE_SK_RUN", "GE_STREAMK")}
    os.environ["GE_TILE"] = "LM" if lm else "LH"
    os.environ.pop("GE_STREAMK", None)
    if run is not None:
        os.environ["GE_SK_RUN"] = str(run)
    else:
        os.environ.pop("GE_SK_RUN", None)
    try:
        info = ge.gemm_epilog_plan_info(bm * tiles, bm, 64 * kt, ("f16", "f16", "f16"), "RELU_BIAS",
                                        compute_units=cus)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    assert info["tiles"] == tiles and info["tile_m"] == bm
    if info["split_workgroups"] == 0:
        return None
    return info["whole_tiles"], info["split_run_ktiles"], info["split_workgroups"]


def xcd_remap(i, g):
    per, rem, x, local = g // 8, g % 8, i % 8, i // 8
    return (x * (per + 1) if x < rem else rem * (per + 1) + (x - rem) * per) + local


def pieces(tiles, kt, cus=256, run=None):
    """(run, kind, tile, kb, nt) in the order one run's workgroup computes them."""
    dp, u, wgs = plan(tiles, kt, cus, run)
    total = (tiles - dp) * kt
    for wid in range(wgs):
        r = xcd_remap(wid, wgs)
        u0 = r * u
        u1 = min(total, u0 + u)
        ts = -(-u0 // kt) * kt
        if u0 < min(ts, u1):
            t = u0 // kt
            yield r, "partial", t, u0 - t * kt, min(ts, u1) - u0
        if ts < u1:
            yield r, "owner", ts // kt, 0, u1 - ts


def check(tiles, kt, cus=256, run=None):
    dp, u, wgs = plan(tiles, kt, cus, run)
    total = (tiles - dp) * kt
    assert wgs <= cus   # every split workgroup resident at once
    assert sorted(xcd_remap(i, wgs) for i in range(wgs)) == list(range(wgs))
    assert wgs * u >= total > (wgs - 1) * u
    cover, owners, partial_of = set(), {}, {}
    last_kind = {}
    for r, kind, t, kb, nt in pieces(tiles, kt, cus, run):
        assert kb + nt <= kt
        for kk in range(kb, kb + nt):
            assert (t, kk) not in cover
            cover.add((t, kk))
        if kind == "owner":
            assert kb == 0 and t not in owners
            owners[t] = r
        else:
            assert kb > 0 and r not in partial_of and r not in last_kind   # partial comes first
            partial_of[r] = t
        last_kind[r] = kind
    assert len(cover) == total
    waited = []
    for t in range(tiles - dp):
        r = owners[t]
        last = min(((t + 1) * kt - 1) // u, wgs - 1)
        partners = list(range(r + 1, last + 1))
        assert sorted(o for o, tt in partial_of.items() if tt == t) == partners
        waited += partners
    # each published flag is waited for by exactly one owner (who then clears it)
    assert sorted(waited) == sorted(partial_of)


def test_sparse_last_round_splits():
    # 4352 x 4096 with 256 x 256 tiles: 272 tiles, the last round holds 16
    dp, u, wgs = plan(272, 64)
    assert (dp, u, wgs) == (256, 16, 64)
    check(272, 64)


def test_two_workgroups_per_cu_rounds():
    # 128 x 128 tiles run two per CU: 352 of them (4096 x 1376) fill one round and do not
    # split; 32 (1024 x 512) still do, in runs of 8 of their 32 k-tiles
    assert plan(352, 64, slots=512) is None
    assert plan(32, 32, slots=512) == (0, 8, 128)
    assert plan(600, 64, slots=512) == (512, 22, 256)
    check(600, 64)


def test_full_or_mostly_full_rounds_do_not_split():
    assert plan(1024, 128) is None and plan(8192, 256) is None and plan(512, 64) is None
    assert plan(688, 64) is None   # 4096 x 11008: the last pass over the CUs is 69% full
    assert plan(255, 64) is None


@pytest.mark.parametrize("tiles", list(range(1, 1100, 13)))
@pytest.mark.parametrize("kt", [2, 3, 5, 8, 33, 64, 128])
def test_schedule_invariants(tiles, kt):
    if plan(tiles, kt) is not None:
        check(tiles, kt)


@pytest.mark.parametrize("tiles", [1, 8, 32, 100, 272])
@pytest.mark.parametrize("kt", [2, 8, 32, 64])
@pytest.mark.parametrize("run", [1, 2, 4, 16, 63])
def test_forced_run_lengths(tiles, kt, run):
    p = plan(tiles, kt, run=run)
    if p is not None:
        check(tiles, kt, run=run)
