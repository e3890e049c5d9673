"""Model of the tile order of the direct-to-LDS kernels (CPU only).

Workgroup ids are renumbered so that each of the 8 XCDs walks a contiguous range of
positions (xcd_remap), and positions are laid out in groups of group_m m-tiles, m
fastest inside a group (raster). The persistent kernel's workgroup w takes ids
w, w + G, w + 2G, ... This model restates that arithmetic and checks that every
tile is computed exactly once for every grid the plan can launch and that the tiles
an XCD runs together form compact blocks (so they share A and B panels in its L2);
the plan's choice of group size is read from the plan itself (gemm_epilog_plan_info)."""
import itertools

import pytest


def xcd_remap(i, g):
    per, rem, x, local = g // 8, g % 8, i % 8, i // 8
    return (x * (per + 1) if x < rem else rem * (per + 1) + (x - rem) * per) + local


def raster(pos, tiles_m, tiles_n, group_m):
    gsz = group_m * tiles_n
    g = pos // gsz
    first_m = g * group_m
    rows = min(tiles_m - first_m, group_m)
    inner = pos - g * gsz
    return first_m + inner % rows, inner // rows


@pytest.mark.parametrize("tiles_m,tiles_n", [(1, 1), (1, 43), (16, 43), (17, 16), (32, 32), (256, 32), (3, 5),
                                             (9, 7), (100, 3)])
@pytest.mark.parametrize("group_m", [1, 4, 8, 16])
def test_every_tile_once(tiles_m, tiles_n, group_m):
    T = tiles_m * tiles_n
    assert sorted(xcd_remap(i, T) for i in range(T)) == list(range(T))
    seen = set()
    for pos in range(T):
        tm, tn = raster(pos, tiles_m, tiles_n, group_m)
        assert 0 <= tm < tiles_m and 0 <= tn < tiles_n
        seen.add((tm, tn))
    assert len(seen) == T


@pytest.mark.parametrize("T", [1, 7, 255, 256, 257, 688, 1024, 8192])
def test_persistent_grid_covers_every_id_once(T, cus=256):
    G = min(T, cus)
    ids = [w + G * j for w in range(G) for j in range((T - w + G - 1) // G)]
    assert sorted(ids) == list(range(T))


def test_concurrent_tiles_of_an_xcd_share_panels():
    # the headline grid (16 x 43 tiles of 256 x 256) on 256 workgroups: in every round
    # the 32 tiles of one XCD touch at most 8 m-tiles and 5 n-tiles (4 when aligned)
    tiles_m, tiles_n, G = 16, 43, 256
    T = tiles_m * tiles_n
    for x, j in itertools.product(range(8), range(3)):
        ids = [w + G * j for w in range(x, G, 8) if w + G * j < T]
        tiles = [raster(xcd_remap(v, T), tiles_m, tiles_n, 8) for v in ids]
        ms, ns = {t[0] for t in tiles}, {t[1] for t in tiles}
        assert len(ms) <= 8 and len(ns) <= 5, (x, j, ms, ns)


def plan_group(m, n, k):
    """The group size the plan itself chooses (host code of the library, no GPU)."""
    import gemm_epilogues_epilog_amd as ge
    return ge.gemm_epilog_plan_info(m, n, k, ("f16", "f16", "f16"), "RELU_BIAS")["group_m"]


def test_group_size_rule():
    # whole-tile plans: groups of 8 m-tiles, or 4 once A outgrows the 256 MB MALL
    assert plan_group(4096, 11008, 4096) == 8       # headline: A is 32 MiB
    assert plan_group(8192, 8192, 8192) == 8        # A is 128 MiB
    assert plan_group(65536, 8192, 16384) == 4      # A is 2 GiB
    assert plan_group(16376, 8192, 8192) == 8 and plan_group(16384, 8192, 8192) == 4   # A of 256 MiB
    # split plans: groups of 4
    assert plan_group(1024, 1024, 4096) == 4
