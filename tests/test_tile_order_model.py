"""Host-side model of the prefill GEMM's XCD-aware tile order (xcd_tile in
gemm.hip): the 1-D grid index L goes to XCD L % 8, and the tile index t
given to it must visit every output tile exactly once, give each XCD one
contiguous range of tiles, and walk the M tiles of one group (gm M tiles, all of them by default) down
one weight panel before the next.
Nothing here runs on a GPU."""
import pytest

XCDS = 8


def xcd_tile(L, tiles_m, tiles_n, gm=None):
    gm = tiles_m if gm is None else gm
    T = tiles_m * tiles_n
    per, rem = divmod(T, XCDS)
    x, local = L % XCDS, L // XCDS
    t = x * (per + 1) + local if x < rem else rem * (per + 1) + (x - rem) * per + local
    grp = t // (gm * tiles_n)
    gsz = min(gm, tiles_m - grp * gm)
    r = t - grp * gm * tiles_n
    tn = r // gsz
    return grp * gm + r - tn * gsz, tn, t


@pytest.mark.parametrize("gm", [None, 1, 3, 4, 8])
@pytest.mark.parametrize("tiles_m,tiles_n", [(16, 224), (16, 16), (1, 1), (3, 5), (9, 7),
                                             (8, 1), (1, 13), (17, 33)])
def test_tile_order_is_a_bijection_with_contiguous_xcd_ranges(tiles_m, tiles_n, gm):
    if gm is not None and gm >= tiles_m:
        gm = None
    T = tiles_m * tiles_n
    seen = set()
    by_xcd = {}
    for L in range(T):
        tm, tn, t = xcd_tile(L, tiles_m, tiles_n, gm)
        assert 0 <= tm < tiles_m and 0 <= tn < tiles_n
        seen.add((tm, tn))
        by_xcd.setdefault(L % XCDS, []).append(t)
    assert len(seen) == T
    start = 0
    for x in range(min(XCDS, T)):
        ts = by_xcd[x]
        assert ts == list(range(start, start + len(ts)))     # in dispatch order, contiguous
        start += len(ts)
    assert start == T


def test_concurrent_tiles_of_an_xcd_share_weight_panels():
    """LLaMA-3-70B gate+up (4096 x 57344 in 256 x 256 tiles): the first 32
    tiles an XCD runs (one per CU) touch 2 weight panels, where the row-major
    grid order touched 28."""
    tiles_m, tiles_n = 16, 224
    for x in range(XCDS):
        Ls = [L for L in range(tiles_m * tiles_n) if L % XCDS == x][:32]
        panels = {xcd_tile(L, tiles_m, tiles_n)[1] for L in Ls}
        assert len(panels) == 2
        rowmajor = {L % tiles_n for L in Ls}
        assert len(rowmajor) == 28
