"""Pins for the oracle's sliding-tile planner: closed-form window counts per
axis, the token permutation, padding and the longest-first order."""
import numpy as np
import pytest

from oracle import sta as S


def _axis_counts(n, r):
    return np.array([min(u + r, n - 1) - max(u - r, 0) + 1 for u in range(n)])


def _closed_form_sizes(tile_grid, window):
    c = [_axis_counts(n, w // 2) for n, w in zip(tile_grid, window)]
    return (c[0][:, None, None] * c[1][None, :, None] * c[2][None, None, :]).ravel()


@pytest.mark.parametrize("grid,real,tile,window,pairs,lo,hi", [
    ((12, 48, 80), (12, 48, 80), (6, 8, 8), (3, 3, 3), 1792, 8, 18),
    ((24, 48, 80), (21, 45, 80), (6, 8, 8), (3, 5, 5), 10560, 18, 75),
])
def test_window_counts_closed_form(grid, real, tile, window, pairs, lo, hi):
    p = S.plan(grid, real, tile, window)
    tg = [g // t for g, t in zip(grid, tile)]
    sizes = np.diff(p.win_off)
    assert np.array_equal(sizes, _closed_form_sizes(tg, window))
    assert len(p.win_idx) == pairs == sizes.sum()
    assert sizes.min() == lo and sizes.max() == hi
    # every list ascending and within the infinity-norm bound
    rad = np.array(window) // 2
    coords = np.array(p.tile_coords)
    for u in range(p.n_tiles):
        lst = p.win_idx[p.win_off[u]:p.win_off[u + 1]]
        assert np.all(np.diff(lst) > 0)
        assert np.all(np.abs(coords[lst] - coords[u]) <= rad)


def test_permutation_and_padding():
    grid, real, tile = (24, 48, 80), (21, 45, 80), (6, 8, 8)
    p = S.plan(grid, real, tile, (3, 5, 5))
    assert p.n_tokens == 92160 and p.tile_tokens == 384 and p.n_tiles == 240
    ok = p.perm >= 0
    assert ok.sum() == 21 * 45 * 80
    assert np.array_equal(np.sort(p.perm[ok]), np.arange(21 * 45 * 80))
    assert np.array_equal(p.kv_valid, ok.astype(np.uint8))
    # first tile is the (6,8,8) box at the origin, raster inside
    t, rem = np.divmod(p.perm[:384], 45 * 80)
    h, w = np.divmod(rem, 80)
    assert np.array_equal(t, np.repeat(np.arange(6), 64))
    assert np.array_equal(h, np.tile(np.repeat(np.arange(8), 8), 6))
    assert np.array_equal(w, np.tile(np.arange(8), 48))
    # a tile cut by the grid's end along h (tile rows 40..47, real rows 0..44):
    # its 5 x 8 real positions of each of its 6 frames first, in raster order,
    # then its 144 padding slots
    u = 5 * 10 + 3                      # tile (0, 5, 3)
    blk = p.perm[u * 384:(u + 1) * 384]
    t, rem = np.divmod(blk[:240], 45 * 80)
    h, w = np.divmod(rem, 80)
    assert np.array_equal(t, np.repeat(np.arange(6), 40))
    assert np.array_equal(h, np.tile(np.repeat(np.arange(40, 45), 8), 6))
    assert np.array_equal(w, np.tile(np.arange(24, 32), 30))
    assert np.all(blk[240:] == -1)
    # every tile: its real tokens are exactly the real points of its 3D box
    for u in range(p.n_tiles):
        ut, uh, uw = u // 60, (u // 10) % 6, u % 10
        box = [(tt * 45 + hh) * 80 + ww for tt in range(6 * ut, min(6 * ut + 6, 21))
               for hh in range(8 * uh, min(8 * uh + 8, 45)) for ww in range(8 * uw, 8 * uw + 8)]
        blk = p.perm[u * 384:(u + 1) * 384]
        assert np.array_equal(blk[:len(box)], np.array(box)) and np.all(blk[len(box):] == -1)
    # gather puts zeros at padding positions
    x = np.arange(21 * 45 * 80, dtype=np.float32)[None, :, None]
    g = S.gather_tokens(x, p.perm)
    assert np.all(g[0, ~ok, 0] == 0) and np.array_equal(g[0, ok, 0], p.perm[ok].astype(np.float32))


def test_lpt_order():
    p = S.plan((24, 48, 80), (21, 45, 80), (6, 8, 8), (3, 5, 5))
    sizes = np.diff(p.win_off)
    s = sizes[p.lpt]
    assert np.all(np.diff(s) <= 0)
    assert np.array_equal(np.sort(p.lpt), np.arange(p.n_tiles))
