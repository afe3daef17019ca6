"""Sliding-tile attention planning by brute force (test infrastructure).

[FPS §2.2] The 3D token grid is cut into M non-overlapping tiles {T_u}; query
tile u attends only to the key tiles v in a local window W(u) defined by an
infinity-norm bound on the distance of tile coordinates, so the work becomes
M * |W(u)| dense tile blocks.  The tile (6, 8, 8) is the page's choice.
[FPS §3.3, item 1] memory access is made contiguous by a block transpose:
tokens are regrouped so that each tile is contiguous.

Readings (the printed window formula is garbled):
  * window sizes are given in tiles per axis, w = (w_t, w_h, w_w); v is in W(u)
    iff |u_a - v_a| <= floor(w_a / 2) on every axis; windows are clipped at the
    grid border (not shifted);
  * kernel token order: tiles in raster order over (tile_t, tile_h, tile_w);
    inside a tile its real tokens in raster order over (dt, dh, dw), then its
    padding slots (the pages make each tile contiguous and leave the order
    inside it open; padding last fills whole key steps and query tiles);
  * a grid that is not a multiple of the tile is zero-padded at the high end;
    padded tokens are not keys (masked) and their outputs are not stored.
"""
import itertools

import numpy as np


class Plan:
    pass


def plan(grid, real_grid, tile, window):
    """Returns a Plan with
       perm      int32 [N]: raster index (real grid) of kernel position p, or -1
                 for padding;
       kv_valid  uint8 [N]: 1 where perm >= 0;
       win_off   int32 [M+1], win_idx int32 [sum |W|]: CSR window lists,
                 ascending tile index per row;
       lpt       int32 [M]: a schedule (no arithmetic depends on it): tiles by
                 decreasing |W(u)|, then by their window list (so that tiles
                 with the same list are adjacent), then by index;
       n_tokens, n_tiles, tile_tokens."""
    T, H, W = grid
    Tr, Hr, Wr = real_grid
    tt, th, tw = tile
    assert T % tt == 0 and H % th == 0 and W % tw == 0
    assert Tr <= T and Hr <= H and Wr <= W
    nt, nh, nw = T // tt, H // th, W // tw
    tiles = list(itertools.product(range(nt), range(nh), range(nw)))
    perm = []
    for (ut, uh, uw) in tiles:
        real = []
        for (dt, dh, dw) in itertools.product(range(tt), range(th), range(tw)):
            t, h, w = ut * tt + dt, uh * th + dh, uw * tw + dw
            if t < Tr and h < Hr and w < Wr:
                real.append((t * Hr + h) * Wr + w)
        perm += real + [-1] * (tt * th * tw - len(real))
    perm = np.array(perm, dtype=np.int32)
    rad = [wa // 2 for wa in window]
    off, idx = [0], []
    for u in tiles:
        for vi, v in enumerate(tiles):
            if all(abs(u[a] - v[a]) <= rad[a] for a in range(3)):
                idx.append(vi)
        off.append(len(idx))
    off = np.array(off, dtype=np.int32)
    sizes = np.diff(off)
    lists = [tuple(idx[off[u]:off[u + 1]]) for u in range(len(tiles))]
    lpt = sorted(range(len(tiles)), key=lambda u: (-sizes[u], lists[u], u))
    p = Plan()
    p.perm = perm
    p.kv_valid = (perm >= 0).astype(np.uint8)
    p.win_off = off
    p.win_idx = np.array(idx, dtype=np.int32)
    p.lpt = np.array(lpt, dtype=np.int32)
    p.n_tokens = len(perm)
    p.n_tiles = len(tiles)
    p.tile_tokens = tt * th * tw
    p.tile_coords = tiles
    return p


def gather_tokens(x_raster, perm):
    """[..., N_real, d] in raster order -> [..., N, d] in kernel order, zeros
    at padding positions."""
    out = np.zeros(x_raster.shape[:-2] + (len(perm), x_raster.shape[-1]), dtype=x_raster.dtype)
    ok = perm >= 0
    out[..., ok, :] = x_raster[..., perm[ok], :]
    return out


def key_blocks_for_tile(p, u, bn):
    """Ascending BN-key tile starts covering the window list of query tile u."""
    starts = []
    for v in p.win_idx[p.win_off[u]:p.win_off[u + 1]]:
        base = int(v) * p.tile_tokens
        starts.extend(range(base, base + p.tile_tokens, bn))
    return starts
