"""Shared test helpers: layout conversions of the library's documented output
layouts, tolerances, and oracle runs on host copies of the inputs."""
import numpy as np

from oracle import attention as OA
from oracle import quant as OQ
from oracle import sta as OS

# Attention parity gate (fp32 accumulate): max-abs and mean-abs error.
MAX_ABS = 1e-2
MEAN_ABS = 1e-3


def _pos_of_token():
    """Position inside a 64-token group of the transposed V codes for token t
    (t = 32a + 8b + 4g + c is stored at 32g + 16a + 4b + c)."""
    t = np.arange(64)
    a, b, g, c = t // 32, (t % 32) // 8, (t % 8) // 4, t % 4
    return 32 * g + 16 * a + 4 * b + c


POS = _pos_of_token()


def vt_to_tokens(vt, n):
    """[..., d, n_alloc] transposed V codes -> [..., n, d] in token order."""
    na = vt.shape[-1]
    idx = (np.arange(na) // 64) * 64 + POS[np.arange(na) % 64]
    tok = vt[..., idx]                       # [..., d, na] in token order
    return np.swapaxes(tok, -1, -2)[..., :n, :]


def oracle_operands(q, k, v, recipe, blk):
    """Oracle quantisation of one (b, h) slice each: returns per-(b,h) Operand
    triples as a nested list [B][H]."""
    B, H = q.shape[:2]
    out = [[None] * H for _ in range(B)]
    for b in range(B):
        for h in range(H):
            if recipe == "fp8":
                qc, qs = OQ.fp8_block_quantize(q[b, h], blk)
                kc, ks = OQ.fp8_block_quantize(k[b, h], blk)
                qo = OA.Operand("fp8_block", qc, qs, blk)
                ko = OA.Operand("fp8_block", kc, ks, blk)
            else:
                qc, qe = OQ.mxfp4_quantize(q[b, h])
                kc, ke = OQ.mxfp4_quantize(k[b, h])
                qo, ko = OA.Operand("mxfp4", qc, qe), OA.Operand("mxfp4", kc, ke)
            if recipe == "mxfp4_pv":
                vc, ve = OQ.mxfp4_token_quantize(v[b, h])
                vo = OA.Operand("mxfp4_tokens", vc, ve)
            else:
                vc, vs = OQ.fp8_channel_quantize(v[b, h])
                vo = OA.Operand("fp8_channel", vc, vs)
            out[b][h] = (qo, ko, vo)
    return out


def compare(got, ref):
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    return float(err.max()), float(err.mean())


def assert_close(got, ref, what=""):
    mx, mean = compare(got, ref)
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    assert mx <= MAX_ABS and mean <= MEAN_ABS, "%s: max-abs %.3g mean-abs %.3g" % (what, mx, mean)
    return mx, mean


def oracle_sta(x, grid, real_grid, tile, window, blk, bn, sm_scale):
    """Oracle sliding-tile attention of raster-order inputs x = (q, k, v)
    [B, H, N_real, d]: tokens regrouped tile-major, FP8 Q/K per blk-token
    block, key tiles of each query tile from its window list; returns
    [B, H, N_real, d] in raster order."""
    op = OS.plan(grid, real_grid, tile, window)
    q, k, v = (OS.gather_tokens(a, op.perm) for a in x)
    B, H = q.shape[:2]
    ops = oracle_operands(q, k, v, "fp8", blk)
    ref = np.zeros(x[0].shape, np.float32)
    for b in range(B):
        for h in range(H):
            qo, ko, vo = ops[b][h]
            for u in range(op.n_tiles):
                rows = np.arange(u * op.tile_tokens, (u + 1) * op.tile_tokens)
                o = OA.recipe_attention(qo, ko, vo, rows, sm_scale=sm_scale, bn=bn, kv_valid=op.kv_valid,
                                        key_blocks=OS.key_blocks_for_tile(op, u, bn))
                keep = op.perm[rows] >= 0
                ref[b, h, op.perm[rows][keep]] = o[keep]
    return ref


V4_SLOT_TOKEN = np.array([8 * ((j % 16) // 4) + 4 * (j // 16) + j % 4 for j in range(32)])


def v4_codes_to_tokens(codes_t, n):
    """GPU MXFP4 V codes [d, n_alloc/2] (two per byte, low nibble first, slot j
    of every 32-token group holding token V4_SLOT_TOKEN[j]) -> [n, d] codes in
    token order."""
    b = np.asarray(codes_t)
    d = b.shape[0]
    nib = np.empty((d, b.shape[1] * 2), np.uint8)
    nib[:, 0::2] = b & 0xF
    nib[:, 1::2] = b >> 4
    g = nib.reshape(d, -1, 32)
    tok = np.empty_like(g)
    tok[:, :, V4_SLOT_TOKEN] = g
    return tok.reshape(d, -1)[:, :n].T


def v4_scales_to_channels(scales, d=128):
    """GPU MXFP4 V scales [n_alloc/32, d] (channel c at 4 (c % 32) + c / 32)
    -> [n_alloc/32, d] in channel order."""
    c = np.arange(d)
    return np.asarray(scales)[:, 4 * (c % 32) + c // 32]
