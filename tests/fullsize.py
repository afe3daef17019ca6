"""Oracle side of the full-size parity tests.

The oracle is run per head in spawned worker processes (CPU only: this module
imports neither torch nor the GPU library).  Workers read the float32 inputs
[1, H, N_real, d] from shared memory created by the test, quantise their
head with the oracle quantizers (after the 3D token reorder for grid
workloads), run the oracle recipe for that head's sampled query rows and
return the rows plus digests of the codes and scales, which the test compares
with digests of the GPU's codes.
"""
import hashlib
from multiprocessing import shared_memory

import numpy as np

from oracle import attention as OA
from oracle import quant as OQ
from oracle import sta as OS
from workloads import CONFIGS

FULL_WINDOW = (99, 99, 99)     # window reaching every tile (dense on a grid)


def digest(*arrays):
    h = hashlib.sha256()
    for a in arrays:
        a = np.ascontiguousarray(a)
        h.update(str(a.dtype).encode())
        h.update(str(a.shape).encode())
        h.update(a.tobytes())
    return h.hexdigest()


def oracle_plan(cfg):
    return OS.plan(cfg.grid, cfg.real_grid, cfg.tile, cfg.window if cfg.window else FULL_WINDOW)


def kernel_positions(plan, tokens):
    """Kernel (tile-major) positions of raster tokens."""
    ok = plan.perm >= 0
    inv = np.empty(int(ok.sum()), np.int64)
    inv[plan.perm[ok]] = np.nonzero(ok)[0]
    return inv[tokens]


def head_job(job):
    """(config name, shm names, shape, head, raster tokens, bn) ->
    (head, tokens, oracle rows [len, d] float32, digests, unquantised rows).
    The unquantised rows are exact softmax attention of the bf16 inputs
    themselves (float64), the path the quantised recipe approximates."""
    name, shm_names, shape, head, tokens, bn = job
    cfg = CONFIGS[name]
    blocks = [shared_memory.SharedMemory(name=n) for n in shm_names]
    try:
        q, k, v = (np.ndarray(shape, np.float32, buffer=b.buf)[0, head].copy() for b in blocks)
    finally:
        for b in blocks:
            b.close()
    kv_valid, plan = None, None
    rows = np.asarray(tokens, np.int64)
    if cfg.grid is not None:
        plan = oracle_plan(cfg)
        q, k, v = (OS.gather_tokens(a[None], plan.perm)[0] for a in (q, k, v))
        kv_valid = plan.kv_valid
        rows = kernel_positions(plan, rows)
    if cfg.recipe == "fp8":
        qc, qs = OQ.fp8_block_quantize(q, cfg.blk)
        kc, ks = OQ.fp8_block_quantize(k, cfg.blk)
        qo, ko = OA.Operand("fp8_block", qc, qs, cfg.blk), OA.Operand("fp8_block", kc, ks, cfg.blk)
    else:
        qc, qs = OQ.mxfp4_quantize(q)
        kc, ks = OQ.mxfp4_quantize(k)
        qo, ko = OA.Operand("mxfp4", qc, qs), OA.Operand("mxfp4", kc, ks)
    if cfg.recipe == "mxfp4_pv":
        vc, vs = OQ.mxfp4_token_quantize(v)
        vo = OA.Operand("mxfp4_tokens", vc, vs)
    else:
        vc, vs = OQ.fp8_channel_quantize(v)
        vo = OA.Operand("fp8_channel", vc, vs)
    digests = {"q": digest(qc, qs), "k": digest(kc, ks), "v": digest(vc, vs)}
    sm = 1.0 / np.sqrt(cfg.d)
    out = np.zeros((len(rows), cfg.d), np.float32)
    if cfg.mode == "sta":
        tiles = rows // plan.tile_tokens
        for u in np.unique(tiles):
            sel = np.nonzero(tiles == u)[0]
            kb = OS.key_blocks_for_tile(plan, int(u), bn)
            out[sel] = OA.recipe_attention(qo, ko, vo, rows[sel], sm_scale=sm, bn=bn,
                                           kv_valid=kv_valid, key_blocks=kb)
    else:
        out[:] = OA.recipe_attention(qo, ko, vo, rows, sm_scale=sm, bn=bn,
                                     causal=cfg.mode == "causal", kv_valid=kv_valid)
    return head, tokens, out, digests, unquantised_rows(cfg, plan, q, k, v, rows, sm)


def unquantised_rows(cfg, plan, q, k, v, rows, sm):
    """softmax(q k^T sm) v for the given kernel-order rows in float64, with the
    workload's key set (causal prefix, sliding-tile window, padding mask)."""
    n = q.shape[0]
    keep = np.ones((len(rows), n), bool)
    if cfg.mode == "causal":
        keep &= np.arange(n)[None, :] <= rows[:, None]
    if plan is not None:
        keep &= plan.kv_valid.astype(bool)[None, :]
        if cfg.mode == "sta":
            tiles = np.arange(n) // plan.tile_tokens
            for x, r in enumerate(rows):
                u = r // plan.tile_tokens
                keep[x] &= np.isin(tiles, plan.win_idx[plan.win_off[u]:plan.win_off[u + 1]])
    return OA.brute_force(q[rows], k, v, sm, mask=keep).astype(np.float32)


U_BF16 = 2.0 ** -8


def sampled_bounds(qh, kh, vh, o, do, lse, sm, rows, cols, causal):
    """First-order bounds of the library's bf16 roundings for dQ[rows],
    dK[cols] and dV[cols]: sm u (P A + |dS|) |K^| for dQ rows, its transpose
    with |Q^| for dK, 2 u P^T |dO| for dV (A = |dO| |V^|^T), from float64
    operands [N, d], the forward output o, dO and lse (log2 units)."""
    l64 = np.asarray(lse, np.float64)
    o, do = np.asarray(o, np.float64), np.asarray(do, np.float64)
    dd = (do * o).sum(axis=1)
    allq = np.arange(qh.shape[0])

    def pmat(ri, ci):
        s = (qh[ri] @ kh[ci].T) * (sm * OA.LOG2E)
        p = np.exp2(s - l64[ri][:, None])
        return np.where(ci[None, :] <= ri[:, None], p, 0.0) if causal else p

    p = pmat(rows, allq)
    w = p * (np.abs(do[rows]) @ np.abs(vh).T) + np.abs(p * (do[rows] @ vh.T - dd[rows][:, None]))
    bq = sm * U_BF16 * (w @ np.abs(kh))
    p = pmat(allq, cols)
    w = p * (np.abs(do) @ np.abs(vh[cols]).T) + np.abs(p * (do @ vh[cols].T - dd[:, None]))
    bk = sm * U_BF16 * (w.T @ np.abs(qh))
    bv = 2 * U_BF16 * (p.T @ np.abs(do))
    return bq, bk, bv


def head_backward_job(job):
    """Backward pass of one head at full size: (config name, shm names of q,
    k, v, dO, shape, head, query rows, keys, bn) -> (head, O [N, d] float32,
    LSE [N] float32, dQ[rows], dK[keys], dV[keys], and the first-order bounds
    of the library's bf16 roundings for those elements).  The oracle forward
    runs for every row (the keys' gradients need all of them)."""
    from oracle import backward as OB
    name, shm_names, shape, head, rows, cols, bn = job
    cfg = CONFIGS[name]
    blocks = [shared_memory.SharedMemory(name=n) for n in shm_names]
    try:
        q, k, v, do = (np.ndarray(shape, np.float32, buffer=b.buf)[0, head].copy() for b in blocks)
    finally:
        for b in blocks:
            b.close()
    qc, qs = OQ.fp8_block_quantize(q, cfg.blk)
    kc, ks = OQ.fp8_block_quantize(k, cfg.blk)
    vc, vs = OQ.fp8_channel_quantize(v)
    qo, ko = OA.Operand("fp8_block", qc, qs, cfg.blk), OA.Operand("fp8_block", kc, ks, cfg.blk)
    vo = OA.Operand("fp8_channel", vc, vs)
    n = q.shape[0]
    sm = 1.0 / np.sqrt(cfg.d)
    causal = cfg.mode == "causal"
    o, lse = OA.recipe_attention(qo, ko, vo, np.arange(n), sm_scale=sm, bn=bn, causal=causal,
                                 return_lse=True)
    qh, kh, vh = OB.dequantized(qo), OB.dequantized(ko), OB.dequantized(vo)
    do = do.astype(np.float64)
    grads = OB.backward_sampled(qh, kh, vh, o, do, lse, sm, rows, cols, causal=causal)
    bounds = sampled_bounds(qh, kh, vh, o, do, lse, sm, rows, cols, causal)
    return head, o, lse, grads, bounds
