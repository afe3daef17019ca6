"""Seeded input generation.

Seeds: 1000 * config.index + {Q: 0, K: 1, V: 2, outlier channels: 3,
gains: 4, row sample: 5}, drawn with numpy.random.default_rng.

Values are N(0, 1) float32.  Workloads with outliers scale 4 of the d channels
of Q and K per head by gains drawn from lognormal(0, 1.5), constant over
tokens; the 4 channel indices come from a seeded permutation per head and are
shared by Q and K of that head, and the gains are drawn independently per
(tensor, head, channel).  bf16 workloads are rounded to bfloat16 (nearest-even,
torch's CPU cast) after the gains.  Outputs are [B, H, N_real, d] in raster
token order, as float32 arrays holding the exact input values, plus the
bfloat16 torch tensors for bf16 workloads.
"""
import numpy as np


def _seed(cfg, k):
    return 1000 * cfg.index + k


def _normal(cfg, k, shape):
    rng = np.random.default_rng(_seed(cfg, k))
    return rng.standard_normal(size=shape, dtype=np.float32)


def make_inputs(cfg, heads=None, as_torch=False):
    """Returns dict(q, k, v) of float32 numpy arrays [B, H, N_real, d].

    heads: optional number of leading heads to keep (smaller test runs draw
    the full tensors' first heads only, so values match the full workload).
    as_torch: also return bf16/f32 torch CPU tensors under 'q_t', 'k_t', 'v_t'.
    """
    B, H, d, n = cfg.B, cfg.H, cfg.d, cfg.n_real
    shape = (B, H, n, d)
    q = _normal(cfg, 0, shape)
    k = _normal(cfg, 1, shape)
    v = _normal(cfg, 2, shape)
    if cfg.outliers:
        rng_c = np.random.default_rng(_seed(cfg, 3))
        chans = np.stack([rng_c.permutation(d)[:4] for _ in range(H)])      # [H, 4]
        rng_g = np.random.default_rng(_seed(cfg, 4))
        gq = rng_g.lognormal(0.0, 1.5, size=(H, 4)).astype(np.float32)
        gk = rng_g.lognormal(0.0, 1.5, size=(H, 4)).astype(np.float32)
        for h in range(H):
            q[:, h, :, chans[h]] *= gq[h][:, None, None]
            k[:, h, :, chans[h]] *= gk[h][:, None, None]
    out = {}
    if heads is not None:
        q, k, v = q[:, :heads].copy(), k[:, :heads].copy(), v[:, :heads].copy()
    if cfg.dtype == "bf16":
        import torch
        ts = [torch.from_numpy(a).to(torch.bfloat16) for a in (q, k, v)]
        q, k, v = (t.float().numpy() for t in ts)
        if as_torch:
            out.update(q_t=ts[0], k_t=ts[1], v_t=ts[2])
    elif as_torch:
        import torch
        out.update(q_t=torch.from_numpy(q), k_t=torch.from_numpy(k), v_t=torch.from_numpy(v))
    out.update(q=q, k=k, v=v)
    return out


def sample_rows(cfg, count=4096):
    """`count` distinct (head, raster token) pairs drawn uniformly over
    H x N_real (seed 1000 * index + 5).  Returns (heads, tokens) int64 arrays."""
    rng = np.random.default_rng(_seed(cfg, 5))
    total = cfg.H * cfg.n_real
    idx = rng.choice(total, size=min(count, total), replace=False)
    return idx // cfg.n_real, idx % cfg.n_real
