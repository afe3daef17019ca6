"""Denoising-step-aware precision/sparsity schedule for sliding-tile FP8
attention ["FP8量化与稀疏性协同加速视频扩散模型", §3.2 (step-aware schedule)
and §5.2 (deployment advice on re-tiling cost)].

Over D denoising steps the page splits the run at t1 = alpha1 * D and
t2 = alpha2 * D (alpha1 = 0.2, alpha2 = 0.7 reported best): early steps
(t <= t1) use a coarse quantisation granularity and a sparse window, middle
steps (t1 < t <= t2), the most error-sensitive ones, a fine granularity and a
dense window, and late steps (t > t2) intermediate settings.  Steps are
counted from 1, as on the page.

The page does not print the granularity or window values of the three
phases (its tables did not survive); the defaults below are this library's
choice: the granularity g is the token block of the per-block FP8 Q/K scales
(384 = one (6, 8, 8) tile, 128, 64) and the window W is in tiles per axis
((3, 3, 3) sparse, (3, 5, 5) medium, every tile for dense).

Plans are built once per window on the host and cached, so a phase change
costs one plan upload (the page reports ~5% overhead for re-tiling and
advises re-planning every 50 steps; with cached plans no periodic re-planning
is needed).  Every step's attention runs in the library's kernels.
"""
from dataclasses import dataclass
from typing import Dict, Optional, Tuple

from . import binding as B
from .api import quantize_qkv

FULL = None                            # a window reaching every tile: dense attention


@dataclass(frozen=True)
class Phase:
    block_tokens: int                   # FP8 Q/K scale granularity g, in tokens
    window: Optional[Tuple[int, int, int]]   # sliding-tile window W in tiles per axis (FULL: dense)


COARSE = Phase(384, (3, 3, 3))
FINE = Phase(64, FULL)
INTERMEDIATE = Phase(128, (3, 5, 5))


class DenoisingSchedule:
    """Attention for step t of a D-step denoising run on one latent grid.

    grid / real_grid / tile: as for `binding.sta_plan` (grid a multiple of the
    tile, real_grid <= grid, tokens given in raster order of real_grid)."""

    def __init__(self, steps, grid, real_grid, tile, alpha1=0.2, alpha2=0.7,
                 early=COARSE, middle=FINE, late=INTERMEDIATE, device="cuda"):
        if steps < 1 or not (0.0 <= alpha1 <= alpha2 <= 1.0):
            raise ValueError("need steps >= 1 and 0 <= alpha1 <= alpha2 <= 1")
        self.steps = int(steps)
        self.t1, self.t2 = alpha1 * steps, alpha2 * steps
        self.grid, self.real_grid, self.tile = tuple(grid), tuple(real_grid), tuple(tile)
        self.early, self.middle, self.late = early, middle, late
        self.device = device
        self._plans: Dict[Tuple[int, int, int], object] = {}

    def phase(self, t):
        """Phase of step t (1 <= t <= steps)."""
        if not 1 <= t <= self.steps:
            raise ValueError("step %d outside 1..%d" % (t, self.steps))
        if t <= self.t1:
            return self.early
        if t <= self.t2:
            return self.middle
        return self.late

    def window_tiles(self, window):
        """A window in tiles per axis; FULL reaches every tile of the grid."""
        if window is FULL:
            return tuple(2 * (g // t) + 1 for g, t in zip(self.grid, self.tile))
        return tuple(int(w) for w in window)

    def plan(self, window):
        """The device plan of a window (built and uploaded once)."""
        key = self.window_tiles(window)
        if key not in self._plans:
            hp = B.sta_plan(self.grid, self.real_grid, self.tile, key)
            self._plans[key] = B.DevicePlan(hp, self.device)
        return self._plans[key]

    def attention(self, q, k, v, t, sm_scale=None):
        """q, k, v: [B, H, N_real, d] device tensors in raster order of
        real_grid; returns float32 [B, H, N_real, d]."""
        ph = self.phase(t)
        dp = self.plan(ph.window)
        qq, kq, vq = quantize_qkv(q, k, v, "fp8", ph.block_tokens, dp.perm, dp.n_tokens)
        return B.attention_sta(qq, kq, vq, dp, sm_scale=sm_scale)
