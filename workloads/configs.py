"""Workload shapes.  They stand in for the pages' workloads, which need model
weights and data that are not available: LLM prefill, and video-diffusion
latents of a 720p Wan2.1-class model (FPSAttention page, §1 and §2.2).

recipe  'fp8'   : Q/K FP8 E4M3 per `blk`-token block, V FP8 per channel
        'mxfp4' : Q/K E2M1 with one E8M0 scale per 32 channels, V FP8 per channel
        'mxfp4_pv': Q/K as 'mxfp4', V MXFP4 along tokens and P requantised to
                  MXFP4 per 32 keys (both products in FP4)
mode    'dense' | 'causal' | 'sta'
grid    (T, H, W) of the zero-padded latent grid, real_grid the unpadded one;
        tokens are given in raster order over real_grid.
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Config:
    name: str
    index: int                  # seed base = 1000 * index
    B: int
    H: int
    d: int
    recipe: str
    blk: int
    mode: str
    dtype: str                  # input dtype: 'f32' or 'bf16'
    outliers: bool
    N: Optional[int] = None     # token count for non-grid workloads
    grid: Optional[Tuple[int, int, int]] = None
    real_grid: Optional[Tuple[int, int, int]] = None
    tile: Optional[Tuple[int, int, int]] = None
    window: Optional[Tuple[int, int, int]] = None
    desc: str = ""

    @property
    def n_real(self):
        if self.real_grid is not None:
            t, h, w = self.real_grid
            return t * h * w
        return self.N

    @property
    def n_kernel(self):
        """Token count in the kernel's order (padded grid for grid workloads)."""
        if self.grid is not None:
            t, h, w = self.grid
            return t * h * w
        return self.N


CONFIGS = {
    "tiny_fp8": Config(
        "tiny_fp8", 1, B=1, H=2, d=64, recipe="fp8", blk=64, mode="dense",
        dtype="f32", outliers=False, N=256,
        desc="tiny dense FP8: B1 H2 N256 d64, fp32 N(0,1), 64-token blocks"),
    "llm_prefill_fp8_causal": Config(
        "llm_prefill_fp8_causal", 2, B=1, H=32, d=128, recipe="fp8", blk=128,
        mode="causal", dtype="bf16", outliers=True, N=8192,
        desc="LLM prefill FP8 causal: B1 H32 N8192 d128, bf16 + 4 outlier channels"),
    "dense_mxfp4_16k": Config(
        "dense_mxfp4_16k", 3, B=1, H=40, d=128, recipe="mxfp4", blk=32,
        mode="dense", dtype="bf16", outliers=True, N=16384,
        desc="dense MXFP4 Q/K: B1 H40 N16384 d128, bf16 + outliers, FP8 V"),
    "dense_mxfp4_pv_16k": Config(
        "dense_mxfp4_pv_16k", 3, B=1, H=40, d=128, recipe="mxfp4_pv", blk=32,
        mode="dense", dtype="bf16", outliers=True, N=16384,
        desc="dense FP4 attention: the 16K MXFP4 shape (same inputs) with V and P in MXFP4 too"),
    "dense_fp8_16k": Config(
        "dense_fp8_16k", 3, B=1, H=40, d=128, recipe="fp8", blk=128,
        mode="dense", dtype="bf16", outliers=True, N=16384,
        desc="dense FP8 twin of the 16K MXFP4 shape (same inputs), 128-token blocks"),
    "sta_46k_fp8": Config(
        "sta_46k_fp8", 4, B=1, H=24, d=128, recipe="fp8", blk=384, mode="sta",
        dtype="bf16", outliers=False, grid=(12, 48, 80), real_grid=(12, 48, 80),
        tile=(6, 8, 8), window=(3, 3, 3),
        desc="STA FP8: grid 12x48x80 (46080 tokens), tiles (6,8,8), window 3x3x3, H24"),
    "video_92k_fp8_dense": Config(
        "video_92k_fp8_dense", 5, B=1, H=40, d=128, recipe="fp8", blk=384,
        mode="dense", dtype="bf16", outliers=True, grid=(24, 48, 80),
        real_grid=(21, 45, 80), tile=(6, 8, 8), window=None,
        desc="video FP8 dense: grid 21x45x80 padded to 24x48x80 (92160), H40"),
    "video_92k_fp8_sta": Config(
        "video_92k_fp8_sta", 5, B=1, H=40, d=128, recipe="fp8", blk=384,
        mode="sta", dtype="bf16", outliers=True, grid=(24, 48, 80),
        real_grid=(21, 45, 80), tile=(6, 8, 8), window=(3, 5, 5),
        desc="video FP8 STA: same inputs, window 3x5x5"),
}


def get(name):
    return CONFIGS[name]
