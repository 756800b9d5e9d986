"""Synthetic workload table for the RainFusion2.0 sparse-attention hot path.

Each entry fixes a latent grid, a window, the head shape, the precision, the
target sparsity and the value model of the synthetic Q/K/V.  The shapes stand
in for the workloads the RainFusion2.0 page shows in its Figure 2 caption
(720p video with HunyuanVideo1.5 / Wan2.2 at 80% sparsity, 1024x1024 image
editing with Qwen-image-edit at 60% sparsity); no model weights are involved.

This module holds plain data only.  Nothing here computes any part of the
method: derived sizes (padded grid, block counts, keep counts) are computed
separately by the HIP library and by the CPU oracle.
"""
from dataclasses import dataclass, field, replace
from typing import Tuple


@dataclass(frozen=True)
class Config:
    name: str
    cid: int                 # seed base: generator seed = 1000 + cid
    B: int
    H: int                   # attention heads
    d: int                   # head dim
    dtype: str               # "bf16" or "f32"
    T: int                   # latent frames (1 for images)
    Hs: int                  # latent height in tokens
    Ws: int                  # latent width in tokens
    wt: int                  # window extent along frames
    wh: int                  # window extent along height
    ww: int                  # window extent along width
    n_text: int = 0          # text tokens appended after the video tokens
    sink: int = 0            # 1 = key blocks of frame 0 always kept
    permute: int = 1         # 1 = 3D window order, 0 = raster blocks
    sparsity: Tuple[int, ...] = (0,)
    values: str = "iid"      # "iid" N(0,1) or "grf" smooth field + noise
    ls: float = 4.0          # spatial correlation length (tokens)
    lt: float = 2.0          # temporal correlation length (frames); 0 = none

    @property
    def N(self) -> int:
        return self.T * self.Hs * self.Ws

    @property
    def layout(self) -> dict:
        """Fields of the C-ABI layout struct, by name."""
        return dict(T=self.T, H=self.Hs, W=self.Ws, wt=self.wt, wh=self.wh,
                    ww=self.ww, n_text=self.n_text, permute=self.permute,
                    sink=self.sink)


# 768 tokens, fp32, CPU-checkable in full.
TINY = Config("tiny-3x16x16-f32", 1, B=1, H=2, d=64, dtype="f32",
              T=3, Hs=16, Ws=16, wt=1, wh=8, ww=8, sink=1,
              sparsity=(50,), values="iid")

# One 64x64 latent frame (a 1024x1024 image after 16x patching), 2D windows.
IMAGE = Config("image-64x64", 2, B=1, H=24, d=128, dtype="bf16",
               T=1, Hs=64, Ws=64, wt=1, wh=8, ww=16, sink=0,
               sparsity=(60,), values="grf", ls=4.0, lt=0.0)

# 720p video latent: 21 frames of 45x80 tokens, padded to 22x48x80.
VIDEO720 = Config("video720-21x45x80", 3, B=1, H=40, d=128, dtype="bf16",
                  T=21, Hs=45, Ws=80, wt=2, wh=8, ww=8, sink=1,
                  sparsity=(80,), values="grf", ls=4.0, lt=2.0)

# Longer video with 512 text tokens that every row attends to.
VIDEO_LONG = Config("video-31x45x80+text512", 4, B=1, H=24, d=128,
                    dtype="bf16", T=31, Hs=45, Ws=80, wt=2, wh=8, ww=8,
                    n_text=512, sink=1, sparsity=(85,), values="grf",
                    ls=4.0, lt=2.0)

# Sparsity sweep on the 720p shape; seed of the 720p case so the tensors match.
SWEEP = replace(VIDEO720, name="video720-sweep", sparsity=(0, 50, 70, 80, 90, 95))
SWEEP_RASTER = replace(SWEEP, name="video720-sweep-raster", permute=0)

CONFIGS = {1: TINY, 2: IMAGE, 3: VIDEO720, 4: VIDEO_LONG, 5: SWEEP}


def get(cid: int) -> Config:
    return CONFIGS[cid]
