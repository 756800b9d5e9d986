"""Timestep policy of a sampling run, at the caller level.

RainFusion keeps the first 10% of the denoising timesteps dense (RainFusion
review page, "Assumptions & free parameters": dense timestep fraction,
Section 4.1) and predicts the sparse mask online at every later step
(RainFusion2.0 page, Abstract: online adaptive sparse attention).  This
module decides, per step, whether a layer's attention runs dense or sparse
and whether its mask is predicted afresh or reused from an earlier step of
the same layer (reuse is an option of this library, off by default:
refresh_every = 1 predicts every step as the pages describe).

Dense steps run the same kernels with sparsity 0, which keeps every tile and
is exact dense attention.
"""
import math
from dataclasses import dataclass

import torch

from . import rf


@dataclass(frozen=True)
class StepPolicy:
    n_steps: int
    dense_fraction: float = 0.10
    sparsity_pct: int = 80
    refresh_every: int = 1

    def __post_init__(self):
        if self.n_steps < 1:
            raise ValueError("n_steps must be >= 1")
        if not 0.0 <= self.dense_fraction <= 1.0:
            raise ValueError("dense_fraction must be in [0, 1]")
        if not 0 <= self.sparsity_pct <= 99:
            raise ValueError("sparsity_pct must be in [0, 99]")
        if self.refresh_every < 1:
            raise ValueError("refresh_every must be >= 1")

    @property
    def n_dense(self) -> int:
        """Leading dense steps: the fraction of the run, rounded up (a run of
        any length with a non-zero fraction starts with a dense step)."""
        return min(self.n_steps, math.ceil(self.dense_fraction * self.n_steps - 1e-9))

    def mode(self, step: int) -> str:
        """'dense', 'predict' (fresh mask) or 'reuse' (the layer's last mask)."""
        if not 0 <= step < self.n_steps:
            raise ValueError(f"step {step} outside [0, {self.n_steps})")
        if step < self.n_dense:
            return "dense"
        return "predict" if (step - self.n_dense) % self.refresh_every == 0 else "reuse"

    def schedule(self):
        return [self.mode(t) for t in range(self.n_steps)]


class SparseAttention:
    """One attention layer under a StepPolicy: owns the plan and the buffers
    of one layout and shape, and the mask of the last predicted step.

    __call__(q, k, v, step) takes raster tensors [B, H, N + n_text, d] and
    returns the attention output in the same order."""

    def __init__(self, layout, policy: StepPolicy, B, H, d, dtype, device):
        self.plan = rf.Plan(layout)
        self.policy = policy
        z = self.plan.sizes
        self.shape = (B, H, z["L"], d)
        Lt, nt, bs = z["Lt"], z["n_tiles"], z["bs"]
        mk = dict(dtype=dtype, device=device)
        # Q is read and O written in raster order by the attention call
        # itself, so only K and V are held permuted.
        self.kp = torch.empty(B, H, Lt, d, **mk)
        self.vt = torch.empty(B, H, nt, d, bs, **mk)
        self.qbar = torch.empty(B, H, z["nb"], d, dtype=torch.float32, device=device)
        self.kbar = torch.empty_like(self.qbar)
        s = policy.sparsity_pct
        self.kept = torch.empty(B, H, self.plan.keep(s)["nnz_per_head"],
                                dtype=torch.int32, device=device)
        self.dense_kept = torch.empty(B, H, self.plan.keep(0)["nnz_per_head"],
                                      dtype=torch.int32, device=device)
        self._have_mask = False
        self._have_dense = False

    def __call__(self, q, k, v, step, out=None):
        if tuple(q.shape) != self.shape:
            raise ValueError(f"expected {self.shape}, got {tuple(q.shape)}")
        mode = self.policy.mode(step)
        rf.permute_means(self.plan, q, xbar=self.qbar, means_only=True)
        rf.permute_means(self.plan, k, out=self.kp, xbar=self.kbar)
        rf.permute(self.plan, v, order=rf.TILES_T, out=self.vt)
        if mode == "dense":
            if not self._have_dense:       # s = 0 keeps every tile: a fixed list
                rf.predict_mask(self.plan, self.qbar, self.kbar, 0, kept=self.dense_kept)
                self._have_dense = True
            kept, s = self.dense_kept, 0
        else:
            if mode == "predict" or not self._have_mask:
                rf.predict_mask(self.plan, self.qbar, self.kbar,
                                self.policy.sparsity_pct, kept=self.kept)
                self._have_mask = True
            kept, s = self.kept, self.policy.sparsity_pct
        return rf.sparse_attn_raster(self.plan, q, self.kp, self.vt, kept, s, out=out)

    def close(self):
        self.plan.close()
