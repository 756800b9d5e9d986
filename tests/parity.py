"""Comparison rules between the HIP path and the fp64 oracle.

  permutation   bit-exact (raw element bits)
  block means   |gpu - oracle| <= 2e-6 + 1e-6 |oracle|   (fp32 vs fp64)
  mask          per row, every block in the symmetric difference of the two
                kept sets must be borderline: |exp(l_j - l_theta) - 1| <= 1e-4
                where l_theta is the oracle's smallest kept non-sink logit;
                rows whose selection is sink-only must match exactly.
  attention     bf16: max-abs <= 2e-2 and mean-abs <= 5e-3 over valid rows;
                fp32: max-abs <= 1e-5.  The oracle row is computed with the
                GPU's kept list, so a legal borderline swap cannot fail it.
  log-sum-exp   bf16: |gpu - oracle| <= 1e-4 + 1e-6 |oracle|.  The kernels
                sum the fp32 weights (the bf16 rounding is applied only to
                the PV operand), so the error is that of fp32 logits from
                the same bf16 operands the oracle reads, a few ulp of the
                dot products of 128 products, and of the fp32 sum.
                fp32: <= 1e-5 + 1e-6 |oracle|.  Pad slots are -inf on both.
  dense mask    bit-exact against the kept rows it copies.
"""
import math

import numpy as np
import torch

from oracle import rainfusion_oracle as orc

BORDER = 1e-4
TOL = {"bf16": (2e-2, 5e-3), "f32": (1e-5, 1e-5)}
LSE_TOL = {"bf16": 1e-4, "f32": 1e-5}


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw element bits of a tensor as a host integer array."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy()
    raise TypeError(t.dtype)


def values(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


def olayout(cfg_or_dict) -> orc.Layout:
    d = cfg_or_dict.layout if hasattr(cfg_or_dict, "layout") else cfg_or_dict
    return orc.Layout(d["T"], d["H"], d["W"], d["wt"], d["wh"], d["ww"],
                      n_text=d["n_text"], permute=d["permute"], sink=d["sink"])


def tiles_t(xp_rows: np.ndarray, lay: orc.Layout) -> np.ndarray:
    """[B, H, Lp, d] rows -> [B, H, n_tiles, d, bs] tile-transposed order."""
    z = orc.sizes(lay)
    B, H, Lp, d = xp_rows.shape
    pad = z["n_tiles"] * z["bs"] - Lp
    x = np.concatenate([xp_rows, np.zeros((B, H, pad, d), xp_rows.dtype)], axis=2)
    return np.ascontiguousarray(
        x.reshape(B, H, z["n_tiles"], z["bs"], d).transpose(0, 1, 2, 4, 3))


def check_means(gpu: np.ndarray, want: np.ndarray):
    err = np.abs(gpu - want)
    bound = 2e-6 + 1e-6 * np.abs(want)
    bad = err > bound
    assert not bad.any(), f"{bad.sum()} means off, worst {err.max():.3e}"


def check_mask(gpu_rows, want_rows, l, lay: orc.Layout, sparsity):
    """Borderline acceptance of the GPU kept lists (per (b, h) list of rows
    in tile order).  Returns the number of borderline swaps."""
    z = orc.sizes(lay)
    nb = z["nb"]
    sinks = set(orc.sink_blocks(lay).tolist())
    _, k_eff = orc.keep_count(nb, sparsity, len(sinks))
    swaps = 0
    for i, (g, o) in enumerate(zip(gpu_rows, want_rows)):
        g = np.asarray(g)
        assert np.all(np.diff(g) > 0), f"row {i} not strictly ascending"
        if i >= nb:
            assert g.tolist() == o.tolist(), f"text row {i}"
            continue
        assert len(g) == k_eff + z["n_text_tiles"], f"row {i} length"
        assert g[k_eff:].tolist() == list(range(nb, z["n_tiles"]))
        gs, os_ = set(g[:k_eff].tolist()), set(o[:k_eff].tolist())
        assert sinks <= gs, f"row {i} misses a sink"
        diff = gs ^ os_
        if not diff:
            continue
        chosen = [j for j in os_ if j not in sinks]
        assert chosen, f"row {i}: sink-only selection differs"
        l_theta = min(l[i, j] for j in chosen)
        for j in diff:
            assert abs(math.expm1(l[i, j] - l_theta)) <= BORDER, \
                f"row {i}: block {j} not borderline ({l[i, j]} vs {l_theta})"
        swaps += len(diff) // 2
    return swaps


def check_attention(gpu_op: np.ndarray, want_op: np.ndarray, valid: np.ndarray,
                    dtype: str):
    """gpu_op, want_op: [Lp, d] of one head (want NaN where not computed);
    valid: bool [Lp] slot validity."""
    computed = ~np.isnan(want_op[:, 0])
    rows = computed & valid
    assert rows.any()
    err = np.abs(gpu_op[rows] - want_op[rows])
    max_abs, mean_abs = TOL[dtype]
    assert err.max() <= max_abs, f"max-abs {err.max():.3e}"
    assert err.mean() <= mean_abs, f"mean-abs {err.mean():.3e}"
    pad = computed & ~valid
    assert np.all(gpu_op[pad] == 0), "pad query rows must be zero"
    return float(err.max()), float(err.mean())


def check_lse(gpu_lse: np.ndarray, want_lse: np.ndarray, valid: np.ndarray,
              dtype: str, tol=None):
    """gpu_lse, want_lse: [Lp] of one head (want NaN where not computed);
    tol: optional per-slot bound replacing the dtype's."""
    computed = ~np.isnan(want_lse)
    rows = computed & valid
    assert rows.any()
    assert np.all(np.isfinite(gpu_lse[rows])), "finite LSE expected at valid slots"
    err = np.abs(gpu_lse[rows] - want_lse[rows])
    bound = (LSE_TOL[dtype] if tol is None else tol[rows]) + 1e-6 * np.abs(want_lse[rows])
    bad = err > bound
    assert not bad.any(), f"{bad.sum()} LSE values off, worst {err.max():.3e}"
    pad = computed & ~valid
    assert np.all(np.isneginf(gpu_lse[pad])), "pad query slots must be -inf"
    return float(err.max())
