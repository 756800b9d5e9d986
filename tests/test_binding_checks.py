"""The binding refuses tensors that do not fit the plan before it calls the
library (the kernels cannot check buffer sizes), and the host functions that
replaced arithmetic in the binding match the oracle.  CPU only: tensors are
host tensors with the device predicate patched, and every hot-path entry of
the library is replaced by one that fails the test if it is reached."""
import ctypes

import numpy as np
import pytest
import torch

from image_diffusion_dits_amd import configs, rf
from oracle import rainfusion_oracle as orc

LAYOUTS = [configs.TINY.layout, configs.VIDEO720.layout, configs.VIDEO_LONG.layout,
           configs.SWEEP_RASTER.layout,
           dict(T=3, H=13, W=21, wt=2, wh=8, ww=8, n_text=77, permute=1, sink=1)]


@pytest.mark.parametrize("lay", LAYOUTS)
@pytest.mark.parametrize("b", [0.0, 0.1, 0.25, 0.5, 1.0])
def test_band_tiles_matches_oracle(lay, b):
    olay = orc.Layout(**lay)
    assert rf.band_tiles_of(lay, b) == orc.band_halfwidth(olay, b)


def test_band_tiles_rejects_bad_bandwidth():
    lay = rf._as_layout(configs.TINY.layout)
    w = ctypes.c_int32()
    L = rf.lib()
    for b in (-0.1, 1.5, float("nan")):
        assert L.rf_band_tiles(ctypes.byref(lay), b, ctypes.byref(w)) == rf.ERR_INVALID_ARG
    assert L.rf_band_tiles(ctypes.byref(lay), 0.25, None) == rf.ERR_INVALID_ARG


def test_plan_keep_count_rejects_a_null_plan():
    k, n = ctypes.c_int32(), ctypes.c_int64()
    L = rf.lib()
    assert L.rf_keep_count(None, 50, ctypes.byref(k), ctypes.byref(n)) == rf.ERR_INVALID_ARG
    assert b"null plan" in L.rf_last_error()


class _HostPlan:
    """sizes, layout and keep() of a plan, from the host functions alone."""

    def __init__(self, lay):
        self.layout = rf._as_layout(lay)
        self.sizes = rf.layout_sizes(lay)
        self.handle = None

    def keep(self, s):
        return rf.keep_count(self.layout, s)


_HOT = {n for n in rf._SIGNATURES if n not in (
    "rf_layout_sizes", "rf_layout_tables", "rf_layout_keep", "rf_band_tiles",
    "rf_tile_rank", "rf_pattern_row_width", "rf_arm_sample_count")}


class _NoLaunch:
    """The real library for host helpers; any GPU entry point fails."""

    def __init__(self, real):
        self._real = real

    def __getattr__(self, name):
        if name in _HOT:
            raise AssertionError(f"{name} reached with a mismatched tensor")
        return getattr(self._real, name)


@pytest.fixture
def host(monkeypatch):
    real = rf.lib()
    monkeypatch.setattr(rf, "_on_device", lambda t: True)
    monkeypatch.setattr(rf, "lib", lambda: _NoLaunch(real))
    monkeypatch.setattr(rf, "_stream", lambda: None)
    return _HostPlan(dict(T=3, H=13, W=21, wt=2, wh=8, ww=8, n_text=77, permute=1,
                          sink=1))


def _z(plan):
    return plan.sizes


def _ops(plan, B=1, H=2, d=64, dt=torch.bfloat16):
    z = _z(plan)
    qp = torch.zeros(B, H, z["Lt"], d, dtype=dt)
    vt = torch.zeros(B, H, z["n_tiles"], d, z["bs"], dtype=dt)
    return qp, qp.clone(), vt


def _kept(plan, s, B=1, H=2):
    return torch.zeros(B, H, plan.keep(s)["nnz_per_head"], dtype=torch.int32)


def test_sparse_attn_refuses_mismatches(host):
    p = host
    qp, kp, vt = _ops(p)
    kept = _kept(p, 20)
    assert _kept(p, 50).numel() < kept.numel()
    cases = {
        "short kept (from a higher sparsity than the call's)": dict(kept=_kept(p, 50)),
        "kept int64": dict(kept=kept.long()),
        "kept not contiguous": dict(kept=torch.zeros(1, 2, 2 * kept.shape[2],
                                                     dtype=torch.int32)[..., ::2]),
        "qp tokens": dict(qp=qp[:, :, :-1].contiguous()),
        "kp dtype": dict(kp=kp.float()),
        "kp heads": dict(kp=torch.zeros(1, 1, *kp.shape[2:], dtype=kp.dtype)),
        "vt rows order": dict(vt=torch.zeros_like(qp)),
        "vt block": dict(vt=vt[..., :64].contiguous()),
        "out shape": dict(out=torch.zeros_like(qp)[:, :1].contiguous()),
    }
    # well-formed arguments pass the checks and reach the library
    with pytest.raises(AssertionError, match="rf_sparse_attn reached"):
        rf.sparse_attn(p, qp, kp, vt, kept, 20)
    for name, over in cases.items():
        a = dict(qp=qp, kp=kp, vt=vt, kept=kept)
        out = over.pop("out", None)
        a.update(over)
        with pytest.raises(ValueError):
            rf.sparse_attn(p, a["qp"], a["kp"], a["vt"], a["kept"], 20, out=out)
    # rows form: width outside [1, n_tiles], wrong tile count
    nt = _z(p)["n_tiles"]
    for rows in (torch.zeros(1, 2, nt, nt + 1, dtype=torch.int32),
                 torch.zeros(1, 2, nt - 1, 4, dtype=torch.int32),
                 torch.zeros(1, 2, nt, 4, dtype=torch.int16)):
        with pytest.raises(ValueError):
            rf.sparse_attn_rows(p, qp, kp, vt, rows)


def test_fp8_attention_refuses_mismatches(host):
    p = host
    z = _z(p)
    B, H, d = 1, 2, 128
    q8 = torch.zeros(B, H, z["Lt"], d, dtype=torch.uint8)
    qs = torch.ones(B, H, z["n_tiles"])
    v8 = torch.zeros(B, H, z["n_tiles"], d, z["bs"], dtype=torch.uint8)
    vs = torch.ones(B, H, d)
    kept = _kept(p, 20)
    good = dict(q8=q8, qs=qs, k8=q8.clone(), ks=qs.clone(), v8=v8, vs=vs, kept=kept)
    bad = {"q8 bf16": dict(q8=q8.to(torch.bfloat16)),
           "k scale per feature": dict(ks=vs),
           "v scale per tile": dict(vs=qs),
           "v8 rows": dict(v8=q8),
           "kept short": dict(kept=_kept(p, 50))}
    with pytest.raises(AssertionError, match="rf_sparse_attn_fp8 reached"):
        rf.sparse_attn_fp8(p, *[good[k] for k in ("q8", "qs", "k8", "ks", "v8", "vs",
                                                  "kept")], 20)
    for name, over in bad.items():
        a = dict(good, **over)
        with pytest.raises(ValueError):
            rf.sparse_attn_fp8(p, a["q8"], a["qs"], a["k8"], a["ks"], a["v8"], a["vs"],
                               a["kept"], 20)
    # The raster-output form: the same operand checks, and its output has
    # one row per token, not per slot.
    args = [good[k] for k in ("q8", "qs", "k8", "ks", "v8", "vs", "kept")]
    with pytest.raises(AssertionError, match="rf_sparse_attn_fp8_raster reached"):
        rf.sparse_attn_fp8_raster(p, *args, 20)
    for name, over in bad.items():
        a = dict(good, **over)
        with pytest.raises(ValueError):
            rf.sparse_attn_fp8_raster(p, a["q8"], a["qs"], a["k8"], a["ks"], a["v8"],
                                      a["vs"], a["kept"], 20)
    if z["Lt"] != z["L"]:
        with pytest.raises(ValueError):
            rf.sparse_attn_fp8_raster(p, *args, 20, out=torch.zeros(B, H, z["Lt"], d,
                                                                    dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        rf.sparse_attn_fp8_raster(p, *args, 20, out=torch.zeros(B, H, z["L"], d))


def test_other_entry_points_refuse_mismatches(host):
    p = host
    z = _z(p)
    B, H, d = 1, 2, 64
    x = torch.zeros(B, H, z["L"], d, dtype=torch.bfloat16)
    qp, kp, vt = _ops(p)
    bar = torch.zeros(B, H, z["nb"], d)
    with pytest.raises(ValueError):                       # raster tokens short
        rf.permute(p, x[:, :, :-1].contiguous())
    with pytest.raises(ValueError):                       # out of the rows order
        rf.permute(p, x, order=rf.TILES_T, out=qp)
    with pytest.raises(ValueError):                       # xbar bf16
        rf.permute_means(p, x, xbar=bar.to(torch.bfloat16))
    with pytest.raises(ValueError):                       # unpermute of raster rows
        rf.unpermute(p, x)
    with pytest.raises(ValueError):                       # kp of another layout
        rf.block_means(p, qp, kp[:, :, :-128].contiguous())
    with pytest.raises(ValueError):                       # kbar with nb - 1 blocks
        rf.predict_mask(p, bar, bar[:, :, 1:].contiguous(), 50)
    with pytest.raises(ValueError):                       # kept for 50% at 20%
        rf.predict_mask(p, bar, bar, 20, kept=_kept(p, 50))
    with pytest.raises(ValueError):                       # recall samples int64
        rf.attention_recall(p, qp, kp, _kept(p, 20), 20, torch.zeros(3, dtype=torch.int64))
    with pytest.raises(ValueError):                       # patterns of one head short
        rf.pattern_mask(p, torch.zeros(1, 2, dtype=torch.int64), 3)
    with pytest.raises(ValueError):                       # fp8 quantize: codes bf16
        rf.quantize_fp8(p, qp, out=torch.zeros_like(qp))
    with pytest.raises(ValueError):                       # fp8 permute: scale per tile for V
        rf.permute_fp8(p, x, order=rf.TILES_T, scale=torch.zeros(B, H, z["n_tiles"]))
    with pytest.raises(ValueError):                       # recalls of different heads
        rf.arm_classify(torch.zeros(1, 2, 5), torch.zeros(1, 3, 5))


def test_raster_attention_refuses_mismatches(host):
    p = host
    z = _z(p)
    B, H, d = 1, 2, 64
    q = torch.zeros(B, H, z["L"], d, dtype=torch.bfloat16)
    qp, kp, vt = _ops(p)
    kept = _kept(p, 20)
    with pytest.raises(AssertionError, match="rf_sparse_attn_raster reached"):
        rf.sparse_attn_raster(p, q, kp, vt, kept, 20)
    for bad in (dict(q=qp), dict(kp=q), dict(kept=_kept(p, 50)),
                dict(out=torch.zeros_like(qp))):
        a = dict(q=q, kp=kp, vt=vt, kept=kept, out=None)
        a.update(bad)
        with pytest.raises(ValueError):
            rf.sparse_attn_raster(p, a["q"], a["kp"], a["vt"], a["kept"], 20, out=a["out"])
    # means only: no rows tensor is needed, and a wrong xbar is still refused
    x = torch.zeros(B, H, z["L"], d, dtype=torch.bfloat16)
    with pytest.raises(AssertionError, match="rf_permute_means reached"):
        rf.permute_means(p, x, means_only=True)
    with pytest.raises(ValueError):
        rf.permute_means(p, x, means_only=True, xbar=torch.zeros(B, H, z["nb"] + 1, d))
