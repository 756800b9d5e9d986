"""Python binding of librf.so (ctypes).  Argument marshalling only: every step
of the path runs in the library's HIP kernels.  Output tensors are
allocated with torch (device memory plumbing) and handed to the library as
raw pointers together with torch's current HIP stream.

The library must have been built (``python -m image_diffusion_dits_amd.build``);
loading fails loudly when it is missing.  There is no fallback path.
"""
import ctypes
import math
import os

import numpy as np
import torch

# RF_LIB selects another build of the library (the debug builds of build.py).
LIB_PATH = os.environ.get("RF_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "librf.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_BUFFER_TOO_SMALL = range(5)
F32, BF16 = 0, 1
ROWS, TILES_T = 0, 1
SPATIAL, TEMPORAL, TEXTURAL = 0, 1, 2

_c_i32, _c_i64, _c_f32, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p


class Layout(ctypes.Structure):
    _fields_ = [(n, _c_i32) for n in
                ("T", "H", "W", "wt", "wh", "ww", "n_text", "permute", "sink")]


class Sizes(ctypes.Structure):
    _fields_ = [("N", _c_i64), ("Np", _c_i64), ("L", _c_i64), ("Lp", _c_i64),
                ("Lt", _c_i64), ("bs", _c_i32), ("nb", _c_i32), ("n_text_tiles", _c_i32),
                ("n_tiles", _c_i32), ("n_sink", _c_i32)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class Keep(ctypes.Structure):
    _fields_ = [("k", _c_i32), ("k_eff", _c_i32), ("row_len_video", _c_i32),
                ("row_len_text", _c_i32), ("nnz_per_head", _c_i64)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class RfError(RuntimeError):
    def __init__(self, status, fn, msg):
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


_P = ctypes.POINTER
_SIGNATURES = {
    "rf_layout_sizes": [_P(Layout), _P(Sizes)],
    "rf_layout_tables": [_P(Layout), _vp, _c_i64, _vp, _c_i64, _vp, _c_i64,
                         _vp, _c_i64],
    "rf_layout_keep": [_P(Layout), _c_i32, _P(Keep)],
    "rf_keep_count": [_vp, _c_i32, _P(_c_i32), _P(_c_i64)],
    "rf_band_tiles": [_P(Layout), ctypes.c_double, _P(_c_i32)],
    "rf_plan_create": [_P(Layout), _P(_vp)],
    "rf_plan_sizes": [_vp, _P(Sizes)],
    "rf_plan_info": [_vp, _P(_c_i64), _P(_c_i64), _P(_c_i32), _P(_c_i32), _P(_c_i32),
                     _P(_c_i32)],
    "rf_permute": [_vp, _vp, _vp, _c_i32, _c_i32, _c_i32, ctypes.c_int,
                   ctypes.c_int, _vp],
    "rf_permute_means": [_vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32,
                         ctypes.c_int, _vp],
    "rf_unpermute": [_vp, _vp, _vp, _c_i32, _c_i32, _c_i32, ctypes.c_int, _vp],
    "rf_block_means": [_vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32,
                       ctypes.c_int, _vp],
    "rf_predict_mask": [_vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _vp,
                        _vp, _vp, _vp],
    "rf_sparse_attn": [_vp, _vp, _vp, _vp, _vp, _c_i32, _vp, _vp, _c_i32,
                       _c_i32, _c_i32, _c_f32, ctypes.c_int, _vp],
    "rf_sparse_attn_raster": [_vp, _vp, _vp, _vp, _vp, _c_i32, _vp, _vp, _c_i32,
                              _c_i32, _c_i32, _c_f32, ctypes.c_int, _vp],
    "rf_attention_recall": [_vp, _vp, _vp, _vp, _c_i32, _vp, _c_i32, _c_i32,
                            _c_i32, _c_i32, _c_f32, ctypes.c_int, _vp, _vp],
    "rf_tile_rank": [_P(Layout), _vp, _c_i64],
    "rf_pattern_row_width": [_P(Layout), _c_i32, _c_i32, _P(_c_i32)],
    "rf_arm_sample_count": [_P(Layout), _c_i32, _c_i32, _P(_c_i32)],
    "rf_sparse_attn_rows": [_vp, _vp, _vp, _vp, _vp, _c_i32, _vp, _vp, _c_i32,
                            _c_i32, _c_i32, _c_f32, ctypes.c_int, _vp],
    "rf_attention_recall_rows": [_vp, _vp, _vp, _vp, _c_i32, _vp, _c_i32,
                                 _c_i32, _c_i32, _c_i32, _c_f32, ctypes.c_int,
                                 _vp, _vp],
    "rf_pattern_mask": [_vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _c_i32,
                        _vp],
    "rf_arm_recall": [_vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                      _c_i32, _c_i32, _c_i32, _c_f32, ctypes.c_int, _vp, _vp],
    "rf_arm_classify": [_vp, _c_i32, _vp, _c_i32, _c_i32, _c_f32, _vp, _vp,
                        _vp],
    "rf_quantize_fp8": [_vp, _vp, ctypes.c_int, _vp, _vp, _c_i32, _c_i32, _c_i32,
                        ctypes.c_int, _vp],
    "rf_permute_fp8": [_vp, _vp, ctypes.c_int, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32,
                       ctypes.c_int, _vp],
    "rf_sparse_attn_fp8": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i32, _vp,
                           _vp, _c_i32, _c_i32, _c_i32, _c_f32, _vp],
    "rf_sparse_attn_fp8_rows": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i32,
                                _vp, _vp, _c_i32, _c_i32, _c_i32, _c_f32, _vp],
    "rf_sparse_attn_fp8_raster": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i32, _vp,
                                  _vp, _c_i32, _c_i32, _c_i32, _c_f32, _vp],
}

_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m image_diffusion_dits_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGNATURES.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.rf_plan_destroy.argtypes = [_vp]
        L.rf_plan_destroy.restype = None
        L.rf_status_str.argtypes = [ctypes.c_int]
        L.rf_status_str.restype = ctypes.c_char_p
        L.rf_last_error.argtypes = []
        L.rf_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status, fn):
    if status != OK:
        raise RfError(status, fn, lib().rf_last_error().decode())


def make_layout(T, H, W, wt, wh, ww, n_text=0, permute=1, sink=0):
    return Layout(T, H, W, wt, wh, ww, n_text, permute, sink)


def _as_layout(lay):
    if isinstance(lay, Layout):
        return lay
    if isinstance(lay, dict):
        return make_layout(**lay)
    return make_layout(*lay)


# ---------------------------------------------------------------- host helpers

def layout_sizes(lay):
    out = Sizes()
    _check(lib().rf_layout_sizes(ctypes.byref(_as_layout(lay)), ctypes.byref(out)),
           "rf_layout_sizes")
    return out.as_dict()


def layout_tables(lay):
    """(slot_src, tok_slot, tile_count, is_sink) as numpy arrays."""
    lay = _as_layout(lay)
    z = layout_sizes(lay)
    slot_src = np.empty(z["Lt"], np.int32)
    tok_slot = np.empty(z["L"], np.int32)
    count = np.empty(z["n_tiles"], np.int32)
    sink = np.empty(z["nb"], np.uint8)
    _check(lib().rf_layout_tables(
        ctypes.byref(lay), slot_src.ctypes.data, slot_src.size,
        tok_slot.ctypes.data, tok_slot.size, count.ctypes.data, count.size,
        sink.ctypes.data, sink.size), "rf_layout_tables")
    return slot_src, tok_slot, count, sink


def keep_count(lay, sparsity_pct):
    """rf_layout_keep: the keep counts of a layout as a dict."""
    out = Keep()
    _check(lib().rf_layout_keep(ctypes.byref(_as_layout(lay)), int(sparsity_pct),
                                ctypes.byref(out)), "rf_layout_keep")
    return out.as_dict()


def band_tiles_of(lay, bandwidth):
    """rf_band_tiles: band half-width in video tiles for a bandwidth fraction."""
    w = _c_i32()
    _check(lib().rf_band_tiles(ctypes.byref(_as_layout(lay)), float(bandwidth),
                               ctypes.byref(w)), "rf_band_tiles")
    return w.value


def tile_rank(lay):
    """Position of each video tile in spatial-major order (numpy int32)."""
    lay = _as_layout(lay)
    out = np.empty(layout_sizes(lay)["nb"], np.int32)
    _check(lib().rf_tile_rank(ctypes.byref(lay), out.ctypes.data, out.size),
           "rf_tile_rank")
    return out


def pattern_row_width(lay, band, tau):
    w = _c_i32()
    _check(lib().rf_pattern_row_width(ctypes.byref(_as_layout(lay)), int(band),
                                      int(tau), ctypes.byref(w)),
           "rf_pattern_row_width")
    return w.value


def arm_sample_count(lay, local, stride):
    n = _c_i32()
    _check(lib().rf_arm_sample_count(ctypes.byref(_as_layout(lay)), int(bool(local)),
                                     int(stride), ctypes.byref(n)),
           "rf_arm_sample_count")
    return n.value


# ---------------------------------------------------------------- plan

class Plan:
    """Device index tables of one layout (rf_plan_create / rf_plan_destroy)."""

    def __init__(self, lay):
        self.layout = _as_layout(lay)
        h = _vp()
        _check(lib().rf_plan_create(ctypes.byref(self.layout), ctypes.byref(h)),
               "rf_plan_create")
        self._h = h
        s = Sizes()
        _check(lib().rf_plan_sizes(h, ctypes.byref(s)), "rf_plan_sizes")
        self.sizes = s.as_dict()

    @property
    def handle(self):
        return self._h

    def keep(self, sparsity_pct):
        return keep_count(self.layout, sparsity_pct)

    def keep_count(self, sparsity_pct):
        """rf_keep_count on the plan: (k_eff, nnz_per_head)."""
        k, n = _c_i32(), _c_i64()
        _check(lib().rf_keep_count(self._h, int(sparsity_pct), ctypes.byref(k),
                                   ctypes.byref(n)), "rf_keep_count")
        return k.value, n.value

    def close(self):
        if getattr(self, "_h", None):
            lib().rf_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------- hot path

def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream():
    return _vp(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return _vp(t.data_ptr())


def _on_device(t):
    return t.is_cuda


def _bhd(x):
    if x.dim() != 4 or not x.is_contiguous() or not _on_device(x):
        raise ValueError("expected a contiguous CUDA tensor [B, H, tokens, d]")
    return x.shape[0], x.shape[1], x.shape[3]


def _need(t, name, shape, dtypes, numel_only=False):
    """Checks one tensor handed to the library against what the plan and the
    call imply, before any launch: the kernels cannot check sizes and would
    read or write past a short buffer.  shape: the expected shape (or, with
    numel_only, the expected element count); dtypes: allowed dtypes."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a tensor")
    if not _on_device(t):
        raise ValueError(f"{name}: expected a CUDA tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected one of {list(dtypes)}")
    if numel_only:
        if t.numel() != shape:
            raise ValueError(f"{name}: {t.numel()} elements, expected {shape}")
    elif tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


_FLOAT = (torch.bfloat16, torch.float32)
_I32 = (torch.int32,)
_F32 = (torch.float32,)
_U8 = (torch.uint8,)


def _rows_operands(plan, qp, kp, name="qp"):
    """B, H, d of permuted RF_ROWS operands qp and kp, checked against the
    plan (both [B, H, Lt, d] of one float dtype)."""
    B, H, d = _bhd(qp)
    Lt = plan.sizes["Lt"]
    _need(qp, name, (B, H, Lt, d), _FLOAT)
    if kp is not None:
        _need(kp, "kp", (B, H, Lt, d), (qp.dtype,))
    return B, H, d


def _kept_operand(plan, kept, B, H, sparsity_pct):
    nnz = plan.keep(sparsity_pct)["nnz_per_head"]
    _need(kept, "kept", B * H * nnz, _I32, numel_only=True)


def _rows_operand(plan, rows, B, H):
    z = plan.sizes
    if rows.dim() != 4:
        raise ValueError("rows: expected [B, H, n_tiles, width]")
    w = rows.shape[-1]
    if not 1 <= w <= z["n_tiles"]:
        raise ValueError(f"rows: width {w} outside [1, {z['n_tiles']}]")
    _need(rows, "rows", (B, H, z["n_tiles"], w), _I32)


def _vt_operand(plan, vt, B, H, d, dtypes):
    z = plan.sizes
    _need(vt, "vt", (B, H, z["n_tiles"], d, z["bs"]), dtypes)


def permute(plan, x, order=ROWS, out=None):
    B, H, d = _bhd(x)
    z = plan.sizes
    if x.shape[2] != z["L"]:
        raise ValueError(f"x has {x.shape[2]} tokens, layout needs {z['L']}")
    shape = (B, H, z["Lt"], d) if order == ROWS else (B, H, z["n_tiles"], d, z["bs"])
    if out is None:
        out = torch.empty(shape, dtype=x.dtype, device=x.device)
    _need(x, "x", (B, H, z["L"], d), _FLOAT)
    _need(out, "out", shape, (x.dtype,))
    _check(lib().rf_permute(plan.handle, _ptr(x), _ptr(out), B, H, d,
                            _dtype_code(x), order, _stream()), "rf_permute")
    return out


def permute_means(plan, x, out=None, xbar=None, means_only=False):
    """Permuted rows of x (RF_ROWS) and the block means, in one pass.  With
    means_only=True no permuted rows are written and only xbar is returned."""
    B, H, d = _bhd(x)
    z = plan.sizes
    if x.shape[2] != z["L"]:
        raise ValueError(f"x has {x.shape[2]} tokens, layout needs {z['L']}")
    if out is None and not means_only:
        out = torch.empty(B, H, z["Lt"], d, dtype=x.dtype, device=x.device)
    if xbar is None:
        xbar = torch.empty(B, H, z["nb"], d, dtype=torch.float32, device=x.device)
    _need(x, "x", (B, H, z["L"], d), _FLOAT)
    if not means_only:
        _need(out, "out", (B, H, z["Lt"], d), (x.dtype,))
    _need(xbar, "xbar", (B, H, z["nb"], d), _F32)
    _check(lib().rf_permute_means(plan.handle, _ptr(x),
                                  None if means_only else _ptr(out), _ptr(xbar), B,
                                  H, d, _dtype_code(x), _stream()),
           "rf_permute_means")
    return xbar if means_only else (out, xbar)


def unpermute(plan, xp, out=None):
    B, H, d = _bhd(xp)
    z = plan.sizes
    if xp.shape[2] != z["Lt"]:
        raise ValueError(f"xp has {xp.shape[2]} slots, layout needs {z['Lt']}")
    if out is None:
        out = torch.empty(B, H, z["L"], d, dtype=xp.dtype, device=xp.device)
    _need(xp, "xp", (B, H, z["Lt"], d), _FLOAT)
    _need(out, "out", (B, H, z["L"], d), (xp.dtype,))
    _check(lib().rf_unpermute(plan.handle, _ptr(xp), _ptr(out), B, H, d,
                              _dtype_code(xp), _stream()), "rf_unpermute")
    return out


def block_means(plan, qp, kp, qbar=None, kbar=None):
    B, H, d = _rows_operands(plan, qp, kp)
    nb = plan.sizes["nb"]
    if qbar is None:
        qbar = torch.empty(B, H, nb, d, dtype=torch.float32, device=qp.device)
    if kbar is None:
        kbar = torch.empty_like(qbar)
    _need(qbar, "qbar", (B, H, nb, d), _F32)
    _need(kbar, "kbar", (B, H, nb, d), _F32)
    _check(lib().rf_block_means(plan.handle, _ptr(qp), _ptr(kp), _ptr(qbar),
                                _ptr(kbar), B, H, d, _dtype_code(qp), _stream()),
           "rf_block_means")
    return qbar, kbar


def predict_mask(plan, qbar, kbar, sparsity_pct, kept=None, logits=False,
                 dense=False):
    """Kept tiles [B, H, nnz_per_head]; with logits=True also the fp32 block
    logits [B, H, nb, nb], with dense=True also the uint8 tile mask
    [B, H, n_tiles, n_tiles], returned in that order after kept."""
    B, H, d = _bhd(qbar)
    nb = plan.sizes["nb"]
    _need(qbar, "qbar", (B, H, nb, d), _F32)
    _need(kbar, "kbar", (B, H, nb, d), _F32)
    kc = plan.keep(sparsity_pct)
    if kept is None:
        kept = torch.empty(B, H, kc["nnz_per_head"], dtype=torch.int32,
                           device=qbar.device)
    _kept_operand(plan, kept, B, H, sparsity_pct)
    lg = mask = None
    if logits:
        nb = plan.sizes["nb"]
        lg = torch.empty(B, H, nb, nb, dtype=torch.float32, device=qbar.device)
    if dense:
        nt = plan.sizes["n_tiles"]
        mask = torch.empty(B, H, nt, nt, dtype=torch.uint8, device=qbar.device)
    _check(lib().rf_predict_mask(plan.handle, _ptr(qbar), _ptr(kbar), B, H, d,
                                 int(sparsity_pct), _ptr(kept),
                                 _ptr(mask) if dense else None,
                                 _ptr(lg) if logits else None,
                                 _stream()), "rf_predict_mask")
    extra = ([lg] if logits else []) + ([mask] if dense else [])
    return (kept, *extra) if extra else kept


def _lse_out(want, qp):
    if not want:
        return None
    B, H, Lt = qp.shape[:3]
    return torch.empty(B, H, Lt, dtype=torch.float32, device=qp.device)


def sparse_attn(plan, qp, kp, vt, kept, sparsity_pct, scale=None, out=None,
                lse=False):
    """Op [B, H, Lt, d]; with lse=True also the fp32 log-sum-exp [B, H, Lt]."""
    B, H, d = _rows_operands(plan, qp, kp)
    _vt_operand(plan, vt, B, H, d, (qp.dtype,))
    _kept_operand(plan, kept, B, H, sparsity_pct)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(qp)
    _need(out, "out", qp.shape, (qp.dtype,))
    lo = _lse_out(lse, qp)
    _check(lib().rf_sparse_attn(plan.handle, _ptr(qp), _ptr(kp), _ptr(vt),
                                _ptr(kept), int(sparsity_pct), _ptr(out),
                                _ptr(lo) if lse else None, B, H,
                                d, float(scale), _dtype_code(qp), _stream()),
           "rf_sparse_attn")
    return (out, lo) if lse else out


def sparse_attn_raster(plan, q, kp, vt, kept, sparsity_pct, scale=None, out=None,
                       lse=False):
    """rf_sparse_attn_raster: raster q [B, H, L, d] in, raster O [B, H, L, d]
    out (and with lse=True the fp32 log-sum-exp [B, H, L], raster order)."""
    B, H, d = _bhd(q)
    z = plan.sizes
    _need(q, "q", (B, H, z["L"], d), _FLOAT)
    _need(kp, "kp", (B, H, z["Lt"], d), (q.dtype,))
    _vt_operand(plan, vt, B, H, d, (q.dtype,))
    _kept_operand(plan, kept, B, H, sparsity_pct)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.shape, (q.dtype,))
    lo = torch.empty(B, H, z["L"], dtype=torch.float32, device=q.device) if lse else None
    _check(lib().rf_sparse_attn_raster(plan.handle, _ptr(q), _ptr(kp), _ptr(vt),
                                       _ptr(kept), int(sparsity_pct), _ptr(out),
                                       _ptr(lo) if lse else None, B, H, d, float(scale),
                                       _dtype_code(q), _stream()),
           "rf_sparse_attn_raster")
    return (out, lo) if lse else out


def attention_recall(plan, qp, kp, kept, sparsity_pct, sample_tiles, scale=None,
                     out=None):
    """Share of each sampled query's dense softmax mass inside its kept tiles.

    sample_tiles: int32 tensor of query-tile ids on the device.  Returns fp32
    [B, H, n_sample, bs] (NaN at pad query slots)."""
    B, H, d = _rows_operands(plan, qp, kp)
    _kept_operand(plan, kept, B, H, sparsity_pct)
    n = sample_tiles.numel()
    _need(sample_tiles, "sample_tiles", n, _I32, numel_only=True)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, n, plan.sizes["bs"]), dtype=torch.float32,
                          device=qp.device)
    _need(out, "out", (B, H, n, plan.sizes["bs"]), _F32)
    _check(lib().rf_attention_recall(plan.handle, _ptr(qp), _ptr(kp), _ptr(kept),
                                     int(sparsity_pct), _ptr(sample_tiles), n, B, H,
                                     d, float(scale), _dtype_code(qp), _ptr(out),
                                     _stream()),
           "rf_attention_recall")
    return out


def sparse_attn_rows(plan, qp, kp, vt, rows, scale=None, out=None, lse=False):
    """rf_sparse_attn on padded kept rows: rows is int32 [B, H, n_tiles, width]."""
    B, H, d = _rows_operands(plan, qp, kp)
    _vt_operand(plan, vt, B, H, d, (qp.dtype,))
    _rows_operand(plan, rows, B, H)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(qp)
    _need(out, "out", qp.shape, (qp.dtype,))
    lo = _lse_out(lse, qp)
    _check(lib().rf_sparse_attn_rows(plan.handle, _ptr(qp), _ptr(kp), _ptr(vt),
                                     _ptr(rows), rows.shape[-1], _ptr(out),
                                     _ptr(lo) if lse else None, B, H,
                                     d, float(scale), _dtype_code(qp), _stream()),
           "rf_sparse_attn_rows")
    return (out, lo) if lse else out


def attention_recall_rows(plan, qp, kp, rows, sample_tiles, scale=None, out=None):
    """rf_attention_recall on padded kept rows [B, H, n_tiles, width]."""
    B, H, d = _rows_operands(plan, qp, kp)
    _rows_operand(plan, rows, B, H)
    n = sample_tiles.numel()
    _need(sample_tiles, "sample_tiles", n, _I32, numel_only=True)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, n, plan.sizes["bs"]), dtype=torch.float32,
                          device=qp.device)
    _need(out, "out", (B, H, n, plan.sizes["bs"]), _F32)
    _check(lib().rf_attention_recall_rows(plan.handle, _ptr(qp), _ptr(kp), _ptr(rows),
                                          rows.shape[-1], _ptr(sample_tiles), n, B,
                                          H, d, float(scale), _dtype_code(qp),
                                          _ptr(out), _stream()),
           "rf_attention_recall_rows")
    return out


def band_tiles(plan, bandwidth):
    """Band half-width in tiles of the plan's layout (rf_band_tiles)."""
    return band_tiles_of(plan.layout, bandwidth)


def pattern_mask(plan, head_pattern, band, tau=2, width=None, out=None):
    """Padded kept rows [B, H, n_tiles, width] of the v1 head patterns.
    head_pattern: int32 [B, H] on the device."""
    if head_pattern.dim() != 2:
        raise ValueError("head_pattern: expected [B, H]")
    B, H = head_pattern.shape
    _need(head_pattern, "head_pattern", (B, H), _I32)
    if width is None:
        width = pattern_row_width(plan.layout, band, tau)
    if out is None:
        out = torch.empty((B, H, plan.sizes["n_tiles"], width), dtype=torch.int32,
                          device=head_pattern.device)
    _rows_operand(plan, out, B, H)
    _check(lib().rf_pattern_mask(plan.handle, _ptr(head_pattern), B, H,
                                 int(band), int(tau), _ptr(out), out.shape[-1],
                                 _stream()), "rf_pattern_mask")
    return out


def arm_recall(plan, qp, kp, local, stride, pattern, band, tau=2, scale=None,
               out=None):
    """Per sampled query, the share of its mass over the sampled keys that
    the pattern keeps: fp32 [B, H, n]."""
    B, H, d = _rows_operands(plan, qp, kp)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    n = arm_sample_count(plan.layout, local, stride)
    if out is None:
        out = torch.empty((B, H, n), dtype=torch.float32, device=qp.device)
    _need(out, "out", (B, H, n), _F32)
    _check(lib().rf_arm_recall(plan.handle, _ptr(qp), _ptr(kp), int(bool(local)),
                               int(stride), int(pattern), int(band), int(tau), B, H,
                               d, float(scale), _dtype_code(qp), _ptr(out),
                               _stream()), "rf_arm_recall")
    return out


def arm_classify(local_recall, global_recall, alpha=0.9, pattern=None, mean=None):
    """Head patterns (int32 [B, H]) and mean recalls (fp32 [B, H, 2]) from
    the two recall samples [B, H, n_local] and [B, H, n_global]."""
    if local_recall.dim() != 3 or global_recall.dim() != 3:
        raise ValueError("recalls: expected [B, H, n]")
    B, H, nl = local_recall.shape
    ng = global_recall.shape[-1]
    _need(local_recall, "local_recall", (B, H, nl), _F32)
    _need(global_recall, "global_recall", (B, H, ng), _F32)
    if pattern is None:
        pattern = torch.empty((B, H), dtype=torch.int32, device=local_recall.device)
    if mean is None:
        mean = torch.empty((B, H, 2), dtype=torch.float32, device=local_recall.device)
    _need(pattern, "pattern", (B, H), _I32)
    _need(mean, "mean", (B, H, 2), _F32)
    _check(lib().rf_arm_classify(_ptr(local_recall), nl, _ptr(global_recall), ng,
                                 B * H, float(alpha), _ptr(pattern), _ptr(mean),
                                 _stream()), "rf_arm_classify")
    return pattern, mean


def arm_patterns(plan, qp, kp, band, local_stride, global_stride, alpha=0.9,
                 tau=2, scale=None):
    """The v1 classifier: recall of the temporal mask on the local sample and
    of the spatial mask on the global sample, then the decision.  Returns
    (head_pattern [B, H], mean recalls [B, H, 2])."""
    loc = arm_recall(plan, qp, kp, True, local_stride, TEMPORAL, band, tau, scale)
    glo = arm_recall(plan, qp, kp, False, global_stride, SPATIAL, band, tau, scale)
    return arm_classify(loc, glo, alpha)


def quantize_fp8(plan, xp, order=ROWS, out=None, scale=None):
    """e4m3 codes (uint8, same shape as xp) and power-of-two scales of a
    permuted bf16 tensor: per tile for RF_ROWS ([B, H, n_tiles]), per
    feature for RF_TILES_T ([B, H, d])."""
    z = plan.sizes
    if xp.dim() != (4 if order == ROWS else 5):
        raise ValueError("xp: expected [B, H, Lt, d] (RF_ROWS) or "
                         "[B, H, n_tiles, d, bs] (RF_TILES_T)")
    B, H = xp.shape[:2]
    d = xp.shape[3]
    shape = (B, H, z["Lt"], d) if order == ROWS else (B, H, z["n_tiles"], d, z["bs"])
    _need(xp, "xp", shape, _FLOAT)
    if out is None:
        out = torch.empty(xp.shape, dtype=torch.uint8, device=xp.device)
    n = z["n_tiles"] if order == ROWS else d
    if scale is None:
        scale = torch.empty((B, H, n), dtype=torch.float32, device=xp.device)
    _need(out, "out", shape, _U8)
    _need(scale, "scale", (B, H, n), _F32)
    _check(lib().rf_quantize_fp8(plan.handle, _ptr(xp), order, _ptr(out), _ptr(scale),
                                 B, H, d, _dtype_code(xp), _stream()), "rf_quantize_fp8")
    return out, scale


def permute_fp8(plan, x, order=ROWS, means=False, out=None, scale=None, xbar=None):
    """Permuted e4m3 codes and scales of a raster bf16 tensor in one pass
    (and, for RF_ROWS with means=True, the block means).  Returns
    (codes, scale) or (codes, scale, xbar)."""
    B, H, d = _bhd(x)
    z = plan.sizes
    if x.shape[2] != z["L"]:
        raise ValueError(f"x has {x.shape[2]} tokens, layout needs {z['L']}")
    shape = (B, H, z["Lt"], d) if order == ROWS else (B, H, z["n_tiles"], d, z["bs"])
    if out is None:
        out = torch.empty(shape, dtype=torch.uint8, device=x.device)
    n = z["n_tiles"] if order == ROWS else d
    if scale is None:
        scale = torch.empty((B, H, n), dtype=torch.float32, device=x.device)
    if means and xbar is None:
        xbar = torch.empty((B, H, z["nb"], d), dtype=torch.float32, device=x.device)
    _need(x, "x", (B, H, z["L"], d), _FLOAT)
    _need(out, "out", shape, _U8)
    _need(scale, "scale", (B, H, n), _F32)
    if means:
        _need(xbar, "xbar", (B, H, z["nb"], d), _F32)
    _check(lib().rf_permute_fp8(plan.handle, _ptr(x), order, _ptr(out), _ptr(scale),
                                _ptr(xbar) if means else None, B, H, d, _dtype_code(x),
                                _stream()), "rf_permute_fp8")
    return (out, scale, xbar) if means else (out, scale)


def _fp8_operands(plan, q8, qs, k8, ks, v8, vs):
    """B, H, d of the e4m3 attention operands, checked against the plan."""
    if q8.dim() != 4:
        raise ValueError("q8: expected [B, H, Lt, d]")
    z = plan.sizes
    B, H, _, d = q8.shape
    _need(q8, "q8", (B, H, z["Lt"], d), _U8)
    _need(k8, "k8", (B, H, z["Lt"], d), _U8)
    _need(qs, "q_scale", (B, H, z["n_tiles"]), _F32)
    _need(ks, "k_scale", (B, H, z["n_tiles"]), _F32)
    _need(v8, "v8", (B, H, z["n_tiles"], d, z["bs"]), _U8)
    _need(vs, "v_scale", (B, H, d), _F32)
    return B, H, d


def sparse_attn_fp8(plan, q8, qs, k8, ks, v8, vs, kept, sparsity_pct, scale=None,
                    out=None, lse=False):
    """Block-sparse attention on e4m3 operands; bf16 output [B, H, Lt, d]
    (and with lse=True the fp32 log-sum-exp [B, H, Lt])."""
    B, H, d = _fp8_operands(plan, q8, qs, k8, ks, v8, vs)
    _kept_operand(plan, kept, B, H, sparsity_pct)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty(q8.shape, dtype=torch.bfloat16, device=q8.device)
    _need(out, "out", q8.shape, (torch.bfloat16,))
    lo = _lse_out(lse, q8)
    _check(lib().rf_sparse_attn_fp8(plan.handle, _ptr(q8), _ptr(qs), _ptr(k8), _ptr(ks),
                                    _ptr(v8), _ptr(vs), _ptr(kept), int(sparsity_pct),
                                    _ptr(out), _ptr(lo) if lse else None, B, H, d,
                                    float(scale), _stream()),
           "rf_sparse_attn_fp8")
    return (out, lo) if lse else out


def sparse_attn_fp8_raster(plan, q8, qs, k8, ks, v8, vs, kept, sparsity_pct, scale=None,
                           out=None, lse=False):
    """rf_sparse_attn_fp8_raster: the FP8 attention with its bf16 output in
    raster order [B, H, L, d] (and with lse=True the fp32 log-sum-exp
    [B, H, L], raster order)."""
    B, H, d = _fp8_operands(plan, q8, qs, k8, ks, v8, vs)
    _kept_operand(plan, kept, B, H, sparsity_pct)
    L = plan.sizes["L"]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, L, d), dtype=torch.bfloat16, device=q8.device)
    _need(out, "out", (B, H, L, d), (torch.bfloat16,))
    lo = torch.empty(B, H, L, dtype=torch.float32, device=q8.device) if lse else None
    _check(lib().rf_sparse_attn_fp8_raster(plan.handle, _ptr(q8), _ptr(qs), _ptr(k8),
                                           _ptr(ks), _ptr(v8), _ptr(vs), _ptr(kept),
                                           int(sparsity_pct), _ptr(out),
                                           _ptr(lo) if lse else None, B, H, d,
                                           float(scale), _stream()),
           "rf_sparse_attn_fp8_raster")
    return (out, lo) if lse else out


def sparse_attn_fp8_rows(plan, q8, qs, k8, ks, v8, vs, rows, scale=None, out=None,
                         lse=False):
    B, H, d = _fp8_operands(plan, q8, qs, k8, ks, v8, vs)
    _rows_operand(plan, rows, B, H)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty(q8.shape, dtype=torch.bfloat16, device=q8.device)
    _need(out, "out", q8.shape, (torch.bfloat16,))
    lo = _lse_out(lse, q8)
    _check(lib().rf_sparse_attn_fp8_rows(plan.handle, _ptr(q8), _ptr(qs), _ptr(k8),
                                         _ptr(ks), _ptr(v8), _ptr(vs), _ptr(rows),
                                         rows.shape[-1], _ptr(out),
                                         _ptr(lo) if lse else None, B, H, d, float(scale),
                                         _stream()), "rf_sparse_attn_fp8_rows")
    return (out, lo) if lse else out


def sparse_attention_fp8(q, k, v, plan, sparsity_pct, scale=None, fused=True):
    """The whole path with the FP8 attention: permute into e4m3 codes and
    pool (one pass per tensor), predict, attend.  fused=True writes the
    output in raster order from the attention kernel; fused=False attends
    in slot order and unpermutes (the same bytes).  Returns (o, kept)."""
    q8, qs, qbar = permute_fp8(plan, q, means=True)
    k8, ks, kbar = permute_fp8(plan, k, means=True)
    v8, vs = permute_fp8(plan, v, order=TILES_T)
    kept = predict_mask(plan, qbar, kbar, sparsity_pct)
    if fused:
        o = sparse_attn_fp8_raster(plan, q8, qs, k8, ks, v8, vs, kept, sparsity_pct,
                                   scale=scale)
        return o, kept
    op = sparse_attn_fp8(plan, q8, qs, k8, ks, v8, vs, kept, sparsity_pct, scale=scale)
    return unpermute(plan, op), kept


def padded_rows(rows):
    """Per-row arrays of padded kept rows [B, H, n_tiles, width] (host copy),
    each cut at its first negative entry."""
    r = rows.detach().cpu().numpy()
    out = []
    for b in range(r.shape[0]):
        per_head = []
        for h in range(r.shape[1]):
            rr = []
            for row in r[b, h]:
                neg = np.flatnonzero(row < 0)
                rr.append(row[:neg[0]] if len(neg) else row)
            per_head.append(rr)
        out.append(per_head)
    return out


def kept_rows(plan, kept, sparsity_pct):
    """Split a flat kept list [B, H, nnz] (on the host) into per-row arrays."""
    kc = plan.keep(sparsity_pct)
    z = plan.sizes
    k = kept.detach().cpu().numpy()
    rows = []
    for b in range(k.shape[0]):
        per_head = []
        for h in range(k.shape[1]):
            flat = k[b, h]
            lv = kc["row_len_video"]
            r = [flat[i * lv:(i + 1) * lv] for i in range(z["nb"])]
            base = z["nb"] * lv
            lt = kc["row_len_text"]
            r += [flat[base + t * lt: base + (t + 1) * lt]
                  for t in range(z["n_text_tiles"])]
            per_head.append(r)
        rows.append(per_head)
    return rows


def sparse_attention(q, k, v, plan, sparsity_pct, scale=None, fused=True):
    """The whole path on raster tensors [B, H, N + n_text, d]: permute,
    pool, predict, attend, unpermute.  Returns (o, kept).  fused=True reads
    Q and writes O in raster order inside the attention call (the query
    means come from a means-only pass); fused=False permutes Q and
    unpermutes O in passes of their own.  Both give the same bytes."""
    kp, kbar = permute_means(plan, k)
    vt = permute(plan, v, order=TILES_T)
    if fused:
        qbar = permute_means(plan, q, means_only=True)
        kept = predict_mask(plan, qbar, kbar, sparsity_pct)
        return sparse_attn_raster(plan, q, kp, vt, kept, sparsity_pct, scale=scale), kept
    qp, qbar = permute_means(plan, q)
    kept = predict_mask(plan, qbar, kbar, sparsity_pct)
    op = sparse_attn(plan, qp, kp, vt, kept, sparsity_pct, scale=scale)
    return unpermute(plan, op), kept
