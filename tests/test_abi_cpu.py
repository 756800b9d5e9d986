"""The C-ABI library without a GPU: it loads, exports every declared symbol,
its host-side tables and keep counts agree with the oracle, and invalid
arguments come back as status codes before any device work."""
import ctypes
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from image_diffusion_dits_amd import configs, rf
from oracle import rainfusion_oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rf.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:rf_status|void|const char\*)\s+(rf_\w+)\s*\(",
                                 text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 13, names
    L = rf.lib()
    for n in names:
        assert hasattr(L, n), n


def _olay(lay):
    return orc.Layout(lay.T, lay.H, lay.W, lay.wt, lay.wh, lay.ww,
                      n_text=lay.n_text, permute=lay.permute, sink=lay.sink)


LAYOUTS = [configs.TINY.layout, configs.IMAGE.layout, configs.VIDEO720.layout,
           configs.VIDEO_LONG.layout, configs.SWEEP_RASTER.layout,
           dict(T=3, H=5, W=7, wt=2, wh=4, ww=8, n_text=37, permute=1, sink=1),
           dict(T=2, H=9, W=11, wt=1, wh=8, ww=8, n_text=0, permute=1, sink=1),
           dict(T=4, H=3, W=10, wt=1, wh=8, ww=8, n_text=70, permute=0, sink=1)]


@pytest.mark.parametrize("lay", LAYOUTS)
def test_host_tables_match_oracle(lay):
    L = rf.make_layout(**lay)
    o = _olay(L)
    z, oz = rf.layout_sizes(L), orc.sizes(o)
    for key in ("N", "Np", "L", "Lp", "bs", "nb", "n_text_tiles", "n_tiles"):
        assert z[key] == oz[key], key
    slot_src, tok_slot, count, sink = rf.layout_tables(L)
    want_slot = orc.slot_of_token(o)
    assert np.array_equal(tok_slot[:oz["N"]], want_slot)
    assert np.array_equal(tok_slot[oz["N"]:], np.arange(oz["Np"], oz["Lp"]))
    valid = orc.slot_valid(o)
    assert z["Lt"] == oz["n_tiles"] * oz["bs"] and len(slot_src) == z["Lt"]
    assert np.array_equal(slot_src[:oz["Lp"]] >= 0, valid)
    assert (slot_src[oz["Lp"]:] == -1).all()
    assert np.array_equal(slot_src[want_slot], np.arange(oz["N"]))
    assert np.array_equal(count[:oz["nb"]], orc.block_counts(o))
    want_sink = np.zeros(oz["nb"], np.uint8)
    want_sink[orc.sink_blocks(o)] = 1
    assert np.array_equal(sink, want_sink)
    assert z["n_sink"] == len(orc.sink_blocks(o))
    for s in (0, 50, 80, 95, 99):
        kc = rf.keep_count(L, s)
        k, keff = orc.keep_count(oz["nb"], s, z["n_sink"])
        assert (kc["k"], kc["k_eff"]) == (k, keff)
        assert kc["row_len_video"] == keff + oz["n_text_tiles"]
        assert kc["nnz_per_head"] == (oz["nb"] * kc["row_len_video"]
                                      + oz["n_text_tiles"] * oz["n_tiles"])


@settings(max_examples=40, deadline=None)
@given(T=st.integers(1, 6), H=st.integers(1, 20), W=st.integers(1, 20),
       win=st.sampled_from([(1, 8, 8), (2, 4, 8), (4, 4, 4), (2, 8, 8),
                            (1, 8, 16), (2, 2, 16), (1, 4, 16)]),
       n_text=st.integers(0, 300), permute=st.integers(0, 1),
       sink=st.integers(0, 1))
def test_host_tables_property(T, H, W, win, n_text, permute, sink):
    L = rf.make_layout(T, H, W, *win, n_text=n_text, permute=permute, sink=sink)
    o = _olay(L)
    slot_src, tok_slot, count, sink_t = rf.layout_tables(L)
    oz = orc.sizes(o)
    assert np.array_equal(tok_slot[:oz["N"]], orc.slot_of_token(o))
    assert np.array_equal(count[:oz["nb"]], orc.block_counts(o))
    assert np.array_equal(np.flatnonzero(sink_t), orc.sink_blocks(o))


def test_invalid_layouts_return_status():
    bad = [dict(T=0, H=4, W=4, wt=1, wh=8, ww=8),
           dict(T=1, H=4, W=4, wt=0, wh=8, ww=8),
           dict(T=1, H=4, W=4, wt=1, wh=8, ww=8, n_text=-1),
           dict(T=1, H=4, W=4, wt=1, wh=8, ww=8, permute=2),
           dict(T=1, H=4, W=4, wt=1, wh=8, ww=8, sink=3)]
    for lay in bad:
        with pytest.raises(rf.RfError) as e:
            rf.layout_sizes(lay)
        assert e.value.status == rf.ERR_INVALID_ARG
    with pytest.raises(rf.RfError) as e:
        rf.layout_sizes(dict(T=1, H=4, W=4, wt=1, wh=4, ww=4))   # bs = 16
    assert e.value.status == rf.ERR_UNSUPPORTED
    with pytest.raises(rf.RfError) as e:
        rf.keep_count(configs.TINY.layout, 100)
    assert e.value.status == rf.ERR_INVALID_ARG
    with pytest.raises(rf.RfError) as e:
        rf.keep_count(configs.TINY.layout, -1)
    assert e.value.status == rf.ERR_INVALID_ARG


def test_table_capacity_is_checked():
    L = rf.make_layout(**configs.TINY.layout)
    z = rf.layout_sizes(L)
    small = np.empty(z["Lt"] - 1, np.int32)
    ok = np.empty(max(z["Lt"], z["L"]), np.int32)
    sink = np.empty(z["nb"], np.uint8)
    st_ = rf.lib().rf_layout_tables(ctypes.byref(L), small.ctypes.data, small.size,
                                    ok.ctypes.data, ok.size, ok.ctypes.data, ok.size,
                                    sink.ctypes.data, sink.size)
    assert st_ == rf.ERR_BUFFER_TOO_SMALL


def test_gpu_entry_points_reject_bad_arguments_without_a_device():
    L = rf.lib()
    buf = ctypes.c_void_p(16)  # never dereferenced: checks fail first
    # Null plan.
    assert L.rf_permute(None, buf, buf, 1, 1, 64, rf.BF16, rf.ROWS, None) == rf.ERR_INVALID_ARG
    assert L.rf_unpermute(None, buf, buf, 1, 1, 64, rf.BF16, None) == rf.ERR_INVALID_ARG
    assert L.rf_block_means(None, buf, buf, buf, buf, 1, 1, 64, rf.BF16, None) == rf.ERR_INVALID_ARG
    assert L.rf_predict_mask(None, buf, buf, 1, 1, 64, 50, buf, None, None, None) == rf.ERR_INVALID_ARG
    assert L.rf_sparse_attn(None, buf, buf, buf, buf, 50, buf, None, 1, 1, 64, 0.125,
                            rf.BF16, None) == rf.ERR_INVALID_ARG
    assert L.rf_attention_recall(None, buf, buf, buf, 50, buf, 1, 1, 1, 64, 0.125,
                                 rf.BF16, buf, None) == rf.ERR_INVALID_ARG
    assert L.rf_sparse_attn_rows(None, buf, buf, buf, buf, 4, buf, None, 1, 1, 64, 0.125,
                                 rf.BF16, None) == rf.ERR_INVALID_ARG
    assert L.rf_attention_recall_rows(None, buf, buf, buf, 4, buf, 1, 1, 1, 64,
                                      0.125, rf.BF16, buf, None) == rf.ERR_INVALID_ARG
    assert L.rf_pattern_mask(None, buf, 1, 1, 2, 2, buf, 8, None) == rf.ERR_INVALID_ARG
    assert L.rf_arm_recall(None, buf, buf, 1, 4, rf.TEMPORAL, 2, 2, 1, 1, 64, 0.125,
                           rf.BF16, buf, None) == rf.ERR_INVALID_ARG
    assert L.rf_quantize_fp8(None, buf, rf.ROWS, buf, buf, 1, 1, 128, rf.BF16,
                             None) == rf.ERR_INVALID_ARG
    assert L.rf_sparse_attn_fp8(None, buf, buf, buf, buf, buf, buf, buf, 50, buf, None, 1, 1,
                                128, 0.125, None) == rf.ERR_INVALID_ARG
    assert L.rf_sparse_attn_fp8_rows(None, buf, buf, buf, buf, buf, buf, buf, 4, buf, None, 1,
                                     1, 128, 0.125, None) == rf.ERR_INVALID_ARG
    assert L.rf_sparse_attn_fp8_raster(None, buf, buf, buf, buf, buf, buf, buf, 50, buf, None,
                                       1, 1, 128, 0.125, None) == rf.ERR_INVALID_ARG
    assert L.rf_sparse_attn_raster(None, buf, buf, buf, buf, 50, buf, None, 1, 1, 64, 0.125,
                                   rf.BF16, None) == rf.ERR_INVALID_ARG
    assert b"null plan" in L.rf_last_error()
    # The classifier needs no plan: its sizes are checked first.
    assert L.rf_arm_classify(buf, 0, buf, 4, 1, 0.9, buf, None, None) == rf.ERR_INVALID_ARG
    assert L.rf_arm_classify(None, 4, buf, 4, 1, 0.9, buf, None, None) == rf.ERR_INVALID_ARG
    assert L.rf_plan_sizes(None, None) == rf.ERR_INVALID_ARG
    assert L.rf_plan_info(None, None, None, None, None, None, None) == rf.ERR_INVALID_ARG
    L.rf_plan_destroy(None)  # no-op
    assert L.rf_status_str(rf.ERR_HIP) == b"HIP runtime error"


def test_plan_create_without_device_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    with pytest.raises(rf.RfError) as e:
        rf.Plan(configs.TINY.layout)
    assert e.value.status == rf.ERR_HIP


@pytest.mark.parametrize("lay", LAYOUTS)
def test_tile_rank_matches_oracle(lay):
    np.testing.assert_array_equal(rf.tile_rank(lay), orc.tile_rank(_olay(rf._as_layout(lay))))


@pytest.mark.parametrize("lay", LAYOUTS)
@pytest.mark.parametrize("b,tau", [(0.0, 1), (0.25, 2), (0.1, 3), (1.0, 4)])
def test_pattern_row_width_holds_the_longest_oracle_row(lay, b, tau):
    """The width is the longest row of the three oracle masks."""
    olay = _olay(rf._as_layout(lay))
    w = orc.band_halfwidth(olay, b)
    longest = 0
    for p in (orc.SPATIAL, orc.TEMPORAL, orc.TEXTURAL):
        rows = orc.pattern_mask(olay, np.array([[p]]), w, tau)[0][0]
        longest = max(longest, max(len(r) for r in rows))
    assert rf.pattern_row_width(lay, w, tau) == longest


@pytest.mark.parametrize("lay", LAYOUTS)
@pytest.mark.parametrize("stride", [1, 3, 64])
def test_arm_sample_count_matches_oracle(lay, stride):
    olay = _olay(rf._as_layout(lay))
    for local in (True, False):
        assert rf.arm_sample_count(lay, local, stride) == len(orc.arm_samples(olay, local, stride))


def test_pattern_helpers_reject_bad_parameters():
    lay = rf._as_layout(configs.TINY.layout)
    w, n = ctypes.c_int32(), ctypes.c_int32()
    L = rf.lib()
    assert L.rf_pattern_row_width(ctypes.byref(lay), -1, 2, ctypes.byref(w)) == rf.ERR_INVALID_ARG
    assert L.rf_pattern_row_width(ctypes.byref(lay), 1, 0, ctypes.byref(w)) == rf.ERR_INVALID_ARG
    assert L.rf_arm_sample_count(ctypes.byref(lay), 1, 0, ctypes.byref(n)) == rf.ERR_INVALID_ARG
    small = np.empty(1, np.int32)
    assert L.rf_tile_rank(ctypes.byref(lay), small.ctypes.data, 1) == rf.ERR_BUFFER_TOO_SMALL


class _HostPlan:
    """The two members of rf.Plan that the row helpers read, from the host
    functions alone (creating a real plan needs a device)."""

    def __init__(self, lay):
        self.layout = lay
        self.sizes = rf.layout_sizes(lay)

    def keep(self, sparsity_pct):
        return rf.keep_count(self.layout, sparsity_pct)


@pytest.mark.parametrize("lay,s", [
    (dict(T=3, H=13, W=21, wt=2, wh=8, ww=8, n_text=77, permute=1, sink=1), 70),
    (dict(T=3, H=7, W=11, wt=1, wh=8, ww=8, n_text=10, permute=0, sink=1), 60),
    (dict(T=2, H=9, W=17, wt=2, wh=8, ww=8, n_text=0, permute=1, sink=0), 0),
])
def test_kept_rows_splits_the_flat_kept_list_into_the_oracle_rows(lay, s):
    """The flat [B, H, nnz] kept list (video rows of equal length, then text
    rows) splits back into the oracle's rows, head by head."""
    import torch
    olay = orc.Layout(**lay)
    B, H, d = 2, 2, 64
    rng = np.random.default_rng(7)
    qbar = rng.standard_normal((B, H, orc.sizes(olay)["nb"], d))
    kbar = rng.standard_normal((B, H, orc.sizes(olay)["nb"], d))
    kept_o, _ = orc.predict_mask(qbar, kbar, olay, s)
    flat = np.stack([np.stack([np.concatenate(kept_o[b][h]) for h in range(H)])
                     for b in range(B)]).astype(np.int32)
    plan = _HostPlan(lay)
    assert flat.shape[2] == plan.keep(s)["nnz_per_head"]
    rows = rf.kept_rows(plan, torch.from_numpy(flat), s)
    for b in range(B):
        for h in range(H):
            assert len(rows[b][h]) == len(kept_o[b][h])
            for got, want in zip(rows[b][h], kept_o[b][h]):
                assert np.array_equal(got, want)


def test_padded_rows_cut_each_row_at_its_first_negative_entry():
    import torch
    r = torch.tensor([[[[3, 5, 9, -1, -1],
                        [0, 1, 2, 3, 4],
                        [-1, 7, 8, -1, -1],
                        [6, -1, 2, -1, 1]]]], dtype=torch.int32)
    out = rf.padded_rows(r)
    want = [[3, 5, 9], [0, 1, 2, 3, 4], [], [6]]
    assert len(out) == 1 and len(out[0]) == 1
    for got, w in zip(out[0][0], want):
        assert got.tolist() == w
