"""Parity of the HIP path (through the C-ABI) with the fp64 oracle.

Every case prints the case name before touching the GPU.  Shapes span several
tiles with ragged windows, partial text tiles, raster blocks, both block
sizes, both head dims and both precisions; the five synthetic workloads run
at full size with all heads checked for the permutation, means and masks and
sampled query tiles for attention (all tiles of two heads).
"""
import os
import sys

import numpy as np
import pytest
import torch

import parity
from image_diffusion_dits_amd import configs, inputs, rf
from oracle import rainfusion_oracle as orc

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def run_gpu(plan, q, k, v, s, logits=False):
    qp, qbar = rf.permute_means(plan, q)
    kp, kbar = rf.permute_means(plan, k)
    vt = rf.permute(plan, v, order=rf.TILES_T)
    kept, lg, dense = rf.predict_mask(plan, qbar, kbar, s, logits=True, dense=True)
    op, lse = rf.sparse_attn(plan, qp, kp, vt, kept, s, lse=True)
    o = rf.unpermute(plan, op)
    torch.cuda.synchronize()
    return dict(qp=qp, kp=kp, vt=vt, qbar=qbar, kbar=kbar, kept=kept,
                logits=lg, dense=dense, op=op, lse=lse, o=o)


def check_case(lay_dict, q, k, v, s, dtype, full_heads=None, sample_tiles=None,
               seed=0, gpu=None, check_lse=True, record=None):
    """Run the GPU path on q, k, v (device tensors) and check it against the
    oracle.  full_heads: heads whose every query tile is checked for
    attention (None = all); other heads get `sample_tiles` random tiles.
    check_lse=False skips the oracle's log-sum-exp (checked on other cases).
    record: optional dict that receives the point's statistics."""
    lay = parity.olayout(lay_dict)
    z = orc.sizes(lay)
    plan = rf.Plan(lay_dict)
    g = gpu if gpu is not None else run_gpu(plan, q, k, v, s)
    # The unfused entry points give the same bytes as the fused one.
    qp2, kp2 = rf.permute(plan, q), rf.permute(plan, k)
    qbar2, kbar2 = rf.block_means(plan, qp2, kp2)
    torch.cuda.synchronize()
    assert torch.equal(qp2, g["qp"]) and torch.equal(kp2, g["kp"])
    torch.testing.assert_close(qbar2, g["qbar"], rtol=1e-6, atol=1e-7)
    torch.testing.assert_close(kbar2, g["kbar"], rtol=1e-6, atol=1e-7)
    del qp2, kp2, qbar2, kbar2
    B, H = q.shape[:2]
    qb, kb, vb = parity.bits(q), parity.bits(k), parity.bits(v)
    qpb, kpb, vtb = parity.bits(g["qp"]), parity.bits(g["kp"]), parity.bits(g["vt"])
    opb, ob = parity.bits(g["op"]), parity.bits(g["o"])
    qbar, kbar = parity.values(g["qbar"]), parity.values(g["kbar"])
    rows = rf.kept_rows(plan, g["kept"], s)
    Lp = z["Lp"]
    op = parity.values(g["op"][:, :, :Lp])
    for name in ("qp", "kp", "op"):        # whole-tile pad rows after Lp
        assert torch.all(g[name][:, :, Lp:] == 0), name
    lse = parity.values(g["lse"]) if ("lse" in g and check_lse) else None
    if lse is not None:
        assert np.all(np.isneginf(lse[:, :, Lp:])), "LSE of whole-tile pad rows"
    dense = g["dense"].cpu().numpy() if "dense" in g else None
    valid = orc.slot_valid(lay)
    rng = np.random.default_rng(seed)
    stats = dict(swaps=0, max_abs=0.0, mean_abs=[])
    for b in range(B):
        for h in range(H):
            sl = (slice(b, b + 1), slice(h, h + 1))
            # permutation, bit-exact
            qpo = orc.permute(qb[sl], lay)
            assert np.array_equal(qpb[sl][..., :Lp, :], qpo), f"Q permutation b{b} h{h}"
            kpo = orc.permute(kb[sl], lay)
            assert np.array_equal(kpb[sl][..., :Lp, :], kpo), f"K permutation b{b} h{h}"
            vpo = orc.permute(vb[sl], lay)
            assert np.array_equal(vtb[sl], parity.tiles_t(vpo, lay)), \
                f"V permutation b{b} h{h}"
            assert np.array_equal(ob[sl], orc.unpermute(opb[sl][..., :Lp, :], lay)), \
                f"unpermutation b{b} h{h}"
            # means
            qv = parity.values(g["qp"][b:b + 1, h:h + 1, :Lp])
            kv = parity.values(g["kp"][b:b + 1, h:h + 1, :Lp])
            qbo, kbo = orc.block_means(qv, lay), orc.block_means(kv, lay)
            parity.check_means(qbar[sl], qbo)
            parity.check_means(kbar[sl], kbo)
            # mask
            kept_o, l = orc.predict_mask(qbo, kbo, lay, s)
            stats["swaps"] += parity.check_mask(rows[b][h], kept_o[0][0],
                                                l[0, 0], lay, s)
            if dense is not None:
                assert np.array_equal(dense[b, h], orc.kept_dense([[rows[b][h]]], lay)[0, 0]), \
                    f"dense mask b{b} h{h}"
            # attention, with the GPU's kept rows
            if full_heads is None or h in full_heads:
                tiles = range(z["n_tiles"])
            else:
                tiles = sorted(rng.choice(z["n_tiles"], size=min(sample_tiles, z["n_tiles"]),
                                          replace=False).tolist())
            vv = parity.values(v[b:b + 1, h:h + 1])
            want = orc.sparse_attention(qv, kv, orc.permute(vv, lay),
                                        [[rows[b][h]]], lay,
                                        query_tiles={(0, 0): tiles})
            mx, mn = parity.check_attention(op[b, h], want[0, 0], valid, dtype)
            if lse is not None:
                want_lse = orc.attention_lse(qv, kv, [[rows[b][h]]], lay,
                                             query_tiles={(0, 0): tiles})
                stats.setdefault("lse", []).append(
                    parity.check_lse(lse[b, h, :Lp], want_lse[0, 0], valid, dtype))
            stats["max_abs"] = max(stats["max_abs"], mx)
            stats["mean_abs"].append(mn)
    plan.close()
    if record is not None:
        record.update(swaps=stats["swaps"], max_abs=stats["max_abs"],
                      mean_abs=float(np.mean(stats["mean_abs"])),
                      lse_max_abs=max(stats.get("lse", [float("nan")])))
    say(f"  swaps={stats['swaps']} max_abs={stats['max_abs']:.3e} "
        f"mean_abs={np.mean(stats['mean_abs']):.3e} "
        f"lse_max_abs={max(stats.get('lse', [float('nan')])):.3e}")
    return g, stats


def _iid(shape, seed, dtype):
    return inputs.random_tensor(shape, seed, device="cuda", dtype=dtype)


EDGE = [
    # name, layout, B, H, d, dtype, sparsity
    ("ragged3d-text77", dict(T=3, H=13, W=21, wt=2, wh=8, ww=8, n_text=77,
                             permute=1, sink=1), 2, 3, 128, torch.bfloat16, 70),
    ("bs64-d64", dict(T=2, H=10, W=9, wt=1, wh=8, ww=8, n_text=0, permute=1,
                      sink=1), 1, 2, 64, torch.bfloat16, 50),
    ("raster-bs64-text10", dict(T=3, H=7, W=11, wt=1, wh=8, ww=8, n_text=10,
                                permute=0, sink=1), 1, 2, 128, torch.bfloat16, 60),
    ("bs128-d64", dict(T=2, H=9, W=17, wt=2, wh=8, ww=8, n_text=0, permute=1,
                       sink=0), 1, 2, 64, torch.bfloat16, 40),
    ("f32-d128-bs128", dict(T=2, H=9, W=17, wt=2, wh=8, ww=8, n_text=5,
                            permute=1, sink=1), 1, 2, 128, torch.float32, 40),
    ("f32-d64-bs64-raster", dict(T=2, H=5, W=30, wt=1, wh=8, ww=8, n_text=64,
                                 permute=0, sink=1), 1, 2, 64, torch.float32, 75),
    ("single-block", dict(T=1, H=8, W=8, wt=1, wh=8, ww=8, n_text=0, permute=1,
                          sink=0), 1, 1, 128, torch.bfloat16, 90),
    ("dense-s0", dict(T=3, H=13, W=21, wt=2, wh=8, ww=8, n_text=77, permute=1,
                      sink=1), 1, 2, 128, torch.bfloat16, 0),
    ("max-s99", dict(T=3, H=13, W=21, wt=2, wh=8, ww=8, n_text=0, permute=1,
                     sink=0), 1, 2, 128, torch.bfloat16, 99),
    ("frames-smaller-than-window", dict(T=4, H=3, W=5, wt=2, wh=8, ww=8, n_text=3,
                                        permute=1, sink=1), 1, 2, 128, torch.bfloat16, 50),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_edge_layouts(case):
    name, lay, B, H, d, dt, s = case
    say(f"[edge] {name} B={B} H={H} d={d} {dt} s={s}")
    L = rf.layout_sizes(lay)["L"]
    q = _iid((B, H, L, d), 11, dt)
    k = _iid((B, H, L, d), 12, dt)
    v = _iid((B, H, L, d), 13, dt)
    check_case(lay, q, k, v, s, "bf16" if dt == torch.bfloat16 else "f32")


def test_tiny_f32_workload():
    cfg = configs.TINY
    say(f"[workload] {cfg.name}")
    q, k, v = (t.cuda() for t in inputs.make_qkv(cfg, "cpu"))
    g, _ = check_case(cfg.layout, q, k, v, cfg.sparsity[0], "f32")
    # the optional logits equal the oracle's block scores
    lay = parity.olayout(cfg)
    Lp = orc.sizes(lay)["Lp"]
    qbo = orc.block_means(parity.values(g["qp"][:, :, :Lp]), lay)
    kbo = orc.block_means(parity.values(g["kp"][:, :, :Lp]), lay)
    l, _ = orc.block_scores(qbo, kbo)
    np.testing.assert_allclose(parity.values(g["logits"]), l, atol=1e-6)


def test_image_bf16_workload():
    cfg = configs.IMAGE
    say(f"[workload] {cfg.name}")
    q, k, v = (t.cuda() for t in inputs.make_qkv(cfg, "cpu"))
    check_case(cfg.layout, q, k, v, cfg.sparsity[0], "bf16")


def test_video720_workload():
    cfg = configs.VIDEO720
    say(f"[workload] {cfg.name} (all heads: permutation, means, mask; "
        f"attention: heads 0 and {cfg.H // 2} in full, 16 tiles elsewhere)")
    q, k, v = inputs.make_qkv(cfg, "cuda")
    check_case(cfg.layout, q, k, v, cfg.sparsity[0], "bf16",
               full_heads={0, cfg.H // 2}, sample_tiles=16)


def test_video_long_text_workload():
    cfg = configs.VIDEO_LONG
    say(f"[workload] {cfg.name}")
    q, k, v = inputs.make_qkv(cfg, "cuda")
    check_case(cfg.layout, q, k, v, cfg.sparsity[0], "bf16",
               full_heads={0, cfg.H // 2}, sample_tiles=16)


def _sweep_record(cfg, s, q, k, v, rec):
    """One JSON line per sweep point (input sha256s, swaps, errors, host),
    appended to $RF_PARITY_RECORD when that is set."""
    path = os.environ.get("RF_PARITY_RECORD")
    if not path:
        return
    import json
    line = dict(workload=cfg.name, sparsity_pct=s, permute=cfg.permute, heads=q.shape[1],
                inputs_sha256={n: inputs.sha256(t) for n, t in (("q", q), ("k", k),
                                                                 ("v", v))},
                nproc=os.cpu_count(), **rec)
    try:
        with open("/proc/cpuinfo") as f:
            line["cpu_model"] = next((l.split(":", 1)[1].strip() for l in f
                                      if l.startswith("model name")), "")
    except OSError:
        pass
    with open(path, "a") as f:
        f.write(json.dumps(line) + "\n")


@pytest.mark.parametrize("permute", [1, 0])
def test_sweep_workload(permute):
    """Every sweep point at the full 40 heads, in window and raster order:
    permutation, means and masks on every head, attention on 3 sampled query
    tiles of every head (the full acceptance is test_sweep_full_acceptance)."""
    cfg = configs.SWEEP if permute else configs.SWEEP_RASTER
    q, k, v = inputs.make_qkv(cfg, "cuda")
    for s in cfg.sparsity:
        say(f"[workload] {cfg.name} s={s} (40 heads; attention: 3 tiles each)")
        rec = {}
        check_case(cfg.layout, q, k, v, s, "bf16", full_heads=set(),
                   sample_tiles=3, seed=s, check_lse=False, record=rec)
        _sweep_record(cfg, s, q, k, v, dict(rec, check="sampled-3"))


@pytest.mark.slow
@pytest.mark.parametrize("permute", [1, 0])
def test_sweep_full_acceptance(permute):
    """The sweep's acceptance at the full 40 heads: masks on every head,
    attention on every query tile of heads 0 and 20 and on 16 sampled tiles
    of every other head, at every sparsity, in window and raster order.  The
    log-sum-exp is left to the other workload tests."""
    cfg = configs.SWEEP if permute else configs.SWEEP_RASTER
    q, k, v = inputs.make_qkv(cfg, "cuda")
    for s in cfg.sparsity:
        say(f"[acceptance] {cfg.name} s={s} (40 heads; attention: heads 0, 20 in full, "
            f"16 tiles elsewhere)")
        rec = {}
        check_case(cfg.layout, q, k, v, s, "bf16", full_heads={0, cfg.H // 2},
                   sample_tiles=16, seed=100 + s, check_lse=False, record=rec)
        _sweep_record(cfg, s, q, k, v, dict(rec, check="full-heads-0-20+16"))


@pytest.mark.parametrize("T,d", [(16, 128), (17, 64), (17, 128), (64, 64)],
                         ids=["nb1024-d128", "nb1088-d64", "nb1088-d128", "nb4096-d64"])
def test_mask_kernel_size_limits(T, d):
    """Frames of 64x64 tokens in 1x8x8 windows give 64 blocks per frame:
    nb = 1024 is the largest row of the MFMA selection kernel, 1088 and 4096
    take the kernel for longer rows (4096 its largest)."""
    lay = dict(T=T, H=64, W=64, wt=1, wh=8, ww=8, n_text=0, permute=1, sink=1)
    z = rf.layout_sizes(lay)
    assert z["nb"] == 64 * T
    say(f"[edge] nb={z['nb']} bs=64 d={d} bf16 s=90 (all blocks: permutation, means, mask; "
        f"attention: 24 sampled tiles)")
    q, k, v = (_iid((1, 1, z["L"], d), sd, torch.bfloat16) for sd in (21, 22, 23))
    check_case(lay, q, k, v, 90, "bf16", full_heads=set(), sample_tiles=24, seed=5)


def test_repeated_runs_are_bitwise_identical():
    cfg = configs.VIDEO720
    say("[determinism] three runs of the 720p case (8 heads)")
    q, k, v = inputs.make_qkv(cfg, "cuda", H=8)
    plan = rf.Plan(cfg.layout)
    outs = [run_gpu(plan, q, k, v, 80) for _ in range(3)]
    def host(t):
        return t.cpu().numpy() if t.dtype in (torch.int32, torch.uint8) else parity.bits(t)
    for key in ("qp", "kp", "vt", "qbar", "kbar", "kept", "dense", "op", "lse", "o"):
        a = host(outs[0][key])
        for other in outs[1:]:
            assert np.array_equal(a, host(other[key])), key
    # The sweep's 80% point is the 720p case itself.
    sw = configs.SWEEP
    q2, k2, v2 = inputs.make_qkv(sw, "cuda", H=8)
    assert torch.equal(q, q2) and torch.equal(k, k2) and torch.equal(v, v2)
    plan.close()


def test_out_of_range_kept_entries_are_skipped():
    """Tile ids outside [0, n_tiles) are ignored by the kernel's own bounds
    check: rows [0, -7, 2, 3] give the attention over tiles 0, 2 and 3."""
    lay = dict(T=2, H=8, W=16, wt=1, wh=8, ww=8, n_text=0, permute=1, sink=0)
    say("[robustness] kept lists with out-of-range ids")
    plan = rf.Plan(lay)
    z = plan.sizes
    olay = parity.olayout(lay)
    for dt in (torch.bfloat16, torch.float32):
        q, k, v = (_iid((1, 1, z["L"], 128), s, dt) for s in (1, 2, 3))
        qp, kp = rf.permute(plan, q), rf.permute(plan, k)
        vt = rf.permute(plan, v, order=rf.TILES_T)
        kept = torch.tensor([[[0, 1, 2, 3]]], dtype=torch.int32)
        kept = kept.repeat(1, 1, z["nb"]).cuda()      # s = 0: rows of nb = 4
        ref = rf.sparse_attn(plan, qp, kp, vt, kept, 0)
        bad = kept.clone()
        bad[0, 0, 1::4] = -7
        bad[0, 0, 5] = 1 << 30                          # row 1: huge id too
        bad[0, 0, 4] = 0
        got = rf.sparse_attn(plan, qp, kp, vt, bad, 0)
        torch.cuda.synchronize()
        rows = [[[np.array([0, 2, 3])] * z["n_tiles"]]]
        Lp = z["Lp"]
        want = orc.sparse_attention(parity.values(qp[:, :, :Lp]),
                                    parity.values(kp[:, :, :Lp]),
                                    orc.permute(parity.values(v), olay), rows, olay)
        parity.check_attention(parity.values(got)[0, 0, :Lp], want[0, 0],
                               orc.slot_valid(olay),
                               "bf16" if dt == torch.bfloat16 else "f32")
        assert not torch.equal(ref, got)
    plan.close()


def test_gpu_argument_errors():
    plan = rf.Plan(configs.TINY.layout)
    z = plan.sizes
    # rf_plan_info gives the sizes of rf_plan_sizes one by one.
    import ctypes
    n, n_p = ctypes.c_int64(), ctypes.c_int64()
    nb, bs, ns, nt = (ctypes.c_int32() for _ in range(4))
    assert rf.lib().rf_plan_info(plan.handle, ctypes.byref(n), ctypes.byref(n_p),
                                 ctypes.byref(nb), ctypes.byref(bs), ctypes.byref(ns),
                                 ctypes.byref(nt)) == 0
    assert (n.value, n_p.value, nb.value, bs.value, ns.value, nt.value) == \
        (z["N"], z["Np"], z["nb"], z["bs"], z["n_sink"], z["n_text_tiles"])
    # rf_keep_count on the plan agrees with rf_layout_keep on its layout.
    for cfg in (configs.TINY, configs.VIDEO_LONG, configs.SWEEP_RASTER):
        p2 = rf.Plan(cfg.layout)
        for s in (0, 50, 80, 95, 99):
            want = rf.keep_count(cfg.layout, s)
            assert p2.keep_count(s) == (want["k_eff"], want["nnz_per_head"])
        with pytest.raises(rf.RfError):
            p2.keep_count(100)
        p2.close()
    x = torch.zeros(1, 2, z["L"], 64, device="cuda")
    with pytest.raises(rf.RfError) as e:
        rf.permute(plan, x[..., :48].contiguous())       # d = 48
    assert e.value.status == rf.ERR_UNSUPPORTED
    L = rf.lib()
    xp = torch.zeros(1, 2, z["Lt"], 64, device="cuda")
    mis = x.view(-1)[1:].data_ptr()                     # 4-byte aligned only
    st = L.rf_permute(plan.handle, mis, xp.data_ptr(), 1, 2, 64, rf.F32,
                      rf.ROWS, None)
    assert st == rf.ERR_INVALID_ARG
    kept = torch.zeros(10, dtype=torch.int32, device="cuda")
    st = L.rf_sparse_attn(plan.handle, xp.data_ptr(), xp.data_ptr(), xp.data_ptr(),
                          kept.data_ptr(), 50, xp.data_ptr(), None, 1, 2, 64, -1.0,
                          rf.F32, None)
    assert st == rf.ERR_INVALID_ARG
    st = L.rf_predict_mask(plan.handle, xp.data_ptr(), xp.data_ptr(), 1, 2, 64, 100,
                           kept.data_ptr(), None, None, None)
    assert st == rf.ERR_INVALID_ARG
    # More than 4096 blocks per row is refused before any launch.
    big = rf.Plan(dict(T=65, H=64, W=64, wt=1, wh=8, ww=8, n_text=0, permute=1, sink=1))
    assert big.sizes["nb"] == 4160
    st = L.rf_predict_mask(big.handle, xp.data_ptr(), xp.data_ptr(), 1, 1, 64, 50,
                           kept.data_ptr(), None, None, None)
    assert st == rf.ERR_UNSUPPORTED and b"4096" in L.rf_last_error()
    big.close()
    # A misaligned LSE buffer is refused before any launch.
    st = L.rf_sparse_attn(plan.handle, xp.data_ptr(), xp.data_ptr(), xp.data_ptr(),
                          kept.data_ptr(), 50, xp.data_ptr(), xp.data_ptr() + 2, 1, 2,
                          64, 0.125, rf.F32, None)
    assert st == rf.ERR_INVALID_ARG and b"lse" in L.rf_last_error()
    plan.close()


PAD_LAYOUTS = [
    # partial tiles in t, h and w, text with a partial tile; bs = 128 and 64
    ("bs128-partial", dict(T=3, H=13, W=21, wt=2, wh=8, ww=8, n_text=77, permute=1,
                           sink=1), 128, 60),
    ("bs64-partial", dict(T=3, H=13, W=21, wt=1, wh=8, ww=8, n_text=77, permute=1,
                          sink=1), 64, 60),
    ("bs128-raster-tail", dict(T=3, H=7, W=11, wt=2, wh=8, ww=8, n_text=0, permute=0,
                               sink=1), 128, 50),
]


@pytest.mark.parametrize("case", PAD_LAYOUTS, ids=[c[0] for c in PAD_LAYOUTS])
def test_permute_writes_zero_pads_and_attention_matches_oracle(case):
    """rf_sparse_attn requires zero pad rows in kp and zero pad columns in
    vt, which rf_permute writes: output buffers pre-filled with finite
    garbage (3.0) hold exact zeros at every pad slot afterwards, and both
    the 128-slot and the 64-slot kernels then match the oracle.  The 64-slot
    kernel masks pad keys itself, so garbage written into the pads after the
    permutation leaves its result unchanged (documented behaviour; the
    128-slot kernels' result is unspecified then and is not tested)."""
    name, lay, bs, s = case
    say(f"[pads] {name} s={s}")
    plan = rf.Plan(lay)
    z = plan.sizes
    assert z["bs"] == bs
    olay = parity.olayout(lay)
    valid = orc.slot_valid(olay)
    valid_lt = np.concatenate([valid, np.zeros(z["Lt"] - z["Lp"], bool)])
    assert not valid_lt.all(), "the layout must have pad slots"
    B, H, d = 1, 2, 128
    q, k, v = (_iid((B, H, z["L"], d), sd, torch.bfloat16) for sd in (51, 52, 53))
    qp = rf.permute(plan, q)
    kp = torch.full((B, H, z["Lt"], d), 3.0, dtype=torch.bfloat16, device="cuda")
    vt = torch.full((B, H, z["n_tiles"], d, bs), 3.0, dtype=torch.bfloat16, device="cuda")
    rf.permute(plan, k, out=kp)
    rf.permute(plan, v, order=rf.TILES_T, out=vt)
    qbar, kbar = rf.block_means(plan, qp, kp)
    kept = rf.predict_mask(plan, qbar, kbar, s)
    op = rf.sparse_attn(plan, qp, kp, vt, kept, s)
    torch.cuda.synchronize()
    pad = torch.from_numpy(~valid_lt).cuda()
    assert torch.all(kp[:, :, pad] == 0), "pad rows of kp"
    vt_slots = vt.permute(0, 1, 2, 4, 3).reshape(B, H, z["Lt"], d)
    assert torch.all(vt_slots[:, :, pad] == 0), "pad columns of vt"
    rows = rf.kept_rows(plan, kept, s)
    Lp = z["Lp"]
    for h in range(H):
        sl = (slice(0, 1), slice(h, h + 1))
        want = orc.sparse_attention(parity.values(qp[sl][..., :Lp, :]),
                                    parity.values(kp[sl][..., :Lp, :]),
                                    orc.permute(parity.values(v[sl]), olay),
                                    [[rows[0][h]]], olay)
        parity.check_attention(parity.values(op[0, h, :Lp]), want[0, 0], valid, "bf16")
    if bs == 64:
        kp[:, :, pad] = 3.0
        vt_slots[:, :, pad] = 3.0
        vt2 = vt_slots.reshape(B, H, z["n_tiles"], bs, d).permute(0, 1, 2, 4, 3).contiguous()
        op2 = rf.sparse_attn(plan, qp, kp, vt2, kept, s)
        torch.cuda.synchronize()
        assert torch.equal(op2, op), "64-slot kernel with garbage pads"
    plan.close()
