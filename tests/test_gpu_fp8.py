"""Parity of the FP8 (OCP e4m3) variant with the fp64 oracle, through the C-ABI.

Quantization is integer work and is compared bit for bit: every code (as its
e4m3 value) and every power-of-two scale equals the oracle's.

Attention: the oracle attends over the dequantized operands with exact
softmax weights; the kernel also rounds each weight to e4m3 (relative error
at most 2^-4 above 2^-6 times its reference weight, absolute at most 2^-10
below) and writes bf16.  To first order a relative weight error of at most
eps moves an output by at most eps / (1 - eps) * sum_j w_j |v_j - o| (w the
normalised weights), and absolute errors of 2^-10 on the weights below 2^-6
of the row maximum move it by at most 2^-10 * sum_small |v_j - o| /
sum_j 2^(l_j - l_max).  The per-element tolerance is that bound plus the
bf16 rounding of the output (2^-8 |o|) and 2e-3 for fp32 accumulation.
On inputs whose weights are exact powers of two inside the e4m3 range the
weights are not rounded at all, and the tolerance is the bf16 one
(max-abs 1e-2, mean-abs 2e-3).

Log-sum-exp: the kernel's sum is that of the rounded weights.  A weight at
least 2^-6 of the row maximum is off by at most eps of itself; a smaller one
by at most min(w, 2^-10) (it rounds to a subnormal step of 2^-9, or to 0),
so the sum's relative error is at most
delta = eps + sum_small min(w_j, 2^-10) / sum_j w_j (w_j = 2^(l_j - l_max))
and the LSE error at most -ln(1 - delta), plus 1e-4 for fp32 logits; -inf
at pad slots.
"""
import math
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


def _e4m3_values(codes_u8: torch.Tensor) -> np.ndarray:
    return codes_u8.cpu().view(torch.float8_e4m3fn).to(torch.float64).numpy()


def check_quant(plan, lay, xp_gpu, order, heads=None):
    """GPU codes and scales against the oracle, bit for bit."""
    x8, sc = rf.quantize_fp8(plan, xp_gpu, order=order)
    torch.cuda.synchronize()
    z = orc.sizes(lay)
    B, H = xp_gpu.shape[:2]
    got = _e4m3_values(x8)
    scales = sc.cpu().numpy().astype(np.float64)
    for b in range(B):
        for h in (range(H) if heads is None else heads):
            if order == rf.ROWS:
                xv = parity.values(xp_gpu[b:b + 1, h:h + 1, :z["Lp"]])
                want, ex = orc.quantize_tiles(xv, lay)
                np.testing.assert_array_equal(scales[b, h], np.exp2(ex[0, 0]))
                codes = want[0, 0] / np.repeat(np.exp2(ex[0, 0]), z["bs"])[:z["Lp"], None]
                np.testing.assert_array_equal(got[b, h, :z["Lp"]], codes)
                assert np.all(got[b, h, z["Lp"]:] == 0)
            else:
                # [tile][d][bs] -> rows [Lt][d] for the oracle
                xv = parity.values(xp_gpu[b:b + 1, h:h + 1]).transpose(0, 1, 2, 4, 3)
                xv = xv.reshape(1, 1, -1, xv.shape[-1])
                want, ex = orc.quantize_channels(xv)
                np.testing.assert_array_equal(scales[b, h], np.exp2(ex[0, 0]))
                g = got[b, h].transpose(0, 2, 1).reshape(-1, xv.shape[-1])
                np.testing.assert_array_equal(g, want[0, 0] / np.exp2(ex[0, 0])[None, :])
    return x8, sc


def fp8_bound(q8v, k8v, v8v, rows_bh, lay, tiles, scale):
    """Per-element tolerances of the header for the listed query tiles of one
    head: (dict tile -> [n_rows, d] for the output, dict tile -> [n_rows]
    for the log-sum-exp); NaN rows are pad queries."""
    z = orc.sizes(lay)
    bs, Lp = z["bs"], z["Lp"]
    valid = orc.slot_valid(lay)
    eps = 2.0 ** -4
    out, out_lse = {}, {}
    for i in tiles:
        rows = np.arange(i * bs, min((i + 1) * bs, Lp))
        tol = np.full((len(rows), q8v.shape[-1]), np.nan)
        tol_lse = np.full(len(rows), np.nan)
        qr = rows[valid[rows]]
        keys = np.concatenate([np.arange(j * bs, min((j + 1) * bs, Lp)) for j in rows_bh[i]])
        keys = keys[valid[keys]]
        s = (q8v[qr] @ k8v[keys].T) * scale / math.log(2.0)    # log2 units
        wrel = np.exp2(s - s.max(axis=1, keepdims=True))
        w = wrel / wrel.sum(axis=1, keepdims=True)
        o = w @ v8v[keys]
        vk = v8v[keys]
        t = np.empty_like(o)
        for a in range(0, len(qr), 8):                        # [8, key, d] at a time
            dev = np.abs(vk[None, :, :] - o[a:a + 8, None, :])
            small = (wrel[a:a + 8] < 2.0 ** -6)[:, :, None]
            t1 = eps / (1 - eps) * np.einsum("qk,qkd->qd", w[a:a + 8], dev)
            t2 = 2.0 ** -10 * (dev * small).sum(axis=1) / wrel[a:a + 8].sum(axis=1)[:, None]
            t[a:a + 8] = t1 + t2
        tol[valid[rows]] = t + 2.0 ** -8 * np.abs(o) + 2e-3
        out[i] = tol
        small = np.where(wrel < 2.0 ** -6, np.minimum(wrel, 2.0 ** -10), 0.0)
        delta = eps + small.sum(axis=1) / wrel.sum(axis=1)
        assert np.all(delta < 0.5), "LSE bound too loose to test"
        tol_lse[valid[rows]] = -np.log1p(-delta) + 1e-4
        out_lse[i] = tol_lse
    return out, out_lse


def run_fp8(plan, q, k, v, s):
    qp, qbar = rf.permute_means(plan, q)
    kp, kbar = rf.permute_means(plan, k)
    vt = rf.permute(plan, v, order=rf.TILES_T)
    kept = rf.predict_mask(plan, qbar, kbar, s)
    q8, qs = rf.quantize_fp8(plan, qp)
    k8, ks = rf.quantize_fp8(plan, kp)
    v8, vs = rf.quantize_fp8(plan, vt, order=rf.TILES_T)
    op, lse = rf.sparse_attn_fp8(plan, q8, qs, k8, ks, v8, vs, kept, s, lse=True)
    torch.cuda.synchronize()
    return dict(qp=qp, kp=kp, vt=vt, kept=kept, op=op, lse=lse)


def check_fp8_attention(lay_dict, q, k, v, s, heads=None, sample_tiles=None, seed=0,
                        scale=None):
    """Quantization bit-exact, then attention within the per-element bound
    on every query tile (sample_tiles None) or a random subset."""
    lay = parity.olayout(lay_dict)
    z = orc.sizes(lay)
    plan = rf.Plan(lay_dict)
    g = run_fp8(plan, q, k, v, s)
    check_quant(plan, lay, g["qp"], rf.ROWS, heads)
    check_quant(plan, lay, g["kp"], rf.ROWS, heads)
    check_quant(plan, lay, g["vt"], rf.TILES_T, heads)
    rows = rf.kept_rows(plan, g["kept"], s)
    Lp = z["Lp"]
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    op = parity.values(g["op"])
    valid = orc.slot_valid(lay)
    rng = np.random.default_rng(seed)
    B, H = q.shape[:2]
    worst, ratio, errs, lse_worst = 0.0, 0.0, [], 0.0
    lse = parity.values(g["lse"])
    assert np.all(np.isneginf(lse[:, :, Lp:])), "LSE of whole-tile pad rows"
    for b in range(B):
        for h in (range(H) if heads is None else heads):
            tiles = (list(range(z["n_tiles"])) if sample_tiles is None else
                     sorted(rng.choice(z["n_tiles"], size=min(sample_tiles, z["n_tiles"]),
                                       replace=False).tolist()))
            qv = parity.values(g["qp"][b:b + 1, h:h + 1, :Lp])
            kv = parity.values(g["kp"][b:b + 1, h:h + 1, :Lp])
            vv = orc.permute(parity.values(v[b:b + 1, h:h + 1]), lay)
            want = orc.sparse_attention_fp8(qv, kv, vv, [[rows[b][h]]], lay, scale=scale,
                                            query_tiles={(0, 0): tiles})[0, 0]
            q8v, _ = orc.quantize_tiles(qv, lay)
            k8v, _ = orc.quantize_tiles(kv, lay)
            v8v, _ = orc.quantize_channels(vv)
            tol, tol_lse = fp8_bound(q8v[0, 0], k8v[0, 0], v8v[0, 0], rows[b][h], lay,
                                     tiles, scale)
            want_lse = orc.attention_lse(q8v, k8v, [[rows[b][h]]], lay, scale=scale,
                                         query_tiles={(0, 0): tiles})[0, 0]
            tl = np.full(Lp, np.nan)
            for i in tiles:
                tl[i * z["bs"]:min((i + 1) * z["bs"], Lp)] = tol_lse[i]
            lse_worst = max(lse_worst, parity.check_lse(lse[b, h, :Lp], want_lse, valid,
                                                        "bf16", tol=tl))
            for i in tiles:
                sl = slice(i * z["bs"], min((i + 1) * z["bs"], Lp))
                gi, wi = op[b, h, sl], want[sl]
                vr = valid[sl]
                assert np.all(gi[~vr] == 0), f"pad rows b{b} h{h} tile {i}"
                err = np.abs(gi[vr] - wi[vr])
                bad = err > tol[i][vr]
                assert not bad.any(), (f"b{b} h{h} tile {i}: {bad.sum()} elements beyond the "
                                       f"bound, worst err {err.max():.3e}")
                worst = max(worst, float(err.max()))
                ratio = max(ratio, float((err / tol[i][vr]).max()))
                errs.append(err.ravel())
    e = np.concatenate(errs)
    say(f"  fp8 attention max_abs={worst:.3e} mean_abs={e.mean():.3e} "
        f"max err/bound={ratio:.3f} lse max_abs={lse_worst:.3e}")
    plan.close()
    return g, e


EDGE = [
    ("ragged3d-text77", dict(T=3, H=13, W=21, wt=2, wh=8, ww=8, n_text=77, permute=1,
                             sink=1), 2, 3, 70),
    ("raster-text40", dict(T=2, H=9, W=17, wt=2, wh=8, ww=8, n_text=40, permute=0,
                           sink=1), 1, 2, 40),
    ("single-tile", dict(T=2, H=8, W=8, wt=2, wh=8, ww=8, n_text=0, permute=1,
                         sink=0), 1, 2, 90),
    ("dense-s0", dict(T=3, H=13, W=21, wt=2, wh=8, ww=8, n_text=77, permute=1,
                      sink=1), 1, 2, 0),
]


def _iid(shape, seed):
    return inputs.random_tensor(shape, seed, device="cuda", dtype=torch.bfloat16)


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_fp8_edge_layouts(case):
    name, lay, B, H, s = case
    say(f"[fp8 edge] {name} B={B} H={H} s={s}")
    L = rf.layout_sizes(lay)["L"]
    q, k, v = (_iid((B, H, L, 128), sd) for sd in (61, 62, 63))
    check_fp8_attention(lay, q, k, v, s)


def test_fp8_exact_weights():
    """Q, K in {-1, 0, 1} on four features and scale ln 2: logits in log2
    units are integers in [-4, 4], the weights exact powers of two, so the
    kernel rounds nothing but the output; every permutation, mask, scale
    and key/value pairing error shows at bf16 tolerance."""
    lay = dict(T=3, H=13, W=21, wt=2, wh=8, ww=8, n_text=77, permute=1, sink=1)
    say("[fp8] exact power-of-two weights")
    z = rf.layout_sizes(lay)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(67)
    q = torch.zeros((1, 3, z["L"], 128), device="cuda")
    k = torch.zeros_like(q)
    q[..., :4] = torch.randint(-1, 2, (1, 3, z["L"], 4), generator=gen, device="cuda").float()
    k[..., :4] = torch.randint(-1, 2, (1, 3, z["L"], 4), generator=gen, device="cuda").float()
    v = _iid((1, 3, z["L"], 128), 69)
    plan = rf.Plan(lay)
    olay = parity.olayout(lay)
    # a 1 in every tile, so that every tile's amax is 1 and its scale 2^-8
    slot_src = rf.layout_tables(lay)[0]
    for t in range(z["n_tiles"]):
        src = slot_src[t * z["bs"]:(t + 1) * z["bs"]]
        tok = int(src[src >= 0][0])
        q[:, :, tok, 0] = 1.0
        k[:, :, tok, 0] = 1.0
    q, k = q.bfloat16(), k.bfloat16()
    s = 70
    g = run_fp8(plan, q, k, v, s)
    rows = rf.kept_rows(plan, g["kept"], s)
    Lp = z["Lp"]
    valid = orc.slot_valid(olay)
    # the attention again with scale ln 2 (integer logits in log2 units)
    q8, qs = rf.quantize_fp8(plan, g["qp"])
    k8, ks = rf.quantize_fp8(plan, g["kp"])
    v8, vs = rf.quantize_fp8(plan, g["vt"], order=rf.TILES_T)
    assert torch.all(qs == 2.0 ** -8) and torch.all(ks == 2.0 ** -8)
    op2 = rf.sparse_attn_fp8(plan, q8, qs, k8, ks, v8, vs, g["kept"], s, scale=math.log(2.0))
    torch.cuda.synchronize()
    op2 = parity.values(op2)
    for h in range(3):
        want = orc.sparse_attention_fp8(parity.values(g["qp"][:, h:h + 1, :Lp]),
                                        parity.values(g["kp"][:, h:h + 1, :Lp]),
                                        orc.permute(parity.values(v[:, h:h + 1]), olay),
                                        [[rows[0][h]]], olay, scale=math.log(2.0))
        err = np.abs(op2[0, h, :Lp][valid] - want[0, 0][valid])
        say(f"  exact-weight head {h}: max_abs={err.max():.3e} mean_abs={err.mean():.3e}")
        assert err.max() <= 1e-2 and err.mean() <= 2e-3
    plan.close()


def test_fp8_image_workload():
    cfg = configs.IMAGE
    say(f"[fp8 workload] {cfg.name} (4 heads, all tiles)")
    q, k, v = inputs.make_qkv(cfg, "cuda", H=4)
    check_fp8_attention(cfg.layout, q, k, v, cfg.sparsity[0])


def test_fp8_video720_workload():
    cfg = configs.VIDEO720
    say(f"[fp8 workload] {cfg.name} (2 heads, 12 sampled tiles)")
    q, k, v = inputs.make_qkv(cfg, "cuda", H=2)
    check_fp8_attention(cfg.layout, q, k, v, cfg.sparsity[0], sample_tiles=12)


def test_fp8_above_1024_blocks():
    """nb = 1088 (34 frames of 64x64 tokens, 2x8x8 windows): quantization
    bit-exact on every tile, attention and LSE on 8 sampled tiles."""
    lay = dict(T=34, H=64, W=64, wt=2, wh=8, ww=8, n_text=0, permute=1, sink=1)
    z = rf.layout_sizes(lay)
    assert z["nb"] == 1088
    say(f"[fp8 edge] nb={z['nb']} (1 head, 8 sampled tiles)")
    q, k, v = (_iid((1, 1, z["L"], 128), sd) for sd in (81, 82, 83))
    check_fp8_attention(lay, q, k, v, 90, sample_tiles=8)


def test_fp8_long_text_workload():
    cfg = configs.VIDEO_LONG
    z = rf.layout_sizes(cfg.layout)
    say(f"[fp8 workload] {cfg.name} (2 heads, sampled tiles incl. text)")
    q, k, v = inputs.make_qkv(cfg, "cuda", H=2)
    check_fp8_attention(cfg.layout, q, k, v, cfg.sparsity[0], sample_tiles=10)


def test_fp8_rows_matches_predicted_bitwise():
    cfg = configs.VIDEO720
    say("[fp8 rows vs predicted] 720p, 4 heads")
    q, k, v = inputs.make_qkv(cfg, "cuda", H=4)
    plan = rf.Plan(cfg.layout)
    z = plan.sizes
    s = 80
    g = run_fp8(plan, q, k, v, s)
    q8, qs = rf.quantize_fp8(plan, g["qp"])
    k8, ks = rf.quantize_fp8(plan, g["kp"])
    v8, vs = rf.quantize_fp8(plan, g["vt"], order=rf.TILES_T)
    kc = plan.keep(s)
    rows = torch.full((1, 4, z["n_tiles"], kc["row_len_video"] + 1), -1, dtype=torch.int32,
                      device="cuda")
    rows[..., :kc["row_len_video"]] = g["kept"].view(1, 4, z["nb"], kc["row_len_video"])
    got, lse = rf.sparse_attn_fp8_rows(plan, q8, qs, k8, ks, v8, vs, rows, lse=True)
    torch.cuda.synchronize()
    assert torch.equal(got, g["op"])
    assert torch.equal(lse, g["lse"])
    plan.close()


def test_fp8_deterministic_and_errors():
    lay = EDGE[0][1]
    z = rf.layout_sizes(lay)
    q, k, v = (_iid((1, 2, z["L"], 128), sd) for sd in (71, 72, 73))
    plan = rf.Plan(lay)
    a = run_fp8(plan, q, k, v, 60)["op"]
    b = run_fp8(plan, q, k, v, 60)["op"]
    assert torch.equal(a, b)
    with pytest.raises(rf.RfError):                      # fp32 input
        rf.quantize_fp8(plan, torch.zeros((1, 2, z["Lt"], 128), device="cuda"))
    plan64 = rf.Plan(dict(T=2, H=8, W=8, wt=1, wh=8, ww=8, n_text=0, permute=1, sink=0))
    x = torch.zeros((1, 1, plan64.sizes["Lt"], 128), dtype=torch.bfloat16, device="cuda")
    x8, xs = rf.quantize_fp8(plan64, x)
    assert torch.all(x8 == 0) and torch.all(xs == 1.0)   # all-zero tiles: scale 1
    v8, vsc = rf.quantize_fp8(plan64, torch.zeros((1, 1, plan64.sizes["n_tiles"], 128, 64),
                                                  dtype=torch.bfloat16, device="cuda"),
                              order=rf.TILES_T)
    kept = torch.zeros((1, 1, plan64.keep(0)["nnz_per_head"]), dtype=torch.int32, device="cuda")
    with pytest.raises(rf.RfError):                      # bs = 64 is not supported
        rf.sparse_attn_fp8(plan64, x8, xs, x8, xs, v8, vsc, kept, 0)
    plan.close()
    plan64.close()


@pytest.mark.parametrize("case", EDGE[:3] + [("video720-2heads", configs.VIDEO720.layout, 1, 2, 80)],
                         ids=[c[0] for c in EDGE[:3]] + ["video720-2heads"])
def test_fused_permute_fp8_matches_two_steps(case):
    """rf_permute_fp8 gives the bytes of rf_permute + rf_quantize_fp8 and the
    means of rf_permute_means."""
    name, lay, B, H, _ = case
    say(f"[fp8 fused permute] {name}")
    z = rf.layout_sizes(lay)
    plan = rf.Plan(lay)
    x = _iid((B, H, z["L"], 128), 77)
    xp, xbar = rf.permute_means(plan, x)
    c1, s1 = rf.quantize_fp8(plan, xp)
    c2, s2, xbar2 = rf.permute_fp8(plan, x, means=True)
    vt = rf.permute(plan, x, order=rf.TILES_T)
    c3, s3 = rf.quantize_fp8(plan, vt, order=rf.TILES_T)
    c4, s4 = rf.permute_fp8(plan, x, order=rf.TILES_T)
    c5, s5 = rf.permute_fp8(plan, x)                     # no means
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(s1, s2) and torch.equal(xbar, xbar2)
    assert torch.equal(c3, c4) and torch.equal(s3, s4)
    assert torch.equal(c1, c5) and torch.equal(s1, s5)
    plan.close()
