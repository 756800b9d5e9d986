"""Benchmark of the RainFusion2.0 sparse-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3]
                    [--sparsity S] [--raster] [--no-cpu-baseline]

One step is one pass of the whole path over one attention call of the
workload: permute K and V (3D windows), pool the block means of Q and K,
predict the mask, block-sparse attention reading Q and writing O in raster
order (the fused path; --unfused permutes Q and unpermutes O in passes of
their own).  With --fp8 the permutations quantize Q, K and V to e4m3 and
the attention writes O in raster order (--unfused: slot order, then an
unpermute pass).  Inputs are synthetic (seeded) and
resident in HBM before timing starts; every output buffer is allocated
beforehand, so the timed region only launches kernels.

Prints one JSON line.  `value` is executed attention TFLOP/s over the whole
step: 4*d*bs^2 FLOP per kept (query tile, key tile) pair, summed over heads,
divided by the step time.  `roofline` reports the attention kernel alone
against the bf16 dense MFMA peak (its duration from HIP events on the
stream it runs on), and `cpu_baseline` times the fp64 oracle on a bounded
sample of the same workload on the host's cores.
"""
import argparse
import hashlib
import json
import os
import re
import shutil
import statistics
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "block-sparse attn TFLOP/s, ms/call @75.6k tok 80% sparse, MFMA util"
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3
PEAK_FP8_TFLOPS = 5000.0        # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0
CSRC = os.path.join(ROOT, "image_diffusion_dits_amd", "csrc")
# Sources each attention kernel is compiled from (its file and the headers it
# includes): stored counter readings apply only while these are unchanged.
KERNEL_SOURCES = {
    "attn_bf16_pp_kernel": ["attn.hip", "tile_common.h", "rf_internal.h"],
    "attn_fp8_pp_kernel": ["attn_fp8.hip", "tile_common.h", "rf_internal.h"],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--sparsity", type=int, default=None)
    ap.add_argument("--raster", action="store_true",
                    help="permutation off (raster blocks)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="one JSON line per workload point (all configurations, the "
                         "720p sparsity sweep in window and raster order)")
    ap.add_argument("--unfused", action="store_true",
                    help="attend in slot order and unpermute O in a pass of its own "
                         "(bf16: and permute Q in a pass of its own)")
    ap.add_argument("--cpu-tiles", type=int, default=660,
                    help="query tiles in the oracle's attention sample")
    ap.add_argument("--cpu-heads", type=int, default=2,
                    help="heads the oracle's sample covers")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after timing, run a plain elementwise copy of "
                         "known size (counter calibration)")
    ap.add_argument("--recall", type=int, default=0, metavar="N",
                    help="instead of the step benchmark, measure the attention "
                         "recall of N sampled query tiles per head at each "
                         "sweep sparsity, permutation on and off")
    ap.add_argument("--schedule", type=int, default=0, metavar="N",
                    help="instead of the step benchmark, time an N-step sampling "
                         "run of one attention layer under the timestep policy "
                         "(first 10%% of steps dense) on the 720p workload")
    ap.add_argument("--refresh", type=int, default=1,
                    help="with --schedule: predict the mask every R sparse steps")
    ap.add_argument("--fp8", action="store_true",
                    help="run the attention on OCP e4m3 operands (the quantization "
                         "of Q, K and V is a stage of the timed step)")
    ap.add_argument("--patterns", action="store_true",
                    help="instead of the step benchmark, time the v1 head-pattern "
                         "path on the 720p workload: ARM recall and decision, "
                         "pattern rows, and block-sparse attention on them")
    ap.add_argument("--heads", type=int, default=None,
                    help="time the workload on this many heads instead of all: one "
                         "GPU's share when the heads are split across GPUs (the "
                         "720p workload's 40 heads over 8 GPUs is --heads 5)")
    ap.add_argument("--clock-vs-data", action="store_true",
                    help="instead of the step benchmark, time the bf16 attention (with "
                         "--fp8 the FP8 one) on the same kept tiles with the synthetic "
                         "operands, with Q and K scaled by 0.01, and with all-zero "
                         "operands, each with the shader clock it holds and the cycles "
                         "per call that gives")
    ap.add_argument("--reference-gemm", action="store_true",
                    help="instead of the step benchmark, time the vendor library's "
                         "dense bf16 GEMM (torch.matmul, 8192^3) on the same GPU, "
                         "with the shader clock it holds: the rate a dense bf16 "
                         "matrix-core kernel reaches on this part")
    return ap.parse_args()


def _time(fn, reps=5):
    """Median milliseconds of fn() over reps runs, HIP events on the current
    stream (the library launches on it)."""
    import numpy as np
    import torch
    fn()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return float(np.median(ts))


def pattern_study():
    """v1 head patterns on the 720p workload (bandwidth 1/4, tau 2, ARM local
    stride 4 and global stride 64, alpha 0.9): times of each stage and the
    attention rate on pattern rows, against the 80% predicted mask."""
    import torch

    from image_diffusion_dits_amd import configs, inputs, rf

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    cfg = configs.VIDEO720
    q, k, v = inputs.make_qkv(cfg, dev)
    plan = rf.Plan(cfg.layout)
    z = plan.sizes
    B, H, d, bs = cfg.B, cfg.H, cfg.d, z["bs"]
    qp, qbar = rf.permute_means(plan, q)
    kp, kbar = rf.permute_means(plan, k)
    vt = rf.permute(plan, v, order=rf.TILES_T)
    band, tau, ls, gs, alpha = rf.band_tiles(plan, 0.25), 2, 4, 64, 0.9
    loc = rf.arm_recall(plan, qp, kp, True, ls, rf.TEMPORAL, band, tau)
    glo = rf.arm_recall(plan, qp, kp, False, gs, rf.SPATIAL, band, tau)
    pat, mean = rf.arm_classify(loc, glo, alpha)
    out = {"metric": "v1 head-pattern path on the 720p workload", "unit": "ms",
           "higher_is_better": False, "data": "synthetic",
           "config": {"workload": cfg.name, "heads": H, "band_tiles": band, "tau": tau,
                      "arm_local_stride": ls, "arm_global_stride": gs, "alpha": alpha,
                      "arm_local_samples": loc.shape[-1],
                      "arm_global_samples": glo.shape[-1]}}
    t_loc = _time(lambda: rf.arm_recall(plan, qp, kp, True, ls, rf.TEMPORAL, band, tau, out=loc))
    t_glo = _time(lambda: rf.arm_recall(plan, qp, kp, False, gs, rf.SPATIAL, band, tau, out=glo))
    t_cls = _time(lambda: rf.arm_classify(loc, glo, alpha, pattern=pat, mean=mean))
    counts = torch.bincount(pat.view(-1).long(), minlength=3).tolist()
    m = mean.view(-1, 2)
    out["arm"] = {"ms_local": round(t_loc, 4), "ms_global": round(t_glo, 4),
                  "ms_classify": round(t_cls, 4),
                  "heads_spatial_temporal_textural": counts,
                  "mean_local_recall": round(float(m[:, 0].mean()), 4),
                  "mean_global_recall": round(float(m[:, 1].mean()), 4)}
    op = torch.empty_like(qp)
    runs = {"arm": pat}
    for name, p in (("spatial", rf.SPATIAL), ("temporal", rf.TEMPORAL),
                    ("textural", rf.TEXTURAL)):
        runs[name] = torch.full((B, H), p, dtype=torch.int32, device=dev)
    width = rf.pattern_row_width(plan.layout, band, tau)
    rows = torch.empty((B, H, z["n_tiles"], width), dtype=torch.int32, device=dev)
    out["patterns"] = {}
    for name, hp in runs.items():
        t_rows = _time(lambda: rf.pattern_mask(plan, hp, band, tau, out=rows))
        pairs = int((rows >= 0).sum())
        t_att = _time(lambda: rf.sparse_attn_rows(plan, qp, kp, vt, rows, out=op))
        tflop = 4.0 * d * bs * bs * pairs / 1e12
        out["patterns"][name] = {
            "ms_rows": round(t_rows, 4), "ms_attn": round(t_att, 3),
            "kept_pair_share": round(pairs / (B * H * z["n_tiles"] ** 2), 4),
            "attn_tflops": round(tflop / (t_att * 1e-3), 1),
            "mfma_frac": round(tflop / (t_att * 1e-3) / PEAK_BF16_TFLOPS, 4)}
        print(f"[patterns] {name}: {out['patterns'][name]}", file=sys.stderr, flush=True)
    kept = rf.predict_mask(plan, qbar, kbar, 80)
    out["predicted_80pct_ms_attn"] = round(
        _time(lambda: rf.sparse_attn(plan, qp, kp, vt, kept, 80, out=op)), 3)
    plan.close()
    print(json.dumps(out))
    return 0


def schedule_study(n_steps, refresh, sparsity):
    """Attention time per step over a sampling run under the timestep policy,
    against an all-dense run; prints one JSON line."""
    import numpy as np
    import torch

    from image_diffusion_dits_amd import configs, inputs
    from image_diffusion_dits_amd.policy import SparseAttention, StepPolicy

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    cfg = configs.VIDEO720
    q, k, v = inputs.make_qkv(cfg, dev)
    pol = StepPolicy(n_steps, dense_fraction=0.10, sparsity_pct=sparsity,
                     refresh_every=refresh)
    layer = SparseAttention(cfg.layout, pol, cfg.B, cfg.H, cfg.d, q.dtype, dev)
    out = torch.empty_like(q)
    for t in sorted({0, pol.n_dense}):         # warm both kinds of step
        if t < n_steps:
            layer(q, k, v, t, out=out)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_steps + 1)]
    ev[0].record()
    for t in range(n_steps):
        layer(q, k, v, t, out=out)
        ev[t + 1].record()
    torch.cuda.synchronize()
    ms = [ev[t].elapsed_time(ev[t + 1]) for t in range(n_steps)]
    modes = pol.schedule()
    by = {m: [x for x, mm in zip(ms, modes) if mm == m] for m in set(modes)}
    dense = float(np.median(by["dense"])) if "dense" in by else None
    mean = float(np.mean(ms))
    layer.close()
    print(json.dumps({
        "metric": "attention ms per sampling step under the timestep policy",
        "unit": "ms", "higher_is_better": False, "data": "synthetic",
        "config": {"workload": cfg.name, "steps": n_steps, "dense_fraction": 0.10,
                   "sparsity_pct": sparsity, "refresh_every": refresh},
        "mean_ms_per_step": round(mean, 3),
        "ms_by_mode": {m: round(float(np.median(x)), 3) for m, x in by.items()},
        "steps_by_mode": {m: len(x) for m, x in by.items()},
        "speedup_vs_all_dense": round(dense / mean, 3) if dense else None}))
    return 0


def recall_study(n_sample):
    """Mean share of each sampled query's dense softmax mass inside its kept
    tiles (the masked recall R'), 720p tensors, permutation on vs off, at the
    sweep sparsities; prints one JSON line."""
    import numpy as np
    import torch

    from image_diffusion_dits_amd import configs, inputs, rf

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    out = {"metric": "attention recall (share of dense softmax mass in kept tiles)",
           "unit": "fraction", "higher_is_better": True, "data": "synthetic",
           "samples_per_head": n_sample, "modes": {}}
    for cfg in (configs.SWEEP, configs.SWEEP_RASTER):
        q, k, _ = inputs.make_qkv(cfg, dev)
        plan = rf.Plan(cfg.layout)
        qp, qbar = rf.permute_means(plan, q)
        kp, kbar = rf.permute_means(plan, k)
        z = plan.sizes
        rng = np.random.default_rng(7)
        tiles = np.sort(rng.choice(z["nb"], size=min(n_sample, z["nb"]), replace=False))
        st = torch.tensor(tiles, dtype=torch.int32, device=dev)
        mode = {}
        for s in cfg.sparsity:
            kept = rf.predict_mask(plan, qbar, kbar, s)
            rec = rf.attention_recall(plan, qp, kp, kept, s, st)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            rf.attention_recall(plan, qp, kp, kept, s, st, out=rec)
            e1.record()
            torch.cuda.synchronize()
            r = rec.cpu().numpy()
            mode[str(s)] = {"kept_tiles_per_row": plan.keep(s)["k_eff"],
                            "mean": round(float(np.nanmean(r)), 5),
                            "p10": round(float(np.nanpercentile(r, 10)), 5),
                            "min": round(float(np.nanmin(r)), 5),
                            "ms": round(e0.elapsed_time(e1), 3)}
            print(f"[recall] {cfg.name} s={s}: {mode[str(s)]}", file=sys.stderr, flush=True)
        out["modes"][cfg.name] = mode
        plan.close()
        del q, k, qp, kp
    print(json.dumps(out))
    return 0


def reference_gemm(n=8192, calls=50):
    """Rate of the vendor library's dense bf16 GEMM (torch.matmul, which
    dispatches to hipBLASLt) on an n x n x n product, timed with HIP events,
    and the shader clock held meanwhile.  Context for the attention's rate:
    this is what a tuned dense matrix-core kernel reaches here, against the
    same 2.5 PFLOP/s peak quoted at 2.4 GHz."""
    import torch

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    g = torch.Generator(device=dev).manual_seed(0)
    x = torch.randn(n, n, device=dev, dtype=torch.bfloat16, generator=g)
    y = torch.randn(n, n, device=dev, dtype=torch.bfloat16, generator=g)
    out = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(10):
        torch.matmul(x, y, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(calls):
        torch.matmul(x, y, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / calls
    clock = ClockSampler()
    with clock:
        t_end = time.perf_counter() + (0.5 if clock.available() else 0.0)
        while time.perf_counter() < t_end:
            for _ in range(10):
                torch.matmul(x, y, out=out)
            torch.cuda.synchronize()
    tflops = 2.0 * n ** 3 / (ms / 1e3) / 1e12
    print(json.dumps({"metric": "dense bf16 GEMM TFLOP/s (torch.matmul, vendor library)",
                      "value": round(tflops, 2), "unit": "TFLOP/s", "n": n,
                      "ms_per_call": round(ms, 4), "calls": calls,
                      "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
                      "peak": PEAK_BF16_TFLOPS, "sclk_mhz": clock.record()}), flush=True)
    return 0


def clock_study(a):
    """The bf16 attention of one workload on three sets of operands that
    share the synthetic data's kept tiles: the synthetic operands, Q and K
    scaled by 0.01 (near-uniform weights), and all-zero operands.  The work
    (tiles, copies, instructions) is the same; the power drawn, and so the
    clock the chip holds, is not.  Each point runs for about two seconds
    with the clock sampled, and reports ms per call, the frac against the
    2.4 GHz peak, and cycles per call (ms x the median clock).  With --fp8
    the FP8 attention runs instead, on each set's e4m3 codes."""
    import torch

    from image_diffusion_dits_amd import configs, inputs, rf

    cfg = configs.get(a.config)
    if cfg.dtype != "bf16":
        print(f"--clock-vs-data times the bf16 or FP8 attention; {cfg.name} is {cfg.dtype}",
              file=sys.stderr)
        return 2
    s = a.sparsity if a.sparsity is not None else (80 if a.config == 5 else cfg.sparsity[0])
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    q, k, v = inputs.make_qkv(cfg, dev, H=a.heads)
    peak = PEAK_FP8_TFLOPS if a.fp8 else PEAK_BF16_TFLOPS
    plan = rf.Plan(cfg.layout)
    z = plan.sizes
    B, H, d = q.shape[0], q.shape[1], q.shape[3]
    qp, qbar = rf.permute_means(plan, q)
    kp, kbar = rf.permute_means(plan, k)
    vt = rf.permute(plan, v, order=rf.TILES_T)
    kept = rf.predict_mask(plan, qbar, kbar, s)
    flop = 4.0 * d * z["bs"] ** 2 * plan.keep(s)["nnz_per_head"] * B * H
    sets = [("synthetic", qp, kp, vt),
            ("q_k_times_0.01", qp * 0.01, kp * 0.01, vt),
            ("zeros", torch.zeros_like(qp), torch.zeros_like(kp), torch.zeros_like(vt))]
    points = []
    for name, qq, kk, vv in sets:
        out = torch.empty_like(qq)
        if a.fp8:
            ops = (*rf.quantize_fp8(plan, qq), *rf.quantize_fp8(plan, kk),
                   *rf.quantize_fp8(plan, vv, order=rf.TILES_T))
            call = lambda: rf.sparse_attn_fp8(plan, *ops, kept, s, out=out)
        else:
            call = lambda: rf.sparse_attn(plan, qq, kk, vv, kept, s, out=out)
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        clock = ClockSampler()
        calls = 0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with clock:
            e0.record()
            t_end = time.perf_counter() + 2.0
            while time.perf_counter() < t_end:
                for _ in range(5):
                    call()
                calls += 5
                torch.cuda.synchronize()
            e1.record()
            torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / calls
        clk = clock.record()
        points.append({"operands": name, "ms_per_call": round(ms, 4), "calls": calls,
                       "frac": round(flop / (ms / 1e3) / 1e12 / peak, 4),
                       "sclk_mhz": clk,
                       "cycles_per_call": (round(ms * clk["median"] * 1e3) if clk else None)})
        print(f"[clock] {name}: {points[-1]}", file=sys.stderr, flush=True)
        del out
    plan.close()
    kind = "FP8" if a.fp8 else "bf16"
    print(json.dumps({"metric": f"{kind} attention time and shader clock against operand values",
                      "workload": cfg.name, "sparsity_pct": s, "heads": H,
                      "exec_tflop_per_call": round(flop / 1e12, 4), "points": points}),
          flush=True)
    return 0


def source_hash(kernel):
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic(kernel, workload):
    """HBM bytes per attention launch from committed rocprofv3 counter runs,
    or None when absent or taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kernel, {})
    except (OSError, ValueError):
        return None
    if kernel not in KERNEL_SOURCES or rec.get("src_sha256") != source_hash(kernel):
        return None
    if rec.get("workload") != workload:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, q, k, v, sparsity, n_tiles_sample, exec_flop_total, fp8=False,
                 n_heads=2):
    """Time the fp64 oracle on the first n_heads heads: the whole of permute,
    means, mask (with fp8, the e4m3 quantization of Q, K, V too) and
    unpermute, plus attention on a sample of query tiles; extrapolate to all
    heads and tiles (heads are independent and every video row keeps the
    same number of tiles)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import rainfusion_oracle as orc

    lay = orc.Layout(**{key: cfg.layout[key] for key in
                        ("T", "H", "W", "wt", "wh", "ww", "n_text", "permute", "sink")})
    z = orc.sizes(lay)
    rng = np.random.default_rng(0)
    tiles = sorted(rng.choice(z["nb"], size=min(n_tiles_sample, z["nb"]),
                              replace=False).tolist())
    H = cfg.H * cfg.B
    n_heads = max(1, min(n_heads, cfg.H))
    fixed = attn = 0.0
    host_cpus = len(os.sched_getaffinity(0))
    # The oracle's matrix products use every host core this process may run on.
    limiter = threadpool_limits(limits=host_cpus)
    for h in range(n_heads):
        f64 = lambda t: t[:1, h:h + 1].cpu().double().numpy()
        qh, kh, vh = f64(q), f64(k), f64(v)
        t0 = time.perf_counter()
        qp, kp, vp = (orc.permute(x, lay) for x in (qh, kh, vh))
        qbar, kbar = orc.block_means(qp, lay), orc.block_means(kp, lay)
        kept, _ = orc.predict_mask(qbar, kbar, lay, sparsity)
        if fp8:      # the oracle's fp8 attention is attention over these values
            qp, _ = orc.quantize_tiles(qp, lay)
            kp, _ = orc.quantize_tiles(kp, lay)
            vp, _ = orc.quantize_channels(vp)
        t1 = time.perf_counter()
        op = orc.sparse_attention(qp, kp, vp, kept, lay, query_tiles={(0, 0): tiles})
        t2 = time.perf_counter()
        op[np.isnan(op)] = 0.0
        orc.unpermute(op, lay)
        t3 = time.perf_counter()
        fixed += (t1 - t0) + (t3 - t2)
        attn += t2 - t1
    per_head_fixed = fixed / n_heads
    per_tile = attn / (n_heads * len(tiles))
    full = H * per_head_fixed + H * z["n_tiles"] * per_tile
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    limiter.unregister()
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f
                          if l.startswith("model name")), "")
    except OSError:
        pass
    return {
        "value": exec_flop_total / full / 1e12,
        "unit": "TFLOP/s",
        # threads the oracle ran on: its BLAS products use them all; the
        # permutation, pooling and selection loops run on one
        "cores": int(threads),
        "host_cpus": host_cpus,
        "nproc": os.cpu_count(),
        "cpu_model": model,
        "kind": "oracle",
        "sample": (f"heads 0-{n_heads - 1} of {H}: permute, means, mask, unpermute in "
                   f"full; attention on {len(tiles)} of {z['n_tiles']} query tiles "
                   f"each; {fixed + attn:.1f} s measured, extrapolated to all heads "
                   f"and tiles ({full:.0f} s per step)"),
    }


def main():
    a = parse()
    if a.recall:
        return recall_study(a.recall)
    if a.schedule:
        return schedule_study(a.schedule, a.refresh,
                              a.sparsity if a.sparsity is not None else 80)
    if a.patterns:
        return pattern_study()
    if a.reference_gemm:
        return reference_gemm()
    if a.clock_vs_data:
        return clock_study(a)
    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported "
              "(every step is independent per head; the multi-GPU layout is "
              "head sharding, not run here)", file=sys.stderr)
        return 2
    import torch

    from image_diffusion_dits_amd import configs, inputs

    if a.sweep:
        return sweep(a)
    cfg = configs.get(a.config)
    if a.raster:
        cfg = configs.SWEEP_RASTER if a.config in (3, 5) else cfg
    s = a.sparsity if a.sparsity is not None else (80 if a.config == 5 else cfg.sparsity[0])
    if a.heads is not None and not 1 <= a.heads <= cfg.H:
        print(f"--heads must be in 1..{cfg.H} for {cfg.name}", file=sys.stderr)
        return 2
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    q, k, v = inputs.make_qkv(cfg, dev, H=a.heads)
    rec, exec_flop = measure(a, cfg, s, q, k, v)
    if not a.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(cfg, q, k, v, s, a.cpu_tiles, exec_flop, a.fp8,
                                           a.cpu_heads)
    print(json.dumps(rec), flush=True)
    return 0


class ClockSampler:
    """Reads the GPU's shader clock (SCLK) with rocm-smi, over and over, while
    the timed steps run, so that each record says at what clock its rate was
    reached.  Under sustained matrix-core load the clock sits well below the
    2.4 GHz the published peaks assume.  Gives None where rocm-smi is absent,
    under a profiler, or when no reading finished in time."""

    PATTERN = re.compile(r"sclk clock level: \S+ \((\d+)Mhz\)")

    def __init__(self):
        self.samples = []
        self._stop = threading.Event()
        self._thread = None

    @staticmethod
    def profiler_attached():
        """True under rocprofv3, whose preloaded library would initialise the
        GPU in the sampler's child processes too."""
        return ("rocprof" in os.environ.get("LD_PRELOAD", "")
                or any(k.startswith("ROCPROF") for k in os.environ))

    def available(self):
        return shutil.which("rocm-smi") is not None and not self.profiler_attached()

    def __enter__(self):
        if self.available():
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def _run(self):
        while not self._stop.is_set():
            try:
                r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True,
                                   text=True, timeout=5)
            except (OSError, subprocess.SubprocessError):
                return
            found = self.PATTERN.findall(r.stdout)
            if found and not self._stop.is_set():
                # The busiest GPU the tool lists (on a one-GPU machine, that GPU).
                self.samples.append(max(int(x) for x in found))

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread is not None:
            self._thread.join(timeout=10)
        return False

    def record(self):
        if not self.samples:
            return None
        return {"median": statistics.median(self.samples), "min": min(self.samples),
                "max": max(self.samples), "samples": len(self.samples)}


def host_info():
    """Host facts recorded beside each measurement."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f
                          if l.startswith("model name")), "")
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "host_cpus": len(os.sched_getaffinity(0)),
            "cpu_model": model}


def sweep(a):
    """One JSON line per (workload, sparsity, order): the tiny fp32 case, the
    image, the 720p and long+text videos at their sparsities, and the 720p
    sweep over sparsity in window and raster order.  Each line carries the
    sha256 of the inputs, so that it can be joined with the parity record of
    the same point."""
    import torch

    from image_diffusion_dits_amd import configs, inputs

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    points = [(configs.TINY, 50), (configs.IMAGE, 60), (configs.VIDEO720, 80),
              (configs.VIDEO_LONG, 85)]
    points += [(configs.SWEEP, sp) for sp in configs.SWEEP.sparsity]
    points += [(configs.SWEEP_RASTER, sp) for sp in configs.SWEEP_RASTER.sparsity]
    host = host_info()
    cache = {}
    for cfg, sp in points:
        if a.fp8 and (cfg.dtype != "bf16" or cfg.d != 128):
            continue                    # the FP8 attention takes d = 128, bf16 inputs
        key = (cfg.cid, cfg.permute)
        if key not in cache:
            cache.clear()
            torch.cuda.empty_cache()
            dev_in = "cpu" if cfg.cid in (1, 2) else dev
            q, k, v = (t.to(dev) for t in inputs.make_qkv(cfg, dev_in))
            cache[key] = (q, k, v, {n: inputs.sha256(t) for n, t in
                                    (("q", q), ("k", k), ("v", v))})
        q, k, v, sha = cache[key]
        rec, _ = measure(a, cfg, sp, q, k, v)
        rec["inputs_sha256"] = sha
        rec["host"] = host
        print(json.dumps(rec), flush=True)
    return 0


def measure(a, cfg, s, q, k, v):
    """Times the step on one workload point; returns (record, executed FLOP
    per call)."""
    import torch

    from image_diffusion_dits_amd import rf

    dev = q.device
    plan = rf.Plan(cfg.layout)
    z = plan.sizes
    kc = plan.keep(s)
    B, H, d = q.shape[0], q.shape[1], q.shape[3]
    bs = z["bs"]

    # Every buffer is allocated before timing.
    qp = torch.empty(B, H, z["Lt"], d, dtype=q.dtype, device=dev)
    kp = torch.empty_like(qp)
    vt = torch.empty(B, H, z["n_tiles"], d, bs, dtype=q.dtype, device=dev)
    qbar = torch.empty(B, H, z["nb"], d, dtype=torch.float32, device=dev)
    kbar = torch.empty_like(qbar)
    kept = torch.empty(B, H, kc["nnz_per_head"], dtype=torch.int32, device=dev)
    op = torch.empty_like(qp)
    o = torch.empty_like(q)
    if a.fp8:
        q8 = torch.empty(qp.shape, dtype=torch.uint8, device=dev)
        k8 = torch.empty_like(q8)
        v8 = torch.empty(vt.shape, dtype=torch.uint8, device=dev)
        qs = torch.empty(B, H, z["n_tiles"], dtype=torch.float32, device=dev)
        ks = torch.empty_like(qs)
        vs = torch.empty(B, H, d, dtype=torch.float32, device=dev)

    fused = not a.unfused
    if a.fp8:
        stages = ["permute_fp8_qk", "permute_fp8_v", "predict_mask", "sparse_attn"]
        if not fused:
            stages.append("unpermute")
    elif fused:
        stages = ["means_q_permute_means_k", "permute_v", "predict_mask", "sparse_attn"]
    else:
        stages = ["permute_means_qk", "permute_v", "predict_mask", "sparse_attn", "unpermute"]
    n_ev = len(stages) + 1

    def step(ev=None):
        marks = iter(range(n_ev))

        def mark():
            i = next(marks)
            if ev is not None:
                ev[i].record()
        mark()
        if a.fp8:
            rf.permute_fp8(plan, q, means=True, out=q8, scale=qs, xbar=qbar)
            rf.permute_fp8(plan, k, means=True, out=k8, scale=ks, xbar=kbar)
            mark()
            rf.permute_fp8(plan, v, order=rf.TILES_T, out=v8, scale=vs)
        elif fused:
            rf.permute_means(plan, q, xbar=qbar, means_only=True)
            rf.permute_means(plan, k, out=kp, xbar=kbar)
            mark()
            rf.permute(plan, v, order=rf.TILES_T, out=vt)
        else:
            rf.permute_means(plan, q, out=qp, xbar=qbar)
            rf.permute_means(plan, k, out=kp, xbar=kbar)
            mark()
            rf.permute(plan, v, order=rf.TILES_T, out=vt)
        mark()
        rf.predict_mask(plan, qbar, kbar, s, kept=kept)
        mark()
        if a.fp8 and fused:
            rf.sparse_attn_fp8_raster(plan, q8, qs, k8, ks, v8, vs, kept, s, out=o)
        elif a.fp8:
            rf.sparse_attn_fp8(plan, q8, qs, k8, ks, v8, vs, kept, s, out=op)
        elif fused:
            rf.sparse_attn_raster(plan, q, kp, vt, kept, s, out=o)
        else:
            rf.sparse_attn(plan, qp, kp, vt, kept, s, out=op)
        mark()
        if not fused:
            rf.unpermute(plan, op, out=o)
            mark()

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region 1: whole steps, wall clock.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        step()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / a.steps

    # Timed region 2: the same steps with HIP events between stages (all
    # kernels run on torch's current stream, which the events are recorded on).
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
           for _ in range(a.steps)]
    torch.cuda.synchronize()
    for i in range(a.steps):
        step(evs[i])
    torch.cuda.synchronize()

    # Region 3, not timed: the same steps for about half a second while the
    # shader clock is sampled (the sampler's subprocesses would otherwise
    # compete with the launches of a short step).
    clock = ClockSampler()
    if clock.available():
        with clock:
            t_end = time.perf_counter() + 0.5
            while time.perf_counter() < t_end:
                for _ in range(max(1, min(a.steps, 50))):
                    step()
                torch.cuda.synchronize()
    stage_ms = {name: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / a.steps
                for j, name in enumerate(stages)}
    ev_step_ms = sum(e[0].elapsed_time(e[n_ev - 1]) for e in evs) / a.steps
    j_attn = stages.index("sparse_attn")
    attn_median = statistics.median(e[j_attn].elapsed_time(e[j_attn + 1]) for e in evs)

    pairs = kc["nnz_per_head"] * B * H
    # Valid work: the (query, key) pairs of kept tiles whose slots both hold a
    # token (the executed count includes the pad slots of partial tiles).
    _, _, tile_count, _ = rf.layout_tables(cfg.layout)
    cnt = torch.from_numpy(tile_count.astype("int64")).to(dev)
    kept_l = kept.view(B * H, -1).long()
    n_tiles = z["n_tiles"]
    rows_t = torch.cat([torch.arange(z["nb"], device=dev).repeat_interleave(kc["row_len_video"]),
                        torch.arange(z["nb"], n_tiles, device=dev).repeat_interleave(kc["row_len_text"])])
    valid_pairs = int((cnt[rows_t][None, :] * cnt[kept_l]).sum())
    exec_flop = 4.0 * d * bs * bs * pairs
    L = z["L"]
    dense_flop = 4.0 * B * H * L * L * d
    attn_s = stage_ms["sparse_attn"] / 1e3
    ms_step = wall * 1e3
    if a.fp8:
        peak = PEAK_FP8_TFLOPS
    else:
        peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    attn_tflops = exec_flop / attn_s / 1e12
    workload = cfg.name + ("" if cfg.permute or cfg.name.endswith("-raster") else "-raster")
    kernel = ("attn_fp8_pp_kernel" if a.fp8 else
              "attn_bf16_pp_kernel" if cfg.dtype == "bf16" else "attn_f32_kernel")
    traffic = stored_traffic(kernel, workload)
    aux_ms = sum(stage_ms[n] for n in stages if n != "sparse_attn")
    esize = 2 if cfg.dtype == "bf16" else 4
    perm_bytes = B * H * (z["L"] + z["Lt"]) * d * esize   # one tensor
    unperm_bytes = B * H * 2 * z["L"] * d * esize
    perm8_bytes = B * H * (z["L"] * esize + z["Lt"]) * d      # bf16 in, e4m3 out
    perm8v_bytes = B * H * (2 * z["L"] * esize + z["Lt"]) * d  # maxima pass, then one pass
    means_bytes = B * H * z["L"] * d * esize                   # read only

    rec = {
        "metric": METRIC,
        "value": round(exec_flop / wall / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if a.fp8 else cfg.dtype,
        "data": "synthetic",
        "config": {
            "workload": workload,
            "path": ("fp8-" if a.fp8 else "") + ("fused" if fused else "five-pass"),
            "batch": B, "heads": H, "head_dim": d,
            "tokens": z["N"], "text_tokens": z["L"] - z["N"],
            "padded_slots": z["Lp"], "block": bs, "blocks": z["nb"],
            "sparsity_pct": s, "kept_tiles_per_row": kc["k_eff"],
            "kept_tile_pairs": pairs, "sink_blocks": z["n_sink"],
        },
        "attn_ms": round(stage_ms["sparse_attn"], 4),
        "attn_ms_median": round(attn_median, 4),
        "attn_exec_tflops": round(attn_tflops, 2),
        "attn_valid_tflops": round(4.0 * d * valid_pairs / attn_s / 1e12, 2),
        "valid_pair_share": round(valid_pairs / (pairs * bs * bs), 4),
        "attn_dense_equiv_tflops": round(dense_flop / attn_s / 1e12, 2),
        "mfma_util": round(attn_tflops / peak, 4),
        "exec_tflop_per_call": round(exec_flop / 1e12, 4),
        "dense_equiv_tflop_per_call": round(dense_flop / 1e12, 4),
        "stages_ms": {n: round(x, 4) for n, x in stage_ms.items()},
        "event_ms_per_step": round(ev_step_ms, 4),
        "mask_plus_perm_over_attn": round(aux_ms / stage_ms["sparse_attn"], 4),
        "hbm_gbs": (dict({
            "permute_fp8_qk": round(2 * perm8_bytes / (stage_ms["permute_fp8_qk"] / 1e3) / 1e9, 1),
            "permute_fp8_v": round(perm8v_bytes / (stage_ms["permute_fp8_v"] / 1e3) / 1e9, 1),
        }, **({} if fused else {
            "unpermute": round(unperm_bytes / (stage_ms["unpermute"] / 1e3) / 1e9, 1)}))
            if a.fp8 else {
            "means_q_permute_means_k": round((means_bytes + perm_bytes) / (
                stage_ms["means_q_permute_means_k"] / 1e3) / 1e9, 1),
            "permute_v": round(perm_bytes / (stage_ms["permute_v"] / 1e3) / 1e9, 1),
        } if fused else {
            "permute_means_qk": round(2 * perm_bytes / (stage_ms["permute_means_qk"] / 1e3) / 1e9, 1),
            "permute_v": round(perm_bytes / (stage_ms["permute_v"] / 1e3) / 1e9, 1),
            "unpermute": round(unperm_bytes / (stage_ms["unpermute"] / 1e3) / 1e9, 1),
        }),
        # Shader clock while the same steps run (rocm-smi samples, region 3);
        # the peaks above are quoted at 2.4 GHz.
        "sclk_mhz": clock.record(),
        "roofline": {
            "kernel": kernel,
            "bound": "mfma",
            "achieved": round(attn_tflops, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / peak, 4),
            "traffic": traffic,
        },
    }
    if a.fp8:
        # Cost of the e4m3 operands: the same step's output against the bf16
        # attention on the same permuted tensors.
        rf.permute(plan, q, out=qp)
        rf.permute(plan, k, out=kp)
        rf.permute(plan, v, order=rf.TILES_T, out=vt)
        ref = rf.unpermute(plan, rf.sparse_attn(plan, qp, kp, vt, kept, s))
        torch.cuda.synchronize()
        diff = (o.float() - ref.float()).abs()
        rec["fp8_vs_bf16_attention"] = {"max_abs": round(float(diff.max()), 5),
                                        "mean_abs": round(float(diff.mean()), 6)}
        rec["config"]["operands"] = ("e4m3: Q, K per-tile and V per-feature "
                                     "power-of-two scales; softmax weights e4m3")
        del ref, diff
    if a.copy_probe:
        # torch.neg reads and writes exactly n*2 bytes: a plain copy kernel
        # whose HBM counters calibrate the attention kernel's.
        n = 1 << 29
        src = torch.ones(n, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        rec["copy_probe_bytes"] = {"read": 2 * n, "write": 2 * n}
    plan.close()
    return rec, exec_flop


if __name__ == "__main__":
    sys.exit(main())
