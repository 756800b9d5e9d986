"""Host logic of bench.py that runs without a GPU: the one-GPU guard, the
shader-clock sampler, the source-keyed traffic record and the argument
guards of the head-share and clock studies."""
import json
import os
import subprocess
import sys
import time
import types

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


SMI_OUT = """
============================ ROCm System Management Interface ============================
=================================== Current clock frequencies ===================================
GPU[0]\t\t: fclk clock level: 0: (1900Mhz)
GPU[0]\t\t: mclk clock level: 0: (2000Mhz)
GPU[0]\t\t: sclk clock level: 1: ({mhz}Mhz)
GPU[0]\t\t: socclk clock level: 0: (28Mhz)
==================================================================================================
"""


def test_clock_sampler_reads_sclk(monkeypatch):
    readings = iter([1700, 1680, 1720, 1700, 1690] + [1700] * 1000)

    def fake_run(cmd, **kw):
        assert cmd[:2] == ["rocm-smi", "--showclocks"]
        time.sleep(0.002)
        return types.SimpleNamespace(stdout=SMI_OUT.format(mhz=next(readings)), returncode=0)

    monkeypatch.setattr(bench.shutil, "which", lambda name: "/usr/bin/" + name)
    monkeypatch.setattr(bench.subprocess, "run", fake_run)
    with bench.ClockSampler() as clock:
        time.sleep(0.1)
    rec = clock.record()
    assert rec is not None and rec["samples"] >= 5
    assert rec["min"] >= 1680 and rec["max"] <= 1720
    assert rec["median"] == 1700          # sclk only: not fclk, mclk or socclk


def test_clock_sampler_without_rocm_smi(monkeypatch):
    monkeypatch.setattr(bench.shutil, "which", lambda name: None)
    with bench.ClockSampler() as clock:
        time.sleep(0.01)
    assert clock.record() is None


def test_clock_sampler_tool_failure_gives_none(monkeypatch):
    def failing_run(cmd, **kw):
        raise subprocess.TimeoutExpired(cmd, 5)

    monkeypatch.setattr(bench.shutil, "which", lambda name: "/usr/bin/" + name)
    monkeypatch.setattr(bench.subprocess, "run", failing_run)
    with bench.ClockSampler() as clock:
        time.sleep(0.01)
    assert clock.record() is None


def test_traffic_record_is_keyed_to_the_kernel_source(tmp_path, monkeypatch):
    kernel = "attn_bf16_pp_kernel"
    good = {kernel: {"src_sha256": bench.source_hash(kernel), "workload": "video720-21x45x80",
                     "hbm_bytes_per_launch": 123}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(good))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.stored_traffic(kernel, "video720-21x45x80") == 123
    assert bench.stored_traffic(kernel, "image-64x64") is None          # other workload
    stale = {kernel: dict(good[kernel], src_sha256="0" * 64)}
    f.write_text(json.dumps(stale))
    assert bench.stored_traffic(kernel, "video720-21x45x80") is None    # kernel changed since
    f.write_text("not json")
    assert bench.stored_traffic(kernel, "video720-21x45x80") is None


def test_clock_sampler_stays_off_under_a_profiler(monkeypatch):
    calls = []
    monkeypatch.setattr(bench.shutil, "which", lambda name: "/usr/bin/" + name)
    monkeypatch.setattr(bench.subprocess, "run", lambda *a, **k: calls.append(a))
    monkeypatch.setenv("ROCPROF_KERNEL_TRACE", "1")
    with bench.ClockSampler() as clock:
        time.sleep(0.01)
    assert clock.record() is None and calls == []


def test_head_share_out_of_range_is_refused():
    for h in ("0", "41"):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--heads", h],
                           capture_output=True, text=True, timeout=300, cwd=ROOT)
        assert r.returncode == 2, r.stderr[-500:]
        assert "--heads must be in 1..40" in r.stderr
        assert r.stdout == ""


def test_clock_study_refuses_an_fp32_workload():
    """--clock-vs-data times the bf16 (or FP8) attention: the fp32 workload
    is refused before any device is touched."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--clock-vs-data",
                        "--config", "1"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "bf16 or FP8" in r.stderr
    assert r.stdout == ""
