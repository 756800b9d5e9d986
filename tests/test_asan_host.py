"""The host side of the library (layout sizes, index tables, keep counts, the
argument checks and error paths of every entry point) under AddressSanitizer:
tests/test_abi_cpu.py and tests/test_binding_checks.py run in a subprocess
against librf_asan.so, with the sanitizer runtime preloaded.  CPU only; the
sanitized build is made (host code only) when missing or older than a
source."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

from image_diffusion_dits_amd import build

HERE = os.path.dirname(os.path.abspath(__file__))


def _stale(lib):
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    srcs = glob.glob(os.path.join(build.CSRC, "*")) + glob.glob(os.path.join(build.INCLUDE, "*"))
    return any(os.path.getmtime(s) > t for s in srcs)


@pytest.mark.skipif(shutil.which(build.HIPCC) is None and not os.path.exists(build.HIPCC),
                    reason="hipcc not available")
def test_host_code_is_clean_under_address_sanitizer():
    lib = os.path.join(build.PKG, build.VARIANTS["asan"][0])
    if _stale(lib):
        build.build(variant="asan")
    runtime = build.asan_runtime()
    assert os.path.exists(runtime), runtime
    env = dict(os.environ, LD_PRELOAD=runtime, RF_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_abi_cpu.py"),
                        os.path.join(HERE, "test_binding_checks.py")],
                       env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
