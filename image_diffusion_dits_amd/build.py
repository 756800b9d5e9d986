"""Build librf.so (the C-ABI HIP library) in-tree for gfx950.

    python -m image_diffusion_dits_amd.build [--verbose] [--poison | --asan]

Compiles every source under csrc/ with hipcc (one object per source, in
parallel) into _build/, then links image_diffusion_dits_amd/librf.so.

Debug builds, each to a library of its own (select one for the binding with
RF_LIB=<path>):
  --poison  librf_poison.so: every attention kernel fills the LDS bytes a
            tile copy will overwrite with NaN before issuing the copy, so an
            operand read not ordered after its copy shows up in parity;
  --asan    librf_asan.so: the host code under AddressSanitizer (the device
            code is built as usual); load it with the sanitizer runtime
            preloaded (asan_runtime() gives its path).
"""
import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "librf.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-I", INCLUDE, "-I", CSRC,
    # Keep the compiler from forming packed fp32 VALU ops.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# Per-source extra hipcc flags (none at present).
EXTRA = {}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


VARIANTS = {
    None: ("librf.so", [], []),
    "poison": ("librf_poison.so", ["-DRF_POISON_LDS"], []),
    # -Xarch_host keeps the sanitizer out of the device code.
    "asan": ("librf_asan.so", ["-Xarch_host", "-fsanitize=address",
                               "-Xarch_host", "-fno-omit-frame-pointer"],
             ["-Xarch_host", "-fsanitize=address"]),
}


def asan_runtime():
    """Path of the AddressSanitizer runtime that librf_asan.so needs preloaded."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    return r.stdout.strip()


def _compile(src, verbose, variant=None):
    build = BUILD if variant is None else os.path.join(BUILD, variant)
    obj = os.path.join(build, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *VARIANTS[variant][1], *EXTRA.get(os.path.basename(src), []),
           "-x", "hip", "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr)
    # The host pass does not know the gfx feature flag; that note is noise.
    out = "\n".join(l for l in out.splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if out and verbose:
        print(out)
    return obj


def build(verbose=False, jobs=None, variant=None):
    name, _, link_flags = VARIANTS[variant]
    lib = os.path.join(PKG, name)
    os.makedirs(BUILD if variant is None else os.path.join(BUILD, variant), exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, variant), srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *link_flags, *objs,
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)
    return lib


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", "-v", action="store_true")
    g = ap.add_mutually_exclusive_group()
    g.add_argument("--poison", action="store_true")
    g.add_argument("--asan", action="store_true")
    a = ap.parse_args(argv)
    print(build(verbose=a.verbose,
                variant="poison" if a.poison else "asan" if a.asan else None))


if __name__ == "__main__":
    sys.exit(main())
