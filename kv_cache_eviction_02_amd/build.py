"""Build step of the H2O library: compiles the HIP kernels and the C ABI into
kv_cache_eviction_02_amd/libh2o.so for gfx950 with hipcc, and the benchmark's
streaming-read probe (not part of the H2O path) into libh2o_probe.so.

    python -m kv_cache_eviction_02_amd.build
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libh2o.so")
SOURCES = ["h2o_api.cpp", "decode.hip", "prefill.hip", "prefill_no_alloc.hip"]
PROBE_LIB = os.path.join(PKG, "libh2o_probe.so")
PROBE_SOURCES = ["read_probe.hip"]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(sources, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-function",
           # keep the compiler from forming packed fp32 instructions
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in sources], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    if verbose and errs:
        print("\n".join(errs), file=sys.stderr)
    os.replace(tmp, lib)
    return lib


def build(verbose=False) -> str:
    """Compile libh2o.so and the benchmark's probe library; returns libh2o.so's path."""
    _compile(SOURCES, LIB, verbose)
    _compile(PROBE_SOURCES, PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
