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


# Per-source flags.  The prefill kernels never form a NaN (masked logits are
# -inf, running maxima start finite), so max() needs no NaN quieting there.
EXTRA_FLAGS = {"prefill.hip": ["-fno-honor-nans"]}
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          # keep the compiler from forming packed fp32 instructions
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    if verbose and errs:
        print("\n".join(errs), file=sys.stderr)


def _compile(sources, lib, verbose):
    """Each source to an object (in parallel), then one shared library."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = [os.path.join(objdir, os.path.basename(lib) + "." + src + ".o") for src in sources]

    def one(i):
        src = sources[i]
        cmd = [hipcc(), f"--offload-arch={ARCH}", *COMMON, *EXTRA_FLAGS.get(src, []), *inc, "-c",
               os.path.join(CSRC, src), "-o", objs[i]]
        _run(cmd, verbose)

    with ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        list(ex.map(one, range(len(sources))))
    tmp = lib + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, lib)
    return lib


def build(verbose=False) -> str:
    """Compile libh2o.so and the benchmark's probe library; returns libh2o.so's path."""
    _compile(SOURCES, LIB, verbose)
    _compile(PROBE_SOURCES, PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
