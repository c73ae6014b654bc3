"""Host-side logic of bench.py: the algorithmic byte count, the source hash
that keys the recorded HBM traffic, and the one-GPU guard (no GPU needed)."""
import json
import os
import subprocess
import sys

import bench
from synth import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_per_step_by_hand():
    # opt30b: U = 64 * 56 units, k = 410 slots, d = 128, bf16
    U, k, d = 3584, 410, 128
    kv = U * k * d * 2 * 2          # every live K and V row
    score = U * k * 8               # score read and write
    new = U * 3 * d * 2             # q, k, v of the decoded token
    out = U * d * 4                 # fp32 output
    admit = U * (2 * d * 2 + 8)     # one admitted row (K, V, score, position)
    ev = U * 4                      # evicted position
    assert bench.alg_bytes_per_step(WORKLOADS["opt30b"]) == kv + score + new + out + admit + ev == 770_574_336
    # E4M3 cache: one byte per element plus a float32 scale per K row and per V row
    kvq = U * k * (d * 2 + 8)
    admit_q = U * (2 * d + 8 + 8)
    assert bench.alg_bytes_per_step(WORKLOADS["opt30b"], "e4m3") == \
        kvq + score + new + out + admit_q + ev == 405_264_384


def test_prefill_flops_count_the_causal_triangle():
    wl = WORKLOADS["opt30b"]
    # P(P+1)/2 dot products of length d, 2 flops each, per unit
    assert bench.prefill_flops(wl) == wl.units * (1024 * 1025 // 2) * 128 * 2


def test_source_hash_ignores_comments_and_layout():
    a = "int f(int x) {\n  return x + 1;  // add one\n}\n/* block\n comment */"
    b = "int f(int x) { return x + 1; }"
    c = "int f(int x) { return x + 2; }"
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(b) != bench.code_text(c)


def test_recorded_traffic_is_used_only_for_the_same_source(tmp_path, monkeypatch):
    rec = {"opt30b": {"source_sha256": bench.decode_source_hash(), "decode_waves": 1,
                      "traffic_bytes_per_launch": 123}}
    f = tmp_path / "t.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.traffic_for("opt30b", 1) == 123
    assert bench.traffic_for("opt30b", 2) is None            # another launch shape
    assert bench.traffic_for("opt30b", 1, "e4m3") is None    # another cache format
    rec["opt30b"]["source_sha256"] = "0" * 64
    f.write_text(json.dumps(rec))
    assert bench.traffic_for("opt30b", 1) is None            # counters taken on other code


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "only --gpus 1" in r.stderr


def test_read_probe_library_exports_and_rejects_bad_arguments():
    """The benchmark's streaming-read probe is built beside libh2o and refuses
    invalid arguments before any HIP call."""
    import ctypes
    path = os.path.join(ROOT, "kv_cache_eviction_02_amd", "libh2o_probe.so")
    assert os.path.exists(path), "build the libraries first (python -m kv_cache_eviction_02_amd.build)"
    lib = ctypes.CDLL(path)
    f = lib.h2o_probe_read
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    f.restype = ctypes.c_int
    assert f(None, 1024, 16, 1024, None) == 1          # no source
    assert f(16, 1024, None, 1024, None) == 1          # no sink
    assert f(16, 1000, 16, 1024, None) == 1            # not whole 16-byte chunks
    assert f(24, 1024, 16, 1024, None) == 1            # misaligned source
    assert f(16, 1024, 16, 0, None) == 1               # no workgroups
