#!/usr/bin/env python3
"""Decode-step throughput of the H2O hot path on one MI355X.

A step is one decode step over the whole batch of a workload: attention over
the k cached slots plus the new token for every (batch, head) unit, score
accumulation, eviction and admission.  Inputs are seeded synthetic tensors
already resident in HBM before the timed region; the prefill that seeds the
cache runs (and is timed) separately.

Prints one JSON line.  `value` is decode steps/s over the timed region (HIP
events on the stream the kernel runs on, synchronised on both sides);
`roofline` reports the decode kernel's algorithmic bytes per launch divided by
its mean launch duration over that region (one launch per step) against the
8 TB/s HBM peak; `cpu_baseline` is the float64 oracle timed on the host's cores on a
bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload opt30b] [--no-cpu-baseline]
"""
import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from synth import WORKLOADS, HEADLINE  # noqa: E402

METRIC = "H2O decode steps/s + achieved HBM GB/s (% peak), OPT-30B-shape heads, 20% KV"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_MFMA_TFLOPS = 157.3
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
DECODE_SOURCES = ["kv_cache_eviction_02_amd/csrc/decode.hip", "kv_cache_eviction_02_amd/csrc/common.h"]


def alg_bytes_per_step(wl, cache="input"):
    """Bytes one decode step must move at minimum: every live K and V row, the
    score read and write, q/k/v of the new token, the fp32 output, one admitted
    row (K, V, score, position) and the evicted position.  An E4M3 cache stores
    one byte per element plus a float32 scale per K row and per V row."""
    U, k, d, e = wl.units, wl.k, wl.head_dim, wl.elem_bytes
    if cache == "e4m3":
        return (U * k * (d * 2 + 8) + U * k * 8 + U * 3 * d * e + U * d * 4
                + U * (2 * d + 8 + 8) + U * 4)
    return (U * k * d * e * 2 + U * k * 8 + U * 3 * d * e + U * d * 4
            + U * (2 * d * e + 8) + U * 4)


PREFILL_CALLS = 7  # warm prefills timed back to back; the mean per call is reported


def prefill_flops(wl):
    """Causal QK^T of the prompt: P(P+1)/2 dot products of length d per unit."""
    P = wl.prompt
    return wl.units * P * (P + 1) * wl.head_dim


def code_text(src):
    """Source text without comments and whitespace: what the compiler sees."""
    import re
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def decode_source_hash():
    """Hash of the decode sources' code (comments and layout ignored)."""
    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()


def traffic_for(wl_name, waves, cache="input"):
    """Measured HBM bytes per decode launch, if recorded for the current source
    (records are keyed by workload, with "/e4m3" appended for an E4M3 cache)."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    ent = rec.get(wl_name if cache == "input" else f"{wl_name}/{cache}")
    if not ent or ent.get("source_sha256") != decode_source_hash() or ent.get("decode_waves") != waves:
        return None
    return ent.get("traffic_bytes_per_launch")


# ---- CPU baseline: the oracle on the host cores (runs before any GPU use) -------

def _oracle_worker(args):
    wl_name, prompt, recent, heavy, policy, units, steps, blas_threads = args
    import dataclasses as dc
    from threadpoolctl import threadpool_limits
    from oracle import decode_step, prefill
    from synth import WORKLOADS as W, gen
    wl = dc.replace(W[wl_name], prompt=prompt, recent=recent, heavy=heavy)
    with threadpool_limits(blas_threads):
        data = []
        pre_s = 0.0
        for u in units:
            b, h = divmod(u, wl.heads)
            Q, K, V = gen.unit_values(wl, b, h, 0, wl.prompt + steps)
            tp = time.perf_counter()
            m, _ = prefill(Q[:wl.prompt], K[:wl.prompt], wl.recent, wl.heavy, wl.scale, policy)
            pre_s += time.perf_counter() - tp
            data.append((Q, K, V, m))
        t0 = time.perf_counter()
        for Q, K, V, m in data:
            for s in range(steps):
                t = wl.prompt + s
                m = decode_step(m, t, Q[t], K, V, wl.recent, wl.heavy, wl.scale, policy=policy).members
        dt = time.perf_counter() - t0
    return len(units) * steps, dt, len(units), pre_s


def host_cpu():
    """(cores this process may run on, CPU model name from /proc/cpuinfo)."""
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return len(os.sched_getaffinity(0)), model


def cpu_baseline(wl, units_per_worker, steps, policy="h2o"):
    """The oracle on every core of the host: at most 16 worker processes (one
    per unit sample share), each with host_cores // workers BLAS threads."""
    import multiprocessing as mp
    host_cores, model = host_cpu()
    workers = min(16, host_cores)
    blas = max(1, host_cores // workers)
    stride = max(1, wl.units // (workers * units_per_worker))
    chosen = list(range(0, wl.units, stride))[:workers * units_per_worker]
    jobs = [(wl.name, wl.prompt, wl.recent, wl.heavy, policy, chosen[i::workers], steps, blas)
            for i in range(workers)]
    jobs = [j for j in jobs if j[5]]
    with mp.get_context("fork").Pool(len(jobs)) as pool:
        res = pool.map(_oracle_worker, jobs)
    unit_steps_per_s = sum(n / dt for n, dt, _, _ in res)
    cpu_work = sum(dt for _, dt, _, _ in res)
    # oracle prefill: per-unit time on one worker, scaled to the whole batch over the workers
    pre_unit_s = sum(ps for _, _, _, ps in res) / sum(nu for _, _, nu, _ in res)
    return {
        "value": unit_steps_per_s / wl.units,
        "unit": "steps/s",
        "cores": len(jobs) * blas,
        "kind": "oracle",
        "host_cores": host_cores,
        "processes": len(jobs),
        "blas_threads_per_process": blas,
        "cpu_model": model,
        "prefill_s": pre_unit_s * wl.units / len(jobs),
        "sample": (f"{len(chosen)} of {wl.units} (batch, head) units x {steps} decode steps "
                   f"after an untimed oracle prefill, float64 numpy, {len(jobs)} processes with "
                   f"{blas} BLAS thread(s) each on {host_cores} host cores; {cpu_work:.1f} s of "
                   f"CPU time; rate scaled to whole-batch steps/s; host CPU: {model}"),
    }


def rocminfo_record():
    """Fields of the first gfx agent in rocminfo's listing (name, clocks and unit
    counts), read before any GPU use in this process; {} when unavailable."""
    import subprocess
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError):
        return {}
    keys = {"Marketing Name": "marketing_name", "Max Clock Freq. (MHz)": "max_clock_mhz",
            "Compute Unit": "compute_units", "SIMDs per CU": "simds_per_cu",
            "Wavefront Size": "wavefront_size", "Max Waves Per CU": "max_waves_per_cu",
            "Shader Engines": "shader_engines"}
    for agent in txt.split("Agent ")[1:]:
        if "gfx9" not in agent or "Device Type:" not in agent or "GPU" not in agent.split("Device Type:")[1][:20]:
            continue
        rec = {}
        for line in agent.splitlines():
            k, _, v = line.strip().partition(":")
            if k.strip() in keys and keys[k.strip()] not in rec:
                v = v.strip().split("(")[0].strip()
                rec[keys[k.strip()]] = int(v) if v.isdigit() else v
        return rec
    return {}


def smi_clocks():
    """Current and top shader and memory clocks reported by rocm-smi (MHz), or {}."""
    import re
    import subprocess
    try:
        txt = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError):
        return {}
    rec = {}
    for name, key in (("sclk", "sclk_mhz"), ("mclk", "mclk_mhz"), ("fclk", "fclk_mhz")):
        m = re.search(rf"{name} clock level:\s*\d+:\s*\(?(\d+)\s*Mhz", txt, re.I)
        if m:
            rec[key] = int(m.group(1))
    return rec


# ---- GPU -----------------------------------------------------------------------

def read_ceiling(stream, gib=4, reps=3):
    """Best HBM read rate (GB/s) of the streaming-read probe (libh2o_probe.so,
    16-byte non-temporal loads, grid-stride) over `gib` GiB, and the workgroup
    count that reached it; None when the probe library is not built."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "kv_cache_eviction_02_amd", "libh2o_probe.so")
    if not os.path.exists(path):
        print(f"[bench] {path} missing: no read ceiling", file=sys.stderr, flush=True)
        return None
    lib = ctypes.CDLL(path)
    lib.h2o_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                   ctypes.c_void_p]
    lib.h2o_probe_read.restype = ctypes.c_int
    nbytes = gib << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    src.fill_(1)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    assert src.data_ptr() % 16 == 0 and nbytes % 16 == 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = (0.0, 0)
    # up to one 16-byte load per thread (2^20 workgroups over 4 GiB), the best shape measured
    for blocks in (4096, 16384, 65536, 262144, 1 << 20):
        def run():
            st = lib.h2o_probe_read(src.data_ptr(), nbytes, sink.data_ptr(), blocks, stream.cuda_stream)
            if st != 0:
                raise RuntimeError(f"h2o_probe_read returned {st}")
        run()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        gbs = reps * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
        best = max(best, (gbs, blocks))
    del src, sink
    return best


def time_torch_flash_attention(prompt, scale, stream, reps=5):
    """Mean time (ms) of torch's flash-attention forward, causal, over the same prompt
    q, k, v ([B, H, P, d] bf16): a measured reference for the prompt-output prefill.
    Only the flash backend is allowed, so nothing falls back to batched products;
    None when that backend is not available."""
    import torch
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel
    q, k, v = prompt
    try:
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            o = F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=scale)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                o = F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=scale)
            e1.record(stream)
            torch.cuda.synchronize()
        del o
        return e0.elapsed_time(e1) / reps
    except RuntimeError as ex:
        print(f"[bench] torch flash attention unavailable: {ex}", file=sys.stderr, flush=True)
        return None


def run_gpu(wl, steps, warmup, waves, copy_mib=0, single_calls=False, split=0, cache="input",
            policy="h2o", streaming=True):
    import torch
    from kv_cache_eviction_02_amd import H2OCache
    from kv_cache_eviction_02_amd.binding import load_library
    from synth.stage import stage_decode, stage_prompt

    load_library()
    dev = "cuda:0"
    torch.cuda.set_device(0)
    dtype = torch.bfloat16 if wl.kv_dtype == "bf16" else torch.float32
    t0 = time.time()
    prompt = stage_prompt(wl, dev)
    dq, dk, dv = stage_decode(wl, 0, warmup + steps, dev)
    torch.cuda.synchronize()
    print(f"[bench] staged inputs in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)

    cache_kind = cache
    # one launch per step, as an autoregressive decoder runs it
    cache = H2OCache(wl.batch, wl.heads, wl.head_dim, wl.recent, wl.heavy, wl.prompt, dtype,
                     wl.scale, device=dev, decode_waves=waves, decode_split=split, cache=cache,
                     policy=policy, steps_mode="per_step")
    stream = torch.cuda.current_stream()
    # The first prefill also loads the kernels' code objects; the warm ones that
    # follow, each rebuilding the same state from the same prompt, are timed
    # one by one and the median is reported (one call varies with the clock).
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    # Back to back, like the decode steps and torch's attention below: the host's
    # enqueueing of one call overlaps the GPU's work on the one before.
    def mean_prefill_ms(**kw):
        cache.prefill(*prompt, **kw)
        torch.cuda.synchronize()
        p0.record(stream)
        for _ in range(PREFILL_CALLS):
            cache.prefill(*prompt, **kw)
        p1.record(stream)
        torch.cuda.synchronize()
        return p0.elapsed_time(p1) / PREFILL_CALLS

    prefill_ms = mean_prefill_ms()
    # The prefill that also returns the prompt's attention output.
    prompt_out = torch.empty((wl.batch, wl.heads, wl.prompt, wl.head_dim), dtype=torch.float32, device=dev)
    prefill_out_ms = mean_prefill_ms(out=prompt_out)
    del prompt_out
    # torch's own causal flash attention over the same prompt, for context (not in
    # counter runs, whose only copies calibrate the byte counters)
    sdpa_ms = time_torch_flash_attention(prompt, wl.scale, stream) \
        if wl.kv_dtype == "bf16" and not copy_mib else None
    prompt_keep = prompt if streaming and not single_calls else None
    del prompt

    for s in range(warmup):
        cache.step(dq[s], dk[s], dv[s])
    out_all = torch.empty((steps, wl.batch, wl.heads, wl.head_dim), dtype=torch.float32, device=dev)
    ev_all = torch.empty((steps, wl.batch, wl.heads), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    r0.record(stream)
    if single_calls:
        for i in range(steps):
            s = warmup + i
            cache.step(dq[s], dk[s], dv[s])
    else:
        cache.steps(dq[warmup:warmup + steps], dk[warmup:warmup + steps], dv[warmup:warmup + steps],
                    out=out_all, evicted=ev_all)
    r1.record(stream)
    torch.cuda.synchronize()
    region_ms = r0.elapsed_time(r1)
    stream_ms = resident_ms = None
    if streaming and not single_calls:
        # the same steps as one persistent launch (known tokens, as in a long-stream run);
        # h2o_decode_steps picks it by itself for small batches (steps_mode "auto")
        pc = H2OCache(wl.batch, wl.heads, wl.head_dim, wl.recent, wl.heavy, wl.prompt, dtype,
                      wl.scale, device=dev, decode_waves=waves, decode_split=split, cache=cache_kind,
                      policy=policy, steps_mode="persistent")
        pc.prefill(*prompt_keep)
        if warmup:
            pc.steps(dq[:warmup], dk[:warmup], dv[:warmup])
        torch.cuda.synchronize()
        r0.record(stream)
        pc.steps(dq[warmup:warmup + steps], dk[warmup:warmup + steps], dv[warmup:warmup + steps],
                 out=out_all, evicted=ev_all)
        r1.record(stream)
        torch.cuda.synchronize()
        stream_ms = r0.elapsed_time(r1)
        pc.close()
        # the same steps with every unit's rows held in LDS across them, when they fit
        rc = H2OCache(wl.batch, wl.heads, wl.head_dim, wl.recent, wl.heavy, wl.prompt, dtype,
                      wl.scale, device=dev, decode_waves=waves, decode_split=split, cache=cache_kind,
                      policy=policy, steps_mode="resident")
        rc.prefill(*prompt_keep)
        if warmup:
            rc.steps(dq[:warmup], dk[:warmup], dv[:warmup])
        if steps > 1 and rc.steps_launch(steps) == "resident":
            torch.cuda.synchronize()
            r0.record(stream)
            rc.steps(dq[warmup:warmup + steps], dk[warmup:warmup + steps], dv[warmup:warmup + steps],
                     out=out_all, evicted=ev_all)
            r1.record(stream)
            torch.cuda.synchronize()
            resident_ms = r0.elapsed_time(r1)
        rc.close()
    del prompt_keep
    copy_gbs = None
    if not copy_mib:
        # device-to-device copy of 2 GiB, as a measured ceiling for context (left out of
        # counter runs, whose copies calibrate the byte counters)
        xc = torch.empty(1 << 30, dtype=torch.int16, device=dev)
        yc = torch.empty_like(xc)
        xc.fill_(1)
        yc.copy_(xc)
        torch.cuda.synchronize()
        r0.record(stream)
        for _ in range(5):
            yc.copy_(xc)
        r1.record(stream)
        torch.cuda.synchronize()
        copy_gbs = 5 * 2 * xc.numel() * 2 / (r0.elapsed_time(r1) * 1e-3) / 1e9
        del xc, yc
        read_best = read_ceiling(stream)
    else:
        read_best = None
    if copy_mib:
        # plain device copy of known size, for scaling the HBM byte counters
        x = torch.empty(copy_mib << 20, dtype=torch.uint8, device=dev)
        y = torch.empty_like(x)
        x.fill_(1)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        del x, y
    waves_used, split_used = cache.launch_shape()
    cache.close()
    props = torch.cuda.get_device_properties(0)
    device = {"name": torch.cuda.get_device_name(0), "arch": getattr(props, "gcnArchName", ""),
              "compute_units": props.multi_processor_count,
              "memory_gib": round(props.total_memory / 2 ** 30, 1)}
    clock = getattr(props, "clock_rate", None)
    if clock:
        device["clock_mhz"] = clock / 1000
    return dict(region_ms=region_ms, stream_ms=stream_ms, resident_ms=resident_ms, prefill_ms=prefill_ms, prefill_out_ms=prefill_out_ms,
                sdpa_ms=sdpa_ms, read_best=read_best, waves=waves_used, split=split_used, device=device, copy_gbs=copy_gbs)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=24)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(WORKLOADS))
    ap.add_argument("--decode-waves", type=int, default=0)
    ap.add_argument("--cache", default="input", choices=["input", "e4m3"],
                    help="cache rows as the input dtype, or E4M3 codes with per-row scales")
    ap.add_argument("--policy", default="h2o", choices=["h2o", "static", "naive"],
                    help="eviction policy: H2O or one of its ablations")
    ap.add_argument("--heavy-only", action="store_true",
                    help="no protected window: recent = 0, heavy = the workload's k")
    ap.add_argument("--prompt", type=int, default=0, help="override the workload's prompt length")
    ap.add_argument("--budget", default="",
                    help="override the workload's budget as RECENT,HEAVY (e.g. a long context)")
    ap.add_argument("--decode-split", type=int, default=0,
                    help="decode workgroups per (batch, head) unit; 0 = library default")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-streaming", action="store_true",
                    help="skip the persistent-launch timing of the same steps")
    ap.add_argument("--single-step-calls", action="store_true",
                    help="one h2o_decode_step call per step instead of one h2o_decode_steps call")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run a device copy of this size (for counter scaling)")
    ap.add_argument("--no-device-tools", action="store_true",
                    help="skip the rocminfo / rocm-smi records (for runs under a profiler, whose "
                         "preload has already opened the GPU)")
    ap.add_argument("--cpu-units-per-worker", type=int, default=32)
    ap.add_argument("--cpu-steps", type=int, default=128)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the H2O decode path has no cross-GPU exchange "
              "((batch, head) units are independent), so only --gpus 1 is supported.",
              file=sys.stderr)
        sys.exit(2)
    wl = WORKLOADS[args.workload]
    if args.prompt:
        wl = dataclasses.replace(wl, prompt=args.prompt)
    if args.budget:
        r, h = (int(x) for x in args.budget.split(","))
        wl = dataclasses.replace(wl, recent=r, heavy=h)
    if args.heavy_only:
        wl = dataclasses.replace(wl, recent=0, heavy=wl.k)
    modified = bool(args.prompt or args.budget or args.heavy_only)
    steps = max(1, args.steps)
    warmup = max(0, args.warmup)
    if warmup + steps > wl.steps:
        warmup = min(warmup, wl.steps - 1)
        steps = max(1, wl.steps - warmup)
        print(f"[bench] {wl.name} has {wl.steps} decode positions: timing {steps} steps",
              file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        t0 = time.time()
        cpu = cpu_baseline(wl, args.cpu_units_per_worker, min(args.cpu_steps, wl.steps), args.policy)
        print(f"[bench] cpu baseline done in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)

    if args.cache == "e4m3" and wl.kv_dtype != "bf16":
        sys.exit("an E4M3 cache takes bf16 inputs")
    # device listing and clocks from the ROCm tools, in child processes, before this
    # process touches the GPU
    agent = {} if args.no_device_tools else rocminfo_record()
    clocks = {} if args.no_device_tools else smi_clocks()
    g = run_gpu(wl, steps, warmup, args.decode_waves, args.copy_calibration_mib, args.single_step_calls,
                args.decode_split, args.cache, args.policy, not args.no_streaming)
    ms_per_step = g["region_ms"] / steps
    # one decode launch per step: the mean launch duration over the timed region
    mean_launch_ms = ms_per_step
    bytes_step = alg_bytes_per_step(wl, args.cache)
    achieved = bytes_step / (mean_launch_ms * 1e-3) / 1e9
    traffic = traffic_for(wl.name, g["waves"], args.cache) \
        if args.policy == "h2o" and not modified and g["split"] == 1 else None
    line = {
        "metric": METRIC,
        "value": 1e3 / ms_per_step,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.kv_dtype if args.cache == "input" else "bf16 in, e4m3 cache",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "batch": wl.batch, "heads": wl.heads, "head_dim": wl.head_dim,
            "prompt": wl.prompt, "k": wl.k, "recent": wl.recent, "heavy": wl.heavy,
            "kv_dtype": wl.kv_dtype, "cache": args.cache, "policy": args.policy,
            "decode_waves": g["waves"],
            "decode_split": g["split"],
            "launch_shape": "explicit" if args.decode_waves or args.decode_split else "automatic",
            "parallelism": "none",
            "launch": ("h2o_decode_step per step" if args.single_step_calls
                       else "h2o_decode_steps, one launch per step"),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": traffic,
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "kernel": "decode_kernel" if g["split"] == 1 else "decode_split_kernel",
            "alg_bytes_per_launch": bytes_step,
            "mean_launch_us": mean_launch_ms * 1e3,
        },
        "prefill": {
            "ms": g["prefill_ms"],
            "timing": f"mean of {PREFILL_CALLS} warm calls, back to back",
            "qk_tflops": prefill_flops(wl) / (g["prefill_ms"] * 1e-3) / 1e12,
            "peak_tflops": PEAK_BF16_TFLOPS if wl.kv_dtype == "bf16" else PEAK_FP32_MFMA_TFLOPS,
            "frac": prefill_flops(wl) / (g["prefill_ms"] * 1e-3) / 1e12 /
                    (PEAK_BF16_TFLOPS if wl.kv_dtype == "bf16" else PEAK_FP32_MFMA_TFLOPS),
            "with_output": {
                "ms": g["prefill_out_ms"],
                # causal QK^T and PV: each P(P+1)/2 dot products of length d per unit
                "tflops": 2 * prefill_flops(wl) / (g["prefill_out_ms"] * 1e-3) / 1e12,
                "out_bytes": wl.units * wl.prompt * wl.head_dim * 4,
                # the same causal QK^T and PV by torch (no column sums, no selection,
                # bf16 output): a measured reference, not part of the path
                "torch_flash_attention": None if g["sdpa_ms"] is None else {
                    "kind": "torch.nn.functional.scaled_dot_product_attention, flash backend, causal",
                    "ms": g["sdpa_ms"],
                    "tflops": 2 * prefill_flops(wl) / (g["sdpa_ms"] * 1e-3) / 1e12,
                },
            },
        },
        "streaming": None if g["stream_ms"] is None else {
            # the same steps over known tokens in one persistent launch
            "launch": "h2o_decode_steps, one launch for all steps",
            "kernel": "decode_multi_kernel",
            "value": 1e3 * steps / g["stream_ms"],
            "unit": "steps/s",
            "ms_per_step": g["stream_ms"] / steps,
            "achieved": bytes_step * steps / (g["stream_ms"] * 1e-3) / 1e9,
            "frac": bytes_step * steps / (g["stream_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
            # the same steps with the rows held in LDS (one launch; none when they do not fit)
            "resident": None if g["resident_ms"] is None else {
                "kernel": "decode_resident_kernel",
                "value": 1e3 * steps / g["resident_ms"],
                "ms_per_step": g["resident_ms"] / steps,
            },
        },
        "copy_ceiling": None if g["copy_gbs"] is None else {
            "kind": "device-to-device copy, 2 GiB read + 2 GiB written (torch)",
            "GBps": g["copy_gbs"], "frac": g["copy_gbs"] / PEAK_HBM_GBS},
        "read_ceiling": None if g["read_best"] is None else {
            "kind": "hand-written streaming read, 16-byte non-temporal loads, grid-stride, 4 GiB, "
                    "best of 2^12-2^20 workgroups of 256 threads (libh2o_probe.so)",
            "GBps": g["read_best"][0], "frac": g["read_best"][0] / PEAK_HBM_GBS,
            "workgroups": g["read_best"][1],
            "decode_frac_of_ceiling": achieved / g["read_best"][0]},
        "cpu_baseline": cpu,
        "device": {**g["device"], "rocminfo": agent, "clocks": clocks},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
