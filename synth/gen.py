"""Seeded synthetic queries, keys and values for the H2O workloads.

Shared by the CPU oracle's tests and the GPU path's tests and benchmark: both
sides consume exactly the same bytes.  Nothing here computes any part of the
H2O method; it only draws inputs.

Recipe (one (batch b, head h) stream at a time, so any unit can be regenerated
on its own, and any range of positions can be drawn without the rest):

* z ~ N(0, 1) i.i.d. float32, drawn in blocks of 4096 positions; block ``i`` of
  tensor ``x`` of unit (b, h) of workload ``c`` uses numpy PCG64 seeded with
  ``SeedSequence([BASE_SEED, c, b, h, x, i])``.
* A skew direction u_h (unit vector, one per head index, shared across the
  batch) makes the attention mass uneven: every query gets ``+1.5 u_h`` and
  key ``p`` gets ``+a_p u_h``.  ``a_p`` depends on the workload:

  - "fraction": ``a_p = 3`` on round(frac * N) positions drawn without
    replacement from all N = prompt + steps positions, else 0;
  - "zipf": ranks rho = a random permutation of 1..N; ``a_p = alpha *
    ln(N / rho_p) / (1.5 * scale)``, so the logit boost is alpha*ln(N/rho) and
    the expected attention multiplier is (N/rho)^alpha (power law in rank);
  - "bursts": round(frac * N / 16) distinct aligned blocks of 16 consecutive
    positions get ``a_p = 3``;
  - "zipf_periodic": as "zipf" over one period (5000 positions) and repeated,
    so the same heavy positions recur every period.

* Values carry no skew.  bf16 workloads round q, k, v to bfloat16
  (round-to-nearest-even) after the skew is added.
"""
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

from .configs import Workload

BASE_SEED = 230614048
BLOCK = 4096
T_Q, T_K, T_V, T_U, T_SKEW = 0, 1, 2, 3, 4


def _rng(*key):
    return np.random.default_rng(np.random.SeedSequence([BASE_SEED, *key]))


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    Inputs here are finite and far from the float32 range limits."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = bits + np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def skew_direction(wl: Workload, head: int) -> np.ndarray:
    g = _rng(wl.cid, head, T_U).standard_normal(wl.head_dim)
    return (g / np.linalg.norm(g)).astype(np.float32)


def skew_amplitudes(wl: Workload, b: int, h: int) -> np.ndarray:
    """a_p for every position 0..N-1 of unit (b, h), float32."""
    n = wl.n_positions
    rng = _rng(wl.cid, b, h, T_SKEW)
    a = np.zeros(n, dtype=np.float64)
    if wl.skew == "fraction":
        cnt = int(round(wl.skew_frac * n))
        a[rng.choice(n, size=cnt, replace=False)] = wl.skew_amp
    elif wl.skew == "zipf":
        rho = rng.permutation(n) + 1
        a = wl.zipf_alpha * np.log(n / rho) / (wl.query_amp * wl.scale)
    elif wl.skew == "bursts":
        nblk = n // wl.burst_len
        cnt = int(round(wl.skew_frac * n / wl.burst_len))
        for blk in rng.choice(nblk, size=cnt, replace=False):
            a[blk * wl.burst_len:(blk + 1) * wl.burst_len] = wl.skew_amp
    elif wl.skew == "zipf_periodic":
        rho = rng.permutation(wl.period) + 1
        per = wl.zipf_alpha * np.log(wl.period / rho) / (wl.query_amp * wl.scale)
        a = per[np.arange(n) % wl.period]
    else:
        raise ValueError(f"unknown skew {wl.skew!r}")
    return a.astype(np.float32)


def _gauss(wl: Workload, b: int, h: int, tensor: int, p0: int, p1: int) -> np.ndarray:
    d = wl.head_dim
    out = np.empty((p1 - p0, d), dtype=np.float32)
    blk = p0 // BLOCK
    while blk * BLOCK < p1:
        z = _rng(wl.cid, b, h, tensor, blk).standard_normal((BLOCK, d), dtype=np.float32)
        lo, hi = max(p0, blk * BLOCK), min(p1, (blk + 1) * BLOCK)
        out[lo - p0:hi - p0] = z[lo - blk * BLOCK:hi - blk * BLOCK]
        blk += 1
    return out


def unit_raw(wl: Workload, b: int, h: int, p0: int, p1: int):
    """Q, K, V of unit (b, h) for positions [p0, p1) before any rounding."""
    if not (0 <= p0 <= p1 <= wl.n_positions):
        raise ValueError("position range outside the workload")
    u = skew_direction(wl, h)
    a = skew_amplitudes(wl, b, h)[p0:p1]
    q = _gauss(wl, b, h, T_Q, p0, p1) + np.float32(wl.query_amp) * u[None, :]
    k = _gauss(wl, b, h, T_K, p0, p1) + a[:, None] * u[None, :]
    v = _gauss(wl, b, h, T_V, p0, p1)
    return q, k, v


def unit_storage(wl: Workload, b: int, h: int, p0: int, p1: int):
    """Q, K, V of one unit as stored on the device: float32 arrays for "f32"
    workloads, bfloat16 bit patterns (uint16) for "bf16" ones."""
    q, k, v = unit_raw(wl, b, h, p0, p1)
    if wl.kv_dtype == "bf16":
        return round_to_bf16_bits(q), round_to_bf16_bits(k), round_to_bf16_bits(v)
    return q, k, v


def unit_values(wl: Workload, b: int, h: int, p0: int, p1: int):
    """Q, K, V of one unit as the exact float64 values of the stored elements."""
    out = []
    for x in unit_storage(wl, b, h, p0, p1):
        if x.dtype == np.uint16:
            x = bf16_bits_to_f32(x)
        out.append(x.astype(np.float64))
    return tuple(out)


def batch_storage(wl: Workload, p0: int, p1: int, units=None, threads=None):
    """Q, K, V for all units (or a list of (b, h) units) and positions [p0, p1).

    Returns three arrays shaped [B, H, p1-p0, d] (or [len(units), p1-p0, d]),
    uint16 bf16 bits or float32."""
    dt = np.uint16 if wl.kv_dtype == "bf16" else np.float32
    if units is None:
        shape = (wl.batch, wl.heads, p1 - p0, wl.head_dim)
        todo = [(b, h) for b in range(wl.batch) for h in range(wl.heads)]
    else:
        todo = list(units)
        shape = (len(todo), p1 - p0, wl.head_dim)
    arrs = [np.empty(shape, dtype=dt) for _ in range(3)]
    flat = [x.reshape(-1, p1 - p0, wl.head_dim) for x in arrs]

    def work(i):
        b, h = todo[i]
        for dst, src in zip(flat, unit_storage(wl, b, h, p0, p1)):
            dst[i] = src

    n = threads or min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(max_workers=n) as ex:
        list(ex.map(work, range(len(todo))))
    return tuple(arrs)
