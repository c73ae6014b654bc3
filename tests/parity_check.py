"""Per-unit comparison of one GPU decode step with the float64 oracle.

Torch-free (numpy, the oracle and the input generator only), so the same check
runs in the test process and in worker processes that never touch the GPU.
The protocol and tolerances are stated in tests/parity.py.
"""
import math
import os

import numpy as np

from oracle import decode_step, dequantize_row_e4m3, members_from_slots, prefill, quantize_row_e4m3
from synth import gen


def ulp32(x):
    x = abs(float(x))
    if x == 0.0:
        return 2.0 ** -149
    return 2.0 ** (math.floor(math.log2(x)) - 23)


def near_tie_tau(lo):
    """Two candidates closer than this may be evicted in either order: the
    literal 1e-5 of the parity bar, or 4 ulp of the lowest score where the fp32
    rounding of the GPU's own score += p alone exceeds it."""
    return max(1e-5, 4 * ulp32(lo))


class Stats:
    """Counts and worst errors of a parity run.

    steps           decode steps checked (each over all sampled units);
    unit_steps      (unit, step) pairs checked;
    near_ties       steps where the GPU's victim differed from the oracle's
                    within the near-tie exemption;
    close_calls     steps whose two lowest candidates were within the
                    exemption's tau (whatever the GPU chose);
    heavy_evictions steps whose victim was not the position leaving the
                    protected window (t - recent): the accumulated-score
                    re-ranking changed a heavy member."""
    FIELDS = ("steps", "unit_steps", "near_ties", "close_calls", "heavy_evictions", "prefill_near_ties",
              "prompt_out_rows")
    MAXES = ("max_out_rel", "max_score_rel", "prompt_out_err_over_tol")

    def __init__(self):
        for f in self.FIELDS:
            setattr(self, f, 0)
        for f in self.MAXES:
            setattr(self, f, 0.0)

    def merge(self, d):
        for f in self.FIELDS:
            setattr(self, f, getattr(self, f) + d.get(f, 0))
        for f in self.MAXES:
            setattr(self, f, max(getattr(self, f), d.get(f, 0.0)))

    def as_dict(self):
        return {f: getattr(self, f) for f in self.FIELDS + self.MAXES}

    def __repr__(self):
        parts = [f"{f}={getattr(self, f)}" for f in self.FIELDS]
        parts += [f"{f}={getattr(self, f):.3g}" for f in self.MAXES]
        return "Stats(" + ", ".join(parts) + ")"


def unit_inputs(wl, u, n_pos, cache_kind):
    """Exact input values of unit u for positions [0, n_pos), and for an E4M3
    cache the stored (dequantized) rows and the codes and scales of every row."""
    b, h = divmod(u, wl.heads)
    vals = gen.unit_values(wl, b, h, 0, n_pos)
    cached, quant = (None, None), None
    if cache_kind == "e4m3":
        qk = [quantize_row_e4m3(row) for row in vals[1]]
        qv = [quantize_row_e4m3(row) for row in vals[2]]
        quant = (np.array([c for c, _ in qk]), np.array([s for _, s in qk], np.float32),
                 np.array([c for c, _ in qv]), np.array([s for _, s in qv], np.float32))
        cached = (np.array([dequantize_row_e4m3(c, s) for c, s in qk]),
                  np.array([dequantize_row_e4m3(c, s) for c, s in qv]))
    return vals, cached, quant


def check_unit_step(wl, policy, vals, cached, t, pos_b, score_b, out, ev, pos_a, score_a, unit=None):
    """Check one unit's step at position t: the oracle, fed the GPU's incoming
    state (pos_b, score_b), against the GPU's output, eviction and outgoing
    state (pos_a, score_a).  Returns this step's counts as a dict."""
    r, h = wl.recent, wl.heavy
    Q, K, V = vals
    Kc, Vc = cached
    members = members_from_slots(pos_b, score_b)
    res = decode_step(members, t, Q[t], K, V, r, h, wl.scale, Kc, Vc, policy)
    d = {"unit_steps": 1}
    scale_o = np.abs(res.out).max()
    err_o = np.abs(out - res.out).max()
    assert err_o <= 2e-3 * scale_o, (unit, t, err_o, scale_o)
    d["max_out_rel"] = float(err_o / scale_o)

    expected = dict(res.members)
    got_ev = int(ev)
    if res.evicted is not None and policy != "static":
        keep = 0.0 if policy == "naive" else 1.0
        pre = {j: keep * members[j] + res.weights[j] for j in members}
        pre[t] = res.weights[t]
        cands = sorted((sc, j) for j, sc in pre.items() if j <= t - r)
        if len(cands) > 1 and cands[1][0] - cands[0][0] < near_tie_tau(cands[0][0]):
            d["close_calls"] = 1
    if res.evicted is None:
        assert got_ev == -1, (unit, t, got_ev)
    elif got_ev != res.evicted:
        # the static victim is fixed by positions alone: no tolerance
        assert policy != "static", (unit, t, got_ev, res.evicted)
        lo = cands[0][0]
        assert len(cands) > 1 and cands[1][0] - lo < near_tie_tau(lo), (unit, t, got_ev, res.evicted, cands[:3])
        assert got_ev in pre and got_ev <= t - r and pre[got_ev] - lo < near_tie_tau(lo), (unit, t, got_ev)
        del expected[got_ev]
        expected[res.evicted] = pre[res.evicted]
        d["near_ties"] = 1
    if got_ev >= 0 and got_ev != t - r:
        d["heavy_evictions"] = 1
    got = members_from_slots(pos_a, score_a)
    assert set(got) == set(expected), (unit, t, sorted(set(got) ^ set(expected)))
    worst = 0.0
    for j, sc in got.items():
        ref = expected[j]
        err = abs(sc - ref)
        assert err <= 2e-3 * ref + 1e-6, (unit, t, j, sc, ref)
        if ref > 1e-3:
            worst = max(worst, err / ref)
    d["max_score_rel"] = worst
    return d


def check_unit_prefill(wl, policy, vals, pos, score, unit=None):
    """Check one unit's cache state after the prefill against the oracle's
    prefill: ring slots hold the newest positions, the kept set is exact except
    for positions whose score lies within tau_pre of the h-th largest score c_h
    among the older positions, and every kept score is within the score bar."""
    P, r, h = wl.prompt, wl.recent, wl.heavy
    Q, K, _ = vals
    ref, c = prefill(Q[:P], K[:P], r, h, wl.scale, policy)
    got = members_from_slots(pos, score)
    d = {}
    for p in range(P - min(P, r), P):
        assert pos[p % r] == p, (unit, p)
    if set(got) != set(ref):
        assert P > r + h, (unit, sorted(set(got) ^ set(ref)))
        c_h = np.sort(c[:P - r])[::-1][h - 1]
        tau = prefill_tau(c_h)
        for j in set(got) ^ set(ref):
            assert abs(c[j] - c_h) <= tau, (unit, j, c[j], c_h, tau)
        assert len(got) == len(ref)
        d["prefill_near_ties"] = 1
    worst = 0.0
    for j, sc in got.items():
        err = abs(sc - c[j])
        assert err <= 2e-3 * c[j] + 1e-6, (unit, j, sc, c[j])
        worst = max(worst, err / max(c[j], 1e-30))
    d["max_score_rel"] = worst
    return d


def prefill_tau(c_h):
    """Near-tie band of the prefill selection at the h-th largest score c_h:
    the literal 1e-5, or 1e-5 relative where fp32 column sums of up to P terms
    in another order than the oracle's can differ by more."""
    return max(1e-5, 1e-5 * c_h)


def check_unit_rows(wl, cache_kind, bits, quant, pos, krows, vrows, kscale=None, vscale=None, unit=None):
    """Every live slot's K and V row equals the input row of the position it
    claims, bit for bit (E4M3: the codes and scale of that row's quantization)."""
    live = np.flatnonzero(pos >= 0)
    p = pos[live]
    if cache_kind == "e4m3":
        qkc, qks, qvc, qvs = quant
        np.testing.assert_array_equal(krows[live], qkc[p], err_msg=f"unit {unit} K codes")
        np.testing.assert_array_equal(vrows[live], qvc[p], err_msg=f"unit {unit} V codes")
        np.testing.assert_array_equal(kscale[live], qks[p], err_msg=f"unit {unit} K scales")
        np.testing.assert_array_equal(vscale[live], qvs[p], err_msg=f"unit {unit} V scales")
        return
    _, Kb, Vb = bits
    np.testing.assert_array_equal(krows[live], Kb[p], err_msg=f"unit {unit} K rows")
    np.testing.assert_array_equal(vrows[live], Vb[p], err_msg=f"unit {unit} V rows")


# ---- worker side of the pooled check ------------------------------------------------

_UNITS = {}
_KEEP = 4   # units whose inputs a worker keeps (about 14 MB each at the largest workload)


def _inputs(wl, u, n_pos, cache_kind):
    key = (wl, u, n_pos, cache_kind)
    if key not in _UNITS:
        if len(_UNITS) >= _KEEP:
            _UNITS.pop(next(iter(_UNITS)))
        b, h = divmod(u, wl.heads)
        vals, cached, quant = unit_inputs(wl, u, n_pos, cache_kind)
        _UNITS[key] = (vals, cached, quant, gen.unit_storage(wl, b, h, 0, n_pos))
    return _UNITS[key]


def pooled_task(kind, wl, u, n_pos, cache_kind, policy, payload):
    """One check of unit u in a worker process, on inputs regenerated from the
    seeds.  kind "steps": payload = [(t, pos_b, score_b, out, ev, pos_a,
    score_a)] over consecutive steps; "prefill": (pos, score); "rows": (pos,
    krows, vrows, kscale, vscale).  Returns ("ok", counts) or ("fail", message)."""
    vals, cached, quant, bits = _inputs(wl, u, n_pos, cache_kind)
    st = Stats()
    try:
        if kind == "steps":
            for rec in payload:
                st.merge(check_unit_step(wl, policy, vals, cached, *rec, unit=u))
        elif kind == "prefill":
            st.merge(check_unit_prefill(wl, policy, vals, *payload, unit=u))
        elif kind == "rows":
            check_unit_rows(wl, cache_kind, bits, quant, *payload, unit=u)
        else:
            raise ValueError(kind)
    except AssertionError as e:
        return ("fail", f"{kind} unit {u}: {e!r}"[:4000])
    return ("ok", st.as_dict())


def pool_workers():
    """Worker processes for the pooled check: the host's cores, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))
