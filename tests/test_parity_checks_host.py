"""Host-side tests of the parity checks themselves (no GPU).

The GPU's results are stood in for by the oracle's own trajectory laid out in
slots, rounded to float32 as the device stores them; the checks must accept
that and reject each planted mistake.  The pooled variant runs the same checks
in spawned worker processes."""
import numpy as np
import pytest

from oracle import prefill, run_trace
from parity_check import (Stats, check_unit_prefill, check_unit_rows, check_unit_step, pooled_task,
                          unit_inputs)
from synth import WORKLOADS, gen

WL = WORKLOADS["tiny_fp32"]


def slots_of(members, k, r=None, t=None):
    """The library's slot layout of a member set before position t: the r
    newest positions in ring slots p % r, the others in slots r, r + 1, ... in
    ascending order; float32 scores, -1 = empty.  Without t, a plain list."""
    pos = np.full(k, -1, dtype=np.int32)
    score = np.zeros(k, dtype=np.float32)
    nxt = r if t is not None else 0
    for p, sc in sorted(members.items()):
        if t is not None and r and p >= t - r:
            s = p % r
        else:
            s, nxt = nxt, nxt + 1
        pos[s] = p
        score[s] = sc
    return pos, score


def oracle_records(unit, steps):
    vals, cached, _ = unit_inputs(WL, unit, WL.n_positions, "input")
    Q, K, V = vals
    seeded, _, res = run_trace(Q, K, V, WL.prompt, steps, WL.recent, WL.heavy, WL.scale)
    recs = []
    prev = seeded
    for s, r in enumerate(res):
        pb, sb = slots_of(prev, WL.k)
        pa, sa = slots_of(r.members, WL.k)
        ev = -1 if r.evicted is None else r.evicted
        recs.append((WL.prompt + s, pb, sb, r.out.astype(np.float32), ev, pa, sa))
        prev = r.members
    return vals, cached, seeded, recs


def test_step_check_accepts_the_oracle_and_counts_heavy_evictions():
    st = Stats()
    for unit in (0, 1):
        vals, cached, _, recs = oracle_records(unit, WL.steps)
        for rec in recs:
            st.merge(check_unit_step(WL, "h2o", vals, cached, *rec, unit=unit))
    assert st.unit_steps == 2 * WL.steps and st.near_ties == 0
    # the tiny trace's evictions are all the position leaving the window
    assert st.heavy_evictions == 0


def test_step_check_counts_a_heavy_eviction():
    # a short prompt and a Zipf key skew: strong decoded tokens outscore heavy
    # members seeded by the prompt
    from synth.configs import Workload
    wl = Workload(901, "short_zipf", 1, 1, 32, 16, 60, 4, 8, "f32", "zipf", zipf_alpha=1.1)
    vals, cached, _ = unit_inputs(wl, 0, wl.n_positions, "input")
    Q, K, V = vals
    seeded, _, res = run_trace(Q, K, V, wl.prompt, wl.steps, wl.recent, wl.heavy, wl.scale)
    st = Stats()
    prev = seeded
    for s, r in enumerate(res):
        t = wl.prompt + s
        rec = (t, *slots_of(prev, wl.k), r.out, r.evicted, *slots_of(r.members, wl.k))
        st.merge(check_unit_step(wl, "h2o", vals, cached, *rec))
        prev = r.members
    assert st.heavy_evictions == sum(r.evicted != wl.prompt + s - wl.recent for s, r in enumerate(res)) > 0


@pytest.mark.parametrize("plant", ["output", "victim", "score", "member"])
def test_step_check_rejects_planted_mistakes(plant):
    vals, cached, _, recs = oracle_records(0, 8)
    t, pb, sb, out, ev, pa, sa = recs[5]
    out, pa, sa = out.copy(), pa.copy(), sa.copy()
    if plant == "output":
        out[3] += 3e-3 * np.abs(out).max()
    elif plant == "victim":
        live = [p for p in pb if 0 <= p <= t - WL.recent and p != ev]
        ev = live[0]
    elif plant == "score":
        sa[np.argmax(sa)] *= 1.003
    else:
        pa[np.argmax(pa)] = t - 1 if t - 1 not in pa else 0
    with pytest.raises(AssertionError):
        check_unit_step(WL, "h2o", vals, cached, t, pb, sb, out, ev, pa, sa)


def test_prefill_check_and_its_near_tie_band():
    vals, _, _ = unit_inputs(WL, 0, WL.n_positions, "input")
    Q, K, _ = vals
    ref, c = prefill(Q[:WL.prompt], K[:WL.prompt], WL.recent, WL.heavy, WL.scale)
    pos, score = slots_of(ref, WL.k, WL.recent, WL.prompt)
    assert check_unit_prefill(WL, "h2o", vals, pos, score)["max_score_rel"] < 1e-6
    # swapping the weakest kept heavy position for the best dropped one is a
    # mistake unless the two scores are within 1e-5 (they are not here)
    pool = range(WL.prompt - WL.recent)
    kept = [j for j in pool if j in ref]
    dropped = [j for j in pool if j not in ref]
    weakest = min(kept, key=lambda j: c[j])
    best = max(dropped, key=lambda j: c[j])
    assert c[weakest] - c[best] > 1e-5
    bad = dict(ref)
    del bad[weakest]
    bad[best] = c[best]
    with pytest.raises(AssertionError):
        check_unit_prefill(WL, "h2o", vals, *slots_of(bad, WL.k, WL.recent, WL.prompt))


def test_row_check_is_bit_exact():
    b, h = 0, 1
    bits = gen.unit_storage(WL, b, h, 0, WL.n_positions)
    pos = np.array([3, 9, -1, 40], dtype=np.int32)
    krows = np.zeros((4, WL.head_dim), np.float32)
    vrows = np.zeros((4, WL.head_dim), np.float32)
    for s, p in enumerate(pos):
        if p >= 0:
            krows[s], vrows[s] = bits[1][p], bits[2][p]
    check_unit_rows(WL, "input", bits, None, pos, krows, vrows)
    vrows[3, 7] = np.nextafter(vrows[3, 7], np.float32(np.inf))
    with pytest.raises(AssertionError):
        check_unit_rows(WL, "input", bits, None, pos, krows, vrows)


def test_pooled_checks_in_spawned_workers():
    """The same checks in worker processes started fresh; a planted mistake
    comes back as a failure message."""
    import multiprocessing as mp
    _, _, seeded, recs = oracle_records(1, 16)
    with mp.get_context("spawn").Pool(2) as pool:
        ok = pool.apply_async(pooled_task, ("steps", WL, 1, WL.n_positions, "input", "h2o", recs)).get(120)
        t, pb, sb, out, ev, pa, sa = recs[3]
        bad = recs[:3] + [(t, pb, sb, out + 1.0, ev, pa, sa)]
        fail = pool.apply_async(pooled_task, ("steps", WL, 1, WL.n_positions, "input", "h2o", bad)).get(120)
        pre = pool.apply_async(pooled_task, ("prefill", WL, 1, WL.n_positions, "input", "h2o",
                                             slots_of(seeded, WL.k, WL.recent, WL.prompt))).get(120)
    assert ok[0] == "ok" and ok[1]["unit_steps"] == 16
    assert fail[0] == "fail" and "steps unit 1" in fail[1]
    assert pre[0] == "ok"
