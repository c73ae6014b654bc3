"""Pins of the float64 CPU oracle to facts the H2O pages and mathematics fix.

Each test checks the oracle against something other than itself: a library
attention routine (torch's scaled_dot_product_attention on the CPU in float64)
for the special cases that reduce to full or sliding-window attention, closed
forms, hand-built exact ties, exhaustive search on tiny inputs, and invariants
of the eviction rule (summary page "H2O: Heavy-Hitter Oracle for Efficient
Generative Inference", "The mechanism" and "Algorithm / figure walkthrough").
"""
import itertools
from collections import defaultdict

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import (causal_attention, decode_step, prefill, prefill_column_sums, prefill_output,
                    prefill_scores,
                    prefill_keep, run_trace)
from synth import WORKLOADS, gen


def sdpa(Q, K, V, scale, mask=None, causal=False):
    q = torch.from_numpy(np.ascontiguousarray(Q, dtype=np.float64))[None, None]
    k = torch.from_numpy(np.ascontiguousarray(K, dtype=np.float64))[None, None]
    v = torch.from_numpy(np.ascontiguousarray(V, dtype=np.float64))[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    return F.scaled_dot_product_attention(q, k, v, attn_mask=m, is_causal=causal,
                                          scale=scale)[0, 0].numpy()


def random_qkv(n, d, seed, spread=1.0):
    rng = np.random.default_rng(seed)
    return tuple(spread * rng.standard_normal((n, d)) for _ in range(3))


def c1_unit(unit):
    wl = WORKLOADS["tiny_fp32"]
    Q, K, V = gen.unit_values(wl, 0, unit, 0, wl.n_positions)
    return wl, Q, K, V


TRACE_CASES = [  # (P, T, r, h, d, seed)
    (24, 30, 4, 6, 8, 1),
    (10, 25, 3, 5, 16, 2),
    (5, 20, 4, 4, 8, 3),      # prompt shorter than the budget
    (3, 15, 4, 2, 8, 4),      # prompt shorter than the protected window
    (30, 20, 1, 7, 8, 5),     # smallest protected window
    (16, 16, 8, 0, 8, 6),     # no heavy slots
]


def all_traces():
    for (P, T, r, h, d, seed) in TRACE_CASES:
        Q, K, V = random_qkv(P + T, d, seed, spread=1.5)
        yield P, T, r, h, 1 / np.sqrt(d), Q, K, V
    for unit in (0, 1):
        wl, Q, K, V = c1_unit(unit)
        yield wl.prompt, wl.steps, wl.recent, wl.heavy, wl.scale, Q, K, V


# --- P1: a budget covering the whole sequence is full causal attention -------

@pytest.mark.parametrize("P,T,r,h", [(12, 10, 4, 30), (5, 9, 8, 10), (3, 8, 2, 12),
                                     (16, 4, 16, 4), (1, 6, 1, 6)])
def test_full_budget_equals_full_causal_attention(P, T, r, h):
    d = 8
    N = P + T
    assert r + h >= N
    Q, K, V = random_qkv(N, d, seed=P * 100 + T, spread=2.0)
    scale = 1 / np.sqrt(d)
    seeded, c, steps = run_trace(Q, K, V, P, T, r, h, scale)

    A_prompt = sdpa(Q[:P], K[:P], np.eye(P), scale, causal=True)
    assert sorted(seeded) == list(range(P))
    np.testing.assert_allclose([seeded[j] for j in range(P)], A_prompt.sum(0),
                               rtol=1e-12, atol=1e-13)

    ref_out = sdpa(Q, K, V, scale, causal=True)
    for s, res in enumerate(steps):
        t = P + s
        assert res.evicted is None
        np.testing.assert_allclose(res.out, ref_out[t], rtol=1e-12, atol=1e-12)

    A = sdpa(Q, K, np.eye(N), scale, causal=True)   # full attention matrix
    final = steps[-1].members
    assert sorted(final) == list(range(N))
    np.testing.assert_allclose([final[j] for j in range(N)], A.sum(0),
                               rtol=1e-12, atol=1e-13)


# --- P2: no heavy slots is sliding-window (Local) attention ------------------

@pytest.mark.parametrize("P,T,k", [(16, 20, 6), (3, 12, 6), (6, 6, 6), (10, 10, 1)])
def test_zero_heavy_equals_sliding_window(P, T, k):
    d = 8
    N = P + T
    Q, K, V = random_qkv(N, d, seed=7 + k, spread=2.0)
    scale = 1 / np.sqrt(d)
    _, _, steps = run_trace(Q, K, V, P, T, k, 0, scale)
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    band = (j <= i) & (j >= i - k)
    ref = sdpa(Q, K, V, scale, mask=band)
    for s, res in enumerate(steps):
        t = P + s
        assert res.evicted == (t - k if t >= k else None)
        np.testing.assert_allclose(res.out, ref[t], rtol=1e-12, atol=1e-12)


# --- P3: Definition 4.3 and irreversible eviction ----------------------------

def test_definition_4_3_invariants():
    for P, T, r, h, scale, Q, K, V in all_traces():
        k = r + h
        seeded, _, steps = run_trace(Q, K, V, P, T, r, h, scale)
        prev = set(seeded)
        assert len(prev) == min(P, k)
        gone = set()
        for s, res in enumerate(steps):
            t = P + s
            cur = set(res.members)
            assert len(cur) == min(t + 1, k)
            assert cur <= prev | {t}
            assert len(cur - prev) <= 1
            assert set(range(max(0, t - r + 1), t + 1)) <= cur
            assert not (cur & gone)
            if res.evicted is not None:
                assert res.evicted in prev and res.evicted not in cur
                gone.add(res.evicted)
            assert (prev | {t}) - cur == ({res.evicted} if res.evicted is not None else set())
            prev = cur


# --- P4: score bounds; P9: mass conservation ---------------------------------

def test_score_bounds_and_mass_conservation():
    for P, T, r, h, scale, Q, K, V in all_traces():
        seeded, _, steps = run_trace(Q, K, V, P, T, r, h, scale)
        evicted_any = len(seeded) < P
        prev = seeded
        total_prev = sum(seeded.values())
        if not evicted_any:
            assert total_prev == pytest.approx(P, rel=1e-12)
        for s, res in enumerate(steps):
            t = P + s
            vals = np.array(list(res.members.values()))
            assert (vals >= 0).all()
            total = vals.sum()
            assert total <= (t + 1) * (1 + 1e-12)
            if res.evicted is None:
                assert total == pytest.approx(total_prev + 1, rel=1e-12)
            else:
                evicted_any = True
                victim_score = prev[res.evicted] + res.weights[res.evicted]
                assert total == pytest.approx(total_prev + 1 - victim_score, rel=1e-12)
            if not evicted_any:
                assert total == pytest.approx(t + 1, rel=1e-12)
            total_prev = total
            prev = res.members


# --- P5: brute-force recomputation of the accumulated scores -----------------

def test_scores_match_non_incremental_recomputation():
    for P, T, r, h, scale, Q, K, V in all_traces():
        seeded, _, steps = run_trace(Q, K, V, P, T, r, h, scale)
        A_prompt = sdpa(Q[:P], K[:P], np.eye(P), scale, causal=True)
        acc = defaultdict(float)
        for j, cj in enumerate(A_prompt.sum(0)):
            acc[j] = cj
        for s, res in enumerate(steps):
            t = P + s
            idx = res.attended
            w = torch.softmax(torch.from_numpy(scale * (K[idx] @ Q[t])), dim=0).numpy()
            for j, wj in zip(idx, w):
                acc[j] += wj
            for j, sc in res.members.items():
                assert sc == pytest.approx(acc[j], rel=1e-11, abs=1e-13)


# --- P6: the eviction maximises the retained accumulated score ---------------

def test_eviction_is_greedy_max_retained_mass():
    for P, T, r, h, scale, Q, K, V in all_traces():
        seeded, _, steps = run_trace(Q, K, V, P, T, r, h, scale)
        prev = seeded
        for s, res in enumerate(steps):
            t = P + s
            pre = {j: prev[j] + res.weights[j] for j in prev}
            pre[t] = res.weights[t]
            if res.evicted is not None:
                cands = [j for j in pre if j <= t - r]
                kept_mass = {v: sum(sc for j, sc in pre.items() if j != v) for v in cands}
                best = max(kept_mass.values())
                # greatest retained mass; among equal masses the older goes
                winners = sorted(v for v in cands if kept_mass[v] == best)
                assert res.evicted == winners[0]
            prev = res.members


# --- P7: closed form under uniform attention ----------------------------------

def test_uniform_attention_closed_form():
    P, T, r, h, d = 64, 64, 16, 16, 8
    k = r + h
    N = P + T
    rng = np.random.default_rng(11)
    Q = np.zeros((N, d))
    K = rng.standard_normal((N, d))
    V = rng.standard_normal((N, d))
    seeded, c, steps = run_trace(Q, K, V, P, T, r, h, 1 / np.sqrt(d))
    H = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, N + 1))])   # harmonic numbers
    np.testing.assert_allclose(c, H[P] - H[np.arange(P)], rtol=1e-13)
    assert sorted(seeded) == list(range(h)) + list(range(P - r, P))
    for s, res in enumerate(steps):
        t = P + s
        assert res.evicted == t - r
        att = list(range(h)) + list(range(t - r, t + 1))
        np.testing.assert_allclose(res.out, V[att].mean(0), rtol=1e-12, atol=1e-13)
    final = steps[-1].members
    assert sorted(final) == list(range(h)) + list(range(N - r, N))
    for j, sc in final.items():
        expect = (H[P] - H[j] if j < P else 0.0) + (N - max(j, P)) / (k + 1)
        assert sc == pytest.approx(expect, rel=1e-12)


# --- P8: exact ties -------------------------------------------------------------

def test_prefill_and_decode_exact_ties_from_dead_keys():
    """Keys far below the row maximum get weight exactly 0.0 in float64, so
    several positions tie at score 0: prefill keeps the newer ones, decode
    evicts the older ones first."""
    d, P, r, h = 8, 24, 4, 6
    alive_pool = {0, 4, 9, 15}
    N = P + 4
    e0 = np.eye(d)[0]
    Q = np.tile(e0, (N, 1))
    rng = np.random.default_rng(5)
    K = rng.standard_normal((N, d))
    K[:, 0] = 0.0                       # alive keys: logit exactly 0
    dead = [j for j in range(P - r) if j not in alive_pool]
    K[dead] = -1e4 * e0                 # dead keys: weight underflows to exactly 0
    V = rng.standard_normal((N, d))
    scale = 1 / np.sqrt(d)
    seeded, c, steps = run_trace(Q, K, V, P, N - P, r, h, scale)
    assert all(c[j] == 0.0 for j in dead)
    assert all(c[j] > 0.0 for j in alive_pool)
    assert sorted(seeded) == sorted(alive_pool) + [18, 19] + list(range(P - r, P))
    assert steps[0].evicted == 18
    assert steps[1].evicted == 19
    assert all(res.evicted not in alive_pool for res in steps)


def test_decode_exact_tie_evicts_oldest():
    r, h = 2, 5
    members = {0: 0.5, 1: 0.25, 2: 0.25, 3: 0.25, 4: 0.75, 5: 0.25, 6: 0.125}
    d = 4
    t = 7
    rng = np.random.default_rng(3)
    K = rng.standard_normal((t + 1, d))
    V = rng.standard_normal((t + 1, d))
    res = decode_step(members, t, np.zeros(d), K, V, r, h, 0.5)
    assert res.evicted == 1
    scores = [res.members[j] for j in (2, 3, 5)]
    assert scores[0] == scores[1] == scores[2] == 0.25 + 1 / 8


def test_prefill_keep_exhaustive_on_tiny_inputs():
    rng = np.random.default_rng(9)
    for trial in range(200):
        P = int(rng.integers(1, 11))
        r = int(rng.integers(1, 4))
        h = int(rng.integers(0, 5))
        c = rng.integers(0, 4, size=P).astype(float)     # small integers: many exact ties
        keep = prefill_keep(c, r, h)
        if P <= r + h:
            assert keep == list(range(P))
            continue
        pool = list(range(P - r))
        best = max(itertools.combinations(pool, h),
                   key=lambda S: (sum(c[j] for j in S), sum(S)))
        assert keep == sorted(best) + list(range(P - r, P))


# --- P10: accumulation matters (naive per-step top-k is a different rule) ------

def test_not_naive_per_step_top_k():
    wl, Q, K, V = c1_unit(0)
    seeded, _, steps = run_trace(Q, K, V, wl.prompt, wl.steps, wl.recent, wl.heavy, wl.scale)
    prev = seeded
    differ = 0
    for s, res in enumerate(steps):
        t = wl.prompt + s
        cands = [j for j in list(prev) + [t] if j <= t - wl.recent]
        naive = min(cands, key=lambda j: (res.weights[j], j))
        differ += naive != res.evicted
        prev = res.members
    assert differ >= 1


# --- prefill column sums: consistency with the attention matrix ----------------

def test_prefill_column_sums_sum_to_prompt_length():
    for n in (1, 2, 7, 64):
        Q, K, _ = random_qkv(n, 16, seed=n, spread=3.0)
        c = prefill_column_sums(Q, K, 0.25)
        assert c.sum() == pytest.approx(n, rel=1e-13)
        A = causal_attention(Q, K, 0.25)
        np.testing.assert_allclose(A, sdpa(Q, K, np.eye(n), 0.25, causal=True), atol=1e-14)
        assert c[-1] == pytest.approx(A[-1, -1])


# --- regression record of the tiny fp32 trajectory -------------------------------

def test_tiny_trace_matches_recorded_trajectory():
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_fp32_trace.json")
    rec = json.load(open(path))
    for u in rec["units"]:
        wl, Q, K, V = c1_unit(u["head"])
        seeded, _, steps = run_trace(Q, K, V, wl.prompt, wl.steps, wl.recent, wl.heavy, wl.scale)
        assert sorted(seeded) == u["prefill_kept"]
        assert [s.evicted for s in steps] == u["evicted"]
        assert sorted(steps[-1].members) == u["final_members"]


def test_stream_trace_matches_recorded_trajectory_and_evicts_heavy_members():
    """The recorded long-stream trajectory (first 2000 steps, heads 0-3) is the
    oracle's own; here its first 400 steps of head 0 are replayed.  Many of its
    evictions remove a heavy member, not the position leaving the window, so it
    separates H2O from Local and from a static Top-K, whose victim is always
    t - recent."""
    import json
    import os
    from oracle import prefill as oracle_prefill
    path = os.path.join(os.path.dirname(__file__), "golden", "llama7b_stream_trace.json")
    rec = json.load(open(path))
    wl = WORKLOADS["llama7b_stream"]
    P, r, h = wl.prompt, wl.recent, wl.heavy
    for u in rec["units"]:
        assert u["heavy_evictions"] == sum(e != P + s - r for s, e in enumerate(u["evicted"])) > 40
    u = rec["units"][0]
    n = 400
    Q, K, V = gen.unit_values(wl, 0, u["head"], 0, P + n)
    members, _ = oracle_prefill(Q[:P], K[:P], r, h, wl.scale)
    assert sorted(members) == u["prefill_kept"]
    for s in range(n):
        res = decode_step(members, P + s, Q[P + s], K, V, r, h, wl.scale)
        assert res.evicted == u["evicted"][s], s
        members = res.members


# --- E4M3 cache rows -------------------------------------------------------------

def test_e4m3_encode_matches_torch_float8_e4m3fn():
    from oracle import e4m3_encode, e4m3_value
    finite = [c for c in range(256) if not np.isnan(e4m3_value(c))]
    vals = e4m3_value(finite)
    order = np.argsort(vals)
    sv = vals[order]
    mids = (sv[:-1] + sv[1:]) / 2            # exact midpoints: ties to even
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.uniform(-448, 448, 20000), rng.normal(0, 1, 20000),
                        rng.normal(0, 0.004, 5000), mids, sv,
                        [448.00003, -448.00003, 463.9]]).astype(np.float32)
    ours = e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_e4m3_round_trip_and_row_quantization_bounds():
    from oracle import dequantize_row_e4m3, e4m3_encode, e4m3_value, quantize_row_e4m3
    for c in range(256):
        v = e4m3_value(c)
        if not np.isnan(v):
            assert e4m3_encode(np.float32(v)) == c
    rng = np.random.default_rng(8)
    for trial in range(200):
        x = (rng.standard_normal(128) * rng.uniform(1e-3, 50)).astype(np.float32)
        codes, s = quantize_row_e4m3(x)
        deq = dequantize_row_e4m3(codes, s)
        amax = np.abs(x).max()
        assert abs(abs(deq[np.argmax(np.abs(x))]) - amax) <= amax * 1e-6   # the peak maps to +-448
        # half a quantum of the code grid, in row units
        bound = np.maximum(np.abs(x) * 2.0 ** -4, s * 2.0 ** -10) * (1 + 1e-6)
        assert np.all(np.abs(deq - x) <= bound)
    codes, s = quantize_row_e4m3(np.zeros(8, dtype=np.float32))
    assert s == 0 and not codes.any()


def test_e4m3_cache_equals_exact_cache_when_rows_are_representable():
    """Rows already on their own E4M3 grid are stored exactly, so the trace with
    an E4M3 cache equals the exact one (checks the cached-row plumbing)."""
    from oracle import e4m3_value
    rng = np.random.default_rng(12)
    P, T, r, h, d = 24, 20, 4, 6, 16
    N = P + T
    finite = np.array([c for c in range(256) if not np.isnan(e4m3_value(c))])
    def grid_rows():
        rows = e4m3_value(rng.choice(finite, size=(N, d)))
        rows[:, 0] = 448.0                        # peak sets the row scale to exactly 1
        return rows * 2.0 ** -6                   # power-of-two scale keeps the grid
    Q = rng.standard_normal((N, d))
    K, V = grid_rows(), grid_rows()
    scale = 1 / np.sqrt(d)
    _, _, exact = run_trace(Q, K, V, P, T, r, h, scale)
    _, _, quant = run_trace(Q, K, V, P, T, r, h, scale, cache="e4m3")
    for a, b in zip(exact, quant):
        assert a.evicted == b.evicted
        np.testing.assert_array_equal(a.out, b.out)


def torch_e4m3_stored_row(x):
    """The row an E4M3 cache holds for input row x, built without the oracle:
    the format the library stores (codes of x * (448 / amax) in float32, row
    scale amax / 448; a zero row stays zero) with torch's own float8_e4m3fn
    rounding, read back in float64."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.abs(x).max())
    if amax == 0:
        return np.zeros(x.shape)
    y = (x * (np.float32(448.0) / amax)).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn)
    return codes.to(torch.float64).numpy() * np.float64(amax / np.float32(448.0))


def test_e4m3_cache_off_grid_rows_attend_stored_members_and_exact_token():
    """Rows off the E4M3 grid with a budget covering the whole sequence: every
    decode step's output is the library attention (torch SDPA, float64) over
    the stored (dequantized) rows of the cached positions plus the decoded
    token's exact row, and the final scores are the prompt's exact column sums
    plus the column sums of those steps' weights (summary, "What to notice when
    reading": H2O composes with quantization of the cached rows).  The two
    other readings (every row exact; the token attending with its stored row)
    give outputs at least a thousand times the tolerance away at every step, so
    either mistake fails here."""
    P, T, d = 10, 14, 16
    N = P + T
    Q, K, V = random_qkv(N, d, seed=31, spread=1.5)
    K = K.astype(np.float32).astype(np.float64)   # float32 inputs, as the library takes them
    V = V.astype(np.float32).astype(np.float64)
    scale = 1 / np.sqrt(d)
    seeded, c, steps = run_trace(Q, K, V, P, T, 4, 30, scale, cache="e4m3")
    Ks = np.array([torch_e4m3_stored_row(row) for row in K])
    Vs = np.array([torch_e4m3_stored_row(row) for row in V])
    assert np.abs(Ks - K).max() > 1e-3            # the rows really are off the grid

    A_prompt = sdpa(Q[:P], K[:P], np.eye(P), scale, causal=True)
    score = np.zeros(N)
    score[:P] = A_prompt.sum(0)
    for s, res in enumerate(steps):
        t = P + s
        assert res.evicted is None
        Kt = np.vstack([Ks[:t], K[t:t + 1]])
        Vt = np.vstack([Vs[:t], V[t:t + 1]])
        ref = sdpa(Q[t:t + 1], Kt, Vt, scale)[0]
        np.testing.assert_allclose(res.out, ref, rtol=1e-12, atol=1e-13)
        w = sdpa(Q[t:t + 1], Kt, np.eye(t + 1), scale)[0]
        score[:t + 1] += w
        # the other readings are clearly different answers
        all_exact = sdpa(Q[t:t + 1], K[:t + 1], V[:t + 1], scale)[0]
        token_stored = sdpa(Q[t:t + 1], Ks[:t + 1], Vs[:t + 1], scale)[0]
        assert np.abs(all_exact - ref).max() > 1e-9 and np.abs(token_stored - ref).max() > 1e-9
    final = steps[-1].members
    assert sorted(final) == list(range(N))
    np.testing.assert_allclose([final[j] for j in range(N)], score, rtol=1e-12, atol=1e-13)


def test_e4m3_cache_stored_rows_decide_the_victim():
    """Hand-built full cache (r = 1: every member is a candidate) whose two
    lowest scores are separated so that only the stated reading evicts position
    0: the members attend with their stored E4M3 rows and the decoded token with
    its exact row.  Attending with the members' exact rows, or with the token's
    stored row, moves the weight enough to evict position 1 instead."""
    d, t, r, h = 2, 3, 1, 2
    scale = 1.0
    q = np.array([0.0, 10.0])
    # position 0 and the token are off the grid (0.3 * 448 = 134.4 is stored as
    # 128); position 1 (0.25 * 448 = 112) and position 2 are on it
    K = {0: np.array([1.0, 0.3]), 1: np.array([1.0, 0.25]), 2: np.array([1.0, 0.0]),
         3: np.array([1.0, 0.3])}
    V = {j: np.array([float(j), 1.0]) for j in K}
    Ks = {j: torch_e4m3_stored_row(K[j]) for j in K}
    Vs = {j: torch_e4m3_stored_row(V[j]) for j in V}
    assert abs(Ks[0][1] - 128 / 448) < 1e-7 and abs(Ks[1][1] - 0.25) < 1e-7

    def weights(k_members, k_token):
        rows = np.vstack([k_members[j] for j in (0, 1, 2)] + [k_token])
        return sdpa(q[None], rows, np.eye(4), scale)[0]
    w_read = weights(Ks, K[3])               # the stated reading
    w_exact = weights(K, K[3])               # members exact
    w_tok = weights(Ks, Ks[3])               # token stored
    th = {name: w[0] - w[1] for name, w in (("read", w_read), ("exact", w_exact), ("tok", w_tok))}
    # position 0 is evicted iff s1 - s0 > w0 - w1; both other readings need a larger gap
    assert th["exact"] > th["read"] and th["tok"] > th["read"]
    gap = th["read"] + 0.5 * (min(th["exact"], th["tok"]) - th["read"])
    members = {0: 1.0, 1: 1.0 + gap, 2: 50.0}
    Kc = {j: dequant for j, dequant in Ks.items()}
    Vc = {j: dequant for j, dequant in Vs.items()}
    from oracle import dequantize_row_e4m3, quantize_row_e4m3
    for j in K:   # the oracle's own quantizer stores the same rows
        np.testing.assert_array_equal(dequantize_row_e4m3(*quantize_row_e4m3(K[j])), Ks[j])
    res = decode_step(members, t, q, K, V, r, h, scale, Kc, Vc)
    assert res.evicted == 0
    np.testing.assert_allclose([res.weights[j] for j in (0, 1, 2, 3)], w_read, rtol=1e-12, atol=1e-15)
    # the same step under each other reading evicts position 1
    assert decode_step(members, t, q, K, V, r, h, scale).evicted == 1
    Kt = dict(Kc)
    Kt[3] = Ks[3]
    assert decode_step(members, t, q, Kt, V, r, h, scale, Kc, Vc).evicted == 1


def test_e4m3_cache_keeps_definition_4_3():
    wl, Q, K, V = c1_unit(0)
    seeded, _, steps = run_trace(Q, K, V, wl.prompt, wl.steps, wl.recent, wl.heavy, wl.scale,
                                 cache="e4m3")
    prev = set(seeded)
    for s, res in enumerate(steps):
        cur = set(res.members)
        assert len(cur) == wl.k and len(cur - prev) <= 1
        prev = cur


# ---- prompt output ---------------------------------------------------------------

@pytest.mark.parametrize("n,d,seed", [(1, 8, 11), (7, 16, 12), (40, 32, 13), (65, 64, 14)])
def test_prefill_output_matches_library_causal_attention(n, d, seed):
    # Full causal attention of the prompt (walkthrough step 1) is exactly what
    # torch's scaled_dot_product_attention computes with is_causal=True.
    Q, K, V = random_qkv(n, d, seed, spread=2.0)
    scale = 1 / np.sqrt(d)
    O = prefill_output(Q, K, V, scale)
    np.testing.assert_allclose(O, sdpa(Q, K, V, scale, causal=True), rtol=1e-12, atol=1e-12)


def test_prefill_output_special_cases():
    Q, K, V = random_qkv(12, 8, 15, spread=3.0)
    O = prefill_output(Q, K, V, 0.5)
    # the first position attends only to itself
    np.testing.assert_allclose(O[0], V[0], rtol=0, atol=1e-14)
    # constant values are reproduced (each attention row sums to one)
    np.testing.assert_allclose(prefill_output(Q, K, np.full_like(V, 3.25), 0.5), 3.25, rtol=0, atol=1e-13)
    # zero queries: position i averages the values of positions 0..i
    Oz = prefill_output(np.zeros_like(Q), K, V, 0.5)
    means = np.cumsum(V, axis=0) / np.arange(1, 13)[:, None]
    np.testing.assert_allclose(Oz, means, rtol=0, atol=1e-13)


# ---- ablation policies (summary, "Prior limits" and "Limitations") -------------

def band_mask(n, allowed):
    """Boolean attention mask: row i may attend the positions allowed(i)."""
    m = np.zeros((n, n), dtype=bool)
    for i in range(n):
        m[i, list(allowed(i))] = True
    return m


def test_heavy_only_uniform_attention_closed_form():
    # r = 0, q = 0: every attended weight is 1/(n+1).  The prompt keeps the h
    # oldest positions (largest harmonic column sums); once full, the new token's
    # weight 1/(h+1) is below every member's score, so it is evicted at once.
    P, T, h, d = 40, 30, 8, 8
    rng = np.random.default_rng(21)
    N = P + T
    Q = np.zeros((N, d))
    K, V = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    seeded, _, steps = run_trace(Q, K, V, P, T, 0, h, 0.5)
    assert sorted(seeded) == list(range(h))
    for s, res in enumerate(steps):
        t = P + s
        assert res.evicted == t
        assert sorted(res.members) == list(range(h))
        np.testing.assert_allclose(res.out, V[list(range(h)) + [t]].mean(0), rtol=1e-12, atol=1e-13)


def test_heavy_only_keeps_definition_4_3_and_admits_strong_tokens():
    # Heavy-only traces: |S| = k once full, at most one change per step.  Every
    # third token's key is aligned with its query, so its own weight is close to
    # one and beats the weakest member; the others are evicted at once.
    P, T, h, d = 12, 60, 6, 8
    Q, K, V = random_qkv(P + T, d, 22, spread=1.0)
    for t in range(P, P + T, 3):
        K[t] = 3.0 * Q[t]
    seeded, _, steps = run_trace(Q, K, V, P, T, 0, h, 1 / np.sqrt(d))
    prev = set(seeded)
    self_evicted = kept = 0
    for s, res in enumerate(steps):
        t = P + s
        cur = set(res.members)
        assert len(cur) == h and len(cur - prev) <= 1
        self_evicted += res.evicted == t
        kept += t in cur
        prev = cur
    assert self_evicted > 0 and kept > 0


def test_static_policy_attends_prefill_heavy_set_plus_window():
    # Static Top-K: after a full prompt the heavy set is the prefill's and never
    # changes; every step attends to it plus the r newest positions, which is
    # torch's attention with that mask.
    P, T, r, h, d = 50, 40, 6, 10, 16
    Q, K, V = random_qkv(P + T, d, 23, spread=2.0)
    scale = 1 / np.sqrt(d)
    seeded, c, steps = run_trace(Q, K, V, P, T, r, h, scale, policy="static")
    heavy0 = sorted(j for j in seeded if j < P - r)
    assert heavy0 == sorted(prefill_keep(c, r, h))[:h]
    N = P + T
    mask = band_mask(N, lambda i: set(heavy0) | set(range(max(0, i - r), i + 1)))
    ref = sdpa(Q, K, V, scale, mask=mask)
    for s, res in enumerate(steps):
        t = P + s
        assert res.evicted == t - r
        np.testing.assert_allclose(res.out, ref[t], rtol=1e-12, atol=1e-12)
    assert sorted(steps[-1].members) == heavy0 + list(range(N - r, N))


def test_static_policy_fills_like_h2o_before_the_cache_is_full():
    # With a short prompt the cache fills by admission under every policy.
    P, T, r, h, d = 4, 30, 4, 8, 8
    Q, K, V = random_qkv(P + T, d, 24, spread=2.0)
    _, _, st = run_trace(Q, K, V, P, T, r, h, 0.4, policy="static")
    _, _, hh = run_trace(Q, K, V, P, T, r, h, 0.4)
    fill = r + h - P  # steps before the first eviction
    for s in range(fill):
        assert st[s].evicted is None and hh[s].evicted is None
        assert st[s].members == hh[s].members
    assert all(res.evicted == P + s - r for s, res in enumerate(st) if s >= fill)


def test_naive_policy_uniform_attention_is_a_sliding_window():
    # Naive per-step Top-K with q = 0: every weight of a step is equal, ties send
    # the older position out, so the cache is always the newest k positions:
    # torch's attention with a band mask of width k + 1.
    P, T, r, h, d = 30, 25, 4, 7, 8
    k = r + h
    rng = np.random.default_rng(25)
    N = P + T
    Q = np.zeros((N, d))
    K, V = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    seeded, c, steps = run_trace(Q, K, V, P, T, r, h, 0.5, policy="naive")
    np.testing.assert_allclose(c, np.full(P, 1.0 / P), rtol=1e-13)
    assert sorted(seeded) == list(range(P - k, P))
    ref = sdpa(Q, K, V, 0.5, mask=band_mask(N, lambda i: range(max(0, i - k), i + 1)))
    for s, res in enumerate(steps):
        t = P + s
        assert res.evicted == t - k
        np.testing.assert_allclose(res.out, ref[t], rtol=1e-12, atol=1e-13)
        for j, sc in res.members.items():
            assert sc == pytest.approx(1.0 / (k + 1), rel=1e-12)


def test_naive_prefill_scores_are_the_last_prompt_row():
    Q, K, _ = random_qkv(20, 8, 26, spread=2.0)
    c = prefill_scores(Q, K, 0.35, "naive")
    e = np.zeros(20)
    e[-1] = 1.0
    last = sdpa(Q, K, np.eye(20), 0.35, causal=True)[-1]
    np.testing.assert_allclose(c, last, rtol=1e-12, atol=1e-15)
    assert c.sum() == pytest.approx(1.0, rel=1e-13)


def test_naive_policy_forgets_accumulated_mass():
    # Hand-built: position 0 collected a large score in the past but gets the
    # smallest weight now.  H2O keeps it (its accumulated score is largest);
    # the naive policy evicts it.
    d = 4
    K = np.array([[5.0, 0, 0, 0], [0, 1.0, 0, 0], [0, 0, 1.0, 0], [0, 0, 0, 1.0]])
    V = np.eye(4)
    q = np.array([-2.0, 1.0, 0.5, 0.2])
    members = {0: 3.0, 1: 0.2, 2: 0.1}
    h2o = decode_step(members, 3, q, K, V, 1, 2, 1.0)
    naive = decode_step(members, 3, q, K, V, 1, 2, 1.0, policy="naive")
    assert naive.evicted == 0 and h2o.evicted != 0
    w = np.exp(K @ q)
    w /= w.sum()
    for j in (1, 2):
        assert naive.members[j] == pytest.approx(w[j], rel=1e-13)


def test_policy_traces_match_recorded_trajectories():
    # regression record of the oracle's ablation policies (tests/golden/make_policy_traces.py)
    import json
    import os
    rec = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tiny_fp32_policy_traces.json")))
    for case in rec["cases"]:
        for u in case["units"]:
            wl, Q, K, V = c1_unit(u["head"])
            seeded, _, steps = run_trace(Q, K, V, wl.prompt, wl.steps, case["recent"], case["heavy"], wl.scale,
                                         policy=case["policy"])
            assert sorted(seeded) == u["prefill_kept"], case["policy"]
            assert [s.evicted for s in steps] == u["evicted"], case["policy"]
            assert sorted(steps[-1].members) == u["final_members"], case["policy"]
