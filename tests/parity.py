"""Step-by-step comparison of the HIP path with the float64 oracle.

Protocol: before every checked decode step the GPU's slot state (pos, score) of
a sample of (batch, head) units is read back; the oracle rebuilds its cache set
from it, runs the same step on the exact input values, and the GPU's output,
eviction, updated scores and post-step membership are compared.  K/V slot rows
are compared bit for bit with the input rows of the positions they claim.

Tolerances:
  * attention output, per unit: max|o_gpu - o_ref| <= 2e-3 * max|o_ref|;
  * scores, per member: |s_gpu - s_ref| <= 2e-3 * s_ref + 1e-6 (the absolute
    floor covers a new token whose weight is tiny);
  * eviction: exact, except when the oracle's two lowest candidate scores are
    closer than tau = max(1e-5, 4 ulp_fp32(lowest)); then the GPU's victim must
    be one of the candidates within tau of the lowest (fp32 rounding of the
    GPU's own score += p is up to half an ulp);
  * prefill: scores as above; the kept set exact except for positions whose
    oracle score lies within tau_pre = max(1e-5, 1e-5 * c_h) of the h-th
    largest score c_h (fp32 column sums over up to P terms);
  * prompt attention output, per element: |o_gpu - o_ref| <= e * (A|V|)_ic + 1e-6
    where (A|V|)_ic = sum_j a_ij |v_jc| from the oracle's attention matrix and
    e = 2^-8 + 2e-4 for bf16 inputs (the probabilities enter the value product
    rounded to bf16: relative error at most 2^-8 each, plus float32 logits,
    exp2 and sums), e = 2e-4 for float32 inputs.

The per-unit checks live in tests/parity_check.py (torch-free).  With a process
pool (make_pool) the oracle side of every check runs in worker processes
that regenerate each unit's inputs from the seeds, while the GPU goes on with
the next steps; the results are the same checks.
"""
import numpy as np
import torch

from oracle import causal_attention
from parity_check import (Stats, check_unit_prefill, check_unit_rows, check_unit_step, pool_workers,
                          pooled_task, ulp32, unit_inputs)  # noqa: F401
from synth import gen
from synth.stage import stage_decode, stage_prompt

from kv_cache_eviction_02_amd import H2OCache


def sample_units(wl, n, seed=0):
    U = wl.units
    if n >= U:
        return list(range(U))
    rng = np.random.default_rng(seed)
    fixed = [0, U - 1, U // 2]
    rest = rng.choice([u for u in range(U) if u not in fixed], size=n - len(fixed), replace=False)
    return sorted(fixed + [int(u) for u in rest])


def torch_dtype(wl):
    return torch.bfloat16 if wl.kv_dtype == "bf16" else torch.float32


def make_pool(workers=None):
    """Worker processes for the oracle side.  They are started fresh (spawn),
    import numpy, the oracle and the generator only, and never touch the GPU."""
    import multiprocessing as mp
    return mp.get_context("spawn").Pool(workers or pool_workers())


class Harness:
    """Runs one workload on the GPU and checks sampled units against the oracle."""

    def __init__(self, wl, units, steps, device="cuda", decode_waves=0, decode_split=0,
                 cache="input", policy="h2o", pool=None):
        self.wl = wl
        self.units = units
        self.steps = steps
        self.device = device
        self.stats = Stats()
        self.cache_kind = cache
        self.policy = policy
        self.pool = pool
        self.pending = []
        U, k = wl.units, wl.k
        self.idx = torch.tensor(units, dtype=torch.long, device=device)
        self.cache = H2OCache(wl.batch, wl.heads, wl.head_dim, wl.recent, wl.heavy,
                              max_prompt=wl.prompt, dtype=torch_dtype(wl), scale=wl.scale,
                              device=device, decode_waves=decode_waves, decode_split=decode_split,
                              cache=cache, policy=policy)
        self.flat = dict(pos=self.cache.pos.view(U, k), score=self.cache.score.view(U, k),
                         k=self.cache.k_slots.view(U, k, -1), v=self.cache.v_slots.view(U, k, -1))
        if cache == "e4m3":
            self.flat["ks"] = self.cache.k_scale.view(U, k)
            self.flat["vs"] = self.cache.v_scale.view(U, k)
        self.n_pos = wl.prompt + steps
        self._inputs = {}

    def inputs(self, u):
        """(exact values, stored E4M3 rows, E4M3 codes and scales, storage bits) of unit u."""
        if u not in self._inputs:
            b, h = divmod(u, self.wl.heads)
            vals, cached, quant = unit_inputs(self.wl, u, self.n_pos, self.cache_kind)
            self._inputs[u] = (vals, cached, quant, gen.unit_storage(self.wl, b, h, 0, self.n_pos))
        return self._inputs[u]

    def gather(self, name):
        return self.flat[name].index_select(0, self.idx).cpu().numpy()

    # ---- pooled checks -----------------------------------------------------------

    def submit(self, kind, u, payload):
        args = (kind, self.wl, u, self.n_pos, self.cache_kind, self.policy, payload)
        self.pending.append(self.pool.apply_async(pooled_task, args))

    def collect(self, keep=0):
        """Wait for all but the newest `keep` pooled checks and merge their counts."""
        while len(self.pending) > keep:
            status, res = self.pending.pop(0).get()
            assert status == "ok", res
            self.stats.merge(res)

    # ---- prefill -------------------------------------------------------------

    def prefill(self, output=False):
        q, k, v = stage_prompt(self.wl, self.device)
        O = self.cache.prefill(q, k, v, output=output)
        torch.cuda.synchronize()
        del q, k, v
        if output:
            U, P, d = self.wl.units, self.wl.prompt, self.wl.head_dim
            O = O.view(U, P, d).index_select(0, self.idx).cpu().numpy()
            self.check_prompt_output(O)
        self.check_prefill()

    def check_prompt_output(self, O):
        wl = self.wl
        P = wl.prompt
        e = 2.0 ** -8 + 2e-4 if wl.kv_dtype == "bf16" else 2e-4
        for i, u in enumerate(self.units):
            Q, K, V = self.inputs(u)[0]
            A = causal_attention(Q[:P], K[:P], wl.scale)
            ref = A @ V[:P]
            tol = e * (A @ np.abs(V[:P])) + 1e-6
            err = np.abs(O[i].astype(np.float64) - ref)
            assert np.all(np.isfinite(O[i])), u
            worst = np.unravel_index(np.argmax(err / tol), err.shape)
            assert np.all(err <= tol), (u, worst, O[i][worst], ref[worst], tol[worst])
            self.stats.prompt_out_rows += P
            self.stats.prompt_out_err_over_tol = max(self.stats.prompt_out_err_over_tol,
                                                     float(np.max(err / tol)))

    def check_prefill(self):
        pos, score = self.gather("pos"), self.gather("score")
        for i, u in enumerate(self.units):
            if self.pool:
                self.submit("prefill", u, (pos[i], score[i]))
            else:
                self.stats.merge(check_unit_prefill(self.wl, self.policy, self.inputs(u)[0], pos[i], score[i],
                                                    unit=u))
        self.check_slot_rows()

    # ---- K/V slot rows ---------------------------------------------------------

    def check_slot_rows(self):
        pos = self.gather("pos")
        ks = self.flat["k"].index_select(0, self.idx).cpu()
        vs = self.flat["v"].index_select(0, self.idx).cpu()
        ksc = vsc = None
        if self.cache_kind == "e4m3":
            ksc, vsc = self.gather("ks"), self.gather("vs")
            ks, vs = ks.numpy(), vs.numpy()
        elif self.wl.kv_dtype == "bf16":
            ks = ks.view(torch.int16).numpy().view(np.uint16)
            vs = vs.view(torch.int16).numpy().view(np.uint16)
        else:
            ks, vs = ks.numpy(), vs.numpy()
        for i, u in enumerate(self.units):
            row = (pos[i], ks[i], vs[i], None if ksc is None else ksc[i], None if vsc is None else vsc[i])
            if self.pool:
                self.submit("rows", u, row)
            else:
                _, _, quant, bits = self.inputs(u)
                check_unit_rows(self.wl, self.cache_kind, bits, quant, *row, unit=u)

    # ---- decode ----------------------------------------------------------------

    def run(self, check_every=1, kv_every=64, chunk=4096, pool_chunk=64):
        wl = self.wl
        recs = {u: [] for u in self.units}
        after = None
        for s0 in range(0, self.steps, chunk):
            s1 = min(self.steps, s0 + chunk)
            dq, dk, dv = stage_decode(wl, s0, s1, self.device)
            for s in range(s0, s1):
                check = (s % check_every == 0) or s == self.steps - 1
                if check:
                    # checking every step: this step's incoming state is the last one's outgoing state
                    before = after if after is not None else (self.gather("pos"), self.gather("score"))
                out, ev = self.cache.step(dq[s - s0], dk[s - s0], dv[s - s0])
                after = None
                if check:
                    t = wl.prompt + s
                    self.stats.steps += 1
                    out = out.view(wl.units, -1).index_select(0, self.idx).cpu().numpy()
                    ev = ev.view(-1).index_select(0, self.idx).cpu().numpy()
                    pos_a, score_a = self.gather("pos"), self.gather("score")
                    if check_every == 1:
                        after = (pos_a, score_a)
                    for i, u in enumerate(self.units):
                        rec = (t, before[0][i], before[1][i], out[i], ev[i], pos_a[i], score_a[i])
                        if self.pool:
                            recs[u].append(rec)
                        else:
                            vals, cached, _, _ = self.inputs(u)
                            self.stats.merge(check_unit_step(wl, self.policy, vals, cached, *rec, unit=u))
                    if self.pool and (len(recs[self.units[0]]) >= pool_chunk or s == self.steps - 1):
                        for u in self.units:
                            self.submit("steps", u, recs[u])
                            recs[u] = []
                        # keep a few chunks in flight, so the host memory they hold stays bounded
                        self.collect(keep=4 * len(self.units))
                if s % kv_every == 0 or s == self.steps - 1:
                    self.check_slot_rows()
                if self.pool and s % 256 == 255:
                    print(f"[parity] {wl.name}: {s + 1} of {self.steps} steps run, "
                          f"{self.stats.unit_steps} unit-steps checked", flush=True)
            del dq, dk, dv
        if self.pool:
            self.collect()
        return self.stats

    def check_step(self, t, before, out, ev):
        """Check the sampled units' step at position t (before: incoming pos, score)."""
        wl = self.wl
        out = out.view(wl.units, -1).index_select(0, self.idx).cpu().numpy()
        ev = ev.view(-1).index_select(0, self.idx).cpu().numpy()
        pos_a, score_a = self.gather("pos"), self.gather("score")
        self.stats.steps += 1
        for i, u in enumerate(self.units):
            vals, cached, _, _ = self.inputs(u)
            self.stats.merge(check_unit_step(wl, self.policy, vals, cached, t, before[0][i], before[1][i],
                                             out[i], ev[i], pos_a[i], score_a[i], unit=u))

    def close(self):
        self.pending = []   # checks still running belong to a run that is being abandoned
        self.cache.close()
