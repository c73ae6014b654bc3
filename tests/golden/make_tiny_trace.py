"""Writes tiny_fp32_trace.json: the oracle's own free-running trajectory on the
tiny fp32 workload (1 x 2 heads, d 64, prompt 64, 64 steps, k 32 = 16 + 16).

The H2O pages print no worked numeric example, so this file is not a value
from the pages: it is a regression record of the oracle (which is pinned by
tests/test_oracle_pins.py), produced by this script, which calls only the
oracle and the input generator.  Run from the repository root:

    python tests/golden/make_tiny_trace.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import run_trace  # noqa: E402
from synth import WORKLOADS, gen  # noqa: E402


def main():
    wl = WORKLOADS["tiny_fp32"]
    units = []
    for h in range(wl.heads):
        Q, K, V = gen.unit_values(wl, 0, h, 0, wl.n_positions)
        seeded, c, steps = run_trace(Q, K, V, wl.prompt, wl.steps, wl.recent, wl.heavy, wl.scale)
        units.append({
            "batch": 0, "head": h,
            "prefill_kept": sorted(seeded),
            "evicted": [s.evicted for s in steps],
            "final_members": sorted(steps[-1].members),
            # smallest gap between the two lowest candidate scores at each step
            "min_gap": [_gap(_pre(steps, i, seeded, wl)) for i in range(len(steps))],
        })
    out = {"workload": wl.name, "source": "oracle/h2o_ref.py via tests/golden/make_tiny_trace.py",
           "units": units}
    with open(os.path.join(os.path.dirname(__file__), "tiny_fp32_trace.json"), "w") as f:
        json.dump(out, f, indent=1)


def _gap(cands):
    """Difference between the two lowest candidate scores."""
    lo = sorted(cands.values())
    return lo[1] - lo[0]


def _pre(steps, i, seeded, wl):
    """Candidate scores at step i after the step's addition, before eviction."""
    prev = seeded if i == 0 else steps[i - 1].members
    res = steps[i]
    t = wl.prompt + i
    pre = {j: prev[j] + res.weights[j] for j in prev}
    pre[t] = res.weights[t]
    return {j: v for j, v in pre.items() if j <= t - wl.recent}


if __name__ == "__main__":
    main()
