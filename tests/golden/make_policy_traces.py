"""Writes tiny_fp32_policy_traces.json: the oracle's own free-running
trajectories on the tiny fp32 workload (1 x 2 heads, d 64, prompt 64, 64
steps) for the ablation policies: static Top-K and naive per-step Top-K with
the workload's budget (16 recent + 16 heavy), and heavy-only (recent = 0,
32 heavy) under the H2O and naive policies.

A regression record of the oracle (pinned by tests/test_oracle_pins.py), not
values from the pages, which print no worked example.  This script calls only
the oracle and the input generator.  Run from the repository root:

    python tests/golden/make_policy_traces.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import run_trace  # noqa: E402
from synth import WORKLOADS, gen  # noqa: E402

CASES = [  # (policy, recent, heavy)
    ("static", 16, 16),
    ("naive", 16, 16),
    ("h2o", 0, 32),
    ("naive", 0, 32),
]


def min_gap(policy, prev, res, t, recent):
    """Smallest gap between the two lowest candidate scores at a step (None for
    the static policy, whose victim is fixed by position)."""
    if policy == "static" or res.evicted is None:
        return None
    keep = 0.0 if policy == "naive" else 1.0
    pre = {j: keep * prev[j] + res.weights[j] for j in prev}
    pre[t] = res.weights[t]
    lo = sorted(v for j, v in pre.items() if j <= t - recent)
    return lo[1] - lo[0]


def main():
    wl = WORKLOADS["tiny_fp32"]
    cases = []
    for policy, recent, heavy in CASES:
        units = []
        for h in range(wl.heads):
            Q, K, V = gen.unit_values(wl, 0, h, 0, wl.n_positions)
            seeded, _, steps = run_trace(Q, K, V, wl.prompt, wl.steps, recent, heavy, wl.scale, policy=policy)
            gaps = []
            prev = seeded
            for i, res in enumerate(steps):
                gaps.append(min_gap(policy, prev, res, wl.prompt + i, recent))
                prev = res.members
            units.append({"batch": 0, "head": h, "prefill_kept": sorted(seeded),
                          "evicted": [s.evicted for s in steps], "final_members": sorted(steps[-1].members),
                          "min_gap": gaps})
        cases.append({"policy": policy, "recent": recent, "heavy": heavy, "units": units})
    out = {"workload": wl.name, "source": "oracle/h2o_ref.py via tests/golden/make_policy_traces.py",
           "cases": cases}
    with open(os.path.join(os.path.dirname(__file__), "tiny_fp32_policy_traces.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
