"""Writes llama7b_stream_trace.json: the oracle's own free-running trajectory
over the first 2000 decode steps of the long-stream workload (LLaMA-7B-shaped
heads, k = 256 = 128 recent + 128 heavy, Zipf skew recurring every 5000
positions) for heads 0-3 of batch 0.

Unlike the tiny trace, many of these evictions remove a heavy member rather
than the position leaving the protected window: the accumulated scores re-rank
the heavy slots (summary "H2O: Heavy-Hitter Oracle for Efficient Generative
Inference", "Algorithm / figure walkthrough", the contrast of Full, Local and
H2O), which a sliding window or a static Top-K never does.

The pages print no worked numeric example, so this is not a value from the
pages: it is a regression record of the oracle (pinned by
tests/test_oracle_pins.py), produced by this script, which calls only the
oracle and the input generator.  Run from the repository root:

    python tests/golden/make_stream_trace.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import decode_step, prefill  # noqa: E402
from synth import WORKLOADS, gen  # noqa: E402

STEPS = 2000
HEADS = (0, 1, 2, 3)


def main():
    wl = WORKLOADS["llama7b_stream"]
    P, r, h = wl.prompt, wl.recent, wl.heavy
    units = []
    for head in HEADS:
        Q, K, V = gen.unit_values(wl, 0, head, 0, P + STEPS)
        members, _ = prefill(Q[:P], K[:P], r, h, wl.scale)
        kept = sorted(members)
        evicted, gaps = [], []
        for s in range(STEPS):
            t = P + s
            res = decode_step(members, t, Q[t], K, V, r, h, wl.scale)
            # candidate scores after the step's addition, before the eviction
            pre = {j: members[j] + res.weights[j] for j in members}
            pre[t] = res.weights[t]
            cands = sorted(v for j, v in pre.items() if j <= t - r)
            gaps.append(float(f"{cands[1] - cands[0]:.3g}"))
            evicted.append(res.evicted)
            members = res.members
        units.append({
            "batch": 0, "head": head,
            "prefill_kept": kept,
            "evicted": evicted,
            "heavy_evictions": sum(e != P + s - r for s, e in enumerate(evicted)),
            "final_members": sorted(members),
            # gap between the two lowest candidate scores at each step (3 digits)
            "min_gap": gaps,
        })
    out = {"workload": wl.name, "steps": STEPS,
           "source": "oracle/h2o_ref.py via tests/golden/make_stream_trace.py", "units": units}
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "llama7b_stream_trace.json"), "w") as f:
        json.dump(out, f, separators=(",", ":"))


if __name__ == "__main__":
    main()
