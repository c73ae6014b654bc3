"""Plain float64 CPU oracle of the H2O (Heavy-Hitter Oracle) decode step and prefill.

TEST INFRASTRUCTURE.  Only the tests, the smoke check of the graft entry and
the CPU-baseline leg of the benchmark may import this module.  The library and
its Python binding never do, and this module imports nothing from them.

Everything works on one (batch, head) unit at a time, in float64, with the
cache held as a set of absolute positions mapped to accumulated scores (no slot
layout).  K and V rows are looked up by absolute position in the caller's
input arrays.

Sources (the pages on H2O; "summary" is the Fanout Daily page "H2O:
Heavy-Hitter Oracle for Efficient Generative Inference", "abstract" the
paper's abstract as carried by the codewithpapers and mlsanity pages):

* summary, "The mechanism", Heavy Hitters: the score of a cached token is the
  sum of the softmax attention weights it has received.
* summary, "The mechanism", H2O eviction and Definition 4.3: a budget of k
  cached tokens; admit while not full; once full admit the newest token and
  evict the lowest-scoring member outside a protected block of recent tokens;
  at most one membership change per step.
* summary, "Algorithm / figure walkthrough", steps 1-5: prefill seeds the
  scores; each decode step attends over the cache, adds the weights into the
  scores, appends the new token, evicts if over budget; memory stays O(k).

Readings taken where the pages leave a step open:

* The token being decoded attends to the cached set plus itself (up to k+1
  keys) before any eviction; this is the only reading under which a budget at
  least the sequence length gives full causal attention.
* The protected window is the r newest positions including the current one,
  so the candidates at step t are the members at positions <= t - r.
* This step's weights are added before the eviction decision; the new token's
  score starts at its own weight.
* Softmax scale is an input (1/sqrt(d) by default on the caller's side).
* One total order (score, position) breaks ties: the eviction argmin takes the
  older position on equal scores, and the prefill top-h keeps the newer one.
* Prefill scores are the column sums of the exact causal attention of the whole
  prompt; if the prompt exceeds k, the newest r prompt positions are kept and
  the h best of the rest by that order.
"""
from collections import namedtuple

import numpy as np

StepResult = namedtuple("StepResult", "out evicted members weights attended")


def causal_attention(Q, K, scale):
    """Row-stochastic causal attention matrix of one unit.

    A[i, j] = exp(s_ij) / sum_{j' <= i} exp(s_ij') with s = scale * Q K^T and
    j <= i (zero above the diagonal).  Rows are shifted by their maximum before
    exponentiation, which leaves the quotient unchanged."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    n = Q.shape[0]
    S = scale * (Q @ K.T)
    S = np.where(np.tril(np.ones((n, n), dtype=bool)), S, -np.inf)
    S = S - S.max(axis=1, keepdims=True)
    E = np.exp(S)
    return E / E.sum(axis=1, keepdims=True)


def prefill_column_sums(Q, K, scale):
    """Accumulated attention of every prompt position after the prompt:
    c_j = sum over query rows i >= j of A[i, j]  (summary, "The mechanism",
    Heavy Hitters; "Algorithm / figure walkthrough", step 1)."""
    return causal_attention(Q, K, scale).sum(axis=0)


def prefill_keep(c, recent, heavy):
    """Positions kept after the prompt (sorted).

    A prompt that fits the budget k = recent + heavy is kept whole.  Otherwise
    the newest ``recent`` positions form the protected block and the ``heavy``
    positions with the largest scores among the older ones are kept, ties going
    to the newer position (summary, "Algorithm / figure walkthrough", step 1;
    "The mechanism", H2O eviction)."""
    n = len(c)
    if n <= recent + heavy:
        return list(range(n))
    older = range(n - recent)
    ranked = sorted(older, key=lambda j: (-c[j], -j))
    return sorted(ranked[:heavy]) + list(range(n - recent, n))


def prefill(Q, K, recent, heavy, scale):
    """Seed the cache from the prompt.  Returns ({position: score}, c)."""
    c = prefill_column_sums(Q, K, scale)
    return {j: float(c[j]) for j in prefill_keep(c, recent, heavy)}, c


def decode_step(members, t, q, K, V, recent, heavy, scale):
    """One H2O decode step for the token at absolute position t.

    ``members`` maps each cached position (< t) to its accumulated score.  K and
    V are indexable by absolute position and hold rows for every member and for
    t itself.  Returns StepResult(out, evicted, members after the step, the
    softmax weight of each attended position, attended positions in order).

    Order of work (summary, "Algorithm / figure walkthrough", steps 2-4):
      1. attend over the members and the new token;
      2. add every weight into that position's score; the new token enters with
         its own weight;
      3. if the cache now exceeds k = recent + heavy, evict the candidate
         (position <= t - recent) with the smallest score, older first on ties.
    """
    q = np.asarray(q, dtype=np.float64)
    attended = sorted(members) + [t]
    Ka = np.asarray([K[j] for j in attended], dtype=np.float64)
    Va = np.asarray([V[j] for j in attended], dtype=np.float64)
    logits = scale * (Ka @ q)
    w = np.exp(logits - logits.max())
    p = w / w.sum()
    out = p @ Va

    after = {j: members[j] + float(p[i]) for i, j in enumerate(attended[:-1])}
    after[t] = float(p[-1])

    evicted = None
    if len(after) > recent + heavy:
        candidates = [j for j in after if j <= t - recent]
        evicted = min(candidates, key=lambda j: (after[j], j))
        del after[evicted]
    weights = {j: float(p[i]) for i, j in enumerate(attended)}
    return StepResult(out, evicted, after, weights, attended)


def run_trace(Q, K, V, prompt, steps, recent, heavy, scale):
    """Prefill on positions [0, prompt) then ``steps`` decode steps.

    Q, K, V hold rows for positions [0, prompt + steps).  Returns
    (members after prefill, prompt column sums, [StepResult per step])."""
    members, c = prefill(Q[:prompt], K[:prompt], recent, heavy, scale)
    seeded = dict(members)
    results = []
    for s in range(steps):
        t = prompt + s
        res = decode_step(members, t, Q[t], K, V, recent, heavy, scale)
        results.append(res)
        members = res.members
    return seeded, c, results


def members_from_slots(pos, score):
    """Cache set held in a slot layout: {pos[s]: score[s]} over slots with pos >= 0."""
    pos = np.asarray(pos)
    score = np.asarray(score, dtype=np.float64)
    live = pos >= 0
    return {int(p): float(s) for p, s in zip(pos[live], score[live])}
