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

Ablation policies the pages contrast with H2O (summary, "Prior limits" and
"Limitations"), each a change of one step of the same loop:

* "static" (static Top-K without heavy-hitter dynamics): the heavy set is
  picked once; after the cache is full the victim is always the position that
  leaves the protected window, so the heavy members never change and the rest
  behaves as a sliding window.  Scores are still accumulated (they decide
  nothing).  While the cache is filling, positions are admitted as under H2O.
* "naive" (per-step Top-K without accumulation): a member's score is only the
  weight it received at the current step; the prefill ranks the prompt
  positions by the attention of the last prompt token alone.
* heavy-only is H2O with recent = 0: no protected window, so the token being
  decoded is a candidate for eviction too (positions <= t - 0).
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


def prefill_output(Q, K, V, scale):
    """Attention output of every prompt position, O = A V with A the causal
    attention matrix of the prompt (summary, "Algorithm / figure walkthrough",
    step 1: the prompt is processed with full attention over its own prefix
    before any eviction)."""
    return causal_attention(Q, K, scale) @ np.asarray(V, dtype=np.float64)


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


POLICIES = ("h2o", "static", "naive")


def prefill_scores(Q, K, scale, policy="h2o"):
    """Score of every prompt position after the prompt: the causal column sums
    (accumulated attention), or for the naive policy the attention the last
    prompt token gives each position."""
    if policy == "naive":
        return causal_attention(Q, K, scale)[-1]
    if policy not in POLICIES:
        raise ValueError(policy)
    return prefill_column_sums(Q, K, scale)


def prefill(Q, K, recent, heavy, scale, policy="h2o"):
    """Seed the cache from the prompt.  Returns ({position: score}, scores)."""
    c = prefill_scores(Q, K, scale, policy)
    return {j: float(c[j]) for j in prefill_keep(c, recent, heavy)}, c


def decode_step(members, t, q, K, V, recent, heavy, scale, K_cached=None, V_cached=None,
                policy="h2o"):
    """One decode step for the token at absolute position t.

    ``members`` maps each cached position (< t) to its score.  K and V are
    indexable by absolute position and hold rows for every member and for t
    itself.  When the cache stores rows in a lossy form, K_cached / V_cached
    give the rows as stored (indexable by position) and are used for the
    members; the token being decoded always attends with its exact row.
    Returns StepResult(out, evicted, members after the step, the softmax weight
    of each attended position, attended positions in order).

    Order of work (summary, "Algorithm / figure walkthrough", steps 2-4):
      1. attend over the members and the new token;
      2. add every weight into that position's score (naive policy: the score
         becomes the weight); the new token enters with its own weight;
      3. if the cache now exceeds k = recent + heavy, evict among the
         candidates (positions <= t - recent): the smallest score, older first
         on ties; under the static policy the newest candidate, the position
         leaving the protected window.
    """
    if policy not in POLICIES:
        raise ValueError(policy)
    q = np.asarray(q, dtype=np.float64)
    attended = sorted(members) + [t]
    Kc = K if K_cached is None else K_cached
    Vc = V if V_cached is None else V_cached
    Ka = np.asarray([Kc[j] for j in attended[:-1]] + [K[t]], dtype=np.float64)
    Va = np.asarray([Vc[j] for j in attended[:-1]] + [V[t]], dtype=np.float64)
    logits = scale * (Ka @ q)
    w = np.exp(logits - logits.max())
    p = w / w.sum()
    out = p @ Va

    keep_old = 0.0 if policy == "naive" else 1.0
    after = {j: keep_old * members[j] + float(p[i]) for i, j in enumerate(attended[:-1])}
    after[t] = float(p[-1])

    evicted = None
    if len(after) > recent + heavy:
        candidates = [j for j in after if j <= t - recent]
        if policy == "static":
            evicted = max(candidates)
        else:
            evicted = min(candidates, key=lambda j: (after[j], j))
        del after[evicted]
    weights = {j: float(p[i]) for i, j in enumerate(attended)}
    return StepResult(out, evicted, after, weights, attended)


def run_trace(Q, K, V, prompt, steps, recent, heavy, scale, cache="exact", policy="h2o"):
    """Prefill on positions [0, prompt) then ``steps`` decode steps.

    Q, K, V hold rows for positions [0, prompt + steps).  cache="e4m3" stores
    every cached row as per-row-scaled E4M3 (quantize_row_e4m3); the prefill
    scores still come from the exact prompt.  Returns (members after prefill,
    prompt scores, [StepResult per step])."""
    members, c = prefill(Q[:prompt], K[:prompt], recent, heavy, scale, policy)
    Kc = Vc = None
    if cache == "e4m3":
        Kc = np.asarray([dequantize_row_e4m3(*quantize_row_e4m3(row)) for row in K])
        Vc = np.asarray([dequantize_row_e4m3(*quantize_row_e4m3(row)) for row in V])
    elif cache != "exact":
        raise ValueError(cache)
    seeded = dict(members)
    results = []
    for s in range(steps):
        t = prompt + s
        res = decode_step(members, t, Q[t], K, V, recent, heavy, scale, Kc, Vc, policy)
        results.append(res)
        members = res.members
    return seeded, c, results


def members_from_slots(pos, score):
    """Cache set held in a slot layout: {pos[s]: score[s]} over slots with pos >= 0."""
    pos = np.asarray(pos)
    score = np.asarray(score, dtype=np.float64)
    live = pos >= 0
    return {int(p): float(s) for p, s in zip(pos[live], score[live])}


# ---- E4M3 cache rows ------------------------------------------------------------
#
# OCP 8-bit floating point, E4M3 variant without infinities: sign, 4 exponent
# bits with bias 7, 3 mantissa bits; exponent 0 holds subnormals (m/8 * 2^-6);
# 0x7F / 0xFF are NaN, so the largest finite magnitude is 448.  Conversion
# rounds to nearest with ties to the even mantissa.  A cached row x is stored
# as codes of x * (448 / amax) with amax = max |x|, and the per-row scale
# amax / 448; both quotients are float32 (the precision the kernel decides the
# codes in).  A row of zeros is stored as zero codes with scale 0.

E4M3_MAX = 448.0


def e4m3_value(codes):
    """float64 value of E4M3 codes (NaN for the two NaN codes)."""
    codes = np.asarray(codes, dtype=np.int64)
    sign = np.where(codes & 0x80, -1.0, 1.0)
    e = (codes >> 3) & 0xF
    m = codes & 7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def e4m3_encode(y):
    """Round float values to E4M3 codes (nearest, ties to even).

    Values up to the midpoint between 448 and the next step of the grid (464)
    round to 448; a row scaled by the float32 quotient 448 / amax can exceed 448
    by an ulp."""
    y = np.asarray(y, dtype=np.float64)
    if np.any(np.abs(y) >= 464.0):
        raise ValueError("value outside the E4M3 range")
    sign = np.signbit(y).astype(np.int64) << 7
    a = np.abs(y)
    codes = np.empty(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormal range: multiples of 2^-9; a result of 8 is the smallest normal, code 8
    codes[sub] = np.rint(a[sub] / 2.0 ** -9).astype(np.int64)
    an = a[~sub]
    e = np.floor(np.log2(an)).astype(np.int64)
    q = np.rint(an / np.exp2(e - 3.0)).astype(np.int64)   # 8 .. 16
    carry = q == 16
    e = e + carry
    q = np.where(carry, 8, q)
    codes[~sub] = ((e + 7) << 3) | (q - 8)
    return (codes | sign).astype(np.uint8)


def quantize_row_e4m3(x):
    """One cached row -> (E4M3 codes, float32 scale)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x)))
    if amax == 0:
        return np.zeros(x.shape, dtype=np.uint8), np.float32(0.0)
    inv = np.float32(E4M3_MAX) / amax
    s = amax / np.float32(E4M3_MAX)
    return e4m3_encode((x * inv).astype(np.float32)), np.float32(s)


def dequantize_row_e4m3(codes, s):
    """Exact float64 value of a stored row: code value times the row scale."""
    return e4m3_value(codes) * np.float64(s)
