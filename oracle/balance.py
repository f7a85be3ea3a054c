"""Oracle: workload statistics (Eq. 2, Eq. 3) and the RunSet policies.

Pins (tests/test_oracle_balance.py):
* effective_workload / utilization -- the review's eight-device example
  (10, 9, ..., 3 -> effective workload 10; u = 52/80 follows from Eq. (3));
  the sum-of-max inequality of [PAPER] §4.1 on random workloads; an
  independent closed form of Eq. (3) on per-layer steps; u of any schedule is
  at least u of the one-(micro-batch, layer)-per-step baseline.
* same_peak_windows -- hand-counted sequences (tests/test_oracle_balance.py).
* schedule -- hand-worked examples (tests/golden/schedule_examples.json) whose
  expected picks are derived by hand there; MaxUtil against an independent
  brute force (exhaustive ``itertools`` search with a different tie-break
  formulation); CumUtil's strict-increase rule checked step by step.
"""
from __future__ import annotations

import itertools
from fractions import Fraction

import numpy as np

B0_ALONE, B1_LOCKSTEP, CUMUTIL, MAXUTIL, DIFFPEAK = 0, 1, 2, 3, 4
POLICIES = {"b0": B0_ALONE, "b1": B1_LOCKSTEP, "cumutil": CUMUTIL, "maxutil": MAXUTIL,
            "diffpeak": DIFFPEAK}


def group_workload(counts: np.ndarray, D: int) -> list:
    """w_d = number of (token, expert) assignments whose expert lies in group d.

    [PAPER] §2.3: w^(l) = (w_1, ..., w_D) is the MoE workload across D devices;
    the even expert-device mapping puts a contiguous block of E/D experts on
    each device ([PAPER] Figure 1).  Reading: assignments are counted, group
    d holds experts [d*E/D, (d+1)*E/D).
    """
    counts = [int(c) for c in np.asarray(counts).reshape(-1)]
    E = len(counts)
    if D < 1 or E % D:
        raise ValueError("E must be a multiple of D")
    g = E // D
    return [sum(counts[d * g:(d + 1) * g]) for d in range(D)]


def effective_workload(w) -> int:
    """[PAPER] Eq. (2): the step waits for the heaviest device, w_hat = max_d w_d."""
    return max(int(v) for v in w)


def combined(ws) -> list:
    """Devicewise sum of several workload vectors run in one step."""
    ws = [list(map(int, w)) for w in ws]
    return [sum(col) for col in zip(*ws)]


def util_of(W) -> Fraction:
    """U of one combined workload vector: sum_d W_d / (D * max_d W_d).

    Eq. (3) of [PAPER] restricted to a single step; 0 for an all-zero vector
    (a step with no work uses nothing; reading for the degenerate case).
    """
    W = [int(v) for v in W]
    mx = max(W)
    if mx == 0:
        return Fraction(0)
    return Fraction(sum(W), len(W) * mx)


def step_stats(ws) -> tuple:
    """(sum_d W_d, max_d W_d, sum_j max_d w_jd) for the micro-batches of one step.

    The third value is the effective workload had each member run alone,
    the right-hand side of the inequality in [PAPER] §4.1 (and the
    "max workload sum" curve of its Figure 6)."""
    W = combined(ws)
    return sum(W), max(W), sum(max(map(int, w)) for w in ws)


def utilization(steps_W, D: int) -> Fraction:
    """[PAPER] Eq. (3) over a sequence of steps:
        u = sum_i sum_d W_{i,d} / (D * sum_i max_d W_{i,d}),
    with W_i the combined workload of step i.  When each step is one layer of
    one batch this is Eq. (3) verbatim."""
    num = sum(sum(int(v) for v in W) for W in steps_W)
    den = sum(max(int(v) for v in W) for W in steps_W)
    return Fraction(num, D * den)


def same_peak_windows(w_layers, run: int) -> tuple:
    """(hits, windows) of the [PAPER] Table 2 statistic for one workload sequence.

    w_layers: the per-layer workload vectors of one micro-batch, in layer
    order.  A window is ``run`` consecutive layers; it is a hit when every
    layer in it has the same peak device.  [PAPER] §1 and §4.1 explain why
    such windows are rare (a hot device in one layer is seldom hot in the
    next).  Readings: the peak device is the lowest index among equal maxima
    (as DiffPeak), and windows are counted per micro-batch.
    """
    peaks = [_argmax_low(w) for w in w_layers]
    windows = max(0, len(peaks) - run + 1)
    hits = 0
    for s in range(windows):
        if all(peaks[s + q] == peaks[s] for q in range(run)):
            hits += 1
    return hits, windows


# ---------------------------------------------------------------- policies
def _pad(chosen, ready, m):
    """Top up a greedy pick to the minimum size m with the lowest-id
    candidates it left out (reading: the pages do not say how the linear
    policies meet the |RunSet| >= m rule)."""
    chosen = list(chosen)
    for j in ready:
        if len(chosen) >= m:
            break
        if j not in chosen:
            chosen.append(j)
    return tuple(sorted(chosen))


def _argmax_low(w) -> int:
    w = [int(v) for v in w]
    best = 0
    for d in range(1, len(w)):
        if w[d] > w[best]:
            best = d
    return best


def schedule(w, ready, m: int, policy: int) -> tuple:
    """Schedule(S, m) of [PAPER] Algorithm 1: pick RunSet from the pool.

    ``w`` is indexable by micro-batch id (each a length-D workload vector),
    ``ready`` the ids of the pool S in any order.  Returns the sorted ids.

    [PAPER] §4.2: |RunSet| >= m; if |S| < m every ready batch runs.
    Policies ([PAPER] §5.2, [REVIEW] §2.4):
      B0_ALONE    -- one batch per step (lowest ready id): no cross-layer
                     combination, the baseline.  Ignores m.
      B1_LOCKSTEP -- every ready batch.  Ignores m.
      CUMUTIL     -- scan ready ids ascending; the first is always taken; a
                     later one joins iff U strictly rises.  Then pad to m.
      MAXUTIL     -- among subsets R of S with |R| >= m (S itself if
                     |S| < m) maximise U; ties: larger |R|, then the
                     lexicographically smallest sorted id tuple.
      DIFFPEAK    -- scan ready ids ascending; the first is always taken; a
                     later one joins iff its peak device (lowest index among
                     equal maxima) is not a peak of a chosen one.  Then pad to m.
    """
    ready = sorted(int(j) for j in ready)
    if not ready:
        raise ValueError("empty pool")
    if m < 1:
        raise ValueError("m must be >= 1")
    if policy == B0_ALONE:
        return (ready[0],)
    if policy == B1_LOCKSTEP or len(ready) < m:
        return tuple(ready)
    if policy == CUMUTIL:
        chosen = [ready[0]]
        for j in ready[1:]:
            before = util_of(combined([w[c] for c in chosen]))
            after = util_of(combined([w[c] for c in chosen] + [w[j]]))
            if after > before:
                chosen.append(j)
        return _pad(chosen, ready, m)
    if policy == DIFFPEAK:
        chosen = [ready[0]]
        peaks = {_argmax_low(w[ready[0]])}
        for j in ready[1:]:
            p = _argmax_low(w[j])
            if p not in peaks:
                chosen.append(j)
                peaks.add(p)
        return _pad(chosen, ready, m)
    if policy == MAXUTIL:
        best, best_u = None, None
        # larger sets first; itertools.combinations yields sorted tuples in
        # lexicographic order, so a strict '>' keeps the tie-break winner
        for size in range(len(ready), m - 1, -1):
            for R in itertools.combinations(ready, size):
                u = util_of(combined([w[j] for j in R]))
                if best_u is None or u > best_u:
                    best, best_u = R, u
        return tuple(best)
    raise ValueError(f"unknown policy {policy}")
