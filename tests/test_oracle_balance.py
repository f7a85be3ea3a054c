"""Pins for the oracle's workload statistics and RunSet policies."""
import itertools
import json
import os
import random
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import balance

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_worked_example_eq2_eq3():
    g = _load("eq2_worked_example.json")
    # feed the example through per-expert counts: 2 experts per device
    counts = []
    for v in g["w"]:
        counts += [v - v // 2, v // 2]
    w = oracle.group_workload(np.array(counts), g["D"])
    assert w == g["w"]
    assert oracle.effective_workload(w) == g["w_hat"]
    u = oracle.utilization([w], g["D"])
    assert u == Fraction(g["u_num"], g["u_den"])
    assert 1 - u == Fraction(35, 100)


def test_group_workload_contiguous_blocks():
    counts = np.arange(12)
    assert oracle.group_workload(counts, 3) == [0 + 1 + 2 + 3, 4 + 5 + 6 + 7, 8 + 9 + 10 + 11]
    assert oracle.group_workload(counts, 12) == list(range(12))
    with pytest.raises(ValueError):
        oracle.group_workload(counts, 5)


def test_eq3_closed_form_per_layer():
    rng = np.random.default_rng(0)
    D, L = 8, 20
    w = rng.integers(0, 50, size=(L, D))
    w[:, 0] += 1
    u = oracle.utilization([list(r) for r in w], D)
    # Eq. (3) written as totals: all work / (devices x sum of per-layer peaks)
    assert u == Fraction(int(w.sum()), D * int(w.max(axis=1).sum()))
    assert Fraction(1, D) <= u <= 1


def test_sum_of_max_inequality():
    rng = np.random.default_rng(1)
    for _ in range(500):
        n, D = rng.integers(1, 7), rng.integers(1, 9)
        ws = rng.integers(0, 30, size=(n, D))
        a, b, c = oracle.step_stats([list(r) for r in ws])
        assert b == ws.sum(axis=0).max() and a == ws.sum()
        assert b <= c == ws.max(axis=1).sum()
        peaks = {int(np.argmax(r)) for r in ws}
        if b < c:
            # strict only when the peaks of the members do not all coincide
            assert len(peaks) > 1


@pytest.mark.parametrize("ex", _load("schedule_examples.json")["examples"], ids=lambda e: e["name"])
def test_schedule_hand_examples(ex):
    ready = ex.get("ready", list(range(len(ex["w"]))))
    for name, want in ex["expect"].items():
        got = oracle.schedule(ex["w"], ready, ex["m"], oracle.POLICIES[name])
        assert list(got) == want, name


def _brute_maxutil(w, ready, m):
    ready = sorted(ready)
    if len(ready) < m:
        return tuple(ready)
    cands = []
    for mask in range(1, 1 << len(ready)):
        R = tuple(ready[i] for i in range(len(ready)) if mask >> i & 1)
        if len(R) < m:
            continue
        W = [sum(w[j][d] for j in R) for d in range(len(w[0]))]
        U = Fraction(sum(W), len(W) * max(W)) if max(W) else Fraction(0)
        cands.append((-U, -len(R), R))
    return min(cands)[2]


def test_maxutil_brute_force():
    rnd = random.Random(2)
    for _ in range(300):
        n, D = rnd.randint(1, 7), rnd.randint(1, 6)
        w = [[rnd.choice([0, 0, 1, 2, 3, 5, 8]) for _ in range(D)] for _ in range(n)]
        ready = [j for j in range(n) if rnd.random() < 0.8] or [0]
        m = rnd.randint(1, n)
        assert oracle.schedule(w, ready, m, balance.MAXUTIL) == _brute_maxutil(w, ready, m)


def test_cumutil_rule_step_by_step():
    rnd = random.Random(3)
    for _ in range(300):
        n, D = rnd.randint(1, 8), rnd.randint(2, 6)
        w = [[rnd.randint(0, 9) for _ in range(D)] for _ in range(n)]
        m = rnd.randint(1, n)
        R = oracle.schedule(w, range(n), m, balance.CUMUTIL)
        # replay the scan: accepted ids raise U strictly, rejected ones do not
        chosen = [0]
        for j in range(1, n):
            cur = balance.util_of(balance.combined([w[c] for c in chosen]))
            new = balance.util_of(balance.combined([w[c] for c in chosen] + [w[j]]))
            if new > cur:
                chosen.append(j)
        assert set(chosen) <= set(R)
        extra = sorted(set(R) - set(chosen))
        rejected = [j for j in range(n) if j not in chosen]
        assert extra == rejected[:len(extra)]
        assert len(R) == max(len(chosen), min(m, n))


def test_any_schedule_not_worse_than_per_layer_baseline():
    """u of every schedule >= u of running each (batch, layer) alone: each
    (j, l) runs in exactly one step and a step's peak is at most the sum of
    its members' peaks ([PAPER] §4.1)."""
    rng = np.random.default_rng(4)
    n, L, D = 3, 3, 4
    wt = rng.integers(0, 6, size=(n, L, D))
    wt[..., 0] += 1
    base = oracle.utilization([wt[j, l] for j in range(n) for l in range(L)], D)
    seen = 0

    def walk(state, steps):
        nonlocal seen
        live = [j for j in range(n) if state[j] < L]
        if not live:
            u = oracle.utilization(steps, D)
            assert u >= base
            seen += 1
            return
        for r in range(1, len(live) + 1):
            for R in itertools.combinations(live, r):
                W = [sum(int(wt[j, state[j], d]) for j in R) for d in range(D)]
                nxt = list(state)
                for j in R:
                    nxt[j] += 1
                walk(tuple(nxt), steps + [W])

    walk((0, 0, 0), [])
    assert seen > 1000


def test_same_peak_windows_hand_counted():
    """Table 2 statistic on a hand-counted sequence.  Peaks per layer:
    0, 0, 1, 0 (a tie, lowest index), 0.  Pairs: (0,0) hit, (0,1), (1,0),
    (0,0) hit -> 2 of 4.  Triples: none of 3.  Single layers: 5 of 5."""
    w = [[5, 1], [6, 2], [1, 7], [3, 3], [9, 0]]
    assert oracle.same_peak_windows(w, 2) == (2, 4)
    assert oracle.same_peak_windows(w, 3) == (0, 3)
    assert oracle.same_peak_windows(w, 1) == (5, 5)
    assert oracle.same_peak_windows(w[:1], 2) == (0, 0)
    # one device hot on every layer: every window is a hit
    assert oracle.same_peak_windows([[0, 4, 1]] * 6, 3) == (4, 4)


def test_same_peak_windows_independent_layers():
    """Layers whose peak device is uniform and independent: the pair rate is
    1/D and the triple rate 1/D^2 (binomial bounds, 6 sigma)."""
    rng = np.random.default_rng(11)
    D, L, reps = 8, 48, 400
    hits2 = win2 = hits3 = win3 = 0
    for _ in range(reps):
        peaks = rng.integers(0, D, L)
        w = [[10 if d == p else int(rng.integers(0, 10)) for d in range(D)] for p in peaks]
        h, n = oracle.same_peak_windows(w, 2)
        hits2, win2 = hits2 + h, win2 + n
        h, n = oracle.same_peak_windows(w, 3)
        hits3, win3 = hits3 + h, win3 + n
    assert win2 == reps * (L - 1) and win3 == reps * (L - 2)
    for hits, n, p in ((hits2, win2, 1 / D), (hits3, win3, 1 / D ** 2)):
        assert abs(hits / n - p) <= 6 * (p * (1 - p) / n) ** 0.5, (hits, n, p)
