"""Pins for the oracle's Algorithm 1 loop on the tiny stack."""
import itertools
from functools import lru_cache

import numpy as np
import pytest

import oracle
import synth
from oracle import balance

CFG = synth.CONFIGS["tiny"]


def _inputs(seed=0):
    w13, w2, _, _ = synth.weights_numpy(CFG, seed)
    w13 = oracle.widen(w13, CFG.dtype)
    w2 = oracle.widen(w2, CFG.dtype)
    h0 = [oracle.widen(synth.hidden(CFG, seed, j), CFG.dtype) for j in range(CFG.n)]

    def logits_fn(j, l):
        return synth.logits(CFG, seed, j, l)
    return h0, logits_fn, w13, w2


def _layer_by_layer(h0, logits_fn, w13, w2):
    outs = {}
    h = [x.copy() for x in h0]
    for j in range(CFG.n):
        for l in range(CFG.L):
            o = oracle.moe_layer(h[j], logits_fn(j, l), CFG.k, w13[l], w2[l])
            outs[(j, l)] = o
            h[j] = o["y"]
    return h, outs


@pytest.mark.parametrize("policy", ["b0", "b1", "cumutil", "maxutil", "diffpeak"])
@pytest.mark.parametrize("m", [1, 2, 3])
def test_engine_outputs_independent_of_policy(policy, m):
    h0, logits_fn, w13, w2 = _inputs()
    ref, outs = _layer_by_layer(h0, logits_fn, w13, w2)
    h, trace, acc, u = oracle.run_engine(h0, logits_fn, CFG.k, CFG.D, w13, w2, m,
                                         oracle.POLICIES[policy])
    for j in range(CFG.n):
        assert np.array_equal(h[j], ref[j])
    # Algorithm 1 invariants: each (j, l) runs once, in layer order
    seen = {j: [] for j in range(CFG.n)}
    for R, layers in trace:
        for j, l in zip(R, layers):
            seen[j].append(l)
    assert all(seen[j] == list(range(CFG.L)) for j in range(CFG.n))
    # u from the device-group workloads of the layer-by-layer run
    wt = [[oracle.group_workload(outs[(j, l)]["counts"], CFG.D) for l in range(CFG.L)]
          for j in range(CFG.n)]
    trace2, acc2, u2 = oracle.run_schedule_only(wt, CFG.n, CFG.L, CFG.D, m,
                                                oracle.POLICIES[policy])
    assert trace2 == trace and acc2 == acc and u2 == u
    base = oracle.utilization([wt[j][l] for j in range(CFG.n) for l in range(CFG.L)], CFG.D)
    assert u >= base
    if policy == "b0":
        assert u == base


def test_min_runset_and_pool_rules():
    rng = np.random.default_rng(9)
    n, L, D = 5, 6, 4
    wt = rng.integers(0, 9, size=(n, L, D)).tolist()
    for policy in ("cumutil", "maxutil", "diffpeak"):
        for m in range(1, n + 1):
            trace, acc, u = oracle.run_schedule_only(wt, n, L, D, m, oracle.POLICIES[policy])
            lj = [0] * n
            for R, layers in trace:
                live = [j for j in range(n) if lj[j] < L]
                assert len(R) >= min(m, len(live)) and set(R) <= set(live)
                assert list(layers) == [lj[j] for j in R]
                for j in R:
                    lj[j] += 1
            assert lj == [L] * n


def test_state_lattice_every_schedule_same_outputs():
    """Brute force over all schedules of the tiny stack (n=3, L=4): every path
    through the (l_0, l_1, l_2) lattice yields the layer-by-layer outputs.

    Each (j, l) output depends only on micro-batch j's own history, so it is
    enough to check every transition (state, RunSet) once: that running the
    RunSet's members together at their layers gives each member's canonical
    output.  Counting the paths confirms the lattice covers 699,121 schedules
    at m=1, 436 at m=2 and 1 at m=3."""
    h0, logits_fn, w13, w2 = _inputs(1)
    ref, outs = _layer_by_layer(h0, logits_fn, w13, w2)
    hist = {(j, 0): h0[j] for j in range(CFG.n)}
    for (j, l), o in outs.items():
        hist[(j, l + 1)] = o["y"]
    n, L = CFG.n, CFG.L
    transitions = 0
    for state in itertools.product(range(L + 1), repeat=n):
        live = [j for j in range(n) if state[j] < L]
        for r in range(1, len(live) + 1):
            for R in itertools.combinations(live, r):
                for j in R:
                    l = state[j]
                    o = oracle.moe_layer(hist[(j, l)], logits_fn(j, l), CFG.k, w13[l], w2[l])
                    assert np.array_equal(o["y"], hist[(j, l + 1)])
                transitions += 1
    assert transitions > 0

    @lru_cache(None)
    def paths(state, m):
        live = [j for j in range(n) if state[j] < L]
        if not live:
            return 1
        tot = 0
        for r in range(min(m, len(live)), len(live) + 1):
            for R in itertools.combinations(live, r):
                nxt = list(state)
                for j in R:
                    nxt[j] += 1
                tot += paths(tuple(nxt), m)
        return tot
    assert [paths((0,) * n, m) for m in (1, 2, 3)] == [699121, 436, 1]
