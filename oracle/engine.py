"""Oracle: one MoE layer end to end, and Algorithm 1 of [PAPER].

Pins (tests/test_oracle_engine.py):
* the loop invariants of [PAPER] §4.1-§4.2 (each l_j rises by one per
  selected step, |RunSet| >= min(m, |S|), termination after L steps per
  batch), checked on every step;
* outputs do not depend on the schedule ([PAPER] §4.1: lossless as long as
  each micro-batch keeps its own layer order), by brute force over every
  path of the (l_0, l_1, l_2) state lattice of a tiny stack;
* the per-layer baseline reproduces Eq. (3) computed layer by layer.
Pins (tests/test_oracle_eq1.py):
* moe_layer equals Eq. (1) of [PAPER] §2.1 evaluated token by token (brute
  force top-k, torch's rms_norm / silu / linear per token, the residual from
  the raw state), with and without the pre-norm block and shared experts;
* run_engine, with the pre-norm block and with the router in front of top-k,
  equals each token followed through every layer alone by that evaluation.
"""
from __future__ import annotations

import numpy as np

from . import moe
from .balance import group_workload, schedule, step_stats, utilization, combined


def moe_layer(h, logits, k, w13_l, w2_l, w13s_l=None, w2s_l=None, prenorm=False,
              eps=1e-6):
    """One MoE layer on hidden rows h (float64 [T, H]).

    [PAPER] §2.1 with attention taken as the identity (h' = h):
        route -> dispatch -> experts -> Eq. (1) combine -> residual.
    prenorm: the experts read rmsnorm(h), the residual is h itself.
    Returns a dict with every intermediate (float64 for values).
    """
    E = w13_l.shape[0]
    xin = moe.rmsnorm(h, eps) if prenorm else h
    idx, gates = moe.route(logits, k)
    counts, offsets, dest, src = moe.dispatch(idx, E)
    xp = moe.permute_rows(xin, src, k)
    yp = moe.expert_ffn(xp, offsets, w13_l, w2_l)
    ysh = None
    if w13s_l is not None and len(w13s_l):
        ysh = [moe.swiglu_expert(xin, w13s_l[s], w2s_l[s]) for s in range(len(w13s_l))]
    y = moe.combine(yp, dest, gates, k, y_shared=ysh, residual=h)
    return dict(idx=idx, gates=gates, counts=counts, offsets=offsets, dest=dest, src=src,
                xp=xp, yp=yp, y_shared=ysh, y=y)


def _algorithm1(n, L, m, policy, start_layers, route_layer, run_layer):
    """The EasyBalance loop ([PAPER] Algorithm 1; [REVIEW] §2.3).

    route_layer(j, l) -> workload vector of micro-batch j at layer l (the
    AttnRouteDispatch of the pages); run_layer(j, l) does MoECompute_Combine
    for j.  The initial RunSet_0 is the whole pool, so every unfinished batch
    is routed before the first Schedule.
    """
    lj = list(start_layers) if start_layers else [0] * n
    S = [j for j in range(n) if lj[j] < L]
    prev = list(S)
    w = {}
    trace, steps_W = [], []
    num = den = sep = 0
    while S:
        for j in prev:
            if lj[j] < L:
                w[j] = route_layer(j, lj[j])
        R = schedule(w, S, m, policy)
        assert len(R) >= min(m, len(S)) or policy == 0
        assert set(R) <= set(S)
        for j in R:
            run_layer(j, lj[j])
        a, b, c = step_stats([w[j] for j in R])
        num, den, sep = num + a, den + b, sep + c
        steps_W.append(combined([w[j] for j in R]))
        trace.append((tuple(R), tuple(lj[j] for j in R)))
        for j in R:
            lj[j] += 1
        S = [j for j in S if lj[j] < L]
        prev = list(R)
    return trace, steps_W, (num, den, sep)


def run_schedule_only(w_table, n, L, D, m, policy, start_layers=None):
    """Algorithm 1 driven by precomputed workloads w_table[j][l] (length D).

    Under the reading that router logits are inputs, routing does not depend
    on the hidden state, so the schedule and u follow from the workloads
    alone.  Returns (trace, (num, den, sep), u) with u an exact Fraction.
    """
    trace, steps_W, acc = _algorithm1(n, L, m, policy, start_layers,
                                      lambda j, l: list(w_table[j][l]), lambda j, l: None)
    return trace, acc, utilization(steps_W, D)


def run_engine(h0, logits_fn, k, D, w13, w2, m, policy, w13s=None, w2s=None,
               start_layers=None, prenorm=False, eps=1e-6, router=None):
    """Algorithm 1 with the full MoE math.

    h0: list of float64 [T_j, H]; logits_fn(j, l) -> float32 [T_j, E];
    w13 [L, E, 2I, H], w2 [L, E, H, I] float64 (shared: [L, S, ...]).
    prenorm: the router and the experts read rmsnorm(h), the residual is h
    (see moe_layer).  router: None (the logits are given by logits_fn), or
    (w_gate [L, E, H], bias [L, E] | None) float64: a micro-batch is routed
    from its current state, z = x W_g[l]^T + b[l] with x the block input
    ([PAPER] §2.1, G(h'_l)), rounded to float32 as the top-k input.
    Returns (h_final list, trace, (num, den, sep), u).
    """
    n, L = len(h0), w13.shape[0]
    h = [np.array(x, dtype=np.float64) for x in h0]
    pending = {}

    def scores(j, l):
        if router is None:
            return logits_fn(j, l)
        x = moe.rmsnorm(h[j], eps) if prenorm else h[j]
        wg, bias = router
        return moe.gate_logits(x, wg[l], None if bias is None else bias[l]).astype(np.float32)

    def route_layer(j, l):
        # AttnRouteDispatch: micro-batch j is at layer l and h[j] is that
        # layer's input; its scores are kept for the layer's run
        z = scores(j, l)
        idx, _ = moe.route(z, k)
        counts, *_ = moe.dispatch(idx, w13.shape[1])
        pending[j] = (l, z)
        return group_workload(counts, D)

    def run_layer(j, l):
        lp, z = pending[j]
        assert lp == l
        out = moe_layer(h[j], z, k, w13[l], w2[l],
                        None if w13s is None else w13s[l], None if w2s is None else w2s[l],
                        prenorm=prenorm, eps=eps)
        h[j] = out["y"]

    trace, steps_W, acc = _algorithm1(n, L, m, policy, start_layers, route_layer, run_layer)
    return h, trace, acc, utilization(steps_W, D)
