"""Algorithm 1 of EasyBalance driven through libcle.

"EasyBalance: Cross-Layer Load Balancing in Distributed MoE Inference",
Algorithm 1 (§4.2): every micro-batch T_j keeps its current layer l_j; each
step routes and dispatches the micro-batches run in the previous step
(AttnRouteDispatch), picks RunSet_i from the pool (Schedule(S, m)), runs the
experts of every RunSet member -- each at its own layer -- in one grouped
launch and combines them (MoECompute_Combine), then advances l_j of the
members and drops finished micro-batches.

Attention is outside the MoE step and taken as the identity, so a layer is
h <- h + MoE_l(h).  Router logits are inputs (one [T, E] block per
(micro-batch, layer)).  All per-micro-batch state lives in HBM; the only
device-to-host traffic per step is the n x D workload matrix the host
scheduler reads (n*D int32).
"""
from __future__ import annotations

import numpy as np
import torch

from . import (BF16, LOOP_STATE_BYTES, OP_DISPATCH, OP_DISPATCH_MANY, OP_FFN, W_PACKED,
               W_ROWMAJOR, LoopDesc, combine, combine_many, dispatch, dispatch_many,
               NORM_EPS, gate_logits_many, grouped_expert_ffn, ids_of, loop_init, loop_step,
               make_desc, mask_of, rmsnorm_many,
               read_loop_state, route, route_many, schedule_step_raw, workload_stats,
               workspace_bytes)


class Engine:
    """Device-resident state of n micro-batches moving through an L-layer MoE stack.

    weights: (w13 [L,E,2I,H], w2 [L,E,H,I], w13_shared | None, w2_shared | None),
    row-major, or all four packed by pack_weights (then packed=True),
    logits: tensor [n, L, T, E] float32 on the device, or None with `gate`;
    h0: tensor [n, T, H];
    gate: None, or (w_gate [L, E, H], bias [L, E] float32 | None): routing
    from the hidden state through the linear router of each layer instead of
    the given logits (w_gate packed too when packed=True).
    prenorm: the router and the experts read the RMS-normalised rows of h
    (kept in xn), the combine adds to h itself (a pre-norm block).
    """

    def __init__(self, weights, logits, h0, D, k, policy, m, start_layers=None, stream=None,
                 fused_gather=True, batched=True, packed=False, device_loop=False, restart=False,
                 log_cap=4096, gate=None, prenorm=False):
        self.w13, self.w2, self.w13s, self.w2s = weights
        self.packed = packed  # the weights were written by pack_weights (bf16)
        self.L, self.E, I2, self.H = self.w13.shape
        self.I = I2 // 2
        self.ns = 0 if self.w13s is None else self.w13s.shape[1]
        self.logits = logits
        self.wg, self.gbias = gate if gate is not None else (None, None)
        if logits is None and self.wg is None:
            raise ValueError("either router logits or a router (gate) is needed")
        self.n, self.T = h0.shape[0], h0.shape[1]
        self.k, self.D, self.policy, self.m = k, D, int(policy), m
        self.start = list(start_layers) if start_layers else [0] * self.n
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        dev, dt = h0.device, h0.dtype
        n, T, H, I, E, A = self.n, self.T, self.H, self.I, self.E, self.T * k
        i32 = dict(dtype=torch.int32, device=dev)
        self.h0 = h0
        self.h = h0.clone()
        self.prenorm = bool(prenorm)
        self.xn = torch.empty_like(self.h) if self.prenorm else None
        self.xin = self.xn if self.prenorm else self.h  # what the router and experts read
        self.idx = torch.empty((n, T, k), **i32)
        self.gates = torch.empty((n, T, k), dtype=torch.float32, device=dev)
        self.counts = torch.zeros((n, E), **i32)
        self.offsets = torch.zeros((n, E + 1), **i32)
        self.dest = torch.empty((n, A), **i32)
        self.src = torch.empty((n, A), **i32)
        # fused_gather: the expert launch reads token rows through src, so the
        # expert-sorted copy xp is never materialised
        self.fused = fused_gather
        # batched: route, dispatch and combine of a whole RunSet in one call
        # each (needs fused_gather: the batched dispatch copies no rows)
        self.batched = batched and fused_gather
        self.xp = None if fused_gather else torch.empty((n, A, H), dtype=dt, device=dev)
        self.act = torch.empty((n, A, I), dtype=dt, device=dev)
        self.yp = torch.empty((n, A, H), dtype=dt, device=dev)
        if self.ns:
            self.act_sh = torch.empty((n, self.ns, T, I), dtype=dt, device=dev)
            self.y_sh = torch.empty((n, self.ns, T, H), dtype=dt, device=dev)
        else:
            self.act_sh = self.y_sh = None
        self.glog = (torch.empty((n, T, E), dtype=torch.float32, device=dev)
                     if self.wg is not None else None)
        self.w_dev = torch.zeros((n, D), **i32)
        self.acc = torch.zeros(4, dtype=torch.int64, device=dev)
        self.w_host = torch.zeros((n, D), dtype=torch.int32).pin_memory()
        self.ws_dispatch = torch.empty(
            max(256, workspace_bytes(OP_DISPATCH_MANY, T, E, k, 0, n)) // 4, dtype=torch.int32,
            device=dev)
        self.ws_ffn = torch.empty(
            max(256, workspace_bytes(OP_FFN, 0, E, 1, self.ns, n)) // 4, dtype=torch.int32,
            device=dev)
        self.descs = [self._desc(j) for j in range(n)]
        # device_loop: the whole step, schedule included, is one cle_loop_step
        # call reading its masks from device memory; the host never waits.
        # restart: when every micro-batch has finished, the loop starts over
        # from h0 inside the same step (for steady-state timing).
        self.device_loop = device_loop
        if device_loop:
            if not self.batched:
                raise ValueError("device_loop needs the fused gather")
            self.restart = bool(restart)
            self.state = torch.zeros(LOOP_STATE_BYTES // 8 + 1, dtype=torch.int64, device=dev)
            self.log = torch.zeros(int(log_cap), dtype=torch.int64, device=dev)
            self.loop_desc = self._loop_desc(D, m)
        self.reset()

    def _loop_desc(self, D, m):
        d = LoopDesc()
        d.n, d.L, d.T, d.E, d.k, d.H, d.I = self.n, self.L, self.T, self.E, self.k, self.H, self.I
        d.D, d.m, d.policy, d.n_shared = D, m, self.policy, self.ns
        d.dtype = 0 if self.h.dtype == torch.bfloat16 else 1
        d.w_layout = W_PACKED if self.packed else W_ROWMAJOR
        d.restart = 1 if self.restart else 0
        if self.wg is not None:
            d.w_gate = self.wg.data_ptr()
            d.gate_bias = None if self.gbias is None else self.gbias.data_ptr()
        for j in range(self.n):
            if self.wg is not None:
                d.gate_logits[j] = self.glog[j].data_ptr()
            else:
                d.logits[j] = self.logits[j].data_ptr()
            d.h[j] = self.h[j].data_ptr()
            d.h0[j] = self.h0[j].data_ptr()
            d.idx[j] = self.idx[j].data_ptr()
            d.gate[j] = self.gates[j].data_ptr()
            d.counts[j] = self.counts[j].data_ptr()
            d.offsets[j] = self.offsets[j].data_ptr()
            d.dest[j] = self.dest[j].data_ptr()
            d.src[j] = self.src[j].data_ptr()
            d.act[j] = self.act[j].data_ptr()
            d.yp[j] = self.yp[j].data_ptr()
            if self.ns:
                d.act_shared[j] = self.act_sh[j].data_ptr()
                d.y_shared[j] = self.y_sh[j].data_ptr()
        d.w13, d.w2 = self.w13.data_ptr(), self.w2.data_ptr()
        d.w13_shared = None if self.w13s is None else self.w13s.data_ptr()
        d.w2_shared = None if self.w2s is None else self.w2s.data_ptr()
        d.ws_dispatch = self.ws_dispatch.data_ptr()
        d.ws_dispatch_bytes = self.ws_dispatch.numel() * 4
        d.ws_ffn = self.ws_ffn.data_ptr()
        d.ws_ffn_bytes = self.ws_ffn.numel() * 4
        d.w = self.w_dev.data_ptr()
        d.log = self.log.data_ptr()
        d.log_cap = self.log.numel()
        d.state = self.state.data_ptr()
        if self.prenorm:
            d.prenorm, d.norm_eps = 1, NORM_EPS
            for j in range(self.n):
                d.xn[j] = self.xn[j].data_ptr()
        return d

    def _desc(self, j):
        if self.fused:
            d = make_desc(0, self.T * self.k, self.offsets[j], None, self.act[j], self.yp[j],
                          x=self.xin[j], src=self.src[j], k=self.k)
        else:
            d = make_desc(0, self.T * self.k, self.offsets[j], self.xp[j], self.act[j],
                          self.yp[j])
        if self.ns:
            d.shared_rows = self.T
            d.x_shared = self.xin[j].data_ptr()
            d.act_shared = self.act_sh[j].data_ptr()
            d.y_shared = self.y_sh[j].data_ptr()
        return d

    def reset(self, h0=None):
        """Back to the start: every micro-batch at its first layer, stats cleared."""
        self.h.copy_(self.h0 if h0 is None else h0)
        self.acc.zero_()
        self.l = list(self.start)
        self.S = [j for j in range(self.n) if self.l[j] < self.L]
        self.prev = list(self.S)
        self.trace = []
        if self.device_loop:
            loop_init(self.state, self.n, self.L, self.start, stream=self.stream)
            self._logged = 0  # log entries already turned into trace entries
            self._shadow = list(self.start)

    @property
    def done(self) -> bool:
        if self.device_loop:
            return read_loop_state(self.state).ready == 0
        return not self.S

    def sync_trace(self):
        """Device loop: append the RunSets logged since the last call to
        `trace`, with each member's layer replayed from the starting layers."""
        st = read_loop_state(self.state)
        total = int(st.acc[3])
        if total - self._logged > self.log.numel():
            raise RuntimeError("RunSet log overwritten: raise log_cap")
        if total > self._logged:
            cap = self.log.numel()
            raw = self.log.cpu().numpy().view(np.uint64)
            for s in range(self._logged, total):
                R = ids_of(int(raw[s % cap]))
                self.trace.append((tuple(R), tuple(self._shadow[j] for j in R)))
                for j in R:
                    self._shadow[j] += 1
                if self.restart and all(v >= self.L for v in self._shadow):
                    self._shadow = list(self.start)
            self._logged = total
        return st

    # ------------------------------------------------------------ one step
    def _scores(self, js):
        """Router logits of the micro-batches js at their current layers: the
        given ones, or from h through each layer's router (one launch)."""
        if self.prenorm:
            rmsnorm_many([self.h[j] for j in js], [self.xn[j] for j in js], stream=self.stream)
        if self.wg is None:
            return [self.logits[j, self.l[j]] for j in js]
        out = [self.glog[j] for j in js]
        bias = None if self.gbias is None else [self.gbias[self.l[j]] for j in js]
        gate_logits_many([self.xin[j] for j in js], [self.wg[self.l[j]] for j in js], out,
                         bias=bias, packed=self.packed, stream=self.stream)
        return out

    def route_dispatch(self, j):
        """AttnRouteDispatch for micro-batch j at its current layer."""
        s = self.stream
        route(self._scores([j])[0], self.k, self.idx[j], self.gates[j], stream=s)
        dispatch(self.idx[j], self.E, self.xin[j], self.counts[j], self.offsets[j], self.dest[j],
                 self.src[j], None if self.fused else self.xp[j], self.ws_dispatch, stream=s)

    def route_dispatch_many(self, js):
        """AttnRouteDispatch for the micro-batches js, each at its current layer,
        one launch per pass."""
        s = self.stream
        idx = [self.idx[j] for j in js]
        route_many(self._scores(js), self.k, idx, [self.gates[j] for j in js], stream=s)
        dispatch_many(idx, self.E, [self.counts[j] for j in js], [self.offsets[j] for j in js],
                      [self.dest[j] for j in js], [self.src[j] for j in js], self.ws_dispatch,
                      stream=s)

    def schedule(self) -> list:
        """Workloads to the host, then Schedule(S, m) in the host library."""
        s = self.stream
        workload_stats(self.counts, self.D, 0, self.w_dev, stream=s)
        self.w_host.copy_(self.w_dev, non_blocking=True)
        s.synchronize()
        R = schedule_step_raw(self.w_host.data_ptr(), self.n, self.D, mask_of(self.S), self.m,
                              self.policy)
        return ids_of(R)

    def moe_compute_combine(self, R, events=None):
        """MoECompute_Combine: one grouped expert launch for every member of R
        (each at its own layer), then the Eq. (1) combine + residual."""
        s = self.stream
        workload_stats(self.counts, self.D, mask_of(R), self.w_dev, self.acc, stream=s)
        descs = []
        for j in R:
            d = self.descs[j]
            d.layer = self.l[j]
            descs.append(d)
        grouped_expert_ffn(descs, self.w13, self.w2, self.ws_ffn, self.w13s, self.w2s,
                           events=events, stream=s, packed=self.packed)
        if self.batched:
            combine_many([self.yp[j] for j in R], [self.dest[j] for j in R],
                         [self.gates[j] for j in R], [self.h[j] for j in R],
                         y_shared=None if self.y_sh is None else [self.y_sh[j] for j in R],
                         residual=[self.h[j] for j in R], stream=s)
            return
        for j in R:
            combine(self.yp[j], self.dest[j], self.gates[j], self.h[j],
                    y_shared=None if self.y_sh is None else self.y_sh[j], residual=self.h[j],
                    stream=s)

    def step(self, events=None, mark=None) -> list:
        """One iteration of the Algorithm 1 loop; returns RunSet_i (None with
        device_loop: the RunSet stays on the device; see sync_trace).

        events: 4 raw hipEvent_t for the expert launch (see grouped_expert_ffn);
        mark: optional callable, called with 0 / 1 before / after the route +
        dispatch launches and with 2 after the combine, on the host as the
        work is enqueued (for timing events on the engine's stream)."""
        if self.device_loop:
            loop_step(self.loop_desc, events, stream=self.stream)
            return None
        todo = [j for j in self.prev if self.l[j] < self.L]
        if mark:
            mark(0)
        if self.batched and todo:
            self.route_dispatch_many(todo)
        else:
            for j in todo:
                self.route_dispatch(j)
        if mark:
            mark(1)
        R = self.schedule()
        layers = [self.l[j] for j in R]
        self.moe_compute_combine(R, events=events)
        if mark:
            mark(2)
        self.trace.append((tuple(R), tuple(layers)))
        for j in R:
            self.l[j] += 1
        self.S = [j for j in self.S if self.l[j] < self.L]
        self.prev = R
        return R

    def run(self, chunk=8):
        """Steps until every micro-batch has finished.  Device loop: steps
        are enqueued `chunk` at a time between checks of the pool (steps
        after the last one find it empty and do nothing)."""
        if self.device_loop:
            if self.restart:
                raise ValueError("run() of a restarting loop never ends")
            while True:
                for _ in range(chunk):
                    self.step()
                if self.sync_trace().ready == 0:
                    return self
        while self.S:
            self.step()
        return self

    def stats(self):
        """(work, effective workload, sum of members' own peaks, steps) and u."""
        if self.device_loop:
            a = [int(v) for v in read_loop_state(self.state).acc]
        else:
            a = [int(v) for v in self.acc.cpu()]
        u = a[0] / (self.D * a[1]) if a[1] else 0.0
        return a, u

    def expert_tokens(self, R) -> int:
        return len(R) * self.T * (self.k + self.ns)
