"""Throughput of the cross-layer MoE step on one MI355X.

A timed step is one whole run of Algorithm 1 of EasyBalance -- every
micro-batch through every layer -- over the Qwen3-30B-A3B-shaped synthetic
stack (48 layers, hidden 2048, 128 experts top-8, SwiGLU intermediate 768,
D = 8 groups, 4 micro-batches of 2048 tokens).  Each of its iterations
routes and dispatches the previous RunSet, takes the workload statistics and
Schedule(S, m) (CumUtil, m = 3), runs one grouped expert launch per GEMM
phase for every RunSet member at its own layer, and the gate-weighted
combine.  By default an iteration is one cle_loop_step (the schedule runs on
the device and the host never waits); --host-loop times host-driven
iterations instead (workloads copied to the host, the host scheduler, then
the launches).  When all micro-batches have passed layer 48 the loop
restarts at layer 0 from the initial hidden states, inside the iteration
that finishes the run, so the timed steps are back-to-back whole runs.

Prints one JSON line (rank 0):
  value      expert tokens/s over the timed whole runs (inputs resident in HBM);
  roofline   the dominant kernel (grouped gate/up GEMM): algorithmic bytes or
             FLOPs per launch / its mean launch time, from start/end HIP
             events that the launch itself records on the library's stream
             during the timed steps;
  cpu_baseline the CPU oracle on (micro-batch, layer) units of the same
             workload, on this host's cores (and on one core).
With --sweep it prints instead the 1-u sweep over n, m/n and D and the
consecutive-layer same-peak counts, one JSON line per (config, D); with
--group-fit, the per-group expert time against the group workload w_d.
"""
from __future__ import annotations

import argparse
import ctypes
import gc
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "expert tokens/s per cross-layer MoE step; % bf16 MFMA peak; under-util 1-u"
PROFILE = os.path.join(ROOT, "profiles", "ffn_gemm_gate_up_qwen3.md")
KERNEL_SOURCES = ("cross_layer_expert_amd/csrc/ffn.hip", "cross_layer_expert_amd/csrc/cle_internal.h")


def measured_traffic(workload: str, algorithmic_per_launch: float):
    """HBM bytes per gate/up launch from the committed rocprofv3 FETCH_SIZE +
    WRITE_SIZE summary, or None when that summary is for another workload,
    the kernel sources changed since the counters were taken, or its launches
    carried different work (algorithmic bytes per launch more than 0.5 %
    apart: another mix of launches than the ones timed here)."""
    try:
        text = open(PROFILE).read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if ":" in line and not line.startswith((" ", "|", "#")):
            key, val = line.split(":", 1)
            fields[key.strip()] = val.split()[0] if val.split() else ""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if fields.get("workload") != workload or fields.get("kernel_source_sha256") != h.hexdigest():
        return None
    alg = float(fields.get("algorithmic_bytes_per_launch", "nan"))
    if not abs(alg - algorithmic_per_launch) <= 0.005 * algorithmic_per_launch:
        return None
    return int(fields["traffic_bytes_per_launch"])


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime already loaded by torch."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def record(self, e, stream_handle):
        assert self.lib.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream_handle)) == 0

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
            out.append(e.value)
        return out

    def ms(self, a, b) -> float:
        f = ctypes.c_float()
        st = self.lib.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(a), ctypes.c_void_p(b))
        assert st == 0, st
        return float(f.value)


def workload_name(cfg) -> str:
    s = (f"{cfg.name}-shaped MoE stack: {cfg.L} layers, hidden {cfg.H}, {cfg.E} experts top-{cfg.k}"
         f", SwiGLU I {cfg.I}, D={cfg.D}, {cfg.n} micro-batches x {cfg.T} tokens")
    if cfg.n_shared:
        s += f", +{cfg.n_shared} shared experts"
    if cfg.bias == "zipf":
        s += f", Zipf({cfg.zipf_s}) skew"
    if cfg.profiles > 1:
        s += f", {cfg.profiles} skew profiles"
    if cfg.start_layers:
        s += ", staggered start layers 3j"
    return s


def setup(cfg, seed, dev):
    import torch
    import synth
    t0 = time.time()
    W = synth.weights_torch(cfg, seed, dev)
    logits = np.stack([np.stack([synth.logits(cfg, seed, j, l) for l in range(cfg.L)])
                       for j in range(cfg.n)])
    lt = torch.from_numpy(logits).to(dev)
    h0 = np.stack([synth.hidden(cfg, seed, j) for j in range(cfg.n)])
    ht = torch.from_numpy(h0.view(np.int16)).to(dev).view(torch.bfloat16)
    torch.cuda.synchronize()
    print(f"[bench] inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    return W, lt, ht, logits, h0


def counts_of(eng, j, l):
    """Per-expert counts of micro-batch j at layer l, from the library's route
    and dispatch kernels (routing depends only on the logits)."""
    import cross_layer_expert_amd as cle
    saved = eng.l[j]
    eng.l[j] = l
    eng.route_dispatch(j)
    eng.l[j] = saved
    return eng.counts[j].clone()


def ffn_work(cfg, members, counts_host):
    """Algorithmic bytes and FLOPs of the two GEMM phases of one grouped launch.

    members: list of (j, layer); counts_host[(j, layer)] = per-expert counts.
    Weights of a distinct (layer, expert) are read once; activations once."""
    H, I = cfg.H, cfg.I
    touched = set()
    rows = 0
    for j, l in members:
        c = counts_host[(j, l)]
        rows += int(c.sum())
        touched.update((l, int(e)) for e in np.flatnonzero(c))
        if cfg.n_shared:
            rows += cfg.n_shared * cfg.T
            touched.update((l, -1 - q) for q in range(cfg.n_shared))
    nw = len(touched)
    b1 = nw * 2 * I * H * 2 + rows * (H * 2 + I * 2)
    b2 = nw * H * I * 2 + rows * (I * 2 + H * 2)
    f1 = 2.0 * rows * H * 2 * I
    f2 = 2.0 * rows * I * H
    return b1, b2, f1, f2


def plan_run(w_table, D, policy, m, start_layers=None):
    """The steps of one whole run of Algorithm 1 with the library's host
    scheduler, from the per-(micro-batch, layer) workloads w_table[j][l]
    (length D): a list of RunSets, each a list of (micro-batch, layer)."""
    import cross_layer_expert_amd as cle
    n, L = len(w_table), len(w_table[0])
    lj = list(start_layers) if start_layers else [0] * n
    S = [j for j in range(n) if lj[j] < L]
    steps = []
    while S:
        w = np.zeros((n, D), np.int32)
        for j in S:
            w[j] = w_table[j][lj[j]]
        R = cle.ids_of(cle.schedule_step(w, cle.mask_of(S), m, policy))
        steps.append([(j, lj[j]) for j in R])
        for j in R:
            lj[j] += 1
        S = [j for j in S if lj[j] < L]
    return steps


def schedule_only_u(w_table, D, policy, m, start_layers=None):
    """1-u of Algorithm 1 over a full run, from the per-(micro-batch, layer)
    workloads w_table[j][l] (length D), with the library's host scheduler.
    Returns (1-u, steps, sum of members' own peaks / sum of step peaks)."""
    num = den = sep = 0
    steps = plan_run(w_table, D, policy, m, start_layers)
    for st in steps:
        w = np.array([w_table[j][l] for j, l in st], np.int64)
        Wd = w.sum(axis=0)
        num += int(Wd.sum())
        den += int(Wd.max())
        sep += int(w.max(axis=1).sum())
    return 1.0 - num / (D * den), len(steps), sep / den


def same_peak(w_table, run):
    """Windows of `run` consecutive layers whose peak group (lowest index among
    equal maxima) is the same on every layer, summed over micro-batches
    (the statistic of the EasyBalance paper's Table 2): (hits, windows)."""
    hits = windows = 0
    for wj in w_table:
        peaks = np.argmax(np.asarray(wj), axis=1)      # first maximum = lowest index
        nwin = max(0, len(peaks) - run + 1)
        if nwin:
            same = np.ones(nwin, bool)
            for q in range(1, run):
                same &= peaks[q:q + nwin] == peaks[:nwin]
            hits += int(same.sum())
        windows += nwin
    return hits, windows


def workload_tables(cfg, seed, dev, n, Ds):
    """{D: int array [n, L, D]}: per-(micro-batch, layer) group workloads from
    the library's route, dispatch and workload-statistics kernels (one batched
    call per micro-batch covers all L layers)."""
    import torch
    import cross_layer_expert_amd as cle
    import synth
    L, T, E, k = cfg.L, cfg.T, cfg.E, cfg.k
    i32 = dict(dtype=torch.int32, device=dev)
    idx = torch.empty((L, T, k), **i32)
    gate = torch.empty((L, T, k), dtype=torch.float32, device=dev)
    counts, offsets = torch.empty((L, E), **i32), torch.empty((L, E + 1), **i32)
    dest, src = torch.empty((L, T * k), **i32), torch.empty((L, T * k), **i32)
    ws = torch.empty(cle.workspace_bytes(cle.OP_DISPATCH_MANY, T, E, k, 0, L) // 4, **i32)
    out = {D: np.zeros((n, L, D), np.int64) for D in Ds}
    for j in range(n):
        lg = torch.from_numpy(np.stack([synth.logits(cfg, seed, j, l) for l in range(L)])).to(dev)
        cle.route_many(list(lg), k, list(idx), list(gate))
        cle.dispatch_many(list(idx), E, list(counts), list(offsets), list(dest), list(src), ws)
        for D in Ds:
            wd = torch.empty((L, D), **i32)
            cle.workload_stats(counts, D, 0, wd)
            out[D][j] = wd.cpu().numpy()
    return out


SWEEP_POLICIES = ("b0", "b1", "cumutil", "maxutil", "diffpeak")


def sweep(seed, dev, configs=("qwen3", "moonlight", "taskshift"), ns=(2, 4, 8, 16),
          ratios=(0.5, 0.75, 1.0), Ds=(2, 4, 8)):
    """1-u of every policy over n, m/n and D, and the consecutive-layer
    same-peak rates; one JSON line per (config, D)."""
    import cross_layer_expert_amd as cle
    import synth
    for name in configs:
        cfg = synth.CONFIGS[name]
        t0 = time.time()
        tables = workload_tables(cfg, seed, dev, max(ns), Ds)
        for D in Ds:
            wt = tables[D]
            line = {"sweep": name, "seed": seed, "D": D, "L": cfg.L, "T": cfg.T, "E": cfg.E,
                    "k": cfg.k, "zipf_s": cfg.zipf_s, "profiles": cfg.profiles}
            sp = {}
            for run in (2, 3):
                h, w = same_peak(wt[:max(ns)], run)
                sp[str(run)] = [h, w, round(h / w, 4) if w else None]
            line["same_peak"] = sp
            pts = []
            for n in ns:
                base = {}
                for pol in ("b0", "b1"):
                    om, st, _ = schedule_only_u(wt[:n], D, cle.POLICIES[pol], 1)
                    base[pol] = (round(om, 4), st)
                for r in ratios:
                    m = max(1, int(r * n))
                    pt = {"n": n, "m": m, "one_minus_u": {}, "steps": {}}
                    for pol in SWEEP_POLICIES:
                        if pol in base:
                            om, st = base[pol]
                        else:
                            om, st, _ = schedule_only_u(wt[:n], D, cle.POLICIES[pol], m)
                            om = round(om, 4)
                        pt["one_minus_u"][pol] = om
                        pt["steps"][pol] = st
                    pts.append(pt)
            line["points"] = pts
            line["seconds"] = round(time.time() - t0, 1)
            print(json.dumps(line), flush=True)


def fit_linear(X, y):
    """Least squares y ~ X @ c (X includes a column of ones for an intercept):
    (c, R^2, median |relative residual|)."""
    X, y = np.asarray(X, np.float64), np.asarray(y, np.float64)
    c, *_ = np.linalg.lstsq(X, y, rcond=None)
    r = y - X @ c
    ss = float(((y - y.mean()) ** 2).sum())
    r2 = 1.0 - float((r ** 2).sum()) / ss if ss > 0 else 1.0
    return c, r2, float(np.median(np.abs(r) / np.maximum(np.abs(y), 1e-30)))


def group_fit(cfg, seed, dev, reps=3, n_sets=96):
    """Eq. (2) of EasyBalance on this GPU: the expert time of one group's share
    of a step, against its workload w_d.

    Under expert parallelism GPU d runs only the segments of group d's experts
    (E/D of them per layer).  Each point here is one grouped expert launch
    (both GEMM phases, timed by the launch's own start/end events) over exactly
    those segments -- the other experts get empty ranges -- for either one
    (micro-batch, layer) unit or a cross-layer set of m units (distinct
    micro-batches at random layers, as a RunSet would be).  Fits
    time = a + b * w_d, and time = a + b * w_d + c * (experts with rows), and
    checks, per unit or set, whether the group with the largest w_d is also the
    slowest.  Points run in a seeded random order, so consecutive launches
    rarely share a layer's weights in the caches."""
    import torch
    import cross_layer_expert_amd as cle
    from cross_layer_expert_amd.engine import Engine
    W, lt, ht, _, _ = setup(cfg, seed, dev)
    packed = cfg.dtype == "bf16"
    Wk = tuple(None if w is None else cle.pack_weights(w) for w in W) if packed else W
    stream = torch.cuda.current_stream()
    eng = Engine(Wk, lt, ht, cfg.D, cfg.k, cle.POLICY_B0_ALONE, 1, stream=stream,
                 packed=packed)
    hip = HipEvents()
    G = cfg.E // cfg.D
    units = [(j, l) for j in range(cfg.n) for l in range(cfg.L)]
    off, src = {}, {}
    for j, l in units:
        saved = eng.l[j]
        eng.l[j] = l
        eng.route_dispatch(j)
        eng.l[j] = saved
        off[(j, l)] = eng.offsets[j].clone()
        src[(j, l)] = eng.src[j].clone()
    torch.cuda.synchronize()
    off_h = {u: o.cpu().numpy().astype(np.int64) for u, o in off.items()}
    # what GPU d would receive of unit u: the rows [lo, hi) of group d's
    # experts, with offsets rebased to 0 (other experts empty)
    gof = {}
    for u, o in off.items():
        oh = off_h[u]
        for d in range(cfg.D):
            lo, hi = int(oh[d * G]), int(oh[(d + 1) * G])
            gof[(u, d)] = (torch.clamp(o, lo, hi) - lo, lo, hi - lo)
    rng = np.random.default_rng(seed + 1000)
    sets = [[(u,) for u in units]]
    m = min(cfg.m, cfg.n)
    multi = []
    for _ in range(n_sets):
        js = rng.choice(cfg.n, size=m, replace=False)
        multi.append(tuple((int(j), int(rng.integers(cfg.L))) for j in js))
    sets.append(multi)

    def work(members, d):
        w = touched = 0
        for u in members:
            oh = off_h[u]
            seg = np.diff(oh[d * G:(d + 1) * G + 1])
            w += int(seg.sum())
            touched += int((seg > 0).sum())
        return w, touched

    results = {}
    for name, group_sets in (("single", sets[0]), ("cross_layer_sets", sets[1])):
        pts = [(s_, d) for s_ in group_sets for d in range(cfg.D)]
        times = np.zeros((reps, len(pts)))
        for r in range(reps):
            order = rng.permutation(len(pts))
            evs = [hip.create(4) for _ in pts]
            for i in order:
                members, d = pts[i]
                descs = []
                for u in members:
                    j, l = u
                    go, lo, rows = gof[(u, d)]
                    dd = cle.FfnDesc.from_buffer_copy(eng.descs[j])
                    dd.layer = l
                    dd.rows = rows
                    dd.offsets = go.data_ptr()
                    dd.src = src[u][lo:].data_ptr()
                    dd.shared_rows = 0
                    dd.x_shared = dd.act_shared = dd.y_shared = None
                    descs.append(dd)
                cle.grouped_expert_ffn(descs, eng.w13, eng.w2, eng.ws_ffn, events=evs[i],
                                       stream=stream, packed=packed)
            torch.cuda.synchronize()
            times[r] = [hip.ms(e[0], e[3]) * 1e3 for e in evs]
        t = np.median(times, axis=0)                       # us per point
        wt = np.array([work(members, d) for members, d in pts], np.float64)
        ones = np.ones(len(pts))
        c1, r2_1, rel1 = fit_linear(np.stack([ones, wt[:, 0]], 1), t)
        c2, r2_2, rel2 = fit_linear(np.stack([ones, wt[:, 0], wt[:, 1]], 1), t)
        tt = t.reshape(len(group_sets), cfg.D)
        ww = wt[:, 0].reshape(len(group_sets), cfg.D)
        slow = tt.argmax(axis=1)
        peak = ww.argmax(axis=1)
        close = tt[np.arange(len(tt)), peak] >= 0.98 * tt.max(axis=1)
        qs = np.quantile(wt[:, 0], np.linspace(0, 1, 9))
        binned = []
        for b in range(8):
            sel = (wt[:, 0] >= qs[b]) & ((wt[:, 0] < qs[b + 1]) | (b == 7))
            if sel.any():
                binned.append([int(qs[b]), int(qs[b + 1]), round(float(t[sel].mean()), 2)])
        results[name] = dict(
            points=len(pts), members=len(group_sets[0]), reps=reps,
            mean_time_us=round(float(t.mean()), 2),
            w_octiles_mean_us=binned,
            w_range=[int(wt[:, 0].min()), int(wt[:, 0].max())],
            time_us_range=[round(float(t.min()), 2), round(float(t.max()), 2)],
            fit_a_b=dict(a_us=round(float(c1[0]), 3), b_us_per_row=round(float(c1[1]), 5),
                         r2=round(r2_1, 4), median_rel_residual=round(rel1, 4)),
            fit_a_b_c=dict(a_us=round(float(c2[0]), 3), b_us_per_row=round(float(c2[1]), 5),
                           c_us_per_expert=round(float(c2[2]), 3), r2=round(r2_2, 4),
                           median_rel_residual=round(rel2, 4)),
            peak_group_is_slowest=round(float((slow == peak).mean()), 4),
            peak_group_within_2pct_of_slowest=round(float(close.mean()), 4),
        )
    print(json.dumps({"metric": "per-group expert time vs w_d (Eq. 2)",
                      "config": {"workload": workload_name(cfg), "group_experts_per_layer": G,
                                 "seed": seed},
                      **results}), flush=True)


def ep_projection(cfg, seed, dev, reps=2):
    """The expert time of whole runs under expert parallelism, projected from
    launches measured on this GPU: D GPUs, GPU d holding group d's experts of
    every layer (E/D per layer), each step waiting for its slowest group
    (EasyBalance's Eq. (2): the step's expert time is set by the peak group).

    For each policy the library's host scheduler plans a whole run from the
    per-(micro-batch, layer) workloads; every step is then launched once per
    group over exactly that group's segments of the step's members (the
    segments GPU d would receive; other experts empty), timed by the launch's
    own events (start of gate/up to end of down), median of `reps` passes in
    a seeded random order.  Reported per policy: steps, 1-u, the projected
    expert time (sum over steps of the slowest group), and the sum over steps
    and groups (the same work done by this one GPU group by group).  Expert
    compute only: no all-to-all, no attention."""
    import torch
    import cross_layer_expert_amd as cle
    from cross_layer_expert_amd.engine import Engine
    W, lt, ht, _, _ = setup(cfg, seed, dev)
    packed = cfg.dtype == "bf16"
    Wk = tuple(None if w is None else cle.pack_weights(w) for w in W) if packed else W
    stream = torch.cuda.current_stream()
    eng = Engine(Wk, lt, ht, cfg.D, cfg.k, cle.POLICY_B0_ALONE, 1, stream=stream,
                 packed=packed)
    hip = HipEvents()
    G = cfg.E // cfg.D
    n, L, D = cfg.n, cfg.L, cfg.D
    off, src = {}, {}
    for j in range(n):
        for l in range(L):
            saved = eng.l[j]
            eng.l[j] = l
            eng.route_dispatch(j)
            eng.l[j] = saved
            off[(j, l)] = eng.offsets[j].clone()
            src[(j, l)] = eng.src[j].clone()
    torch.cuda.synchronize()
    off_h = {u: o.cpu().numpy().astype(np.int64) for u, o in off.items()}
    gof, w_table = {}, [[None] * L for _ in range(n)]
    for u, o in off.items():
        oh = off_h[u]
        w_table[u[0]][u[1]] = np.array([oh[(d + 1) * G] - oh[d * G] for d in range(D)], np.int32)
        for d in range(D):
            lo, hi = int(oh[d * G]), int(oh[(d + 1) * G])
            gof[(u, d)] = (torch.clamp(o, lo, hi) - lo, lo, hi - lo)
    policies = [("b0", cle.POLICY_B0_ALONE, 1), ("b1", cle.POLICY_B1_LOCKSTEP, n),
                ("cumutil", cle.POLICY_CUMUTIL, min(cfg.m, n)),
                ("maxutil", cle.POLICY_MAXUTIL, min(cfg.m, n))]
    plans = {name: plan_run(w_table, D, pol, m, cfg.start_layers) for name, pol, m in policies}
    pts = [(name, s_, d) for name, _, _ in policies for s_ in range(len(plans[name]))
           for d in range(D)]
    rng = np.random.default_rng(seed + 2000)
    times = np.zeros((reps, len(pts)))
    for r in range(reps):
        evs = [hip.create(4) for _ in pts]
        for i in rng.permutation(len(pts)):
            name, s_, d = pts[i]
            descs = []
            for u in plans[name][s_]:
                j, l = u
                go, lo, rows = gof[(u, d)]
                dd = cle.FfnDesc.from_buffer_copy(eng.descs[j])
                dd.layer = l
                dd.rows = rows
                dd.offsets = go.data_ptr()
                dd.src = src[u][lo:].data_ptr()
                dd.shared_rows = 0
                dd.x_shared = dd.act_shared = dd.y_shared = None
                descs.append(dd)
            cle.grouped_expert_ffn(descs, eng.w13, eng.w2, eng.ws_ffn, events=evs[i],
                                   stream=stream, packed=packed)
        torch.cuda.synchronize()
        times[r] = [hip.ms(e[0], e[3]) * 1e3 for e in evs]
    t = np.median(times, axis=0)
    res, idx = {}, 0
    for name, _, _ in policies:
        ns = len(plans[name])
        tt = t[idx:idx + ns * D].reshape(ns, D)
        idx += ns * D
        num = den = 0
        for st in plans[name]:
            Wd = np.sum([w_table[j][l] for j, l in st], axis=0)
            num += int(Wd.sum())
            den += int(Wd.max())
        res[name] = dict(steps=ns, one_minus_u=round(1.0 - num / (D * den), 4),
                         projected_ep_expert_ms=round(float(tt.max(axis=1).sum()) / 1e3, 3),
                         one_gpu_group_by_group_ms=round(float(tt.sum()) / 1e3, 3))
    b0 = res["b0"]["projected_ep_expert_ms"]
    for name in res:
        res[name]["vs_b0"] = round(res[name]["projected_ep_expert_ms"] / b0, 4)
    print(json.dumps({"metric": "projected expert-parallel expert time per whole run "
                                "(sum over steps of the slowest group's measured launch)",
                      "config": {"workload": workload_name(cfg), "D": D, "m": cfg.m,
                                 "seed": seed, "reps": reps},
                      "policies": res}), flush=True)


def cpu_baseline(cfg, W, logits, h0, budget_s, threads=None, gate=None, prenorm=True):
    """The CPU oracle on (micro-batch, layer) units of the same workload:
    route, dispatch, float64 SwiGLU experts (numpy matmul) and the combine of
    micro-batch 0 at layers 0, 1, ... until budget_s of oracle time is spent.
    threads: BLAS threads (None = every core this process may run on)."""
    import torch
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=threads if threads else cores):
        used = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        done_tok, spent, units = 0, 0.0, 0
        j = 0
        for l in range(cfg.L):
            w13 = oracle.widen(W[0][l].cpu().view(torch.int16).numpy().view(np.uint16), "bf16")
            w2 = oracle.widen(W[1][l].cpu().view(torch.int16).numpy().view(np.uint16), "bf16")
            ws = [None, None]
            if W[2] is not None:
                ws = [oracle.widen(W[q][l].cpu().view(torch.int16).numpy().view(np.uint16), "bf16")
                      for q in (2, 3)]
            x = oracle.widen(h0[j], "bf16")
            if gate is not None:
                wg = oracle.widen(gate[0][l].cpu().view(torch.int16).numpy().view(np.uint16),
                                  "bf16")
                gb = gate[1][l].cpu().numpy()
            t0 = time.perf_counter()
            xin = oracle.rmsnorm(x) if prenorm else x
            z = (logits[j, l] if gate is None
                 else oracle.gate_logits(xin, wg, gb).astype(np.float32))
            out = oracle.moe_layer(x, z, cfg.k, w13, w2, ws[0], ws[1], prenorm=prenorm)
            dt = time.perf_counter() - t0
            assert np.isfinite(out["y"]).all()
            spent += dt
            done_tok += cfg.T * (cfg.k + cfg.n_shared)
            units += 1
            del w13, w2, ws
            if spent >= budget_s:
                break
    return dict(value=round(done_tok / spent, 1), unit="expert tokens/s", cores=int(used),
                kind="oracle",
                sample=f"{units} (micro-batch, layer) unit(s) of the {cfg.name} workload "
                       f"(micro-batch 0, layers 0..{units - 1}; {done_tok} expert tokens; "
                       f"{'rmsnorm, ' if prenorm else ''}"
                       f"{'router, ' if gate is not None else ''}route, dispatch, float64 "
                       f"SwiGLU experts, combine); {spent:.1f} s")


def run_length(Wk, lt, ht, cfg, policy, m, stream, packed, gate_k, prenorm):
    """Iterations of Algorithm 1 in one whole run (every micro-batch through
    every layer), from one device-driven run on the same inputs."""
    from cross_layer_expert_amd.engine import Engine
    e = Engine(Wk, lt, ht, cfg.D, cfg.k, policy, m, start_layers=cfg.start_layers,
               stream=stream, packed=packed, device_loop=True, gate=gate_k, prenorm=prenorm)
    e.run(chunk=max(1, cfg.L // 2))
    n = len(e.trace)
    del e
    return n


def launch_stats(name, g1, g2, W):
    """Mean time, TFLOP/s, GB/s and binding-roofline fractions of the two GEMM
    phases over launches with algorithmic work W = (bytes1, bytes2, flops1,
    flops2), summed over the same launches."""
    B1, B2, F1, F2 = W
    t1, t2 = sum(g1) / 1e3, sum(g2) / 1e3
    K = len(g1)

    def binding(F, B, t):
        return max(F / (BF16_PEAK_TFLOPS * 1e12), B / (HBM_PEAK_GBS * 1e9)) / t

    out = {}
    for ph, g, t, B, F in (("gate_up", g1, t1, B1, F1), ("down", g2, t2, B2, F2)):
        out[ph] = dict(mean_us=round(t / K * 1e6, 2), median_us=round(float(np.median(g)) * 1e3, 2),
                       tflops=round(F / t / 1e12, 1), mfma_peak_frac=round(F / t / 1e12 / BF16_PEAK_TFLOPS, 4),
                       gbs=round(B / t / 1e9, 1), hbm_frac=round(B / t / 1e9 / HBM_PEAK_GBS, 4),
                       binding_roofline_frac=round(binding(F, B, t), 4),
                       bound="mfma" if F / B > BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
                       else "hbm")
    return out


def vendor_gemm(dev, groups, rows, H, I, reps=10):
    """Same-box context for the MFMA fractions (not part of the path): the
    vendor libraries' bf16 batched GEMM (torch.bmm through hipBLASLt and
    through rocBLAS; the faster is reported) on uniform batches of `groups`
    experts x `rows` rows at the expert shapes, gate/up [rows, H] x [H, 2I]
    and down [rows, I] x [I, H], timed with events on torch's stream.
    Operands are contiguous (batched products with a transposed right operand
    are avoided on this platform)."""
    import torch
    libs = (("hipblaslt", "cublaslt"), ("rocblas", "cublas"))
    before = torch.backends.cuda.preferred_blas_library()
    out = {}
    try:
        for name, K, N in (("gate_up", H, 2 * I), ("down", I, H)):
            a = torch.randn(groups, rows, K, device=dev).to(torch.bfloat16)
            b = torch.randn(groups, K, N, device=dev).to(torch.bfloat16).contiguous()
            c = torch.empty(groups, rows, N, device=dev, dtype=torch.bfloat16)
            per = {}
            for lib, key in libs:
                torch.backends.cuda.preferred_blas_library(key)
                for _ in range(3):
                    torch.bmm(a, b, out=c)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    torch.bmm(a, b, out=c)
                e1.record()
                torch.cuda.synchronize()
                per[lib] = e0.elapsed_time(e1) / reps
            lib = min(per, key=per.get)
            tf = 2.0 * groups * rows * K * N / (per[lib] * 1e-3) / 1e12
            out[name] = dict(shape=f"{groups} x ({rows} x {K}) x ({K} x {N})", library=lib,
                             mean_us=round(per[lib] * 1e3, 1),
                             us_by_library={k: round(v * 1e3, 1) for k, v in per.items()},
                             tflops=round(tf, 1), mfma_peak_frac=round(tf / BF16_PEAK_TFLOPS, 4))
            del a, b, c
    finally:
        torch.backends.cuda.preferred_blas_library(before)
    torch.cuda.empty_cache()
    return out


def hbm_stream(dev, gib=4, reps=5):
    """Same-box context for the HBM fractions (not part of the path): the rate
    of torch's device copy over a `gib` GiB bf16 tensor (bytes read +
    written)."""
    import torch
    n = gib << 29
    a = torch.empty(n, dtype=torch.bfloat16, device=dev).normal_()
    b = torch.empty_like(a)
    out = {}
    for name, fn, nbytes in (("copy", lambda: b.copy_(a), 4 * n),):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = dict(gbs=round(nbytes / (ms * 1e-3) / 1e9, 1),
                         hbm_frac=round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
    out["bytes"] = 2 * n
    del a, b
    torch.cuda.empty_cache()
    return out


def prefill_leg(Wk, seed, dev, stream, policy_name, prenorm):
    """The long-prefill shape (2 micro-batches x 16384 tokens) on the same
    48 x 128-expert weight stack: one whole device-driven run after a warm-up
    run, with the expert launches' own events; per-phase MFMA fractions."""
    import torch
    import cross_layer_expert_amd as cle
    import synth
    from cross_layer_expert_amd.engine import Engine
    pcfg = synth.CONFIGS["prefill"]
    t0 = time.time()
    lg = np.stack([np.stack([synth.logits(pcfg, seed, j, l) for l in range(pcfg.L)])
                   for j in range(pcfg.n)])
    lt = torch.from_numpy(lg).to(dev)
    del lg
    h0 = np.stack([synth.hidden(pcfg, seed, j) for j in range(pcfg.n)])
    ht = torch.from_numpy(h0.view(np.int16)).to(dev).view(torch.bfloat16)
    policy = cle.POLICIES[policy_name]
    eng = Engine(Wk, lt, ht, pcfg.D, pcfg.k, policy, pcfg.m, stream=stream, packed=True,
                 device_loop=True, prenorm=prenorm)
    eng.run(chunk=pcfg.L // 2)                       # warm-up run
    n_iter = len(eng.trace)
    eng.reset()
    hip = HipEvents()
    evs = [hip.create(4) for _ in range(n_iter)]
    torch.cuda.synchronize()
    gc.collect()
    gc.disable()
    s0 = time.perf_counter()
    for i in range(n_iter):
        eng.step(events=evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - s0
    gc.enable()
    eng.sync_trace()
    steps = [list(zip(R, layers)) for R, layers in eng.trace]
    assert eng.sync_trace().ready == 0 and len(steps) == n_iter
    counts_host = {}
    for (j, l) in sorted({jl for R in steps for jl in R}):
        counts_host[(j, l)] = counts_of(eng, j, l).cpu().numpy()
    W = [0.0, 0.0, 0.0, 0.0]
    for R in steps:
        W = [a + b for a, b in zip(W, ffn_work(pcfg, R, counts_host))]
    g1 = [hip.ms(e[0], e[1]) for e in evs]
    g2 = [hip.ms(e[2], e[3]) for e in evs]
    tok = sum(len(R) * pcfg.T * pcfg.k for R in steps)
    out = dict(workload=workload_name(pcfg), policy=policy_name, m=pcfg.m,
               iterations=n_iter, run_ms=round(elapsed * 1e3, 2),
               expert_tokens_per_s=round(tok / elapsed, 1),
               gemm_mfma_peak_frac=round((W[2] + W[3]) / (sum(g1) + sum(g2)) / 1e9
                                         / BF16_PEAK_TFLOPS, 4))
    out.update(launch_stats("prefill", g1, g2, W))
    del eng, lt, ht
    torch.cuda.empty_cache()
    # the vendor GEMM at the mean expert shape of one (micro-batch, layer)
    # unit: every expert of a layer with T * k / E rows
    ven = vendor_gemm(dev, pcfg.E, pcfg.T * pcfg.k // pcfg.E, pcfg.H, pcfg.I)
    for ph in ("gate_up", "down"):
        ven[ph]["ours_over_vendor"] = round(out[ph]["mfma_peak_frac"] / ven[ph]["mfma_peak_frac"], 3)
    out["vendor_gemm"] = ven
    out["setup_s"] = round(time.time() - t0 - elapsed, 1)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20,
                    help="timed steps; a step is one whole Algorithm 1 run (every micro-batch "
                         "through every layer)")
    ap.add_argument("--warmup", type=int, default=3, help="untimed whole runs before timing")
    ap.add_argument("--config", default="qwen3")
    ap.add_argument("--policy", default="cumutil")
    ap.add_argument("--m", type=int, default=None)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the whole-run comparison, 1-u and long-prefill passes")
    ap.add_argument("--no-prefill", action="store_true", help="skip the long-prefill leg")
    ap.add_argument("--host-loop", action="store_true",
                    help="time the host-driven step (schedule on the host after a wait for the "
                         "workloads) instead of the device-driven one")
    ap.add_argument("--gate", action="store_true",
                    help="route from the hidden state through each layer's linear router "
                         "(+ per-layer expert bias) instead of the given router logits")
    ap.add_argument("--no-prenorm", action="store_true",
                    help="experts read the raw hidden state (no RMS-normalised block input; "
                         "the residual stream then overflows bf16 in the last layers)")
    ap.add_argument("--sweep", action="store_true",
                    help="print the 1-u sweep over n, m/n and D (one JSON line per config and D) "
                         "instead of the timed step")
    ap.add_argument("--group-fit", action="store_true",
                    help="print the per-group expert time against w_d (one group's share of "
                         "each unit, as one GPU of an expert-parallel step) instead of the step")
    ap.add_argument("--ep-projection", action="store_true",
                    help="print the projected expert-parallel expert time of whole runs per "
                         "policy (each step's slowest group, measured per group) instead of "
                         "the step")
    ap.add_argument("--calib-copy", action="store_true",
                    help="first run a plain 1 GiB device copy (HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only; the expert-parallel sharding over "
              "several GPUs is a design, not code (set --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import cross_layer_expert_amd as cle
    import synth
    from cross_layer_expert_amd.engine import Engine

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.sweep:
        sweep(args.seed, dev)
        return
    cfg = synth.CONFIGS[args.config]
    if args.group_fit:
        group_fit(cfg, args.seed, dev)
        return
    if args.ep_projection:
        ep_projection(cfg, args.seed, dev)
        return
    m = args.m if args.m is not None else cfg.m
    policy = cle.POLICIES[args.policy]
    if cfg.start_layers and args.policy == "cumutil" and args.m is None:
        policy, m = cle.POLICY_B1_LOCKSTEP, cfg.n     # decode: the staggered 16-layer step

    if args.calib_copy:
        a = torch.empty(1 << 29, dtype=torch.int16, device=dev)   # 1 GiB
        b = torch.empty_like(a)
        a.fill_(1)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    W, lt, ht, logits, h0 = setup(cfg, args.seed, dev)
    stream = torch.cuda.current_stream()
    prenorm = not args.no_prenorm
    gate = gate_k = None
    if args.gate:
        # routing from the hidden state: each layer's linear router (+ bias)
        gate = (synth.gate_weights_torch(cfg, args.seed, dev),
                torch.from_numpy(synth.gate_bias(cfg, args.seed)).to(dev))
        lt = None
    # bf16: the expert launch reads a packed copy of the weights (a one-time
    # re-layout; results are bitwise those of the row-major weights, which the
    # CPU oracle keeps using)
    packed = cfg.dtype == "bf16"
    Wk = tuple(None if w is None else cle.pack_weights(w) for w in W) if packed else W
    if gate is not None:
        gate_k = (cle.pack_weights(gate[0]) if packed else gate[0], gate[1])
    torch.cuda.synchronize()
    K, Wm = args.steps, args.warmup
    device_loop = not args.host_loop
    # a timed step is one whole run of Algorithm 1; every run of the same
    # inputs takes the same iterations
    n_iter = run_length(Wk, lt, ht, cfg, policy, m, stream, packed, gate_k, prenorm)
    # device loop: every iteration is one cle_loop_step (schedule on the
    # device, no host wait); when all micro-batches finish, the loop restarts
    # from h0 inside that iteration
    eng = Engine(Wk, lt, ht, cfg.D, cfg.k, policy, m, start_layers=cfg.start_layers,
                 stream=stream, packed=packed, device_loop=device_loop, restart=device_loop,
                 log_cap=max(4096, (Wm + K) * n_iter + 64), gate=gate_k, prenorm=prenorm)
    hip = HipEvents()

    def one_step(e, events=None):
        if not e.device_loop and e.done:
            e.reset()
        return e.step(events=events)

    for _ in range(Wm * n_iter):
        one_step(eng)
    torch.cuda.synchronize()

    # the expert launches take their own start/end events (no marker between
    # kernels); Python's cyclic collector stays off while the steps run
    NI = K * n_iter
    evs = [hip.create(4) for _ in range(NI)]
    steps = []
    gc.collect()
    gc.disable()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(NI):
        one_step(eng, events=evs[i])
        if not device_loop:
            R, layers = eng.trace[-1]
            steps.append(list(zip(R, layers)))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gc.enable()
    if device_loop:
        eng.sync_trace()
        steps = [list(zip(R, layers)) for R, layers in eng.trace[-NI:]]
        assert len(eng.trace) == (Wm + K) * n_iter
    # every timed run takes each micro-batch through its remaining layers once
    units_per_run = sum(cfg.L - s for s in (cfg.start_layers or [0] * cfg.n))
    assert sum(len(R) for R in steps) == K * units_per_run

    # host-driven iterations (host schedule after a wait for the workloads) on
    # the same buffers: one timed whole run for comparison, then a pass with
    # markers around route + dispatch and after the combine (markers cost a
    # few us of stream time each, so they stay out of the timed steps above)
    hst = eng if not device_loop else Engine(
        Wk, lt, ht, cfg.D, cfg.k, policy, m, start_layers=cfg.start_layers, stream=stream,
        packed=packed, gate=gate_k, prenorm=prenorm)
    hst.reset()
    hst.run()
    hst.reset()
    torch.cuda.synchronize()
    gc.collect()
    gc.disable()
    h0t = time.perf_counter()
    hst.run()
    torch.cuda.synchronize()
    host_ms = (time.perf_counter() - h0t) * 1e3
    gc.enable()
    C = min(NI, 40)
    cev = [hip.create(4) for _ in range(C)]
    marks = [hip.create(3) for _ in range(C)]
    sh = stream.cuda_stream
    routed, csteps = [], []
    hst.reset()
    for i in range(C):
        if hst.done:
            hst.reset()
        routed.append([(j, hst.l[j]) for j in hst.prev if hst.l[j] < hst.L])
        hst.step(events=cev[i], mark=lambda q, i=i: hip.record(marks[i][q], sh))
        csteps.append(hst.trace[-1][0])
    torch.cuda.synchronize()

    tok = sum(len(R) * cfg.T * (cfg.k + cfg.n_shared) for R in steps)
    value = tok / elapsed
    g1 = [hip.ms(e[0], e[1]) for e in evs]
    g2 = [hip.ms(e[2], e[3]) for e in evs]

    # algorithmic work of every timed launch (counts recomputed by the library)
    need = sorted({jl for R in steps for jl in R})
    counts_host = {}
    if gate is None:
        for (j, l) in need:
            counts_host[(j, l)] = counts_of(eng, j, l).cpu().numpy()
    else:
        # routing depends on the hidden state: replay one whole run host-driven
        # (bitwise the same run) and read each member's counts
        rep = Engine(Wk, lt, ht, cfg.D, cfg.k, policy, m, start_layers=cfg.start_layers,
                     stream=stream, packed=packed, gate=gate_k, prenorm=prenorm)
        replayed = []
        while not rep.done:
            R = rep.step()
            replayed.append(list(zip(R, [rep.l[j] - 1 for j in R])))
            for j in R:
                counts_host.setdefault((j, rep.l[j] - 1), rep.counts[j].cpu().numpy())
        assert replayed * K == steps, "replay differs from the timed run"
        del rep
    Wk_ = [0.0, 0.0, 0.0, 0.0]
    for R in steps:
        Wk_ = [a + b for a, b in zip(Wk_, ffn_work(cfg, R, counts_host))]
    B1, B2, F1, F2 = Wk_
    t1, t2 = sum(g1) / 1e3, sum(g2) / 1e3
    ai1 = F1 / B1
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if ai1 < ridge:
        ach = B1 / NI / (t1 / NI) / 1e9
        roof = dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(ach / HBM_PEAK_GBS, 4))
    else:
        ach = F1 / NI / (t1 / NI) / 1e12
        roof = dict(bound="mfma", achieved=round(ach, 1), peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(ach / BF16_PEAK_TFLOPS, 4))
    default_run = args.policy == "cumutil" and args.m is None and args.seed == 0 and \
        not args.gate and prenorm and device_loop
    trf = measured_traffic(cfg.name, B1 / NI) if default_run else None
    roof["traffic"] = trf
    roof.update(kernel="ffn_gemm_bf16<1> (grouped gate/up + SwiGLU)",
                mean_launch_us=round(t1 / NI * 1e6, 2),
                algorithmic_bytes_per_launch=int(B1 / NI), flops_per_launch=int(F1 / NI))
    if trf:
        roof["traffic_over_algorithmic"] = round(trf / (B1 / NI), 4)

    gemm_tflops = (F1 + F2) / (t1 + t2) / 1e12

    # route + dispatch of the previous RunSet, and the combine, from events on
    # the same stream (stream time between the events)
    esz = 2 if cfg.dtype == "bf16" else 4
    T, k, H, E, ns = cfg.T, cfg.k, cfg.H, cfg.E, cfg.n_shared
    rd_unit = T * E * 4 + T * k * 8 + T * k * 4 + T * k * 8 + 2 * E * 4
    if gate is not None:   # router: hidden rows and weights in, logits out and back in
        rd_unit += T * H * esz + E * H * esz + T * E * 4
    if prenorm:            # the block input: raw rows in, normalised rows out
        rd_unit += 2 * T * H * esz
    cb_unit = T * k * H * esz + T * k * 8 + (1 + ns) * T * H * esz + T * H * esz
    rd_ms = [hip.ms(mk[0], mk[1]) for mk, r in zip(marks, routed) if r]
    rd_bytes = sum(len(r) for r in routed) * rd_unit
    cb_ms = [hip.ms(e[3], mk[2]) for e, mk in zip(cev, marks)]
    cb_bytes = sum(len(R) for R in csteps) * cb_unit
    t_rd, t_cb = sum(rd_ms) / 1e3, sum(cb_ms) / 1e3
    extras = dict(
        iterations_per_step=n_iter,
        ms_per_iteration=round(elapsed / NI * 1e3, 4),
        gemm_tflops=round(gemm_tflops, 1),
        mfma_peak_frac=round(gemm_tflops / BF16_PEAK_TFLOPS, 4),
        gemm_hbm_gbs=round((B1 + B2) / (t1 + t2) / 1e9, 1),
        gemm_binding_roofline_frac=round(
            max((F1 + F2) / (BF16_PEAK_TFLOPS * 1e12), (B1 + B2) / (HBM_PEAK_GBS * 1e9))
            / (t1 + t2), 4),
    )
    extras.update(launch_stats(cfg.name, g1, g2, Wk_))
    extras.update(
        route_dispatch=dict(mean_us=round(t_rd / max(len(rd_ms), 1) * 1e6, 2),
                            gbs=round(rd_bytes / t_rd / 1e9, 1) if t_rd else None,
                            bytes_per_microbatch=rd_unit),
        combine=dict(mean_us=round(t_cb / C * 1e6, 2), gbs=round(cb_bytes / t_cb / 1e9, 1),
                     bytes_per_microbatch=cb_unit),
        ffn_share_of_step=round((t1 + t2) / elapsed, 3),
        loop="device" if device_loop else "host",
        host_loop_ms_per_step=round(host_ms, 3),
    )

    if not args.no_extras and gate is None:
        # per-(micro-batch, layer) workloads of the whole stack -> 1-u per policy
        w_table = [[None] * cfg.L for _ in range(cfg.n)]
        for j in range(cfg.n):
            for l in range(cfg.L):
                c = counts_of(eng, j, l).view(1, -1)
                wd = torch.empty((1, cfg.D), dtype=torch.int32, device=dev)
                cle.workload_stats(c, cfg.D, 0, wd)
                w_table[j][l] = wd.cpu().numpy()[0]
        uu = {}
        for name in SWEEP_POLICIES:
            one_minus_u, nsteps, ratio = schedule_only_u(w_table, cfg.D, cle.POLICIES[name], m,
                                                         cfg.start_layers)
            uu[name] = dict(one_minus_u=round(one_minus_u, 4), steps=nsteps)
        extras["under_util"] = uu
    if not args.no_extras:
        # measured whole runs: cross-layer (timed policy) vs one (j, l) per step
        runs = {}
        # one (j, l) per step; all micro-batches at the same layer (on one GPU
        # the fastest: a layer's weights are read once for every micro-batch);
        # the timed policy
        cands = [("b0", cle.POLICY_B0_ALONE, 1), ("b1", cle.POLICY_B1_LOCKSTEP, cfg.n),
                 (args.policy, policy, m)]
        seen = set()
        for name, pol, mm in cands:
            if (pol, mm) in seen:
                continue
            seen.add((pol, mm))
            for dl in (False, True):
                e2 = Engine(Wk, lt, ht, cfg.D, cfg.k, pol, mm, start_layers=cfg.start_layers,
                            stream=stream, packed=packed, device_loop=dl, gate=gate_k,
                            prenorm=prenorm)
                e2.step()
                e2.reset()
                torch.cuda.synchronize()
                s0 = time.perf_counter()
                e2.run(chunk=max(1, cfg.L // 2)) if dl else e2.run()
                torch.cuda.synchronize()
                runs[name + ("_device" if dl else "_host")] = dict(
                    ms=round((time.perf_counter() - s0) * 1e3, 2), steps=len(e2.trace),
                    one_minus_u=round(1 - e2.stats()[1], 4))
                del e2
        extras["whole_run"] = runs
    pre = synth.CONFIGS["prefill"]
    same_stack = (cfg.L, cfg.E, cfg.H, cfg.I, cfg.n_shared, cfg.dtype) == (
        pre.L, pre.E, pre.H, pre.I, pre.n_shared, pre.dtype)
    if not args.no_extras and not args.no_prefill and same_stack and cfg.name != "prefill" \
            and gate is None:
        extras["prefill"] = prefill_leg(Wk, args.seed, dev, stream, "cumutil", prenorm)
    if not args.no_extras and cfg.dtype == "bf16":
        extras["hbm_stream"] = hbm_stream(dev)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, W, logits, h0, args.cpu_budget, gate=gate, prenorm=prenorm)
        cpu["one_core"] = cpu_baseline(cfg, W, logits, h0, args.cpu_budget / 2, threads=1,
                                       gate=gate, prenorm=prenorm)

    routing = ("hidden state routed through seeded per-layer linear routers plus a Zipf "
               "expert bias" if gate is not None else
               f"seeded router logits N(0,1) + {'Zipf' if cfg.bias == 'zipf' else 'normal'} "
               f"per-layer expert bias")
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "expert tokens/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(elapsed / K * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": f"synthetic ({routing}, N(0,1) hidden, N(0,0.02) weights); a step is one "
                f"whole Algorithm 1 run of {n_iter} iterations",
        "config": {"workload": workload_name(cfg), "policy": args.policy if policy != 1 else "b1",
                   "schedule": "device" if device_loop else "host",
                   "routing": "hidden state through the router" if gate is not None
                   else "given router logits",
                   "block": "pre-norm (experts read RMS-normalised rows)" if prenorm
                   else "raw hidden state",
                   "m": m, "seed": args.seed, "parallelism": "single GPU"},
        "roofline": roof, "cpu_baseline": cpu,
    }
    out.update(extras)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
