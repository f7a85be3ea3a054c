"""The batched entry points (cle_route_many, cle_dispatch_many,
cle_combine_many) against the oracle and against the per-micro-batch calls.

Bars: indices, dispatch outputs and combine outputs bit-exact with the
per-micro-batch calls (same kernels, one launch); routing and dispatch
bit-exact with the oracle, gates included; the
batched engine bitwise equal to the per-micro-batch engine over whole runs.
"""
import numpy as np
import pytest
import torch

import cross_layer_expert_amd as cle
import oracle
import synth
from cross_layer_expert_amd.engine import Engine
from gpu_helpers import bits_of, device, to_dev

pytestmark = pytest.mark.gpu


def _skewed_ids(rng, T, k, E, skew):
    p = np.arange(1, E + 1, dtype=np.float64) ** (-skew)
    p = p[rng.permutation(E)]
    p /= p.sum()
    return rng.choice(E, size=(T, k), p=p).astype(np.int32)


@pytest.mark.parametrize("n,T,E,k", [(3, 2048, 128, 8), (64, 5, 8, 2), (1, 33, 1000, 7),
                                     (5, 129, 64, 6), (4, 1, 4, 4)])
def test_route_many(n, T, E, k):
    dev = device()
    rng = np.random.default_rng(n * 1000 + T)
    z = rng.standard_normal((n, T, E)).astype(np.float32)
    z[0, 0, :] = 1.5                      # an all-tie row: lower expert ids win
    zt = torch.from_numpy(z).to(dev)
    idx = torch.full((n, T, k), -7, dtype=torch.int32, device=dev)
    gate = torch.full((n, T, k), -1.0, dtype=torch.float32, device=dev)
    print(f"[route_many] n={n} T={T} E={E} k={k}", flush=True)
    cle.route_many(list(zt), k, list(idx), list(gate))
    idx1 = torch.empty_like(idx)
    gate1 = torch.empty_like(gate)
    for j in range(n):
        cle.route(zt[j], k, idx1[j], gate1[j])
    torch.cuda.synchronize()
    assert torch.equal(idx, idx1) and np.array_equal(bits_of(gate), bits_of(gate1))
    for j in range(n):
        ridx, rgate = oracle.route(z[j], k)
        assert np.array_equal(idx[j].cpu().numpy(), ridx), j
        assert np.array_equal(gate[j].cpu().numpy().view(np.int32), rgate.view(np.int32)), j


@pytest.mark.parametrize("n,T,k,E,skew", [(3, 2048, 8, 128, 1.1), (64, 7, 3, 16, 2.0),
                                          (2, 1000, 6, 1024, 0.5), (1, 1, 1, 1, 0.0),
                                          (8, 4097, 2, 7, 3.0), (2, 5000, 8, 128, 1.1)])
def test_dispatch_many(n, T, k, E, skew):
    dev = device()
    rng = np.random.default_rng(T + n)
    ids = np.stack([_skewed_ids(rng, T, k, E, skew) for _ in range(n)])
    if n > 1 and T * k > 4:               # dropped ids in one micro-batch
        ids[1].flat[[0, 3]] = [-1, E]
    it = torch.from_numpy(ids).to(dev)
    i32 = dict(dtype=torch.int32, device=dev)
    counts, offsets = torch.full((n, E), -9, **i32), torch.full((n, E + 1), -9, **i32)
    dest, src = torch.full((n, T * k), -9, **i32), torch.full((n, T * k), -9, **i32)
    ws = torch.empty(cle.workspace_bytes(cle.OP_DISPATCH_MANY, T, E, k, 0, n) // 4, **i32)
    print(f"[dispatch_many] n={n} T={T} k={k} E={E}", flush=True)
    cle.dispatch_many(list(it), E, list(counts), list(offsets), list(dest), list(src), ws)
    torch.cuda.synchronize()
    x = torch.zeros((T, 8), dtype=torch.float32, device=dev)
    ws1 = torch.empty(cle.workspace_bytes(cle.OP_DISPATCH, T, E, k) // 4, **i32)
    for j in range(n):
        if ((ids[j] >= 0) & (ids[j] < E)).all():
            # (dropped ids: the per-micro-batch call below, itself checked
            # against the oracle on the valid subset elsewhere, is the reference)
            rc, ro, rd, rs = oracle.dispatch(ids[j], E)
            assert np.array_equal(counts[j].cpu().numpy(), rc), j
            assert np.array_equal(offsets[j].cpu().numpy(), ro), j
            assert np.array_equal(dest[j].cpu().numpy(), rd), j
            assert np.array_equal(src[j].cpu().numpy(), rs), j
        c1, o1 = torch.empty(E, **i32), torch.empty(E + 1, **i32)
        d1, s1 = torch.empty(T * k, **i32), torch.empty(T * k, **i32)
        cle.dispatch(it[j], E, x, c1, o1, d1, s1, None, ws1)
        torch.cuda.synchronize()
        assert torch.equal(c1, counts[j]) and torch.equal(o1, offsets[j])
        assert torch.equal(d1, dest[j]) and torch.equal(s1, src[j])


@pytest.mark.parametrize("n,T,k,E,H,ns,dtype,res", [
    (3, 2048, 8, 128, 2048, 0, "bf16", True), (8, 1024, 6, 64, 2048, 2, "bf16", True),
    (64, 3, 2, 8, 64, 0, "f32", False), (2, 37, 12, 16, 72, 1, "bf16", True)])
def test_combine_many(n, T, k, E, H, ns, dtype, res):
    dev = device()
    rng = np.random.default_rng(T + H + n)
    gates, dests, yps, yshs, hs = [], [], [], [], []
    for _ in range(n):
        z = rng.standard_normal((T, E)).astype(np.float32)
        idx, g = oracle.route(z, k)
        dests.append(oracle.dispatch(idx, E)[2])
        gates.append(g)
        yps.append(synth.store(rng.standard_normal((T * k, H)).astype(np.float32), dtype))
        yshs.append(synth.store(rng.standard_normal((ns, T, H)).astype(np.float32), dtype))
        hs.append(synth.store(rng.standard_normal((T, H)).astype(np.float32), dtype))
    yp = [to_dev(a, dtype, dev) for a in yps]
    dt = [torch.from_numpy(a).to(dev) for a in dests]
    gt = [torch.from_numpy(a).to(dev) for a in gates]
    ysh = [to_dev(a, dtype, dev) for a in yshs] if ns else None
    h_many = [to_dev(a, dtype, dev) for a in hs]
    h_one = [to_dev(a, dtype, dev) for a in hs]
    out_many = h_many if res else [torch.empty_like(a) for a in h_many]
    out_one = h_one if res else [torch.empty_like(a) for a in h_one]
    print(f"[combine_many] n={n} T={T} k={k} H={H} ns={ns} {dtype}", flush=True)
    cle.combine_many(yp, dt, gt, out_many, y_shared=ysh, residual=h_many if res else None)
    for j in range(n):
        cle.combine(yp[j], dt[j], gt[j], out_one[j], y_shared=None if ysh is None else ysh[j],
                    residual=h_one[j] if res else None)
    torch.cuda.synchronize()
    for j in range(n):
        assert np.array_equal(bits_of(out_many[j]), bits_of(out_one[j])), j
    # one member against the oracle (the per-member call is tested there too)
    j = n - 1
    ref = oracle.combine(oracle.widen(yps[j], dtype), dests[j], gates[j], k,
                         y_shared=list(oracle.widen(yshs[j], dtype)) if ns else None,
                         residual=oracle.widen(hs[j], dtype) if res else None)
    got = oracle.widen(bits_of(out_many[j]).view(np.uint16) if dtype == "bf16"
                       else out_many[j].cpu().numpy(), dtype)
    tol = 2.0 ** -8 if dtype == "bf16" else 1e-6
    assert np.all(np.abs(got - ref) <= tol * np.abs(ref) + 1e-6 * np.abs(ref).max() * (k + ns + 1))


@pytest.mark.parametrize("name,policy", [("tiny", "cumutil"), ("tiny", "maxutil"),
                                         ("qwen3-small", "cumutil")])
def test_engine_batched_equals_per_microbatch(name, policy):
    """Whole runs: the batched engine and the per-micro-batch engine give
    bitwise-equal hidden states, workloads, statistics and schedules."""
    dev = device()
    cfg = (synth.small(synth.CONFIGS["qwen3"], L=6, T=256) if name == "qwen3-small"
           else synth.CONFIGS[name])
    W = synth.weights_torch(cfg, 4, dev)
    logits = np.stack([np.stack([synth.logits(cfg, 4, j, l) for l in range(cfg.L)])
                       for j in range(cfg.n)])
    h0 = np.stack([synth.hidden(cfg, 4, j) for j in range(cfg.n)])
    lt, ht = torch.from_numpy(logits).to(dev), to_dev(h0, cfg.dtype, dev)
    print(f"[engine] {name} {policy}", flush=True)
    runs = []
    for batched in (True, False):
        eng = Engine(W, lt, ht, cfg.D, cfg.k, cle.POLICIES[policy], cfg.m,
                     batched=batched).run()
        runs.append((bits_of(eng.h), eng.stats()[0], list(eng.trace)))
    assert np.array_equal(runs[0][0], runs[1][0])
    assert runs[0][1] == runs[1][1] and runs[0][2] == runs[1][2]
