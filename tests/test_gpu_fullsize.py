"""Parity at full workload sizes, in the launch configuration bench.py times.

One cross-layer step with every micro-batch at a different layer (the hidden
states at those layers are seeded inputs, so the oracle needs nothing from
the GPU):
  * routing indices and dispatch permutation: bit-exact, every token;
  * workloads and step statistics: exact;
  * expert outputs of sampled segments (hottest, median, smallest non-empty)
    and combined outputs of sampled tokens: max-abs 2e-2, normwise 1e-2;
and for the Qwen3-shaped stack the whole cross-layer run (device-driven) is bitwise equal
to the run with one (micro-batch, layer) per step, with finite hidden states
after all 48 layers.  Launch configuration of bench.py: packed weights,
pre-norm block (the experts read the RMS-normalised rows, compared here from
the GPU's own bf16 normalised rows after checking those against the oracle's
normalisation), device-driven step.
"""
import gc

import numpy as np
import pytest
import torch

import cross_layer_expert_amd as cle
import oracle
import synth
from cross_layer_expert_amd.engine import Engine
from gpu_helpers import bits_of, check_close, device, f32_ulp_diff, to_dev, to_host

pytestmark = pytest.mark.gpu

TOL = (2e-2, 1e-2)


def _w(t):
    return oracle.widen(to_host(t), "bf16")


def _setup(cfg, seed, start):
    dev = device()
    W = synth.weights_torch(cfg, seed, dev)
    logits = np.stack([np.stack([synth.logits(cfg, seed, j, l) for l in range(cfg.L)])
                       for j in range(cfg.n)])
    # seeded hidden states "at" the starting layers (tag = layer): inputs
    h0 = np.stack([synth.hidden(cfg, seed, j, tag=1000 + start[j]) for j in range(cfg.n)])
    return dev, W, logits, h0


def _one_cross_layer_step(name, start):
    cfg = synth.CONFIGS[name]
    seed = 2
    print(f"[fullsize] {name}: setup", flush=True)
    dev, W, logits, h0 = _setup(cfg, seed, start)
    # the launch configuration bench.py times: packed weights, pre-norm block,
    # device-driven step
    Wk = tuple(None if w is None else cle.pack_weights(w) for w in W)
    eng = Engine(Wk, torch.from_numpy(logits).to(dev), to_dev(h0, "bf16", dev), cfg.D, cfg.k,
                 cle.POLICY_B1_LOCKSTEP, cfg.n, start_layers=start, packed=True, prenorm=True,
                 device_loop=True)
    eng.step()
    eng.sync_trace()
    torch.cuda.synchronize()
    R = list(eng.trace[-1][0])
    assert R == list(range(cfg.n)), R
    del Wk
    print(f"[fullsize] {name}: step done, layers {start}", flush=True)
    w13, w2, w13s, w2s = W
    wrows = []
    for j in range(cfg.n):
        l = start[j]
        z = logits[j, l]
        ridx, rg = oracle.route(z, cfg.k)
        assert np.array_equal(eng.idx[j].cpu().numpy(), ridx), f"route idx j={j}"
        u = f32_ulp_diff(eng.gates[j].cpu().numpy(), rg)
        assert u.max() <= 1 and (u > 0).sum() <= max(1, u.size // 10000), f"gates j={j}"
        counts, offsets, dest, src = oracle.dispatch(ridx, cfg.E)
        assert np.array_equal(eng.counts[j].cpu().numpy(), counts)
        assert np.array_equal(eng.offsets[j].cpu().numpy(), offsets)
        assert np.array_equal(eng.dest[j].cpu().numpy(), dest)
        assert np.array_equal(eng.src[j].cpu().numpy(), src)
        wrows.append(oracle.group_workload(counts, cfg.D))
        # the experts read the GPU's normalised rows (one bf16 rounding of the
        # oracle's), the residual is the raw state
        x = oracle.widen(h0[j], "bf16")
        xn = oracle.widen(to_host(eng.xn[j]), "bf16")
        rn = oracle.rmsnorm(x, cle.NORM_EPS)
        assert np.all(np.abs(xn - rn) <= (2.0 ** -8 + 1e-5) * np.abs(rn) + 1e-30)
        # sampled segments: hottest, median non-empty, smallest non-empty
        nz = np.flatnonzero(counts)
        order = nz[np.argsort(counts[nz], kind="stable")]
        for e in sorted({int(order[-1]), int(order[len(order) // 2]), int(order[0])}):
            a, b = int(offsets[e]), int(offsets[e + 1])
            xs = xn[src[a:b] // cfg.k]
            ref = oracle.swiglu_expert(xs, _w(w13[l, e]), _w(w2[l, e]))
            got = oracle.widen(to_host(eng.yp[j][a:b]), "bf16")
            check_close(got, ref, *TOL, what=f"{name} j={j} l={l} e={e} rows={b - a}")
        # sampled tokens: the full layer output of one token from inputs only
        rng = np.random.default_rng(j)
        for t in rng.choice(cfg.T, 3, replace=False):
            xt = xn[t:t + 1]
            yp = np.concatenate([oracle.swiglu_expert(xt, _w(w13[l, int(e)]), _w(w2[l, int(e)]))
                                 for e in ridx[t]])
            ysh = None
            if cfg.n_shared:
                ysh = [oracle.swiglu_expert(xt, _w(w13s[l, q]), _w(w2s[l, q]))
                       for q in range(cfg.n_shared)]
            ref = oracle.combine(yp, np.arange(cfg.k), rg[t:t + 1], cfg.k, y_shared=ysh,
                                 residual=x[t:t + 1])
            got = oracle.widen(to_host(eng.h[j][t:t + 1]), "bf16")
            check_close(got, ref, *TOL, what=f"{name} j={j} token {t}")
    # statistics of the step (B1: every micro-batch in one step)
    acc, _ = eng.stats()
    a, b, c = oracle.step_stats(wrows)
    assert acc == [a, b, c, 1]
    del eng, W
    gc.collect()
    torch.cuda.empty_cache()


def test_qwen3_cross_layer_step():
    _one_cross_layer_step("qwen3", [0, 11, 30, 47])


def test_moonlight_cross_layer_step():
    _one_cross_layer_step("moonlight", [0, 3, 7, 10, 14, 18, 21, 25])


def test_decode_staggered_step():
    _one_cross_layer_step("decode", list(synth.CONFIGS["decode"].start_layers))


def test_prefill_cross_layer_step():
    _one_cross_layer_step("prefill", [5, 40])


def test_qwen3_full_run_cross_layer_equals_layer_by_layer():
    cfg = synth.CONFIGS["qwen3"]
    dev = device()
    W = synth.weights_torch(cfg, 0, dev)
    logits = np.stack([np.stack([synth.logits(cfg, 0, j, l) for l in range(cfg.L)])
                       for j in range(cfg.n)])
    h0 = np.stack([synth.hidden(cfg, 0, j) for j in range(cfg.n)])
    lt, ht = torch.from_numpy(logits).to(dev), to_dev(h0, "bf16", dev)
    print("[fullsize] qwen3 full runs", flush=True)
    W = tuple(None if w is None else cle.pack_weights_inplace(w) for w in W)
    kw = dict(packed=True, prenorm=True)
    base = Engine(W, lt, ht, cfg.D, cfg.k, cle.POLICY_B0_ALONE, 1, **kw).run()
    ref = bits_of(base.h)
    assert np.isfinite(oracle.widen(ref.view(np.uint16), "bf16")).all()
    acc0, u0 = base.stats()
    for policy in ("cumutil", "maxutil"):
        eng = Engine(W, lt, ht, cfg.D, cfg.k, cle.POLICIES[policy], cfg.m, device_loop=True,
                     **kw).run()
        assert np.array_equal(bits_of(eng.h), ref), policy
        acc, u = eng.stats()
        assert acc[0] == acc0[0] and acc[2] == acc0[2] and u > u0
        print(f"[fullsize] {policy}: {acc[3]} steps, 1-u {1 - u:.4f} vs per-layer {1 - u0:.4f}",
              flush=True)
    del base, eng, W
    gc.collect()
    torch.cuda.empty_cache()
