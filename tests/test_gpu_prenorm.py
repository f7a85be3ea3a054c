"""The pre-norm MoE block: experts and router read RMS-normalised rows
(cle_rmsnorm_many), the combine adds to the raw hidden state.

Bars: the normalised rows within one bf16 rounding (2^-8 relative, plus the
float32 sum) of the float64 oracle, or 1e-6 relative in f32, bitwise
reproducible and in place; device-driven pre-norm runs bitwise equal to
host-driven ones (given logits and routed through the router); a token
followed through the layers by the oracle stays within the chained
tolerance; and over a full 48-layer stack the hidden state stays finite
(without the norm it overflows bf16 there).
"""
import numpy as np
import pytest
import torch

import cross_layer_expert_amd as cle
import oracle
import synth
from cross_layer_expert_amd.engine import Engine
from gpu_helpers import bits_of, check_close, device, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,T,H,dtype", [(3, 2048, 2048, "bf16"), (2, 37, 72, "bf16"),
                                         (1, 1, 8, "bf16"), (2, 16, 64, "f32")])
def test_rmsnorm_vs_oracle(n, T, H, dtype):
    dev = device()
    rng = np.random.default_rng(T + H)
    xs = [synth.store((rng.standard_normal((T, H)) * rng.uniform(0.01, 50, (T, 1)))
                      .astype(np.float32), dtype) for _ in range(n)]
    xt = [to_dev(a, dtype, dev) for a in xs]
    yt = [torch.empty_like(a) for a in xt]
    print(f"[rmsnorm] n={n} T={T} H={H} {dtype}", flush=True)
    cle.rmsnorm_many(xt, yt)
    again = [a.clone() for a in xt]
    cle.rmsnorm_many(again, again)                       # in place
    torch.cuda.synchronize()
    for j in range(n):
        assert np.array_equal(bits_of(again[j]), bits_of(yt[j]))
        ref = oracle.rmsnorm(oracle.widen(xs[j], dtype), cle.NORM_EPS)
        got = oracle.widen(to_host(yt[j]), dtype)
        rel = 2.0 ** -8 + 1e-5 if dtype == "bf16" else 1e-6
        assert np.all(np.abs(got - ref) <= rel * np.abs(ref) + 1e-30)


def _cfg(name):
    base = synth.CONFIGS[name.split("-")[0]]
    return synth.small(base, L=6, T=256)


@pytest.mark.parametrize("name,gated", [("qwen3-small", False), ("qwen3-small", True),
                                        ("moonlight-small", True)])
def test_prenorm_loop_equals_host_driven(name, gated):
    dev = device()
    cfg = _cfg(name)
    W = tuple(None if w is None else cle.pack_weights(w) for w in synth.weights_torch(cfg, 2, dev))
    h0 = to_dev(np.stack([synth.hidden(cfg, 2, j) for j in range(cfg.n)]), "bf16", dev)
    if gated:
        gate = (cle.pack_weights(synth.gate_weights_torch(cfg, 2, dev)),
                torch.from_numpy(synth.gate_bias(cfg, 2)).to(dev))
        lt = None
    else:
        gate = None
        lt = torch.from_numpy(np.stack([np.stack([synth.logits(cfg, 2, j, l) for l in range(cfg.L)])
                                        for j in range(cfg.n)])).to(dev)
    print(f"[prenorm loop] {name} gated={gated}", flush=True)
    kw = dict(packed=True, gate=gate, prenorm=True)
    host = Engine(W, lt, h0, cfg.D, cfg.k, cle.POLICY_CUMUTIL, cfg.m, **kw).run()
    dl = Engine(W, lt, h0, cfg.D, cfg.k, cle.POLICY_CUMUTIL, cfg.m, device_loop=True, **kw).run()
    torch.cuda.synchronize()
    assert dl.trace == host.trace and dl.stats()[0] == host.stats()[0]
    assert np.array_equal(bits_of(dl.h), bits_of(host.h))


def test_prenorm_sampled_chain_vs_oracle():
    """Three tokens followed through 4 layers by the oracle, from the seeded
    inputs alone: rmsnorm, route, SwiGLU experts, Eq. (1), residual."""
    dev = device()
    cfg = synth.small(synth.CONFIGS["qwen3"], L=4, T=128, n=2)
    W = synth.weights_torch(cfg, 1, dev)
    logits = np.stack([np.stack([synth.logits(cfg, 1, j, l) for l in range(cfg.L)])
                       for j in range(cfg.n)])
    h0 = np.stack([synth.hidden(cfg, 1, j) for j in range(cfg.n)])
    eng = Engine(W, torch.from_numpy(logits).to(dev), to_dev(h0, "bf16", dev), cfg.D, cfg.k,
                 cle.POLICY_CUMUTIL, 1, prenorm=True).run()
    got = oracle.widen(to_host(eng.h[1]), "bf16")
    for t in (0, 63, 127):
        x = oracle.widen(h0[1, t:t + 1], "bf16")
        for l in range(cfg.L):
            xn = oracle.rmsnorm(x, cle.NORM_EPS)
            idx, gates = oracle.route(logits[1, l, t:t + 1], cfg.k)
            yp = np.concatenate([
                oracle.swiglu_expert(xn, oracle.widen(to_host(W[0][l, int(e)]), "bf16"),
                                     oracle.widen(to_host(W[1][l, int(e)]), "bf16"))
                for e in idx[0]])
            x = oracle.combine(yp, np.arange(cfg.k), gates, cfg.k, residual=x)
        check_close(got[t:t + 1], x, 2e-2 * cfg.L ** 0.5, 1e-2,
                    what=f"pre-norm token {t} after {cfg.L} layers")


@pytest.mark.parametrize("gated", [False, True])
def test_full_stack_stays_finite_with_prenorm(gated):
    """48 Qwen3-shaped layers (512 tokens per micro-batch): with the pre-norm
    block the hidden state stays finite and of moderate size."""
    dev = device()
    cfg = synth.small(synth.CONFIGS["qwen3"], T=512)
    W = tuple(cle.pack_weights(w) if w is not None else None for w in synth.weights_torch(cfg, 0, dev))
    h0 = to_dev(np.stack([synth.hidden(cfg, 0, j) for j in range(cfg.n)]), "bf16", dev)
    if gated:
        gate, lt = (cle.pack_weights(synth.gate_weights_torch(cfg, 0, dev)),
                    torch.from_numpy(synth.gate_bias(cfg, 0)).to(dev)), None
    else:
        gate = None
        lt = torch.from_numpy(np.stack([np.stack([synth.logits(cfg, 0, j, l) for l in range(cfg.L)])
                                        for j in range(cfg.n)])).to(dev)
    print(f"[prenorm] full stack gated={gated}", flush=True)
    eng = Engine(W, lt, h0, cfg.D, cfg.k, cle.POLICY_CUMUTIL, cfg.m, packed=True, gate=gate,
                 prenorm=True, device_loop=True).run()
    h = eng.h.float()
    assert torch.isfinite(h).all()
    rms = h.pow(2).mean().sqrt().item()
    print(f"[prenorm] rms of h after {cfg.L} layers: {rms:.3f}; 1-u {1 - eng.stats()[1]:.4f}",
          flush=True)
    assert 0.5 < rms < 50


@pytest.mark.parametrize("policy", ["cumutil", "maxutil"])
def test_prenorm_whole_run_vs_oracle(policy):
    """The block bench.py times (pre-norm, packed weights, device-driven loop)
    over a whole Algorithm 1 run against the oracle's run_engine with the
    pre-norm block, on a reduced stack of the Qwen3 structure: the schedule
    and the Eq. (3) accumulators exactly, the final hidden states within the
    tolerance chained over the layers (the GPU rounds h to bf16 after every
    layer)."""
    dev = device()
    cfg = synth.small(synth.CONFIGS["qwen3"], L=6, T=128, n=4, H=512, I=256, E=32, k=4, m=3)
    W = synth.weights_torch(cfg, 3, dev)
    logits = np.stack([np.stack([synth.logits(cfg, 3, j, l) for l in range(cfg.L)])
                       for j in range(cfg.n)])
    h0 = np.stack([synth.hidden(cfg, 3, j) for j in range(cfg.n)])
    Wk = tuple(None if w is None else cle.pack_weights(w) for w in W)
    print(f"[prenorm run] {policy}", flush=True)
    eng = Engine(Wk, torch.from_numpy(logits).to(dev), to_dev(h0, "bf16", dev), cfg.D, cfg.k,
                 cle.POLICIES[policy], cfg.m, packed=True, prenorm=True, device_loop=True).run()
    torch.cuda.synchronize()
    w13, w2 = oracle.widen(to_host(W[0]), "bf16"), oracle.widen(to_host(W[1]), "bf16")
    h_ref, trace, acc, u = oracle.run_engine(
        [oracle.widen(h, "bf16") for h in h0], lambda j, l: logits[j, l], cfg.k, cfg.D, w13, w2,
        cfg.m, oracle.POLICIES[policy], prenorm=True, eps=cle.NORM_EPS)
    assert eng.trace == trace, "schedule differs from the oracle's Algorithm 1"
    a, ug = eng.stats()
    assert a[:3] == list(acc) and a[3] == len(trace)
    for j in range(cfg.n):
        check_close(oracle.widen(to_host(eng.h[j]), "bf16"), h_ref[j], 2e-2 * cfg.L ** 0.5, 1e-2,
                    what=f"h[{j}] after {cfg.L} layers ({policy})")
