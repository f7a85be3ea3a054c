"""Routing from the hidden state: router logits z = h W_g^T + b
(cle_gate_logits_many) in front of top-k, and the engine routed through it.

Bars:
* logits within the float32-accumulation bound of the float64 oracle,
  |dz| <= H * 2^-24 * sum_h |x_h w_eh| + 2^-24 |b_e| (bf16 products are exact
  in float32; only the sum rounds), and bitwise reproducible, batched equal
  to per-micro-batch, packed equal to row-major;
* routing of the GPU logits bit-exact with the oracle's routing of the same
  logits (indices and gates);
* the selection valid against the oracle logits up to twice the bound
  (near-ties may flip: several answers are correct, so validity is checked);
* device-driven runs routed through the gate bitwise equal to host-driven.
"""
import numpy as np
import pytest
import torch

import cross_layer_expert_amd as cle
import oracle
import synth
from cross_layer_expert_amd.engine import Engine
from gpu_helpers import bits_of, device, to_dev, to_host

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _bound(x, w, b):
    """Elementwise error bound of float32 accumulation over H terms."""
    H = x.shape[1]
    s = np.abs(x) @ np.abs(w).T
    return H * U * s + (U * np.abs(b)[None, :] if b is not None else 0.0) + 1e-30


def _check_routing(z_gpu, z_ref, bound, idx_gpu, k):
    # the GPU's top-k of its own logits is the oracle's, bit for bit
    ridx, _ = oracle.route(z_gpu, k)
    assert np.array_equal(idx_gpu, ridx)
    # and a valid top-k of the exact logits up to twice the bound
    T, E = z_ref.shape
    rows = np.arange(T)[:, None]
    sel = np.zeros((T, E), bool)
    sel[rows, idx_gpu] = True
    worst_in = np.where(sel, z_ref + 2 * bound, np.inf).min(axis=1)
    best_out = np.where(~sel, z_ref, -np.inf).max(axis=1)
    assert np.all(worst_in >= best_out)
    flips = int((np.sort(oracle.route(z_ref, k)[0], axis=1) != np.sort(idx_gpu, axis=1)).any(axis=1).sum())
    return flips


@pytest.mark.parametrize("n,T,H,E,k,dtype,use_bias,packed", [
    (3, 2048, 2048, 128, 8, "bf16", True, True),     # Qwen3 shape, three micro-batches
    (2, 1024, 2048, 64, 6, "bf16", True, False),     # Moonlight shape
    (2, 1024, 2048, 64, 6, "bf16", True, True),      # Moonlight shape, packed router
    (2, 37, 256, 64, 4, "bf16", False, False),       # ragged T
    (1, 1, 128, 1024, 8, "bf16", True, True),        # one token, 1024 experts
    (2, 16, 64, 8, 2, "f32", True, False),           # tiny f32
])
def test_gate_logits_and_routing(n, T, H, E, k, dtype, use_bias, packed):
    dev = device()
    rng = np.random.default_rng(T + H + E)
    xs = [synth.store(rng.standard_normal((T, H)).astype(np.float32), dtype) for _ in range(n)]
    ws = [synth.store((rng.standard_normal((E, H)) / np.sqrt(H)).astype(np.float32), dtype)
          for _ in range(n)]
    bs = [rng.standard_normal(E).astype(np.float32) if use_bias else None for _ in range(n)]
    xt = [to_dev(a, dtype, dev) for a in xs]
    wt = [to_dev(a, dtype, dev) for a in ws]
    wk = [cle.pack_weights(w) for w in wt] if packed else wt
    bt = [torch.from_numpy(b).to(dev) for b in bs] if use_bias else None
    z = [torch.full((T, E), float("nan"), dtype=torch.float32, device=dev) for _ in range(n)]
    print(f"[gate] n={n} T={T} H={H} E={E} {dtype} bias={use_bias} packed={packed}", flush=True)
    cle.gate_logits_many(xt, wk, z, bias=bt, packed=packed)
    z1 = [torch.empty_like(a) for a in z]
    for j in range(n):                                  # one micro-batch per call
        cle.gate_logits_many([xt[j]], [wk[j]], [z1[j]], bias=None if bt is None else [bt[j]],
                             packed=packed)
    if packed:                                          # row-major weights, same bits
        z2 = [torch.empty_like(a) for a in z]
        cle.gate_logits_many(xt, wt, z2, bias=bt)
    idx = torch.empty((n, T, k), dtype=torch.int32, device=dev)
    gate = torch.empty((n, T, k), dtype=torch.float32, device=dev)
    cle.route_many(z, k, list(idx), list(gate))
    torch.cuda.synchronize()
    for j in range(n):
        assert np.array_equal(bits_of(z[j]), bits_of(z1[j]))
        if packed:
            assert np.array_equal(bits_of(z[j]), bits_of(z2[j]))
        x64, w64 = oracle.widen(xs[j], dtype), oracle.widen(ws[j], dtype)
        ref = oracle.gate_logits(x64, w64, bs[j])
        zg = z[j].cpu().numpy()
        bound = _bound(x64, w64, bs[j])
        err = np.abs(zg - ref)
        print(f"[gate] j={j} max|dz|={err.max():.3e} max bound={bound.max():.3e} "
              f"max err/bound={(err / bound).max():.3e}", flush=True)
        assert np.all(err <= bound)
        flips = _check_routing(zg, ref, bound, idx[j].cpu().numpy(), k)
        _, rg = oracle.route(zg, k)
        assert np.array_equal(gate[j].cpu().numpy().view(np.int32), rg.view(np.int32))
        print(f"[gate] j={j} tokens whose top-k set differs from the exact logits': {flips}",
              flush=True)


def _cfg(name):
    if name == "tiny":
        return synth.CONFIGS["tiny"]
    base = synth.CONFIGS[name.split("-")[0]]
    if name.startswith("decode"):
        return synth.small(base, L=12, T=64, n=6, start_layers=tuple(2 * j for j in range(6)), m=4)
    return synth.small(base, L=6, T=256)


def _gated_inputs(cfg, seed, packed):
    dev = device()
    if cfg.dtype == "f32":
        W = [None if w is None else to_dev(w, "f32", dev) for w in synth.weights_numpy(cfg, seed)]
        wg = to_dev(synth.gate_weights_numpy(cfg, seed), "f32", dev)
    else:
        W = synth.weights_torch(cfg, seed, dev)
        wg = synth.gate_weights_torch(cfg, seed, dev)
    if packed:
        W = tuple(None if w is None else cle.pack_weights(w) for w in W)
        wg = cle.pack_weights(wg)
    gb = torch.from_numpy(synth.gate_bias(cfg, seed)).to(dev)
    h0 = np.stack([synth.hidden(cfg, seed, j) for j in range(cfg.n)])
    return W, (wg, gb), to_dev(h0, cfg.dtype, dev)


@pytest.mark.parametrize("name,policy", [("tiny", "cumutil"), ("tiny", "maxutil"),
                                         ("qwen3-small", "cumutil"), ("moonlight-small", "diffpeak"),
                                         ("decode-small", "b1")])
def test_gated_loop_equals_host_driven(name, policy):
    cfg = _cfg(name)
    packed = cfg.dtype == "bf16"
    W, gate, ht = _gated_inputs(cfg, 3, packed)
    print(f"[gated loop] {name} {policy}", flush=True)
    host = Engine(W, None, ht, cfg.D, cfg.k, cle.POLICIES[policy], cfg.m,
                  start_layers=cfg.start_layers, packed=packed, gate=gate).run()
    dl = Engine(W, None, ht, cfg.D, cfg.k, cle.POLICIES[policy], cfg.m,
                start_layers=cfg.start_layers, packed=packed, gate=gate, device_loop=True).run()
    torch.cuda.synchronize()
    assert dl.trace == host.trace
    assert dl.stats()[0] == host.stats()[0]
    assert np.array_equal(bits_of(dl.h), bits_of(host.h))


def test_gated_step_routes_from_hidden_state():
    """The first step of a gated engine: every micro-batch's routing comes
    from its hidden state through its layer's router (checked against the
    oracle as above), and after the step the hidden states of the members
    changed while the others did not."""
    cfg = _cfg("qwen3-small")
    W, (wg, gb), ht = _gated_inputs(cfg, 5, False)
    eng = Engine(W, None, ht, cfg.D, cfg.k, cle.POLICY_CUMUTIL, cfg.m, gate=(wg, gb))
    h_before = to_host(eng.h).copy()
    R = eng.step()
    torch.cuda.synchronize()
    for j in range(cfg.n):
        x64 = oracle.widen(h_before[j], "bf16")
        w64 = oracle.widen(to_host(wg[0]), "bf16")
        b = gb[0].cpu().numpy()
        ref = oracle.gate_logits(x64, w64, b)
        zg = eng.glog[j].cpu().numpy()
        bound = _bound(x64, w64, b)
        assert np.all(np.abs(zg - ref) <= bound)
        _check_routing(zg, ref, bound, eng.idx[j].cpu().numpy(), cfg.k)
    h_after = to_host(eng.h)
    for j in range(cfg.n):
        assert np.array_equal(h_after[j], h_before[j]) == (j not in R)
