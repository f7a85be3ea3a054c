"""The device-driven loop: Schedule(S, m) on the device (cle_schedule_step_device)
and whole steps with device-resident masks (cle_loop_step).

Bars: the device schedule equals the oracle's Schedule(S, m) (and the host
library's) exactly, on hand examples and on random workloads full of ties,
up to MaxUtil's largest pool; a device-driven run is bitwise equal to the
host-driven run of the same inputs (hidden states, RunSets with their
layers, statistics) for every policy, with shared experts and with
staggered start layers; a restarting loop replays the first run exactly.
"""
import json
import os
import random

import numpy as np
import pytest
import torch

import cross_layer_expert_amd as cle
import oracle
import synth
from cross_layer_expert_amd.engine import Engine
from gpu_helpers import bits_of, device, to_dev

pytestmark = pytest.mark.gpu

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _dev_schedule(w, ready, m, policy):
    dev = device()
    wt = torch.from_numpy(np.ascontiguousarray(w, dtype=np.int32)).to(dev)
    out = torch.full((1,), -1, dtype=torch.int64, device=dev)
    cle.schedule_step_device(wt, cle.mask_of(ready), m, policy, out)
    return cle.ids_of(int(out.cpu().numpy().view(np.uint64)[0]))


def test_schedule_device_hand_examples():
    with open(os.path.join(GOLD, "schedule_examples.json")) as f:
        examples = json.load(f)["examples"]
    for ex in examples:
        ready = ex.get("ready", list(range(len(ex["w"]))))
        for name, want in ex["expect"].items():
            print(f"[sched dev] {ex['name']} {name}", flush=True)
            assert _dev_schedule(ex["w"], ready, ex["m"], cle.POLICIES[name]) == want


@pytest.mark.parametrize("policy", sorted(cle.POLICIES))
def test_schedule_device_random(policy):
    rnd = random.Random(len(policy))
    pol = cle.POLICIES[policy]
    print(f"[sched dev] random {policy}", flush=True)
    for case in range(150):
        n = rnd.randint(1, 12 if policy == "maxutil" else 64)
        D = rnd.choice([1, 2, 3, 8, 17, 64])
        w = np.array([[rnd.choice([0, 0, 1, 2, 3, 5, 8, 1000]) for _ in range(D)]
                      for _ in range(n)], dtype=np.int32)
        ready = [j for j in range(n) if rnd.random() < 0.8] or [n - 1]
        m = rnd.randint(1, n)
        want = list(oracle.schedule(w.tolist(), ready, m, pol))
        got = _dev_schedule(w, ready, m, pol)
        host = cle.ids_of(cle.schedule_step(w, cle.mask_of(ready), m, pol))
        assert got == want == host, (case, n, D, m, ready)


def test_schedule_device_maxutil_large_pools():
    """Large workloads (sums reach 2^33, cross products 2^66) and pools of 16
    against the oracle; the largest pool (20, 2^20 subsets) against the host
    library, which the oracle pins elsewhere."""
    rng = np.random.default_rng(9)
    for pool, m in ((16, 1), (16, 9), (20, 1), (20, 10)):
        w = rng.integers(0, 1 << 28, size=(pool, 8)).astype(np.int32)
        w[3] = w[5]                       # a duplicate row: ties between subsets
        print(f"[sched dev] maxutil pool {pool} m={m}", flush=True)
        got = _dev_schedule(w, list(range(pool)), m, cle.POLICY_MAXUTIL)
        host = cle.ids_of(cle.schedule_step(w, (1 << pool) - 1, m, cle.POLICY_MAXUTIL))
        assert got == host
        if pool <= 16:
            assert got == list(oracle.schedule(w.tolist(), range(pool), m, cle.POLICY_MAXUTIL))


def _inputs(cfg, seed):
    dev = device()
    if cfg.dtype == "f32":
        W = [None if w is None else to_dev(w, "f32", dev) for w in synth.weights_numpy(cfg, seed)]
    else:
        W = synth.weights_torch(cfg, seed, dev)
    logits = np.stack([np.stack([synth.logits(cfg, seed, j, l) for l in range(cfg.L)])
                       for j in range(cfg.n)])
    h0 = np.stack([synth.hidden(cfg, seed, j) for j in range(cfg.n)])
    return W, torch.from_numpy(logits).to(dev), to_dev(h0, cfg.dtype, dev)


CASES = [("tiny", p) for p in sorted(cle.POLICIES)] + [
    ("qwen3-small", "cumutil"), ("qwen3-small", "maxutil"), ("moonlight-small", "cumutil"),
    ("decode-small", "diffpeak"), ("decode-small", "b1")]


def _cfg(name):
    if name == "tiny":
        return synth.CONFIGS["tiny"]
    base = synth.CONFIGS[name.split("-")[0]]
    over = dict(L=6, T=256)
    if name.startswith("decode"):
        over = dict(L=12, T=64, n=6, start_layers=tuple(2 * j for j in range(6)), m=4)
    return synth.small(base, **over)


@pytest.mark.parametrize("name,policy", CASES)
def test_loop_equals_host_driven(name, policy):
    cfg = _cfg(name)
    W, lt, ht = _inputs(cfg, 6)
    m = cfg.m
    packed = cfg.dtype == "bf16"
    Wk = tuple(None if w is None else cle.pack_weights(w) for w in W) if packed else W
    print(f"[loop] {name} {policy}", flush=True)
    host = Engine(Wk, lt, ht, cfg.D, cfg.k, cle.POLICIES[policy], m,
                  start_layers=cfg.start_layers, packed=packed).run()
    dl = Engine(Wk, lt, ht, cfg.D, cfg.k, cle.POLICIES[policy], m,
                start_layers=cfg.start_layers, packed=packed, device_loop=True).run()
    torch.cuda.synchronize()
    assert dl.trace == host.trace
    assert dl.stats()[0] == host.stats()[0]
    assert np.array_equal(bits_of(dl.h), bits_of(host.h))
    st = cle.read_loop_state(dl.state)
    assert st.ready == 0 and st.todo == 0 and list(st.layer)[:cfg.n] == [cfg.L] * cfg.n
    # the workloads the last schedule saw are those of the host path
    assert np.array_equal(dl.w_dev.cpu().numpy(), host.w_dev.cpu().numpy())


@pytest.mark.parametrize("name,prenorm,gated", [("qwen3-small", False, False), ("tiny", False, False),
                                                 ("qwen3-small", True, True)])
def test_loop_restart_replays_first_run(name, prenorm, gated):
    """The step that finishes the last micro-batch restarts the loop (the
    combine writes h <- h0 there): the states are h0 again, and the next run
    replays the first one step for step (f32 tiles; bf16 with the pre-norm
    block and routing through the router)."""
    cfg = _cfg(name)
    W, lt, ht = _inputs(cfg, 8)
    packed = cfg.dtype == "bf16"
    Wk = tuple(None if w is None else cle.pack_weights(w) for w in W) if packed else tuple(W)
    kw = dict(packed=packed, prenorm=prenorm)
    if gated:
        dev = device()
        kw["gate"] = (cle.pack_weights(synth.gate_weights_torch(cfg, 8, dev)),
                      torch.from_numpy(synth.gate_bias(cfg, 8)).to(dev))
        lt = None
    print(f"[loop] restart {name} prenorm={prenorm} gated={gated}", flush=True)
    one = Engine(Wk, lt, ht, cfg.D, cfg.k, cle.POLICY_CUMUTIL, cfg.m, **kw).run()
    steps = len(one.trace)
    rs = Engine(Wk, lt, ht, cfg.D, cfg.k, cle.POLICY_CUMUTIL, cfg.m, device_loop=True,
                restart=True, **kw)
    for _ in range(steps):
        rs.step()
    st = rs.sync_trace()
    assert st.restarts == 1 and rs.trace == one.trace
    assert np.array_equal(bits_of(rs.h), bits_of(ht))          # back to h0
    part = Engine(Wk, lt, ht, cfg.D, cfg.k, cle.POLICY_CUMUTIL, cfg.m, **kw)
    for _ in range(5):
        part.step()
        rs.step()
    rs.sync_trace()
    assert rs.trace[steps:] == part.trace
    assert np.array_equal(bits_of(rs.h), bits_of(part.h))
    assert np.array_equal(bits_of(rs.h), bits_of(part.h))
    acc = rs.stats()[0]
    assert acc[3] == steps + 5 and acc[:3] == [a + b for a, b in
                                                zip(one.stats()[0][:3], part.stats()[0][:3])]
