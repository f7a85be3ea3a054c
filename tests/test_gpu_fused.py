"""The fused gate/up -> down launch for thin segments (cle_set_fused_thin_rows):
segments of 1 .. 16 rows run in one launch (one workgroup per segment, both
phases) and the rest in the two phase launches.  Outputs are bitwise those of
the unfused launches -- for ragged segments around the threshold, with rows
read in place through the dispatch permutation or from an expert-sorted copy,
and for a whole device-driven run -- and within the element-wise bound of the
float64 oracle."""
import numpy as np
import pytest
import torch

import cross_layer_expert_amd as cle
import oracle
import synth
from cross_layer_expert_amd.engine import Engine
from gpu_helpers import bits_of, check_bound, device, swiglu_bound, to_dev, to_host
from test_gpu_tiles import _case

pytestmark = pytest.mark.gpu

SIZES = [0, 1, 2, 15, 16, 17, 31, 64, 128, 129, 300, 3, 7, 0, 11, 16]


def _run(case, rows):
    cle.set_fused_thin_rows(rows)
    try:
        for t in case["keep"]:
            t["yp"].fill_(7.0)
            t["act"].fill_(7.0)
        cle.grouped_expert_ffn(case["descs"], case["W"][0], case["W"][1], case["ws"], packed=True)
        torch.cuda.synchronize()
    finally:
        cle.set_fused_thin_rows(-1)
    return [(bits_of(t["act"]), bits_of(t["yp"])) for t in case["keep"]]


@pytest.mark.parametrize("fused_gather", [False, True])
def test_fused_thin_bitwise_and_oracle(fused_gather):
    rng = np.random.default_rng(4)
    sizes = [SIZES, list(rng.permutation(SIZES)), [1] * len(SIZES)]
    print(f"[fused] gather={fused_gather}", flush=True)
    case = _case(2048, 768, len(SIZES), 2, [1, 0, 1], sizes, seed=7, fused=fused_gather)
    off = _run(case, 0)
    on = _run(case, 16)
    for j, (a, b) in enumerate(zip(off, on)):
        rows = case["refs"][j][3]
        assert np.array_equal(a[0][:rows], b[0][:rows]) and np.array_equal(a[1][:rows], b[1][:rows])
    w13, w2 = case["w"]
    for j, (t, (x, offsets, l, rows)) in enumerate(zip(case["keep"], case["refs"])):
        got = oracle.widen(to_host(t["yp"])[:rows], "bf16")
        for e in range(len(offsets) - 1):
            a, b = int(offsets[e]), int(offsets[e + 1])
            if b > a:
                we13, we2 = oracle.widen(w13[l, e], "bf16"), oracle.widen(w2[l, e], "bf16")
                check_bound(got[a:b], oracle.swiglu_expert(x[a:b], we13, we2),
                            swiglu_bound(x[a:b], we13, we2, "bf16"), quiet=True,
                            what=f"fused desc {j} expert {e} rows {b - a}")


def test_fused_thin_engine_run_bitwise():
    """A device-driven run of the Qwen3 structure (many thin segments) with the
    fused launch equals the run without it, bit for bit."""
    dev = device()
    cfg = synth.small(synth.CONFIGS["qwen3"], L=4, T=256, n=4)
    W = tuple(None if w is None else cle.pack_weights(w) for w in synth.weights_torch(cfg, 5, dev))
    lt = torch.from_numpy(np.stack([np.stack([synth.logits(cfg, 5, j, l) for l in range(cfg.L)])
                                    for j in range(cfg.n)])).to(dev)
    ht = to_dev(np.stack([synth.hidden(cfg, 5, j) for j in range(cfg.n)]), "bf16", dev)
    outs = []
    for rows in (0, 16):
        cle.set_fused_thin_rows(rows)
        try:
            eng = Engine(W, lt, ht, cfg.D, cfg.k, cle.POLICY_CUMUTIL, cfg.m, packed=True,
                         prenorm=True, device_loop=True).run()
            torch.cuda.synchronize()
        finally:
            cle.set_fused_thin_rows(-1)
        outs.append((eng.trace, bits_of(eng.h)))
    assert outs[0][0] == outs[1][0]
    assert np.array_equal(outs[0][1], outs[1][1])
