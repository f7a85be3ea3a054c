"""Packed expert weights (cle_pack_weights, CLE_W_PACKED).

Bars: the packed tensor equals an independent host re-layout of the
documented format element for element; the grouped expert launch with packed
weights is bitwise equal to the launch with the row-major weights (the packed
blocks land in LDS byte for byte as the row-major ones do); a whole engine run
with packed weights is bitwise equal to one with row-major weights.
"""
import numpy as np
import pytest
import torch

import cross_layer_expert_amd as cle
import synth
from cross_layer_expert_amd.engine import Engine
from gpu_helpers import bits_of, device, to_dev

pytestmark = pytest.mark.gpu


def _packed_reference(w):
    """Host re-layout of [M, R, K] uint16 by the format's definition: blocks of
    16 rows x 64 K in (row block, K block) order, two 8-row groups per block,
    chunk c of row r of a group at position r * 8 + (c ^ r)."""
    M, R, K = w.shape
    out = np.empty(M * R * K, dtype=w.dtype)
    q = 0
    for m in range(M):
        for rb in range(R // 16):
            for kb in range(K // 64):
                for g in range(2):
                    for pos in range(64):
                        r, c = pos // 8, None
                        # position pos holds chunk c with (c ^ r) == pos % 8
                        c = (pos % 8) ^ r
                        row = rb * 16 + g * 8 + r
                        col = kb * 64 + c * 8
                        out[q:q + 8] = w[m, row, col:col + 8]
                        q += 8
    return out.reshape(M, R, K)


@pytest.mark.parametrize("M,R,K", [(1, 16, 64), (3, 48, 192), (2, 1536, 128)])
def test_pack_layout(M, R, K):
    dev = device()
    rng = np.random.default_rng(R + K)
    w = rng.integers(0, 1 << 16, size=(M, R, K), dtype=np.uint16)
    t = torch.from_numpy(w.view(np.int16)).to(dev).view(torch.bfloat16)
    print(f"[pack] M={M} R={R} K={K}", flush=True)
    p = cle.pack_weights(t)
    torch.cuda.synchronize()
    got = bits_of(p).view(np.uint16)
    assert np.array_equal(got, _packed_reference(w))
    # in place, a few matrices at a time, gives the same bytes
    t2 = t.clone()
    cle.pack_weights_inplace(t2, mats_per_chunk=2)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(t2), bits_of(p))


def _ffn(H, I, E, L, ns, layers, sizes_list, packed_too=True, seed=3):
    dev = device()
    rng = np.random.default_rng(seed)
    cfg = synth.Config("case", L=L, H=H, E=E, k=1, I=I, D=1, n=len(layers), T=1, dtype="bf16",
                       n_shared=ns)
    W = [None if w is None else to_dev(w, "bf16", dev) for w in synth.weights_numpy(cfg, seed)]
    Wp = [None if w is None else cle.pack_weights(w) for w in W]
    outs = []
    for weights, packed in ((W, False), (Wp, True)):
        descs, keep = [], []
        for l, sizes in zip(layers, sizes_list):
            rows = int(sum(sizes))
            off = torch.from_numpy(np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)).to(dev)
            g = np.random.default_rng(seed + l)        # same inputs for both layouts
            xp = to_dev(synth.store(g.standard_normal((rows, H)).astype(np.float32), "bf16"),
                        "bf16", dev)
            Ts = max(rows // 2, 1)
            xs = to_dev(synth.store(g.standard_normal((Ts, H)).astype(np.float32), "bf16"),
                        "bf16", dev) if ns else None
            act = torch.zeros((rows, I), dtype=torch.bfloat16, device=dev)
            yp = torch.zeros((rows, H), dtype=torch.bfloat16, device=dev)
            acts = torch.zeros((ns, Ts, I), dtype=torch.bfloat16, device=dev) if ns else None
            ys = torch.zeros((ns, Ts, H), dtype=torch.bfloat16, device=dev) if ns else None
            keep.append((off, xp, xs, act, yp, acts, ys))
            descs.append(cle.make_desc(l, rows, off, xp, act, yp, Ts if ns else 0, xs, acts, ys))
        ws = torch.empty(cle.workspace_bytes(cle.OP_FFN, 0, E, 1, ns, len(descs)) // 4,
                         dtype=torch.int32, device=dev)
        cle.grouped_expert_ffn(descs, weights[0], weights[1], ws, weights[2], weights[3],
                               packed=packed)
        torch.cuda.synchronize()
        outs.append([bits_of(t) for k in keep for t in k[3:] if t is not None])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("H,I,ns", [(128, 64, 0), (256, 128, 0), (128, 192, 1), (2048, 768, 0),
                                     (512, 640, 0), (1280, 256, 0)])
def test_ffn_packed_equals_rowmajor(H, I, ns):
    """Wide and narrow tiles, shared experts, the Qwen3 reduction lengths and
    the other K-loop tails of the wide tiles."""
    print(f"[ffn packed] H={H} I={I} ns={ns}", flush=True)
    E = 8
    sizes = [[0, 1, 63, 64, 65, 130, 7, 0], [200, 0, 0, 0, 0, 0, 0, 3], [16] * 8]
    _ffn(H, I, E, 3, ns, [2, 0, 1], sizes)


def test_engine_packed_equals_rowmajor():
    dev = device()
    cfg = synth.small(synth.CONFIGS["qwen3"], L=4, T=256)
    W = synth.weights_torch(cfg, 5, dev)
    Wp = tuple(None if w is None else cle.pack_weights(w) for w in W)
    logits = np.stack([np.stack([synth.logits(cfg, 5, j, l) for l in range(cfg.L)])
                       for j in range(cfg.n)])
    h0 = np.stack([synth.hidden(cfg, 5, j) for j in range(cfg.n)])
    lt, ht = torch.from_numpy(logits).to(dev), to_dev(h0, "bf16", dev)
    print("[engine packed] qwen3-small", flush=True)
    a = Engine(W, lt, ht, cfg.D, cfg.k, cle.POLICY_CUMUTIL, cfg.m).run()
    b = Engine(Wp, lt, ht, cfg.D, cfg.k, cle.POLICY_CUMUTIL, cfg.m, packed=True).run()
    assert np.array_equal(bits_of(a.h), bits_of(b.h)) and a.trace == b.trace
