"""cle_grouped_expert_ffn_noalloc (the expert launch without a workspace
argument, for callers that cannot allocate) against cle_grouped_expert_ffn
on the same inputs: bitwise equal outputs on two calls in a row, the second
with a smaller input (fewer descriptors and rows, so stale contents of the
library's fixed scratch from the first call would show), for bf16 packed
weights (with the row map) and float32; sizes past the fixed scratch are
rejected before anything runs."""
import numpy as np
import pytest
import torch

import cross_layer_expert_amd as cle
import synth
from gpu_helpers import bits_of, device, to_dev

pytestmark = pytest.mark.gpu


def _inputs(dtype, H, I, E, L, layers, sizes_list, seed):
    dev = device()
    rng = np.random.default_rng(seed)
    cfg = synth.Config("case", L=L, H=H, E=E, k=1, I=I, D=1, n=len(layers), T=1, dtype=dtype)
    w13, w2, _, _ = synth.weights_numpy(cfg, seed)
    W13, W2 = to_dev(w13, dtype, dev), to_dev(w2, dtype, dev)
    packed = dtype == "bf16"
    if packed:
        W13, W2 = cle.pack_weights(W13), cle.pack_weights(W2)
    keep, descs = [], []
    for l, sizes in zip(layers, sizes_list):
        rows = int(sum(sizes))
        offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
        ntok = -(-max(rows, 1) // 2)
        x = synth.store(rng.standard_normal((ntok, H)).astype(np.float32), dtype)
        src = rng.permutation(ntok * 2)[:rows].astype(np.int32)
        t = dict(offsets=torch.from_numpy(offsets).to(dev), x=to_dev(x, dtype, dev),
                 src=torch.from_numpy(src).to(dev))
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        t["act"] = torch.full((max(rows, 1), I), 3.0, dtype=tdt, device=dev)
        t["yp"] = torch.full((max(rows, 1), H), 3.0, dtype=tdt, device=dev)
        keep.append(t)
        descs.append(cle.make_desc(l, rows, t["offsets"], None, t["act"], t["yp"], x=t["x"],
                                   src=t["src"], k=2))
    return dict(W=(W13, W2), packed=packed, keep=keep, descs=descs, E=E)


def _outputs(case):
    return [(bits_of(t["act"]), bits_of(t["yp"])) for t in case["keep"]]


def _both(case):
    dev = device()
    W13, W2 = case["W"]
    ws = torch.empty(cle.workspace_bytes(cle.OP_FFN, 0, case["E"], 1, 0, len(case["descs"])) // 4,
                     dtype=torch.int32, device=dev)
    for t in case["keep"]:
        t["act"].fill_(3.0)
        t["yp"].fill_(3.0)
    cle.grouped_expert_ffn(case["descs"], W13, W2, ws, packed=case["packed"])
    torch.cuda.synchronize()
    ref = _outputs(case)
    for t in case["keep"]:
        t["act"].fill_(3.0)
        t["yp"].fill_(3.0)
    cle.grouped_expert_ffn_noalloc(case["descs"], W13, W2, packed=case["packed"])
    torch.cuda.synchronize()
    got = _outputs(case)
    for (ra, ry), (ga, gy) in zip(ref, got):
        assert np.array_equal(ga, ra) and np.array_equal(gy, ry)


@pytest.mark.parametrize("dtype,H,I", [("bf16", 2048, 768), ("bf16", 512, 256), ("f32", 64, 128)])
def test_noalloc_equals_workspace_call_twice(dtype, H, I):
    E = 16
    rng = np.random.default_rng(H)
    big = [list(rng.integers(0, 300, E)) for _ in range(5)]
    small = [[0, 3, 129, 0, 1] + [0] * (E - 5)]
    print(f"[noalloc] {dtype} H={H} I={I}: 5 descriptors, then 1", flush=True)
    _both(_inputs(dtype, H, I, E, 3, [2, 0, 1, 2, 0], big, seed=1))
    _both(_inputs(dtype, H, I, E, 3, [1], small, seed=2))


def test_noalloc_rejects_sizes_past_its_scratch():
    dev = device()
    E = 1024
    z = torch.zeros(E + 1, dtype=torch.int32, device=dev)
    yp = torch.zeros((1, 128), dtype=torch.bfloat16, device=dev)
    W = torch.zeros((1, E, 2 * 64, 128), dtype=torch.bfloat16, device="meta")
    need = cle.workspace_bytes(cle.OP_FFN, 0, E, 1, 0, 64)
    assert need > cle.NOALLOC_SCRATCH_BYTES
    descs = [cle.make_desc(0, 0, z, yp, yp, yp) for _ in range(64)]
    arr = (cle.FfnDesc * 64)(*descs)
    st = cle._lib.cle_grouped_expert_ffn_noalloc(arr, 64, yp.data_ptr(), yp.data_ptr(), None,
                                                 None, 1, E, 0, 128, 64, cle.BF16,
                                                 cle.W_ROWMAJOR, None, None)
    assert st == cle.EUNSUPPORTED
    del W
