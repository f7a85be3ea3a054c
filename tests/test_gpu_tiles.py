"""The output tiles of the bf16 expert launch (cle_set_expert_tile): 128 x 256,
256 x 256 and 128 x 512 give bitwise the same results on ragged segments of
several micro-batches at different layers, and every one matches the float64
oracle element by element within the rounding-error bound of the expert FFN
(tests/gpu_helpers.py).  With many more tiles than workgroups, the per-XCD
tile claims cover every tile exactly once: each XCD's claim counter ends at
the size of its tile range (one claim per tile run), and every output row is
checked."""
import numpy as np
import pytest
import torch

import cross_layer_expert_amd as cle
import oracle
import synth
from gpu_helpers import bits_of, check_bound, device, swiglu_bound, to_dev, to_host

pytestmark = pytest.mark.gpu

TILES = ("128x256", "256x256", "128x512")
XCDS = 8
CLAIMS = 16  # int32 offset of the per-XCD claim counters in the workspace header


def _case(H, I, E, L, layers, sizes_list, seed, fused):
    dev = device()
    rng = np.random.default_rng(seed)
    cfg = synth.Config("case", L=L, H=H, E=E, k=1, I=I, D=1, n=len(layers), T=1, dtype="bf16")
    w13, w2, _, _ = synth.weights_numpy(cfg, seed)
    W13p = cle.pack_weights(to_dev(w13, "bf16", dev))
    W2p = cle.pack_weights(to_dev(w2, "bf16", dev))
    keep, descs, refs = [], [], []
    k = 2
    for j, (l, sizes) in enumerate(zip(layers, sizes_list)):
        rows = int(sum(sizes))
        offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
        t = dict(offsets=torch.from_numpy(offsets).to(dev))
        t["act"] = torch.full((max(rows, 1), I), 7.0, dtype=torch.bfloat16, device=dev)
        t["yp"] = torch.full((max(rows, 1), H), 7.0, dtype=torch.bfloat16, device=dev)
        if fused:
            # rows read in place through a row map, as the engine does
            ntok = -(-max(rows, 1) // k)
            x = synth.store(rng.standard_normal((ntok, H)).astype(np.float32), "bf16")
            src = rng.permutation(ntok * k)[:rows].astype(np.int32)
            xp = x[src // k]
            t["x"], t["src"] = to_dev(x, "bf16", dev), torch.from_numpy(src).to(dev)
            d = cle.make_desc(l, rows, t["offsets"], None, t["act"], t["yp"], x=t["x"],
                              src=t["src"], k=k)
        else:
            xp = synth.store(rng.standard_normal((rows, H)).astype(np.float32), "bf16")
            t["xp"] = to_dev(xp, "bf16", dev)
            d = cle.make_desc(l, rows, t["offsets"], t["xp"], t["act"], t["yp"])
        keep.append(t)
        descs.append(d)
        refs.append((oracle.widen(xp, "bf16"), offsets, l, rows))
    ws = torch.zeros(cle.workspace_bytes(cle.OP_FFN, 0, E, 1, 0, len(descs)) // 4,
                     dtype=torch.int32, device=dev)
    return dict(descs=descs, keep=keep, refs=refs, W=(W13p, W2p), w=(w13, w2), ws=ws)


def _run(case, tile):
    cle.set_expert_tile(tile)
    try:
        for t in case["keep"]:
            # both phases' outputs start as a sentinel, so a tile that a
            # shape's order skips cannot reuse an earlier run's Act rows
            t["act"].fill_(7.0)
            t["yp"].fill_(7.0)
        cle.grouped_expert_ffn(case["descs"], case["W"][0], case["W"][1], case["ws"], packed=True)
        torch.cuda.synchronize()
    finally:
        cle.set_expert_tile("default")
    return [bits_of(t["yp"]) for t in case["keep"]]


def _check_oracle(case, what):
    w13, w2 = case["w"]
    for j, (t, (x, offsets, l, rows)) in enumerate(zip(case["keep"], case["refs"])):
        got = oracle.widen(to_host(t["yp"])[:rows], "bf16")
        for e in range(len(offsets) - 1):
            a, b = int(offsets[e]), int(offsets[e + 1])
            if b == a:
                continue
            we13, we2 = oracle.widen(w13[l, e], "bf16"), oracle.widen(w2[l, e], "bf16")
            ref = oracle.swiglu_expert(x[a:b], we13, we2)
            check_bound(got[a:b], ref, swiglu_bound(x[a:b], we13, we2, "bf16"),
                        what=f"{what} desc {j} layer {l} expert {e} rows {b - a}")


RAGGED = [0, 1, 15, 16, 17, 127, 128, 129, 255, 256, 300, 0, 700, 2, 64, 33]


# (512, 384): three gate/up column tiles on the 256-row tiles, whose groups run
# in blocks of two column tiles, so the last block is one column tile wide
@pytest.mark.parametrize("H,I", [(2048, 768), (512, 256), (1024, 512), (512, 384)])
@pytest.mark.parametrize("fused", [False, True])
def test_tiles_bitwise_equal_and_match_oracle(H, I, fused):
    E = len(RAGGED)
    rng = np.random.default_rng(H + I)
    sizes = [RAGGED, list(rng.permutation(RAGGED)), [5] * E]
    print(f"[tiles] H={H} I={I} fused={fused}", flush=True)
    case = _case(H, I, E, 3, [2, 0, 2], sizes, seed=H + I + fused, fused=fused)
    outs = {tile: _run(case, tile) for tile in TILES}
    for tile in TILES[1:]:
        for j in range(len(sizes)):
            rows = case["refs"][j][3]
            assert np.array_equal(outs[tile][j][:rows], outs[TILES[0]][j][:rows]), (tile, j)
    _check_oracle(case, f"H={H} I={I}")


@pytest.mark.parametrize("tile", TILES)
def test_claimed_tiles_cover_every_tile(tile):
    """Several thousand tiles per phase over one workgroup per CU: each XCD's
    range is longer than its workgroups, so most tiles are claimed."""
    H, I, E = 512, 256, 8
    rng = np.random.default_rng(5)
    sizes_list = []
    for j in range(4):
        p = np.arange(1, E + 1, dtype=np.float64) ** -1.2
        sizes_list.append(list(rng.multinomial(24000, p[rng.permutation(E)] / p.sum())))
    print(f"[claims] tile {tile}", flush=True)
    case = _case(H, I, E, 2, [1, 0, 1, 0], sizes_list, seed=9, fused=True)
    _run(case, tile)
    ws = case["ws"].cpu().numpy()
    for phase in (0, 1):
        total = int(ws[phase])
        per = -(-total // XCDS)
        want = [min(total, x * per + per) - min(total, x * per) for x in range(XCDS)]
        got = ws[CLAIMS + XCDS * phase: CLAIMS + XCDS * (phase + 1)].tolist()
        print(f"[claims] phase {phase + 1}: {total} tiles, claims {got}", flush=True)
        assert total >= 2 * 256, total          # more tiles than workgroups
        assert got == want
    _check_oracle(case, f"claims {tile}")
