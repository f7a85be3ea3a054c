"""GPU parity of each libcle entry point against the CPU oracle, through the
C ABI, on seeded inputs that span several tiles, ragged tails and the
degenerate cases of the method.

Bars: routing indices, gates, dispatch outputs, workloads and statistics
are bit-exact; expert outputs are within the element-wise rounding-error
bound of the expert FFN (gpu_helpers.swiglu_bound) of the float64 oracle,
and bf16 ones also within max-abs 2e-2 and normwise relative 1e-2 (the
workload's stated tolerance); float32 paths also within 1e-5.
"""
import numpy as np
import pytest
import torch

import cross_layer_expert_amd as cle
import oracle
import synth
from gpu_helpers import (bits_of, check_bound, check_close, device, f32_ulp_diff,
                         swiglu_bound, to_dev, to_host)

pytestmark = pytest.mark.gpu

BF16_MAX_ABS, BF16_REL = 2e-2, 1e-2
F32_TOL = 1e-5


# ---------------------------------------------------------------- route
def _route_case(z, k):
    dev = device()
    T, E = z.shape
    zt = torch.from_numpy(np.ascontiguousarray(z, np.float32)).to(dev)
    idx = torch.full((T, k), -7, dtype=torch.int32, device=dev)
    gate = torch.full((T, k), -1.0, dtype=torch.float32, device=dev)
    cle.route(zt, k, idx, gate)
    torch.cuda.synchronize()
    ridx, rgate = oracle.route(z, k)
    gi, gg = idx.cpu().numpy(), gate.cpu().numpy()
    assert np.array_equal(gi, ridx), f"route indices differ (T={T} E={E} k={k})"
    ulps = f32_ulp_diff(gg, rgate)
    nbad = int((ulps > 0).sum())
    print(f"[route] T={T} E={E} k={k}: gate mismatches {nbad}/{gg.size}, max ulp {ulps.max()}",
          flush=True)
    assert np.array_equal(gg.view(np.int32), rgate.view(np.int32)), "gates differ (bits)"


@pytest.mark.parametrize("name", ["tiny", "qwen3", "moonlight", "taskshift"])
def test_route_configs(name):
    cfg = synth.CONFIGS[name]
    for j, l in [(0, 0), (cfg.n - 1, cfg.L - 1)]:
        _route_case(synth.logits(cfg, 0, j, l), cfg.k)


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (5, 8, 8), (33, 1024, 8), (7, 1000, 7),
                                   (130, 64, 1), (3, 65, 64), (2051, 128, 8)])
def test_route_shapes(T, E, k):
    rng = np.random.default_rng(T * 7 + E)
    _route_case(rng.standard_normal((T, E)).astype(np.float32), k)


def test_route_ties_and_signed_zero():
    rng = np.random.default_rng(11)
    z = (np.round(rng.standard_normal((257, 16)) * 2) / 2).astype(np.float32)
    z[0] = 0.0
    z[1, :8] = -0.0
    z[2] = 1.5
    _route_case(z, 5)


def test_route_empty():
    dev = device()
    z = torch.zeros((0, 8), dtype=torch.float32, device=dev)
    cle.route(z, 2, torch.empty((0, 2), dtype=torch.int32, device=dev),
              torch.empty((0, 2), dtype=torch.float32, device=dev))
    torch.cuda.synchronize()


# ---------------------------------------------------------------- dispatch
def _dispatch_case(idx, E, H, dtype, seed=0):
    dev = device()
    T, k = idx.shape
    A = T * k
    x = synth.store(np.random.default_rng(seed).standard_normal((T, H)).astype(np.float32), dtype)
    xt = to_dev(x, dtype, dev)
    idt = torch.from_numpy(np.ascontiguousarray(idx, np.int32)).to(dev)
    counts = torch.full((E,), -5, dtype=torch.int32, device=dev)
    offsets = torch.full((E + 1,), -5, dtype=torch.int32, device=dev)
    dest = torch.full((max(A, 1),), -5, dtype=torch.int32, device=dev)
    src = torch.full((max(A, 1),), -5, dtype=torch.int32, device=dev)
    xp = torch.full((max(A, 1), H), 3.0, dtype=xt.dtype, device=dev)
    ws = torch.empty(max(64, cle.workspace_bytes(cle.OP_DISPATCH, T, E, k) // 4),
                     dtype=torch.int32, device=dev)
    cle.dispatch(idt, E, xt, counts, offsets, dest, src, xp, ws)
    torch.cuda.synchronize()
    return x, counts.cpu().numpy(), offsets.cpu().numpy(), dest.cpu().numpy()[:A], \
        src.cpu().numpy()[:A], to_host(xp)[:A]


@pytest.mark.parametrize("T,k,E,H,dtype,skew", [
    (16, 2, 8, 64, "f32", 0.0), (2048, 8, 128, 2048, "bf16", 1.1), (1024, 6, 64, 256, "bf16", 1.0),
    (1000, 3, 7, 64, "bf16", 0.0), (333, 8, 1024, 64, "f32", 0.5), (77, 1, 1, 64, "bf16", 0.0),
    (129, 8, 128, 128, "bf16", 3.0), (1, 1, 4, 64, "f32", 0.0), (4097, 4, 16, 64, "bf16", 2.0),
    # up to 4096 chunk-histogram entries (chunks x E) each scatter block does
    # the scan itself; past that a scan launch does it: both sides of the
    # limit for E = 128 and E = 1024, E = 300 (two experts per thread), the
    # long-prefill size and many chunks of few experts
    (4096, 8, 128, 64, "bf16", 1.1), (4500, 8, 128, 64, "bf16", 1.1),
    (512, 8, 1024, 64, "bf16", 0.3), (513, 8, 1024, 64, "bf16", 0.3), (700, 5, 300, 64, "f32", 1.0),
    (16384, 8, 128, 64, "bf16", 1.1), (32769, 1, 5, 64, "f32", 0.0), (3000, 11, 1024, 64, "bf16", 0.3)])
def test_dispatch_matches_oracle(T, k, E, H, dtype, skew):
    rng = np.random.default_rng(T + E)
    # skewed expert ids: Zipf-like weights over a random permutation
    p = np.arange(1, E + 1, dtype=np.float64) ** (-skew)
    p = p[rng.permutation(E)]
    p /= p.sum()
    idx = rng.choice(E, size=(T, k), p=p).astype(np.int32)
    print(f"[dispatch] T={T} k={k} E={E} H={H} {dtype}", flush=True)
    x, counts, offsets, dest, src, xp = _dispatch_case(idx, E, H, dtype)
    rc, ro, rd, rs = oracle.dispatch(idx, E)
    assert np.array_equal(counts, rc) and np.array_equal(offsets, ro)
    assert np.array_equal(dest, rd) and np.array_equal(src, rs)
    assert np.array_equal(xp, oracle.moe.permute_rows(x, rs, k))  # bit copy


def test_dispatch_route_chain_qwen3_shape():
    """route -> dispatch on one (micro-batch, layer) of the Qwen3-shaped workload."""
    cfg = synth.CONFIGS["qwen3"]
    z = synth.logits(cfg, 0, 2, 17)
    ridx, _ = oracle.route(z, cfg.k)
    x, counts, offsets, dest, src, xp = _dispatch_case(ridx, cfg.E, cfg.H, "bf16", seed=3)
    rc, ro, rd, rs = oracle.dispatch(ridx, cfg.E)
    assert np.array_equal(counts, rc) and np.array_equal(dest, rd) and np.array_equal(src, rs)
    assert np.array_equal(xp, x[rs // cfg.k])


# the scan in the scatter blocks, then a scan launch (9 chunks x 600 experts)
@pytest.mark.parametrize("T,E", [(50, 8), (3000, 600)])
def test_dispatch_out_of_range_ids_are_dropped(T, E):
    k, H = 3, 64
    rng = np.random.default_rng(5)
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    bad = [(0, 1), (7, 0), (T - 1, 2), (20, 1)]
    for t, s in bad:
        idx[t, s] = [-1, E, 1 << 30, -100][bad.index((t, s))]
    x, counts, offsets, dest, src, xp = _dispatch_case(idx, E, H, "f32")
    valid = (idx >= 0) & (idx < E)
    flat = idx.reshape(-1)
    keep = np.flatnonzero(valid.reshape(-1))
    # the valid assignments are sorted exactly as the oracle sorts them alone
    rc, ro, rd, rs = oracle.dispatch(flat[keep].reshape(-1, 1), E)
    assert np.array_equal(counts, rc) and np.array_equal(offsets, ro)
    nv = keep.size
    assert np.array_equal(src[:nv], keep[rs]) and np.all(src[nv:] == -1)
    assert np.all(dest[~valid.reshape(-1)] == -1)
    assert np.array_equal(dest[keep], rd)
    assert np.all(xp[nv:] == 0)


def test_dispatch_empty():
    x, counts, offsets, dest, src, xp = _dispatch_case(np.zeros((0, 2), np.int32), 8, 64, "bf16")
    assert np.all(counts == 0) and np.all(offsets == 0)


# ---------------------------------------------------------------- workload stats
@pytest.mark.parametrize("n,E,D", [(3, 8, 4), (4, 128, 8), (8, 64, 8), (64, 128, 128),
                                   (1, 1, 1), (16, 1024, 8)])
def test_workload_stats(n, E, D):
    dev = device()
    rng = np.random.default_rng(n * E + D)
    counts = rng.integers(0, 300, size=(n, E)).astype(np.int32)
    if n > 1:
        counts[1] = 0
    ct = torch.from_numpy(counts).to(dev)
    w = torch.full((n, D), -1, dtype=torch.int32, device=dev)
    acc = torch.zeros(4, dtype=torch.int64, device=dev)
    masks = [0, 1, (1 << n) - 1, int(rng.integers(1, 1 << min(n, 62)))]
    want = [0, 0, 0, 0]
    ref_w = [oracle.group_workload(counts[j], D) for j in range(n)]
    for mask in masks:
        cle.workload_stats(ct, D, mask, w, acc)
        R = cle.ids_of(mask)
        if R:
            a, b, c = oracle.step_stats([ref_w[j] for j in R])
            want = [want[0] + a, want[1] + b, want[2] + c, want[3] + 1]
    torch.cuda.synchronize()
    assert w.cpu().numpy().tolist() == ref_w
    assert acc.cpu().numpy().tolist() == want


def test_workload_stats_worked_example():
    """The eight-device example of Eq. (2): 10, 9, ..., 3 -> 10; u = 52/80."""
    dev = device()
    counts = np.array([[5, 5, 5, 4, 4, 4, 4, 3, 3, 3, 3, 2, 2, 2, 2, 1]], np.int32)
    w = torch.zeros((1, 8), dtype=torch.int32, device=dev)
    acc = torch.zeros(4, dtype=torch.int64, device=dev)
    cle.workload_stats(torch.from_numpy(counts).to(dev), 8, 1, w, acc)
    torch.cuda.synchronize()
    assert w.cpu().numpy().tolist() == [[10, 9, 8, 7, 6, 5, 4, 3]]
    assert acc.cpu().numpy().tolist() == [52, 10, 10, 1]


# ---------------------------------------------------------------- combine
@pytest.mark.parametrize("T,k,E,H,ns,dtype,res", [
    (16, 2, 8, 64, 0, "f32", True), (2048, 8, 128, 2048, 0, "bf16", True),
    (1024, 6, 64, 2048, 2, "bf16", True), (37, 3, 5, 72, 1, "bf16", False),
    (5, 1, 1, 8, 0, "f32", False), (9, 12, 16, 64, 1, "bf16", True),
    (6, 9, 9, 16, 0, "f32", True)])
def test_combine(T, k, E, H, ns, dtype, res):
    dev = device()
    rng = np.random.default_rng(T + H)
    z = rng.standard_normal((T, E)).astype(np.float32)
    idx, gates = oracle.route(z, k)
    _, _, dest, _ = oracle.dispatch(idx, E)
    yp = synth.store(rng.standard_normal((T * k, H)).astype(np.float32), dtype)
    ysh = synth.store(rng.standard_normal((ns, T, H)).astype(np.float32), dtype) if ns else None
    h = synth.store(rng.standard_normal((T, H)).astype(np.float32), dtype)
    ref = oracle.combine(oracle.widen(yp, dtype), dest, gates, k,
                         y_shared=None if ysh is None else list(oracle.widen(ysh, dtype)),
                         residual=oracle.widen(h, dtype) if res else None)
    ht = to_dev(h, dtype, dev)
    out = ht if res else torch.empty_like(ht)      # in place over the residual
    cle.combine(to_dev(yp, dtype, dev), torch.from_numpy(dest).to(dev),
                torch.from_numpy(gates).to(dev), out,
                y_shared=None if ysh is None else to_dev(ysh, dtype, dev),
                residual=ht if res else None)
    torch.cuda.synchronize()
    got = oracle.widen(to_host(out), dtype)
    # float32 accumulation of at most k + ns + 1 terms, then one rounding
    scale = np.abs(ref).max()
    if dtype == "bf16":
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6 * scale * (k + ns + 1))
    else:
        assert np.all(np.abs(got - ref) <= 1e-6 * np.abs(ref) + 1e-6 * scale * (k + ns + 1))


# ---------------------------------------------------------------- grouped expert FFN
def _segment_idx(sizes, k, rng):
    """Expert ids whose per-expert counts are exactly `sizes` (T*k = sum)."""
    ids = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(sizes)])
    rng.shuffle(ids)
    # keep the k slots of a token distinct where possible by a stable re-deal
    return ids.reshape(-1, k)


def _ffn_case(dtype, H, I, E, L, ns, layers, sizes_list, seed=0, T_shared=None):
    dev = device()
    rng = np.random.default_rng(seed)
    cfg = synth.Config("case", L=L, H=H, E=E, k=1, I=I, D=1, n=len(layers), T=1, dtype=dtype,
                       n_shared=ns)
    w13, w2, w13s, w2s = synth.weights_numpy(cfg, seed)
    W13, W2 = to_dev(w13, dtype, dev), to_dev(w2, dtype, dev)
    W13s = to_dev(w13s, dtype, dev) if ns else None
    W2s = to_dev(w2s, dtype, dev) if ns else None
    descs, keep, refs = [], [], []
    for j, (l, sizes) in enumerate(zip(layers, sizes_list)):
        rows = int(sum(sizes))
        offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
        xp = synth.store(rng.standard_normal((rows, H)).astype(np.float32), dtype)
        Ts = T_shared if T_shared is not None else max(rows // 2, 1)
        xs = synth.store(rng.standard_normal((Ts, H)).astype(np.float32), dtype) if ns else None
        t = dict(offsets=torch.from_numpy(offsets).to(dev), xp=to_dev(xp, dtype, dev))
        t["act"] = torch.full((max(rows, 1), I), 7.0, dtype=t["xp"].dtype, device=dev)
        t["yp"] = torch.full((max(rows, 1), H), 7.0, dtype=t["xp"].dtype, device=dev)
        if ns:
            t["xs"] = to_dev(xs, dtype, dev)
            t["acts"] = torch.empty((ns, Ts, I), dtype=t["xp"].dtype, device=dev)
            t["ys"] = torch.empty((ns, Ts, H), dtype=t["xp"].dtype, device=dev)
        keep.append(t)
        descs.append(cle.make_desc(l, rows, t["offsets"], t["xp"], t["act"], t["yp"],
                                   Ts if ns else 0, t.get("xs"), t.get("acts"), t.get("ys")))
        x64 = oracle.widen(xp, dtype)
        w13l, w2l = oracle.widen(w13[l], dtype), oracle.widen(w2[l], dtype)
        ref_y = oracle.expert_ffn(x64, offsets, w13l, w2l)
        bnd_y = np.zeros_like(ref_y)
        for e in range(E):
            a, b = int(offsets[e]), int(offsets[e + 1])
            if b > a:
                bnd_y[a:b] = swiglu_bound(x64[a:b], w13l[e], w2l[e], dtype)
        ref_sh = bnd_sh = None
        if ns:
            xs64 = oracle.widen(xs, dtype)
            pairs = [(oracle.widen(w13s[l, q], dtype), oracle.widen(w2s[l, q], dtype))
                     for q in range(ns)]
            ref_sh = [oracle.swiglu_expert(xs64, a13, a2) for a13, a2 in pairs]
            bnd_sh = [swiglu_bound(xs64, a13, a2, dtype) for a13, a2 in pairs]
        refs.append((ref_y, ref_sh, rows, bnd_y, bnd_sh))
    ws = torch.empty(cle.workspace_bytes(cle.OP_FFN, 0, E, 1, ns, len(descs)) // 4,
                     dtype=torch.int32, device=dev)
    return dict(descs=descs, keep=keep, refs=refs, W=(W13, W2, W13s, W2s), ws=ws, dtype=dtype)


def _run_ffn(case, which=None):
    W13, W2, W13s, W2s = case["W"]
    descs = case["descs"] if which is None else [case["descs"][j] for j in which]
    cle.grouped_expert_ffn(descs, W13, W2, case["ws"], W13s, W2s)
    torch.cuda.synchronize()


def _check_ffn(case):
    dtype = case["dtype"]
    tol = (BF16_MAX_ABS, BF16_REL) if dtype == "bf16" else (F32_TOL, F32_TOL)
    for j, (t, (ref_y, ref_sh, rows, bnd_y, bnd_sh)) in enumerate(zip(case["keep"],
                                                                      case["refs"])):
        got = oracle.widen(to_host(t["yp"])[:rows], dtype)
        check_bound(got, ref_y, bnd_y, what=f"yp[{j}]")
        check_close(got, ref_y, *tol, what=f"yp[{j}]")
        if ref_sh is not None:
            gs = oracle.widen(to_host(t["ys"]), dtype)
            for q, r in enumerate(ref_sh):
                check_bound(gs[q], r, bnd_sh[q], what=f"y_shared[{j},{q}]")
                check_close(gs[q], r, *tol, what=f"y_shared[{j},{q}]")


SIZES_A = [0, 1, 63, 64, 65, 130, 7, 0]           # empty, single row, tile edges, multi-tile
SIZES_B = [200, 0, 0, 0, 0, 0, 0, 3]              # one hot expert
SIZES_C = [16, 16, 16, 16, 16, 16, 16, 16]


@pytest.mark.parametrize("H,I", [(128, 64), (256, 128), (128, 192)])
def test_ffn_bf16_cross_layer(H, I):
    print(f"[ffn] bf16 H={H} I={I}", flush=True)
    case = _ffn_case("bf16", H, I, 8, 3, 0, [2, 0, 1], [SIZES_A, SIZES_B, SIZES_C])
    _run_ffn(case)
    _check_ffn(case)


@pytest.mark.parametrize("H,I", [(256, 384), (512, 640), (768, 128), (1280, 256)])
def test_ffn_bf16_k_loop_tails(H, I):
    """The 8-wavefront tiles at every K-loop tail they can meet: K / 64 =
    4, 8, 12, 20 (gate/up) and 6, 10, 2, 4 (down), i.e. tails of 4, 3 and 2
    steps after zero, one or several whole rounds of three, and the short-K
    path whose prologue re-requests its last stage."""
    print(f"[ffn tails] bf16 H={H} I={I}", flush=True)
    case = _ffn_case("bf16", H, I, 8, 2, 0, [1, 0], [SIZES_A, SIZES_B], seed=11)
    _run_ffn(case)
    _check_ffn(case)


@pytest.mark.parametrize("n_desc,E", [(20, 8), (3, 1024)])
def test_ffn_plan_beyond_one_planner_table(n_desc, E):
    """Plans the one planner workgroup cannot keep in LDS: 20 descriptors (two
    planner launches) and 3 x 1024 segments (more than it holds)."""
    rng = np.random.default_rng(n_desc + E)
    sizes_list = []
    for j in range(n_desc):
        sizes = np.zeros(E, np.int64)
        hot = rng.choice(E, min(E, 6), replace=False)
        sizes[hot] = rng.integers(0, 150, size=hot.size)
        sizes_list.append(list(sizes))
    layers = [int(v) for v in rng.integers(0, 3, size=n_desc)]
    print(f"[ffn plan] n_desc={n_desc} E={E}", flush=True)
    case = _ffn_case("bf16", 128, 64, E, 3, 0, layers, sizes_list, seed=2)
    _run_ffn(case)
    _check_ffn(case)


def test_ffn_bf16_shared_experts():
    case = _ffn_case("bf16", 128, 128, 8, 2, 2, [1, 0], [SIZES_A, SIZES_C], seed=4, T_shared=70)
    _run_ffn(case)
    _check_ffn(case)


def test_ffn_bf16_qwen3_dims():
    """Full H=2048, I=768 reduction lengths on a few hundred rows."""
    sizes = [0] * 32
    rng = np.random.default_rng(8)
    for e in rng.choice(32, 20, replace=False):
        sizes[e] = int(rng.integers(1, 90))
    sizes[5] = 300
    case = _ffn_case("bf16", 2048, 768, 32, 1, 0, [0], [sizes], seed=5)
    _run_ffn(case)
    _check_ffn(case)


def test_ffn_f32_tiny():
    case = _ffn_case("f32", 64, 128, 8, 4, 0, [3, 0, 2], [SIZES_A, SIZES_B, SIZES_C], seed=2)
    _run_ffn(case)
    _check_ffn(case)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ffn_rows_independent_of_launch_mates(dtype):
    """A micro-batch's outputs are bitwise the same alone or in a joint launch."""
    case = _ffn_case(dtype, 128, 128, 8, 3, 0, [2, 0, 1], [SIZES_A, SIZES_B, SIZES_C], seed=6)
    _run_ffn(case)
    joint = [bits_of(t["yp"]) for t in case["keep"]]
    for j in range(3):
        case["keep"][j]["yp"].fill_(0)
        _run_ffn(case, which=[j])
        assert np.array_equal(bits_of(case["keep"][j]["yp"]), joint[j])
    _run_ffn(case, which=[2, 0])
    assert np.array_equal(bits_of(case["keep"][0]["yp"]), joint[0])
    assert np.array_equal(bits_of(case["keep"][2]["yp"]), joint[2])


@pytest.mark.parametrize("dtype,k", [("bf16", 1), ("bf16", 3), ("f32", 2)])
def test_ffn_reads_rows_through_src(dtype, k):
    """Rows read in place through the dispatch permutation (xp = NULL) give the
    same bits as rows read from a materialised xp, and match the oracle."""
    dev = device()
    H, I, E, L = (256, 128, 8, 2) if dtype == "bf16" else (64, 128, 8, 2)
    rng = np.random.default_rng(21 + k)
    sizes = [5, 0, 70, 1, 200, 16, 33, 0]
    rows = sum(sizes)
    ntok = -(-rows // k)
    x = synth.store(rng.standard_normal((ntok, H)).astype(np.float32), dtype)
    src = rng.permutation(ntok * k)[:rows].astype(np.int32)   # any assignment ids
    xp = x[src // k]
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    cfg = synth.Config("case", L=L, H=H, E=E, k=1, I=I, D=1, n=1, T=1, dtype=dtype)
    w13, w2, _, _ = synth.weights_numpy(cfg, 3)
    W13, W2 = to_dev(w13, dtype, dev), to_dev(w2, dtype, dev)
    t_off = torch.from_numpy(offsets).to(dev)
    outs = []
    for fused in (False, True):
        act = torch.zeros((rows, I), dtype=W13.dtype, device=dev)
        yp = torch.zeros((rows, H), dtype=W13.dtype, device=dev)
        if fused:
            # the descriptor holds raw addresses: keep its tensors alive
            xt, st = to_dev(x, dtype, dev), torch.from_numpy(src).to(dev)
            d = cle.make_desc(1, rows, t_off, None, act, yp, x=xt, src=st, k=k)
            keep = (xt, st)
        else:
            xpt = to_dev(xp, dtype, dev)
            d = cle.make_desc(1, rows, t_off, xpt, act, yp)
            keep = (xpt, )
        ws = torch.empty(cle.workspace_bytes(cle.OP_FFN, 0, E, 1, 0, 1) // 4, dtype=torch.int32,
                         device=dev)
        cle.grouped_expert_ffn([d], W13, W2, ws)
        torch.cuda.synchronize()
        outs.append(bits_of(yp))
        del keep
    assert np.array_equal(outs[0], outs[1])
    x64, w13l, w2l = (oracle.widen(a, dtype) for a in (xp, w13[1], w2[1]))
    ref = oracle.expert_ffn(x64, offsets, w13l, w2l)
    got = oracle.widen(outs[1].view(np.uint16) if dtype == "bf16" else outs[1].view(np.float32),
                       dtype)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            check_bound(got[a:b], ref[a:b], swiglu_bound(x64[a:b], w13l[e], w2l[e], dtype),
                        what=f"fused {dtype} k={k} e={e}")
    tol = (BF16_MAX_ABS, BF16_REL) if dtype == "bf16" else (F32_TOL, F32_TOL)
    check_close(got, ref, *tol, what=f"fused {dtype} k={k}")
