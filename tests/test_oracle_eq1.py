"""Pins for the oracle's composition of one MoE layer and of Algorithm 1.

"EasyBalance: Cross-Layer Load Balancing in Distributed MoE Inference",
§2.1, Eq. (1): the MoE output of a token is the gate-weighted sum of the
outputs of its top-k experts, and the layer adds it to the token's state.
Here that sum is evaluated one token at a time, with nothing shared with the
oracle's batched pipeline (route -> dispatch -> permute -> segment FFN ->
combine): the top-k by a brute-force sort, the gates with ``math.exp`` in
slot order, each expert by torch's ``silu`` / ``linear`` on the token's own
row, the block input by torch's ``rms_norm``.  A dropped term, a wrong row
index (``src % k`` or ``src`` for ``src // k``), the experts reading the raw
state instead of the normalised one, or the residual taken from the
normalised rows all fail these checks.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import moe

EPS = 1e-6


def _topk_gates(z_row, k):
    """Brute-force top-k of one float32 logit row, (logit desc, id asc), and
    the softmax over the k chosen logits rounded to float32."""
    zr = [float(np.float32(v)) for v in z_row]
    ids = sorted(range(len(zr)), key=lambda e: (-zr[e], e))[:k]
    ex = [math.exp(zr[e] - zr[ids[0]]) for e in ids]
    tot = 0.0
    for v in ex:
        tot += v
    return ids, [float(np.float32(v / tot)) for v in ex]


def _expert(x_row, w13, w2):
    """One SwiGLU expert on one row, through torch (float64)."""
    I = w2.shape[1]
    xt = torch.from_numpy(np.ascontiguousarray(x_row))[None, :]
    t13 = torch.from_numpy(np.ascontiguousarray(w13))
    act = F.silu(F.linear(xt, t13[:I])) * F.linear(xt, t13[I:])
    return F.linear(act, torch.from_numpy(np.ascontiguousarray(w2)))[0].numpy()


def _block_input(h_row, prenorm):
    if not prenorm:
        return h_row
    ht = torch.from_numpy(np.ascontiguousarray(h_row))
    return F.rms_norm(ht, (ht.shape[0],), eps=EPS).numpy()


def eq1_token(h_row, z_row, k, w13_l, w2_l, w13s_l=None, w2s_l=None, prenorm=False):
    """h_row + MoE(h_row) for one token (Eq. (1) plus the shared experts of
    gate weight 1 and the residual of the layer)."""
    x = _block_input(h_row, prenorm)
    ids, gates = _topk_gates(z_row, k)
    y = np.array(h_row, dtype=np.float64)
    for e, g in zip(ids, gates):
        y = y + g * _expert(x, w13_l[e], w2_l[e])
    if w13s_l is not None:
        for q in range(len(w13s_l)):
            y = y + _expert(x, w13s_l[q], w2s_l[q])
    return y


def _stack(rng, L, E, H, I, ns, std=0.15):
    w13 = rng.normal(0, std, (L, E, 2 * I, H))
    w2 = rng.normal(0, std, (L, E, H, I))
    if ns:
        return w13, w2, rng.normal(0, std, (L, ns, 2 * I, H)), rng.normal(0, std, (L, ns, H, I))
    return w13, w2, None, None


# tiny: the tiny stack's shape; moonlight-small: Moonlight's structure (top-6
# of 16 here, two shared experts) at a small hidden size
SHAPES = {"tiny": dict(T=16, H=64, E=8, k=2, I=128, ns=0),
          "moonlight-small": dict(T=24, H=64, E=16, k=6, I=96, ns=2)}


@pytest.mark.parametrize("prenorm", [False, True])
@pytest.mark.parametrize("shape", list(SHAPES))
def test_moe_layer_is_eq1_token_by_token(shape, prenorm):
    s = SHAPES[shape]
    rng = np.random.default_rng(31 + len(shape) + prenorm)
    T, H, E, k, I, ns = s["T"], s["H"], s["E"], s["k"], s["I"], s["ns"]
    w13, w2, w13s, w2s = _stack(rng, 1, E, H, I, ns)
    # rows far from unit RMS, so that the normalised rows differ from h
    h = rng.standard_normal((T, H)) * rng.uniform(0.2, 4.0, (T, 1))
    z = rng.standard_normal((T, E)).astype(np.float32)
    out = oracle.moe_layer(h, z, k, w13[0], w2[0], None if w13s is None else w13s[0],
                           None if w2s is None else w2s[0], prenorm=prenorm, eps=EPS)
    for t in range(T):
        want = eq1_token(h[t], z[t], k, w13[0], w2[0], None if w13s is None else w13s[0],
                         None if w2s is None else w2s[0], prenorm=prenorm)
        np.testing.assert_allclose(out["y"][t], want, rtol=1e-12, atol=1e-12)
    # the experts' MoE part is far from negligible here (a check that reads
    # the residual alone would not pass)
    assert np.abs(out["y"] - h).max() > 1e-2


def test_permute_rows_hand_example():
    """k = 3: assignment a belongs to token a // 3.  src = [5, 0, 7, 3, 1]
    gives tokens [1, 0, 2, 1, 0] (src % 3 would give [2, 0, 1, 0, 1])."""
    x = np.array([[0.0, 0.5], [10.0, 10.5], [20.0, 20.5]])
    xp = moe.permute_rows(x, np.array([5, 0, 7, 3, 1]), 3)
    assert xp.tolist() == [[10.0, 10.5], [0.0, 0.5], [20.0, 20.5], [10.0, 10.5], [0.0, 0.5]]


@pytest.mark.parametrize("T,k,E", [(9, 3, 5), (16, 2, 8), (7, 6, 16)])
def test_dispatch_and_permute_place_every_assignment(T, k, E):
    """Row dest[t*k + s] of the expert-sorted rows is token t's row and lies in
    expert idx[t, s]'s segment."""
    rng = np.random.default_rng(T * k + E)
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    counts, offsets, dest, src = oracle.dispatch(idx, E)
    x = rng.standard_normal((T, 4))
    xp = moe.permute_rows(x, src, k)
    for t in range(T):
        for s in range(k):
            p = int(dest[t * k + s])
            assert np.array_equal(xp[p], x[t])
            e = int(idx[t, s])
            assert offsets[e] <= p < offsets[e + 1]


def _token_chain(h0_row, layers, z_of_layer, k, w13, w2, w13s, w2s, prenorm):
    y = np.array(h0_row, dtype=np.float64)
    for l in layers:
        y = eq1_token(y, z_of_layer(l, y), k, w13[l], w2[l],
                      None if w13s is None else w13s[l], None if w2s is None else w2s[l],
                      prenorm=prenorm)
    return y


@pytest.mark.parametrize("policy,m", [("cumutil", 2), ("maxutil", 1), ("b0", 1)])
@pytest.mark.parametrize("prenorm", [False, True])
def test_run_engine_is_per_token_chain(policy, m, prenorm):
    """Algorithm 1 with given logits: every token's final state equals the
    token followed through all layers alone (Eq. (1) and the residual per
    layer), whatever the schedule; with shared experts."""
    rng = np.random.default_rng(5 + prenorm)
    n, L, T, H, E, k, I, ns, D = 3, 3, 8, 32, 8, 3, 48, 1, 4
    w13, w2, w13s, w2s = _stack(rng, L, E, H, I, ns)
    h0 = [rng.standard_normal((T, H)) * 2.5 for _ in range(n)]
    logits = rng.standard_normal((n, L, T, E)).astype(np.float32)
    h, trace, acc, u = oracle.run_engine(h0, lambda j, l: logits[j, l], k, D, w13, w2, m,
                                         oracle.POLICIES[policy], w13s, w2s, prenorm=prenorm,
                                         eps=EPS)
    for j in range(n):
        for t in range(T):
            want = _token_chain(h0[j][t], range(L), lambda l, y, j=j, t=t: logits[j, l, t], k,
                                w13, w2, w13s, w2s, prenorm)
            np.testing.assert_allclose(h[j][t], want, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("prenorm", [False, True])
def test_run_engine_with_router_is_per_token_chain(prenorm):
    """Routing from the state through each layer's router, z = x W_g^T + b
    with x the block input: the scores (hence the routing) of a token depend
    on its own row only, so each token followed alone through the layers --
    scoring its own row at every layer -- gives the engine's final state."""
    rng = np.random.default_rng(77 + prenorm)
    n, L, T, H, E, k, I, D = 3, 4, 6, 32, 8, 2, 40, 4
    w13, w2, _, _ = _stack(rng, L, E, H, I, 0)
    wg = rng.normal(0, 1 / math.sqrt(H), (L, E, H))
    bias = rng.normal(0, 1.0, (L, E))
    h0 = [rng.standard_normal((T, H)) * 2.0 for _ in range(n)]
    h, trace, acc, u = oracle.run_engine(h0, None, k, D, w13, w2, 2, oracle.POLICIES["cumutil"],
                                         prenorm=prenorm, eps=EPS, router=(wg, bias))

    def z_tok(l, y):
        x = _block_input(y, prenorm)
        z = np.array([sum(float(a) * float(b) for a, b in zip(x, wg[l, e])) + bias[l, e]
                      for e in range(E)])
        return z.astype(np.float32)

    for j in range(n):
        for t in range(T):
            want = _token_chain(h0[j][t], range(L), z_tok, k, w13, w2, None, None, prenorm)
            np.testing.assert_allclose(h[j][t], want, rtol=1e-11, atol=1e-11)
    # every (micro-batch, layer) ran exactly once, in layer order
    seen = {j: [] for j in range(n)}
    for R, layers in trace:
        for j, l in zip(R, layers):
            seen[j].append(l)
    assert all(seen[j] == list(range(L)) for j in range(n))
