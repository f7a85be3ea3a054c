"""Pins for the oracle's routing, dispatch, expert FFN and combine.

Each check compares the oracle with something other than itself: a brute
force, a library routine, a closed form or an invariant fixed by the
definition on the pages.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import moe


def _rand_logits(rng, T, E, ties=False):
    z = rng.standard_normal((T, E)).astype(np.float32)
    if ties:
        # quantise so that exact ties are common
        z = (np.round(z * 2) / 2).astype(np.float32)
    return z


@pytest.mark.parametrize("T,E,k,ties", [(7, 8, 2, False), (9, 8, 2, True), (5, 16, 5, True),
                                        (6, 128, 8, False), (4, 64, 6, True), (3, 1, 1, False)])
def test_route_matches_brute_force(T, E, k, ties):
    rng = np.random.default_rng(T * 100 + E)
    z = _rand_logits(rng, T, E, ties)
    idx, gates = oracle.route(z, k)
    for t in range(T):
        # brute force: full sort with an explicit key (value desc, id asc)
        ids = sorted(range(E), key=lambda e: (-float(z[t, e]), e))[:k]
        assert list(idx[t]) == ids
        zs = [float(z[t, e]) for e in ids]
        ex = [math.exp(v - zs[0]) for v in zs]
        tot = 0.0
        for v in ex:
            tot += v
        want = np.array([v / tot for v in ex], dtype=np.float32)
        np.testing.assert_array_equal(gates[t], want)


def test_route_planted_ties_prefer_low_id():
    z = np.zeros((2, 6), np.float32)
    z[0] = [1, 3, 3, 0, 3, -1]
    z[1] = [0, 0, 0, 0, 0, 0]
    idx, gates = oracle.route(z, 3)
    assert idx[0].tolist() == [1, 2, 4]
    assert idx[1].tolist() == [0, 1, 2]
    np.testing.assert_array_equal(gates[1], np.float32(1 / 3))
    # -0.0 and +0.0 are equal logits: lower id first
    z2 = np.array([[-0.0, 0.0, -1.0]], np.float32)
    assert oracle.route(z2, 2)[0][0].tolist() == [0, 1]


def test_route_full_k_is_softmax():
    rng = np.random.default_rng(3)
    z = _rand_logits(rng, 11, 8)
    idx, gates = oracle.route(z, 8)
    ref = scipy.special.softmax(z.astype(np.float64), axis=1)
    got = np.zeros_like(ref)
    np.put_along_axis(got, idx.astype(np.int64), gates.astype(np.float64), axis=1)
    np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-7)


def test_route_gates_sum_to_one_and_shift_invariant():
    rng = np.random.default_rng(4)
    z = _rand_logits(rng, 50, 32)
    idx, gates = oracle.route(z, 6)
    s = gates.astype(np.float64).sum(axis=1)
    assert np.all(np.abs(s - 1.0) <= 6 * np.finfo(np.float32).eps)
    assert np.all(np.diff(gates, axis=1) <= 0)          # slot order = descending gate
    idx2, gates2 = oracle.route(z + np.float32(0.5), 6)  # exact shift on these values
    assert np.array_equal(idx, idx2)
    np.testing.assert_allclose(gates, gates2, rtol=2e-7)


@pytest.mark.parametrize("T,k,E", [(16, 2, 8), (33, 3, 5), (100, 8, 128), (1, 1, 1)])
def test_dispatch_is_stable_argsort(T, k, E):
    rng = np.random.default_rng(T + E)
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    counts, offsets, dest, src = oracle.dispatch(idx, E)
    flat = idx.reshape(-1)
    ref_src = np.argsort(flat, kind="stable")
    assert np.array_equal(src, ref_src)
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and offsets[-1] == T * k
    assert np.all(np.diff(offsets) == counts)
    assert np.array_equal(dest[src], np.arange(T * k))
    # rows of each segment are the experts' own, in increasing assignment order
    for e in range(E):
        seg = src[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)


def test_swiglu_closed_form():
    # H = I = 1: y = w2 * silu(wg x) * (wu x); with wg x = ln 3, silu = 0.75 ln 3
    x = np.array([[2.0]])
    wg, wu, w2 = math.log(3) / 2.0, -1.5, 0.25
    w13 = np.array([[wg], [wu]])
    y = moe.swiglu_expert(x, w13, np.array([[w2]]))
    assert y.shape == (1, 1)
    assert abs(y[0, 0] - w2 * 0.75 * math.log(3) * (wu * 2.0)) < 1e-15


def test_swiglu_matches_torch_nonsquare():
    rng = np.random.default_rng(5)
    c, H, I = 7, 12, 5
    x = rng.standard_normal((c, H))
    w13 = rng.standard_normal((2 * I, H))
    w2 = rng.standard_normal((H, I))
    got = moe.swiglu_expert(x, w13, w2)
    tx, t13, t2 = (torch.from_numpy(a) for a in (x, w13, w2))
    ref = torch.nn.functional.linear(
        torch.nn.functional.silu(torch.nn.functional.linear(tx, t13[:I])) *
        torch.nn.functional.linear(tx, t13[I:]), t2).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    assert np.all(moe.swiglu_expert(x, np.zeros_like(w13), w2) == 0)


def test_expert_ffn_single_expert_is_dense_mlp():
    rng = np.random.default_rng(6)
    T, k, E, H, I = 10, 1, 4, 8, 6
    idx = np.full((T, k), 2, np.int32)
    counts, offsets, dest, src = oracle.dispatch(idx, E)
    x = rng.standard_normal((T, H))
    w13 = rng.standard_normal((E, 2 * I, H))
    w2 = rng.standard_normal((E, H, I))
    yp = oracle.expert_ffn(x[src // k], offsets, w13, w2)
    tx = torch.from_numpy(x)
    dense = torch.nn.functional.linear(
        torch.nn.functional.silu(tx @ torch.from_numpy(w13[2, :I]).T) *
        (tx @ torch.from_numpy(w13[2, I:]).T), torch.from_numpy(w2[2])).numpy()
    np.testing.assert_allclose(yp, dense, rtol=1e-12, atol=1e-12)


def test_combine_identity_experts_and_hand_example():
    rng = np.random.default_rng(7)
    T, k, E, H = 12, 3, 6, 5
    z = _rand_logits(rng, T, E)
    idx, gates = oracle.route(z, k)
    counts, offsets, dest, src = oracle.dispatch(idx, E)
    x = rng.standard_normal((T, H))
    xp = x[src // k]
    # experts that return their input: Y = X * sum(gates) ~= X
    y = oracle.combine(xp, dest, gates, k)
    np.testing.assert_allclose(y, x * gates.astype(np.float64).sum(1, keepdims=True), rtol=1e-15)
    np.testing.assert_allclose(y, x, rtol=1e-6, atol=1e-6)
    # hand example: one token, two slots, a shared expert and a residual
    yp = np.array([[1.0, 2.0], [10.0, 20.0]])
    out = oracle.combine(yp, np.array([1, 0]), np.array([[0.75, 0.25]], np.float32), 2,
                         y_shared=[np.array([[100.0, 200.0]])], residual=np.array([[5.0, 6.0]]))
    assert out.tolist() == [[0.75 * 10 + 0.25 * 1 + 100 + 5, 0.75 * 20 + 0.25 * 2 + 200 + 6]]


def test_widen_bf16_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F80], np.uint16)
    v = oracle.widen(bits, "bf16")
    assert v[0] == 1.0 and v[1] == -1.0 and v[2] == 3.140625 and v[3] == 0.0
    assert math.copysign(1.0, v[4]) == -1.0 and math.isinf(v[5])


def test_gate_logits_special_cases():
    """Router scores: one-hot router rows pick hidden columns plus the bias
    (a closed form); zero weights leave only the bias, so routing follows
    the bias ranking; relabelling the experts permutes the score columns."""
    rng = np.random.default_rng(4)
    T, H, E = 7, 12, 5
    h = rng.standard_normal((T, H))
    cols = [3, 0, 11, 3, 7]
    w = np.zeros((E, H))
    for e, c in enumerate(cols):
        w[e, c] = 1.0
    b = np.array([0.5, -1.0, 0.0, 2.0, 0.25])
    z = oracle.gate_logits(h, w, b)
    for t in range(T):
        for e, c in enumerate(cols):
            assert z[t, e] == h[t, c] + b[e]
    z0 = oracle.gate_logits(h, np.zeros((E, H)), b)
    assert np.array_equal(z0, np.broadcast_to(b, (T, E)))
    idx, _ = oracle.route(z0.astype(np.float32), 2)
    assert (idx == [3, 0]).all()                     # the two largest biases, every token
    wr = rng.standard_normal((E, H))
    perm = rng.permutation(E)
    assert np.allclose(oracle.gate_logits(h, wr[perm], b[perm]),
                       oracle.gate_logits(h, wr, b)[:, perm], rtol=0, atol=1e-12)
    assert oracle.gate_logits(h, w).shape == (T, E)   # no bias


def test_rmsnorm_closed_forms():
    """[3, 4] has mean square 12.5, so it maps to [3, 4] / sqrt(12.5); a
    constant row maps to +-1 (eps = 0); outputs have unit mean square and do
    not change when the row is scaled by a positive factor."""
    y = oracle.rmsnorm(np.array([[3.0, 4.0]]), eps=0.0)
    assert np.allclose(y, [[3 / math.sqrt(12.5), 4 / math.sqrt(12.5)]], rtol=0, atol=1e-15)
    assert np.array_equal(oracle.rmsnorm(np.full((2, 6), -2.5), eps=0.0), -np.ones((2, 6)))
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 64)) * rng.uniform(0.1, 10, (5, 1))
    y = oracle.rmsnorm(x, eps=0.0)
    assert np.allclose(np.mean(y * y, axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.allclose(oracle.rmsnorm(7.5 * x, eps=0.0), y, rtol=0, atol=1e-12)
    # eps damps only rows of tiny scale
    assert np.allclose(oracle.rmsnorm(x, eps=1e-6), y, rtol=1e-5, atol=0)
