"""Oracle: routing, dispatch, expert FFN and combine (one MoE layer).

Pins (tests/test_oracle_moe.py):
* route      -- brute force on every row (Python ``sorted`` with an explicit
                key), planted exact ties, k = E reducing to scipy's softmax,
                gates summing to 1, shift invariance.
* dispatch   -- numpy's stable argsort (a library counting-sort equivalent),
                permutation / monotonicity invariants.
* swiglu     -- a 1x1 closed form (silu(ln 3) = 0.75 ln 3), torch's
                ``F.silu``/``F.linear`` on non-square shapes, zero weights.
* expert_ffn -- one expert holding every token equals the dense SwiGLU MLP.
* combine    -- Yp = Xp gives Y = X * sum(gates); a hand-worked example;
                shared-expert and residual terms.
* rmsnorm    -- a hand-worked row ([3, 4]); constant rows give +-1; outputs
                have unit mean square; positive scaling leaves them unchanged.
* gate_logits -- one-hot router rows pick hidden columns (closed form); zero
                weights leave the bias; relabelling experts permutes columns.
"""
from __future__ import annotations

import numpy as np


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> float64 values.  bf16 arrays arrive as uint16 bit
    patterns; their float32 value is the pattern shifted into the high half."""
    if dtype == "bf16":
        u32 = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u32.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def rmsnorm(h: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """The MoE block's normalised input rows: h / sqrt(mean(h^2) + eps).

    [PAPER] §2.1 writes the layer as h_{l+1} = h'_l + MLP(h'_l); reading: the
    experts and the router read the RMS-normalised rows of h'_l (unit weight,
    as in pre-norm transformer blocks) while the residual keeps h'_l."""
    h = np.asarray(h, dtype=np.float64)
    return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)


def gate_logits(h: np.ndarray, w_gate: np.ndarray, bias=None) -> np.ndarray:
    """Router scores of the tokens h [T, H] (float64): z = h W_g^T + b, [T, E].

    [PAPER] §2.1: top-k selects from G(h'_l); G is taken as a linear router
    with weights W_g [E, H] (row e scores expert e) and an optional fixed
    per-expert offset b [E] (the synthetic skew; reading R2's bias).
    Evaluated in float64 on the exact values of the stored weights."""
    z = np.asarray(h, dtype=np.float64) @ np.asarray(w_gate, dtype=np.float64).T
    if bias is not None:
        z = z + np.asarray(bias, dtype=np.float64)[None, :]
    return z


def route(logits: np.ndarray, k: int):
    """Router top-k with renormalised softmax gates.

    [PAPER] §2.1: ``W_l, I_l = topk(G(h'_l))``.  G is not defined on the
    pages; the logits are given.  Readings taken here:
      * selection is on the logits, ordered by (logit descending, expert id
        ascending) -- slot s holds the s-th expert in that order;
      * gates are the softmax restricted to the k selected logits,
        g_s = exp(z_s - z_0) / sum_r exp(z_r - z_0), evaluated in float64 with
        the sum taken in slot order, then rounded once to float32.
    Logits must be finite.

    Returns (idx int32 [T, k], gates float32 [T, k]).
    """
    z = np.asarray(logits, dtype=np.float32).astype(np.float64)
    T, E = z.shape
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    # stable sort of -z: equal logits keep ascending expert id
    order = np.argsort(-z, axis=1, kind="stable")[:, :k]
    zs = np.take_along_axis(z, order, axis=1)
    ex = np.exp(zs - zs[:, :1])
    total = np.zeros(T, dtype=np.float64)
    for s in range(k):                      # slot order
        total = total + ex[:, s]
    gates = (ex / total[:, None]).astype(np.float32)
    return order.astype(np.int32), gates


def dispatch(idx: np.ndarray, E: int):
    """Per-expert histogram, exclusive prefix sum and stable permutation.

    [PAPER] §2.2: tokens are sent to the devices of their experts (the
    all-to-all dispatch); here the destination is a buffer grouped by expert.
    [EP-ATLAS] §1: T_e = number of tokens routed to expert e.

    Assignment a = t*k + s (token t, slot s) goes to row
        dest[a] = offsets[e] + #{a' < a : idx[a'] = e},  e = idx[a],
    i.e. a stable counting sort; src is the inverse permutation.

    Returns (counts int32 [E], offsets int32 [E+1], dest int32 [A],
    src int32 [A]).
    """
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    A = flat.size
    counts = np.zeros(E, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    nxt = offsets[:E].copy()
    dest = np.empty(A, dtype=np.int64)
    for a in range(A):
        e = flat[a]
        dest[a] = nxt[e]
        nxt[e] += 1
    src = np.empty(A, dtype=np.int64)
    src[dest] = np.arange(A)
    return (counts.astype(np.int32), offsets.astype(np.int32),
            dest.astype(np.int32), src.astype(np.int32))


def permute_rows(x: np.ndarray, src: np.ndarray, k: int) -> np.ndarray:
    """Xp[p] = X[src[p] // k]: the row of the token behind assignment src[p]."""
    return np.asarray(x)[np.asarray(src, dtype=np.int64) // k]


def _silu(x: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def swiglu_expert(x: np.ndarray, w13: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """One SwiGLU expert on rows x (float64).

    The expert form is not on the pages (they write expert_i abstractly,
    [PAPER] Eq. (1)); the workload names SwiGLU with intermediate I:
        G = x W_gate^T, U = x W_up^T, y = (silu(G) * U) W_down^T,
    silu(v) = v / (1 + e^-v), no biases.  w13 is [2I, H] with the gate rows
    first, w2 is [H, I].
    """
    I = w2.shape[1]
    g = x @ w13[:I].T
    u = x @ w13[I:].T
    return (_silu(g) * u) @ w2.T


def expert_ffn(xp: np.ndarray, offsets: np.ndarray, w13_layer: np.ndarray,
               w2_layer: np.ndarray) -> np.ndarray:
    """Apply each expert e to its segment xp[offsets[e]:offsets[e+1]].

    xp, w13_layer [E, 2I, H], w2_layer [E, H, I] are float64.  Rows past
    offsets[E] (none when every id is valid) stay zero.
    """
    yp = np.zeros((xp.shape[0], w2_layer.shape[1]), dtype=np.float64)
    E = w13_layer.shape[0]
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            yp[a:b] = swiglu_expert(xp[a:b], w13_layer[e], w2_layer[e])
    return yp


def combine(yp: np.ndarray, dest: np.ndarray, gates: np.ndarray, k: int,
            y_shared=None, residual=None) -> np.ndarray:
    """Gate-weighted sum of the expert outputs of each token.

    [PAPER] Eq. (1): MLP(h'_l) = sum_{i in I_l} W_{l,i} * expert_i(h'_l).
    Slot order, then shared experts (gate 1) in index order, then the
    residual h'_l ([PAPER] §2.1: h_{l+1} = h'_l + MLP(h'_l)).  float64.
    """
    gates = np.asarray(gates, dtype=np.float32).astype(np.float64)
    T = gates.shape[0]
    dest = np.asarray(dest, dtype=np.int64).reshape(T, k)
    y = np.zeros((T, yp.shape[1]), dtype=np.float64)
    for s in range(k):
        y = y + gates[:, s:s + 1] * yp[dest[:, s]]
    if y_shared is not None:
        for ysh in y_shared:
            y = y + ysh
    if residual is not None:
        y = y + residual
    return y
