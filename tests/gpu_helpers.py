"""Shared plumbing for the GPU tests: moving seeded inputs to the device and
results back.  No arithmetic of the method lives here."""
import numpy as np
import pytest
import torch


def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU (torch.cuda.is_available() is False)")
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, dtype: str, dev):
    """Storage array (float32, or uint16 bf16 bit patterns) -> device tensor."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def to_host(t) -> np.ndarray:
    """Device tensor -> storage array (bf16 as uint16 bit patterns)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bits_of(t) -> np.ndarray:
    """Raw bit patterns of a device tensor, for bitwise comparisons."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy()
    return t.numpy()


def check_close(got, ref, max_abs, rel_norm, what=""):
    """Elementwise max-abs and normwise relative error ||got-ref|| / ||ref||."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0, 0.0
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    d = np.abs(got - ref)
    ma = float(d.max())
    nr = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    print(f"[check] {what}: max_abs={ma:.3e} rel_norm={nr:.3e}", flush=True)
    assert ma <= max_abs, f"{what}: max abs error {ma} > {max_abs}"
    assert nr <= rel_norm, f"{what}: relative error {nr} > {rel_norm}"
    return ma, nr


def f32_ulp_diff(a, b) -> np.ndarray:
    """|a - b| in units in the last place of float32 (same-sign finite values)."""
    ia = np.asarray(a, dtype=np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, dtype=np.float32).view(np.int32).astype(np.int64)
    return np.abs(ia - ib)


# ---------------------------------------------------------------- element-wise error bounds
# Rounding-error model of the GPU expert FFN against the float64 oracle.  The
# GPU takes products of the stored operand values exactly, sums them in
# float32, rounds Act to the storage type (bf16: unit roundoff 2^-8) and the
# output once more.  Rounding errors are treated as independent, zero-mean
# and bounded, so a sum of n rounding errors e_i * a_i is below
# lam * u * ||a||_2 except with probability 2 exp(-lam^2 / 2) (Hoeffding's
# inequality; the probabilistic error analysis of Higham and Mary, 2019).
# With lam = 8 that probability is 2.5e-14 per element.  Deterministic parts
# (the error Act carries into the second product) are bounded by
# Cauchy-Schwarz.
LAM = 8.0
U32 = 2.0 ** -24


def storage_u(dtype):
    return 2.0 ** -8 if dtype == "bf16" else U32


def swiglu_bound(x, w13, w2, dtype):
    """Element-wise bound on |GPU - float64 SwiGLU expert| for rows x (float64
    [r, H]) and one expert's weights (float64 w13 [2I, H], w2 [H, I])."""
    I = w2.shape[1]
    H = x.shape[1]
    us = storage_u(dtype)
    # the bound itself is evaluated in float32 (it needs no more precision)
    x, w13, w2 = (np.asarray(a, dtype=np.float32) for a in (x, w13, w2))
    wg, wu = w13[:I], w13[I:]
    g = x @ wg.T
    u = x @ wu.T
    nx = np.linalg.norm(x, axis=1, keepdims=True)
    eg = LAM * np.sqrt(H) * U32 * nx * np.linalg.norm(wg, axis=1)[None, :]
    eu = LAM * np.sqrt(H) * U32 * nx * np.linalg.norm(wu, axis=1)[None, :]
    with np.errstate(over="ignore"):
        s = g / (1.0 + np.exp(-g))
    act = s * u
    dact = 1.1 * np.abs(u) * eg + np.abs(s) * eu + 4 * U32 * np.abs(act)
    y = act @ w2.T
    nw2 = np.linalg.norm(w2, axis=1)[None, :]
    t1 = (act * act) @ (w2 * w2).T
    b = (us * np.abs(y) + LAM * us * np.sqrt(t1)
         + LAM * np.sqrt(I) * U32 * np.linalg.norm(act, axis=1, keepdims=True) * nw2
         + np.linalg.norm(dact, axis=1, keepdims=True) * nw2)
    return b.astype(np.float64) * (1.0 + 1e-5) + 1e-30


def check_bound(got, ref, bound, what="", quiet=False):
    """|got - ref| <= bound element by element (and finite); prints (unless
    quiet) and returns the largest ratio of error to bound."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    r = np.abs(got - ref) / bound
    worst = float(r.max())
    i = np.unravel_index(int(r.argmax()), r.shape)
    if not quiet:
        print(f"[bound] {what}: max |err|/bound = {worst:.3f} (err {abs(got[i] - ref[i]):.3e}, "
              f"ref {ref[i]:.3e})", flush=True)
    assert worst <= 1.0, f"{what}: error {abs(got[i] - ref[i])} above bound {bound[i]} at {i}"
    return worst
