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
