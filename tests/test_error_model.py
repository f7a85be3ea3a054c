"""The element-wise error bound the GPU parity tests use for expert outputs
(tests/gpu_helpers.py: swiglu_bound) against an emulation of the GPU
arithmetic on the CPU: products of bf16 values summed in float32, Act
rounded to bf16, the output rounded to bf16.  The emulation must stay well
inside the bound, and the bound must be tight enough that one wrong row, two
swapped rows or a 5 % error on one row fail it (the absolute 2e-2 bar of the
workload's tolerance misses all three on small outputs)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import swiglu_bound


def _bf(a):
    return synth.bf16_to_f32(synth.bf16_bits(np.asarray(a, np.float32))).astype(np.float64)


def _emulated_gpu(x, w13, w2):
    I = w2.shape[1]
    f32 = np.float32
    g = (x.astype(f32) @ w13[:I].T.astype(f32)).astype(np.float64)
    u = (x.astype(f32) @ w13[I:].T.astype(f32)).astype(np.float64)
    act = _bf(g / (1.0 + np.exp(-g)) * u)
    return _bf(act.astype(f32) @ w2.T.astype(f32))


@pytest.mark.parametrize("H,I,rows", [(2048, 768, 150), (128, 64, 200), (512, 256, 90)])
def test_bound_holds_and_is_tight(H, I, rows):
    rng = np.random.default_rng(H + I)
    x = _bf(rng.standard_normal((rows, H)))
    w13 = _bf(rng.normal(0, 0.02, (2 * I, H)))
    w2 = _bf(rng.normal(0, 0.02, (H, I)))
    ref = oracle.swiglu_expert(x, w13, w2)
    got = _emulated_gpu(x, w13, w2)
    b = swiglu_bound(x, w13, w2, "bf16")
    ratio = np.abs(got - ref) / b
    assert ratio.max() < 0.5, ratio.max()
    bad = got.copy()
    bad[[0, 1]] = bad[[1, 0]]
    assert (np.abs(bad - ref) / b).max() > 1.0
    bad = got.copy()
    bad[3] *= 1.05
    assert (np.abs(bad - ref) / b).max() > 1.0
    bad = got.copy()
    bad[7] = _emulated_gpu(x[8:9], w13, w2)[0]
    assert (np.abs(bad - ref) / b).max() > 1.0


def test_float32_bound_holds():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((40, 64)).astype(np.float32).astype(np.float64)
    w13 = rng.normal(0, 0.02, (256, 64)).astype(np.float32).astype(np.float64)
    w2 = rng.normal(0, 0.02, (64, 128)).astype(np.float32).astype(np.float64)
    ref = oracle.swiglu_expert(x, w13, w2)
    f32 = np.float32
    g = x.astype(f32) @ w13[:128].T.astype(f32)
    u = x.astype(f32) @ w13[128:].T.astype(f32)
    act = (g / (f32(1) + np.exp(-g)) * u).astype(f32)
    got = (act @ w2.T.astype(f32)).astype(np.float64)
    b = swiglu_bound(x, w13, w2, "f32")
    assert (np.abs(got - ref) / b).max() < 0.5
