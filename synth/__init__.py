"""Seeded synthetic inputs for the cross-layer MoE step.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no routing, no sorting, no expert math, no statistics).
Both the CPU oracle checks and the GPU path receive the same arrays from here,
so neither side generates the other's inputs.

Workload recipe (stand-in for the LongBench-driven routing of the paper, whose
data and trained weights are not available):

* hidden states  ~ N(0, 1), rounded once to the path's storage type;
* router logits  = N(0, 1) + a per-layer expert bias;
  - "normal" bias: N(0, std) per (layer, expert);
  - "zipf" bias: b[e] = -s * ln(rank(e)), rank = 1 + position of e in a
    per-layer uniform permutation, so softmax(b) is exactly Zipf(s) over the
    experts;
* weights        ~ N(0, 0.02) (second parameter read as the standard
  deviation), rounded once to the storage type.

Every tensor family comes from its own numpy ``SeedSequence`` child keyed by
(family, micro-batch, layer), so any single (micro-batch, layer) slice can be
regenerated alone.  Large weight stacks are drawn on the GPU with a seeded
``torch.Generator`` (see ``weights_torch``), and copied back slice by slice when
a check needs them.
"""
from __future__ import annotations

import dataclasses
import numpy as np

# family tags for SeedSequence spawn keys
_FAM_PERM = 1
_FAM_LOGIT = 2
_FAM_HIDDEN = 3
_FAM_WEIGHT = 4
_FAM_BIAS = 5
_FAM_GATE = 6


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    L: int            # MoE layers
    H: int            # hidden size
    E: int            # routed experts per layer
    k: int            # experts per token
    I: int            # SwiGLU intermediate size
    D: int            # logical expert groups (devices in the expert-parallel reading)
    n: int            # micro-batches
    T: int            # tokens per micro-batch
    dtype: str        # "bf16" or "f32"
    bias: str = "zipf"          # "zipf" or "normal"
    zipf_s: float = 1.1
    bias_std: float = 2.0
    n_shared: int = 0           # always-on shared experts per layer
    profiles: int = 1           # distinct per-layer hot-expert permutations
    start_layers: tuple = ()    # staggered starting layers (empty = all at 0)
    m: int = 1                  # minimum RunSet size

    @property
    def A(self) -> int:
        """Routed (token, expert) assignments per micro-batch."""
        return self.T * self.k

    def profile_of(self, j: int) -> int:
        return j % self.profiles


def _m_default(n: int) -> int:
    return max(1, (3 * n) // 4)


CONFIGS = {
    "tiny": Config("tiny", L=4, H=64, E=8, k=2, I=128, D=4, n=3, T=16, dtype="f32",
                   bias="normal", bias_std=2.0, m=2),
    "qwen3": Config("qwen3", L=48, H=2048, E=128, k=8, I=768, D=8, n=4, T=2048, dtype="bf16",
                    bias="zipf", zipf_s=1.1, m=_m_default(4)),
    "moonlight": Config("moonlight", L=26, H=2048, E=64, k=6, I=1408, D=8, n=8, T=1024,
                        dtype="bf16", bias="zipf", zipf_s=1.0, n_shared=2, m=_m_default(8)),
    "taskshift": Config("taskshift", L=48, H=2048, E=128, k=8, I=768, D=8, n=6, T=2048,
                        dtype="bf16", bias="zipf", zipf_s=1.3, profiles=3, m=_m_default(6)),
    "decode": Config("decode", L=48, H=2048, E=128, k=8, I=768, D=8, n=16, T=64, dtype="bf16",
                     bias="zipf", zipf_s=1.1, start_layers=tuple(3 * j for j in range(16)),
                     m=_m_default(16)),
    "prefill": Config("prefill", L=48, H=2048, E=128, k=8, I=768, D=8, n=2, T=16384,
                      dtype="bf16", bias="zipf", zipf_s=1.1, m=1),
}


def small(cfg: Config, **over) -> Config:
    """A copy of ``cfg`` with some fields replaced (for reduced test sizes)."""
    return dataclasses.replace(cfg, **over)


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=tuple(key)))


# ---------------------------------------------------------------- bf16 storage
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return the
    16-bit patterns as uint16.  Storage conversion only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    r = np.where(nan, 0x7FC0, r)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def store(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 array -> storage array (float32, or uint16 bf16 bit patterns)."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits(x)
    raise ValueError(dtype)


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """storage array -> exact float32 values."""
    return bf16_to_f32(a) if dtype == "bf16" else np.asarray(a, dtype=np.float32)


# ---------------------------------------------------------------- router inputs
def expert_bias(cfg: Config, seed: int, profile: int, layer: int) -> np.ndarray:
    """Per-layer expert bias added to the router logits, float64 [E]."""
    if cfg.bias == "normal":
        return _rng(seed, _FAM_BIAS, profile, layer).normal(0.0, cfg.bias_std, cfg.E)
    perm = _rng(seed, _FAM_PERM, profile, layer).permutation(cfg.E)
    rank = np.empty(cfg.E, dtype=np.float64)
    rank[perm] = np.arange(1, cfg.E + 1, dtype=np.float64)
    return -cfg.zipf_s * np.log(rank)


def logits(cfg: Config, seed: int, j: int, layer: int, T: int | None = None) -> np.ndarray:
    """Router logits of micro-batch ``j`` at ``layer``: float32 [T, E]."""
    T = cfg.T if T is None else T
    z = _rng(seed, _FAM_LOGIT, j, layer).standard_normal((T, cfg.E))
    z = z + expert_bias(cfg, seed, cfg.profile_of(j), layer)[None, :]
    return z.astype(np.float32)


def hidden(cfg: Config, seed: int, j: int, T: int | None = None, tag: int = 0) -> np.ndarray:
    """Hidden state of micro-batch ``j`` in storage form [T, H]."""
    T = cfg.T if T is None else T
    x = _rng(seed, _FAM_HIDDEN, j, tag).standard_normal((T, cfg.H), dtype=np.float32)
    return store(x, cfg.dtype)


# ---------------------------------------------------------------- expert weights
def weights_numpy(cfg: Config, seed: int, layers: int | None = None):
    """Expert weights in storage form, drawn on the CPU (small configs only).

    Returns (w13 [L, E, 2I, H], w2 [L, E, H, I], w13_sh [L, S, 2I, H] | None,
    w2_sh [L, S, H, I] | None).  Rows [0, I) of a w13 slice are the gate
    projection and rows [I, 2I) the up projection.
    """
    L = cfg.L if layers is None else layers
    r = _rng(seed, _FAM_WEIGHT, 0, 0)
    w13 = store(r.normal(0.0, 0.02, (L, cfg.E, 2 * cfg.I, cfg.H)).astype(np.float32), cfg.dtype)
    w2 = store(r.normal(0.0, 0.02, (L, cfg.E, cfg.H, cfg.I)).astype(np.float32), cfg.dtype)
    if cfg.n_shared:
        w13s = store(r.normal(0.0, 0.02, (L, cfg.n_shared, 2 * cfg.I, cfg.H)).astype(np.float32),
                     cfg.dtype)
        w2s = store(r.normal(0.0, 0.02, (L, cfg.n_shared, cfg.H, cfg.I)).astype(np.float32),
                    cfg.dtype)
    else:
        w13s = w2s = None
    return w13, w2, w13s, w2s


def weights_torch(cfg: Config, seed: int, device, layers: int | None = None):
    """Expert weights drawn on ``device`` with a seeded torch generator.

    Same layout as ``weights_numpy``; torch tensors of dtype bfloat16 (or
    float32).  Every (layer, expert) slice is distinct.  Drawn one layer at a
    time to bound the float32 temporary.
    """
    import torch

    L = cfg.L if layers is None else layers
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000003 + 17)

    def draw(shape):
        out = torch.empty(shape, dtype=tdt, device=device)
        for l in range(shape[0]):
            tmp = torch.randn(shape[1:], generator=g, device=device, dtype=torch.float32)
            out[l].copy_(tmp.mul_(0.02))
            del tmp
        return out

    w13 = draw((L, cfg.E, 2 * cfg.I, cfg.H))
    w2 = draw((L, cfg.E, cfg.H, cfg.I))
    if cfg.n_shared:
        w13s = draw((L, cfg.n_shared, 2 * cfg.I, cfg.H))
        w2s = draw((L, cfg.n_shared, cfg.H, cfg.I))
    else:
        w13s = w2s = None
    return w13, w2, w13s, w2s


# ---------------------------------------------------------------- router weights
# Routing from the hidden state: z = h W_g^T + b.  W_g ~ N(0, 1/sqrt(H)) so that
# h W_g^T of an N(0, 1) hidden row is about N(0, 1) -- the noise part of the
# given-logits recipe -- and b is that recipe's per-layer expert bias (profile
# 0), so routing from h has the same skew structure.
def gate_bias(cfg: Config, seed: int) -> np.ndarray:
    """Per-layer expert bias of the router, float32 [L, E]."""
    return np.stack([expert_bias(cfg, seed, 0, l) for l in range(cfg.L)]).astype(np.float32)


def gate_weights_numpy(cfg: Config, seed: int) -> np.ndarray:
    """Router weights [L, E, H] in storage form (small configs)."""
    r = _rng(seed, _FAM_GATE, 0, 0)
    w = r.normal(0.0, 1.0 / np.sqrt(cfg.H), (cfg.L, cfg.E, cfg.H)).astype(np.float32)
    return store(w, cfg.dtype)


def gate_weights_torch(cfg: Config, seed: int, device):
    """Router weights [L, E, H] drawn on ``device`` with a seeded generator."""
    import torch

    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000003 + 29)
    out = torch.empty((cfg.L, cfg.E, cfg.H), dtype=tdt, device=device)
    for l in range(cfg.L):
        tmp = torch.randn((cfg.E, cfg.H), generator=g, device=device, dtype=torch.float32)
        out[l].copy_(tmp.mul_(1.0 / float(np.sqrt(cfg.H))))
    return out
