"""Python binding of libcle.so, the cross-layer MoE expert step for MI355X.

Argument marshalling only: every step of the path runs in the library's HIP
kernels (or, for ``schedule_step``, its host C++).  Tensors are torch tensors
on the GPU; PyTorch provides device memory and streams.  If ``libcle.so`` is
missing or fails to load, importing this package raises -- there is no
fallback implementation.  ``CLE_LIBRARY`` names another build of the same
library to load instead (for comparing builds); it must exist too.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("CLE_LIBRARY") or os.path.join(_PKG, "libcle.so")

OK, EINVAL, EHIP, EWORKSPACE, EUNSUPPORTED = 0, -1, -2, -3, -4
BF16, F32 = 0, 1
POLICY_B0_ALONE, POLICY_B1_LOCKSTEP, POLICY_CUMUTIL, POLICY_MAXUTIL, POLICY_DIFFPEAK = range(5)
POLICIES = {"b0": 0, "b1": 1, "cumutil": 2, "maxutil": 3, "diffpeak": 4}
OP_DISPATCH, OP_FFN, OP_DISPATCH_MANY = 1, 2, 3
W_ROWMAJOR, W_PACKED = 0, 1
MAX_E, MAX_MICROBATCHES, MAX_MAXUTIL_POOL, MAX_DESC = 1024, 64, 20, 64


class CleError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")
        self.status = status


def _load():
    # torch ships a HIP runtime with the same soname as ROCm's; loading torch
    # first makes libcle bind to that one runtime, so torch's streams and
    # device pointers are valid in the library.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m cross_layer_expert_amd.build` (hipcc, gfx950)")
    return ctypes.CDLL(LIB_PATH)


_lib = _load()

_i32, _i64, _u64, _sz, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t, ctypes.c_void_p


class FfnDesc(ctypes.Structure):
    """Mirror of ``cle_ffn_desc``."""
    _fields_ = [("layer", _i32), ("rows", _i32), ("offsets", _vp), ("xp", _vp), ("act", _vp),
                ("yp", _vp), ("shared_rows", _i32), ("x_shared", _vp), ("act_shared", _vp),
                ("y_shared", _vp), ("x", _vp), ("src", _vp), ("k", _i32)]


_P64 = _vp * 64


class LoopState(ctypes.Structure):
    """Mirror of ``cle_loop_state`` (read back from device memory)."""
    _fields_ = [("layer", _i32 * 64), ("run_layer", _i32 * 64), ("start", _i32 * 64),
                ("ready", _u64), ("todo", _u64), ("runset", _u64), ("acc", _i64 * 4),
                ("n", _i32), ("L", _i32), ("restarts", _i32), ("restarted", _i32)]


class LoopDesc(ctypes.Structure):
    """Mirror of ``cle_loop_desc``."""
    _fields_ = [(f, _i32) for f in ("n", "L", "T", "E", "k", "H", "I", "D", "m", "policy",
                                    "n_shared", "dtype", "w_layout", "restart")] + \
               [(f, _P64) for f in ("logits", "h", "h0", "idx", "gate", "counts", "offsets",
                                    "dest", "src", "act", "yp", "act_shared", "y_shared")] + \
               [("w13", _vp), ("w2", _vp), ("w13_shared", _vp), ("w2_shared", _vp),
                ("ws_dispatch", _vp), ("ws_dispatch_bytes", _sz), ("ws_ffn", _vp),
                ("ws_ffn_bytes", _sz), ("w", _vp), ("log", _vp), ("log_cap", _i64),
                ("state", _vp), ("w_gate", _vp), ("gate_bias", _vp), ("gate_logits", _P64),
                ("prenorm", _i32), ("norm_eps", ctypes.c_float), ("xn", _P64)]


LOOP_STATE_BYTES = ctypes.sizeof(LoopState)

_sig = {
    "cle_schedule_step_device": (_i32, [_vp, _i32, _i32, _u64, _i32, _i32, _vp, _vp]),
    "cle_loop_init": (_i32, [_vp, _i32, _i32, ctypes.POINTER(_i32), _vp]),
    "cle_loop_step": (_i32, [ctypes.POINTER(LoopDesc), ctypes.POINTER(_vp), _vp]),
    "cle_gate_logits_many": (_i32, [_i32, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp,
                                    _vp]),
    "cle_rmsnorm_many": (_i32, [_i32, _vp, _vp, _i32, _i32, ctypes.c_float, _i32, _vp]),
    "cle_route": (_i32, [_vp, _i32, _i32, _i32, _vp, _vp, _vp]),
    "cle_route_many": (_i32, [_i32, _vp, _i32, _i32, _i32, _vp, _vp, _vp]),
    "cle_dispatch_many": (_i32, [_i32, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _sz,
                                 _vp]),
    "cle_combine_many": (_i32, [_i32, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _i32, _vp, _vp,
                                _i32, _vp]),
    "cle_dispatch": (_i32, [_vp, _i32, _i32, _i32, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp,
                            _vp, _sz, _vp]),
    "cle_grouped_expert_ffn": (_i32, [ctypes.POINTER(FfnDesc), _i32, _vp, _vp, _vp, _vp, _i32,
                                      _i32, _i32, _i32, _i32, _i32, _i32, _vp, _sz,
                                      ctypes.POINTER(_vp), _vp]),
    "cle_pack_weights": (_i32, [_vp, _vp, _i64, _i32, _i32, _i32, _vp]),
    "cle_set_expert_tile": (_i32, [_i32]),
    "cle_set_fused_thin_rows": (_i32, [_i32]),
    "cle_grouped_expert_ffn_noalloc": (_i32, [ctypes.POINTER(FfnDesc), _i32, _vp, _vp, _vp, _vp,
                                              _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                              ctypes.POINTER(_vp), _vp]),
    "cle_combine": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _vp, _i32, _vp, _vp, _i32, _vp]),
    "cle_workload_stats": (_i32, [_vp, _i32, _i32, _i32, _u64, _vp, _vp, _vp]),
    "cle_schedule_step": (_i32, [ctypes.POINTER(_i32), _i32, _i32, _u64, _i32, _i32,
                                 ctypes.POINTER(_u64)]),
    "cle_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "cle_status_string": (ctypes.c_char_p, [_i32]),
    "cle_version": (ctypes.c_char_p, []),
}
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def status_string(s: int) -> str:
    return _lib.cle_status_string(int(s)).decode()


def version() -> str:
    return _lib.cle_version().decode()


def _check(fn, st):
    if st != OK:
        raise CleError(fn, st)


def _ptr(t):
    """Device (or host) address of a tensor, or None."""
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _dt(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def workspace_bytes(op, T=0, E=1, k=1, n_shared=0, n_desc=1) -> int:
    return int(_lib.cle_workspace_bytes(op, T, E, k, n_shared, n_desc))


# ---------------------------------------------------------------- entry points
def route(logits, k, topk_idx, topk_gate, stream=None):
    T, E = logits.shape
    _check("cle_route", _lib.cle_route(_ptr(logits), T, E, k, _ptr(topk_idx), _ptr(topk_gate),
                                       _stream(stream)))


def dispatch(topk_idx, E, x, counts, offsets, dest, src, xp, ws, stream=None):
    """xp may be None: the row copy is skipped (the expert launch then reads
    the rows of x through src)."""
    T, k = topk_idx.shape
    H = x.shape[1]
    _check("cle_dispatch", _lib.cle_dispatch(
        _ptr(topk_idx), T, k, E, _ptr(x), H, _dt(x), _ptr(counts), _ptr(offsets), _ptr(dest),
        _ptr(src), _ptr(xp), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def _ptrs(ts):
    """HOST array of device addresses (None -> NULL), kept alive by the caller's
    reference to the returned ctypes array for the duration of the call."""
    return (_vp * len(ts))(*[None if t is None else t.data_ptr() for t in ts])


def route_many(logits, k, topk_idx, topk_gate, stream=None):
    """logits, topk_idx, topk_gate: equal-length lists of per-micro-batch tensors."""
    n = len(logits)
    T, E = logits[0].shape
    _check("cle_route_many", _lib.cle_route_many(
        n, _ptrs(logits), T, E, k, _ptrs(topk_idx), _ptrs(topk_gate), _stream(stream)))


NORM_EPS = 1e-6


def rmsnorm_many(x, y, eps=NORM_EPS, stream=None):
    """y_j = x_j / sqrt(mean(x_j^2, rows) + eps); lists of [T, H] tensors."""
    n = len(x)
    T, H = x[0].shape
    _check("cle_rmsnorm_many", _lib.cle_rmsnorm_many(n, _ptrs(x), _ptrs(y), T, H, float(eps),
                                                     _dt(x[0]), _stream(stream)))


def gate_logits_many(x, w_gate, logits, bias=None, packed=False, stream=None):
    """Router logits z_j = x_j w_gate_j^T + bias_j.  x: list of [T, H]; w_gate:
    list of [E, H] (each micro-batch's layer; packed=True if written by
    pack_weights); logits: list of [T, E] float32 out; bias: None or a list
    of [E] float32 tensors (entries may be None)."""
    n = len(x)
    T, H = x[0].shape
    E = w_gate[0].shape[0]
    _check("cle_gate_logits_many", _lib.cle_gate_logits_many(
        n, _ptrs(x), _ptrs(w_gate), None if bias is None else _ptrs(bias), T, H, E, _dt(x[0]),
        W_PACKED if packed else W_ROWMAJOR, _ptrs(logits), _stream(stream)))


def dispatch_many(topk_idx, E, counts, offsets, dest, src, ws, stream=None):
    """Per-micro-batch lists; no row copy (the expert launch reads rows through src)."""
    n = len(topk_idx)
    T, k = topk_idx[0].shape
    _check("cle_dispatch_many", _lib.cle_dispatch_many(
        n, _ptrs(topk_idx), T, k, E, _ptrs(counts), _ptrs(offsets), _ptrs(dest), _ptrs(src),
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def combine_many(yp, dest, topk_gate, y, y_shared=None, residual=None, stream=None):
    """Per-micro-batch lists; y_shared / residual: None or lists (entries may be None)."""
    n = len(yp)
    T, k = topk_gate[0].shape
    H = y[0].shape[-1]
    ns = 0 if y_shared is None or y_shared[0] is None else y_shared[0].shape[0]
    _check("cle_combine_many", _lib.cle_combine_many(
        n, _ptrs(yp), _ptrs(dest), _ptrs(topk_gate), T, k, H,
        None if y_shared is None else _ptrs(y_shared), ns,
        None if residual is None else _ptrs(residual), _ptrs(y), _dt(y[0]), _stream(stream)))


def make_desc(layer, rows, offsets, xp, act, yp, shared_rows=0, x_shared=None, act_shared=None,
              y_shared=None, x=None, src=None, k=0) -> FfnDesc:
    """One micro-batch of a grouped expert launch.  Pass xp=None with x, src,
    k to read the expert-sorted rows of x in place."""
    return FfnDesc(layer, rows, _ptr(offsets), _ptr(xp), _ptr(act), _ptr(yp), shared_rows,
                   _ptr(x_shared), _ptr(act_shared), _ptr(y_shared), _ptr(x), _ptr(src), k)


def grouped_expert_ffn(descs, w13, w2, ws, w13_shared=None, w2_shared=None, events=None,
                       stream=None, packed=False):
    """descs: list of FfnDesc.  w13 [L, E, 2I, H], w2 [L, E, H, I] (shapes of the
    row-major tensors; packed=True when all four were written by pack_weights).
    events: None or 4 raw hipEvent_t handles (ints): start and end of the
    gate/up kernel, then of the down kernel."""
    L, E, I2, H = w13.shape
    ns = 0 if w13_shared is None else w13_shared.shape[1]
    arr = (FfnDesc * len(descs))(*descs)
    ev = None
    if events is not None:
        if len(events) != 4:
            raise ValueError("events: 4 hipEvent_t handles")
        ev = (_vp * 4)(*events)
    _check("cle_grouped_expert_ffn", _lib.cle_grouped_expert_ffn(
        arr, len(descs), _ptr(w13), _ptr(w2), _ptr(w13_shared), _ptr(w2_shared), L, E, ns, H,
        I2 // 2, _dt(w13), W_PACKED if packed else W_ROWMAJOR, _ptr(ws),
        ws.numel() * ws.element_size(), ev, _stream(stream)))


NOALLOC_SCRATCH_BYTES = 1 << 20


def grouped_expert_ffn_noalloc(descs, w13, w2, w13_shared=None, w2_shared=None, events=None,
                               stream=None, packed=False):
    """grouped_expert_ffn without a workspace: the library's own fixed scratch
    (one per GPU) is used; concurrent calls on one GPU race."""
    L, E, I2, H = w13.shape
    ns = 0 if w13_shared is None else w13_shared.shape[1]
    arr = (FfnDesc * len(descs))(*descs)
    ev = None
    if events is not None:
        if len(events) != 4:
            raise ValueError("events: 4 hipEvent_t handles")
        ev = (_vp * 4)(*events)
    _check("cle_grouped_expert_ffn_noalloc", _lib.cle_grouped_expert_ffn_noalloc(
        arr, len(descs), _ptr(w13), _ptr(w2), _ptr(w13_shared), _ptr(w2_shared), L, E, ns, H,
        I2 // 2, _dt(w13), W_PACKED if packed else W_ROWMAJOR, ev, _stream(stream)))


TILE_DEFAULT, TILE_128X256, TILE_256X256, TILE_128X512 = 0, 1, 2, 3
TILES = {"default": 0, "128x256": 1, "256x256": 2, "128x512": 3}


def set_expert_tile(tile):
    """Output tile of the bf16 expert launches (process-wide; results are
    bitwise the same for every tile): an int or a name of TILES."""
    _check("cle_set_expert_tile", _lib.cle_set_expert_tile(TILES.get(tile, tile)
                                                           if isinstance(tile, str) else tile))


def set_fused_thin_rows(rows):
    """Fused gate/up -> down launch for routed segments of 1 .. rows rows
    (process-wide; 0 off, -1 the environment decides; results bitwise the same)."""
    _check("cle_set_fused_thin_rows", _lib.cle_set_fused_thin_rows(int(rows)))


def pack_weights(src, dst=None, stream=None):
    """Packed copy of a bf16 weight tensor [..., R, K] (the matrices are the
    last two dimensions); dst: a tensor of the same size, or None for a new one."""
    import torch
    if dst is None:
        dst = torch.empty_like(src)
    R, K = src.shape[-2], src.shape[-1]
    n = src.numel() // (R * K)
    _check("cle_pack_weights", _lib.cle_pack_weights(_ptr(src), _ptr(dst), n, R, K, _dt(src),
                                                     _stream(stream)))
    return dst


def pack_weights_inplace(t, mats_per_chunk=64, stream=None):
    """Pack a bf16 weight tensor [..., R, K] in place, through a scratch copy of
    at most mats_per_chunk matrices at a time (so no second full-size copy)."""
    R, K = t.shape[-2], t.shape[-1]
    flat = t.view(-1, R, K)
    for a in range(0, flat.shape[0], mats_per_chunk):
        part = flat[a:a + mats_per_chunk]
        part.copy_(pack_weights(part, stream=stream))
    return t


def combine(yp, dest, topk_gate, y, y_shared=None, residual=None, stream=None):
    T, k = topk_gate.shape
    H = y.shape[-1]
    ns = 0 if y_shared is None else y_shared.shape[0]
    _check("cle_combine", _lib.cle_combine(
        _ptr(yp), _ptr(dest), _ptr(topk_gate), T, k, H, _ptr(y_shared), ns, _ptr(residual),
        _ptr(y), _dt(y), _stream(stream)))


def workload_stats(counts, D, runset_mask, w, acc=None, stream=None):
    n, E = counts.shape
    _check("cle_workload_stats", _lib.cle_workload_stats(
        _ptr(counts), n, E, D, int(runset_mask), _ptr(w), _ptr(acc), _stream(stream)))


def schedule_step(w, ready_mask, m, policy) -> int:
    """w: host int32 array [n, D].  Returns the RunSet bitmask."""
    w = np.ascontiguousarray(w, dtype=np.int32)
    n, D = w.shape
    out = _u64(0)
    _check("cle_schedule_step", _lib.cle_schedule_step(
        w.ctypes.data_as(ctypes.POINTER(_i32)), n, D, int(ready_mask), m, int(policy),
        ctypes.byref(out)))
    return int(out.value)


def schedule_step_raw(w_ptr, n, D, ready_mask, m, policy) -> int:
    """Same as schedule_step with w given as a host address (pinned buffer)."""
    out = _u64(0)
    _check("cle_schedule_step", _lib.cle_schedule_step(
        ctypes.cast(w_ptr, ctypes.POINTER(_i32)), n, D, int(ready_mask), m, int(policy),
        ctypes.byref(out)))
    return int(out.value)


def mask_of(ids) -> int:
    m = 0
    for j in ids:
        m |= 1 << int(j)
    return m


def ids_of(mask: int) -> list:
    return [j for j in range(64) if mask >> j & 1]


# ---------------------------------------------------------------- device-driven loop
def schedule_step_device(w, ready_mask, m, policy, runset, stream=None):
    """w: device int32 [n, D]; runset: device tensor of >= 8 bytes (uint64 out)."""
    n, D = w.shape
    _check("cle_schedule_step_device", _lib.cle_schedule_step_device(
        _ptr(w), n, D, int(ready_mask), m, int(policy), _ptr(runset), _stream(stream)))


def loop_init(state, n, L, start=None, stream=None):
    """state: device tensor of >= LOOP_STATE_BYTES bytes (8-byte aligned)."""
    st = None
    if start is not None:
        st = (_i32 * n)(*[int(v) for v in start])
    _check("cle_loop_init", _lib.cle_loop_init(_ptr(state), n, L, st, _stream(stream)))


def loop_step(desc, events=None, stream=None):
    """desc: a LoopDesc; events: None or 4 hipEvent_t handles (see grouped_expert_ffn)."""
    ev = None
    if events is not None:
        if len(events) != 4:
            raise ValueError("events: 4 hipEvent_t handles")
        ev = (_vp * 4)(*events)
    _check("cle_loop_step", _lib.cle_loop_step(ctypes.byref(desc), ev, _stream(stream)))


def read_loop_state(state) -> LoopState:
    """Copy the state back (synchronises the current stream with the copy)."""
    raw = state.view(__import__("torch").uint8)[:LOOP_STATE_BYTES].cpu().numpy()
    return LoopState.from_buffer_copy(raw.tobytes())
