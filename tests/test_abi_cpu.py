"""CPU-side checks of libcle.so: it loads, exports every symbol the header
declares, validates arguments on the host, and its host scheduler matches the
oracle bit for bit.  No GPU compute is issued here."""
import json
import os
import random
import re

import numpy as np
import pytest

import cross_layer_expert_amd as cle
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cle.h")


def test_every_declared_symbol_is_exported():
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:cle_status|size_t|const char\*)\s+(cle_\w+)\s*\(", text,
                              re.M))
    assert {"cle_route", "cle_dispatch", "cle_grouped_expert_ffn", "cle_combine",
            "cle_workload_stats", "cle_schedule_step", "cle_workspace_bytes",
            "cle_route_many", "cle_dispatch_many", "cle_combine_many", "cle_pack_weights",
            "cle_schedule_step_device", "cle_loop_init", "cle_loop_step"} <= declared
    for name in declared:
        assert hasattr(cle._lib, name), name
    assert cle.version().count(".") == 2


def test_status_strings():
    for s in (cle.OK, cle.EINVAL, cle.EHIP, cle.EWORKSPACE, cle.EUNSUPPORTED):
        assert cle.status_string(s)
    assert cle.status_string(123) == "unknown status"


def test_workspace_bytes():
    assert cle.workspace_bytes(cle.OP_DISPATCH, 2048, 128, 8) == 16 * 128 * 4
    assert cle.workspace_bytes(cle.OP_DISPATCH, 0, 8, 2) == 256
    assert cle.workspace_bytes(cle.OP_DISPATCH, 10, 2000, 2) == 0
    b = cle.workspace_bytes(cle.OP_FFN, 0, 128, 1, 0, 4)
    assert b >= 256 + 4 * 128 * 56 and b % 256 == 0
    assert cle.workspace_bytes(cle.OP_FFN, 0, 64, 1, 2, 65) == 0
    assert cle.workspace_bytes(99, 1, 1, 1) == 0
    # one dispatch workspace per micro-batch of a cle_dispatch_many call
    one = cle.workspace_bytes(cle.OP_DISPATCH, 2048, 128, 8)
    assert cle.workspace_bytes(cle.OP_DISPATCH_MANY, 2048, 128, 8, 0, 3) == 3 * one
    assert cle.workspace_bytes(cle.OP_DISPATCH_MANY, 100, 7, 3, 0, 64) == \
        64 * cle.workspace_bytes(cle.OP_DISPATCH, 100, 7, 3)
    assert cle.workspace_bytes(cle.OP_DISPATCH_MANY, 16, 8, 2, 0, 0) == 0
    assert cle.workspace_bytes(cle.OP_DISPATCH_MANY, 16, 8, 2, 0, 65) == 0


def test_invalid_arguments_rejected_on_host():
    """Each call fails validation before any HIP call (null device pointers
    are never dereferenced)."""
    L = cle._lib
    assert L.cle_route(None, 4, 8, 9, None, None, None) == cle.EINVAL     # k > E
    assert L.cle_route(None, 4, 2000, 1, None, None, None) == cle.EINVAL  # E > max
    assert L.cle_route(None, 0, 8, 2, None, None, None) == cle.OK         # T == 0: nothing to do
    assert L.cle_dispatch(None, 4, 2, 8, None, 12, 0, None, None, None, None, None, None, 0,
                          None) == cle.EINVAL                              # H % 8
    assert L.cle_combine(None, None, None, 4, 2, 64, None, 0, None, None, 7, None) == cle.EINVAL
    assert L.cle_workload_stats(None, 2, 8, 3, 0, None, None, None) == cle.EINVAL
    assert L.cle_workload_stats(8, 2, 8, 3, 0, 8, None, None) == cle.EINVAL  # E % D
    assert L.cle_workload_stats(8, 2, 8, 4, 0b100, 8, 8, None) == cle.EINVAL  # mask bit >= n
    d = (cle.FfnDesc * 1)(cle.FfnDesc(0, 8, 16, 16, 16, 16, 0, None, None, None))
    assert L.cle_grouped_expert_ffn(d, 1, 16, 16, None, None, 2, 8, 0, 96, 64, 1, 0, None, 0,
                                    None, None) == cle.EINVAL              # f32: H % 64
    assert L.cle_grouped_expert_ffn(d, 1, 16, 16, None, None, 2, 8, 0, 64, 64, 0, 0, None, 0,
                                    None, None) == cle.EINVAL              # bf16: H % 128
    assert L.cle_grouped_expert_ffn(d, 1, 16, 16, None, None, 2, 8, 0, 128, 64, 0, 0, None, 0,
                                    None, None) == cle.EWORKSPACE
    assert L.cle_grouped_expert_ffn(d, 1, 16, 16, None, None, 2, 8, 0, 128, 64, 1, 1, None, 0,
                                    None, None) == cle.EINVAL              # packed needs bf16
    assert L.cle_grouped_expert_ffn(d, 1, 16, 16, None, None, 2, 8, 0, 128, 64, 0, 2, None, 0,
                                    None, None) == cle.EINVAL              # unknown layout
    assert L.cle_pack_weights(16, 4096, 1, 24, 64, 0, None) == cle.EINVAL  # R % 16
    assert L.cle_pack_weights(16, 4096, 1, 16, 96, 0, None) == cle.EINVAL  # K % 64
    assert L.cle_pack_weights(16, 4096, 1, 16, 64, 1, None) == cle.EINVAL  # f32
    assert L.cle_pack_weights(16, 1024, 1, 16, 64, 0, None) == cle.EINVAL  # overlapping
    assert L.cle_pack_weights(None, None, 0, 16, 64, 0, None) == cle.OK    # nothing to pack
    d[0].layer = 2
    assert L.cle_grouped_expert_ffn(d, 1, 16, 16, None, None, 2, 8, 0, 128, 64, 0, 0, None, 0,
                                    None, None) == cle.EINVAL              # layer >= L


def test_batched_calls_validate_on_host():
    """The _many entry points reject bad counts, NULL pointer arrays, NULL
    entries and short workspaces before any HIP call; T == 0 is a no-op."""
    import ctypes
    L = cle._lib
    vp = ctypes.c_void_p

    def arr(*v):
        return (vp * len(v))(*v)

    one, null1 = arr(16), arr(None)
    three = arr(16, 32, 48)
    # route_many(n, logits, T, E, k, idx, gate, stream)
    assert L.cle_route_many(0, one, 4, 8, 2, one, one, None) == cle.EINVAL     # n < 1
    assert L.cle_route_many(65, one, 4, 8, 2, one, one, None) == cle.EINVAL    # n > 64
    assert L.cle_route_many(1, None, 4, 8, 2, one, one, None) == cle.EINVAL    # no array
    assert L.cle_route_many(1, null1, 4, 8, 2, one, one, None) == cle.EINVAL   # NULL entry
    assert L.cle_route_many(1, one, 4, 8, 9, one, one, None) == cle.EINVAL     # k > E
    assert L.cle_route_many(3, three, 0, 8, 2, three, three, None) == cle.OK   # T == 0
    # dispatch_many(n, idx, T, k, E, counts, offsets, dest, src, ws, ws_bytes, stream)
    need = cle.workspace_bytes(cle.OP_DISPATCH_MANY, 4, 8, 2, 0, 3)
    assert L.cle_dispatch_many(3, three, 4, 2, 8, three, three, three, three, 256, need - 1,
                               None) == cle.EWORKSPACE
    assert L.cle_dispatch_many(3, three, 4, 2, 8, three, three, three, three, 255, need,
                               None) == cle.EWORKSPACE                        # unaligned ws
    assert L.cle_dispatch_many(3, three, 4, 2, 8, three, arr(16, None, 48), three, three, 256,
                               need, None) == cle.EINVAL                      # NULL offsets entry
    assert L.cle_dispatch_many(1, one, 4, 2, 2000, one, one, one, one, 256, 1 << 20,
                               None) == cle.EINVAL                            # E > max
    # combine_many(n, yp, dest, gate, T, k, H, y_shared, n_shared, residual, y, dt, stream)
    assert L.cle_combine_many(1, one, one, one, 4, 2, 12, None, 0, None, one, 0,
                              None) == cle.EINVAL                             # H % 8
    assert L.cle_combine_many(1, one, one, one, 4, 2, 64, None, 1, None, one, 0,
                              None) == cle.EINVAL                             # shared, no array
    assert L.cle_combine_many(1, one, one, one, 4, 2, 64, None, 0, None, arr(8), 0,
                              None) == cle.EINVAL                             # y not 16-aligned
    assert L.cle_combine_many(1, one, one, one, 4, 2, 64, None, 0, None, one, 5,
                              None) == cle.EINVAL                             # dtype
    assert L.cle_combine_many(2, arr(16, 32), arr(16, 32), arr(16, 32), 0, 2, 64, None, 0,
                              None, arr(16, 32), 0, None) == cle.OK           # T == 0


def test_schedule_step_errors():
    w = np.ones((4, 2), np.int32)
    with pytest.raises(cle.CleError):
        cle.schedule_step(w, 0, 1, cle.POLICY_CUMUTIL)          # empty pool
    with pytest.raises(cle.CleError):
        cle.schedule_step(w, 0b10000, 1, cle.POLICY_CUMUTIL)    # bit >= n
    with pytest.raises(cle.CleError):
        cle.schedule_step(w, 0b1111, 0, cle.POLICY_CUMUTIL)     # m < 1
    with pytest.raises(cle.CleError):
        cle.schedule_step(w, 0b1111, 5, cle.POLICY_CUMUTIL)     # m > n
    with pytest.raises(cle.CleError):
        cle.schedule_step(w, 0b1111, 1, 9)                       # policy
    with pytest.raises(cle.CleError):
        cle.schedule_step(-w, 0b1111, 1, cle.POLICY_B1_LOCKSTEP)  # negative workload
    big = np.ones((24, 2), np.int32)
    with pytest.raises(cle.CleError) as e:
        cle.schedule_step(big, (1 << 24) - 1, 2, cle.POLICY_MAXUTIL)
    assert e.value.status == cle.EUNSUPPORTED
    # a pool smaller than m never needs the exhaustive search
    assert cle.schedule_step(big, (1 << 24) - 1, 24, cle.POLICY_MAXUTIL) == (1 << 24) - 1


def test_schedule_hand_examples():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "schedule_examples.json")))
    for ex in g["examples"]:
        w = np.array(ex["w"], np.int32)
        ready = ex.get("ready", list(range(len(w))))
        for name, want in ex["expect"].items():
            got = cle.schedule_step(w, cle.mask_of(ready), ex["m"], cle.POLICIES[name])
            assert cle.ids_of(got) == want, (ex["name"], name)


@pytest.mark.parametrize("policy", ["b0", "b1", "cumutil", "maxutil", "diffpeak"])
def test_schedule_matches_oracle_random(policy):
    rnd = random.Random(hash(policy) & 0xffff)
    for trial in range(400):
        n = rnd.randint(1, 12 if policy == "maxutil" else 40)
        D = rnd.randint(1, 9)
        hot = rnd.random() < 0.5
        w = np.array([[rnd.randint(0, 50) if not hot or rnd.random() < 0.3 else rnd.randint(0, 3)
                       for _ in range(D)] for _ in range(n)], np.int32)
        if rnd.random() < 0.1:
            w[rnd.randrange(n)] = 0            # an empty micro-batch
        ready = [j for j in range(n) if rnd.random() < 0.7] or [rnd.randrange(n)]
        m = rnd.randint(1, n)
        got = cle.ids_of(cle.schedule_step(w, cle.mask_of(ready), m, cle.POLICIES[policy]))
        want = list(oracle.schedule([list(r) for r in w], ready, m, oracle.POLICIES[policy]))
        assert got == want, (trial, w.tolist(), ready, m)


def test_maxutil_large_pool_matches_oracle():
    rnd = random.Random(5)
    for _ in range(3):
        n, D = 16, 8
        w = np.array([[rnd.randint(0, 300) for _ in range(D)] for _ in range(n)], np.int32)
        got = cle.ids_of(cle.schedule_step(w, (1 << n) - 1, 12, cle.POLICY_MAXUTIL))
        want = list(oracle.schedule([list(r) for r in w], range(n), 12, oracle.POLICIES["maxutil"]))
        assert got == want


def test_loop_structs_match_header(tmp_path):
    """The ctypes mirrors of cle_loop_state and cle_loop_desc have the C
    layout: every field offset and both sizes, from a C program built with
    the system compiler against include/cle.h."""
    import ctypes
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lines = []
    for cname, py in (("cle_loop_state", cle.LoopState), ("cle_loop_desc", cle.LoopDesc)):
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    src = tmp_path / "layout.c"
    src.write_text("#include <stdio.h>\n#include <stddef.h>\n#include \"cle.h\"\n"
                   "int main(void) {\n" + "\n".join(lines) + "\nreturn 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = {}
    for line in subprocess.run([str(exe)], check=True, capture_output=True,
                               text=True).stdout.splitlines():
        c, f, v = line.split()
        got[(c, f)] = int(v)
    for cname, py in (("cle_loop_state", cle.LoopState), ("cle_loop_desc", cle.LoopDesc)):
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)


def test_loop_calls_validate_on_host():
    """cle_loop_init / cle_loop_step / cle_schedule_step_device reject bad
    arguments before anything is enqueued."""
    import ctypes
    L = cle._lib
    i32 = ctypes.c_int32
    assert L.cle_loop_init(None, 4, 8, None, None) == cle.EINVAL            # no state
    assert L.cle_loop_init(4, 4, 8, None, None) == cle.EINVAL               # unaligned
    assert L.cle_loop_init(256, 0, 8, None, None) == cle.EINVAL             # n < 1
    assert L.cle_loop_init(256, 65, 8, None, None) == cle.EINVAL            # n > 64
    assert L.cle_loop_init(256, 2, 8, (i32 * 2)(0, 9), None) == cle.EINVAL  # start > L
    assert L.cle_loop_step(None, None, None) == cle.EINVAL

    def desc(**over):
        d = cle.LoopDesc()
        d.n, d.L, d.T, d.E, d.k, d.H, d.I, d.D, d.m = 2, 4, 16, 8, 2, 128, 64, 4, 1
        d.policy, d.dtype, d.w_layout = cle.POLICY_CUMUTIL, cle.BF16, cle.W_ROWMAJOR
        for f in ("logits", "h", "h0", "idx", "gate", "counts", "offsets", "dest", "src",
                  "act", "yp"):
            arr = getattr(d, f)
            for j in range(2):
                arr[j] = 4096 * (j + 1)
        d.w13, d.w2, d.state = 1 << 20, 1 << 21, 1 << 22
        d.ws_dispatch, d.ws_dispatch_bytes = 1 << 23, 1 << 20
        d.ws_ffn, d.ws_ffn_bytes = 1 << 24, 1 << 20
        for k, v in over.items():
            setattr(d, k, v)
        return d

    def step(d):
        return L.cle_loop_step(ctypes.byref(d), None, None)

    assert step(desc(n=0)) == cle.EINVAL
    assert step(desc(D=3)) == cle.EINVAL                      # E % D
    assert step(desc(D=128, E=128, k=2)) == cle.EINVAL        # D > 64
    assert step(desc(m=3)) == cle.EINVAL                      # m > n
    assert step(desc(policy=7)) == cle.EINVAL
    assert step(desc(restart=2)) == cle.EINVAL
    assert step(desc(prenorm=2)) == cle.EINVAL
    assert step(desc(prenorm=1, norm_eps=1e-6)) == cle.EINVAL   # xn entries missing
    assert step(desc(w_gate=1 << 26, E=96, D=4)) == cle.EINVAL  # gate: E % 64 (bf16)
    assert step(desc(I=96)) == cle.EINVAL                     # I % 64 (expert launch)
    assert step(desc(state=None)) == cle.EINVAL
    assert step(desc(ws_dispatch_bytes=0)) == cle.EWORKSPACE
    assert step(desc(ws_ffn_bytes=0)) == cle.EWORKSPACE
    assert step(desc(log=1 << 25, log_cap=0)) == cle.EINVAL
    d = desc()
    d.yp[1] = None
    assert step(d) == cle.EINVAL                              # NULL entry
    d = desc(n_shared=1)
    assert step(d) == cle.EINVAL                              # shared buffers missing
    d = desc(n=21, m=1, policy=cle.POLICY_MAXUTIL)
    assert step(d) == cle.EUNSUPPORTED                        # MaxUtil pool > 20
    # cle_schedule_step_device(w, n, D, ready, m, policy, runset, stream)
    S = L.cle_schedule_step_device
    assert S(None, 2, 2, 3, 1, 2, 256, None) == cle.EINVAL
    assert S(256, 2, 65, 3, 1, 2, 256, None) == cle.EINVAL    # D > 64
    assert S(256, 2, 2, 0, 1, 2, 256, None) == cle.EINVAL     # empty pool
    assert S(256, 2, 2, 4, 1, 2, 256, None) == cle.EINVAL     # bit beyond n
    assert S(256, 2, 2, 3, 3, 2, 256, None) == cle.EINVAL     # m > n
    assert S(256, 21, 2, (1 << 21) - 1, 1, 3, 256, None) == cle.EUNSUPPORTED


def test_gate_logits_validate_on_host():
    """cle_gate_logits_many(n, x, w_gate, bias, T, H, E, dt, w_layout, logits, stream)."""
    import ctypes
    L = cle._lib
    vp = ctypes.c_void_p

    def arr(*v):
        return (vp * len(v))(*v)

    one = arr(256)
    G = L.cle_gate_logits_many
    assert G(0, one, one, None, 16, 128, 64, cle.BF16, 0, one, None) == cle.EINVAL    # n < 1
    assert G(65, one, one, None, 16, 128, 64, cle.BF16, 0, one, None) == cle.EINVAL   # n > 64
    assert G(1, None, one, None, 16, 128, 64, cle.BF16, 0, one, None) == cle.EINVAL   # no x
    assert G(1, arr(None), one, None, 16, 128, 64, cle.BF16, 0, one, None) == cle.EINVAL
    assert G(1, one, one, None, 16, 96, 64, cle.BF16, 0, one, None) == cle.EINVAL     # H % 128
    assert G(1, one, one, None, 16, 128, 96, cle.BF16, 0, one, None) == cle.EINVAL    # E % 64
    assert G(1, one, one, None, 16, 128, 2048, cle.BF16, 0, one, None) == cle.EINVAL  # E > max
    assert G(1, one, one, None, 16, 64, 8, cle.F32, cle.W_PACKED, one, None) == cle.EINVAL
    assert G(1, one, one, None, -1, 128, 64, cle.BF16, 0, one, None) == cle.EINVAL    # T < 0
    assert G(1, one, arr(8), None, 16, 128, 64, cle.BF16, 0, one, None) == cle.EINVAL  # unaligned
    assert G(1, one, one, None, 16, 128, 64, 7, 0, one, None) == cle.EINVAL           # dtype


def test_rmsnorm_and_prenorm_validate_on_host():
    import ctypes
    L = cle._lib
    vp = ctypes.c_void_p
    one = (vp * 1)(256)
    N = L.cle_rmsnorm_many
    assert N(0, one, one, 4, 64, 1e-6, cle.BF16, None) == cle.EINVAL      # n < 1
    assert N(1, None, one, 4, 64, 1e-6, cle.BF16, None) == cle.EINVAL     # no x
    assert N(1, one, (vp * 1)(None), 4, 64, 1e-6, cle.BF16, None) == cle.EINVAL
    assert N(1, one, one, 4, 60, 1e-6, cle.BF16, None) == cle.EINVAL      # H % 8
    assert N(1, one, one, -1, 64, 1e-6, cle.BF16, None) == cle.EINVAL     # T < 0
    assert N(1, one, one, 4, 64, -1.0, cle.BF16, None) == cle.EINVAL      # eps < 0
    assert N(1, one, one, 4, 64, float("nan"), cle.BF16, None) == cle.EINVAL
    assert N(1, (vp * 1)(8), one, 4, 64, 1e-6, cle.BF16, None) == cle.EINVAL  # unaligned
    assert N(1, one, one, 0, 64, 1e-6, cle.BF16, None) == cle.OK          # T == 0: nothing
