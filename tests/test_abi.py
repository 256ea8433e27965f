"""C-ABI checks that need no GPU: the library loads, exports every function
include/moe.h declares, sizes workspaces on the host and rejects bad
arguments before enqueuing anything."""
import ctypes
import os
import re

import pytest

from routing_dispatch_grouped_router_amd import binding as B
from routing_dispatch_grouped_router_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libmoe.so is not built (run __graft_entry__.build())")
    return B.lib()


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert len(declared) >= 12
    assert sorted(B.EXPORTS) == declared
    for name in declared:
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert "gfx950" in B.version()
    assert lib.moe_status_string(0) == b"ok"
    assert lib.moe_status_string(-4) == b"workspace too small"


def _status(fn, *args):
    return getattr(B.lib(), fn)(*args)


def _prob(**kw):
    base = dict(T=64, d=128, E=8, k=2, H=128, act="bf16")
    base.update(kw)
    return B.problem(base["T"], base["d"], base["E"], base["k"], base["H"], base["act"],
                     logits_given=kw.get("logits_given", False), identity=kw.get("identity", False))


@pytest.mark.parametrize("kw,code", [
    (dict(k=9), -2), (dict(k=0), -2), (dict(E=1025, k=2), -2), (dict(T=0), -2),
    (dict(d=96), -2), (dict(H=32), -2), (dict(act="mxfp8", d=192), -2),
    (dict(k=17, E=32), -2), (dict(act="mxfp8", identity=True, d=128), -3),
])
def test_bad_shapes_rejected(lib, kw, code):
    p = _prob(**kw)
    n = ctypes.c_size_t()
    assert lib.moe_workspace_bytes(ctypes.byref(p), ctypes.byref(n)) == code


def test_bad_dtype_and_flags(lib):
    p = _prob()
    p.act_dtype = 7
    n = ctypes.c_size_t()
    assert lib.moe_workspace_bytes(ctypes.byref(p), ctypes.byref(n)) == -3
    p = _prob()
    p.flags = 64
    assert lib.moe_workspace_bytes(ctypes.byref(p), ctypes.byref(n)) == -3
    assert lib.moe_workspace_bytes(None, ctypes.byref(n)) == -1


@pytest.mark.parametrize("T, d, E, k, H, act, identity, code", [
    (512, 256, 8, 2, 256, "bf16", False, 0),      # the fused bf16 FFN: a | b kept
    (512, 128, 8, 2, 128, "bf16", False, 0),
    (512, 64, 8, 2, 256, "bf16", False, -3),      # d_model < 128: no fused FFN
    (512, 256, 8, 2, 64, "bf16", False, -3),      # d_hidden < 128
    (512, 256, 8, 2, 256, "f32", False, -3),
    (512, 256, 8, 2, 256, "mxfp8", False, 0),     # the MXFP8 GEMM1 keeps them too
    (512, 256, 8, 2, 256, "bf16", True, -3),      # identity experts compute no a | b
])
def test_keep_gate_up_flag(lib, T, d, E, k, H, act, identity, code):
    """MOE_KEEP_GATE_UP is valid for the fused bf16 FFN's problems and MXFP8;
    there the forward workspace grows by the T k 2H bf16 pre-activations, and
    the backward workspace does not change."""
    p = B.problem(T, d, E, k, H, act, logits_given=True, identity=identity, keep_gate_up=True)
    n = ctypes.c_size_t()
    assert lib.moe_workspace_bytes(ctypes.byref(p), ctypes.byref(n)) == code
    if code:
        assert lib.moe_backward_workspace_bytes(ctypes.byref(p), ctypes.byref(n)) == code
        return
    plain = B.problem(T, d, E, k, H, act, logits_given=True)
    ab = T * k * 2 * H * 2
    assert B.workspace_bytes(p) - B.workspace_bytes(plain) == -(-ab // 256) * 256
    assert B.backward_workspace_bytes(p) == B.backward_workspace_bytes(plain)


def test_null_pointers_rejected_before_any_launch(lib):
    p = _prob(logits_given=True)
    V = ctypes.c_void_p
    fake = V(0x1000)   # never dereferenced: validation fails first
    assert lib.moe_route(ctypes.byref(p), None, None, None, fake, fake, fake, fake, fake, fake,
                         None, fake, 1 << 30, None) == -1
    assert lib.moe_dispatch(ctypes.byref(p), fake, None, fake, None, None) == -1
    assert lib.moe_combine(ctypes.byref(p), fake, fake, None, fake, None) == -1
    assert lib.moe_forward(ctypes.byref(p), None, None, fake, fake, fake, None, None, None, None,
                           None, None, fake, 1 << 30, None) == -1
    # the host-synchronising variant needs its host buffer
    assert lib.moe_forward_host_sync(ctypes.byref(p), fake, None, fake, fake, fake, None, None, None, None,
                                     None, None, fake, 1 << 30, None, None) == -1
    pm = _prob(act="mxfp8", logits_given=True)
    assert lib.moe_dispatch(ctypes.byref(pm), fake, fake, fake, None, None) == -1
    assert lib.moe_grouped_swiglu(ctypes.byref(pm), fake, None, fake, fake, fake, fake, 1 << 30,
                                  None) == -1


def test_small_workspace_rejected(lib):
    p = _prob(logits_given=True)
    need = B.workspace_bytes(p)
    fake = ctypes.c_void_p(0x1000)
    assert lib.moe_forward(ctypes.byref(p), fake, None, fake, fake, fake, None, None, None, None,
                           None, None, fake, need - 1, None) == -4
    host = (ctypes.c_int32 * p.n_experts)()
    assert lib.moe_forward_host_sync(ctypes.byref(p), fake, None, fake, fake, fake, None, None, None, None,
                                     None, None, fake, need - 1, None, ctypes.cast(host, ctypes.c_void_p)) == -4
    assert lib.moe_route(ctypes.byref(p), None, None, fake, fake, fake, fake, fake, fake, fake,
                         None, fake, 16, None) == -4


@pytest.mark.parametrize("cap,code", [(0, 0), (8, 0), (256, 0), (64, 0), (-8, -7), (4, -7), (12, -7),
                                      (264, -7)])
def test_gemm_grid_cap_range(lib, cap, code):
    assert lib.moe_set_gemm_grid_cap(cap) == code
    assert lib.moe_set_gemm_grid_cap(0) == 0


@pytest.mark.parametrize("flags,code", [(0, 0), (1, 0), (2, 0), (3, 0), (4, -7), (-1, -7)])
def test_test_flags_range(lib, flags, code):
    assert lib.moe_set_test_flags(flags) == code
    assert lib.moe_set_test_flags(0) == 0


def test_fused_status_host_checks(lib):
    # argument checks run on the host before any device access
    p = B.problem(64, 128, 8, 2, 128, "bf16", logits_given=True)
    st = ctypes.c_int32(123)
    fake = ctypes.c_void_p(0x1000)
    assert lib.moe_fused_status(ctypes.byref(p), None, 1 << 20, 0, ctypes.byref(st), None) == -1
    assert lib.moe_fused_status(ctypes.byref(p), fake, 1 << 20, 0, None, None) == -1
    assert lib.moe_fused_status(ctypes.byref(p), fake, 1 << 20, 5, ctypes.byref(st), None) == -7
    assert lib.moe_fused_status(ctypes.byref(p), fake, 16, 0, ctypes.byref(st), None) == -4
    assert lib.moe_fused_status(ctypes.byref(p), fake, 16, 1, ctypes.byref(st), None) == -4
    # no fused launch for this shape (d, H >= 128 needed): OK without touching the device
    small = B.problem(64, 64, 8, 2, 64, "bf16", logits_given=True)
    assert lib.moe_fused_status(ctypes.byref(small), fake, 1 << 20, 0, ctypes.byref(st), None) == 0
    assert st.value == 0


def test_route_noalloc_host_checks(lib):
    # a problem whose routing scratch exceeds MOE_ROUTE_SCRATCH_BYTES is rejected before any device access
    p = B.problem(8192, 64, 1024, 16, 64, "bf16", logits_given=True)
    fake = ctypes.c_void_p(0x1000)
    assert lib.moe_route_noalloc(ctypes.byref(p), None, None, *([fake] * 7), None, None) == -4
    assert lib.moe_route_noalloc(ctypes.byref(p), None, None, None, *([fake] * 6), None, None) == -1


def test_kernel_times_without_profiled_forward(lib):
    n = ctypes.c_int32()
    assert lib.moe_set_profiling(0) == 0
    assert lib.moe_kernel_times(None, None, 0, ctypes.byref(n)) == -6


@pytest.mark.parametrize("name", W.CONFIG_ORDER)
def test_workspace_and_packed_sizes(lib, name):
    w = W.CONFIGS[name]
    p = B.problem(w.T, w.d, w.E, w.k, w.H, w.act, logits_given=w.router != "learned")
    R = w.T * w.k
    elem = {"f32": 4, "bf16": 2, "mxfp8": 1}[w.act]
    ws = B.workspace_bytes(p)
    # at least h and ye of R rows, and xe unless the fused bf16 FFN reads the
    # token rows in place (bf16 with d_model, d_hidden >= 128: no dispatched copy)
    gathers = w.act == "bf16" and w.d >= 128 and w.H >= 128
    # MXFP8 with d_model >= 256 keeps one code row per token instead of per routed row
    xe = 0 if gathers else (w.T if w.act == "mxfp8" and w.d >= 256 else R) * w.d * elem
    assert ws >= xe + R * w.H * elem + R * w.d * (4 if w.act == "f32" else 2)
    assert ws < xe + R * w.H * elem + R * w.d * 4 + 16 * R + (1 << 26)
    pw = B.packed_weight_bytes(p)
    want = 3 * w.E * w.d * w.H * elem
    if w.act == "mxfp8":
        want = want * 33 // 32          # one E8M0 byte per 32 elements
    assert want <= pw < want + 4 * 256


def test_backward_rejects_identity_nulls_and_small_workspaces(lib):
    n = ctypes.c_size_t()
    pm = _prob(act="mxfp8", d=128, H=128)
    assert lib.moe_backward_workspace_bytes(ctypes.byref(pm), ctypes.byref(n)) == 0
    pi = _prob(identity=True)
    assert lib.moe_backward_workspace_bytes(ctypes.byref(pi), ctypes.byref(n)) == -3
    p = _prob(logits_given=True)
    assert lib.moe_backward_workspace_bytes(ctypes.byref(p), ctypes.byref(n)) == 0
    bws = n.value
    assert bws >= p.T * p.top_k * (2 * p.d_hidden + p.d_model + p.d_hidden) * 2
    assert lib.moe_backward_weight_bytes(ctypes.byref(p), ctypes.byref(n)) == 0
    assert n.value >= p.n_experts * p.d_model * 2 * p.d_hidden * 2
    fws = B.workspace_bytes(p)
    fake = ctypes.c_void_p(0x1000)
    # p, dy, x, w_router, packed_w, packed_bwd, idx, gate, offsets, pos, fwd_ws, fwd_ws_bytes,
    # dx, dlogits, dw_gate, dw_up, dw_down, dw_router, ws, ws_bytes, stream
    args = [ctypes.byref(p), fake, fake, None, fake, fake, None, None, None, None, fake, fws,
            fake, fake, fake, fake, fake, None, fake, bws, None]
    # a bf16 block with d_model, d_hidden >= 128 keeps no dispatched rows in its
    # forward workspace, so the backward needs x even with given logits
    no_x = list(args)
    no_x[2] = None
    assert lib.moe_backward(*no_x) == -1
    bad_fwd = list(args)
    bad_fwd[11] = fws - 1
    assert lib.moe_backward(*bad_fwd) == -4
    bad_ws = list(args)
    bad_ws[19] = bws - 1
    assert lib.moe_backward(*bad_ws) == -4
    no_dy = list(args)
    no_dy[1] = None
    assert lib.moe_backward(*no_dy) == -1
    # learned router: x, w_router and dw_router are required
    pl = _prob()
    args_l = list(args)
    args_l[0] = ctypes.byref(pl)
    assert lib.moe_backward(*args_l) == -1
