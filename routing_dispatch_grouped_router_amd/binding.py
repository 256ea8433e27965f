"""Thin ctypes binding of libmoe.so (C ABI in include/moe.h).

Argument marshalling only: every step of the block runs in the library's HIP
kernels.  torch provides device memory (output tensors are allocated with
torch on the input's device) and the stream (torch's current stream, so
torch.cuda events and synchronisation see the library's work).  Nothing here
falls back to a CPU or torch implementation: if the library is not built, or a
call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_F32, MOE_BF16, MOE_MXFP8 = 0, 1, 2
ACT = {"f32": MOE_F32, "bf16": MOE_BF16, "mxfp8": MOE_MXFP8}
MOE_LOGITS_GIVEN, MOE_IDENTITY_EXPERTS, MOE_KEEP_GATE_UP = 1, 2, 4

# every function the header declares, for the export check
EXPORTS = ["moe_version", "moe_status_string", "moe_workspace_bytes", "moe_packed_weight_bytes",
           "moe_pack_weights", "moe_route", "moe_dispatch", "moe_grouped_swiglu", "moe_combine",
           "moe_forward", "moe_forward_host_sync", "moe_set_profiling", "moe_kernel_times",
           "moe_set_gemm_grid_cap", "moe_backward_workspace_bytes", "moe_backward_weight_bytes",
           "moe_pack_weights_backward", "moe_backward", "moe_set_test_flags", "moe_route_noalloc",
           "moe_fused_status"]


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = lib().moe_status_string(status).decode()
        super().__init__(f"{fn} failed with status {status}: {msg}")


class Problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("d_hidden", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("flags", ctypes.c_int32)]

    @property
    def act(self) -> str:
        return {v: k for k, v in ACT.items()}[self.act_dtype]


def problem(T, d, E, k, H, act, logits_given=False, identity=False, keep_gate_up=False) -> Problem:
    flags = ((MOE_LOGITS_GIVEN if logits_given else 0) | (MOE_IDENTITY_EXPERTS if identity else 0)
             | (MOE_KEEP_GATE_UP if keep_gate_up else 0))
    return Problem(T, d, E, k, H, ACT[act], flags)


_LIB = None
_P = ctypes.c_void_p
_SZ = ctypes.c_size_t
_I32 = ctypes.c_int32


def lib():
    """Load libmoe.so; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                               "or python -m routing_dispatch_grouped_router_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        PP = ctypes.POINTER(Problem)
        L.moe_version.restype = ctypes.c_char_p
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [_I32]
        L.moe_workspace_bytes.argtypes = [PP, ctypes.POINTER(_SZ)]
        L.moe_packed_weight_bytes.argtypes = [PP, ctypes.POINTER(_SZ)]
        L.moe_pack_weights.argtypes = [PP, _P, _P, _P, _P, _P]
        L.moe_route.argtypes = [PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]
        L.moe_route_noalloc.argtypes = [PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
        L.moe_dispatch.argtypes = [PP, _P, _P, _P, _P, _P]
        L.moe_grouped_swiglu.argtypes = [PP, _P, _P, _P, _P, _P, _P, _SZ, _P]
        L.moe_combine.argtypes = [PP, _P, _P, _P, _P, _P]
        L.moe_forward.argtypes = [PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]
        L.moe_forward_host_sync.argtypes = [PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P, _P]
        L.moe_set_profiling.argtypes = [_I32]
        L.moe_set_gemm_grid_cap.argtypes = [_I32]
        L.moe_set_test_flags.argtypes = [_I32]
        L.moe_fused_status.argtypes = [PP, _P, _SZ, _I32, ctypes.POINTER(_I32), _P]
        L.moe_backward_workspace_bytes.argtypes = [PP, ctypes.POINTER(_SZ)]
        L.moe_backward_weight_bytes.argtypes = [PP, ctypes.POINTER(_SZ)]
        L.moe_pack_weights_backward.argtypes = [PP, _P, _P, _P, _P, _P]
        L.moe_backward.argtypes = [PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P, _P, _P, _P, _P, _P,
                                   _P, _SZ, _P]
        L.moe_kernel_times.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_float),
                                       _I32, ctypes.POINTER(_I32)]
        for name in EXPORTS:
            if name not in ("moe_version", "moe_status_string"):
                getattr(L, name).restype = _I32
        _LIB = L
    return _LIB


def _check(fn: str, status: int):
    if status != 0:
        raise MoeError(fn, status)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t) -> torch.device:
    return t.device


def storage_dtype(act: str) -> torch.dtype:
    return torch.float32 if act == "f32" else torch.bfloat16


def out_dtype(act: str) -> torch.dtype:
    return torch.float32 if act == "f32" else torch.bfloat16


def _expect(t, shape, dtype, name):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name}: expected {tuple(shape)} {dtype}, got {tuple(t.shape)} {t.dtype}")


# ----------------------------------------------------------------------------- host-only queries


def workspace_bytes(p: Problem) -> int:
    n = _SZ()
    _check("moe_workspace_bytes", lib().moe_workspace_bytes(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def packed_weight_bytes(p: Problem) -> int:
    n = _SZ()
    _check("moe_packed_weight_bytes", lib().moe_packed_weight_bytes(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def new_workspace(p: Problem, device) -> torch.Tensor:
    return torch.empty(workspace_bytes(p), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------------------- entry points


def pack_weights(p: Problem, w_gate, w_up, w_down, stream=None) -> torch.Tensor:
    dt = storage_dtype(p.act)
    E, d, H = p.n_experts, p.d_model, p.d_hidden
    _expect(w_gate, (E, d, H), dt, "w_gate")
    _expect(w_up, (E, d, H), dt, "w_up")
    _expect(w_down, (E, H, d), dt, "w_down")
    packed = torch.empty(packed_weight_bytes(p), dtype=torch.uint8, device=w_gate.device)
    _check("moe_pack_weights", lib().moe_pack_weights(ctypes.byref(p), _ptr(w_gate), _ptr(w_up),
                                                      _ptr(w_down), _ptr(packed), _stream(stream)))
    return packed


def route(p: Problem, x=None, w_router=None, logits=None, ws=None, stream=None, stats=False) -> dict:
    """Returns dict(logits, idx, gate, counts, offsets, pos, row_token) as device tensors,
    plus router_stats [E + 2] (mean router probability per expert, balance scalar,
    worst-case imbalance) when stats=True."""
    T, E, k, d = p.T, p.n_experts, p.top_k, p.d_model
    dev = (logits if logits is not None else x).device
    if p.flags & MOE_LOGITS_GIVEN:
        _expect(logits, (T, E), torch.float32, "logits")
    else:
        _expect(x, (T, d), storage_dtype(p.act), "x")
        _expect(w_router, (d, E), storage_dtype(p.act), "w_router")
        logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    out = dict(logits=logits,
               idx=torch.empty((T, k), dtype=torch.int32, device=dev),
               gate=torch.empty((T, k), dtype=torch.float32, device=dev),
               counts=torch.empty((E,), dtype=torch.int32, device=dev),
               offsets=torch.empty((E + 1,), dtype=torch.int32, device=dev),
               pos=torch.empty((T, k), dtype=torch.int32, device=dev),
               row_token=torch.empty((T * k,), dtype=torch.int32, device=dev),
               router_stats=torch.empty((E + 2,), dtype=torch.float32, device=dev) if stats else None)
    ws = new_workspace(p, dev) if ws is None else ws
    _check("moe_route", lib().moe_route(
        ctypes.byref(p), _ptr(x), _ptr(w_router), _ptr(logits), _ptr(out["idx"]), _ptr(out["gate"]),
        _ptr(out["counts"]), _ptr(out["offsets"]), _ptr(out["pos"]), _ptr(out["row_token"]),
        _ptr(out["router_stats"]), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def route_outputs(p: Problem, device, stats=False) -> dict:
    """Output tensors of route / route_noalloc for problem p (logits included)."""
    T, E, k = p.T, p.n_experts, p.top_k
    return dict(logits=torch.empty((T, E), dtype=torch.float32, device=device),
                idx=torch.empty((T, k), dtype=torch.int32, device=device),
                gate=torch.empty((T, k), dtype=torch.float32, device=device),
                counts=torch.empty((E,), dtype=torch.int32, device=device),
                offsets=torch.empty((E + 1,), dtype=torch.int32, device=device),
                pos=torch.empty((T, k), dtype=torch.int32, device=device),
                row_token=torch.empty((T * k,), dtype=torch.int32, device=device),
                router_stats=torch.empty((E + 2,), dtype=torch.float32, device=device) if stats else None)


def route_noalloc(p: Problem, out: dict, x=None, w_router=None, stream=None) -> dict:
    """moe_route_noalloc into the caller's tensors `out` (as route_outputs makes
    them; with MOE_LOGITS_GIVEN out["logits"] holds the input logits).  Neither
    this function nor the library allocates device memory."""
    T, E, k, d = p.T, p.n_experts, p.top_k, p.d_model
    _expect(out["logits"], (T, E), torch.float32, "logits")
    if not p.flags & MOE_LOGITS_GIVEN:
        _expect(x, (T, d), storage_dtype(p.act), "x")
        _expect(w_router, (d, E), storage_dtype(p.act), "w_router")
    for name, shape in (("idx", (T, k)), ("pos", (T, k)), ("counts", (E,)), ("offsets", (E + 1,)),
                        ("row_token", (T * k,))):
        _expect(out[name], shape, torch.int32, name)
    _expect(out["gate"], (T, k), torch.float32, "gate")
    if out.get("router_stats") is not None:
        _expect(out["router_stats"], (E + 2,), torch.float32, "router_stats")
    _check("moe_route_noalloc", lib().moe_route_noalloc(
        ctypes.byref(p), _ptr(x), _ptr(w_router), _ptr(out["logits"]), _ptr(out["idx"]), _ptr(out["gate"]),
        _ptr(out["counts"]), _ptr(out["offsets"]), _ptr(out["pos"]), _ptr(out["row_token"]),
        _ptr(out.get("router_stats")), _stream(stream)))
    return out


def dispatch(p: Problem, x, pos, stream=None):
    """Returns (xe, xe_scale); xe_scale is None unless MXFP8, else uint8
    [d/128, R, 4]: the four E8M0 scales of each 128-wide slice of a row."""
    T, d, k = p.T, p.d_model, p.top_k
    R = T * k
    _expect(x, (T, d), storage_dtype(p.act), "x")
    _expect(pos, (T, k), torch.int32, "pos")
    if p.act == "mxfp8":
        xe = torch.empty((R, d), dtype=torch.uint8, device=x.device)
        xs = torch.empty((d // 128, R, 4), dtype=torch.uint8, device=x.device)   # slice-major scales
    else:
        xe = torch.empty((R, d), dtype=storage_dtype(p.act), device=x.device)
        xs = None
    _check("moe_dispatch", lib().moe_dispatch(ctypes.byref(p), _ptr(x), _ptr(pos), _ptr(xe), _ptr(xs),
                                              _stream(stream)))
    return xe, xs


def grouped_swiglu(p: Problem, xe, xe_scale, packed, offsets, ws=None, stream=None):
    R, d = p.T * p.top_k, p.d_model
    _expect(offsets, (p.n_experts + 1,), torch.int32, "offsets")
    ye = torch.empty((R, d), dtype=out_dtype(p.act), device=xe.device)
    ws = new_workspace(p, xe.device) if ws is None else ws
    _check("moe_grouped_swiglu", lib().moe_grouped_swiglu(
        ctypes.byref(p), _ptr(xe), _ptr(xe_scale), _ptr(packed), _ptr(offsets), _ptr(ye), _ptr(ws),
        ws.numel(), _stream(stream)))
    return ye


def combine(p: Problem, ye, gate, pos, stream=None):
    T, d, k = p.T, p.d_model, p.top_k
    _expect(ye, (T * k, d), out_dtype(p.act), "ye")
    _expect(gate, (T, k), torch.float32, "gate")
    _expect(pos, (T, k), torch.int32, "pos")
    y = torch.empty((T, d), dtype=out_dtype(p.act), device=ye.device)
    _check("moe_combine", lib().moe_combine(ctypes.byref(p), _ptr(ye), _ptr(gate), _ptr(pos), _ptr(y),
                                            _stream(stream)))
    return y


class Forward:
    """Preallocated state for repeated moe_forward calls (fixed buffer addresses)."""

    def __init__(self, p: Problem, device, debug_outputs: bool = True, host_sync: bool = False,
                 stats: bool = False):
        """host_sync: call moe_forward_host_sync (counts copied to a pinned host
        buffer and waited for before the grouped GEMMs) instead of moe_forward.
        stats: also compute the router statistics into self.router_stats [E + 2]."""
        self.p = p
        self.host_sync = host_sync
        self.host_counts = (torch.empty((p.n_experts,), dtype=torch.int32, pin_memory=True)
                            if host_sync else None)
        T, E, k, d = p.T, p.n_experts, p.top_k, p.d_model
        self.ws = new_workspace(p, device)
        self.y = torch.empty((T, d), dtype=out_dtype(p.act), device=device)
        self.logits = torch.empty((T, E), dtype=torch.float32, device=device)
        self.debug = debug_outputs
        self.router_stats = (torch.empty((E + 2,), dtype=torch.float32, device=device) if stats else None)
        if debug_outputs:
            self.idx = torch.empty((T, k), dtype=torch.int32, device=device)
            self.gate = torch.empty((T, k), dtype=torch.float32, device=device)
            self.counts = torch.empty((E,), dtype=torch.int32, device=device)
            self.offsets = torch.empty((E + 1,), dtype=torch.int32, device=device)
            self.pos = torch.empty((T, k), dtype=torch.int32, device=device)
        else:
            self.idx = self.gate = self.counts = self.offsets = self.pos = None

    def __call__(self, x, packed=None, w_router=None, logits=None, stream=None):
        p = self.p
        _expect(x, (p.T, p.d_model), storage_dtype(p.act), "x")
        if p.flags & MOE_LOGITS_GIVEN:
            _expect(logits, (p.T, p.n_experts), torch.float32, "logits")
            if logits.data_ptr() != self.logits.data_ptr():
                self.logits.copy_(logits)
        else:
            _expect(w_router, (p.d_model, p.n_experts), storage_dtype(p.act), "w_router")
        args = (ctypes.byref(p), _ptr(x), _ptr(w_router), _ptr(self.logits), _ptr(packed), _ptr(self.y),
                _ptr(self.idx), _ptr(self.gate), _ptr(self.counts), _ptr(self.offsets), _ptr(self.pos),
                _ptr(self.router_stats), _ptr(self.ws), self.ws.numel(), _stream(stream))
        if self.host_sync:
            _check("moe_forward_host_sync", lib().moe_forward_host_sync(
                *args, ctypes.c_void_p(self.host_counts.data_ptr())))
        else:
            _check("moe_forward", lib().moe_forward(*args))
        return self.y


def forward(p: Problem, x, packed=None, w_router=None, logits=None, stream=None, host_sync=False,
            stats=False) -> dict:
    f = Forward(p, x.device, host_sync=host_sync, stats=stats)
    y = f(x, packed=packed, w_router=w_router, logits=logits, stream=stream)
    return dict(y=y, logits=f.logits, idx=f.idx, gate=f.gate, counts=f.counts, offsets=f.offsets,
                pos=f.pos, host_counts=f.host_counts, router_stats=f.router_stats)


def set_profiling(enable: bool):
    _check("moe_set_profiling", lib().moe_set_profiling(1 if enable else 0))


def backward_workspace_bytes(p: Problem) -> int:
    n = _SZ()
    _check("moe_backward_workspace_bytes", lib().moe_backward_workspace_bytes(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def backward_weight_bytes(p: Problem) -> int:
    n = _SZ()
    _check("moe_backward_weight_bytes", lib().moe_backward_weight_bytes(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def pack_weights_backward(p: Problem, w_gate, w_up, w_down, stream=None) -> torch.Tensor:
    """The backward weight cache (moe_pack_weights_backward)."""
    dt = storage_dtype(p.act)
    E, d, H = p.n_experts, p.d_model, p.d_hidden
    _expect(w_gate, (E, d, H), dt, "w_gate")
    _expect(w_up, (E, d, H), dt, "w_up")
    _expect(w_down, (E, H, d), dt, "w_down")
    out = torch.empty(backward_weight_bytes(p), dtype=torch.uint8, device=w_gate.device)
    _check("moe_pack_weights_backward", lib().moe_pack_weights_backward(
        ctypes.byref(p), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(out), _stream(stream)))
    return out


class Backward:
    """Preallocated gradients and workspace for moe_backward of a Forward's last call."""

    def __init__(self, p: Problem, device):
        self.p = p
        T, E, d, H = p.T, p.n_experts, p.d_model, p.d_hidden
        self.ws = torch.empty(backward_workspace_bytes(p), dtype=torch.uint8, device=device)
        self.dx = torch.empty((T, d), dtype=out_dtype(p.act), device=device)
        self.dlogits = torch.empty((T, E), dtype=torch.float32, device=device)
        self.dw_gate = torch.empty((E, d, H), dtype=torch.float32, device=device)
        self.dw_up = torch.empty((E, d, H), dtype=torch.float32, device=device)
        self.dw_down = torch.empty((E, H, d), dtype=torch.float32, device=device)
        self.dw_router = (None if p.flags & MOE_LOGITS_GIVEN
                          else torch.empty((d, E), dtype=torch.float32, device=device))

    def __call__(self, fwd: "Forward", dy, packed, packed_bwd, x=None, w_router=None, stream=None):
        p = self.p
        dt = storage_dtype(p.act)
        _expect(dy, (p.T, p.d_model), dt, "dy")
        if not p.flags & MOE_LOGITS_GIVEN:
            _expect(x, (p.T, p.d_model), dt, "x")
            _expect(w_router, (p.d_model, p.n_experts), dt, "w_router")
        elif x is not None:
            _expect(x, (p.T, p.d_model), dt, "x")
        _check("moe_backward", lib().moe_backward(
            ctypes.byref(p), _ptr(dy), _ptr(x), _ptr(w_router), _ptr(packed), _ptr(packed_bwd),
            _ptr(fwd.idx), _ptr(fwd.gate), _ptr(fwd.offsets), _ptr(fwd.pos), _ptr(fwd.ws), fwd.ws.numel(),
            _ptr(self.dx), _ptr(self.dlogits), _ptr(self.dw_gate), _ptr(self.dw_up), _ptr(self.dw_down),
            _ptr(self.dw_router), _ptr(self.ws), self.ws.numel(), _stream(stream)))
        return dict(dx=self.dx, dlogits=self.dlogits, dw_gate=self.dw_gate, dw_up=self.dw_up,
                    dw_down=self.dw_down, dw_router=self.dw_router)


def set_gemm_grid_cap(cap: int):
    """Cap the grouped GEMMs' persistent grid at `cap` workgroups (multiple of 8, <= 256; 0 = no cap)."""
    _check("moe_set_gemm_grid_cap", lib().moe_set_gemm_grid_cap(int(cap)))


MOE_TEST_FFN_WAIT, MOE_TEST_FFN_GIVE_UP = 1, 2
MOE_STATUS_FORWARD, MOE_STATUS_BACKWARD = 0, 1


def set_test_flags(flags: int):
    """Test hooks of the fused bf16 grouped GEMMs (MOE_TEST_FFN_WAIT: every dependent tile waits
    for its rows before starting, the path taken when they are not yet done; MOE_TEST_FFN_GIVE_UP:
    every such wait ends at once as if its bound had been reached); 0 clears them."""
    _check("moe_set_test_flags", lib().moe_set_test_flags(int(flags)))


def fused_status(p: Problem, ws, which=MOE_STATUS_FORWARD, stream=None) -> int:
    """MOE_OK (0) or MOE_ERR_STATE (-6) from the error word of the last fused grouped-GEMM launch
    on workspace ws (synchronises on the stream)."""
    st = _I32()
    _check("moe_fused_status", lib().moe_fused_status(ctypes.byref(p), _ptr(ws), ws.numel(), int(which),
                                                      ctypes.byref(st), _stream(stream)))
    return st.value


def kernel_times() -> list[tuple[str, float]]:
    """(stage name, milliseconds) of the last profiled moe_forward (synchronises on it)."""
    names = (ctypes.c_char_p * 16)()
    ms = (ctypes.c_float * 16)()
    n = _I32()
    _check("moe_kernel_times", lib().moe_kernel_times(names, ms, 16, ctypes.byref(n)))
    return [(names[i].decode(), float(ms[i])) for i in range(n.value)]


def version() -> str:
    return lib().moe_version().decode()
