"""Parity of the block backward (moe_backward) against the CPU oracle (marked gpu).

The oracle is fed the routing the GPU forward produced (for the learned
router, the float32 logits it computed; routing itself is checked bit-exact
by the forward tests) and differentiates its own forward of that routing.

Bars (normwise relative = max|got - ref| / max|ref|, per output): float32
1e-5; bf16 2e-2 (as the forward outputs); MXFP8 blocks, whose backward runs in
bf16 on the dequantised activations and the forward's MXFP8 weight values,
2e-2.  Two calls are bitwise equal.
"""
import numpy as np
import pytest
import torch

from oracle import moe_backward as BW
from oracle import moe_oracle as O
from oracle import mxfp8 as MX
from routing_dispatch_grouped_router_amd import binding as B
from routing_dispatch_grouped_router_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"f32": 1e-5, "bf16": 2e-2, "mxfp8": 2e-2}


def _f64(t):
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy().astype(np.float64)


def _check(name, got, ref, act):
    ref = np.asarray(ref, np.float64)
    scale = np.max(np.abs(ref))
    err = np.max(np.abs(got - ref))
    if scale == 0:
        assert err == 0, f"{name}: expected zeros, max |got| {err:.3e}"
        return
    assert err / scale <= TOL[act], f"{name}: normwise rel err {err / scale:.3e} > {TOL[act]}"


CASES = [
    W.Workload("bwd_f32_learned", T=333, d=192, E=12, k=3, H=128, act="f32", router="learned", seed=4001),
    W.Workload("bwd_f32_random", T=300, d=128, E=8, k=2, H=192, act="f32", router="random", seed=4002),
    W.Workload("bwd_f32_dense_E1", T=257, d=128, E=1, k=1, H=320, act="f32", router="random", seed=4003),
    W.Workload("bwd_bf16_learned", T=1000, d=256, E=8, k=4, H=192, act="bf16", router="learned", seed=4004),
    W.Workload("bwd_bf16_e32_random", T=777, d=384, E=32, k=4, H=320, act="bf16", router="random", seed=4005),
    W.Workload("bwd_bf16_zipf", T=1500, d=256, E=16, k=8, H=128, act="bf16", router="zipf", seed=4006),
    W.Workload("bwd_bf16_empty", T=200, d=128, E=8, k=2, H=128, act="bf16", router="random", seed=4007,
               empty_experts=(0, 3, 7)),
    W.Workload("bwd_bf16_k_eq_E", T=130, d=64, E=4, k=4, H=128, act="bf16", router="random", seed=4008),
    W.Workload("bwd_bf16_tk_lt_E", T=3, d=64, E=16, k=2, H=64, act="bf16", router="random", seed=4009),
    W.Workload("bwd_mx_random", T=600, d=256, E=16, k=4, H=256, act="mxfp8", router="random", seed=4010,
               outlier_frac=0.01),
    W.Workload("bwd_mx_learned", T=400, d=256, E=8, k=2, H=128, act="mxfp8", router="learned", seed=4011),
    W.Workload("bwd_mx_empty", T=70, d=128, E=8, k=2, H=128, act="mxfp8", router="random", seed=4012,
               empty_experts=(1, 6), outlier_frac=0.05),
    W.Workload("bwd_bf16_max_E_k", T=700, d=64, E=1024, k=16, H=64, act="bf16", router="random", seed=4013),
    W.Workload("bwd_f32_max_E_k_learned", T=300, d=64, E=1024, k=16, H=64, act="f32", router="learned",
               seed=4014),
]


def _run(w, keep=False):
    host = W.make_inputs(w)
    dev = {k: (None if v is None else v.to(DEV)) for k, v in host.items()}
    p = B.problem(w.T, w.d, w.E, w.k, w.H, w.act, logits_given=w.router != "learned", keep_gate_up=keep)
    packed = B.pack_weights(p, dev["w_gate"], dev["w_up"], dev["w_down"])
    packed_bwd = B.pack_weights_backward(p, dev["w_gate"], dev["w_up"], dev["w_down"])
    fwd = B.Forward(p, DEV)
    fwd(dev["x"], packed=packed, w_router=dev["w_router"], logits=dev["logits"])
    rng = np.random.default_rng(w.seed + 17)
    dy_host = torch.from_numpy(rng.standard_normal((w.T, w.d)).astype(np.float32)).to(B.storage_dtype(w.act))
    dy = dy_host.to(DEV)
    bwd = B.Backward(p, DEV)
    outs = []
    for _ in range(2):
        g = bwd(fwd, dy, packed, packed_bwd, x=dev["x"], w_router=dev["w_router"])
        torch.cuda.synchronize()
        outs.append({k: (None if v is None else v.clone()) for k, v in g.items()})
    return host, fwd, dy_host, outs


@pytest.mark.parametrize("w", CASES, ids=[c.name for c in CASES])
def test_backward_against_oracle(w):
    print(f"[backward] {w.describe()}", flush=True)
    host, fwd, dy_host, outs = _run(w)
    for k in outs[0]:
        if outs[0][k] is not None:
            assert torch.equal(outs[0][k], outs[1][k]), f"{k} differs between two calls"
    _against_oracle(w, host, fwd, dy_host, outs[0])


def _against_oracle(w, host, fwd, dy_host, g):
    logits = _f64(fwd.logits)
    wg, wu, wd = (W.as_f64(host[n]) for n in ("w_gate", "w_up", "w_down"))
    x = W.as_f64(host["x"])
    fo = O.forward(x, w.E, w.k, w.act, wg, wu, wd, logits=logits)
    assert np.array_equal(fo["idx"], fwd.idx.cpu().numpy()), "routing differs from the oracle's"
    wr = W.as_f64(host["w_router"]) if w.router == "learned" else None
    if w.act == "mxfp8":   # the forward's weight values: MXFP8 blocks along each GEMM's contraction axis
        q = [O.expert_weights(wg, wu, wd, e, "mxfp8") for e in range(w.E)]
        wg, wu, wd = (np.stack([t[i] for t in q]) for i in range(3))
    ref = BW.backward(x, W.as_f64(dy_host), fo, w.act, wg, wu, wd, w_router=wr)
    for name in ("dx", "dlogits", "dw_gate", "dw_up", "dw_down"):
        _check(name, _f64(g[name]), ref[name], w.act)
    if wr is not None:
        _check("dw_router", _f64(g["dw_router"]), ref["dw_router"], w.act)
    if w.E == 1:
        assert torch.count_nonzero(g["dlogits"]) == 0


# --------------------------------------------------------------------------- full size


class _LazyF64:
    """Per-expert float64 view of a stored weight stack, converted on access."""

    def __init__(self, t):
        self.t = t

    def __getitem__(self, e):
        return W.as_f64(self.t[e])


def _sample_tokens(T, seed=0, n=24):
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(8, T - 8), size=n - 16, replace=False)
    return np.unique(np.concatenate([np.arange(8), np.arange(T - 8, T), mid])).astype(np.int64)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["bf16_e8", "bf16_e128_random", "bf16_e64_zipf", "mxfp8_e128"])
def test_full_size_backward(name):
    """The backward at the benchmark's block sizes, run as bench.py runs it:
    dx and dlogits on sampled tokens, every token's router gradient summing to
    zero and vanishing off the selected experts, and one 32-wide block of
    hidden units of dW_gate, dW_up and dW_down for the first and the last
    non-empty expert, all against the oracle."""
    w = W.CONFIGS[name]
    print(f"[full backward] {w.describe()}", flush=True)
    host, fwd, dy_host, outs = _run(w)
    g = outs[0]
    idx = fwd.idx.cpu().numpy().astype(np.int64)
    gate = _f64(fwd.gate)
    pos = fwd.pos.cpu().numpy().astype(np.int64)
    offsets = fwd.offsets.cpu().numpy().astype(np.int64)
    dy = W.as_f64(dy_host)
    wr = W.as_f64(host["w_router"]) if w.router == "learned" else None
    lw = [_LazyF64(host[n]) for n in ("w_gate", "w_up", "w_down")]
    # every token: zero off the selected experts, rows summing to zero
    dl = _f64(g["dlogits"])
    mask = np.ones_like(dl, dtype=bool)
    np.put_along_axis(mask, idx, False, axis=1)
    assert np.all(dl[mask] == 0.0)
    assert np.max(np.abs(dl.sum(axis=1))) <= 1e-5 * max(1e-30, np.max(np.abs(dl)))
    # sampled tokens
    toks = _sample_tokens(w.T)
    x64 = W.as_f64(host["x"][torch.from_numpy(toks)])
    xs = np.zeros((w.T, w.d))
    xs[toks] = x64
    ref = BW.backward_tokens(xs, dy, idx, gate, toks, w.E, w.act, *lw, w_router=wr)
    _check("dx (sampled tokens)", _f64(g["dx"])[toks], ref["dx"], w.act)
    _check("dlogits (sampled tokens)", dl[toks], ref["dlogits"], w.act)
    # one block of hidden units of two experts' weight gradients
    counts = np.diff(offsets)
    live = np.nonzero(counts)[0]
    row_token = np.empty(w.R, np.int64)
    slot = np.empty(w.R, np.int64)
    row_token[pos.reshape(-1)] = np.repeat(np.arange(w.T), w.k)
    slot[pos.reshape(-1)] = np.tile(np.arange(w.k), w.T)
    rng = np.random.default_rng(7)
    for e in (int(live[0]), int(live[-1])):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        t = row_token[lo:hi]
        rows = W.as_f64(host["x"][torch.from_numpy(t)])
        if w.act == "mxfp8":
            rows = MX.fake_quantize(rows, axis=1)
        dye = BW.store(gate[t, slot[lo:hi]][:, None] * dy[t], w.act)
        wg, wu, wd = O.expert_weights(*lw, e, w.act)
        hb = int(rng.integers(0, w.H // 32)) * 32
        hc = np.arange(hb, hb + 32)
        c = BW.weight_grad_columns(rows, dye, wg, wu, wd, w.act, hc)
        _check(f"dw_gate[{e}][:, {hb}:+32]", _f64(g["dw_gate"][e][:, hb:hb + 32]), c["dw_gate"], w.act)
        _check(f"dw_up[{e}][:, {hb}:+32]", _f64(g["dw_up"][e][:, hb:hb + 32]), c["dw_up"], w.act)
        _check(f"dw_down[{e}][{hb}:+32]", _f64(g["dw_down"][e][hb:hb + 32]), c["dw_down"], w.act)


@pytest.mark.parametrize("cap", [0, 8], ids=["full_grid", "cap8"])
def test_backward_chain_wait_path(cap):
    """The bf16 backward runs dh, da | db and dxe as one fused launch whose
    dependent tiles wait on per-M-tile counters; forcing every dependent tile
    through the wait-and-restart path (and a capped grid) leaves every gradient
    bitwise unchanged."""
    w = W.Workload("bwd_chain", T=1200, d=512, E=8, k=2, H=384, act="bf16", router="learned", seed=3401)
    print(f"[backward chain wait path] cap={cap} {w.describe()}", flush=True)
    try:
        B.set_gemm_grid_cap(cap)
        _, _, _, normal = _run(w)
        B.set_test_flags(B.MOE_TEST_FFN_WAIT)
        _, _, _, waited = _run(w)
    finally:
        B.set_test_flags(0)
        B.set_gemm_grid_cap(0)
    for k in normal[0]:
        if normal[0][k] is not None:
            assert torch.equal(normal[0][k], waited[0][k]), f"{k} changed on the wait-and-restart path"


# --------------------------------------------------------------------------- kept pre-activations

KEEP_CASES = [c for c in CASES if c.act == "bf16" and c.d >= 128 and c.H >= 128]


def _kept_gate_up(fwd, w):
    """a | b as the forward stored them: the last region of its workspace,
    [T k][2H] bf16 (the workspace layout puts it after every other region)."""
    n = w.R * 2 * w.H * 2
    off = fwd.ws.numel() - (-(-n // 256) * 256)
    return fwd.ws[off:off + n].view(torch.bfloat16).view(w.R, 2 * w.H)


def _packed_gate_up_ref(host, fwd, w):
    """xe W_gate | xe W_up per expert-major row in float64, columns in the
    packed order (32 gate then 32 up hidden units per 64)."""
    pos = fwd.pos.cpu().numpy().astype(np.int64)
    offsets = fwd.offsets.cpu().numpy().astype(np.int64)
    row_token = np.empty(w.R, np.int64)
    row_token[pos.reshape(-1)] = np.repeat(np.arange(w.T), w.k)
    x = W.as_f64(host["x"])
    ref = np.zeros((w.R, 2 * w.H))
    for e in range(w.E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        xe = x[row_token[lo:hi]]
        a = xe @ W.as_f64(host["w_gate"][e])
        b = xe @ W.as_f64(host["w_up"][e])
        n = hi - lo
        ref[lo:hi] = np.stack([a.reshape(n, w.H // 32, 32), b.reshape(n, w.H // 32, 32)], axis=2).reshape(n, 2 * w.H)
    return ref


def _check_kept(w):
    host, fwd0, _, rec = _run(w)
    host, fwd1, _, kept = _run(w, keep=True)
    assert torch.equal(fwd0.y, fwd1.y), "keeping a | b changed the forward output"
    for k in rec[0]:
        if rec[0][k] is not None:
            assert torch.equal(rec[0][k], kept[0][k]), f"{k}: kept a | b and recompute differ"
    return host, fwd1


@pytest.mark.parametrize("w", KEEP_CASES, ids=[c.name for c in KEEP_CASES])
def test_backward_kept_gate_up(w):
    """MOE_KEEP_GATE_UP: the forward's fused FFN stores a | b (checked against
    xe W1 in float64, in the packed column order), the backward reads them
    instead of recomputing, and y and every gradient equal the recomputing
    path's bit for bit."""
    print(f"[backward kept a|b] {w.describe()}", flush=True)
    host, fwd = _check_kept(w)
    ab = _kept_gate_up(fwd, w).float().cpu().numpy().astype(np.float64)
    _check("stored a | b", ab, _packed_gate_up_ref(host, fwd, w), w.act)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["bf16_e8", "bf16_e128_random"])
def test_full_size_backward_kept_gate_up(name):
    """The same bitwise agreement at the 8-expert and 128-expert benchmark
    blocks (the latter with a partial last M tile in most experts)."""
    w = W.CONFIGS[name]
    print(f"[full backward kept a|b] {w.describe()}", flush=True)
    _check_kept(w)


MX_KEEP_CASES = [c for c in CASES if c.act == "mxfp8"]


@pytest.mark.parametrize("w", MX_KEEP_CASES, ids=[c.name for c in MX_KEEP_CASES])
def test_backward_kept_gate_up_mxfp8(w):
    """MOE_KEEP_GATE_UP on MXFP8 blocks: the MXFP8 GEMM1 stores its gate/up
    accumulators as bf16 a | b (checked against the MXFP8 values of xe and W1
    multiplied in float64), the forward output is unchanged, and the backward
    from the stored a | b meets the oracle's bars like the recomputing one."""
    print(f"[backward kept a|b mxfp8] {w.describe()}", flush=True)
    host, fwd0, _, _ = _run(w)
    host, fwd, dy_host, outs = _run(w, keep=True)
    assert torch.equal(fwd0.y, fwd.y), "keeping a | b changed the forward output"
    for k in outs[0]:
        if outs[0][k] is not None:
            assert torch.equal(outs[0][k], outs[1][k]), f"{k} differs between two calls"
    _against_oracle(w, host, fwd, dy_host, outs[0])
    # the stored a | b: MXFP8 token rows times the MXFP8 expert weights
    pos = fwd.pos.cpu().numpy().astype(np.int64)
    offsets = fwd.offsets.cpu().numpy().astype(np.int64)
    row_token = np.empty(w.R, np.int64)
    row_token[pos.reshape(-1)] = np.repeat(np.arange(w.T), w.k)
    xq = MX.fake_quantize(W.as_f64(host["x"]), axis=1)
    wg, wu, wd = (W.as_f64(host[n]) for n in ("w_gate", "w_up", "w_down"))
    ref = np.zeros((w.R, 2 * w.H))
    for e in range(w.E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        qg, qu, _ = O.expert_weights(wg, wu, wd, e, "mxfp8")
        xe = xq[row_token[lo:hi]]
        a, b, n = xe @ qg, xe @ qu, hi - lo
        ref[lo:hi] = np.stack([a.reshape(n, w.H // 32, 32), b.reshape(n, w.H // 32, 32)], axis=2).reshape(n, 2 * w.H)
    ab = _kept_gate_up(fwd, w).float().cpu().numpy().astype(np.float64)
    _check("stored a | b", ab, ref, "bf16")


@pytest.mark.parametrize("name", ["small_bf16_e8", "small_mxfp8"])
def test_kept_gate_up_host_sync(name):
    """moe_forward_host_sync keeps the same a | b as moe_forward (and the same y)."""
    w = W.get(name)
    print(f"[kept a|b host-sync] {w.describe()}", flush=True)
    host = W.make_inputs(w)
    dev = {k: (None if v is None else v.to(DEV)) for k, v in host.items()}
    p = B.problem(w.T, w.d, w.E, w.k, w.H, w.act, logits_given=w.router != "learned", keep_gate_up=True)
    packed = B.pack_weights(p, dev["w_gate"], dev["w_up"], dev["w_down"])
    outs = []
    for sync in (False, True):
        f = B.Forward(p, DEV, host_sync=sync)
        f(dev["x"], packed=packed, w_router=dev["w_router"], logits=dev["logits"])
        torch.cuda.synchronize()
        outs.append(f)
    assert torch.equal(outs[0].y, outs[1].y)
    assert torch.equal(_kept_gate_up(outs[0], w), _kept_gate_up(outs[1], w))
