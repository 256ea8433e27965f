"""Failure reporting of the fused bf16 grouped GEMMs' bounded waits (marked gpu).

The forward expert FFN and the backward's data-gradient chain each run their
GEMMs in one persistent launch whose dependent tiles wait, for a bounded time,
on counters raised by the tiles that produce their rows.  A tile that stops
waiting must not write a plausible value: it writes NaN and raises an error
word that moe_fused_status reports.  The test hook MOE_TEST_FFN_GIVE_UP makes
every wait give up at once without looking at the counters (with
MOE_TEST_FFN_WAIT every dependent tile takes the wait path), so the failure
path runs with every kernel finishing normally.  A following call without the
hooks clears the error and is correct again.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from routing_dispatch_grouped_router_amd import binding as B
from routing_dispatch_grouped_router_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
FORCED = B.MOE_TEST_FFN_WAIT | B.MOE_TEST_FFN_GIVE_UP


@pytest.fixture
def flags():
    yield B.set_test_flags
    B.set_test_flags(0)
    B.set_gemm_grid_cap(0)


def _inputs(w, keep=False):
    host = W.make_inputs(w)
    dev = {k: (None if v is None else v.to(DEV)) for k, v in host.items()}
    p = B.problem(w.T, w.d, w.E, w.k, w.H, w.act, logits_given=w.router != "learned", keep_gate_up=keep)
    return host, dev, p


@pytest.mark.parametrize("cap", [0, 8], ids=["full_grid", "cap8"])
def test_forward_give_up_is_reported(cap, flags):
    w = W.Workload("giveup_fwd", T=1500, d=512, E=8, k=2, H=384, act="bf16", router="random", seed=3501)
    print(f"[fused give-up forward] cap={cap} {w.describe()}", flush=True)
    host, dev, p = _inputs(w)
    B.set_gemm_grid_cap(cap)
    packed = B.pack_weights(p, dev["w_gate"], dev["w_up"], dev["w_down"])
    f = B.Forward(p, DEV)
    flags(FORCED)
    f(dev["x"], packed=packed, logits=dev["logits"])
    assert B.fused_status(p, f.ws) == -6, "a wait that gave up was not reported"
    torch.cuda.synchronize()
    # every GEMM2 tile gave up: all of ye, hence all of y, is NaN (no finite wrong value)
    assert torch.isnan(f.y.float()).all(), "outputs of tiles that gave up are not NaN"
    flags(0)
    f(dev["x"], packed=packed, logits=dev["logits"])
    assert B.fused_status(p, f.ws) == 0, "the error word was not cleared by the next call"
    torch.cuda.synchronize()
    wg, wu, wd = (W.as_f64(host[n]) for n in ("w_gate", "w_up", "w_down"))
    ref = O.forward(W.as_f64(host["x"]), w.E, w.k, w.act, wg, wu, wd, logits=W.as_f64(host["logits"]))
    y = f.y.float().cpu().numpy().astype(np.float64)
    assert np.max(np.abs(y - ref["y"])) / np.max(np.abs(ref["y"])) <= 2e-2


def test_grouped_swiglu_give_up_is_reported(flags):
    w = W.Workload("giveup_gs", T=1000, d=256, E=16, k=4, H=256, act="bf16", router="zipf", seed=3502)
    print(f"[fused give-up grouped_swiglu] {w.describe()}", flush=True)
    _, dev, p = _inputs(w)
    packed = B.pack_weights(p, dev["w_gate"], dev["w_up"], dev["w_down"])
    ws = B.new_workspace(p, DEV)
    r = B.route(p, logits=dev["logits"], ws=ws)
    xe, _ = B.dispatch(p, dev["x"], r["pos"])
    flags(FORCED)
    ye = B.grouped_swiglu(p, xe, None, packed, r["offsets"], ws=ws)
    assert B.fused_status(p, ws) == -6
    torch.cuda.synchronize()
    assert torch.isnan(ye.float()).all()
    flags(0)
    ye = B.grouped_swiglu(p, xe, None, packed, r["offsets"], ws=ws)
    assert B.fused_status(p, ws) == 0
    torch.cuda.synchronize()
    assert torch.isfinite(ye.float()).all()


@pytest.mark.parametrize("keep", [False, True], ids=["recompute", "kept_gate_up"])
def test_backward_give_up_is_reported(keep, flags):
    w = W.Workload("giveup_bwd", T=1200, d=512, E=8, k=2, H=384, act="bf16", router="learned", seed=3503)
    print(f"[fused give-up backward] keep={keep} {w.describe()}", flush=True)
    _, dev, p = _inputs(w, keep)
    packed = B.pack_weights(p, dev["w_gate"], dev["w_up"], dev["w_down"])
    packed_bwd = B.pack_weights_backward(p, dev["w_gate"], dev["w_up"], dev["w_down"])
    fwd = B.Forward(p, DEV)
    fwd(dev["x"], packed=packed, w_router=dev["w_router"])
    assert B.fused_status(p, fwd.ws) == 0
    dy = torch.randn((w.T, w.d), generator=torch.Generator().manual_seed(7)).to(torch.bfloat16).to(DEV)
    bwd = B.Backward(p, DEV)
    flags(FORCED)
    g = bwd(fwd, dy, packed, packed_bwd, x=dev["x"], w_router=dev["w_router"])
    assert B.fused_status(p, bwd.ws, which=B.MOE_STATUS_BACKWARD) == -6
    torch.cuda.synchronize()
    # the phases that wait gave up (gate/up and input gradient; with kept a | b
    # the input gradient): dx holds NaN in every row
    assert torch.isnan(g["dx"].float()).any(dim=1).all()
    flags(0)
    g = bwd(fwd, dy, packed, packed_bwd, x=dev["x"], w_router=dev["w_router"])
    assert B.fused_status(p, bwd.ws, which=B.MOE_STATUS_BACKWARD) == 0
    torch.cuda.synchronize()
    assert torch.isfinite(g["dx"].float()).all()


def test_status_without_fused_launch():
    # MXFP8 and float32 blocks run no fused launch: nothing waits, the status is OK
    for act, d in (("mxfp8", 256), ("f32", 128)):
        p = B.problem(64, d, 8, 2, 128, act, logits_given=True)
        ws = B.new_workspace(p, DEV)
        assert B.fused_status(p, ws) == 0
