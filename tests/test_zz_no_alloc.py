"""moe_route_noalloc (routing without a workspace argument: its scratch lives in
a library-owned device array) against moe_route, through the C ABI (marked
gpu).

Two calls in a row on one device, the second with fewer tokens, each compared
with moe_route on the same inputs.  Both entry points run the same kernels, so
every output must match bit for bit (float outputs compared as bit patterns).
"""
import ctypes

import pytest
import torch

from routing_dispatch_grouped_router_amd import binding as B
from routing_dispatch_grouped_router_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
NAMES = ("logits", "idx", "gate", "counts", "offsets", "pos", "row_token", "router_stats")


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


def _compare_one(w, stats):
    host = W.make_inputs(w)
    p = B.problem(w.T, w.d, w.E, w.k, w.H, w.act, logits_given=w.router != "learned")
    x = host["x"].to(DEV)
    wr = None if host["w_router"] is None else host["w_router"].to(DEV)
    lg = None if host["logits"] is None else host["logits"].to(DEV)
    ref = B.route(p, x=x, w_router=wr, logits=lg, stats=stats)
    out = B.route_outputs(p, DEV, stats=stats)
    if lg is not None:
        out["logits"].copy_(lg)
    else:
        out["logits"].fill_(float("nan"))   # must be overwritten by the router logits
    for name in NAMES[1:]:
        if out[name] is not None:
            out[name].fill_(-7)              # every output must be overwritten
    B.route_noalloc(p, out, x=x, w_router=wr)
    torch.cuda.synchronize()
    print(f"route_noalloc vs route: {w.describe()} stats={stats}", flush=True)
    for name in NAMES:
        a, b = ref[name], out[name]
        if a is None:
            assert b is None, name
            continue
        assert torch.equal(_bits(a), _bits(b)), f"{w.name}: {name} differs from moe_route"
    assert int(out["counts"].sum().item()) == w.T * w.k


# bf16 learned router with E not a multiple of 8: the transposed router weights
# are part of the scratch; then given logits at the MXFP8 block's routing shape
# (32768 tokens, 128 experts, top-4) with the router statistics, whose partial
# sums are the largest part of the scratch.
LEARNED = W.Workload("noalloc_bf16_e20", T=5000, d=256, E=20, k=4, H=64, act="bf16", router="learned", seed=3001)
GIVEN = W.Workload("noalloc_e128_random", T=32768, d=128, E=128, k=4, H=128, act="bf16", router="random",
                   seed=3002)


@pytest.mark.parametrize("w,stats", [(LEARNED, True), (GIVEN, True), (GIVEN, False)],
                         ids=["bf16_learned_e20", "given_e128_stats", "given_e128"])
def test_noalloc_matches_route_two_calls(w, stats):
    _compare_one(w, stats)                    # first call on this device: sets the scratch up
    _compare_one(W.scaled(w, 1234), stats)    # second call, fewer tokens, same array


def test_noalloc_rejects_oversized_problem():
    # 8192 tokens x 1024 experts: the probability partials alone take 8 MiB > MOE_ROUTE_SCRATCH_BYTES
    p = B.problem(8192, 64, 1024, 16, 64, "bf16", logits_given=True)
    out = B.route_outputs(p, DEV, stats=True)
    st = B.lib().moe_route_noalloc(ctypes.byref(p), None, None, *(ctypes.c_void_p(out[n].data_ptr())
                                                                  for n in NAMES), None)
    assert st == -4
