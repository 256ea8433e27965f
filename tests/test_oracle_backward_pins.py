"""Pins of the backward oracle to facts outside itself (no GPU).

* central finite differences of the unrounded forward (every gradient output,
  both router modes) on tiny blocks whose routing has a clear margin;
* torch autograd of an independently written float64 forward on a larger block;
* closed forms: one expert (the router gradient vanishes), k = E (the router
  gradient is the plain softmax backward, checked with scipy);
* storage: dx representable in bf16, weight and router gradients in float32,
  intermediates (dye) unrounded, and the rounded oracle within bf16 error of
  the exact one.
"""
import numpy as np
import pytest
import scipy.special
import torch

from oracle import moe_backward as BW
from oracle import moe_oracle as O


def _block(T, d, E, k, H, seed, learned):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    wg = rng.standard_normal((E, d, H)) / np.sqrt(d)
    wu = rng.standard_normal((E, d, H)) / np.sqrt(d)
    wd = rng.standard_normal((E, H, d)) / np.sqrt(H)
    dy = rng.standard_normal((T, d))
    if learned:
        wr = rng.standard_normal((d, E))
        return dict(x=x, wg=wg, wu=wu, wd=wd, dy=dy, wr=wr, logits=None)
    return dict(x=x, wg=wg, wu=wu, wd=wd, dy=dy, wr=None, logits=rng.standard_normal((T, E)) * 2)


def _margin(logits, k):
    s = -np.sort(-np.asarray(logits), axis=1)
    if k == s.shape[1]:
        return np.inf
    return float(np.min(s[:, k - 1] - s[:, k]))


def _loss(b, E, k, **over):
    p = {**b, **over}
    f = BW.forward_f64(p["x"], E, k, p["wg"], p["wu"], p["wd"], w_router=p["wr"], logits=p["logits"])
    return float(np.sum(f["y"] * b["dy"]))


def _fd(b, E, k, name, eps=1e-6):
    base = b[name]
    g = np.zeros_like(base)
    it = np.nditer(base, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        hi = base.copy()
        lo = base.copy()
        hi[i] += eps
        lo[i] -= eps
        g[i] = (_loss(b, E, k, **{name: hi}) - _loss(b, E, k, **{name: lo})) / (2 * eps)
    return g


def _analytic(b, E, k):
    f = BW.forward_f64(b["x"], E, k, b["wg"], b["wu"], b["wd"], w_router=b["wr"], logits=b["logits"])
    return BW.backward(b["x"], b["dy"], f, "f64", b["wg"], b["wu"], b["wd"], w_router=b["wr"]), f


@pytest.mark.parametrize("learned", [False, True])
@pytest.mark.parametrize("T,d,E,k,H,seed", [(5, 4, 4, 2, 3, 11), (6, 3, 3, 3, 2, 12), (4, 4, 5, 1, 3, 13)])
def test_backward_matches_finite_differences(T, d, E, k, H, seed, learned):
    b = _block(T, d, E, k, H, seed, learned)
    g, f = _analytic(b, E, k)
    assert _margin(f["logits"], k) > 1e-3, "routing too close to a tie for finite differences"
    pairs = [("x", "dx"), ("wg", "dw_gate"), ("wu", "dw_up"), ("wd", "dw_down")]
    pairs.append(("wr", "dw_router") if learned else ("logits", "dlogits"))
    for name, out in pairs:
        num = _fd(b, E, k, name)
        err = np.max(np.abs(num - g[out]))
        assert err <= 1e-6 * max(1.0, np.max(np.abs(num))), f"{out}: finite-difference error {err:.2e}"


def _torch_forward(x, wg, wu, wd, logits, k):
    """Independent float64 torch forward: per-token loop over the selected experts."""
    idx = torch.topk(logits.detach(), k, dim=1, sorted=True).indices   # no ties in these inputs
    sel = torch.gather(logits, 1, idx)
    g = torch.softmax(sel, dim=1)
    ys = []
    for t in range(x.shape[0]):
        acc = torch.zeros(x.shape[1], dtype=x.dtype)
        for j in range(k):
            e = int(idx[t, j])
            a = x[t] @ wg[e]
            u = x[t] @ wu[e]
            acc = acc + g[t, j] * ((torch.nn.functional.silu(a) * u) @ wd[e])
        ys.append(acc)
    return torch.stack(ys)


@pytest.mark.parametrize("learned", [False, True])
def test_backward_matches_torch_autograd(learned):
    T, d, E, k, H = 40, 16, 6, 3, 12
    b = _block(T, d, E, k, H, 21, learned)
    g, f = _analytic(b, E, k)
    tt = {n: torch.tensor(b[n], dtype=torch.float64, requires_grad=True) for n in ("x", "wg", "wu", "wd")}
    if learned:
        wr = torch.tensor(b["wr"], dtype=torch.float64, requires_grad=True)
        logits = tt["x"] @ wr
    else:
        logits = torch.tensor(b["logits"], dtype=torch.float64, requires_grad=True)
    y = _torch_forward(tt["x"], tt["wg"], tt["wu"], tt["wd"], logits, k)
    (y * torch.tensor(b["dy"])).sum().backward()
    for name, out in [("x", "dx"), ("wg", "dw_gate"), ("wu", "dw_up"), ("wd", "dw_down")]:
        np.testing.assert_allclose(g[out], tt[name].grad.numpy(), rtol=0, atol=1e-10)
    if learned:
        np.testing.assert_allclose(g["dw_router"], wr.grad.numpy(), rtol=0, atol=1e-10)
    else:
        np.testing.assert_allclose(g["dlogits"], logits.grad.numpy(), rtol=0, atol=1e-12)


def test_single_expert_router_gradient_vanishes():
    b = _block(9, 4, 1, 1, 3, 31, learned=True)
    g, _ = _analytic(b, 1, 1)
    assert np.all(g["dlogits"] == 0.0)
    assert np.all(g["dw_router"] == 0.0)


def test_all_experts_selected_is_softmax_backward():
    T, E = 7, 4
    b = _block(T, 4, E, E, 3, 41, learned=False)
    g, f = _analytic(b, E, E)
    # dgate[t, j] belongs to expert idx[t, j]; scatter to expert order
    dp = np.zeros((T, E))
    np.put_along_axis(dp, f["idx"].astype(np.int64), g["dgate"], axis=1)
    p = scipy.special.softmax(b["logits"], axis=1)
    want = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
    np.testing.assert_allclose(g["dlogits"], want, rtol=0, atol=1e-13)


def test_bf16_storage_points():
    T, d, E, k, H = 24, 16, 4, 2, 8
    b = _block(T, d, E, k, H, 51, learned=False)
    rb = {n: O.round_bf16(b[n]) for n in ("x", "wg", "wu", "wd", "dy")}
    fwd = O.forward(rb["x"], E, k, "bf16", rb["wg"], rb["wu"], rb["wd"], logits=O.round_f32(b["logits"]))
    g = BW.backward(rb["x"], rb["dy"], fwd, "bf16", rb["wg"], rb["wu"], rb["wd"])
    # outputs in their declared types; intermediates (dye, dgate) are not rounded
    assert np.array_equal(g["dx"], O.round_bf16(g["dx"]))
    for out in ("dw_gate", "dw_up", "dw_down", "dlogits"):
        assert np.array_equal(g[out], O.round_f32(g[out])), out
    assert np.array_equal(g["dye"], fwd["gate"].reshape(-1)[np.argsort(fwd["pos"].reshape(-1))][:, None]
                          * rb["dy"][fwd["row_token"]])
    # within bf16 error of the unrounded chain rule on the same routing
    exact = BW.backward(rb["x"], rb["dy"], fwd, "f64", rb["wg"], rb["wu"], rb["wd"])
    for out in ("dx", "dw_gate", "dw_up", "dw_down", "dlogits"):
        rel = np.max(np.abs(g[out] - exact[out])) / np.max(np.abs(exact[out]))
        assert rel < 3e-2, (out, rel)


@pytest.mark.parametrize("act,learned", [("f32", True), ("bf16", False), ("bf16", True), ("mxfp8", False)])
def test_sampled_helpers_equal_the_whole_block(act, learned):
    """backward_tokens and weight_grad_columns (used for large blocks) give the
    same values as the whole-block backward."""
    T, d, E, k, H = 30, 64, 4, 2, 64
    b = _block(T, d, E, k, H, 61, learned)
    rb = {n: (O.round_bf16(b[n]) if act != "f32" else O.round_f32(b[n])) for n in ("x", "wg", "wu", "wd", "dy")}
    wr = None
    if learned:
        wr = O.round_bf16(b["wr"]) if act != "f32" else O.round_f32(b["wr"])
        logits = O.router_logits(rb["x"], wr)
    else:
        logits = O.round_f32(b["logits"])
    fwd = O.forward(rb["x"], E, k, act, rb["wg"], rb["wu"], rb["wd"], logits=logits)
    q = [O.expert_weights(rb["wg"], rb["wu"], rb["wd"], e, act) for e in range(E)]
    wg, wu, wd = (np.stack([t[i] for t in q]) for i in range(3))
    g = BW.backward(rb["x"], rb["dy"], fwd, act, wg, wu, wd, w_router=wr)
    toks = np.array([0, 3, 17, 29])
    s = BW.backward_tokens(rb["x"], rb["dy"], fwd["idx"], fwd["gate"], toks, E, act, rb["wg"], rb["wu"], rb["wd"],
                           w_router=wr)
    np.testing.assert_array_equal(s["dx"], g["dx"][toks])
    np.testing.assert_array_equal(s["dlogits"], g["dlogits"][toks])
    off = fwd["offsets"]
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        hc = np.arange(32, 64)
        c = BW.weight_grad_columns(fwd["xe"][lo:hi], g["dye"][lo:hi], wg[e], wu[e], wd[e], act, hc)
        np.testing.assert_allclose(c["dw_gate"], g["dw_gate"][e][:, hc], rtol=1e-6, atol=1e-6)
        np.testing.assert_allclose(c["dw_up"], g["dw_up"][e][:, hc], rtol=1e-6, atol=1e-6)
        np.testing.assert_allclose(c["dw_down"], g["dw_down"][e][hc, :], rtol=1e-6, atol=1e-6)
