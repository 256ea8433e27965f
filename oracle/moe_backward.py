"""Plain CPU oracle of the routed MoE block's backward pass.  TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import or call this module; the product path never does.  It shares no
code with the HIP library.

The report's pages describe the block's training step only by its parts: the
dispatch and combine are each other's transposes (a combine's backward moves
gradient rows to the experts as a dispatch does, a dispatch's backward sums
them back per token), the expert FFNs run as grouped GEMMs in both directions
(data gradients with the routed rows grouped by expert, weight gradients
contracting over each expert's rows), and block forwards are re-executed in
the backward ("Supercharging Olmo-core ...", "Section 24: Conclusion",
Evidence 7 (MXFP8 weight gradients: dequantise, then a bf16 grouped GEMM) and
Evidence 11 (recompute repeats dispatch and combine)).  No formula is printed;
the gradients below are the chain rule applied to the forward this package's
``moe_oracle`` defines:

    y[t]  = sum_j g[t, j] ye[pos[t, j]]
    ye[r] = h[r] Wd[e],  h = silu(a) * b,  a = xe[r] Wg[e],  b = xe[r] Wu[e]
    g[t, :] = softmax of the k selected logits of token t
              (the renormalised full softmax: the full denominator cancels)

    dgate[t, j] = dy[t] . ye[pos[t, j]]
    dye[pos[t, j]] = g[t, j] dy[t]
    dh = dye Wd^T;  da = dh * b * silu'(a);  db = dh * silu(a)
    dxe = da Wg^T + db Wu^T
    dWd[e] = sum over e's rows of h^T dye;  dWg[e] = xe^T da;  dWu[e] = xe^T db
    dL[t, e_j] = g[t, j] (dgate[t, j] - sum_i g[t, i] dgate[t, i]),  0 for
                 experts not selected (top-k selection is piecewise constant)
    dx[t] = sum_j dxe[pos[t, j]]  (+ dL[t] W_r^T for the learned router)
    dW_r = x^T dL

Precision: the pages fix no rounding points for the backward, so the chain
rule above runs in float64 without rounding any intermediate (dgate, dye, the
recomputed a and b, dh, da, db, dxe).  What enters as stored is what the
forward stored: the dispatched rows xe, h (rounded to the forward's h storage
type, as the forward oracle rounds it) and ye, and the inputs themselves.
Only the outputs are rounded, to their declared types: dx to the activation
type, dlogits and the weight gradients to float32.  With ``act='f64'`` no
rounding happens anywhere (used by the finite-difference pins).

MXFP8 blocks: the report found that MXFP8 weight gradients are fastest as a
dequantise followed by bf16 grouped GEMMs (Evidence 7); the backward here does
the whole block that way.  The saved activations are the forward's MXFP8
values (exact in bf16), the weights are the forward's MXFP8 weight values
(the caller passes them, e.g. from ``moe_oracle.expert_weights``), and dx is
stored in bf16.
"""
from __future__ import annotations

import numpy as np

from . import moe_oracle as F
from . import mxfp8


def store(v, act: str) -> np.ndarray:
    """Storage of the input gradient dx ('f64' keeps float64 exactly; MXFP8
    blocks store it in bf16)."""
    if act == "f64":
        return np.asarray(v, dtype=np.float64)
    return F.store(v, "bf16" if act == "mxfp8" else act)


def store_f32(v, act: str) -> np.ndarray:
    """float32 storage of the outputs that are float32 for every activation
    type (dlogits, weight gradients)."""
    if act == "f64":
        return np.asarray(v, dtype=np.float64)
    return F.round_f32(v)


def sigmoid(z) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def silu_grad(z) -> np.ndarray:
    """d silu(z) / dz = s (1 + z (1 - s)), s = sigmoid(z)."""
    s = sigmoid(z)
    return s * (1.0 + np.asarray(z, np.float64) * (1.0 - s))


def forward_f64(x, n_experts: int, k: int, w_gate, w_up, w_down, w_router=None, logits=None) -> dict:
    """The forward with no rounding at all (routing as ``moe_oracle.route``)."""
    x = np.asarray(x, dtype=np.float64)
    if logits is None:
        logits = x @ np.asarray(w_router, np.float64)
    logits = np.asarray(logits, dtype=np.float64)
    idx = F.select_topk(logits, k)
    sel = np.take_along_axis(logits, idx.astype(np.int64), axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    g = z / z.sum(axis=1, keepdims=True)
    counts, offsets, pos, row_token = F.route_metadata(idx, n_experts)
    T = x.shape[0]
    d = x.shape[1]
    xe = np.empty((T * k, d))
    xe[pos.reshape(-1)] = np.repeat(x, k, axis=0)
    ye = np.zeros_like(xe)
    for e in range(n_experts):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            a = xe[lo:hi] @ np.asarray(w_gate[e], np.float64)
            b = xe[lo:hi] @ np.asarray(w_up[e], np.float64)
            ye[lo:hi] = (F.silu(a) * b) @ np.asarray(w_down[e], np.float64)
    y = np.einsum("tk,tkd->td", g, ye[pos.astype(np.int64)])
    return dict(logits=logits, idx=idx, gate=g, counts=counts, offsets=offsets, pos=pos,
                row_token=row_token, xe=xe, ye=ye, y=y)


def combine_backward(dy, ye, gate, pos, act: str):
    """dgate[t, j] = dy[t] . ye[pos[t, j]] and dye[pos[t, j]] = gate[t, j] dy[t] (exact).
    ``act`` is unused: both are intermediates of the chain rule."""
    dy = np.asarray(dy, dtype=np.float64)
    ye = np.asarray(ye, dtype=np.float64)
    gate = np.asarray(gate, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    T, k = pos.shape
    dgate = np.einsum("td,tkd->tk", dy, ye[pos])
    dye = np.zeros((T * k, dy.shape[1]))
    dye[pos.reshape(-1)] = (gate[:, :, None] * dy[:, None, :]).reshape(T * k, -1)
    return dgate, dye


def router_backward(dgate, gate, idx, n_experts: int, act: str) -> np.ndarray:
    """dL [T, E] through the softmax over the selected logits; zero elsewhere
    (the dlogits output, stored float32)."""
    dgate = np.asarray(dgate, dtype=np.float64)
    gate = np.asarray(gate, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    inner = np.sum(gate * dgate, axis=1, keepdims=True)
    dsel = gate * (dgate - inner)
    dL = np.zeros((T, n_experts))
    np.put_along_axis(dL, idx, dsel, axis=1)
    return store_f32(dL, act)


def expert_backward(rows, dye_rows, wg, wu, wd, act: str):
    """Backward of one expert's SwiGLU FFN on its rows.

    Returns (drows, dwg, dwu, dwd): drows (the rows' share of dxe) exact,
    weight gradients float32.  a and b are recomputed exactly from the rows; h
    is the value the forward stored.
    """
    a = rows @ wg
    b = rows @ wu
    h = F.silu(a) * b
    if act != "f64":
        h = F.store(h, F.intermediate_dtypes(act)[0])   # as the forward stored it (MXFP8: blocks along H)
    dh = dye_rows @ wd.T
    da = dh * b * silu_grad(a)
    db = dh * F.silu(a)
    drows = da @ wg.T + db @ wu.T
    return drows, store_f32(rows.T @ da, act), store_f32(rows.T @ db, act), store_f32(h.T @ dye_rows, act)


def backward(x, dy, fwd: dict, act: str, w_gate, w_up, w_down, w_router=None) -> dict:
    """Gradients of sum(y * dy) for the block whose forward is ``fwd``.

    ``fwd`` holds (from ``moe_oracle.forward`` or ``forward_f64``) idx, gate,
    offsets, pos, xe and ye.  Returns dict(dx [T, d], dlogits [T, E], dw_gate /
    dw_up [E, d, H], dw_down [E, H, d], dw_router [d, E] or None, dgate, dye).
    """
    x = np.asarray(x, dtype=np.float64)
    idx, gate, offsets, pos = fwd["idx"], fwd["gate"], fwd["offsets"], np.asarray(fwd["pos"], np.int64)
    xe, ye = np.asarray(fwd["xe"], np.float64), np.asarray(fwd["ye"], np.float64)
    E = len(offsets) - 1
    T, k = pos.shape
    dgate, dye = combine_backward(dy, ye, gate, pos, act)
    dL = router_backward(dgate, gate, idx, E, act)
    d = x.shape[1]
    H = np.asarray(w_gate[0]).shape[1]
    dxe = np.zeros_like(xe)
    dwg = np.zeros((E, d, H))
    dwu = np.zeros((E, d, H))
    dwd = np.zeros((E, H, d))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        wg = np.asarray(w_gate[e], np.float64)
        wu = np.asarray(w_up[e], np.float64)
        wd = np.asarray(w_down[e], np.float64)
        dxe[lo:hi], dwg[e], dwu[e], dwd[e] = expert_backward(xe[lo:hi], dye[lo:hi], wg, wu, wd, act)
    dx = dxe[pos].sum(axis=1)
    dwr = None
    if w_router is not None:
        wr = np.asarray(w_router, np.float64)
        dx = dx + dL @ wr.T
        dwr = store_f32(x.T @ dL, act)
    return dict(dx=store(dx, act), dlogits=dL, dw_gate=dwg, dw_up=dwu, dw_down=dwd, dw_router=dwr,
                dgate=dgate, dye=dye)


# ----------------------------------------------------------------------------- sampled outputs (large blocks)


def backward_tokens(x, dy, idx, gate, tokens, n_experts: int, act: str, w_gate, w_up, w_down,
                    w_router=None) -> dict:
    """dx and dlogits of the listed tokens only, given the block's routing.

    Every routed row passes through its expert independently, so a token's
    gradient rows depend only on its own rows; this evaluates ``backward``'s
    definitions for those rows (expert weights indexed per expert, e.g. lazily
    converted stacks).  Returns dict(dx [n, d], dlogits [n, E], dgate [n, k]).
    """
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    gate = np.asarray(gate, dtype=np.float64)
    tokens = np.asarray(tokens, dtype=np.int64)
    k = idx.shape[1]
    rows = x[tokens]
    if act == "mxfp8":
        rows = mxfp8.fake_quantize(rows, axis=1)
    cache = {}
    dgate = np.zeros((len(tokens), k))
    drows = np.zeros((len(tokens), k, x.shape[1]))
    for i, t in enumerate(tokens):
        for j in range(k):
            e = int(idx[t, j])
            if e not in cache:
                cache[e] = F.expert_weights(w_gate, w_up, w_down, e, act)
            wg, wu, wd = cache[e]
            ye = F.expert_ffn(rows[i:i + 1], wg, wu, wd, act)[0]
            dgate[i, j] = np.dot(dy[t], ye)
            dye = gate[t, j] * dy[t]
            drows[i, j] = expert_backward(rows[i:i + 1], dye[None, :], wg, wu, wd, act)[0][0]
    dL = router_backward(dgate, gate[tokens], idx[tokens], n_experts, act)
    dx = drows.sum(axis=1)
    if w_router is not None:
        dx = dx + dL @ np.asarray(w_router, np.float64).T
    return dict(dx=store(dx, act), dlogits=dL, dgate=dgate)


def weight_grad_columns(rows, dye_rows, wg, wu, wd, act: str, hcols) -> dict:
    """Columns hcols of one expert's dW_gate and dW_up and rows hcols of its
    dW_down, from all of the expert's rows (rows: the dispatched values, dye_rows:
    the gated output gradients, in the expert's row order).  For MXFP8 blocks
    hcols must be whole 32-wide blocks of hidden units (h is quantised in
    blocks along H).  Equal to the same entries of ``expert_backward``.
    """
    rows = np.asarray(rows, np.float64)
    dye_rows = np.asarray(dye_rows, np.float64)
    hc = np.asarray(hcols, np.int64)
    a = rows @ wg[:, hc]
    b = rows @ wu[:, hc]
    h = F.silu(a) * b
    if act != "f64":
        h = F.store(h, F.intermediate_dtypes(act)[0])
    dh = dye_rows @ wd[hc, :].T
    da = dh * b * silu_grad(a)
    db = dh * F.silu(a)
    return dict(dw_gate=store_f32(rows.T @ da, act), dw_up=store_f32(rows.T @ db, act),
                dw_down=store_f32(h.T @ dye_rows, act))
