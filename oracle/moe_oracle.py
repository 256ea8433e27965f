"""Plain CPU oracle of the routed MoE block forward.  TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import or call this module; the product path never does.  It shares no
code with the HIP library.

What it computes, in the order the report's pages describe the routed block
("Olmo-core 3: an open training stack for trillion-parameter MoE", section
"Why a big MoE is a systems problem": a router sends each token to a few
experts; section "Olmo-core 3's answer": rowwise dispatch writes each token row
straight into its expert's buffer, grouped GEMMs run the uneven per-expert
shapes without padding; "Supercharging Olmo-core ...", Abstract: routing
metadata stays on the device, dispatch and combine avoid a permutation):

1. router logits   L = x . W_r                         (learned router)
2. top-k selection ranked by logit, ties to the lower expert index,
   gates = softmax over all experts, renormalised over the selected k
3. counts[e], offsets = exclusive prefix sum, positions pos[t, j] = offsets[e]
   + number of earlier tokens routed to e (a stable counting sort by expert)
4. dispatch        xe[pos[t, j]] = x[t]            (MXFP8: quantised row)
5. expert FFN      ye = (silu(xe W_gate) * (xe W_up)) W_down, per expert
6. combine         y[t] = sum_j gate[t, j] * ye[pos[t, j]]

and, beside step 3, the router statistics (mean router probability per expert,
the Switch-style load-balancing scalar and the worst-case load imbalance).

The pages give no formula for the router, the gate or the expert FFN; the
readings taken (softmax-then-renormalise gates, SwiGLU experts, lowest-index
tie-break, stored precision of each intermediate) are the workload definitions
these kernels are built for and are listed with the design notes.

Arithmetic is float64 on exactly representable stored inputs; every value that
is *stored* in a lower precision (logits and gates fp32; h, ye, y in the
activation dtype) is rounded to that precision at the point it is stored.
Parity of the expert FFN and of y is unpinned except by the special cases the
tests check (E = 1 dense FFN, identity experts): the pages print no worked
numerical example.
"""
from __future__ import annotations

import numpy as np

from . import mxfp8

# ----------------------------------------------------------------------------- rounding


def round_f32(v) -> np.ndarray:
    """Round to the nearest float32 (ties to even) and return as float64."""
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_bf16(v) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (8 significant bits, ties to even).

    bfloat16 keeps the float32 exponent range, so a normal value f * 2**ex
    (f in [0.5, 1)) is quantised to multiples of 2**(ex - 8); below the
    smallest normal 2**-126 the quantum stays 2**-133.
    """
    v = np.asarray(v, dtype=np.float64)
    _, ex = np.frexp(v)
    qexp = np.maximum(ex - 8, -133)
    return np.ldexp(np.rint(np.ldexp(v, -qexp)), qexp)


def store(v, dtype: str) -> np.ndarray:
    """Values as held in memory of the given storage type ('f32', 'bf16' or 'mxfp8')."""
    if dtype == "f32":
        return round_f32(v)
    if dtype == "bf16":
        return round_bf16(v)
    if dtype == "mxfp8":
        return mxfp8.fake_quantize(v, axis=-1)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------- step 1


def router_logits(x, w_router) -> np.ndarray:
    """L = x . W_r in float64, stored as float32.  x [T, d], W_r [d, E]."""
    return round_f32(np.asarray(x, np.float64) @ np.asarray(w_router, np.float64))


# ----------------------------------------------------------------------------- step 2


def select_topk(logits, k: int) -> np.ndarray:
    """Indices of the k largest logits per token, ordered by (logit desc, index asc).

    A stable sort of -L keeps equal logits in ascending expert order, which is
    the lowest-index tie-break.  -0.0 and +0.0 compare equal.  Returns int32 [T, k].
    """
    L = np.asarray(logits, dtype=np.float64)
    order = np.argsort(-L, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def gates(logits, idx) -> np.ndarray:
    """Softmax over all E experts, then renormalised over the selected k, stored fp32."""
    L = np.asarray(logits, dtype=np.float64)
    z = L - L.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(p, np.asarray(idx, np.int64), axis=1)
    return round_f32(sel / sel.sum(axis=1, keepdims=True))


def route(logits, k: int):
    idx = select_topk(logits, k)
    return idx, gates(logits, idx)


# ----------------------------------------------------------------------------- step 3


def route_metadata(idx, n_experts: int):
    """counts [E], offsets [E+1], pos [T, k], row_token [T*k] (all int32).

    Rows of one expert are ordered by ascending token index and experts are
    laid out back to back with no padding.  pos is obtained from a stable sort
    of the token-major list of routed expert ids: equal ids keep token order.
    """
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    flat = idx.reshape(-1)
    counts = np.bincount(flat, minlength=n_experts).astype(np.int64)
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    order = np.argsort(flat, kind="stable")           # route ids in destination order
    pos = np.empty(T * k, dtype=np.int64)
    pos[order] = np.arange(T * k)
    row_token = (order // k).astype(np.int32)
    return (counts.astype(np.int32), offsets.astype(np.int32),
            pos.reshape(T, k).astype(np.int32), row_token)


def router_stats(logits, counts, k: int) -> dict:
    """Router statistics of one block, in float64.

    The report asks that requested route counts be inspected directly next to
    the Switch-style load-balancing scalar, a cross term of soft router scores
    and hard expert counts that can fall while the imbalance of the requested
    routes grows ("Supercharging Olmo-core ...", "Section 24: Conclusion", 24.3
    and Evidence 9 / Figure 45).  The pages print no formula for the scalar;
    the Switch-Transformer form is taken:

        P_e   = mean over tokens of softmax(L[t])[e]      (all E experts)
        f_e   = counts[e] / (T k)                          (share of routed rows)
        lbl   = E * sum_e f_e P_e                          (1 when both are uniform)
        imbalance = max_e counts[e] / (T k / E)            (worst-case load / mean load)

    Returns P [E], lbl, imbalance (float64).
    """
    L = np.asarray(logits, dtype=np.float64)
    T, E = L.shape
    z = np.exp(L - L.max(axis=1, keepdims=True))
    p = z / z.sum(axis=1, keepdims=True)
    P = p.mean(axis=0)
    c = np.asarray(counts, dtype=np.float64)
    f = c / (T * k)
    return {"P": P, "lbl": float(E * np.sum(f * P)), "imbalance": float(c.max() / (T * k / E))}


# ----------------------------------------------------------------------------- step 4


def dispatch(x, pos, act: str):
    """Expert-major buffer xe[pos[t, j]] = x[t].

    For 'f32' / 'bf16' the rows are copied unchanged (returned as float64 of
    the stored values).  For 'mxfp8' each row is quantised along d, and the
    function returns (codes uint8 [R, d], scales uint8 [R, d/32]).
    """
    x = np.asarray(x, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    T, k = pos.shape
    d = x.shape[1]
    src = np.repeat(np.arange(T), k)
    dst = pos.reshape(-1)
    if act in ("f32", "bf16"):
        xe = np.empty((T * k, d), dtype=np.float64)
        xe[dst] = x[src]
        return xe
    if act == "mxfp8":
        q, s = mxfp8.quantize(x, axis=1)
        xq = np.empty((T * k, d), dtype=np.uint8)
        xs = np.empty((T * k, d // mxfp8.BLOCK), dtype=np.uint8)
        xq[dst] = q[src]
        xs[dst] = s[src]
        return xq, xs
    raise ValueError(act)


# ----------------------------------------------------------------------------- step 5


def silu(z) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_weights(w_gate, w_up, w_down, e: int, act: str):
    """Float64 values of expert e's stored weights.

    'f32'/'bf16': the given (already representable) values.  'mxfp8': the
    weights as stored in MXFP8, blocks of 32 along each GEMM's contraction
    axis (d for W_gate/W_up [d, H], H for W_down [H, d]).
    """
    wg = np.asarray(w_gate[e], dtype=np.float64)
    wu = np.asarray(w_up[e], dtype=np.float64)
    wd = np.asarray(w_down[e], dtype=np.float64)
    if act == "mxfp8":
        wg = mxfp8.fake_quantize(wg, axis=0)
        wu = mxfp8.fake_quantize(wu, axis=0)
        wd = mxfp8.fake_quantize(wd, axis=0)
    return wg, wu, wd


def intermediate_dtypes(act: str):
    """(h storage, ye storage) for an activation type: f32 -> f32/f32,
    bf16 -> bf16/bf16, mxfp8 -> mxfp8 (blocks along H) / bf16."""
    return {"f32": ("f32", "f32"), "bf16": ("bf16", "bf16"), "mxfp8": ("mxfp8", "bf16")}[act]


def expert_ffn(rows, wg, wu, wd, act: str) -> np.ndarray:
    """SwiGLU FFN of one expert on its rows: ye = (silu(rows Wg) * (rows Wu)) Wd.

    rows [n, d] float64 (the dispatched values, dequantised for MXFP8),
    wg/wu [d, H], wd [H, d].  h and ye are stored in the activation's
    intermediate precision.
    """
    h_dt, ye_dt = intermediate_dtypes(act)
    a = rows @ wg
    b = rows @ wu
    h = store(silu(a) * b, h_dt)
    return store(h @ wd, ye_dt)


def experts(xe_values, offsets, w_gate, w_up, w_down, act: str) -> np.ndarray:
    """Apply each expert to its segment [offsets[e], offsets[e+1]) of the dispatched buffer."""
    xe_values = np.asarray(xe_values, dtype=np.float64)
    R, d = xe_values.shape
    ye = np.zeros((R, d), dtype=np.float64)
    E = len(offsets) - 1
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        wg, wu, wd = expert_weights(w_gate, w_up, w_down, e, act)
        ye[lo:hi] = expert_ffn(xe_values[lo:hi], wg, wu, wd, act)
    return ye


# ----------------------------------------------------------------------------- step 6


def combine(ye, gate, pos, out_dtype: str) -> np.ndarray:
    """y[t] = sum_j gate[t, j] * ye[pos[t, j]] (float64), stored in out_dtype."""
    ye = np.asarray(ye, dtype=np.float64)
    gate = np.asarray(gate, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    y = np.einsum("tk,tkd->td", gate, ye[pos])
    return store(y, out_dtype)


def out_dtype(act: str) -> str:
    return "f32" if act == "f32" else "bf16"


# ----------------------------------------------------------------------------- whole block


def forward(x, n_experts: int, k: int, act: str, w_gate, w_up, w_down,
            w_router=None, logits=None):
    """The whole block.  Exactly one of ``w_router`` / ``logits`` is given.

    Returns a dict with logits, idx, gate, counts, offsets, pos, row_token,
    xe (float64 values; for MXFP8 also xe_q / xe_s), ye and y.
    """
    x = np.asarray(x, dtype=np.float64)
    if logits is None:
        logits = router_logits(x, w_router)
    logits = np.asarray(logits, dtype=np.float64)
    idx, g = route(logits, k)
    counts, offsets, pos, row_token = route_metadata(idx, n_experts)
    out = dict(logits=logits, idx=idx, gate=g, counts=counts, offsets=offsets, pos=pos,
               row_token=row_token)
    if act == "mxfp8":
        xq, xs = dispatch(x, pos, act)
        out["xe_q"], out["xe_s"] = xq, xs
        xe_vals = mxfp8.dequantize(xq, xs, axis=1)
    else:
        xe_vals = dispatch(x, pos, act)
    out["xe"] = xe_vals
    out["ye"] = experts(xe_vals, offsets, w_gate, w_up, w_down, act)
    out["y"] = combine(out["ye"], g, pos, out_dtype(act))
    return out


def forward_tokens(x, idx, gate, tokens, act: str, w_gate, w_up, w_down) -> np.ndarray:
    """y for a subset of tokens only, given their routing.

    Each (token, slot) row passes through its expert independently of every
    other row, so y[t] depends only on x[t], the token's routing and the
    weights; this evaluates the same steps 4-6 for the listed tokens, the rows
    routed to one expert together (one expert's weights at a time).
    Returns [len(tokens), d] in the output storage type.
    """
    x = np.asarray(x, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    gate = np.asarray(gate, dtype=np.float64)
    tokens = np.asarray(tokens, dtype=np.int64)
    rows = x[tokens]
    if act == "mxfp8":
        rows = mxfp8.fake_quantize(rows, axis=1)
    k = idx.shape[1]
    sel = idx[tokens]                                   # [n, k] experts of the listed tokens
    ye = np.zeros((len(tokens), k, x.shape[1]), dtype=np.float64)
    for e in np.unique(sel):
        ii, jj = np.nonzero(sel == e)
        wg, wu, wd = expert_weights(w_gate, w_up, w_down, int(e), act)
        ye[ii, jj] = expert_ffn(rows[ii], wg, wu, wd, act)
    y = np.einsum("tk,tkd->td", gate[tokens], ye)
    return store(y, out_dtype(act))
