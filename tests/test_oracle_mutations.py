"""Planted mistakes in the CPU oracle must be caught by its pins.

Each case monkeypatches one oracle function with a plausible bug (a dropped
term, a wrong sign or index, a swapped operand, an unstable tie-break) and
checks that at least one of the pin tests fails against it.  Everything runs on
the CPU; nothing here touches the HIP library.
"""
import numpy as np
import pytest

import tests.test_oracle_backward_pins as PB
import tests.test_oracle_pins as P
from oracle import moe_backward as BW
from oracle import moe_oracle as O
from oracle import mxfp8 as MX


def _fails(fn, *args, **kwargs):
    try:
        fn(*args, **kwargs)
    except AssertionError:
        return True
    return False


def _gates_not_renormalised(logits, idx):
    L = np.asarray(logits, np.float64)
    p = np.exp(L - L.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    return O.round_f32(np.take_along_axis(p, np.asarray(idx, np.int64), 1))


def _topk_unstable(logits, k):
    # ascending stable sort reversed: equal logits end up in descending index order
    L = np.asarray(logits, np.float64)
    return np.argsort(L, axis=1, kind="stable")[:, ::-1][:, :k].astype(np.int32)


def _ffn_swapped(rows, wg, wu, wd, act):
    h_dt, ye_dt = O.intermediate_dtypes(act)
    h = O.store(O.silu(rows @ wu) * (rows @ wg), h_dt)     # gate and up swapped
    return O.store(h @ wd, ye_dt)


def _ffn_no_silu(rows, wg, wu, wd, act):
    h_dt, ye_dt = O.intermediate_dtypes(act)
    h = O.store((rows @ wg) * (rows @ wu), h_dt)
    return O.store(h @ wd, ye_dt)


def _combine_ungated(ye, gate, pos, out_dtype):
    return O.store(np.asarray(ye, np.float64)[np.asarray(pos)].sum(1), out_dtype)


def _metadata_off_by_one(idx, n_experts):
    # segment start taken from the inclusive scan: every position shifted by its expert's count
    c, o, p, r = _orig_metadata(idx, n_experts)
    p_bad = (p + c[np.asarray(idx, np.int64)]) % int(o[-1])
    return c, o, p_bad.astype(np.int32), r


_orig_metadata = O.route_metadata


def _metadata_unstable(idx, n_experts):
    idx = np.asarray(idx, np.int64)
    T, k = idx.shape
    flat = idx.reshape(-1)
    counts = np.bincount(flat, minlength=n_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    order = np.lexsort((-(np.arange(T * k) // k), flat))   # descending token order within expert
    pos = np.empty(T * k, np.int64)
    pos[order] = np.arange(T * k)
    return (counts.astype(np.int32), offsets.astype(np.int32),
            pos.reshape(T, k).astype(np.int32), (order // k).astype(np.int32))


def _round_away(u):
    u = np.asarray(u, np.float64)
    a = np.abs(u)
    _, ex = np.frexp(a)
    qe = np.maximum(ex - 1, -6) - 3
    q = np.ldexp(np.floor(np.ldexp(a, -qe) + 0.5), qe)          # ties away from zero
    return np.copysign(np.minimum(q, 448.0), u)


def _shared_exp_ceil(amax):
    amax = np.asarray(amax, np.float64)
    se = np.ceil(np.log2(np.maximum(amax, 1e-300) / 448.0))
    return np.clip(np.where(amax == 0, -127, se), -127, 127).astype(np.int64)


def _decode_fnuz(codes):
    c = np.asarray(codes, np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8, -7), np.ldexp(1 + m / 8, e - 8))
    return s * np.where((c & 0x7F) == 0x7F, np.nan, mag)


def _stats_counts_over_tokens(logits, counts, k):
    # f_e = counts / T instead of counts / (T k): the scalar scales with k
    r = _orig_stats(logits, counts, k)
    T = np.asarray(logits).shape[0]
    E = np.asarray(logits).shape[1]
    r["lbl"] = float(E * np.sum(np.asarray(counts, np.float64) / T * r["P"]))
    return r


def _stats_topk_probabilities(logits, counts, k):
    # P from the renormalised top-k gates instead of the full softmax
    idx = O.select_topk(logits, k)
    g = O.gates(logits, idx)
    L = np.asarray(logits, np.float64)
    T, E = L.shape
    dense = np.zeros((T, E))
    np.put_along_axis(dense, np.asarray(idx, np.int64), g, axis=1)
    P = dense.mean(0)
    c = np.asarray(counts, np.float64)
    return {"P": P, "lbl": float(E * np.sum(c / (T * k) * P)), "imbalance": float(c.max() / (T * k / E))}


_orig_stats = O.router_stats
_orig_expert_weights = O.expert_weights
_orig_combine = O.combine

_orig_expert_backward = BW.expert_backward
_orig_router_backward = BW.router_backward
_orig_combine_backward = BW.combine_backward


def _silu_grad_sigmoid_only(z):
    return BW.sigmoid(z)


def _expert_bwd_swapped_wgrads(rows, dye_rows, wg, wu, wd, act):
    drows, dwg, dwu, dwd = _orig_expert_backward(rows, dye_rows, wg, wu, wd, act)
    return drows, dwu, dwg, dwd


def _expert_bwd_dxe_gate_only(rows, dye_rows, wg, wu, wd, act):
    # the up projection's share of dxe dropped
    a = rows @ wg
    b = rows @ wu
    dh = dye_rows @ wd.T
    da = dh * b * BW.silu_grad(a)
    _, dwg, dwu, dwd = _orig_expert_backward(rows, dye_rows, wg, wu, wd, act)
    return BW.store(da @ wg.T, act), dwg, dwu, dwd


def _router_bwd_uncentred(dgate, gate, idx, n_experts, act):
    dgate = np.asarray(dgate, np.float64)
    gate = np.asarray(gate, np.float64)
    idx = np.asarray(idx, np.int64)
    dL = np.zeros((idx.shape[0], n_experts))
    np.put_along_axis(dL, idx, gate * dgate, axis=1)
    return BW.store_f32(dL, act)


def _combine_bwd_ungated(dy, ye, gate, pos, act):
    return _orig_combine_backward(dy, ye, np.ones_like(np.asarray(gate, np.float64)), pos, act)


def _weights_blocked_along_n(w_gate, w_up, w_down, e, act):
    # MXFP8 weight blocks taken along the GEMM output axis instead of its contraction axis
    wg, wu, wd = (np.asarray(w[e], np.float64) for w in (w_gate, w_up, w_down))
    if act == "mxfp8":
        wg, wu, wd = (MX.fake_quantize(w, axis=1) for w in (wg, wu, wd))
    return wg, wu, wd


def _weights_of_next_expert(w_gate, w_up, w_down, e, act):
    # expert e's rows multiplied by expert e + 1's weights (an index shifted by one)
    return _orig_expert_weights(w_gate, w_up, w_down, (e + 1) % np.asarray(w_gate).shape[0], act)


def _combine_slots_reversed(ye, gate, pos, out_dtype):
    # gate j applied to the row of slot k - 1 - j
    return _orig_combine(ye, np.asarray(gate, np.float64)[:, ::-1], pos, out_dtype)


WEIGHT_PINS = [
    lambda gd: P.test_mxfp8_weights_blocked_along_contraction_axis(),
]

BACKWARD_PINS = [
    lambda gd: [PB.test_backward_matches_finite_differences(*c, learned) for c in
                [(5, 4, 4, 2, 3, 11), (4, 4, 5, 1, 3, 13)] for learned in (False, True)],
    lambda gd: [PB.test_backward_matches_torch_autograd(learned) for learned in (False, True)],
    lambda gd: PB.test_all_experts_selected_is_softmax_backward(),
]

ROUTING_PINS = [
    lambda gd: P.test_route_worked_example(gd),
    lambda gd: [P.test_topk_brute_force_with_ties(E, k) for E, k in [(3, 2), (4, 3), (5, 2)]],
    lambda gd: P.test_gates_special_cases(),
    lambda gd: [P.test_route_metadata_brute_force(T, E, k) for T, E, k in [(5, 3, 2), (40, 7, 3)]],
    lambda gd: P.test_forced_empty_experts_have_equal_offsets(),
]
EXPERT_PINS = [
    lambda gd: [P.test_single_expert_top1_is_dense_swiglu(a) for a in ("f32", "bf16")],
    lambda gd: P.test_identity_experts_round_trip(),
    lambda gd: [P.test_expert_relabelling_invariance(a) for a in ("f32", "bf16")],
    lambda gd: [P.test_routed_block_equals_dense_gate_matrix(a, t) for a, t in (("f32", 1e-6), ("bf16", 1e-2))],
]
STATS_PINS = [
    lambda gd: P.test_router_stats_hand_examples(),
    lambda gd: P.test_router_stats_uniform_and_invariants(),
    lambda gd: P.test_router_stats_scalar_can_fall_while_imbalance_stays(),
]
MX_PINS = [
    lambda gd: P.test_e4m3_golden_values(gd),
    lambda gd: P.test_e4m3_round_matches_exhaustive_search(),
    lambda gd: P.test_quantize_hand_blocks(),
    lambda gd: P.test_quantize_error_bound_and_blocks_independent(),
]

MUTATIONS = [
    ("gates not renormalised", O, "gates", _gates_not_renormalised, ROUTING_PINS),
    ("top-k ties to the higher index", O, "select_topk", _topk_unstable, ROUTING_PINS),
    ("positions from the inclusive scan", O, "route_metadata", _metadata_off_by_one, ROUTING_PINS),
    ("rows of an expert in reverse token order", O, "route_metadata", _metadata_unstable, ROUTING_PINS),
    ("gate and up projections swapped", O, "expert_ffn", _ffn_swapped, EXPERT_PINS),
    ("SiLU dropped", O, "expert_ffn", _ffn_no_silu, EXPERT_PINS),
    ("combine ignores gates", O, "combine", _combine_ungated, EXPERT_PINS),
    ("load share over tokens, not routed rows", O, "router_stats", _stats_counts_over_tokens, STATS_PINS),
    ("router probability from the top-k gates", O, "router_stats", _stats_topk_probabilities, STATS_PINS),
    ("E4M3 ties rounded away from zero", MX, "e4m3_round", _round_away, MX_PINS),
    ("ceil-based shared exponent", MX, "shared_exponent", _shared_exp_ceil, MX_PINS),
    ("FNUZ decode instead of OCP FN", MX, "e4m3_decode", _decode_fnuz, MX_PINS),
    ("MXFP8 weights blocked along the output axis", O, "expert_weights", _weights_blocked_along_n, WEIGHT_PINS),
    ("rows multiplied by the next expert's weights", O, "expert_weights", _weights_of_next_expert, EXPERT_PINS),
    ("gates applied to the slots in reverse", O, "combine", _combine_slots_reversed, EXPERT_PINS),
    ("SiLU gradient taken as the sigmoid", BW, "silu_grad", _silu_grad_sigmoid_only, BACKWARD_PINS),
    ("gate and up weight gradients swapped", BW, "expert_backward", _expert_bwd_swapped_wgrads, BACKWARD_PINS),
    ("dxe without the up projection's share", BW, "expert_backward", _expert_bwd_dxe_gate_only, BACKWARD_PINS),
    ("router gradient without the centring term", BW, "router_backward", _router_bwd_uncentred, BACKWARD_PINS),
    ("combine backward ignores gates", BW, "combine_backward", _combine_bwd_ungated, BACKWARD_PINS),
]


@pytest.mark.parametrize("name,mod,attr,bad,pins", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, golden_dir, name, mod, attr, bad, pins):
    monkeypatch.setattr(mod, attr, bad)
    if mod is MX and attr == "e4m3_decode":
        monkeypatch.setattr(MX, "_POS_VALUES", bad(np.arange(0x7F)))
    caught = [_fails(pin, golden_dir) for pin in pins]
    assert any(caught), f"no pin caught: {name}"
