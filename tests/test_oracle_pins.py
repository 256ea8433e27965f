"""Pins of the CPU oracle to facts outside itself (no GPU).

Each test checks the oracle against something it does not compute itself:
the OCP MX v1.0 E4M3 table, the 33/32 payload ratio printed in the report
(Section 24: Conclusion, Evidence 10), exhaustive search over all codes,
brute-force loops on tiny inputs, textbook/library special cases (scipy
softmax, torch SiLU dense FFN), and invariants of the routing definition.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

from oracle import moe_oracle as O
from oracle import mxfp8 as MX

# ----------------------------------------------------------------------------- MXFP8 format


def _read_table(path):
    rows = []
    for line in open(path):
        line = line.split("#")[0].strip()
        if line:
            c, v = line.split()
            rows.append((int(c, 16), float(v)))
    return rows


def test_e4m3_golden_values(golden_dir):
    for code, val in _read_table(os.path.join(golden_dir, "e4m3_ocp.txt")):
        got = MX.e4m3_decode(code)
        if math.isnan(val):
            assert math.isnan(got), hex(code)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)


def test_e4m3_exhaustive_structure():
    vals = MX.e4m3_decode(np.arange(256))
    nan = np.isnan(vals)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    pos = vals[:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes must increase strictly"
    assert np.array_equal(vals[0x80:0xFF], -pos), "negative codes mirror positive ones"
    assert pos.max() == 448.0 and pos[1] == 2.0 ** -9
    # every finite value is a multiple of 2^-9 with at most 4 significant bits
    assert np.all(np.ldexp(pos, 9) == np.rint(np.ldexp(pos, 9)))


def _brute_round(u, table):
    """Nearest finite E4M3 value by exhaustive search; ties to the even code; saturate."""
    a = abs(u)
    if a >= 448.0:
        return math.copysign(448.0, u)
    diffs = np.abs(table - a)
    best = np.flatnonzero(diffs == diffs.min())
    if len(best) > 1:
        best = [c for c in best if c % 2 == 0]
    return math.copysign(float(table[best[0]]), u)


def test_e4m3_round_matches_exhaustive_search():
    table = MX.e4m3_decode(np.arange(0x7F))
    rng = np.random.default_rng(0)
    mids = (table[1:] + table[:-1]) / 2                      # exact ties
    samples = np.concatenate([
        table, -table, mids, -mids,
        rng.uniform(-500, 500, 3000),
        rng.uniform(-0.05, 0.05, 3000),
        np.ldexp(rng.uniform(-1, 1, 3000), rng.integers(-12, 10, 3000)),
        [448.0, 449.0, 463.99, 464.0, 470.0, 1e6, -1e6, 2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11],
    ])
    got = MX.e4m3_round(samples)
    want = np.array([_brute_round(u, table) for u in samples])
    assert np.array_equal(got, want)


def test_e4m3_encode_round_trips_every_code():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    vals = MX.e4m3_decode(codes)
    assert np.array_equal(MX.e4m3_encode(vals), codes)


def test_quantize_hand_blocks():
    # all-zero block -> smallest scale 2^-127 (code 0), zero elements
    q, s = MX.quantize(np.zeros((1, 32)))
    assert s.tolist() == [[0]] and q.tolist() == [[0] * 32]
    # amax 448 -> shared exponent 0 (code 127); 1.0625 and 1.1875 are exact
    # E4M3 half-way points and round to even (1.0 / 1.25); -3 -> 0xC4
    blk = np.zeros(32)
    blk[:4] = [448.0, 1.0625, 1.1875, -3.0]
    q, s = MX.quantize(blk[None])
    assert s.tolist() == [[127]]
    assert q[0, :4].tolist() == [0x7E, 0x38, 0x3A, 0xC4]
    # same block times 2^5 -> same codes, scale code 132
    q2, s2 = MX.quantize(blk[None] * 32)
    assert s2.tolist() == [[132]] and np.array_equal(q2, q)
    # amax 500: floor(log2 500) = 8 -> scale 2^0; 500 saturates to 448
    blk = np.full(32, 1.0)
    blk[7] = 500.0
    q, s = MX.quantize(blk[None])
    assert s.tolist() == [[127]] and q[0, 7] == 0x7E and q[0, 0] == 0x38
    # a tiny negative value that rounds to zero keeps its sign
    blk = np.zeros(32)
    blk[0], blk[1] = 448.0, -2.0 ** -12
    q, _ = MX.quantize(blk[None])
    assert q[0, 1] == 0x80


def test_quantize_error_bound_and_blocks_independent():
    rng = np.random.default_rng(1)
    v = rng.standard_normal((64, 256)) * np.exp(rng.uniform(-8, 8, (64, 1)))
    v[3, 40] *= 64
    deq = MX.fake_quantize(v, axis=1)
    blocks = v.reshape(64, 8, 32)
    amax = np.abs(blocks).max(-1, keepdims=True)
    scale = np.ldexp(1.0, np.floor(np.log2(amax)).astype(int) - 8)
    # half a quantum of the element's own binade (relative 2^-4), or 2^-10 * scale in
    # the subnormal range, or the excess over 448 * scale where the element saturates
    # (amax / scale lies in [256, 512), so elements above 448 * scale clamp)
    err = np.abs(deq.reshape(64, 8, 32) - blocks)
    bound = np.maximum.reduce([np.abs(blocks) * 2.0 ** -4, scale * 2.0 ** -10 + 0 * blocks,
                               np.abs(blocks) - 448.0 * scale])
    assert np.all(err <= bound)
    sat = np.abs(blocks) > 448.0 * scale
    assert sat.any() and np.all(np.abs(deq.reshape(64, 8, 32))[sat] == (448.0 * scale + 0 * blocks)[sat])
    # quantising one block does not depend on the others
    deq2 = MX.fake_quantize(v[:, 32:64], axis=1)
    assert np.array_equal(deq2, deq[:, 32:64])


def test_mxfp8_payload_is_33_over_32(golden_dir):
    lines = dict(l.split() for l in open(os.path.join(golden_dir, "mxfp8_payload.txt"))
                 if l.strip() and not l.startswith("#"))
    want = Fraction(lines["mxfp8_bytes_per_value"])
    v = np.random.default_rng(2).standard_normal((7, 2048))
    q, s = MX.quantize(v, axis=1)
    assert Fraction(q.nbytes + s.nbytes, v.size) == want
    assert Fraction(lines["bf16_bytes_per_value"]) == 2


# ----------------------------------------------------------------------------- rounding


def test_round_bf16_matches_torch_on_fp32_values():
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        np.ldexp(rng.uniform(-1, 1, 5000), rng.integers(-140, 120, 5000)).astype(np.float32)])
    # add exact bf16 half-way points
    base = torch.from_numpy(v[:2000]).to(torch.bfloat16).float().numpy().astype(np.float64)
    _, ex = np.frexp(base)
    ties = (base + np.ldexp(1.0, ex - 9)).astype(np.float32)
    v = np.concatenate([v, ties])
    want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_bf16(v.astype(np.float64))
    assert np.array_equal(got, want)


# ----------------------------------------------------------------------------- routing


def _eval_logits(exprs):
    out = []
    for row in exprs:
        out.append([float(np.float32(eval(e, {"__builtins__": {}, "log": math.log}))) for e in row])
    return np.array(out, dtype=np.float32).astype(np.float64)


def test_route_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "route_worked.json")))
    L = _eval_logits(g["logits_exprs"])
    idx, gate = O.route(L, g["k"])
    assert idx.tolist() == g["idx"]
    want_gate = np.array([[float(Fraction(f)) for f in r] for r in g["gate"]])
    assert np.max(np.abs(gate - want_gate)) < 1e-6
    counts, offsets, pos, row_token = O.route_metadata(idx, g["E"])
    assert counts.tolist() == g["counts"]
    assert offsets.tolist() == g["offsets"]
    assert pos.tolist() == g["pos"]
    assert row_token.tolist() == g["row_token"]


def _brute_topk(row, k):
    """Exhaustive search over ordered k-tuples of distinct experts: the tuple whose
    (logit, -index) key sequence is lexicographically largest."""
    best, best_key = None, None
    for perm in itertools.permutations(range(len(row)), k):
        key = [(row[e], -e) for e in perm]
        if best_key is None or key > best_key:
            best, best_key = perm, key
    return list(best)


@pytest.mark.parametrize("E,k", [(1, 1), (3, 2), (4, 1), (4, 3), (5, 5), (5, 2)])
def test_topk_brute_force_with_ties(E, k):
    rng = np.random.default_rng(10 * E + k)
    L = rng.integers(-2, 3, size=(8, E)).astype(np.float64)
    L[L == 0] = np.where(rng.random((L == 0).sum()) < 0.5, -0.0, 0.0)   # signed zeros tie
    L[0] = rng.standard_normal(E)
    idx = O.select_topk(L, k)
    for t in range(L.shape[0]):
        assert idx[t].tolist() == _brute_topk([float(v) + 0.0 for v in L[t]], k)


def test_topk_properties_large():
    rng = np.random.default_rng(4)
    T, E, k = 500, 64, 8
    L = rng.integers(0, 4, size=(T, E)).astype(np.float64)
    idx = O.select_topk(L, k)
    for t in range(T):
        sel = set(idx[t].tolist())
        assert len(sel) == k
        uns = [u for u in range(E) if u not in sel]
        for s in sel:
            for u in uns:
                assert L[t, s] > L[t, u] or (L[t, s] == L[t, u] and s < u)
        for a, b in zip(idx[t][:-1], idx[t][1:]):
            assert L[t, a] > L[t, b] or (L[t, a] == L[t, b] and a < b)


def test_gates_special_cases():
    rng = np.random.default_rng(5)
    L = rng.standard_normal((50, 6)).astype(np.float32).astype(np.float64)
    # k = E: the textbook softmax over all experts, in descending-logit order
    idx, g = O.route(L, 6)
    sm = scipy.special.softmax(L, axis=1)
    assert np.max(np.abs(g - np.take_along_axis(sm, idx.astype(np.int64), 1))) < 1e-7
    # k = 1: the single gate is exactly 1
    _, g1 = O.route(L, 1)
    assert np.all(g1 == 1.0)
    # renormalised gates sum to one and are non-increasing
    _, g3 = O.route(L, 3)
    assert np.max(np.abs(g3.sum(1) - 1)) < 1e-6
    assert np.all(np.diff(g3, axis=1) <= 0)
    # shifting all logits of a token leaves selection and gates unchanged
    idx4, g4 = O.route(L, 3)
    idx5, g5 = O.route(L + 0.5, 3)
    assert np.array_equal(idx4, idx5) and np.max(np.abs(g4 - g5)) < 1e-6


def _brute_positions(idx, E):
    T, k = len(idx), len(idx[0])
    counts = [0] * E
    for t in range(T):
        for j in range(k):
            counts[idx[t][j]] += 1
    offsets = [0]
    for e in range(E):
        offsets.append(offsets[-1] + counts[e])
    pos = [[0] * k for _ in range(T)]
    for t in range(T):
        for j in range(k):
            e = idx[t][j]
            earlier = sum(1 for tp in range(t) if e in list(idx[tp]))
            pos[t][j] = offsets[e] + earlier
    return counts, offsets, pos


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (5, 3, 2), (8, 4, 4), (40, 7, 3), (3, 16, 2)])
def test_route_metadata_brute_force(T, E, k):
    rng = np.random.default_rng(T * 100 + E)
    L = rng.standard_normal((T, E))
    idx = O.select_topk(L, k)
    counts, offsets, pos, row_token = O.route_metadata(idx, E)
    bc, bo, bp = _brute_positions(idx.tolist(), E)
    assert counts.tolist() == bc and offsets.tolist() == bo and pos.tolist() == bp
    assert sum(bc) == T * k
    assert sorted(pos.reshape(-1).tolist()) == list(range(T * k))
    for t in range(T):
        for j in range(k):
            assert row_token[pos[t, j]] == t


def test_forced_empty_experts_have_equal_offsets():
    rng = np.random.default_rng(6)
    L = rng.standard_normal((100, 8))
    L[:, [2, 5]] = -1e4
    idx = O.select_topk(L, 3)
    counts, offsets, _, _ = O.route_metadata(idx, 8)
    assert counts[2] == 0 and counts[5] == 0
    assert offsets[2] == offsets[3] and offsets[5] == offsets[6]
    assert offsets[-1] == 300


# ----------------------------------------------------------------------------- dispatch


def test_dispatch_rows_bitwise():
    rng = np.random.default_rng(7)
    T, d, E, k = 37, 64, 5, 2
    x = O.round_bf16(rng.standard_normal((T, d)))
    idx = O.select_topk(rng.standard_normal((T, E)), k)
    _, _, pos, row_token = O.route_metadata(idx, E)
    xe = O.dispatch(x, pos, "bf16")
    for t in range(T):
        for j in range(k):
            assert np.array_equal(xe[pos[t, j]], x[t])
    assert np.array_equal(xe, x[row_token])
    xq, xs = O.dispatch(x, pos, "mxfp8")
    q, s = MX.quantize(x, axis=1)
    assert np.array_equal(xq, q[row_token]) and np.array_equal(xs, s[row_token])
    assert xs.shape == (T * k, d // 32)


# ----------------------------------------------------------------------------- experts / combine


def _torch_dense_swiglu(x, wg, wu, wd):
    xt, g, u, dn = (torch.from_numpy(np.asarray(a, np.float64)) for a in (x, wg, wu, wd))
    return (torch.nn.functional.silu(xt @ g) * (xt @ u) @ dn).numpy()


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_single_expert_top1_is_dense_swiglu(act):
    """E = 1, k = 1: every token goes to the one expert with gate 1, so the block
    is the dense SwiGLU FFN (checked against torch's SiLU and matmul)."""
    rng = np.random.default_rng(8)
    T, d, H = 23, 48, 80                     # d != H so a transposed operand cannot pass
    rnd = O.round_f32 if act == "f32" else O.round_bf16
    x = rnd(rng.standard_normal((T, d)))
    wg = rnd(rng.standard_normal((1, d, H)) * 0.2)
    wu = rnd(rng.standard_normal((1, d, H)) * 0.2)
    wd = rnd(rng.standard_normal((1, H, d)) * 0.2)
    out = O.forward(x, 1, 1, act, wg, wu, wd, logits=rng.standard_normal((T, 1)))
    want = _torch_dense_swiglu(x, wg[0], wu[0], wd[0])
    tol = 1e-6 if act == "f32" else 2e-2
    assert np.max(np.abs(out["y"] - want)) <= tol * np.max(np.abs(want))
    assert np.all(out["gate"] == 1.0)


@pytest.mark.parametrize("act,tol", [("f32", 1e-6), ("bf16", 1e-2), ("mxfp8", 0.12)])
def test_routed_block_equals_dense_gate_matrix(act, tol):
    """The routed block is the dense mixture sum_e G[t, e] SwiGLU_e(x[t]) with G
    the renormalised softmax of each token's k largest logits and zero
    elsewhere (Olmo-core report, Figure 5 and Section 24: the routed rows are
    this sum computed only where G is non-zero).  Written here in torch over
    every (token, expert) pair with torch's topk, softmax and SiLU, so the
    oracle's grouping, positions, weight indexing and combine are checked
    against a formulation that has none of them.  MXFP8 is compared with the
    unquantised mixture at a bar that E4M3's 3-bit mantissa leaves room for."""
    rng = np.random.default_rng(31)
    T, d, E, k, H = 90, 64, 6, 2, 96          # d != H and E > k: transposes and wrong experts fail
    rnd = O.round_f32 if act == "f32" else O.round_bf16
    x = rnd(rng.standard_normal((T, d)))
    wg = rnd(rng.standard_normal((E, d, H)) * 0.15)
    wu = rnd(rng.standard_normal((E, d, H)) * 0.15)
    wd = rnd(rng.standard_normal((E, H, d)) * 0.15)
    logits = O.round_f32(rng.standard_normal((T, E)))
    out = O.forward(x, E, k, act, wg, wu, wd, logits=logits)

    lt = torch.from_numpy(logits)
    top = torch.topk(lt, k, dim=1)
    G = torch.zeros(T, E, dtype=torch.float64)
    G.scatter_(1, top.indices, torch.softmax(top.values, dim=1))
    xt = torch.from_numpy(x)
    y = torch.zeros(T, d, dtype=torch.float64)
    for e in range(E):
        g, u, dn = (torch.from_numpy(np.asarray(a[e], np.float64)) for a in (wg, wu, wd))
        y += G[:, e:e + 1] * ((torch.nn.functional.silu(xt @ g) * (xt @ u)) @ dn)
    want = y.numpy()
    err = np.linalg.norm(out["y"] - want) / np.linalg.norm(want)
    assert err <= tol, err
    assert np.array_equal(np.sort(out["idx"], axis=1), np.sort(top.indices.numpy(), axis=1))


def test_identity_experts_round_trip():
    """With ye := xe the combine returns sum_j g_j x[t] = x[t]: bit-exact in bf16
    because the renormalised gates sum to 1 within far less than a bf16 half-ulp."""
    rng = np.random.default_rng(9)
    T, d, E, k = 200, 64, 16, 4
    x = O.round_bf16(rng.standard_normal((T, d)))
    idx, g = O.route(rng.standard_normal((T, E)).astype(np.float32), k)
    _, _, pos, _ = O.route_metadata(idx, E)
    xe = O.dispatch(x, pos, "bf16")
    assert np.array_equal(O.combine(xe, g, pos, "bf16"), x)
    xf = O.round_f32(rng.standard_normal((T, d)))
    y = O.combine(O.dispatch(xf, pos, "f32"), g, pos, "f32")
    assert np.max(np.abs(y - xf)) <= 1e-6 * np.max(np.abs(xf))
    # k = 1: combine is a pure gather
    idx1, g1 = O.route(rng.standard_normal((T, E)), 1)
    _, _, pos1, _ = O.route_metadata(idx1, E)
    assert np.array_equal(O.combine(O.dispatch(x, pos1, "bf16"), g1, pos1, "bf16"), x)


def _small_problem(act, seed=11, T=60, d=64, E=6, k=2, H=96):
    rng = np.random.default_rng(seed)
    rnd = O.round_f32 if act == "f32" else O.round_bf16
    x = rnd(rng.standard_normal((T, d)))
    L = rng.standard_normal((T, E)).astype(np.float32).astype(np.float64)
    wg = rnd(rng.standard_normal((E, d, H)) * 0.1)
    wu = rnd(rng.standard_normal((E, d, H)) * 0.1)
    wd = rnd(rng.standard_normal((E, H, d)) * 0.1)
    return x, L, wg, wu, wd


@pytest.mark.parametrize("act", ["f32", "bf16", "mxfp8"])
def test_expert_relabelling_invariance(act):
    """Renaming experts (permuting logit columns and weight stacks together) must
    not change y: catches reading another expert's segment or weights."""
    x, L, wg, wu, wd = _small_problem(act if act != "mxfp8" else "bf16")
    E = L.shape[1]
    perm = np.random.default_rng(12).permutation(E)
    y1 = O.forward(x, E, 2, act, wg, wu, wd, logits=L)["y"]
    inv = np.argsort(perm)
    y2 = O.forward(x, E, 2, act, wg[perm], wu[perm], wd[perm], logits=L[:, perm])["y"]
    assert np.array_equal(y1, y2)
    assert not np.array_equal(inv, np.arange(E))


@pytest.mark.parametrize("act", ["f32", "bf16", "mxfp8"])
def test_token_permutation_equivariance(act):
    x, L, wg, wu, wd = _small_problem(act if act != "mxfp8" else "bf16")
    E = L.shape[1]
    perm = np.random.default_rng(13).permutation(x.shape[0])
    y1 = O.forward(x, E, 2, act, wg, wu, wd, logits=L)["y"]
    y2 = O.forward(x[perm], E, 2, act, wg, wu, wd, logits=L[perm])["y"]
    assert np.array_equal(y1[perm], y2)


@pytest.mark.parametrize("act", ["f32", "bf16", "mxfp8"])
def test_forward_tokens_matches_full_forward(act):
    """The per-token evaluation (used for sampled checks at full size) equals the
    segment-wise grouped evaluation."""
    x, L, wg, wu, wd = _small_problem(act if act != "mxfp8" else "bf16")
    E = L.shape[1]
    full = O.forward(x, E, 2, act, wg, wu, wd, logits=L)
    toks = np.array([0, 5, 17, 59])
    part = O.forward_tokens(x, full["idx"], full["gate"], toks, act, wg, wu, wd)
    assert np.array_equal(part, full["y"][toks])


def test_combine_uses_gates_linearly():
    """Doubling W_down doubles every y exactly (powers of two commute with rounding)."""
    x, L, wg, wu, wd = _small_problem("bf16")
    E = L.shape[1]
    y1 = O.forward(x, E, 2, "bf16", wg, wu, wd, logits=L)["y"]
    y2 = O.forward(x, E, 2, "bf16", wg, wu, 2 * wd, logits=L)["y"]
    assert np.array_equal(2 * y1, y2)


def test_learned_router_logits_are_a_matmul():
    rng = np.random.default_rng(14)
    x = O.round_bf16(rng.standard_normal((9, 32)))
    wr = O.round_bf16(rng.standard_normal((32, 5)) * 0.02)
    L = O.router_logits(x, wr)
    want = (torch.from_numpy(x) @ torch.from_numpy(wr)).numpy()
    assert np.max(np.abs(L - want)) <= 1e-6 * np.max(np.abs(want))
    assert np.array_equal(L, L.astype(np.float32).astype(np.float64))


# ----------------------------------------------------------------------------- router statistics


def test_router_stats_hand_examples():
    """Two tokens, two experts, top-1, logits chosen so the softmax is in quarters."""
    l3 = math.log(3.0)
    # token 0 prefers expert 1 (3/4), token 1 prefers expert 0 (3/4): balanced
    s = O.router_stats(np.array([[0.0, l3], [l3, 0.0]]), np.array([1, 1]), k=1)
    assert np.allclose(s["P"], [0.5, 0.5], rtol=0, atol=1e-15)
    assert abs(s["lbl"] - 1.0) < 1e-15 and s["imbalance"] == 1.0
    # both tokens prefer expert 0 with probability 3/4: f = (1, 0), P = (3/4, 1/4)
    s = O.router_stats(np.array([[l3, 0.0], [l3, 0.0]]), np.array([2, 0]), k=1)
    assert np.allclose(s["P"], [0.75, 0.25], rtol=0, atol=1e-15)
    assert abs(s["lbl"] - 1.5) < 1e-15 and s["imbalance"] == 2.0


def test_router_stats_uniform_and_invariants():
    rng = np.random.default_rng(5)
    T, E, k = 64, 8, 2
    # equal logits: P uniform; perfectly balanced counts give lbl = imbalance = 1
    s = O.router_stats(np.zeros((T, E)), np.full(E, T * k // E), k)
    assert np.allclose(s["P"], 1.0 / E, rtol=0, atol=1e-15)
    assert abs(s["lbl"] - 1.0) < 1e-14 and s["imbalance"] == 1.0
    # P is a probability vector; lbl is at most E * max(P) and at least E * min(P)
    L = rng.normal(size=(T, E)) * 3.0
    idx, _ = O.route(L, k)
    counts, _, _, _ = O.route_metadata(idx, E)
    s = O.router_stats(L, counts, k)
    assert abs(s["P"].sum() - 1.0) < 1e-12 and (s["P"] > 0).all()
    assert E * s["P"].min() - 1e-12 <= s["lbl"] <= E * s["P"].max() + 1e-12
    assert s["imbalance"] == counts.max() / (T * k / E)
    # shifting every logit of a token by a constant changes nothing
    s2 = O.router_stats(L + rng.normal(size=(T, 1)) * 10.0, counts, k)
    assert np.allclose(s2["P"], s["P"], rtol=1e-12, atol=0) and abs(s2["lbl"] - s["lbl"]) < 1e-12


def test_router_stats_scalar_can_fall_while_imbalance_stays():
    """The cross-term property the report warns about: with the hard counts
    fixed (same top-1 choices), moving soft score mass between experts changes
    the scalar while the worst-case imbalance is unchanged."""
    T, E = 8, 4
    # every token routes to expert 0 (imbalance E), but with varying confidence
    sharp = np.zeros((T, E))
    sharp[:, 0] = 4.0
    soft = np.zeros((T, E))
    soft[:, 0] = 0.5
    counts = np.array([T, 0, 0, 0])
    for L in (sharp, soft):
        assert (O.select_topk(L, 1)[:, 0] == 0).all()
    a, b = O.router_stats(sharp, counts, 1), O.router_stats(soft, counts, 1)
    assert a["imbalance"] == b["imbalance"] == E
    assert b["lbl"] < a["lbl"]
    # with all rows on expert 0, lbl = E * P_0 exactly
    p0 = math.exp(0.5) / (math.exp(0.5) + 3.0)
    assert abs(b["lbl"] - E * p0) < 1e-14


def test_mxfp8_weights_blocked_along_contraction_axis():
    """MXFP8 expert weights are quantised in blocks of 32 along each GEMM's
    contraction axis: d for W_gate / W_up [d, H], H for W_down [H, d] (axis 0
    of each).  Hand-built 32 x 32 matrices, all v = 11 * 2^-10 except 384 at
    [0, 0]: the block holding 384 has shared exponent floor(log2 384) - 8 = 0,
    so its other entries go to the subnormal grid m * 2^-9, where v / 2^-9 =
    5.5 is a tie that rounds to the even 6 (6 * 2^-9); every other block has
    amax v, shared exponent floor(log2 v) - 8 = -15, and v / 2^-15 = 352 is an
    E4M3 value, so v stays exact.  Blocking along the contraction axis
    coarsens column 0 below the 384; blocking along the output axis would
    coarsen row 0 instead."""
    v = 11 * 2.0 ** -10
    w = np.full((1, 32, 32), v)
    w[0, 0, 0] = 384.0
    for q in O.expert_weights(w, w.copy(), w.copy(), 0, "mxfp8"):
        assert q[0, 0] == 384.0
        assert np.all(q[1:, 0] == 6 * 2.0 ** -9), "the contraction-axis block of [0, 0] is not coarsened"
        assert np.all(q[0, 1:] == v), "an output-axis block was coarsened"
        assert np.all(q[1:, 1:] == v)
