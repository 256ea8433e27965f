"""Parity of the HIP path against the CPU oracle on an MI355X (marked gpu).

Bars: routing indices, counts, offsets, positions, row_token and dispatched
rows (including MXFP8 codes and scales) bit-exact; gates within 1e-5
absolute; outputs within max-abs 1e-5 (float32), normwise relative 2e-2
(bf16) and 6e-2 (MXFP8), where normwise relative = max|out - ref| / max|ref|.
Routing of learned-router blocks is checked as a function of the float32
logits the GPU computed (the oracle re-routes those logits); the logits
themselves are checked against the oracle's float64 product.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from oracle import mxfp8 as MX
from routing_dispatch_grouped_router_amd import binding as B
from routing_dispatch_grouped_router_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
Y_TOL = {"f32": ("abs", 1e-5), "bf16": ("rel", 2e-2), "mxfp8": ("rel", 6e-2)}


def _np(t):
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def _f64(t):
    return _np(t).astype(np.float64)


def scales_rowmajor(xs):
    """MXFP8 scales from the library's slice-major [cols/128][rows][4] layout to
    [rows][cols/32] (the oracle's)."""
    S, R, _ = xs.shape
    return xs.transpose(1, 0, 2).reshape(R, 4 * S)


def check_y(act, out, ref, what="y"):
    kind, tol = Y_TOL[act]
    err = np.max(np.abs(out - ref))
    if kind == "abs":
        assert err <= tol, f"{what}: max abs err {err:.3e} > {tol}"
    else:
        rel = err / max(np.max(np.abs(ref)), 1e-30)
        assert rel <= tol, f"{what}: normwise rel err {rel:.3e} > {tol}"


def problem_of(w, identity=False):
    return B.problem(w.T, w.d, w.E, w.k, w.H, w.act, logits_given=w.router != "learned",
                     identity=identity)


def device_inputs(w):
    host = W.make_inputs(w)
    dev = {k: (None if v is None else v.to(DEV)) for k, v in host.items()}
    return host, dev


def check_routing(w, gpu, logits64):
    """gpu: dict of device tensors from moe_route / moe_forward."""
    idx, gate = O.route(logits64, w.k)
    counts, offsets, pos, row_token = O.route_metadata(idx, w.E)
    assert np.array_equal(_np(gpu["idx"]), idx), "topk_idx"
    assert np.max(np.abs(_f64(gpu["gate"]) - gate)) <= 1e-5, "topk_gate"
    assert np.array_equal(_np(gpu["counts"]), counts), "counts"
    assert np.array_equal(_np(gpu["offsets"]), offsets), "offsets"
    assert np.array_equal(_np(gpu["pos"]), pos), "pos"
    if gpu.get("row_token") is not None:
        assert np.array_equal(_np(gpu["row_token"]), row_token), "row_token"
    assert int(counts.sum()) == w.T * w.k
    return idx, gate, counts, offsets, pos


def check_logits(w, host, gpu_logits):
    if w.router != "learned":
        assert torch.equal(gpu_logits.cpu(), host["logits"])
        return host["logits"].double().numpy()
    want = O.router_logits(W.as_f64(host["x"]), W.as_f64(host["w_router"]))
    got = _f64(gpu_logits)
    assert np.max(np.abs(got - want)) <= 1e-5 * max(1.0, np.max(np.abs(want))), "router logits"
    return got


STATS_TOL = 1e-5   # relative, float32 sums of at most a few thousand probabilities in fixed order


def check_router_stats(w, stats, logits64, counts):
    """stats: device float32 [E + 2] (P_e, balance scalar, worst-case imbalance)."""
    ref = O.router_stats(logits64, counts, w.k)
    got = _f64(stats)
    E = w.E
    assert np.max(np.abs(got[:E] - ref["P"])) <= STATS_TOL * np.max(ref["P"]), "P_e"
    assert abs(got[E] - ref["lbl"]) <= STATS_TOL * ref["lbl"], "balance scalar"
    assert abs(got[E + 1] - ref["imbalance"]) <= 1e-6 * ref["imbalance"], "imbalance"


def oracle_weights(host):
    return (W.as_f64(host["w_gate"]), W.as_f64(host["w_up"]), W.as_f64(host["w_down"]))


SMALL_NAMES = ["tiny_f32"] + list(W.SMALL)


@pytest.mark.parametrize("name", SMALL_NAMES)
def test_stages_against_oracle(name):
    w = W.get(name)
    print(f"[stages] {w.describe()}", flush=True)
    host, dev = device_inputs(w)
    p = problem_of(w)
    ws = B.new_workspace(p, DEV)
    r = B.route(p, x=dev["x"], w_router=dev["w_router"], logits=dev["logits"], ws=ws, stats=True)
    torch.cuda.synchronize()
    L = check_logits(w, host, r["logits"])
    idx, gate, counts, offsets, pos = check_routing(w, r, L)
    check_router_stats(w, r["router_stats"], L, counts)

    x64 = W.as_f64(host["x"])
    xe, xs = B.dispatch(p, dev["x"], r["pos"])
    if w.act == "mxfp8":
        xq_ref, xs_ref = O.dispatch(x64, pos, "mxfp8")
        assert np.array_equal(_np(xe), xq_ref), "MXFP8 codes"
        assert np.array_equal(scales_rowmajor(_np(xs)), xs_ref), "MXFP8 scales"
        xe_vals = MX.dequantize(xq_ref, xs_ref, axis=1)
    else:
        xe_ref = O.dispatch(x64, pos, w.act)
        assert np.array_equal(_f64(xe), xe_ref), "dispatched rows"
        xe_vals = xe_ref

    packed = B.pack_weights(p, dev["w_gate"], dev["w_up"], dev["w_down"])
    ye = B.grouped_swiglu(p, xe, xs, packed, r["offsets"], ws=ws)
    wg, wu, wd = oracle_weights(host)
    ye_ref = O.experts(xe_vals, offsets, wg, wu, wd, w.act)
    check_y(w.act, _f64(ye), ye_ref, "ye")

    y = B.combine(p, ye, r["gate"], r["pos"])
    y_from_gpu_ye = O.combine(_f64(ye), _f64(r["gate"]), pos, O.out_dtype(w.act))
    # combine alone: float32 accumulation of identical inputs -> within output rounding
    tol = 1e-6 if w.act == "f32" else 2 ** -7
    assert np.max(np.abs(_f64(y) - y_from_gpu_ye)) <= tol * max(1.0, np.max(np.abs(y_from_gpu_ye)))
    check_y(w.act, _f64(y), O.combine(ye_ref, gate, pos, O.out_dtype(w.act)))

    # the whole block gives bitwise the staged result (for bf16 with d, H >= 128
    # moe_forward's GEMM reads the token rows of x in place of the dispatched copy)
    out = B.forward(p, dev["x"], packed=packed, w_router=dev["w_router"], logits=dev["logits"])
    torch.cuda.synchronize()
    assert torch.equal(out["y"], y), "moe_forward differs from the staged calls"


@pytest.mark.parametrize("name", SMALL_NAMES)
def test_forward_against_oracle(name):
    w = W.get(name)
    print(f"[forward] {w.describe()}", flush=True)
    host, dev = device_inputs(w)
    p = problem_of(w)
    packed = B.pack_weights(p, dev["w_gate"], dev["w_up"], dev["w_down"])
    out = B.forward(p, dev["x"], packed=packed, w_router=dev["w_router"], logits=dev["logits"])
    torch.cuda.synchronize()
    L = check_logits(w, host, out["logits"])
    check_routing(w, out, L)
    wg, wu, wd = oracle_weights(host)
    ref = O.forward(W.as_f64(host["x"]), w.E, w.k, w.act, wg, wu, wd, logits=L)
    check_y(w.act, _f64(out["y"]), ref["y"])


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_identity_experts_round_trip(act):
    w = W.Workload("identity", T=300, d=256, E=16, k=4, H=64, act=act, router="random", seed=77)
    print(f"[identity] {w.describe()}", flush=True)
    host, dev = device_inputs(w)
    p = problem_of(w, identity=True)
    out = B.forward(p, dev["x"], logits=dev["logits"])
    y = _f64(out["y"])
    x = W.as_f64(host["x"])
    if act == "bf16":
        assert np.array_equal(y, x)
    else:
        assert np.max(np.abs(y - x)) <= 1e-6 * np.max(np.abs(x))


@pytest.mark.parametrize("name", ["small_bf16_zipf", "small_f32_learned", "small_mxfp8"])
def test_deterministic_bitwise(name):
    w = W.get(name)
    print(f"[determinism] {w.describe()}", flush=True)
    host, dev = device_inputs(w)
    p = problem_of(w)
    packed = B.pack_weights(p, dev["w_gate"], dev["w_up"], dev["w_down"])
    f = B.Forward(p, DEV)
    outs = []
    for _ in range(2):
        f(dev["x"], packed=packed, w_router=dev["w_router"], logits=dev["logits"])
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (f.y, f.idx, f.gate, f.counts, f.offsets, f.pos, f.logits)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["tiny_f32", "small_bf16_e8", "small_mxfp8", "edge_empty_experts",
                                  "small_f32_learned"])
def test_host_sync_variant_matches(name):
    """moe_forward_host_sync runs the same kernels after one host wait: every
    output is bit-identical to moe_forward's, and the host copy of the counts
    equals the oracle's counts."""
    w = W.get(name)
    print(f"[host-sync] {w.describe()}", flush=True)
    host, dev = device_inputs(w)
    p = problem_of(w)
    packed = B.pack_weights(p, dev["w_gate"], dev["w_up"], dev["w_down"])
    outs = []
    for sync in (False, True):
        f = B.Forward(p, DEV, host_sync=sync)
        f(dev["x"], packed=packed, w_router=dev["w_router"], logits=dev["logits"])
        torch.cuda.synchronize()
        outs.append(f)
    a, b = outs
    for name_t in ("y", "logits", "idx", "gate", "counts", "offsets", "pos"):
        assert torch.equal(getattr(a, name_t), getattr(b, name_t)), name_t
    L = _f64(a.logits) if w.router == "learned" else W.as_f64(host["logits"])
    idx, _ = O.route(L, w.k)
    counts, _, _, _ = O.route_metadata(idx, w.E)
    assert np.array_equal(b.host_counts.numpy(), counts)


@pytest.mark.parametrize("name", ["small_bf16_zipf", "small_f32_learned", "edge_empty_experts", "edge_k_eq_E",
                                  "edge_one_token", "edge_ties", "edge_max_E_k", "edge_max_E_k_learned_f32"])
def test_router_stats_forward(name):
    """Router statistics from moe_forward: equal to the oracle's, bit-identical
    across calls and to moe_route's, and computing them changes no other output."""
    w = W.get(name)
    print(f"[router-stats] {w.describe()}", flush=True)
    host, dev = device_inputs(w)
    p = problem_of(w)
    packed = B.pack_weights(p, dev["w_gate"], dev["w_up"], dev["w_down"])
    plain = B.Forward(p, DEV)
    plain(dev["x"], packed=packed, w_router=dev["w_router"], logits=dev["logits"])
    f = B.Forward(p, DEV, stats=True)
    runs = []
    for _ in range(2):
        f(dev["x"], packed=packed, w_router=dev["w_router"], logits=dev["logits"])
        torch.cuda.synchronize()
        runs.append(f.router_stats.clone())
    assert torch.equal(runs[0], runs[1])
    for name_t in ("y", "idx", "gate", "counts", "offsets", "pos", "logits"):
        assert torch.equal(getattr(plain, name_t), getattr(f, name_t)), name_t
    L = _f64(f.logits) if w.router == "learned" else W.as_f64(host["logits"])
    check_router_stats(w, f.router_stats, L, _np(f.counts))
    r = B.route(p, x=dev["x"], w_router=dev["w_router"], logits=f.logits if w.router != "learned" else None,
                stats=True)
    torch.cuda.synchronize()
    if w.router != "learned":
        assert torch.equal(r["router_stats"], f.router_stats)


def test_graph_capture_replay():
    w = W.get("small_bf16_e32_random")
    print(f"[graph] {w.describe()}", flush=True)
    host, dev = device_inputs(w)
    p = problem_of(w)
    packed = B.pack_weights(p, dev["w_gate"], dev["w_up"], dev["w_down"])
    f = B.Forward(p, DEV)
    f(dev["x"], packed=packed, logits=dev["logits"])
    torch.cuda.synchronize()
    eager = f.y.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        f(dev["x"], packed=packed, logits=f.logits)     # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        f(dev["x"], packed=packed, logits=f.logits)
    for i in range(4):
        f.y.fill_(float("nan"))
        scratch = torch.randn(1024, device=DEV) * i      # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(f.y, eager), f"replay {i}"
        del scratch


# ----------------------------------------------------------------------------- full-size configurations

N_SAMPLE = 24


class _LazyF64:
    """Per-expert float64 view of a stored weight stack, converted on access
    (the full stacks of the large configurations do not fit in float64)."""

    def __init__(self, t):
        self.t = t

    def __getitem__(self, e):
        return W.as_f64(self.t[e])


def _sample_tokens(T, seed=0):
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(8, T - 8), size=N_SAMPLE - 16, replace=False) if T > 32 else []
    return np.unique(np.concatenate([np.arange(min(8, T)), np.arange(max(0, T - 8), T), mid])).astype(np.int64)


def _tile_tokens(offsets, row_token, T, block=128, seed=0):
    """Tokens that cover every `block`-row piece of every expert segment (one
    routed row drawn from each piece, so every M tile of the grouped GEMMs is
    checked), plus the first and last 8 tokens."""
    rng = np.random.default_rng(seed)
    toks = [np.arange(min(8, T)), np.arange(max(0, T - 8), T)]
    for e in range(len(offsets) - 1):
        for r0 in range(int(offsets[e]), int(offsets[e + 1]), block):
            r1 = min(r0 + block, int(offsets[e + 1]))
            toks.append(np.array([row_token[int(rng.integers(r0, r1))]]))
    return np.unique(np.concatenate(toks)).astype(np.int64)


@pytest.mark.slow
@pytest.mark.parametrize("name", W.CONFIG_ORDER)
def test_full_size_config(name):
    """The five block configurations at full size, run exactly as the benchmark
    runs them (moe_forward with packed weights): routing checked bit-exactly on
    every token, y against the oracle on tokens that cover every 128-row piece
    of every expert segment (so every output tile of both grouped GEMMs)."""
    w = W.CONFIGS[name]
    print(f"[full] {w.describe()}", flush=True)
    host, dev = device_inputs(w)
    p = problem_of(w)
    packed = B.pack_weights(p, dev["w_gate"], dev["w_up"], dev["w_down"])
    f = B.Forward(p, DEV, stats=True)
    f(dev["x"], packed=packed, w_router=dev["w_router"], logits=dev["logits"])
    torch.cuda.synchronize()
    gpu = dict(idx=f.idx, gate=f.gate, counts=f.counts, offsets=f.offsets, pos=f.pos)
    if w.router == "learned":
        L = _f64(f.logits)
        rows = _sample_tokens(w.T, 1)
        want = O.router_logits(W.as_f64(host["x"][torch.from_numpy(rows)]), W.as_f64(host["w_router"]))
        assert np.max(np.abs(L[rows] - want)) <= 1e-5 * max(1.0, np.max(np.abs(want)))
    else:
        L = check_logits(w, host, f.logits)
    idx, gate, counts, offsets, pos = check_routing(w, gpu, L)
    check_router_stats(w, f.router_stats, L, counts)
    _, _, _, row_token = O.route_metadata(idx, w.E)
    toks = _tile_tokens(offsets, row_token, w.T)
    print(f"[full] y checked on {len(toks)} tokens", flush=True)
    ref = O.forward_tokens(W.as_f64(host["x"]), idx, gate, toks, w.act, _LazyF64(host["w_gate"]),
                           _LazyF64(host["w_up"]), _LazyF64(host["w_down"]))
    check_y(w.act, _f64(f.y)[toks], ref)
    yall = _f64(f.y)
    assert np.all(np.isfinite(yall))


@pytest.mark.slow
@pytest.mark.parametrize("name", [n for n in W.CONFIG_ORDER if n != "tiny_f32"])
def test_full_size_dispatch_bitexact(name):
    """The whole dispatched buffer of each large block, through moe_route and
    moe_dispatch at full size: bf16 rows equal x[row_token] bit for bit, and
    moe_forward, whose grouped GEMM reads those rows of x in place, equals the
    staged grouped SwiGLU and combine on them bit for bit (every output tile);
    MXFP8 codes and scales equal the oracle quantiser's for every row, and
    moe_forward, which quantises each token once and reads its code rows in
    place, equals the staged path on them bit for bit."""
    w = W.CONFIGS[name]
    print(f"[full dispatch] {w.describe()}", flush=True)
    host, dev = device_inputs(w)
    p = problem_of(w)
    r = B.route(p, x=dev["x"], w_router=dev["w_router"], logits=dev["logits"])
    xe, xs = B.dispatch(p, dev["x"], r["pos"])
    torch.cuda.synchronize()
    L = _f64(r["logits"]) if w.router == "learned" else W.as_f64(host["logits"])
    idx, _ = O.route(L, w.k)
    _, _, pos, row_token = O.route_metadata(idx, w.E)
    assert np.array_equal(_np(r["row_token"]), row_token), "row_token"
    if w.act != "mxfp8":
        rt = torch.from_numpy(row_token.astype(np.int64)).to(DEV)
        assert torch.equal(xe, dev["x"][rt]), "dispatched rows differ from x[row_token]"
        # moe_forward reads these rows from x in place (no copy): every output
        # tile equals the staged grouped SwiGLU on the dispatched buffer, bitwise
        packed = B.pack_weights(p, dev["w_gate"], dev["w_up"], dev["w_down"])
        ye = B.grouped_swiglu(p, xe, xs, packed, r["offsets"])
        y = B.combine(p, ye, r["gate"], r["pos"])
        del xe, ye
        out = B.forward(p, dev["x"], packed=packed, w_router=dev["w_router"], logits=dev["logits"])
        torch.cuda.synchronize()
        assert torch.equal(out["y"], y), "moe_forward differs from dispatch + grouped SwiGLU + combine"
        return
    q_gpu = _np(xe)
    s_gpu = scales_rowmajor(_np(xs))
    x64 = W.as_f64(host["x"])
    for t0 in range(0, w.T, 4096):
        t1 = min(w.T, t0 + 4096)
        q, sc = MX.quantize(x64[t0:t1], axis=1)
        for j in range(w.k):
            rows = pos[t0:t1, j]
            assert np.array_equal(q_gpu[rows], q), f"MXFP8 codes, tokens {t0}..{t1} slot {j}"
            assert np.array_equal(s_gpu[rows], sc), f"MXFP8 scales, tokens {t0}..{t1} slot {j}"
    # moe_forward quantises each token once and GEMM1 reads those code rows
    # through row_token: every output tile equals the staged path on the
    # dispatched codes and scales, bit for bit
    packed = B.pack_weights(p, dev["w_gate"], dev["w_up"], dev["w_down"])
    ye = B.grouped_swiglu(p, xe, xs, packed, r["offsets"])
    y = B.combine(p, ye, r["gate"], r["pos"])
    del xe, xs, ye
    out = B.forward(p, dev["x"], packed=packed, w_router=dev["w_router"], logits=dev["logits"])
    torch.cuda.synchronize()
    assert torch.equal(out["y"], y), "moe_forward differs from dispatch + grouped SwiGLU + combine"


# ----------------------------------------------------------------------------- MXFP8 packing


def _unpack_w1(packed_w1, E, d, H):
    """Undo the documented gate/up interleave: packed row n -> (gate|up, column h)."""
    n = np.arange(2 * H)
    h = 32 * (n // 64) + n % 32
    is_up = (n // 32) % 2 == 1
    gate = np.empty((E, H, d), packed_w1.dtype)
    up = np.empty((E, H, d), packed_w1.dtype)
    gate[:, h[~is_up]] = packed_w1[:, n[~is_up]]
    up[:, h[is_up]] = packed_w1[:, n[is_up]]
    return gate, up


@pytest.mark.parametrize("act", ["bf16", "mxfp8"])
def test_packed_weight_layout(act):
    w = W.Workload("pack", T=4, d=256, E=3, k=2, H=384 if act == "bf16" else 256, act=act,
                   router="random", seed=5)
    host, dev = device_inputs(w)
    p = problem_of(w)
    packed = B.pack_weights(p, dev["w_gate"], dev["w_up"], dev["w_down"])
    buf = packed.cpu().numpy()
    E, d, H = w.E, w.d, w.H
    al = lambda x: (x + 255) // 256 * 256
    if act == "bf16":
        n1, n2 = E * 2 * H * d * 2, E * d * H * 2
        w1 = buf[:n1].view(np.uint16).reshape(E, 2 * H, d)
        w2 = buf[al(n1):al(n1) + n2].view(np.uint16).reshape(E, d, H)
        bits = lambda t: t.view(torch.int16).numpy().view(np.uint16)
        g, u = _unpack_w1(w1, E, d, H)
        assert np.array_equal(g, bits(host["w_gate"]).transpose(0, 2, 1))
        assert np.array_equal(u, bits(host["w_up"]).transpose(0, 2, 1))
        assert np.array_equal(w2, bits(host["w_down"]).transpose(0, 2, 1))
    else:
        n1, n2 = E * 2 * H * d, E * d * H
        o1, o2 = 0, al(n1)
        o3 = o2 + al(n2)
        o4 = o3 + al(n1 // 32)
        w1 = buf[o1:o1 + n1].reshape(E, 2 * H, d)
        w2 = buf[o2:o2 + n2].reshape(E, d, H)
        # slice-major [E][K/128][N][4] -> [E][N][K/32]
        s1 = buf[o3:o3 + n1 // 32].reshape(E, d // 128, 2 * H, 4).transpose(0, 2, 1, 3).reshape(E, 2 * H, d // 32)
        s2 = buf[o4:o4 + n2 // 32].reshape(E, H // 128, d, 4).transpose(0, 2, 1, 3).reshape(E, d, H // 32)
        gq, uq = _unpack_w1(w1, E, d, H)
        gs, us = _unpack_w1(s1, E, d // 32, H)
        for e in range(E):
            for (codes, scales, src) in ((gq[e], gs[e], host["w_gate"][e]), (uq[e], us[e], host["w_up"][e]),
                                         (w2[e], s2[e], host["w_down"][e])):
                q_ref, s_ref = MX.quantize(W.as_f64(src), axis=0)     # blocks along K
                assert np.array_equal(codes, q_ref.T), "E4M3 codes"
                assert np.array_equal(scales, s_ref.T), "E8M0 scales"


# --------------------------------------------------------------------------- grid cap
#
# moe_set_gemm_grid_cap bounds the persistent grid of the bf16 and MXFP8
# grouped GEMMs.  Each output tile is still computed whole, in the same K
# order, by whichever workgroup takes it, so capped and uncapped results are
# bit-identical; with a small cap every workgroup walks many tiles, and rounds
# end on ragged tails.

CAP_CASES = [
    # dense single expert, 9 ragged M tiles over 8 workgroups
    ("bf16_dense_cap8", W.Workload("cap_bf16_dense", T=2200, d=1024, E=1, k=1, H=256, act="bf16",
                                   router="random", seed=3101), 8),
    ("bf16_e8_cap40", W.Workload("cap_bf16_e8", T=1500, d=512, E=8, k=2, H=384, act="bf16",
                                 router="random", seed=3103), 40),
    ("bf16_sparse_cap16", W.Workload("cap_bf16_sparse", T=1000, d=768, E=64, k=2, H=256, act="bf16",
                                     router="random", seed=3102, empty_experts=tuple(range(8, 64))), 16),
    ("mxfp8_dense_cap8", W.Workload("cap_mx_dense", T=2200, d=1024, E=1, k=1, H=512, act="mxfp8",
                                    router="random", seed=3104, outlier_frac=0.01), 8),
    ("mxfp8_e16_cap24", W.Workload("cap_mx_e16", T=1200, d=512, E=16, k=4, H=256, act="mxfp8",
                                   router="zipf", seed=3105), 24),
    # d = 384: GEMM2's second N tile holds 128 columns, whose missing half the
    # epilogue drops; 4 K-tiles per GEMM2 tile, 3 tiles per workgroup
    ("mxfp8_ragged_n_cap8", W.Workload("cap_mx_rn", T=1500, d=384, E=4, k=2, H=512, act="mxfp8",
                                       router="random", seed=3106, outlier_frac=0.01), 8),
]


@pytest.fixture
def grid_cap():
    yield B.set_gemm_grid_cap
    B.set_gemm_grid_cap(0)


@pytest.mark.parametrize("case,w,cap", CAP_CASES, ids=[c[0] for c in CAP_CASES])
def test_grid_cap_bitwise_and_oracle(case, w, cap, grid_cap):
    print(f"[grid cap] {case} cap={cap} {w.describe()}", flush=True)
    host, dev = device_inputs(w)
    p = problem_of(w)
    packed = B.pack_weights(p, dev["w_gate"], dev["w_up"], dev["w_down"])
    ref_out = B.forward(p, dev["x"], packed=packed, w_router=dev["w_router"], logits=dev["logits"])
    torch.cuda.synchronize()
    y0 = ref_out["y"].clone()
    grid_cap(cap)
    out = B.forward(p, dev["x"], packed=packed, w_router=dev["w_router"], logits=dev["logits"])
    torch.cuda.synchronize()
    assert torch.equal(out["y"], y0), "capped grid changed y"
    L = W.as_f64(host["logits"]) if w.router != "learned" else _f64(out["logits"])
    check_routing(w, out, L)
    wg, wu, wd = oracle_weights(host)
    ref = O.forward(W.as_f64(host["x"]), w.E, w.k, w.act, wg, wu, wd, logits=L)
    check_y(w.act, _f64(out["y"]), ref["y"])


# ----------------------------------------------------------------------------- fused bf16 FFN counters

@pytest.mark.parametrize("cap", [0, 8], ids=["full_grid", "cap8"])
def test_fused_ffn_counters_reset_between_calls(cap, grid_cap):
    """The bf16 expert FFN runs GEMM1 and GEMM2 in one launch whose GEMM2 tiles
    wait on per-M-tile counters in the workspace.  Two calls through the same
    workspace with different inputs and routing must each give the result of a
    fresh workspace: stale counters from the first call would let GEMM2 read
    the first call's h."""
    wa = W.Workload("ffn_a", T=1500, d=512, E=8, k=2, H=384, act="bf16", router="random", seed=3201)
    wb = W.Workload("ffn_b", T=1500, d=512, E=8, k=2, H=384, act="bf16", router="zipf", seed=3202)
    print(f"[fused ffn] cap={cap} {wa.describe()} then {wb.describe()}", flush=True)
    grid_cap(cap)
    ha, da = device_inputs(wa)
    hb, db = device_inputs(wb)
    p = problem_of(wa)
    packed = B.pack_weights(p, da["w_gate"], da["w_up"], da["w_down"])
    f = B.Forward(p, DEV)
    f(da["x"], packed=packed, logits=da["logits"])
    f(db["x"], packed=packed, logits=db["logits"])
    torch.cuda.synchronize()
    y_reused = f.y.clone()
    fresh = B.Forward(p, DEV)
    fresh(db["x"], packed=packed, logits=db["logits"])
    torch.cuda.synchronize()
    assert torch.equal(y_reused, fresh.y), "second call through a reused workspace differs"
    wg, wu, wd = oracle_weights(ha)
    ref = O.forward(W.as_f64(hb["x"]), wb.E, wb.k, wb.act, wg, wu, wd, logits=W.as_f64(hb["logits"]))
    check_y(wb.act, _f64(y_reused), ref["y"])
    # the standalone grouped FFN entry point, twice through one workspace
    ws = B.new_workspace(p, DEV)
    ra = B.route(p, logits=da["logits"], ws=ws)
    rb = B.route(p, logits=db["logits"], ws=ws)
    xe_a, _ = B.dispatch(p, da["x"], ra["pos"])
    xe_b, _ = B.dispatch(p, db["x"], rb["pos"])
    B.grouped_swiglu(p, xe_a, None, packed, ra["offsets"], ws=ws)
    ye_b = B.grouped_swiglu(p, xe_b, None, packed, rb["offsets"], ws=ws)
    ye_fresh = B.grouped_swiglu(p, xe_b, None, packed, rb["offsets"])
    torch.cuda.synchronize()
    assert torch.equal(ye_b, ye_fresh), "grouped_swiglu through a reused workspace differs"


@pytest.fixture
def ffn_wait_flag():
    yield B.set_test_flags
    B.set_test_flags(0)


FFN_WAIT_CASES = [
    ("e8_full", W.Workload("ffnw_e8", T=1500, d=512, E=8, k=2, H=384, act="bf16", router="random", seed=3301), 0),
    ("e8_cap8", W.Workload("ffnw_e8c", T=1500, d=512, E=8, k=2, H=384, act="bf16", router="random", seed=3302), 8),
    ("sparse_cap16", W.Workload("ffnw_sp", T=1000, d=768, E=64, k=2, H=256, act="bf16", router="random", seed=3303,
                                empty_experts=tuple(range(8, 64))), 16),
    ("zipf_full", W.Workload("ffnw_zipf", T=2048, d=1024, E=16, k=4, H=512, act="bf16", router="zipf",
                             seed=3304), 0),
]


@pytest.mark.parametrize("case,w,cap", FFN_WAIT_CASES, ids=[c[0] for c in FFN_WAIT_CASES])
def test_fused_ffn_wait_path(case, w, cap, grid_cap, ffn_wait_flag):
    """Every GEMM2 tile of the fused FFN forced through the wait-and-restart
    path (the one taken when its rows are not yet done at the early check)
    gives bitwise the output of the normal path, and the oracle's."""
    print(f"[fused ffn wait path] {case} cap={cap} {w.describe()}", flush=True)
    grid_cap(cap)
    host, dev = device_inputs(w)
    p = problem_of(w)
    packed = B.pack_weights(p, dev["w_gate"], dev["w_up"], dev["w_down"])
    normal = B.forward(p, dev["x"], packed=packed, w_router=dev["w_router"], logits=dev["logits"])
    torch.cuda.synchronize()
    y0 = normal["y"].clone()
    ffn_wait_flag(B.MOE_TEST_FFN_WAIT)
    waited = B.forward(p, dev["x"], packed=packed, w_router=dev["w_router"], logits=dev["logits"])
    torch.cuda.synchronize()
    assert torch.equal(waited["y"], y0), "wait-and-restart path changed y"
    wg, wu, wd = oracle_weights(host)
    ref = O.forward(W.as_f64(host["x"]), w.E, w.k, w.act, wg, wu, wd, logits=W.as_f64(host["logits"]))
    check_y(w.act, _f64(waited["y"]), ref["y"])
