"""Benchmark of the routed MoE block forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--no-cpu-baseline]

A step is one moe_forward (router -> top-k -> counts/offsets/positions ->
dispatch -> grouped SwiGLU GEMMs -> combine) over one synthetic batch whose
inputs already sit in HBM.  W untimed steps, then exactly K steps between two
device synchronisations; one JSON line is printed.  Per-kernel durations come
from HIP events the library records on the forward's own stream during K
further steps run just before the timed ones (the events add small gaps
between kernels, so those steps are reported separately and are not the
headline); the dominant kernel is reported against its roofline.
The CPU baseline times the float64 oracle on a bounded sample of the same
batch on the host cores.

Beside the main figure the line carries three comparison measurements, each
outside the K timed steps: per-step times with the caches flushed before
every step (cold_cache), the same block through the host-synchronising path
(host_sync_variant: counts copied to the host and waited for before the
grouped GEMMs), and the block with router statistics enabled.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from routing_dispatch_grouped_router_amd import binding as B  # noqa: E402
from routing_dispatch_grouped_router_amd import workloads as W  # noqa: E402

METRIC = "MoE-block fwd tokens/s on 1 MI355X; grouped-GEMM % MFMA peak; dispatch % HBM"
DEFAULT_CONFIG = "bf16_e64_zipf"   # the largest block that fits one GPU

# MI355X published peaks
HBM_GBPS = 8000.0
MFMA_TFLOPS = {"bf16": 2500.0, "mxfp8": 5000.0}
FP32_VECTOR_TFLOPS = 157.3


def elem_bytes(act: str) -> int:
    return {"f32": 4, "bf16": 2, "mxfp8": 1}[act]


def stage_models(w: W.Workload) -> dict:
    """Algorithmic work of one launch of each kernel: (bound, amount, unit, peak)."""
    R, T, d, E, k, H = w.R, w.T, w.d, w.E, w.k, w.H
    bin_ = 4 if w.act == "f32" else 2                 # x storage
    bxe = elem_bytes(w.act)
    bye = 4 if w.act == "f32" else 2
    scale_b = R * d // 32 if w.act == "mxfp8" else 0
    gemm_bound, gemm_peak = (("alu", FP32_VECTOR_TFLOPS) if w.act == "f32"
                             else ("mfma", MFMA_TFLOPS[w.act]))
    return {
        "router_logits": ("hbm", T * d * bin_ + d * E * bin_ + T * E * 4, "GB/s", HBM_GBPS),
        "route_topk": ("hbm", T * E * 4 + R * 4 * 4 + ((T + 255) // 256) * E * 4, "GB/s", HBM_GBPS),
        "route_scan": ("hbm", 3 * ((T + 255) // 256) * E * 4 + (2 * E + 1) * 4, "GB/s", HBM_GBPS),
        # positions only (the fused bf16 FFN reads token rows in place): ranks,
        # expert ids and block bases in, positions and row_token out
        "route_finalize": ("hbm", R * 4 * 4 + ((T + 255) // 256) * E * 4, "GB/s", HBM_GBPS),
        "dispatch": ("hbm", T * d * bin_ + R * d * bxe + scale_b + R * 4 * 3 + R * 4, "GB/s", HBM_GBPS),
        # MXFP8 rows in place: each token quantised once (codes + scales, positions
        # finalised), then the scale dwords laid out per expert-major row
        "quantize": ("hbm", T * d * bin_ + T * d + T * d // 32 + R * 4 * 4, "GB/s", HBM_GBPS),
        "scale_gather": ("hbm", R * 4 + 2 * (R * d // 32), "GB/s", HBM_GBPS),
        "gemm1_gate_up_swiglu": (gemm_bound, 4.0 * R * d * H, "TFLOP/s", gemm_peak),
        "gemm2_down": (gemm_bound, 2.0 * R * H * d, "TFLOP/s", gemm_peak),
        # bf16: both projections in one launch
        "grouped_ffn": (gemm_bound, 6.0 * R * d * H, "TFLOP/s", gemm_peak),
        "combine": ("hbm", R * d * bye + R * 8 + T * d * bye, "GB/s", HBM_GBPS),
    }


def stage_rooflines(models: dict, stages) -> dict:
    """Each timed stage (name, ms) against its roofline: achieved = the stage's
    algorithmic work per launch / its time, frac = achieved / peak."""
    out = {}
    for name, ms in stages:
        bound, amount, unit, peak = models[name]
        ach = (amount / (ms * 1e-3) / 1e9) if unit == "GB/s" else (amount / (ms * 1e-3) / 1e12)
        out[name] = {"ms": round(ms, 5), "bound": bound, "achieved": round(ach, 2), "unit": unit,
                     "peak": peak, "frac": round(ach / peak, 4)}
    return out


def roofline_entry(models: dict, stage_out: dict, dom: str, traffic) -> dict:
    """The JSON line's `roofline` object for the dominant kernel `dom`."""
    bound, _, unit, peak = models[dom]
    ach = stage_out[dom]["achieved"]
    return {"kernel": dom, "bound": bound, "achieved": ach, "peak": peak, "unit": unit,
            "frac": round(ach / peak, 4), "traffic": traffic}


def block_bound_ms(w: W.Workload, models: dict) -> float:
    """The block's roofline time: each step of the method at its own peak
    (router logits for a learned router, routing, dispatch, both expert GEMMs,
    combine), whether or not this block materialises the dispatched copy."""
    steps = ["route_topk", "route_scan", "dispatch", "gemm1_gate_up_swiglu", "gemm2_down", "combine"]
    if w.router == "learned":
        steps.insert(0, "router_logits")
    total = 0.0
    for name in steps:
        _, work, unit, peak = models[name]
        total += work / (peak * (1e9 if unit == "GB/s" else 1e12)) * 1e3
    return total


def source_digest(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "gemm1_gate_up_swiglu": ["routing_dispatch_grouped_router_amd/csrc/gemm_pipe.hip",
                             "routing_dispatch_grouped_router_amd/csrc/grouped_sched.h"],
    "gemm2_down": ["routing_dispatch_grouped_router_amd/csrc/gemm_pipe.hip",
                   "routing_dispatch_grouped_router_amd/csrc/grouped_sched.h"],
    "grouped_ffn": ["routing_dispatch_grouped_router_amd/csrc/gemm_pipe.hip",
                    "routing_dispatch_grouped_router_amd/csrc/grouped_sched.h"],
    "dispatch": ["routing_dispatch_grouped_router_amd/csrc/dispatch.hip"],
    "combine": ["routing_dispatch_grouped_router_amd/csrc/dispatch.hip"],
}


def measured_traffic(config: str, kernel: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None
    if there is none or the kernel's source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path) or kernel not in KERNEL_SOURCES:
        return None
    try:
        entries = json.load(open(path))
    except (OSError, ValueError):
        return None
    want = source_digest(KERNEL_SOURCES[kernel])
    for e in entries:
        if e.get("config") == config and e.get("kernel") == kernel and e.get("source_digest") == want:
            return e.get("bytes_per_launch")
    return None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def single_thread_tiny() -> dict:
    """The oracle on the whole 256-token float32 block with one BLAS thread:
    one warm-up, then the median of three runs."""
    from oracle import moe_oracle as O
    from threadpoolctl import threadpool_limits
    w = W.CONFIGS["tiny_f32"]
    h = W.make_inputs(w)
    args = [W.as_f64(h[n]) for n in ("x", "w_gate", "w_up", "w_down")]
    wr = W.as_f64(h["w_router"])
    times = []
    with threadpool_limits(limits=1):
        for _ in range(4):
            t0 = time.perf_counter()
            O.forward(args[0], w.E, w.k, w.act, *args[1:], w_router=wr)
            times.append(time.perf_counter() - t0)
    ms = sorted(times[1:])[1] * 1e3
    return {"workload": w.describe(), "ms": round(ms, 3), "tokens_per_s": round(w.T / (ms * 1e-3), 1),
            "threads": 1}


def cpu_baseline(w: W.Workload, host: dict, budget_s: float = 12.0) -> dict:
    """Times the oracle (float64 NumPy) on the first tokens of the same batch."""
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = len(os.sched_getaffinity(0))
    wg, wu, wd = (W.as_f64(host[n]) for n in ("w_gate", "w_up", "w_down"))
    wr = W.as_f64(host["w_router"]) if host["w_router"] is not None else None

    def run(n):
        x = W.as_f64(host["x"][:n])
        lg = None if host["logits"] is None else host["logits"][:n].double().numpy()
        t0 = time.perf_counter()
        O.forward(x, w.E, w.k, w.act, wg, wu, wd, w_router=wr, logits=lg)
        return time.perf_counter() - t0

    n = min(w.T, 256)
    dt = run(n)
    while dt < budget_s / 4 and n < w.T:
        n = min(w.T, max(n * 2, int(n * budget_s / 3 / max(dt, 1e-3))))
        dt = run(n)
    reps, total, toks = 1, dt, n
    while total < budget_s * 0.6 and reps < 5:
        total += run(n)
        toks += n
        reps += 1
    return {"value": toks / total, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": len(os.sched_getaffinity(0)),
            "sample": f"oracle.forward (float64 NumPy) on the first {n} of {w.T} tokens of the "
                      f"{w.name} batch, {reps} run(s), {total:.1f} s",
            "single_thread_tiny_f32": single_thread_tiny()}


def cold_cache_steps(step, dev, steps: int) -> dict:
    """Per-step times with the L2s and the 256 MB Infinity Cache flushed first:
    a 512 MiB buffer is rewritten before every step, outside the step's events."""
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    times = []
    for i in range(steps):
        flush.fill_(i & 0xFF)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step()
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b))
    del flush
    t = sorted(times)
    q = lambda f: t[min(len(t) - 1, int(f * (len(t) - 1) + 0.5))]
    return {"ms_per_step_median": round(q(0.5), 5), "p10": round(q(0.1), 5), "p90": round(q(0.9), 5),
            "flush": "512 MiB device write before each step"}


def copy_ceiling(step, dev, models: dict, reps: int = 10) -> dict:
    """The HBM rate a plain device copy reaches in the cache state dispatch and
    combine run in: for each of the two stages, a copy moving the stage's
    algorithmic bytes (half read, half written) is timed right after a forward
    step, so the caches hold the step's dirty lines as they do for the stage;
    median over `reps` steps."""
    out = {}
    for stage in ("dispatch", "combine"):
        nbytes = int(models[stage][1])
        half = max(nbytes // 2, 1 << 20)
        src = torch.empty(half, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        times = []
        for _ in range(reps):
            step()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            dst.copy_(src)
            b.record()
            b.synchronize()
            times.append(a.elapsed_time(b))
        ms = sorted(times)[len(times) // 2]
        gbps = 2 * half / (ms * 1e-3) / 1e9
        out[stage] = {"bytes": 2 * half, "ms": round(ms, 5), "gbps": round(gbps, 1),
                      "frac_of_peak": round(gbps / HBM_GBPS, 4)}
        del src, dst
    out["note"] = "plain device copy of the stage's bytes right after a forward step (median of 10)"
    return out


def dispatch_standalone(p, d_in, dev, models: dict, reps: int = 20) -> dict:
    """moe_dispatch alone on this block's routing: `reps` launches back to back
    between two HIP events.  For blocks whose moe_forward materialises no
    dispatched copy (the fused bf16 FFN reads token rows in place) this is the
    row-wise dispatch of the staged API, measured outside the timed steps."""
    r = B.route(p, x=d_in["x"], w_router=d_in["w_router"], logits=d_in["logits"])
    B.dispatch(p, d_in["x"], r["pos"])
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        B.dispatch(p, d_in["x"], r["pos"])
    b.record()
    b.synchronize()
    ms = a.elapsed_time(b) / reps
    nbytes = models["dispatch"][1]
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 5), "achieved": round(gbps, 1), "unit": "GB/s", "peak": HBM_GBPS,
            "frac": round(gbps / HBM_GBPS, 4), "reps": reps,
            "note": "moe_dispatch of this block's rows, launched alone (not part of moe_forward here)"}


def determinism_check(step, f) -> dict:
    """Two checks run with every full benchmark: two forward steps of the block
    give bitwise the same y, and on a block with planted logit ties
    (edge_ties: 2048 tokens, 64 experts, top-8, logits from 3 integer levels)
    every token's selection is ordered by (logit descending, index ascending)
    and no unselected expert beats or ties-with-a-lower-index a selected one."""
    step()
    y0 = f.y.clone()
    step()
    torch.cuda.synchronize()
    same = bool(torch.equal(f.y, y0))
    wt = W.SMALL["edge_ties"]
    h = W.make_inputs(wt)
    pt = B.problem(wt.T, wt.d, wt.E, wt.k, wt.H, wt.act, logits_given=True)
    r = B.route(pt, logits=h["logits"].to(f.y.device))
    torch.cuda.synchronize()
    L = h["logits"].numpy()
    idx = r["idx"].cpu().numpy()
    ok = True
    ties = 0
    for t in range(wt.T):
        sel = idx[t]
        key = [(-float(L[t, e]), int(e)) for e in sel]
        ok &= key == sorted(key) and len(set(sel.tolist())) == wt.k
        last = key[-1]
        for e in range(wt.E):
            if e not in sel:
                ok &= (-float(L[t, e]), e) > last
        ties += int(np.sum(L[t] == L[t, sel[-1]]) > 1)
    return {"bitwise_repeat": same, "ties_lowest_index": bool(ok), "tokens_with_ties_at_kth": ties,
            "tie_block": wt.describe()}


def host_sync_steps(p, d_in, packed, dev, steps: int, warmup: int, ms_device: float) -> dict:
    """The same block through moe_forward_host_sync (counts copied to the host and
    waited for before the grouped GEMMs), timed like the main loop."""
    f = B.Forward(p, dev, debug_outputs=False, host_sync=True)
    if p.flags & B.MOE_LOGITS_GIVEN:
        f.logits.copy_(d_in["logits"])
    run = lambda: f(d_in["x"], packed=packed, w_router=d_in["w_router"], logits=f.logits)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    B.set_profiling(True)      # the host wait measured by the library's events, in separate steps
    for _ in range(min(steps, 20)):
        run()
    stages = dict(B.kernel_times())
    B.set_profiling(False)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        run()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    return {"ms_per_step": round(ms, 5), "host_count_wait_ms": round(stages.get("host_count_wait", 0.0), 5),
            "slowdown_vs_device_resident": round(ms / ms_device, 4)}


def router_stats_steps(p, d_in, packed, dev, steps: int, warmup: int, ms_device: float) -> dict:
    """The block with the router statistics computed in the routing pass, and their values."""
    f = B.Forward(p, dev, debug_outputs=False, stats=True)
    if p.flags & B.MOE_LOGITS_GIVEN:
        f.logits.copy_(d_in["logits"])
    run = lambda: f(d_in["x"], packed=packed, w_router=d_in["w_router"], logits=f.logits)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        run()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    st = f.router_stats.cpu().numpy()
    E = p.n_experts
    return {"ms_per_step": round(ms, 5), "overhead_ms": round(ms - ms_device, 5),
            "balance_scalar": float(st[E]), "worst_case_imbalance": float(st[E + 1]),
            "mean_router_prob_min_max": [float(st[:E].min()), float(st[:E].max())]}


def _timed(run, steps: int, warmup: int) -> float:
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        run()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def kept_gate_up_steps(w, d_in, packed, dev, steps: int, warmup: int, ms_device: float, bwd: dict) -> dict:
    """The block with MOE_KEEP_GATE_UP (the forward stores a | b, the backward
    reads them instead of recomputing xe W1), forward and backward timed like
    the main loop and set against the recomputing path's."""
    p = B.problem(w.T, w.d, w.E, w.k, w.H, w.act, logits_given=w.router != "learned", keep_gate_up=True)
    f = B.Forward(p, dev, debug_outputs=False)
    if p.flags & B.MOE_LOGITS_GIVEN:
        f.logits.copy_(d_in["logits"])
    ms_f = _timed(lambda: f(d_in["x"], packed=packed, w_router=d_in["w_router"], logits=f.logits), steps, warmup)
    packed_bwd = B.pack_weights_backward(p, d_in["w_gate"], d_in["w_up"], d_in["w_down"])
    g = torch.Generator(device="cpu").manual_seed(w.seed + 17)
    dy = torch.randn((w.T, w.d), generator=g).to(B.storage_dtype(w.act)).to(dev)
    b = B.Backward(p, dev)
    ms_b = _timed(lambda: b(f, dy, packed, packed_bwd, x=d_in["x"], w_router=d_in["w_router"]), steps, warmup)
    # useful FLOPs without the recompute: data gradients 6 R d H, weight gradients 6 R d H
    flops = 12.0 * w.R * w.d * w.H + (2 * 2.0 * w.T * w.d * w.E if w.router == "learned" else 0.0)
    tf = flops / (ms_b * 1e-3) / 1e12
    return {"forward_ms_per_step": round(ms_f, 5), "forward_vs_recompute_path": round(ms_f / ms_device, 4),
            "backward_ms_per_step": round(ms_b, 5),
            "backward_vs_recompute_path": round(ms_b / bwd["ms_per_step"], 4),
            "forward_plus_backward_vs_recompute_path": round((ms_f + ms_b) / (ms_device + bwd["ms_per_step"]), 4),
            "backward_useful_tflops": round(tf, 2), "backward_frac_of_peak": round(tf / 2500.0, 4),
            "extra_forward_workspace_bytes": B.workspace_bytes(p) - B.workspace_bytes(
                B.problem(w.T, w.d, w.E, w.k, w.H, w.act, logits_given=w.router != "learned"))}


def keeps_gate_up(w) -> bool:
    return (w.act == "bf16" and w.d >= 128 and w.H >= 128) or w.act == "mxfp8"


def backward_steps(w, p, d_in, packed, f, dev, steps: int, warmup: int, ms_device: float) -> dict:
    """moe_backward of the last forward (f's workspace), timed like the main loop.

    Useful FLOPs (the arithmetic the block's gradients require, recompute
    excluded): the data gradients 2 R d H (down) + 4 R d H (gate/up), the
    weight gradients 2 R d H + 4 R d H, plus the router's 2 T d E twice for the
    learned router.  Executed FLOPs add the gate/up recompute's 4 R d H."""
    packed_bwd = B.pack_weights_backward(p, d_in["w_gate"], d_in["w_up"], d_in["w_down"])
    g = torch.Generator(device="cpu").manual_seed(w.seed + 17)
    dy = torch.randn((w.T, w.d), generator=g).to(B.storage_dtype(w.act)).to(dev)
    bwd = B.Backward(p, dev)
    ms = _timed(lambda: bwd(f, dy, packed, packed_bwd, x=d_in["x"], w_router=d_in["w_router"]), steps, warmup)
    router = 2 * 2.0 * w.T * w.d * w.E if w.router == "learned" else 0.0
    useful = 12.0 * w.R * w.d * w.H + router
    executed = useful + 4.0 * w.R * w.d * w.H
    peak = 157.3 if w.act == "f32" else 2500.0   # MXFP8 blocks run their backward in bf16
    tf = useful / (ms * 1e-3) / 1e12
    return {"ms_per_step": round(ms, 5), "tokens_per_s": round(w.T / (ms * 1e-3), 1),
            "useful_tflops": round(tf, 2), "frac_of_peak": round(tf / peak, 4),
            "executed_tflops": round(executed / (ms * 1e-3) / 1e12, 2),
            "peak_tflops": peak, "vs_forward": round(ms / ms_device, 3)}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default=DEFAULT_CONFIG, choices=sorted(W.ALL))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--main-only", action="store_true",
                    help="skip the comparison measurements (cold cache, host-synchronising path, router "
                         "statistics), e.g. under a profiler")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one step captured in a HIP graph instead of eager launches")
    ap.add_argument("--with-backward", action="store_true",
                    help="also time moe_backward when --main-only is given")
    ap.add_argument("--calibration-copy-mb", type=int, default=0,
                    help="before the timed steps, run one plain device copy of this many MiB (a known "
                         "byte count that calibrates HBM counters such as FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the routed block: this build has no "
              "multi-GPU path (no collectives, no sharding); run with --gpus 1.", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        return 2
    dev = "cuda:0"
    w = W.ALL[args.config]
    host = W.make_inputs(w)
    d_in = {k: (None if v is None else v.to(dev)) for k, v in host.items()}
    p = B.problem(w.T, w.d, w.E, w.k, w.H, w.act, logits_given=w.router != "learned")
    packed = B.pack_weights(p, d_in["w_gate"], d_in["w_up"], d_in["w_down"])
    f = B.Forward(p, dev, debug_outputs=False)
    if p.flags & B.MOE_LOGITS_GIVEN:
        f.logits.copy_(d_in["logits"])

    def step():
        f(d_in["x"], packed=packed, w_router=d_in["w_router"], logits=f.logits)

    for _ in range(args.warmup):
        step()
    if args.calibration_copy_mb > 0:
        n = args.calibration_copy_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    torch.cuda.synchronize()
    # per-stage breakdown: K eager steps with the library's HIP events between kernels
    B.set_profiling(True)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    ms_eager = start.elapsed_time(stop) / args.steps
    stages = B.kernel_times()
    B.set_profiling(False)
    # the timed K steps, without profiling events: eager launches, or with
    # --graph replays of one step captured in a HIP graph (fixed buffer addresses)
    run = step
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(3):
            graph.replay()
        run = graph.replay
    torch.cuda.synchronize()
    start.record()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = start.elapsed_time(stop)
    ms_step = ms_total / args.steps

    models = stage_models(w)
    stage_out = stage_rooflines(models, stages)
    dom = max(stages, key=lambda s: s[1])[0]
    traffic = measured_traffic(w.name, dom)
    gemm_ms = sum(ms for n, ms in stages if n.startswith("gemm") or n == "grouped_ffn")
    disp_alone = None if "dispatch" in stage_out else dispatch_standalone(p, d_in, dev, models)
    bound_ms = block_bound_ms(w, models)
    gemm_peak = models["gemm1_gate_up_swiglu"][3]
    flops = w.expert_flops + w.router_flops
    result = {
        "metric": METRIC,
        "value": round(w.T * args.steps / (ms_total * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.act,
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02^2) weights)",
        "config": {"workload": w.describe(), "T": w.T, "d_model": w.d, "n_experts": w.E, "top_k": w.k,
                   "d_hidden": w.H, "router": w.router, "parallelism": "single GPU"},
        "roofline": roofline_entry(models, stage_out, dom, traffic),
        "block_tflops": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "block_roofline": {"bound_ms": round(bound_ms, 5), "frac": round(bound_ms / ms_step, 4),
                           "note": "sum of each step's algorithmic work at its peak (HBM 8 TB/s, MFMA dense peak)"},
        "grouped_gemm_frac_of_peak": round(6.0 * w.R * w.d * w.H / (gemm_ms * 1e-3) / 1e12 / gemm_peak, 4)
        if gemm_ms > 0 else None,
        "dispatch_frac_of_hbm": (stage_out["dispatch"] if disp_alone is None else disp_alone)["frac"]
        if "dispatch" in stage_out or disp_alone is not None else None,
        "combine_frac_of_hbm": stage_out.get("combine", {}).get("frac"),
        "launch": "HIP graph replay, one moe_forward per step" if args.graph else "eager, one moe_forward per step",
        "ms_per_step_with_stage_events": round(ms_eager, 5),
        "stages": stage_out,
        **({"dispatch_standalone": disp_alone} if disp_alone is not None else {}),
        "host_wall_s": round(wall, 4),
    }
    if not args.main_only:
        result["cold_cache"] = cold_cache_steps(step, dev, args.steps)
        result["copy_ceiling"] = copy_ceiling(step, dev, models)
        result["host_sync_variant"] = host_sync_steps(p, d_in, packed, dev, args.steps, args.warmup, ms_step)
        result["determinism"] = determinism_check(step, f)
        result["with_router_stats"] = router_stats_steps(p, d_in, packed, dev, args.steps, args.warmup, ms_step)
        result["backward"] = backward_steps(w, p, d_in, packed, f, dev, args.steps, args.warmup, ms_step)
    elif args.with_backward:
        result["backward"] = backward_steps(w, p, d_in, packed, f, dev, args.steps, args.warmup, ms_step)
    if "backward" in result and keeps_gate_up(w):
        result["kept_gate_up"] = kept_gate_up_steps(w, d_in, packed, dev, args.steps, args.warmup, ms_step,
                                                    result["backward"])
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, host)
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
