"""Host-side logic of bench.py (no GPU): the per-stage work model, the
roofline object of the JSON line and the block's roofline time.

The expected totals are the algorithmic work per forward of the four large
blocks, computed from their shapes: expert FLOP 6 R d H, dispatch bytes
T d b_x + R d b_xe (+ R d / 32 scale bytes) + 16 R (ranks and expert ids in,
positions and row_token out), combine bytes R d b_ye + 8 R + T d b_y."""
import pytest

import bench
from routing_dispatch_grouped_router_amd import workloads as W

TOTALS = {   # expert GFLOP, dispatch MB, combine MB, block roofline ms at peak
    "bf16_e8": (412.3, 168.3, 168.0, 0.2113),
    "bf16_e128_random": (824.6, 336.6, 336.1, 0.4151),
    "bf16_e64_zipf": (4947.8, 1210.1, 1209.0, 2.2823),
    "mxfp8_e128": (1649.3, 413.1, 672.1, 0.4679),
}


@pytest.mark.parametrize("name", list(TOTALS))
def test_stage_models_match_the_block_totals(name):
    w = W.CONFIGS[name]
    m = bench.stage_models(w)
    gflop, disp_mb, comb_mb, _ = TOTALS[name]
    assert m["gemm1_gate_up_swiglu"][1] + m["gemm2_down"][1] == pytest.approx(gflop * 1e9, rel=1e-3)
    assert m["grouped_ffn"][1] == pytest.approx(gflop * 1e9, rel=1e-3)
    assert m["dispatch"][1] == pytest.approx(disp_mb * 1e6, rel=2e-3)
    assert m["combine"][1] == pytest.approx(comb_mb * 1e6, rel=1e-3)
    peak = 5000.0 if w.act == "mxfp8" else 2500.0
    assert m["grouped_ffn"][2:] == ("TFLOP/s", peak)
    assert m["combine"][2:] == ("GB/s", 8000.0)


@pytest.mark.parametrize("name", list(TOTALS))
def test_block_bound(name):
    w = W.CONFIGS[name]
    assert bench.block_bound_ms(w, bench.stage_models(w)) == pytest.approx(TOTALS[name][3], rel=1e-3)


def test_roofline_entry_takes_the_dominant_kernels_own_peak():
    w = W.CONFIGS["bf16_e64_zipf"]
    m = bench.stage_models(w)
    stages = [("route_topk", 0.0175), ("route_scan", 0.0079), ("grouped_ffn", 4.132), ("combine", 0.2145)]
    out = bench.stage_rooflines(m, stages)
    r = bench.roofline_entry(m, out, "grouped_ffn", 123)
    assert (r["bound"], r["unit"], r["peak"], r["traffic"]) == ("mfma", "TFLOP/s", 2500.0, 123)
    assert r["achieved"] == pytest.approx(6.0 * w.R * w.d * w.H / 4.132e-3 / 1e12, rel=1e-4)
    assert r["frac"] == pytest.approx(r["achieved"] / 2500.0, abs=1e-4)
    c = out["combine"]
    assert (c["unit"], c["peak"]) == ("GB/s", 8000.0)
    assert c["frac"] == pytest.approx(m["combine"][1] / 0.2145e-3 / 1e9 / 8000.0, abs=1e-4)
