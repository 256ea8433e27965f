"""Workload shapes and seeded synthetic inputs for the routed MoE block.

This module holds no step of the block's computation: it only draws inputs.
Both the HIP path's tests/benchmark and the CPU oracle are fed from it.

Draws use NumPy's PCG64 (``default_rng(seed)``) in float32, in the order
x, router weights (or router logits), W_gate, W_up, W_down, outlier mask.
Values that are stored in bfloat16 are rounded to nearest-even by torch.
Weights are N(0, 0.02^2), activations N(0, 1).  No value is zero-filled or
constant: GEMM timings depend on operand values (report Section 24.2 /
Evidence 8 measured a large swing between random and all-zero operands).
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

ACT_F32, ACT_BF16, ACT_MXFP8 = "f32", "bf16", "mxfp8"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int              # tokens
    d: int              # d_model
    E: int              # experts
    k: int              # top-k
    H: int              # expert SwiGLU hidden size
    act: str            # 'f32' | 'bf16' | 'mxfp8'
    router: str         # 'learned' (L = x W_r) | 'random' (i.i.d. N(0,1) logits) | 'zipf'
    seed: int
    zipf_s: float = 1.2
    outlier_frac: float = 0.0     # fraction of activations multiplied by outlier_scale
    outlier_scale: float = 64.0
    empty_experts: tuple = ()     # experts whose logits get -1e4 (forced empty)
    tie_levels: int = 0           # >0: logits drawn from this many integer levels (planted ties)

    @property
    def R(self) -> int:
        return self.T * self.k

    @property
    def expert_flops(self) -> float:
        """Useful FLOPs of the expert FFNs: 2*R*d*2H (gate+up) + 2*R*H*d (down)."""
        return 6.0 * self.R * self.d * self.H

    @property
    def router_flops(self) -> float:
        return 2.0 * self.T * self.d * self.E if self.router == "learned" else 0.0

    def describe(self) -> str:
        return (f"{self.name}: {self.act} T={self.T} d={self.d} E={self.E} k={self.k} "
                f"H={self.H} router={self.router}")


# The five block configurations the kernels are built and measured for.
CONFIGS = {
    "tiny_f32": Workload("tiny_f32", T=256, d=128, E=8, k=2, H=256, act=ACT_F32,
                         router="learned", seed=1001),
    "bf16_e8": Workload("bf16_e8", T=8192, d=2048, E=8, k=4, H=1024, act=ACT_BF16,
                        router="learned", seed=1002),
    "bf16_e128_random": Workload("bf16_e128_random", T=16384, d=2048, E=128, k=4, H=1024,
                                 act=ACT_BF16, router="random", seed=1003),
    "bf16_e64_zipf": Workload("bf16_e64_zipf", T=16384, d=4096, E=64, k=8, H=1536,
                              act=ACT_BF16, router="zipf", seed=1004),
    "mxfp8_e128": Workload("mxfp8_e128", T=32768, d=2048, E=128, k=4, H=1024, act=ACT_MXFP8,
                           router="random", seed=1005, outlier_frac=0.01),
}
CONFIG_ORDER = ["tiny_f32", "bf16_e8", "bf16_e128_random", "bf16_e64_zipf", "mxfp8_e128"]

# Small cases for parity at sizes the oracle finishes in seconds, and edge cases.
SMALL = {
    "small_bf16_e8": Workload("small_bf16_e8", T=1000, d=256, E=8, k=4, H=192, act=ACT_BF16,
                              router="learned", seed=2001),
    "small_bf16_e32_random": Workload("small_bf16_e32_random", T=777, d=384, E=32, k=4, H=320,
                                      act=ACT_BF16, router="random", seed=2002),
    "small_bf16_zipf": Workload("small_bf16_zipf", T=1500, d=256, E=16, k=8, H=128,
                                act=ACT_BF16, router="zipf", seed=2003),
    "small_mxfp8": Workload("small_mxfp8", T=600, d=256, E=16, k=4, H=256, act=ACT_MXFP8,
                            router="random", seed=2004, outlier_frac=0.01),
    "small_f32_learned": Workload("small_f32_learned", T=333, d=192, E=12, k=3, H=128,
                                  act=ACT_F32, router="learned", seed=2005),
    "edge_empty_experts": Workload("edge_empty_experts", T=200, d=128, E=8, k=2, H=128,
                                   act=ACT_BF16, router="random", seed=2006,
                                   empty_experts=(0, 3, 7)),
    "edge_tk_lt_E": Workload("edge_tk_lt_E", T=3, d=64, E=16, k=2, H=64, act=ACT_BF16,
                             router="random", seed=2007),
    "edge_one_token": Workload("edge_one_token", T=1, d=128, E=4, k=4, H=64, act=ACT_F32,
                               router="random", seed=2008),
    "edge_k_eq_E": Workload("edge_k_eq_E", T=130, d=64, E=4, k=4, H=128, act=ACT_BF16,
                            router="random", seed=2009),
    "edge_dense_E1": Workload("edge_dense_E1", T=257, d=192, E=1, k=1, H=320, act=ACT_F32,
                              router="random", seed=2010),
    "edge_ties": Workload("edge_ties", T=2048, d=64, E=64, k=8, H=64, act=ACT_BF16,
                          router="random", seed=2011, tie_levels=3),
    "edge_mxfp8_empty": Workload("edge_mxfp8_empty", T=70, d=128, E=8, k=2, H=128,
                                 act=ACT_MXFP8, router="random", seed=2012,
                                 empty_experts=(1, 6), outlier_frac=0.05),
    # learned routers whose expert count is not a multiple of 8 (W_r transposed first) or
    # spans several 16-expert tiles of the router GEMM
    "small_bf16_learned_e12": Workload("small_bf16_learned_e12", T=600, d=256, E=12, k=3, H=128,
                                       act=ACT_BF16, router="learned", seed=2016),
    "small_bf16_learned_e20": Workload("small_bf16_learned_e20", T=700, d=384, E=20, k=4, H=128,
                                       act=ACT_BF16, router="learned", seed=2017),
    "small_bf16_learned_e64": Workload("small_bf16_learned_e64", T=900, d=256, E=64, k=6, H=128,
                                       act=ACT_BF16, router="learned", seed=2018),
    "small_mxfp8_learned_e20": Workload("small_mxfp8_learned_e20", T=500, d=256, E=20, k=2, H=128,
                                        act=ACT_MXFP8, router="learned", seed=2019, outlier_frac=0.01),
    "small_mxfp8_learned_e64": Workload("small_mxfp8_learned_e64", T=400, d=384, E=64, k=4, H=256,
                                        act=ACT_MXFP8, router="learned", seed=2020),
    # the largest expert count and top-k the library supports (1024, 16): many tiny segments
    "edge_max_E_k": Workload("edge_max_E_k", T=700, d=64, E=1024, k=16, H=64, act=ACT_BF16,
                             router="random", seed=2013),
    "edge_max_E_k_learned_f32": Workload("edge_max_E_k_learned_f32", T=300, d=64, E=1024, k=16, H=64,
                                         act=ACT_F32, router="learned", seed=2014),
    "edge_max_E_k_mxfp8": Workload("edge_max_E_k_mxfp8", T=500, d=128, E=1024, k=16, H=128,
                                   act=ACT_MXFP8, router="random", seed=2015),
}

ALL = {**CONFIGS, **SMALL}


def get(name: str) -> Workload:
    return ALL[name]


def scaled(w: Workload, T: int) -> Workload:
    """Same workload with a different token count (for bounded samples)."""
    return dataclasses.replace(w, name=f"{w.name}[T={T}]", T=T)


def _storage_dtype(act: str) -> torch.dtype:
    return torch.float32 if act == ACT_F32 else torch.bfloat16


def _to_storage(a: np.ndarray, act: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t if act == ACT_F32 else t.to(torch.bfloat16)


def make_inputs(w: Workload, seed: int | None = None) -> dict:
    """Seeded synthetic inputs on the host as torch CPU tensors.

    x [T, d] and the expert weights W_gate/W_up [E, d, H], W_down [E, H, d] are
    float32 for act 'f32' and bfloat16 otherwise (MXFP8 weights are quantised
    from these bfloat16 values by the library's weight packing).  Router weights
    W_r [d, E] (learned router) share that dtype; router logits [T, E] (random
    and Zipf routers) are float32.
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    x = rng.standard_normal((w.T, w.d), dtype=np.float32)
    w_router = None
    logits = None
    if w.router == "learned":
        w_router = rng.standard_normal((w.d, w.E), dtype=np.float32) * np.float32(0.02)
    else:
        if w.tie_levels:
            logits = rng.integers(0, w.tie_levels, size=(w.T, w.E)).astype(np.float32)
            # also plant signed zeros, which must compare equal
            logits[logits == 0] = np.where(rng.random((logits == 0).sum()) < 0.5, -0.0, 0.0)
        else:
            logits = rng.standard_normal((w.T, w.E), dtype=np.float32)
        if w.router == "zipf":
            ranks = np.arange(1, w.E + 1, dtype=np.float64)
            weight = ranks ** (-w.zipf_s)
            bias = np.log(weight / weight.sum())          # log of the Zipf rank weight
            logits = (logits.astype(np.float64) + bias[None, :]).astype(np.float32)
        for e in w.empty_experts:
            logits[:, e] = np.float32(-1e4)
    w_gate = rng.standard_normal((w.E, w.d, w.H), dtype=np.float32) * np.float32(0.02)
    w_up = rng.standard_normal((w.E, w.d, w.H), dtype=np.float32) * np.float32(0.02)
    w_down = rng.standard_normal((w.E, w.H, w.d), dtype=np.float32) * np.float32(0.02)
    if w.outlier_frac > 0:
        mask = rng.random((w.T, w.d)) < w.outlier_frac
        x = np.where(mask, x * np.float32(w.outlier_scale), x).astype(np.float32)
    if w.router == "learned" and w.empty_experts:
        raise ValueError("forced-empty experts need given logits")
    return dict(
        x=_to_storage(x, w.act),
        w_router=None if w_router is None else _to_storage(w_router, w.act),
        logits=None if logits is None else torch.from_numpy(logits),
        w_gate=_to_storage(w_gate, w.act),
        w_up=_to_storage(w_up, w.act),
        w_down=_to_storage(w_down, w.act),
    )


def as_f64(t: torch.Tensor | None) -> np.ndarray | None:
    """Exact float64 values of a stored tensor (for feeding the oracle)."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()


def mean_rows_per_expert(w: Workload) -> float:
    return w.R / w.E


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


__all__ = ["Workload", "CONFIGS", "CONFIG_ORDER", "SMALL", "ALL", "get", "scaled",
           "make_inputs", "as_f64", "ceil_div"]
