"""Seeded synthetic inputs for the top-k routed MoE layer forward.

This module is shared by the tests, the benchmark and the smoke check. It
draws tensors and converts their storage format. It holds none of the layer's
arithmetic: no routing, no expert FFN and no combine.

Workload shapes follow the models the MoE pages describe. The layer is the
``MoE(d, d_ff, n_experts, top_k, n_shared)`` module from "混合专家 MoE"
(anrans ai-infra handbook), section "实现：逐 token 与按专家分组" (moe.py).
The shapes are:

* tiny          fp32, N=64, d=128, d_ff=256, E=8, k=2, 1 shared expert
* mixtral       bf16, N=4096, d=4096, d_ff=14336, E=8, k=2 (Mixtral 8x7B-shaped prefill)
* dsv3_prefill  bf16, N=8192, d=7168, d_ff=2048, E=256, k=8, 1 shared expert,
                selection-only bias (DeepSeek-V3-shaped; the handbook's
                "负载均衡" section describes the aux-loss-free bias)
* dsv3_decode   the dsv3_prefill layer with N=64 (the first 64 rows of its x)
* switch_cap    bf16, N=16384, d=2048, d_ff=8192, E=128, k=1, capacity 160 with
                a Zipf-like logit skew (Switch-style capacity and dropping, from
                the notes' section "容量因子 (Capacity Factor) 与 Token 丢弃策略")
* p2_shape      fp32, N=50, d=64, d_ff=128, E=16, k=4, 1 shared expert (the
                handbook's own naive-vs-grouped check)

Value recipe, shared by every layer:

* x ~ N(0, 1)
* router W_r ~ N(0, 1/d)
* gate and up ~ N(0, 1/d)
* down ~ N(0, 1/d_ff)
* shared experts use the same recipe

The second argument of N is the variance. Every tensor has its own
``numpy.random.SeedSequence(seed, spawn_key=(layer, tensor, index))`` stream,
so any one expert, or any 64-row block of x, can be regenerated alone. Draws
are fp32. bf16 layers round them to bf16 (round to nearest, ties to even) and
keep the raw 16-bit patterns (``uint16``).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional

import numpy as np

X_BLOCK_ROWS = 64  # x is drawn in blocks of this many rows, one stream each

# tensor ids inside a layer's seed tree
_T_ROUTER, _T_GATE, _T_UP, _T_DOWN = 1, 2, 3, 4
_T_SGATE, _T_SUP, _T_SDOWN = 5, 6, 7
_T_SELECT_BIAS, _T_SKEW_PERM = 8, 9
_T_X = 10


@dataclass(frozen=True)
class MoEConfig:
    name: str
    n_tokens: int
    d_model: int
    d_ff: int
    n_experts: int
    top_k: int
    n_shared: int = 0
    d_ff_shared: int = 0
    capacity: int = 0            # <= 0: unlimited
    dtype: str = "bf16"          # "bf16" or "f32" (x and every weight)
    select_bias: float = 0.0     # > 0: b ~ U(-v, v), used for selection only
    logit_skew: float = 0.0      # > 0: logit_bias = v * ln(1/rank) over a seeded permutation
    renormalize: bool = True
    layer_id: int = 0            # seed tree of the layer tensors
    x_id: int = 0                # seed tree of x
    seed: int = 0

    @property
    def copies(self) -> int:
        return self.n_tokens * self.top_k


def capacity_for(n_tokens: int, top_k: int, n_experts: int, factor: float) -> int:
    """C = ceil(factor * N * k / E), the per-expert buffer size."""
    return int(math.ceil(factor * n_tokens * top_k / n_experts))


CONFIGS: Dict[str, MoEConfig] = {
    "tiny": MoEConfig("tiny", 64, 128, 256, 8, 2, n_shared=1, d_ff_shared=256,
                      dtype="f32", layer_id=100, x_id=100),
    "mixtral": MoEConfig("mixtral", 4096, 4096, 14336, 8, 2, layer_id=101, x_id=101),
    "dsv3_prefill": MoEConfig("dsv3_prefill", 8192, 7168, 2048, 256, 8, n_shared=1,
                              d_ff_shared=2048, select_bias=0.1, layer_id=102, x_id=102),
    # same layer tensors and same x stream as dsv3_prefill: x = its first 64 rows
    "dsv3_decode": MoEConfig("dsv3_decode", 64, 7168, 2048, 256, 8, n_shared=1,
                             d_ff_shared=2048, select_bias=0.1, layer_id=102, x_id=102),
    "switch_cap": MoEConfig("switch_cap", 16384, 2048, 8192, 128, 1,
                            capacity=capacity_for(16384, 1, 128, 1.25),
                            logit_skew=1.5, layer_id=104, x_id=104),
    "p2_shape": MoEConfig("p2_shape", 50, 64, 128, 16, 4, n_shared=1, d_ff_shared=128,
                          dtype="f32", layer_id=105, x_id=105),
}


# ---------------------------------------------------------------- storage format

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the same values as fp32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(a: np.ndarray) -> np.ndarray:
    """Stored tensor (uint16 bf16 bits or fp32) -> fp64 values, exactly."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------- streams

def _rng(cfg: MoEConfig, tree: int, tensor: int, index: int) -> np.random.Generator:
    ss = np.random.SeedSequence(cfg.seed, spawn_key=(tree, tensor, index))
    return np.random.Generator(np.random.PCG64(ss))


def _normal(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    z = np.empty(shape, dtype=np.float32)
    rng.standard_normal(out=z, dtype=np.float32)
    z *= np.float32(std)
    return f32_to_bf16_bits(z) if dtype == "bf16" else z


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ---------------------------------------------------------------- public API

@dataclass
class Layer:
    """One layer's weights in storage format (uint16 bf16 bits or fp32)."""
    cfg: MoEConfig
    w_router: np.ndarray                      # [E, d]
    w_gate: np.ndarray                        # [E, d_ff, d]
    w_up: np.ndarray                          # [E, d_ff, d]
    w_down: np.ndarray                        # [E, d, d_ff]
    s_gate: Optional[np.ndarray] = None       # [S, d_ff_s, d]
    s_up: Optional[np.ndarray] = None         # [S, d_ff_s, d]
    s_down: Optional[np.ndarray] = None       # [S, d, d_ff_s]
    logit_bias: Optional[np.ndarray] = None   # [E] fp32, added to the logits
    select_bias: Optional[np.ndarray] = None  # [E] fp32, selection only


def make_router(cfg: MoEConfig) -> np.ndarray:
    return _normal(_rng(cfg, cfg.layer_id, _T_ROUTER, 0), (cfg.n_experts, cfg.d_model),
                   cfg.d_model ** -0.5, cfg.dtype)


def make_expert(cfg: MoEConfig, e: int, shared: bool = False):
    """(gate [d_ff, d], up [d_ff, d], down [d, d_ff]) of routed expert e, or shared expert e."""
    d = cfg.d_model
    f = cfg.d_ff_shared if shared else cfg.d_ff
    tg, tu, td = (_T_SGATE, _T_SUP, _T_SDOWN) if shared else (_T_GATE, _T_UP, _T_DOWN)
    g = _normal(_rng(cfg, cfg.layer_id, tg, e), (f, d), d ** -0.5, cfg.dtype)
    u = _normal(_rng(cfg, cfg.layer_id, tu, e), (f, d), d ** -0.5, cfg.dtype)
    dn = _normal(_rng(cfg, cfg.layer_id, td, e), (d, f), f ** -0.5, cfg.dtype)
    return g, u, dn


def make_biases(cfg: MoEConfig):
    """(logit_bias, select_bias), each fp32 [E] or None.

    logit_bias[e] = skew * ln(1 / rank_e), rank_e = 1 + position of e in a
    seeded permutation of the experts (a Zipf-like preference).
    select_bias[e] ~ U(-v, v).
    """
    E = cfg.n_experts
    lb = sb = None
    if cfg.logit_skew > 0:
        perm = _rng(cfg, cfg.layer_id, _T_SKEW_PERM, 0).permutation(E)
        rank = np.empty(E, dtype=np.float64)
        rank[perm] = np.arange(1, E + 1, dtype=np.float64)
        lb = (cfg.logit_skew * np.log(1.0 / rank)).astype(np.float32)
    if cfg.select_bias > 0:
        v = cfg.select_bias
        sb = _rng(cfg, cfg.layer_id, _T_SELECT_BIAS, 0).uniform(-v, v, size=E).astype(np.float32)
    return lb, sb


def make_layer(cfg: MoEConfig, workers: Optional[int] = None) -> Layer:
    E, d, f = cfg.n_experts, cfg.d_model, cfg.d_ff
    st = np.uint16 if cfg.dtype == "bf16" else np.float32
    wg = np.empty((E, f, d), dtype=st)
    wu = np.empty((E, f, d), dtype=st)
    wd = np.empty((E, d, f), dtype=st)

    def fill(e):
        wg[e], wu[e], wd[e] = make_expert(cfg, e)

    with ThreadPoolExecutor(workers or _workers()) as ex:
        list(ex.map(fill, range(E)))
    lay = Layer(cfg, make_router(cfg), wg, wu, wd)
    if cfg.n_shared > 0:
        fs = cfg.d_ff_shared
        lay.s_gate = np.empty((cfg.n_shared, fs, d), dtype=st)
        lay.s_up = np.empty((cfg.n_shared, fs, d), dtype=st)
        lay.s_down = np.empty((cfg.n_shared, d, fs), dtype=st)
        for s in range(cfg.n_shared):
            lay.s_gate[s], lay.s_up[s], lay.s_down[s] = make_expert(cfg, s, shared=True)
    lay.logit_bias, lay.select_bias = make_biases(cfg)
    return lay


def make_x(cfg: MoEConfig, workers: Optional[int] = None) -> np.ndarray:
    """x [N, d], drawn in 64-row blocks (block b has its own stream)."""
    N, d = cfg.n_tokens, cfg.d_model
    st = np.uint16 if cfg.dtype == "bf16" else np.float32
    x = np.empty((N, d), dtype=st)
    nb = (N + X_BLOCK_ROWS - 1) // X_BLOCK_ROWS

    def fill(b):
        r0 = b * X_BLOCK_ROWS
        r1 = min(N, r0 + X_BLOCK_ROWS)
        blk = _normal(_rng(cfg, cfg.x_id, _T_X, b), (X_BLOCK_ROWS, d), 1.0, cfg.dtype)
        x[r0:r1] = blk[: r1 - r0]

    with ThreadPoolExecutor(workers or _workers()) as ex:
        list(ex.map(fill, range(nb)))
    return x


def small_config(name: str = "case", **kw) -> MoEConfig:
    """A custom config for tests (fresh seed trees unless given)."""
    base = dict(name=name, n_tokens=37, d_model=64, d_ff=64, n_experts=6, top_k=2,
                layer_id=900, x_id=900)
    base.update(kw)
    return MoEConfig(**base)


def with_(cfg: MoEConfig, **kw) -> MoEConfig:
    return replace(cfg, **kw)

