"""Helpers for the GPU parity tests: the oracle on the same seeded inputs, and
the comparison rules.

The rules:
* Routing. The GPU top-k must equal the oracle's on every token whose fp64
  gap s_(k) - s_(k+1) is at least 1e-6. Fewer than 0.1% of tokens may differ,
  and each one must be such a near-tie.
* Integer outputs (counts, offsets, perm, slot_pos, the dropped set). These
  must be bit-exact against the oracle's grouping of the GPU's own top-k
  (forced routing).
* y. Per row, max |y_gpu - y_ref| <= 1e-2 * rms(y_ref row). y_ref is the
  forced-routing oracle. A row whose reference is all zero must be exactly
  zero.
* prob_sum. Relative error <= 1e-5 per expert. The balance statistic is
  within 1e-6 relative.
"""
from __future__ import annotations

import numpy as np
import torch

import moe_inputs as mi
from oracle import moe_oracle as O

NEAR_TIE = 1e-6
Y_TOL = 1e-2


class F64View:
    """Indexable view of a stacked weight tensor that upcasts one expert at a time, cached."""

    def __init__(self, arr, cache=True):
        self.arr = arr
        self.cache = {} if cache else None

    def __len__(self):
        return len(self.arr)

    def __getitem__(self, e):
        e = int(e)
        if self.cache is None:
            return mi.to_f64(self.arr[e])
        if e not in self.cache:
            self.cache[e] = mi.to_f64(self.arr[e])
        return self.cache[e]


class Fp8View(F64View):
    """Like F64View, but each expert matrix is quantised to FP8 by the oracle
    (per-row scales) and dequantised: the weights the FP8 layer computes with."""

    def __getitem__(self, e):
        e = int(e)
        if self.cache is not None and e in self.cache:
            return self.cache[e]
        codes, scales = O.quantize_fp8_rows(mi.bf16_bits_to_f32(self.arr[e]))
        w = O.dequantize_fp8_rows(codes, scales)
        if self.cache is not None:
            self.cache[e] = w
        return w


class Int4View(F64View):
    """Like F64View, but each expert matrix is quantised to int4 by the oracle
    (per-row scales) and dequantised: the weights the int4 layer computes with."""

    def __getitem__(self, e):
        e = int(e)
        if self.cache is not None and e in self.cache:
            return self.cache[e]
        codes, scales = O.quantize_int4_rows(mi.bf16_bits_to_f32(self.arr[e]))
        w = O.dequantize_int4_rows(codes, scales)
        if self.cache is not None:
            self.cache[e] = w
        return w


def oracle_views(layer: mi.Layer, cache_routed=False, fp8=False, quant=None):
    """quant: None (the stored weights), "fp8" or "int4" (fp8=True means "fp8")."""
    quant = "fp8" if fp8 else quant
    V = {None: F64View, "fp8": Fp8View, "int4": Int4View}[quant]
    ws = tuple(V(a, cache=cache_routed) for a in (layer.w_gate, layer.w_up, layer.w_down))
    shared = None
    if layer.s_gate is not None:
        shared = tuple(V(a) for a in (layer.s_gate, layer.s_up, layer.s_down))
    return ws, shared


def oracle_route(cfg: mi.MoEConfig, layer: mi.Layer, x: np.ndarray) -> O.Routing:
    return O.route(mi.to_f64(x), mi.to_f64(layer.w_router), cfg.top_k, layer.logit_bias,
                   layer.select_bias, cfg.renormalize)


def oracle_y(cfg, layer, x, idx, rows, form, routing: O.Routing = None, fp8=False, quant=None):
    """Forced-routing oracle output on `rows` for the given idx (quant "fp8"/"int4": quantised
    expert weights; fp8=True means "fp8")."""
    (wg, wu, wd), shared = oracle_views(layer, cache_routed=(form == "per_token"), fp8=fp8, quant=quant)
    x64 = mi.to_f64(x)
    if routing is None:
        routing = oracle_route(cfg, layer, x)
    idx = np.asarray(idx, dtype=np.int64)
    w = np.take_along_axis(routing.probs, idx, axis=1)
    if cfg.renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    g = O.group(idx, cfg.n_experts, cfg.capacity)
    round_h = cfg.dtype == "bf16"
    if form == "per_token":
        return O.forward_per_token(x64, idx, w, g.slot_pos >= 0, wg, wu, wd, shared=shared,
                                   round_h=round_h, rows=rows)
    return O.forward_grouped(x64, idx, w, g, wg, wu, wd, shared=shared, round_h=round_h, rows=rows)


def check_routing(gpu_idx: np.ndarray, ref: O.Routing):
    """Returns the number of tokens whose top-k differs (all near-ties)."""
    N = gpu_idx.shape[0]
    mism = np.any(gpu_idx != ref.idx, axis=1)
    n = int(mism.sum())
    if n:
        gaps = ref.gap[mism]
        assert np.all(gaps < NEAR_TIE), f"top-k differs on tokens with gap >= 1e-6: {gaps[gaps >= NEAR_TIE]}"
        assert n < 1e-3 * N, f"{n} of {N} tokens differ (limit: < 0.1%)"
    return n


def check_weights(gpu_w, gpu_idx, ref: O.Routing, renormalize=True):
    same = np.all(gpu_idx == ref.idx, axis=1)
    np.testing.assert_allclose(gpu_w[same], ref.w[same], rtol=2e-5, atol=1e-7)


def check_grouping(gpu, idx, E, C):
    g = O.group(idx, E, C)
    np.testing.assert_array_equal(gpu["counts"], g.counts)
    np.testing.assert_array_equal(gpu["offsets"], g.offsets)
    nk = int(g.offsets[-1])
    np.testing.assert_array_equal(gpu["perm"][:nk], g.perm)
    np.testing.assert_array_equal(gpu["slot_pos"], g.slot_pos)
    return g


def check_y(y_gpu: np.ndarray, y_ref: np.ndarray, tol=Y_TOL):
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    err = np.max(np.abs(y_gpu - y_ref), axis=1)
    rms = np.sqrt(np.mean(y_ref ** 2, axis=1))
    zero = rms == 0
    assert np.all(y_gpu[zero] == 0), "rows with an all-zero reference must be exactly zero"
    bad = ~zero & (err > tol * rms)
    assert not np.any(bad), (f"{bad.sum()} rows exceed {tol}*rms; worst ratio "
                             f"{np.max(err[~zero] / rms[~zero]):.3e}")
    return float(np.max(err[~zero] / rms[~zero])) if np.any(~zero) else 0.0


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def sample_rows(N: int, n: int, seed: int = 1234) -> np.ndarray:
    """A seeded sample of rows that always includes the first and last row."""
    if n >= N:
        return np.arange(N)
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(N, size=n - 2, replace=False).tolist()) | {0, N - 1}
    return np.array(sorted(rows))
