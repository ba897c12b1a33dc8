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
  zero. Where an element of h lies so close to a bf16 midpoint that an fp32
  evaluation may round it either way (oracle h_rounding_band), both
  roundings are correct: a row that fails the bound passes if some choice
  of roundings for exactly those elements (oracle y_rounding_flips) brings
  it within the bound. A row with no such element gets no slack.
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
    expert weights; fp8=True means "fp8"). The oracle's own forced-routing mode gives the
    weights and the grouping."""
    (wg, wu, wd), shared = oracle_views(layer, cache_routed=(form == "per_token"), fp8=fp8, quant=quant)
    return O.moe_layer(mi.to_f64(x), mi.to_f64(layer.w_router), wg, wu, wd, cfg.top_k, shared=shared,
                       logit_bias=layer.logit_bias, select_bias=layer.select_bias, capacity=cfg.capacity,
                       renormalize=cfg.renormalize, round_h=(cfg.dtype == "bf16"), form=form, rows=rows,
                       forced_idx=np.asarray(idx, dtype=np.int64)).y


def rounding_flips(cfg, layer, x, idx, fp8=False, quant=None):
    """t -> the ambiguous h elements of token t's row and how each moves y_t (oracle
    y_rounding_flips), under the forced routing idx. None for fp32 layers (h is not rounded)."""
    if cfg.dtype != "bf16":
        return None
    quant = "fp8" if fp8 else quant
    (wg, wu, wd), shared = oracle_views(layer, fp8=fp8, quant=quant)
    res = O.moe_layer(mi.to_f64(x), mi.to_f64(layer.w_router), wg, wu, wd, cfg.top_k,
                      logit_bias=layer.logit_bias, select_bias=layer.select_bias, capacity=cfg.capacity,
                      renormalize=cfg.renormalize, form="none", forced_idx=np.asarray(idx, dtype=np.int64))
    k = cfg.top_k
    x64 = mi.to_f64(x)

    def flips(t):
        copies = [(res.routing.w[t, j], wg[e], wu[e], wd[e])
                  for j, e in enumerate(res.routing.idx[t]) if res.grouping.slot_pos[t * k + j] >= 0]
        return O.y_rounding_flips(x64[t], copies, shared, scaled=quant is not None)
    return flips


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


def _within(y_gpu_row, y_ref_row, tol):
    rms = np.sqrt(np.mean(y_ref_row ** 2))
    err = np.max(np.abs(y_gpu_row - y_ref_row))
    return err <= tol * rms, err / rms


def _bf16_key(v):
    """An integer that orders bf16 values and steps by one between neighbours (+0 and -0 alike)."""
    b = mi.f32_to_bf16_bits(np.asarray(v, dtype=np.float32)).astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def rounding_witness(y_gpu_row, y_ref_row, fl: O.YFlips, tol=Y_TOL):
    """A choice of correct roundings h_i in [lo_i, hi_i] for the ambiguous elements under which
    y_gpu lies within tol * rms of y_ref + sum_i V[i] (h_i - ref_i); returns the changes
    h_i - ref_i, or None. When every element has two candidates and there are at most 14, every
    choice is tried; otherwise the least-squares fit of y_gpu - y_ref by the rows of V (nearly
    orthogonal) gives each element's change, rounded to bf16 and clipped to its range."""
    y_gpu_row = np.asarray(y_gpu_row, dtype=np.float64)
    m = fl.V.shape[0]
    if m == 0:
        return None
    lo, hi = fl.lo - fl.ref, fl.hi - fl.ref
    if m <= 14 and np.all(_bf16_key(fl.hi) - _bf16_key(fl.lo) == 1):   # two candidates each
        step = np.where(lo == 0, hi, lo)
        C = ((np.arange(1 << m)[:, None] >> np.arange(m)[None, :]) & 1).astype(np.float64) * step[None, :]
        refs = y_ref_row[None, :] + C @ fl.V
        err = np.max(np.abs(y_gpu_row[None, :] - refs), axis=1)
        ok = err <= tol * np.sqrt(np.mean(refs ** 2, axis=1))
        if np.any(ok):
            return C[int(np.argmax(ok))]
    dh = np.linalg.lstsq(fl.V.T, y_gpu_row - y_ref_row, rcond=None)[0]
    h = np.clip(O.bf16_round(fl.ref + dh), fl.lo, fl.hi)
    c = h - fl.ref
    return c if _within(y_gpu_row, y_ref_row + c @ fl.V, tol)[0] else None


def check_y(y_gpu: np.ndarray, y_ref: np.ndarray, tol=Y_TOL, flips=None, tokens=None):
    """Per-row bound. flips (from rounding_flips) and tokens (the token of each row) let a row that
    fails pass when some choice of other correct roundings for its ambiguous h elements brings it
    within the bound; without them, or for a row with no ambiguous element, there is no slack.
    Returns the worst ratio err / rms over the rows (against the chosen roundings)."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    err = np.max(np.abs(y_gpu - y_ref), axis=1)
    rms = np.sqrt(np.mean(y_ref ** 2, axis=1))
    zero = rms == 0
    assert np.all(y_gpu[zero] == 0), "rows with an all-zero reference must be exactly zero"
    ratio = np.where(zero, 0.0, err / np.where(zero, 1.0, rms))
    bad = np.nonzero(~zero & (err > tol * rms))[0]
    still = []
    for i in bad:
        if flips is None:
            still.append(i)
            continue
        t = int(i if tokens is None else tokens[i])
        fl = flips(t)
        c = rounding_witness(y_gpu[i], y_ref[i], fl, tol)
        if c is None:
            still.append(i)
            continue
        ratio[i] = _within(y_gpu[i], y_ref[i] + c @ fl.V, tol)[1]
        print(f"row {i} (token {t}): {ratio[i]:.3e} of rms against the roundings chosen for "
              f"{int(np.sum(c != 0))} of its {fl.V.shape[0]} ambiguous h elements (strict: {err[i] / rms[i]:.3e})")
    assert not still, (f"{len(still)} rows exceed {tol}*rms; worst ratio "
                       f"{np.max(err[still] / rms[still]):.3e}")
    return float(np.max(ratio)) if ratio.size else 0.0


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def stratified_rows(grouping: O.Grouping, k: int, n_tokens: int, block: int = 64, seed: int = 1234):
    """Tokens such that every block of `block` consecutive rows of every expert segment (in
    grouped order) holds at least one of their copies, and every block of `block` tokens (the
    rows of a shared expert) holds one of them; plus the first and last token. Any tile of the
    grouped GEMMs that holds at least `block` rows of a segment, or starts at a multiple of
    `block` within it, therefore holds a checked row. Returns (tokens, cells covered, cells)."""
    rng = np.random.default_rng(seed)
    toks = {0, n_tokens - 1}
    cells = 0
    offs = grouping.offsets
    for e in range(offs.shape[0] - 1):
        a, b = int(offs[e]), int(offs[e + 1])
        for r0 in range(a, b, block):
            r = int(rng.integers(r0, min(b, r0 + block)))
            toks.add(int(grouping.perm[r]) // k)
            cells += 1
    for t0 in range(0, n_tokens, block):
        toks.add(int(rng.integers(t0, min(n_tokens, t0 + block))))
        cells += 1
    rows = np.array(sorted(t for t in toks if 0 <= t < n_tokens))
    return rows, cells


def sample_rows(N: int, n: int, seed: int = 1234) -> np.ndarray:
    """A seeded sample of rows that always includes the first and last row."""
    if n >= N:
        return np.arange(N)
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(N, size=n - 2, replace=False).tolist()) | {0, N - 1}
    return np.array(sorted(rows))
