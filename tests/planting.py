"""Layers with an element of h planted next to a bf16 rounding midpoint.

h = silu(g) * u is rounded to bf16 before the down projection. When its
exact value lies within an fp32 evaluation's error of the midpoint between
two bf16 neighbours, both roundings are correct. These helpers move u, by
changing a few entries of a bf16 weight row of W_up by a few bf16 steps,
until h lies as close to a midpoint as the pair search can bring it. They
call the oracle (silu, bf16_round) and run on the CPU only.
"""
from __future__ import annotations

import numpy as np

import moe_inputs as mi
from oracle import moe_oracle as O


def _bf16_bits(v: np.ndarray) -> np.ndarray:
    return mi.f32_to_bf16_bits(np.asarray(v, dtype=np.float32))


def _bf16_values(bits: np.ndarray) -> np.ndarray:
    return mi.bf16_bits_to_f32(np.asarray(bits, dtype=np.uint16)).astype(np.float64)


def _stepped(w: np.ndarray, m: int) -> np.ndarray:
    """bf16 values w moved m bf16 steps away from zero (m < 0: toward zero; never across it)."""
    bits = _bf16_bits(w).astype(np.int64)
    mag = np.clip((bits & 0x7FFF) + m, 1, 0x7F7F)
    return _bf16_values(((bits & 0x8000) | mag).astype(np.uint16))


def _neighbour_toward(ref: float, t: float) -> float:
    """The bf16 neighbour of the bf16 value ref on t's side (away from zero if |t| > |ref|)."""
    bits = int(_bf16_bits(np.array([ref]))[0])
    mag = bits & 0x7FFF
    mag = mag + 1 if abs(t) > abs(ref) else max(mag - 1, 0)
    sign = (bits & 0x8000) if ref != 0 else (0x8000 if t < 0 else 0)
    return float(_bf16_values(np.array([sign | mag], dtype=np.uint16))[0])


def plant_midpoint(x: np.ndarray, wg_row: np.ndarray, wu_row: np.ndarray, target=None, steps: int = 8):
    """A copy of wu_row (bf16 values) with at most two entries moved by at most `steps` bf16
    steps, so that h = silu(x . wg_row) * (x . wu_row) lies as close as the search can bring it
    to the bf16 rounding midpoint nearest `target` (default: nearest h). x, wg_row and wu_row
    hold bf16 values. Returns (new wu_row, h, midpoint)."""
    x = np.asarray(x, dtype=np.float64)
    wu = np.asarray(wu_row, dtype=np.float64).copy()
    s = float(O.silu(x @ np.asarray(wg_row, dtype=np.float64)))
    h = s * float(x @ wu)
    t = h if target is None else float(target)
    ref = float(O.bf16_round(t))
    nb = _neighbour_toward(ref, t)
    mid = 0.5 * (ref + nb)
    need = mid / s - float(x @ wu)          # the change of u that puts h on the midpoint
    # single moves: (change of u, entry, new value)
    deltas, ents, vals = [], [], []
    for m in list(range(-steps, 0)) + list(range(1, steps + 1)):
        nv = _stepped(wu, m)
        deltas.append(x * (nv - wu))
        ents.append(np.arange(wu.shape[0]))
        vals.append(nv)
    deltas = np.concatenate(deltas)
    ents = np.concatenate(ents)
    vals = np.concatenate(vals)
    keep = deltas != 0
    deltas, ents, vals = deltas[keep], ents[keep], vals[keep]
    best = (abs(need), None, None)
    # one move
    i = int(np.argmin(np.abs(deltas - need)))
    if abs(deltas[i] - need) < best[0]:
        best = (abs(deltas[i] - need), i, None)
    # two moves on different entries: sorted two-sum search
    order = np.argsort(deltas)
    sd = deltas[order]
    pos = np.searchsorted(sd, need - sd)
    for off in (-1, 0):
        j = np.clip(pos + off, 0, sd.shape[0] - 1)
        err = np.abs(sd + sd[j] - need)
        ok = ents[order] != ents[order[j]]
        err = np.where(ok, err, np.inf)
        a = int(np.argmin(err))
        if err[a] < best[0]:
            best = (err[a], int(order[a]), int(order[j[a]]))
    _, a, b = best
    for c in (a, b):
        if c is not None:
            wu[ents[c]] = vals[c]
    h = s * float(x @ wu)
    return wu, h, mid


def planted_layer(n_tokens: int = 16, d: int = 64, d_ff: int = 64, n_experts: int = 4, seed: int = 0):
    """A bf16 layer (k = 1, every token routed to expert 0 by a zero router) in which token t's
    h column t is about 16.06, next to the midpoint 16.0625 of the bf16 values 16 and 16.125,
    and dominates y_t: a one-step rounding difference there moves y_t by about 2% of its rms.
    Returns (cfg, layer, x) in storage format, plus the planted (token, column) pairs."""
    cfg = mi.small_config("planted", n_tokens=n_tokens, d_model=d, d_ff=d_ff, n_experts=n_experts, top_k=1,
                          dtype="bf16", layer_id=780 + seed, x_id=780 + seed)
    layer, x = mi.make_layer(cfg), mi.make_x(cfg)
    layer.w_router[:] = 0   # equal logits: ties go to the lowest index, so every token takes expert 0
    X = mi.to_f64(x)
    wg = mi.to_f64(layer.w_gate[0])
    wu = mi.to_f64(layer.w_up[0])
    planted = []
    for t in range(min(n_tokens, d_ff)):
        n2 = float(X[t] @ X[t])
        wg[t] = _bf16_values(_bf16_bits(X[t] * (4.0 / n2)))            # g ~ 4
        g = float(X[t] @ wg[t])
        wu[t] = _bf16_values(_bf16_bits(X[t] * (16.06 / (float(O.silu(g)) * n2))))  # h ~ 16.06
        wu[t], h, mid = plant_midpoint(X[t], wg[t], wu[t], target=16.06)
        planted.append((t, t, h, mid))
    layer.w_gate[0] = _bf16_bits(wg)
    layer.w_up[0] = _bf16_bits(wu)
    return cfg, layer, x, planted
