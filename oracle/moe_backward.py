"""Plain CPU oracle for the backward pass of the top-k routed MoE layer.

Test infrastructure only, like moe_oracle.py (whose forward pieces it uses):
the tests and the benchmark's CPU-baseline leg may call it, the GPU path
never does. numpy float64 throughout.

The function differentiated is the forward layer of "混合专家 MoE" (anrans
ai-infra handbook), section "实现：逐 token 与按专家分组" (``route`` and
``forward_grouped``), with the selection frozen: the top-k indices and the
dropped set are taken from the forward pass and are not differentiated (they
are piecewise constant). The scalar whose gradient is returned is

    L = sum_{t,c} dy[t, c] * y[t, c] + aux_coef * stat,

where stat is the balance statistic of the section "负载均衡",
E * sum_e f_e * P_e with P_e = (1/N) sum_t p[t, e], and f_e (the routed
counts over N*k) held constant. Readings where the pages are silent:

* the rounding of h to bf16 (bf16 layers) passes the gradient unchanged
  (straight-through): the backward uses the rounded h where h itself
  appears (the down-projection weight gradient) and the exact SwiGLU
  derivative of the unrounded gate and up values;
* a dropped copy (capacity, the notes "混合专家模型 (MoE)..." section 三.1)
  contributes nothing to y, so it sends no gradient into its expert and
  its combine weight gets none; it still counts in the renormalisation
  denominator of its token's selected probabilities;
* the selection-only bias gets no gradient (it only chooses).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from oracle import moe_oracle as O

F64 = np.float64


@dataclass
class Grads:
    dx: np.ndarray            # [N, d]
    dw_router: np.ndarray     # [E, d]
    d_logit_bias: np.ndarray  # [E]
    dw_gate: np.ndarray       # [E, F, d]
    dw_up: np.ndarray         # [E, F, d]
    dw_down: np.ndarray       # [E, d, F]
    ds_gate: Optional[np.ndarray] = None   # [S, Fs, d]
    ds_up: Optional[np.ndarray] = None
    ds_down: Optional[np.ndarray] = None   # [S, d, Fs]


def sigmoid(z):
    z = np.asarray(z, dtype=F64)
    return 1.0 / (1.0 + np.exp(-z))


def silu_grad(z):
    """d/dz (z * sigmoid(z)) = sigmoid(z) * (1 + z * (1 - sigmoid(z)))."""
    s = sigmoid(z)
    return s * (1.0 + np.asarray(z, dtype=F64) * (1.0 - s))


def renorm_backward(dw, w, ssum):
    """w_j = p_j / sum_i p_i over a token's selected probabilities:
    dp_j = (dw_j - sum_i dw_i w_i) / sum_i p_i."""
    return (dw - np.sum(dw * w, axis=1, keepdims=True)) / ssum


def softmax_backward(p, dp):
    """p = softmax(l): dl = p * (dp - sum_e dp_e p_e)."""
    return p * (dp - np.sum(dp * p, axis=1, keepdims=True))


# the grouping whose dropped copies the backward leaves out (the forward's)
_grouping = O.group


def expert_backward_terms(X, dO, w_gate, w_up, w_down, round_h: bool):
    """The rows expert_backward's products are taken over, for one SwiGLU expert over the rows
    X [M, d] with output gradient dO [M, d]: h = silu(X Wg^T) * (X Wu^T) (bf16-rounded if
    round_h), O = h Wd^T. Returns (G, H, dH, dG, dU), each [M, F]."""
    X = np.asarray(X, dtype=F64)
    Wg, Wu, Wd = (np.asarray(a, dtype=F64) for a in (w_gate, w_up, w_down))
    G = X @ Wg.T
    U = X @ Wu.T
    H = O.silu(G) * U
    if round_h:
        H = O.bf16_round(H)
    dH = dO @ Wd                        # O = H Wd^T  ->  dH = dO Wd
    dG = dH * U * silu_grad(G)          # h = silu(G) * U
    dU = dH * O.silu(G)
    return G, H, dH, dG, dU


def expert_backward(X, dO, w_gate, w_up, w_down, round_h: bool):
    """Returns (dX [M, d], dWg [F, d], dWu [F, d], dWd [d, F]) for the expert of
    expert_backward_terms."""
    X = np.asarray(X, dtype=F64)
    Wg, Wu = (np.asarray(a, dtype=F64) for a in (w_gate, w_up))
    _, H, _, dG, dU = expert_backward_terms(X, dO, Wg, Wu, w_down, round_h)
    return dG @ Wg + dU @ Wu, dG.T @ X, dU.T @ X, dO.T @ H


def layer_backward(x, w_router, w_gate, w_up, w_down, idx, dy, *, shared=None, logit_bias=None,
                   capacity: int = 0, renormalize: bool = True, round_h: bool = False,
                   aux_coef: float = 0.0) -> Grads:
    """Gradients of L (module docstring) for the layer whose forward chose `idx` [N, k].

    w_gate, w_up: [E, F, d]; w_down: [E, d, F]; shared: (s_gate, s_up, s_down) or None.
    """
    x = np.asarray(x, dtype=F64)
    dy = np.asarray(dy, dtype=F64)
    Wr = np.asarray(w_router, dtype=F64)
    idx = np.asarray(idx, dtype=np.int64)
    N, k = idx.shape
    E = Wr.shape[0]
    # forward quantities the chain rule needs: p, the selected probabilities and their sum
    p = O.softmax(O.router_logits(x, Wr, logit_bias))
    sel = np.take_along_axis(p, idx, axis=1)
    ssum = sel.sum(axis=1, keepdims=True)
    w = sel / ssum if renormalize else sel
    g = _grouping(idx, E, capacity)
    Wg, Wu, Wd = (np.stack([np.asarray(a[e], dtype=F64) for e in range(E)]) for a in (w_gate, w_up, w_down))
    dx = np.zeros_like(x)
    dWg, dWu, dWd = np.zeros_like(Wg), np.zeros_like(Wu), np.zeros_like(Wd)
    dw = np.zeros((N, k))                           # gradient of the combine weights (0 for dropped copies)
    for e in range(E):
        copies = g.perm[g.offsets[e]:g.offsets[e + 1]]
        if len(copies) == 0:
            continue
        t, j = copies // k, copies % k
        Xe = x[t]
        He = O.silu(Xe @ Wg[e].T) * (Xe @ Wu[e].T)
        if round_h:
            He = O.bf16_round(He)
        Oe = He @ Wd[e].T                           # this expert's output rows, before the weight
        dw[t, j] = np.sum(dy[t] * Oe, axis=1)       # y_t += w_tj * O
        dXe, dWg[e], dWu[e], dWd[e] = expert_backward(Xe, w[t, j][:, None] * dy[t], Wg[e], Wu[e], Wd[e],
                                                      round_h)
        np.add.at(dx, t, dXe)
    ds = None
    if shared is not None:
        sg, su, sd = shared
        S = len(sg)
        ds = [np.zeros((S,) + np.shape(sg[0])), np.zeros((S,) + np.shape(su[0])), np.zeros((S,) + np.shape(sd[0]))]
        for s in range(S):
            dXs, ds[0][s], ds[1][s], ds[2][s] = expert_backward(x, dy, sg[s], su[s], sd[s], round_h)
            dx += dXs
    # router: combine weights -> selected probabilities -> all probabilities -> logits
    dsel = renorm_backward(dw, w, ssum) if renormalize else dw
    dp = np.zeros_like(p)
    np.put_along_axis(dp, idx, dsel, axis=1)          # the k selected experts are distinct
    if aux_coef:
        f = O.expert_counts(idx, E) / (N * k)
        dp += aux_coef * E * f[None, :] / N           # stat = E sum_e f_e (1/N) sum_t p[t, e]
    dl = softmax_backward(p, dp)
    dx += dl @ Wr
    return Grads(dx=dx, dw_router=dl.T @ x, d_logit_bias=dl.sum(axis=0), dw_gate=dWg, dw_up=dWu, dw_down=dWd,
                 ds_gate=None if ds is None else ds[0], ds_up=None if ds is None else ds[1],
                 ds_down=None if ds is None else ds[2])


def layer_loss(x, w_router, w_gate, w_up, w_down, idx, dy, *, shared=None, logit_bias=None,
               capacity: int = 0, renormalize: bool = True, round_h: bool = False,
               aux_coef: float = 0.0) -> float:
    """L = <dy, y> + aux_coef * stat for the frozen selection idx (the function layer_backward
    differentiates), from the forward oracle's grouped form."""
    x = np.asarray(x, dtype=F64)
    idx = np.asarray(idx, dtype=np.int64)
    N, k = idx.shape
    E = np.shape(w_router)[0]
    p = O.softmax(O.router_logits(x, w_router, logit_bias))
    w = np.take_along_axis(p, idx, axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    g = O.group(idx, E, capacity)
    y = O.forward_grouped(x, idx, w, g, w_gate, w_up, w_down, shared=shared, round_h=round_h)
    L = float(np.sum(np.asarray(dy, dtype=F64) * y))
    if aux_coef:
        L += aux_coef * O.balance_stat(O.expert_counts(idx, E), p.sum(axis=0), N, k)
    return L


def layer_backward_sampled(x, w_router, w_gate, w_up, w_down, idx, dy, tokens, experts, *, shared=None,
                           logit_bias=None, capacity: int = 0, renormalize: bool = True, round_h: bool = False,
                           aux_coef: float = 0.0):
    """Part of layer_backward's result, reading only the expert weights that part needs (for
    layers whose weights do not fit in memory in fp64; w_gate etc. may be lazy per-expert views):

    * dx[tokens] (each token's row is its own: its kept copies' expert rows, the shared
      experts' rows and its router row);
    * the weight gradients (dWg, dWu, dWd) of every expert in `experts` (from all its kept rows);
    * every shared expert's weight gradients (None without shared experts).

    Returns (dx_rows [len(tokens), d], {e: (dWg, dWu, dWd)}, (ds_gate, ds_up, ds_down) or None).
    The steps are layer_backward's, applied to the rows and experts asked for."""
    x = np.asarray(x, dtype=F64)
    dy = np.asarray(dy, dtype=F64)
    Wr = np.asarray(w_router, dtype=F64)
    idx = np.asarray(idx, dtype=np.int64)
    tokens = np.asarray(tokens, dtype=np.int64)
    N, k = idx.shape
    E = Wr.shape[0]
    p = O.softmax(O.router_logits(x, Wr, logit_bias))
    sel = np.take_along_axis(p, idx, axis=1)
    ssum = sel.sum(axis=1, keepdims=True)
    w = sel / ssum if renormalize else sel
    g = _grouping(idx, E, capacity)
    kept = (g.slot_pos >= 0).reshape(N, k)

    weights = {}
    for e in experts:
        copies = g.perm[g.offsets[e]:g.offsets[e + 1]]
        if len(copies) == 0:
            F, d = np.shape(w_gate[e])
            weights[e] = (np.zeros((F, d)), np.zeros((F, d)), np.zeros((d, F)))
            continue
        t, j = copies // k, copies % k
        weights[e] = expert_backward(x[t], w[t, j][:, None] * dy[t], w_gate[e], w_up[e], w_down[e], round_h)[1:]

    # the sampled tokens' kept copies, grouped by expert
    dx = np.zeros((len(tokens), x.shape[1]))
    dw = np.zeros((len(tokens), k))
    for e in np.unique(idx[tokens]):
        ii, jj = np.nonzero((idx[tokens] == e) & kept[tokens])
        if len(ii) == 0:
            continue
        t = tokens[ii]
        Wg, Wu, Wd = (np.asarray(a[e], dtype=F64) for a in (w_gate, w_up, w_down))
        He = O.silu(x[t] @ Wg.T) * (x[t] @ Wu.T)
        if round_h:
            He = O.bf16_round(He)
        dw[ii, jj] = np.sum(dy[t] * (He @ Wd.T), axis=1)
        dXe = expert_backward(x[t], w[t, jj][:, None] * dy[t], Wg, Wu, Wd, round_h)[0]
        np.add.at(dx, ii, dXe)
    ds = None
    if shared is not None:
        sg, su, sd = shared
        ds = ([], [], [])
        for s in range(len(sg)):
            dXs, a, b, c = expert_backward(x, dy, sg[s], su[s], sd[s], round_h)
            dx += dXs[tokens]
            for lst, v in zip(ds, (a, b, c)):
                lst.append(v)
        ds = tuple(np.stack(v) for v in ds)
    dsel = renorm_backward(dw, w[tokens], ssum[tokens]) if renormalize else dw
    dp = np.zeros((len(tokens), E))
    np.put_along_axis(dp, idx[tokens], dsel, axis=1)
    if aux_coef:
        f = O.expert_counts(idx, E) / (N * k)
        dp += aux_coef * E * f[None, :] / N
    dx += softmax_backward(p[tokens], dp) @ Wr
    return dx, weights, ds
