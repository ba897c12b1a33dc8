"""Pins of the backward oracle (oracle/moe_backward.py), CPU only.

* central finite differences of the frozen-selection loss, entry by entry,
  for every parameter of a small layer with a shared expert, capacity
  dropping, a logit bias and the balance term;
* torch autograd of the same loss, written with torch ops (fp64);
* E = 1, k = 1: the dense SwiGLU FFN's gradients from torch, and no router
  gradient (a one-expert softmax is constant);
* capacity 1: each expert's weight gradients come from its one kept row.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

from oracle import moe_backward as B
from oracle import moe_oracle as O


def small_layer(rng, N=6, d=8, F=5, E=4, k=2, S=1, Fs=3):
    x = rng.standard_normal((N, d))
    wr = rng.standard_normal((E, d)) * 0.7
    wg = rng.standard_normal((E, F, d)) / np.sqrt(d)
    wu = rng.standard_normal((E, F, d)) / np.sqrt(d)
    wd = rng.standard_normal((E, d, F)) / np.sqrt(F)
    shared = None
    if S:
        shared = (rng.standard_normal((S, Fs, d)) / np.sqrt(d), rng.standard_normal((S, Fs, d)) / np.sqrt(d),
                  rng.standard_normal((S, d, Fs)) / np.sqrt(Fs))
    lb = rng.standard_normal(E) * 0.3
    dy = rng.standard_normal((N, d))
    idx = O.route(x, wr, k, lb).idx
    return x, wr, wg, wu, wd, shared, lb, dy, idx


def fd_check(args, kw, grads, eps=1e-6, rtol=1e-6, atol=1e-8):
    x, wr, wg, wu, wd, shared, lb, dy, idx = args

    def loss(x_=x, wr_=wr, wg_=wg, wu_=wu, wd_=wd, sh_=shared, lb_=lb):
        return B.layer_loss(x_, wr_, wg_, wu_, wd_, idx, dy, shared=sh_, logit_bias=lb_, **kw)

    def central(name, arr, rebuild):
        out = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            a, b = arr.copy(), arr.copy()
            a[i] += eps
            b[i] -= eps
            out[i] = (loss(**rebuild(a)) - loss(**rebuild(b))) / (2 * eps)
        return out

    checks = [("dx", x, lambda a: dict(x_=a), grads.dx),
              ("dw_router", wr, lambda a: dict(wr_=a), grads.dw_router),
              ("d_logit_bias", lb, lambda a: dict(lb_=a), grads.d_logit_bias),
              ("dw_gate", wg, lambda a: dict(wg_=a), grads.dw_gate),
              ("dw_up", wu, lambda a: dict(wu_=a), grads.dw_up),
              ("dw_down", wd, lambda a: dict(wd_=a), grads.dw_down)]
    if shared is not None:
        checks += [("ds_gate", shared[0], lambda a: dict(sh_=(a, shared[1], shared[2])), grads.ds_gate),
                   ("ds_up", shared[1], lambda a: dict(sh_=(shared[0], a, shared[2])), grads.ds_up),
                   ("ds_down", shared[2], lambda a: dict(sh_=(shared[0], shared[1], a)), grads.ds_down)]
    for name, arr, rebuild, got in checks:
        np.testing.assert_allclose(got, central(name, arr, rebuild), rtol=rtol, atol=atol, err_msg=name)


@pytest.mark.parametrize("renormalize", [True, False])
def test_backward_matches_finite_differences(renormalize):
    rng = np.random.default_rng(60 + renormalize)
    args = small_layer(rng)
    x, wr, wg, wu, wd, shared, lb, dy, idx = args
    kw = dict(capacity=2, renormalize=renormalize, aux_coef=0.7)
    assert np.any(O.group(idx, 4, 2).slot_pos < 0), "the case must drop a copy"
    grads = B.layer_backward(x, wr, wg, wu, wd, idx, dy, shared=shared, logit_bias=lb, **kw)
    fd_check(args, kw, grads)


def torch_loss(x, wr, wg, wu, wd, shared, lb, dy, idx, capacity, aux_coef):
    """The frozen-selection loss with torch ops (fp64), for autograd."""
    N, k = idx.shape
    E = wr.shape[0]
    p = torch.softmax(x @ wr.T + lb, dim=1)
    sel = torch.gather(p, 1, torch.from_numpy(idx))
    w = sel / sel.sum(dim=1, keepdim=True)
    keep = O.capacity_keep(idx, E, capacity).reshape(N, k)
    y = torch.zeros_like(x)
    for t in range(N):
        for j in range(k):
            if keep[t, j]:
                e = int(idx[t, j])
                h = Fn.silu(x[t] @ wg[e].T) * (x[t] @ wu[e].T)
                y[t] = y[t] + w[t, j] * (h @ wd[e].T)
    for s in range(shared[0].shape[0]):
        y = y + (Fn.silu(x @ shared[0][s].T) * (x @ shared[1][s].T)) @ shared[2][s].T
    counts = torch.from_numpy(O.expert_counts(idx, E).astype(np.float64))
    stat = E * torch.sum(counts / (N * k) * p.sum(dim=0) / N)
    return torch.sum(dy * y) + aux_coef * stat


def test_backward_matches_torch_autograd():
    rng = np.random.default_rng(62)
    x, wr, wg, wu, wd, shared, lb, dy, idx = small_layer(rng, N=9, d=16, F=12, E=5, k=3, S=1, Fs=8)
    grads = B.layer_backward(x, wr, wg, wu, wd, idx, dy, shared=shared, logit_bias=lb, capacity=4,
                             aux_coef=0.25)
    T = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    tx, twr, twg, twu, twd, tlb = T(x), T(wr), T(wg), T(wu), T(wd), T(lb)
    tsh = tuple(T(a) for a in shared)
    L = torch_loss(tx, twr, twg, twu, twd, tsh, tlb, torch.from_numpy(dy), idx, 4, 0.25)
    L.backward()
    for got, t in ((grads.dx, tx), (grads.dw_router, twr), (grads.d_logit_bias, tlb), (grads.dw_gate, twg),
                   (grads.dw_up, twu), (grads.dw_down, twd), (grads.ds_gate, tsh[0]), (grads.ds_up, tsh[1]),
                   (grads.ds_down, tsh[2])):
        np.testing.assert_allclose(got, t.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_one_expert_is_dense_ffn_backward():
    rng = np.random.default_rng(63)
    N, d, F = 7, 8, 6
    x = rng.standard_normal((N, d))
    wg, wu, wd = rng.standard_normal((1, F, d)), rng.standard_normal((1, F, d)), rng.standard_normal((1, d, F))
    dy = rng.standard_normal((N, d))
    idx = np.zeros((N, 1), dtype=np.int64)
    g = B.layer_backward(x, rng.standard_normal((1, d)), wg, wu, wd, idx, dy, aux_coef=0.5)
    T = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    tx, tg, tu, td = T(x), T(wg[0]), T(wu[0]), T(wd[0])
    y = Fn.linear(Fn.silu(Fn.linear(tx, tg)) * Fn.linear(tx, tu), td)
    torch.sum(torch.from_numpy(dy) * y).backward()
    np.testing.assert_allclose(g.dx, tx.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g.dw_gate[0], tg.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g.dw_up[0], tu.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g.dw_down[0], td.grad.numpy(), rtol=1e-11, atol=1e-12)
    assert not g.dw_router.any() and not g.d_logit_bias.any()


def test_capacity_one_uses_only_the_kept_row():
    rng = np.random.default_rng(64)
    x, wr, wg, wu, wd, _, lb, dy, idx = small_layer(rng, N=8, E=3, k=2, S=0)
    N, k = idx.shape
    g = B.layer_backward(x, wr, wg, wu, wd, idx, dy, logit_bias=lb, capacity=1)
    grp = O.group(idx, 3, 1)
    p = O.softmax(O.router_logits(x, wr, lb))
    sel = np.take_along_axis(p, idx, axis=1)
    w = sel / sel.sum(axis=1, keepdims=True)
    for e in range(3):
        c = grp.perm[grp.offsets[e]:grp.offsets[e + 1]]
        assert len(c) == 1
        t, j = c[0] // k, c[0] % k
        _, dWg, dWu, dWd = B.expert_backward(x[t:t + 1], w[t, j] * dy[t:t + 1], wg[e], wu[e], wd[e], False)
        np.testing.assert_allclose(g.dw_gate[e], dWg, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(g.dw_up[e], dWu, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(g.dw_down[e], dWd, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("renormalize,S", [(True, 1), (False, 0)])
def test_sampled_backward_equals_full(renormalize, S):
    """The sampled form returns the same rows and experts as the full backward."""
    rng = np.random.default_rng(65 + S)
    x, wr, wg, wu, wd, shared, lb, dy, idx = small_layer(rng, N=11, d=8, F=6, E=5, k=2, S=S, Fs=4)
    kw = dict(shared=shared, logit_bias=lb, capacity=3, renormalize=renormalize, round_h=True, aux_coef=0.4)
    full = B.layer_backward(x, wr, wg, wu, wd, idx, dy, **kw)
    tokens = [10, 0, 4, 7]
    experts = list(range(5))
    dx, weights, ds = B.layer_backward_sampled(x, wr, wg, wu, wd, idx, dy, tokens, experts, **kw)
    np.testing.assert_allclose(dx, full.dx[tokens], rtol=1e-12, atol=1e-14)
    for e in experts:
        for got, ref in zip(weights[e], (full.dw_gate[e], full.dw_up[e], full.dw_down[e])):
            np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)
    if S:
        for got, ref in zip(ds, (full.ds_gate, full.ds_up, full.ds_down)):
            np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)
    else:
        assert ds is None
