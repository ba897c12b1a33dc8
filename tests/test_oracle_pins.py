"""Pins of the CPU oracle against what the MoE pages and the mathematics fix.

Each test checks the oracle against something other than itself: a value
the pages print, a closed form, an invariant, a library routine for a
special case, or brute force on tiny inputs. Section names refer to
"混合专家 MoE" (anrans ai-infra handbook) unless stated otherwise.
"""
import itertools
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import moe_inputs as mi
from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                key, v = line.split("=")
                vals[key] = float(v)
    return vals


def rand_layer(rng, E, d, f, S=0):
    wg = rng.standard_normal((E, f, d)) / math.sqrt(d)
    wu = rng.standard_normal((E, f, d)) / math.sqrt(d)
    wd = rng.standard_normal((E, d, f)) / math.sqrt(f)
    shared = None
    if S:
        shared = (rng.standard_normal((S, f, d)) / math.sqrt(d),
                  rng.standard_normal((S, f, d)) / math.sqrt(d),
                  rng.standard_normal((S, d, f)) / math.sqrt(f))
    return wg, wu, wd, shared


# ------------------------------------------------------------------ softmax

def test_softmax_matches_scipy_and_sums_to_one():
    rng = np.random.default_rng(1)
    l = rng.standard_normal((40, 13)) * 5
    p = O.softmax(l)
    np.testing.assert_allclose(p, scipy.special.softmax(l, axis=1), rtol=1e-14, atol=0)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-15)


def test_softmax_closed_forms():
    # E = 1: p = 1 exactly. Equal logits: p = 1/E (exact for E a power of two).
    assert np.all(O.softmax(np.array([[3.7], [-2.0]])) == 1.0)
    for E in (2, 8, 256):
        p = O.softmax(np.zeros((3, E)))
        assert np.all(p == 1.0 / E)
    # a zero router gives equal logits
    x = np.random.default_rng(0).standard_normal((5, 16))
    assert np.all(O.softmax(O.router_logits(x, np.zeros((8, 16)))) == 1.0 / 8)


def test_router_logits_is_linear_layer():
    # nn.Linear(d, E, bias=False) gives x W^T; the optional bias enters additively
    rng = np.random.default_rng(2)
    x, W, b = rng.standard_normal((7, 12)), rng.standard_normal((5, 12)), rng.standard_normal(5)
    ref = torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(W), torch.from_numpy(b))
    np.testing.assert_allclose(O.router_logits(x, W, b), ref.numpy(), rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------ top-k

def topk_bruteforce(s, k):
    """The counting definition: rank_e = #{e': s_e' > s_e or (s_e' == s_e and e' < e)}."""
    E = len(s)
    rank = [sum(1 for f in range(E) if s[f] > s[e] or (s[f] == s[e] and f < e)) for e in range(E)]
    chosen = sorted((r, e) for e, r in enumerate(rank) if r < k)
    return [e for _, e in chosen]


def test_topk_bruteforce_exhaustive_with_ties():
    # every score vector over a 3-level alphabet for E <= 5 (exact ties planted), all k
    levels = [0.0, 0.25, 0.5]
    for E in range(1, 6):
        rows = np.array(list(itertools.product(levels, repeat=E)))
        for k in range(1, E + 1):
            got = O.topk_order(rows, k)
            for r, g in zip(rows, got):
                assert list(g) == topk_bruteforce(list(r), k)


def test_topk_random_e8_k3():
    rng = np.random.default_rng(3)
    s = rng.integers(0, 4, size=(500, 8)).astype(float) / 4  # many ties
    got = O.topk_order(s, 3)
    for r, g in zip(s, got):
        assert list(g) == topk_bruteforce(list(r), 3)


def test_selection_bias_picks_but_does_not_weight():
    # "负载均衡": the bias only changes which experts are chosen, not their weights
    rng = np.random.default_rng(4)
    x, W = rng.standard_normal((30, 16)), rng.standard_normal((8, 16)) * 0.2
    b = np.zeros(8)
    b[7] = 10.0  # expert 7 always chosen
    r = O.route(x, W, 2, select_bias=b, renormalize=False)
    assert np.all(r.idx[:, 0] == 7)
    p = O.softmax(O.router_logits(x, W))
    np.testing.assert_array_equal(r.w[:, 0], p[:, 7])


# ------------------------------------------------------------------ weights

def test_renormalised_weights_sum_to_one_and_special_k():
    rng = np.random.default_rng(5)
    x, W = rng.standard_normal((64, 32)), rng.standard_normal((8, 32))
    for k in (1, 2, 3, 8):
        r = O.route(x, W, k)
        np.testing.assert_allclose(r.w.sum(axis=1), 1.0, rtol=0, atol=4e-16)
        if k == 1:
            assert np.all(r.w == 1.0)
        if k == 8:  # dense-output mixture: all experts, weights = p
            np.testing.assert_allclose(np.take_along_axis(r.probs, r.idx, 1), r.w, rtol=1e-15)
            np.testing.assert_allclose(np.sort(r.idx, axis=1), np.tile(np.arange(8), (64, 1)))


def test_router_figure_weights():
    g = read_golden("router_figure.txt")
    E = int(g["n_experts"])
    p = np.array([0.31, 0.05, 0.07, 0.19, 0.08, 0.1, 0.12, 0.08])  # two selected carry 0.31 : 0.19
    r = O.route(np.ones((1, 1)), np.log(p)[:, None], int(g["top_k"]))  # logits = log p
    assert list(r.idx[0]) == [0, 3]
    np.testing.assert_allclose(r.w[0], [g["w0"], g["w1"]], rtol=1e-14)


# ------------------------------------------------------------------ grouping / capacity

def test_counts_perm_offsets_against_library_sort():
    rng = np.random.default_rng(6)
    N, k, E = 200, 3, 11
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(N)])
    g = O.group(idx, E, 0)
    np.testing.assert_array_equal(g.counts, np.bincount(idx.ravel(), minlength=E))
    assert g.counts.sum() == N * k
    np.testing.assert_array_equal(g.perm, np.argsort(idx.ravel(), kind="mergesort"))
    np.testing.assert_array_equal(g.offsets, np.concatenate([[0], np.cumsum(g.counts)]))
    assert np.all(g.slot_pos[g.perm] == np.arange(N * k))


def capacity_bruteforce(idx, E, C):
    """keep copy c iff #{c' < c : expert(c') == expert(c)} < C."""
    flat = idx.ravel()
    return np.array([np.sum(flat[:c] == flat[c]) < C for c in range(len(flat))])


@pytest.mark.parametrize("C", [1, 2, 5, 17])
def test_capacity_bruteforce(C):
    rng = np.random.default_rng(7 + C)
    N, k, E = 60, 2, 5
    p = np.array([0.5, 0.2, 0.15, 0.1, 0.05])
    idx = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(N)])
    g = O.group(idx, E, C)
    keep = capacity_bruteforce(idx, E, C)
    np.testing.assert_array_equal(g.slot_pos >= 0, keep)
    np.testing.assert_array_equal(g.kept, np.minimum(g.counts, C))
    assert g.kept.sum() + np.sum(~keep) == N * k
    for e in range(E):  # each segment lists its kept copies in increasing copy id
        seg = g.perm[g.offsets[e]:g.offsets[e + 1]]
        assert np.all(np.diff(seg) > 0) and np.all(idx.ravel()[seg] == e)


def test_capacity_special_cases():
    rng = np.random.default_rng(8)
    N, k, E, d, f = 24, 2, 4, 16, 16
    x = rng.standard_normal((N, d))
    Wr = rng.standard_normal((E, d))
    wg, wu, wd, shared = rand_layer(rng, E, d, f, S=1)
    base = O.moe_layer(x, Wr, wg, wu, wd, k, shared=shared, capacity=0)
    big = O.moe_layer(x, Wr, wg, wu, wd, k, shared=shared, capacity=N * k)
    np.testing.assert_array_equal(base.y, big.y)
    np.testing.assert_array_equal(base.grouping.perm, big.grouping.perm)
    # C = 0 is "no limit" in the ABI; a buffer of 1 with every token on one expert keeps one copy
    one = O.group(np.zeros((N, 1), dtype=int), E, 1)
    assert one.kept.tolist() == [1, 0, 0, 0] and one.perm.tolist() == [0]
    # everything dropped: y is the shared expert alone
    lr = O.moe_layer(x, Wr, wg, wu, wd, 1, shared=shared, forced_idx=np.zeros((N, 1), int),
                     capacity=1)
    only_shared = O.swiglu_expert(x, shared[0][0], shared[1][0], shared[2][0], False)
    np.testing.assert_allclose(lr.y[1:], only_shared[1:], rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------ experts

def torch_swiglu(x, g, u, d):
    F = torch.nn.functional
    tx = torch.from_numpy(x)
    return F.linear(F.silu(F.linear(tx, torch.from_numpy(g))) * F.linear(tx, torch.from_numpy(u)),
                    torch.from_numpy(d)).numpy()


def test_silu_matches_libraries():
    z = np.linspace(-40, 40, 2001)
    np.testing.assert_allclose(O.silu(z), z * scipy.special.expit(z), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(O.silu(z), torch.nn.functional.silu(torch.from_numpy(z)).numpy(),
                               rtol=1e-14, atol=1e-300)


def test_e1_k1_is_dense_swiglu_ffn():
    # one expert, top-1: the MoE layer is the dense FFN it replaces ("结构")
    rng = np.random.default_rng(9)
    N, d, f = 33, 24, 40
    x = rng.standard_normal((N, d))
    wg, wu, wd, _ = rand_layer(rng, 1, d, f)
    for form in ("per_token", "grouped"):
        lr = O.moe_layer(x, rng.standard_normal((1, d)), wg, wu, wd, 1, form=form)
        np.testing.assert_allclose(lr.y, torch_swiglu(x, wg[0], wu[0], wd[0]), rtol=1e-12, atol=1e-13)


def test_shared_expert_adds_dense_ffn():
    rng = np.random.default_rng(10)
    N, d, f, E, k = 20, 16, 24, 5, 2
    x = rng.standard_normal((N, d))
    Wr = rng.standard_normal((E, d))
    wg, wu, wd, shared = rand_layer(rng, E, d, f, S=2)
    a = O.moe_layer(x, Wr, wg, wu, wd, k, shared=shared).y
    b = O.moe_layer(x, Wr, wg, wu, wd, k).y
    dense = sum(torch_swiglu(x, shared[0][s], shared[1][s], shared[2][s]) for s in range(2))
    np.testing.assert_allclose(a - b, dense, rtol=1e-11, atol=1e-12)


def test_single_copy_against_torch_expert():
    # y_t = w * Expert_e(x_t) for one routed copy, expert applied by torch
    rng = np.random.default_rng(11)
    N, d, f, E = 6, 16, 32, 3
    x = rng.standard_normal((N, d))
    Wr = rng.standard_normal((E, d))
    wg, wu, wd, _ = rand_layer(rng, E, d, f)
    lr = O.moe_layer(x, Wr, wg, wu, wd, 1)
    for t in range(N):
        e = lr.routing.idx[t, 0]
        np.testing.assert_allclose(lr.y[t], torch_swiglu(x[t:t + 1], wg[e], wu[e], wd[e])[0],
                                   rtol=1e-12, atol=1e-13)
    # k = 2: weights from the renormalised softmax, checked against torch's topk
    lr2 = O.moe_layer(x, Wr, wg, wu, wd, 2)
    tp = torch.softmax(torch.from_numpy(x @ Wr.T), -1)
    tw, ti = tp.topk(2, -1)
    tw = tw / tw.sum(-1, keepdim=True)
    for t in range(N):
        ref = sum(tw[t, j].item() * torch_swiglu(x[t:t + 1], wg[ti[t, j]], wu[ti[t, j]], wd[ti[t, j]])[0]
                  for j in range(2))
        np.testing.assert_allclose(lr2.y[t], ref, rtol=1e-12, atol=1e-13)


# y on general inputs: properties that hold for any input, and the single-expert case, which reduces to
# torch's dense SwiGLU FFN

def _general_layer(rng, N=37, d=24, f=40, E=7, k=3, S=1):
    x = rng.standard_normal((N, d))
    Wr = rng.standard_normal((E, d)) * 0.5
    wg, wu, wd, shared = rand_layer(rng, E, d, f, S=S)
    lb = rng.uniform(-0.3, 0.3, E)
    sb = rng.uniform(-0.05, 0.05, E)
    return x, Wr, wg, wu, wd, shared, lb, sb


@pytest.mark.parametrize("C,renorm,round_h", [(0, True, False), (5, True, True), (9, False, False)])
def test_y_superposition_over_experts(C, renorm, round_h):
    # The routing does not read the down projections, so zeroing every expert's but e's keeps the
    # routing and the dropped set, and leaves expert e's share of y: the shares sum to y less the
    # shared experts. Without rounding of h, the share of e on token t is w[t, j] times torch's dense
    # SwiGLU of expert e at x_t for the kept copy of t in slot j with idx[t, j] = e, and 0 when t has
    # no kept copy on e.
    rng = np.random.default_rng(31)
    x, Wr, wg, wu, wd, shared, lb, sb = _general_layer(rng)
    N, E, k = x.shape[0], Wr.shape[0], 3
    kw = dict(logit_bias=lb, select_bias=sb, capacity=C, renormalize=renorm, round_h=round_h)
    full = O.moe_layer(x, Wr, wg, wu, wd, k, shared=shared, **kw)
    idx, w = full.routing.idx, full.routing.w
    keep = (full.grouping.slot_pos >= 0).reshape(N, k)
    if C:
        assert (~keep).any(), "the capacity must drop copies"
    total = O.moe_layer(x, Wr, wg, wu, np.zeros_like(wd), k, shared=shared, **kw).y  # the shared experts
    for e in range(E):
        wd_e = np.zeros_like(wd)
        wd_e[e] = wd[e]
        ye = O.moe_layer(x, Wr, wg, wu, wd_e, k, **kw).y
        total = total + ye
        if round_h:
            continue
        ffn = torch_swiglu(x, wg[e], wu[e], wd[e])
        for t in range(N):
            ref = sum(w[t, j] * ffn[t] for j in range(k) if idx[t, j] == e and keep[t, j])
            if isinstance(ref, int):
                assert np.all(ye[t] == 0.0)
            else:
                np.testing.assert_allclose(ye[t], ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(total, full.y, rtol=1e-12, atol=1e-12)
    if shared is not None and not round_h:
        dense = sum(torch_swiglu(x, shared[0][s], shared[1][s], shared[2][s]) for s in range(len(shared[0])))
        np.testing.assert_allclose(O.moe_layer(x, Wr, wg, wu, np.zeros_like(wd), k, shared=shared, **kw).y, dense,
                                   rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("C", [0, 6])
def test_y_invariant_under_expert_relabelling(C):
    # Relabel the experts (router rows, both biases and every expert weight, by one permutation): the
    # scores move with their experts, so every token picks the same experts in the same slots, the same
    # copies compete for capacity, and y and the statistic stay as they are; counts move with the labels.
    rng = np.random.default_rng(32)
    x, Wr, wg, wu, wd, shared, lb, sb = _general_layer(rng)
    k = 3
    a = O.moe_layer(x, Wr, wg, wu, wd, k, shared=shared, logit_bias=lb, select_bias=sb, capacity=C)
    pi = rng.permutation(Wr.shape[0])
    b = O.moe_layer(x, Wr[pi], wg[pi], wu[pi], wd[pi], k, shared=shared, logit_bias=lb[pi], select_bias=sb[pi],
                    capacity=C)
    np.testing.assert_array_equal(pi[b.routing.idx], a.routing.idx)
    np.testing.assert_array_equal(b.grouping.counts, a.grouping.counts[pi])
    np.testing.assert_allclose(b.y, a.y, rtol=1e-12, atol=1e-13)
    assert abs(b.stat - a.stat) <= 1e-12 * abs(a.stat)


def test_y_follows_token_order_without_capacity():
    # Without a capacity each token's output depends on its own row alone: permuting the tokens
    # permutes the rows of y (and of idx and w).
    rng = np.random.default_rng(33)
    x, Wr, wg, wu, wd, shared, lb, sb = _general_layer(rng)
    k = 3
    a = O.moe_layer(x, Wr, wg, wu, wd, k, shared=shared, logit_bias=lb, select_bias=sb)
    sig = rng.permutation(x.shape[0])
    b = O.moe_layer(x[sig], Wr, wg, wu, wd, k, shared=shared, logit_bias=lb, select_bias=sb)
    np.testing.assert_array_equal(b.routing.idx, a.routing.idx[sig])
    np.testing.assert_allclose(b.y, a.y[sig], rtol=1e-12, atol=1e-13)


def test_naive_equals_grouped_page_shape():
    g = read_golden("naive_vs_grouped.txt")
    cfg = mi.CONFIGS["p2_shape"]
    assert (cfg.n_tokens, cfg.d_model, cfg.d_ff, cfg.n_experts, cfg.top_k) == (
        g["n_tokens"], g["d_model"], g["d_ff"], g["n_experts"], g["top_k"])
    lay = mi.make_layer(cfg)
    x = mi.to_f64(mi.make_x(cfg))
    sh = (mi.to_f64(lay.s_gate), mi.to_f64(lay.s_up), mi.to_f64(lay.s_down))
    args = (x, mi.to_f64(lay.w_router), mi.to_f64(lay.w_gate), mi.to_f64(lay.w_up), mi.to_f64(lay.w_down),
            cfg.top_k)
    a = O.moe_layer(*args, shared=sh, form="per_token").y
    b = O.moe_layer(*args, shared=sh, form="grouped").y
    assert np.max(np.abs(a - b)) <= g["atol"]
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)  # fp64: far tighter than the page's 1e-5


def test_naive_equals_grouped_with_capacity_and_rounding():
    rng = np.random.default_rng(12)
    N, d, f, E, k = 48, 32, 64, 6, 3
    x = mi.to_f64(mi.f32_to_bf16_bits(rng.standard_normal((N, d)).astype(np.float32)))
    Wr = rng.standard_normal((E, d)) * 0.3
    wg, wu, wd, shared = rand_layer(rng, E, d, f, S=1)
    for C in (0, 5, 13):
        a = O.moe_layer(x, Wr, wg, wu, wd, k, shared=shared, capacity=C, round_h=True).y
        b = O.moe_layer(x, Wr, wg, wu, wd, k, shared=shared, capacity=C, round_h=True, form="grouped").y
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_grouped_on_row_subset_equals_per_token():
    rng = np.random.default_rng(18)
    N, d, f, E, k = 40, 16, 32, 5, 2
    x = rng.standard_normal((N, d))
    Wr = rng.standard_normal((E, d))
    wg, wu, wd, shared = rand_layer(rng, E, d, f, S=1)
    rows = np.array([39, 0, 17, 5])
    for C in (0, 6):
        a = O.moe_layer(x, Wr, wg, wu, wd, k, shared=shared, capacity=C, rows=rows).y
        b = O.moe_layer(x, Wr, wg, wu, wd, k, shared=shared, capacity=C, rows=rows, form="grouped").y
        full = O.moe_layer(x, Wr, wg, wu, wd, k, shared=shared, capacity=C, form="grouped").y
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(b, full[rows], rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------ statistic

def test_balance_stat_uniform_probs_is_one():
    rng = np.random.default_rng(13)
    for E, k, N in ((8, 2, 64), (16, 4, 50), (256, 8, 33)):
        counts = np.bincount(rng.integers(0, E, N * k), minlength=E)
        prob_sum = np.full(E, N / E)
        assert O.balance_stat(counts, prob_sum, N, k) == pytest.approx(1.0, abs=1e-14)


def test_balance_stat_uniform_counts_is_one():
    rng = np.random.default_rng(14)
    E, k, N = 8, 2, 64
    p = rng.dirichlet(np.ones(E), size=N)
    counts = np.full(E, N * k // E)
    assert O.balance_stat(counts, p.sum(0), N, k) == pytest.approx(1.0, abs=1e-14)


def test_balance_stat_one_hot_is_E():
    for E in (4, 16, 128):
        N = 10
        counts = np.zeros(E)
        counts[3] = N
        prob_sum = np.zeros(E)
        prob_sum[3] = N
        assert O.balance_stat(counts, prob_sum, N, 1) == E


def test_balance_stat_skewed_page_case():
    g = read_golden("skewed_aux.txt")
    N, E, H = int(g["n_tokens"]), int(g["n_experts"]), int(g["hot"])
    probs = np.zeros((N, E))
    probs[:, :H] = g["p_hot"]
    bad_idx = np.tile(np.arange(H), (N, 1))
    counts = O.expert_counts(bad_idx, E)
    assert O.balance_stat(counts, probs.sum(0), N, H) == g["value"]


def test_balance_stat_random_router_near_one():
    # the page: a randomly initialised router gives about 1
    rng = np.random.default_rng(15)
    N, d, E, k = 4000, 64, 16, 4
    x = rng.standard_normal((N, d))
    Wr = rng.standard_normal((E, d)) * 0.02
    r = O.route(x, Wr, k)
    stat = O.balance_stat(O.expert_counts(r.idx, E), r.probs.sum(0), N, k)
    assert abs(stat - 1.0) < 0.05


# ------------------------------------------------------------------ bf16 rounding

def _all_bf16_values():
    bits = np.arange(0, 0x7F80, dtype=np.uint32)  # +0 .. largest finite
    return (bits << 16).view(np.float32).astype(np.float64)


def test_bf16_round_is_nearest_even_bruteforce():
    vals = _all_bf16_values()
    rng = np.random.default_rng(16)
    a = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-40, 38, 20000),
        (vals[1:200] + vals[:199]) / 2,            # exact ties in the subnormal range
        (vals[30000:30200] + vals[30001:30201]) / 2,  # exact ties among normals
    ])
    a = a[np.abs(a) < vals[-1]]
    r = O.bf16_round(a)
    m = np.abs(a)
    j = np.searchsorted(vals, m)                    # vals[j-1] < m <= vals[j]
    lo, hi = vals[np.maximum(j - 1, 0)], vals[j]
    dlo, dhi = m - lo, hi - m
    lo_even = (np.maximum(j - 1, 0) % 2) == 0
    expect = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo_even, lo, hi)))
    expect = np.where(m == hi, hi, expect)
    np.testing.assert_array_equal(np.abs(r), expect)
    np.testing.assert_array_equal(np.signbit(r), np.signbit(a))  # zeros keep their sign


def test_bf16_round_matches_torch_on_fp32():
    rng = np.random.default_rng(17)
    a = (rng.standard_normal(100000) * 3).astype(np.float32)
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.bf16_round(a.astype(np.float64)), ref)


# ------------------------------------------------------------------ parameter model

def test_exercise_parameter_count():
    import bench
    g = read_golden("exercise_params.txt")
    per = bench.expert_params(int(g["d_model"]), int(g["d_ff"]))
    total = g["n_experts"] * per * g["layers"]
    active = g["top_k"] * per * g["layers"]
    assert round(total / 1e9, 2) == g["total_billions_2dp"]
    assert round(active / 1e9, 2) == g["active_billions_2dp"]


# ------------------------------------------------------------------ FP8 (E4M3) expert weights

def _fp8_finite_values():
    """The 127 finite non-negative e4m3fn values, ascending (from torch's decode)."""
    v = torch.arange(128, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    return v[~np.isnan(v)]


def test_fp8_decode_matches_torch_all_codes():
    c = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(c).view(torch.float8_e4m3fn).double().numpy()
    got = O.fp8_e4m3_decode(c)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    np.testing.assert_array_equal(got[fin], ref[fin])
    np.testing.assert_array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))
    assert O.fp8_e4m3_decode(np.uint8(0x7E)) == O.FP8_MAX


def test_fp8_encode_is_nearest_even_bruteforce():
    vals = _fp8_finite_values()                   # 0 .. 448, code i <-> vals[i]
    rng = np.random.default_rng(30)
    a = np.concatenate([
        rng.uniform(0, 464, 20000),
        rng.standard_normal(20000) * np.exp2(rng.uniform(-14, 8, 20000)),
        (vals[:-1] + vals[1:]) / 2,                 # every exact tie between neighbours
        vals,                                      # every value itself
    ])
    a = a[np.abs(a) <= 464]
    codes = O.fp8_e4m3_encode(a)
    m = np.abs(a)
    j = np.clip(np.searchsorted(vals, m), 1, len(vals) - 1)   # vals[j-1] < m <= vals[j]
    lo, hi = vals[j - 1], vals[j]
    dlo, dhi = m - lo, hi - m
    lo_even = ((j - 1) % 2) == 0                  # even code <-> even mantissa
    near = np.where(dlo < dhi, j - 1, np.where(dhi < dlo, j, np.where(lo_even, j - 1, j)))
    near = np.where(m == hi, j, near)
    near = np.where(m > vals[-1], len(vals) - 1, near)  # (448, 464]: saturate to 448
    np.testing.assert_array_equal(codes & 0x7F, near)
    np.testing.assert_array_equal((codes >> 7).astype(bool), np.signbit(a))


def test_fp8_encode_matches_torch_cast():
    rng = np.random.default_rng(31)
    v = (rng.standard_normal(100000) * np.exp2(rng.uniform(-14, 8, 100000))).astype(np.float32)
    v = v[np.abs(v) <= 448]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(O.fp8_e4m3_encode(v), ref)


def test_fp8_row_quantisation_invariants():
    rng = np.random.default_rng(32)
    w = mi.bf16_bits_to_f32(mi.f32_to_bf16_bits((rng.standard_normal((64, 96)) *
                                                 np.exp2(rng.uniform(-8, 4, (64, 1)))).astype(np.float32)))
    w[5] = 0.0                                     # an all-zero row
    codes, scale = O.quantize_fp8_rows(w)
    assert codes.dtype == np.uint8 and scale.dtype == np.float32
    assert scale[5] == 0 and not codes[5].any()
    deq = O.dequantize_fp8_rows(codes, scale)
    nz = scale > 0
    # the largest magnitude of each row maps to the largest code
    amax_col = np.argmax(np.abs(w), axis=1)
    assert np.all(np.abs(O.fp8_e4m3_decode(codes[np.arange(64), amax_col]))[nz] == O.FP8_MAX)
    # error within half a code step of the scaled value (normal: 2**-4 relative; subnormal: 2**-10 * scale)
    ratio = np.abs(w.astype(np.float64)) / np.where(nz, scale, 1.0)[:, None]
    half_step = np.where(ratio >= 2.0 ** -6, np.exp2(np.floor(np.log2(np.maximum(ratio, 1e-300))) - 4), 2.0 ** -10)
    err = np.abs(deq - w) / np.where(nz, scale, 1.0)[:, None]
    assert np.all(err[nz] <= half_step[nz] * (1 + 1e-6) + 1e-7 * ratio[nz])


def test_fp8_layer_is_dense_ffn_with_dequantised_weights():
    # E=1, k=1 with FP8 weights: the dense SwiGLU FFN on weights decoded by torch's float8_e4m3fn
    rng = np.random.default_rng(33)
    N, d, f = 17, 32, 48
    x = rng.standard_normal((N, d))
    wg, wu, wd, _ = rand_layer(rng, 1, d, f)
    deq, tdeq = [], []
    for w in (wg[0], wu[0], wd[0]):
        c, s = O.quantize_fp8_rows(w)
        deq.append(O.dequantize_fp8_rows(c, s)[None])
        tdeq.append(torch.from_numpy(c).view(torch.float8_e4m3fn).double().numpy() * s.astype(np.float64)[:, None])
    lr = O.moe_layer(x, rng.standard_normal((1, d)), deq[0], deq[1], deq[2], 1)
    np.testing.assert_allclose(lr.y, torch_swiglu(x, tdeq[0], tdeq[1], tdeq[2]), rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------ training-side router statistics

def test_z_loss_closed_forms_and_scipy():
    rng = np.random.default_rng(50)
    l = rng.standard_normal((40, 9)) * 3
    ref = np.mean(scipy.special.logsumexp(l, axis=1) ** 2)
    assert abs(O.z_loss(l) - ref) <= 1e-12 * ref
    # equal logits c over E experts: logsumexp = c + ln E
    assert abs(O.z_loss(np.full((5, 7), 2.5)) - (2.5 + math.log(7)) ** 2) <= 1e-12
    # one expert: logsumexp = the logit itself
    one = rng.standard_normal((11, 1))
    assert abs(O.z_loss(one) - np.mean(one[:, 0] ** 2)) <= 1e-12
    assert O.z_loss(np.zeros((0, 4))) == 0.0
    # shift invariance of the softmax does not hold for z: adding c to every logit adds c to logsumexp
    assert abs(O.z_loss(l + 1.0) - np.mean((scipy.special.logsumexp(l, axis=1) + 1.0) ** 2)) <= 1e-10


def test_importance_bincount_and_closed_forms():
    rng = np.random.default_rng(51)
    idx = rng.integers(0, 6, (50, 2))
    w = rng.random((50, 2))
    imp = O.importance(idx, w, 8)
    ref = np.zeros(8)
    for t in range(50):
        for j in range(2):
            ref[idx[t, j]] += w[t, j]
    np.testing.assert_allclose(imp, ref, rtol=1e-14)
    assert imp[6] == 0 and imp[7] == 0
    # equal importance everywhere -> 0; everything on one expert -> E - 1
    E = 5
    uni = O.importance(np.tile(np.arange(E), (4, 1)), np.full((4, E), 0.2), E)
    assert O.importance_cv2(uni) == 0.0
    hot = O.importance(np.zeros((9, 1), dtype=int), np.ones((9, 1)), E)
    assert abs(O.importance_cv2(hot) - (E - 1)) <= 1e-12
    assert O.importance_cv2(np.zeros(E)) == 0.0


def test_select_bias_update_bruteforce():
    rng = np.random.default_rng(52)
    E, N, k = 12, 30, 2                       # mean load N*k/E = 5
    counts = np.array([5, 0, 6, 4, 5, 12, 1, 5, 7, 3, 5, 7])
    b = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    g = 1e-3
    out = O.update_select_bias(b, counts, N, k, g)
    assert out.dtype == np.float32
    for e in range(E):
        if counts[e] > 5:
            expect = np.float32(b[e] - np.float32(g))
        elif counts[e] < 5:
            expect = np.float32(b[e] + np.float32(g))
        else:
            expect = b[e]
        assert out[e] == expect, e


# ------------------------------------------------------------------ int4 expert weights (W4A16)

def _int4_test_rows(rng):
    w = mi.bf16_bits_to_f32(mi.f32_to_bf16_bits((rng.standard_normal((64, 128)) *
                                                 np.exp2(rng.uniform(-8, 4, (64, 1)))).astype(np.float32)))
    w[5] = 0.0                                               # an all-zero row
    w[7] = 0.0
    w[7, :8] = [7.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5]    # scale 1: every other entry an exact tie
    w[9] = 0.0
    w[9, 3] = -3.0                                           # a negative maximum, alone in its row
    return w


def test_int4_quantisation_is_nearest_even_bruteforce():
    w = _int4_test_rows(np.random.default_rng(40))
    q, s = O.quantize_int4_rows(w)
    assert q.dtype == np.int8 and s.dtype == np.float32
    nz = s > 0
    ratio = (w.astype(np.float32) / np.where(nz, s, np.float32(1))[:, None]).astype(np.float32).astype(np.float64)
    cand = np.arange(-7, 8, dtype=np.float64)
    dist = np.abs(ratio[..., None] - cand)                   # distance to every code
    best = dist.min(axis=-1, keepdims=True)
    tied = dist == best
    # among the nearest codes take the even one (a tie is between neighbours, so exactly one is even)
    pick = np.where(tied.sum(-1) > 1, np.argmax(tied & (cand % 2 == 0), axis=-1), np.argmax(tied, axis=-1))
    expect = cand[pick].astype(np.int8)
    expect[~nz] = 0
    np.testing.assert_array_equal(q, expect)
    np.testing.assert_array_equal(q[7, :8], [7, 0, 2, 2, 0, -2, -2, 4])
    assert s[7] == 1.0 and s[5] == 0 and not q[5].any()


def test_int4_row_quantisation_invariants():
    w = _int4_test_rows(np.random.default_rng(41))
    q, s = O.quantize_int4_rows(w)
    assert np.all(np.abs(q) <= 7)
    nz = s > 0
    amax_col = np.argmax(np.abs(w), axis=1)
    top = q[np.arange(64), amax_col].astype(np.int64)
    np.testing.assert_array_equal(np.abs(top)[nz], 7)        # the row maximum maps to +-7
    np.testing.assert_array_equal(np.sign(top)[nz], np.sign(w[np.arange(64), amax_col])[nz])
    assert q[9, 3] == -7 and s[9] == np.float32(3.0) / np.float32(7.0)
    deq = O.dequantize_int4_rows(q, s)
    err = np.abs(deq - w)
    assert np.all(err[nz] <= (0.5 * s[nz, None].astype(np.float64)) * (1 + 1e-6) + 1e-12)


def test_int4_packing_matches_worked_block_and_round_trips():
    k = np.arange(64)
    q = ((k % 15) - 7).astype(np.int8)[None]
    packed = O.pack_int4_rows(q)
    assert packed.shape == (1, 32) and packed.dtype == np.uint8
    for line in open(os.path.join(GOLDEN, "int4_block.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        off, hexbytes = line.split(":")
        want = [int(b, 16) for b in hexbytes.split()]
        np.testing.assert_array_equal(packed[0, int(off):int(off) + len(want)], want)
    rng = np.random.default_rng(42)
    qq = rng.integers(-7, 8, (6, 192)).astype(np.int8)   # the code range [-7, 7]
    np.testing.assert_array_equal(O.unpack_int4_rows(O.pack_int4_rows(qq), 192), qq)
    # all-zero codes are bytes 0x00; -7 and 7 differ only in the sign bit
    assert np.all(O.pack_int4_rows(np.zeros((2, 64), np.int8)) == 0x00)
    assert np.all(O.pack_int4_rows(np.full((1, 64), -7, np.int8)) == 0xFF)
    assert np.all(O.pack_int4_rows(np.full((1, 64), 7, np.int8)) == 0x77)


def test_int4_layer_is_dense_ffn_with_dequantised_weights():
    # E=1, k=1 with int4 weights: the dense SwiGLU FFN on weights rebuilt as code * scale by torch
    rng = np.random.default_rng(43)
    N, d, f = 17, 64, 128
    x = rng.standard_normal((N, d))
    wg, wu, wd, _ = rand_layer(rng, 1, d, f)
    deq, tdeq = [], []
    for w in (wg[0], wu[0], wd[0]):
        q, s = O.quantize_int4_rows(w)
        deq.append(O.dequantize_int4_rows(q, s)[None])
        tdeq.append((torch.from_numpy(q.astype(np.int64)).double() * torch.from_numpy(s.astype(np.float64))[:, None]).numpy())
    lr = O.moe_layer(x, rng.standard_normal((1, d)), deq[0], deq[1], deq[2], 1)
    np.testing.assert_allclose(lr.y, torch_swiglu(x, tdeq[0], tdeq[1], tdeq[2]), rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------ near-tie gap of the router

def test_route_gap_planted_scores():
    # p = (0.4, 0.3, 0.2, 0.1) planted as logits log p; selection bias b = (0, 0, 0.12, 0.25), so the
    # scores s = p + b = (0.4, 0.3, 0.32, 0.35) rank 0, 3, 2, 1. The gap is the k-th largest s minus
    # the (k+1)-th, on s, not on p: k=1: 0.4 - 0.35; k=2: 0.35 - 0.32; k=3: 0.32 - 0.3; k=E: none.
    p = np.array([0.4, 0.3, 0.2, 0.1])
    b = np.array([0.0, 0.0, 0.12, 0.25])
    want = {1: 0.05, 2: 0.03, 3: 0.02}
    for k, g in want.items():
        r = O.route(np.ones((1, 1)), np.log(p)[:, None], k, select_bias=b)
        assert list(r.idx[0]) == [0, 3, 2, 1][:k]
        assert abs(r.gap[0] - g) < 1e-12, (k, r.gap[0], g)
    assert np.isinf(O.route(np.ones((1, 1)), np.log(p)[:, None], 4, select_bias=b).gap[0])
    # without the bias the gap is taken on p itself: 0.3 - 0.2 for k = 2
    assert abs(O.route(np.ones((1, 1)), np.log(p)[:, None], 2).gap[0] - 0.1) < 1e-12


def test_route_gap_is_the_selection_margin():
    # the gap equals min over the chosen experts of s minus max over the others (a set margin,
    # independent of any sort), with and without a selection bias
    rng = np.random.default_rng(21)
    x, W = rng.standard_normal((200, 16)), rng.standard_normal((10, 16)) * 0.5
    for b in (None, rng.uniform(-0.1, 0.1, 10)):
        for k in (1, 3, 9):
            r = O.route(x, W, k, select_bias=b)
            s = r.probs + (0.0 if b is None else b[None, :])
            chosen = np.zeros_like(s, dtype=bool)
            np.put_along_axis(chosen, r.idx, True, axis=1)
            margin = np.where(chosen, s, np.inf).min(1) - np.where(chosen, -np.inf, s).max(1)
            np.testing.assert_allclose(r.gap, margin, rtol=0, atol=1e-15)


def test_forced_routing_weights_bruteforce():
    # forced routing keeps p and takes the weights at the given experts, renormalised or not
    rng = np.random.default_rng(22)
    x, W = rng.standard_normal((40, 8)), rng.standard_normal((6, 8))
    r = O.route(x, W, 3, select_bias=rng.uniform(-0.1, 0.1, 6))
    idx = rng.integers(0, 6, size=(40, 3))
    for renorm in (True, False):
        f = O.forced_routing(r, idx, renorm)
        for t in range(40):
            want = [r.probs[t, e] for e in idx[t]]
            if renorm:
                want = [v / sum(want) for v in want]
            np.testing.assert_allclose(f.w[t], want, rtol=1e-15)
        np.testing.assert_array_equal(f.probs, r.probs)
    same = O.forced_routing(r, r.idx, True)
    np.testing.assert_allclose(same.w, r.w, rtol=1e-15)


# ------------------------------------------------------------------ two correct roundings of h

def test_h_band_planted_midpoint():
    # h planted within ~1e-6 of a bf16 step from the midpoint of 16 and 16.125: both roundings
    # are correct, and they are the only ones
    import planting as PL
    cfg, layer, x, planted = PL.planted_layer()
    X = mi.to_f64(x)
    b = O.h_rounding_band(X, mi.to_f64(layer.w_gate[0]), mi.to_f64(layer.w_up[0]))
    for t, f, h, mid in planted:
        assert abs(h - mid) < 1e-5 * 0.125
        assert b.amb[t, f]
        assert (b.lo[t, f], b.hi[t, f]) == (16.0, 16.125)
        assert b.ref[t, f] == O.bf16_round(h)
    # lo and hi are the bf16 roundings of h -+ bound (brute force over the bf16 grid: the nearest
    # grid value, ties to the even pattern); an element whose interval holds no midpoint has one
    bits = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    vals = mi.bf16_bits_to_f32(bits)
    fin = np.isfinite(vals)
    grid, gbits = vals[fin].astype(np.float64), bits[fin]
    order = np.argsort(grid, kind="stable")
    grid, gbits = grid[order], gbits[order]

    def nearest(v):
        i = np.searchsorted(grid, v)
        c = [j for j in (i - 1, i) if 0 <= j < grid.shape[0]]
        best = min(abs(grid[j] - v) for j in c)
        tie = [j for j in c if abs(grid[j] - v) == best]
        return grid[tie[0]] if len(tie) == 1 else grid[[j for j in tie if gbits[j] % 2 == 0][0]]
    rng = np.random.default_rng(24)
    for t, f in [(0, 20), (3, 40), (5, 63)] + [(p[0], p[1]) for p in planted[:3]] + \
            [tuple(v) for v in rng.integers(0, [16, 64], size=(20, 2))]:
        assert b.lo[t, f] == nearest(b.h[t, f] - b.bound[t, f])
        assert b.hi[t, f] == nearest(b.h[t, f] + b.bound[t, f])
        assert b.amb[t, f] == (b.lo[t, f] != b.hi[t, f])


def _fp32_eval(X, W, parts):
    """An fp32 evaluation of X @ W^T in the bound's model: exact groups of 16, fp32 accumulators
    in K order, K cut into `parts` pieces added at the end."""
    f32 = np.float32
    K = X.shape[1]
    cuts = np.linspace(0, K // 16, parts + 1).astype(int) * 16
    tot = np.zeros((X.shape[0], W.shape[0]), f32)
    for p in range(parts):
        acc = np.zeros_like(tot)
        for c in range(cuts[p], cuts[p + 1], 16):
            acc = (acc + (X[:, c:c + 16] @ W[:, c:c + 16].T).astype(f32)).astype(f32)
        tot = (tot + acc).astype(f32)
    return tot


def test_h_band_contains_fp32_evaluations():
    # the bound holds for fp32 evaluations in the modelled orders (one piece and eight pieces), and
    # every element that such an evaluation rounds differently from the oracle is marked ambiguous
    rng = np.random.default_rng(23)
    f32 = np.float32
    for d, F in ((64, 128), (512, 256), (2048, 64)):
        X = O.bf16_round(rng.standard_normal((24, d)))
        Wg = O.bf16_round(rng.standard_normal((F, d)) / math.sqrt(d))
        Wu = O.bf16_round(rng.standard_normal((F, d)) / math.sqrt(d))
        b = O.h_rounding_band(X, Wg, Wu)
        assert b.amb.mean() < 0.15
        for parts in (1, 8):
            g, u = _fp32_eval(X, Wg, parts), _fp32_eval(X, Wu, parts)
            e = np.exp(-g.astype(np.float64)).astype(f32)
            h = (g / (f32(1) + e) * u).astype(f32).astype(np.float64)
            assert np.all(np.abs(h - b.h) <= b.bound)
            hb = O.bf16_round(h)
            assert np.all((b.lo <= hb) & (hb <= b.hi))
            assert np.all(b.amb[hb != b.ref])


def test_y_rounding_flips_bruteforce():
    # y with one ambiguous h element rounded to lo or hi instead of ref is y + V[i] * (h - ref)
    import planting as PL
    cfg, layer, x, planted = PL.planted_layer()
    X = mi.to_f64(x)
    wg, wu, wd = (mi.to_f64(a[0]) for a in (layer.w_gate, layer.w_up, layer.w_down))
    for t in (0, 7):
        fl = O.y_rounding_flips(X[t], [(0.75, wg, wu, wd)])
        b = O.h_rounding_band(X[t:t + 1], wg, wu)
        cols = np.nonzero(b.amb[0])[0]
        assert fl.V.shape == (cols.shape[0], cfg.d_model) and t in cols
        np.testing.assert_array_equal(fl.lo, b.lo[0, cols])
        np.testing.assert_array_equal(fl.hi, b.hi[0, cols])
        y0 = 0.75 * (wd @ b.ref[0])
        for i, f in enumerate(cols):
            for v in (fl.lo[i], fl.hi[i]):
                h = b.ref[0].copy()
                h[f] = v
                np.testing.assert_allclose(y0 + fl.V[i] * (v - fl.ref[i]), 0.75 * (wd @ h), rtol=0, atol=1e-13)
    # a shared expert adds its own rows with weight 1
    a = O.y_rounding_flips(X[0], [], shared=([wg], [wu], [wd]))
    c = O.y_rounding_flips(X[0], [(1.0, wg, wu, wd)])
    np.testing.assert_array_equal(a.V, c.V)
    np.testing.assert_array_equal(a.lo, c.lo)
