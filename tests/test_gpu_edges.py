"""GPU edge cases, each entry point through the C ABI, and determinism.

Small seeded layers, compared with the CPU oracle. Covered:
* N = 1, and N not a multiple of the router's 32-token tile;
* N = 0 (empty input);
* all logits equal (zero router), where ties go to the lower expert index;
* E = 1 with k = 1, and k = E;
* capacity 1, a capacity that drops, and one that drops nothing;
* no renormalisation;
* grouped GEMM segments of length 0, 1 and tile +- 1, for both tile shapes
  and fp32;
* bitwise determinism across two runs;
* a large router (N = 2048, E = 256, d = 1024) whose logits GEMM splits its K loops;
* a top-1 layer of 4099 tokens (the combine's four-token workgroups, the last one partial);
* capacities of 150 and 100 rows, whose gate|up runs one 160-row tile per expert;
* a seeded random sweep of 16 small layers, every knob drawn at once (bf16 and fp32).
* the staged entry points against moe_forward.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import sparse_mixture_experts_44_amd as moe
from sparse_mixture_experts_44_amd.layer import MoELayer, to_device
from oracle import moe_oracle as O

import parity as P
from test_gpu_parity import check_all, run_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def small(name, **kw):
    base = dict(n_tokens=45, d_model=128, d_ff=192, n_experts=8, top_k=2, dtype="bf16",
                layer_id=700, x_id=700)
    base.update(kw)
    return mi.MoEConfig(name=name, **base)


CASES = {
    "n1": small("n1", n_tokens=1),
    "ragged_n": small("ragged_n", n_tokens=97, n_shared=1, d_ff_shared=64),
    "e1k1": small("e1k1", n_experts=1, top_k=1),
    "k_eq_e": small("k_eq_e", n_experts=4, top_k=4),
    "cap1": small("cap1", n_tokens=40, top_k=1, capacity=1),
    "cap_drops": small("cap_drops", n_tokens=300, n_experts=16, top_k=2, capacity=20, logit_skew=1.5),
    "cap_large": small("cap_large", n_tokens=64, capacity=64 * 2),
    "no_renorm": small("no_renorm", renormalize=False, select_bias=0.05),
    "fp32_k3": small("fp32_k3", dtype="f32", n_experts=12, top_k=3, n_shared=2, d_ff_shared=128),
    "wide_e": small("wide_e", n_tokens=70, n_experts=512, top_k=32, d_model=64, d_ff=64),
    "bf16_big_tiles": small("bf16_big_tiles", n_tokens=700, n_experts=4, top_k=2, d_model=256,
                            d_ff=256, n_shared=1, d_ff_shared=128),
    # router logits on the matrix cores with 8 tiles of K = 1024: the K loops split over extra workgroups
    "wide_router": small("wide_router", n_tokens=2048, n_experts=256, top_k=8, d_model=1024, d_ff=64),
    # 256 rows per expert on average, but a selection bias piles them on a few experts (tall and
    # short segments in one launch of 256-row tiles), and a shared expert
    "large_and_small": small("large_and_small", n_tokens=2048, n_experts=32, top_k=4, d_model=256, d_ff=256,
                             n_shared=1, d_ff_shared=128, select_bias=0.1),
    # a top-1 layer with 4099 tokens: the combine takes four tokens per workgroup, the last one ragged,
    # and a capacity drops copies
    "top1_many": small("top1_many", n_tokens=4099, n_experts=16, top_k=1, d_model=128, d_ff=64,
                       capacity=300, logit_skew=1.0),
    # a capacity of 65-160 rows with 64-191 mean rows per expert: gate|up on one 160-row tile per
    # expert and weight tile. C = 150 (the last 32-row block ragged) with d_ff = 320 (the second
    # 256-column n-tile partial); C = 100 (the tile's fifth block empty), skewed so most experts fill up
    "cap150_tall": small("cap150_tall", n_tokens=2048, n_experts=16, top_k=1, d_model=256, d_ff=320,
                         capacity=150, logit_skew=1.0),
    "cap100_tall": small("cap100_tall", n_tokens=1200, n_experts=16, top_k=2, d_model=192, d_ff=256,
                         capacity=100, logit_skew=1.5, n_shared=1, d_ff_shared=128),
}


@pytest.mark.parametrize("name", list(CASES))
def test_edge_layer(name):
    cfg = CASES[name]
    layer, x = mi.make_layer(cfg), mi.make_x(cfg)
    gpu = run_gpu(cfg, layer, x)
    check_all(cfg, layer, x, gpu, per_token_rows=np.arange(min(cfg.n_tokens, 16)))


def test_zero_router_ties_to_lower_index():
    cfg = small("ties", n_tokens=33, n_experts=8, top_k=3)
    layer, x = mi.make_layer(cfg), mi.make_x(cfg)
    layer.w_router[:] = 0
    gpu = run_gpu(cfg, layer, x)
    assert np.all(gpu["topk_idx"] == np.array([0, 1, 2]))
    np.testing.assert_allclose(gpu["topk_w"], 1.0 / 3, rtol=1e-6)
    np.testing.assert_allclose(gpu["prob_sum"], 33 / 8, rtol=1e-12)
    check_all(cfg, layer, x, gpu)


def test_empty_input():
    cfg = small("empty", n_tokens=0, n_shared=1, d_ff_shared=64)
    layer = mi.make_layer(cfg)
    L = MoELayer.from_numpy(moe.shape_for(cfg), layer)
    o = L.out
    o.prob_sum.fill_(7.0)
    o.counts.fill_(7)
    o.balance_stat.fill_(7.0)
    L.forward(torch.empty(0, cfg.d_model, dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()
    assert torch.all(o.prob_sum == 0) and torch.all(o.counts == 0) and torch.all(o.offsets == 0)
    assert o.balance_stat.item() == 0.0


def test_deterministic_bitwise():
    cfg = small("det", n_tokens=1000, n_experts=32, top_k=4, d_model=256, d_ff=256, n_shared=1,
                d_ff_shared=128, capacity=140, select_bias=0.05)
    layer, x = mi.make_layer(cfg), mi.make_x(cfg)
    a, b = run_gpu(cfg, layer, x), run_gpu(cfg, layer, x)
    for k in a:
        np.testing.assert_array_equal(a[k].view(np.uint8), b[k].view(np.uint8), err_msg=k)


def test_deterministic_bitwise_small_batch():
    """A decode-sized batch: the last select workgroup adds the probability sums (its counter
    cleared by the logits launch each call), and the gate|up tail tiles split along K. Three
    calls in a row give the same bits."""
    cfg = small("det_small", n_tokens=64, n_experts=64, top_k=6, d_model=512, d_ff=256, n_shared=1,
                d_ff_shared=128, select_bias=0.05)
    layer, x = mi.make_layer(cfg), mi.make_x(cfg)
    runs = [run_gpu(cfg, layer, x) for _ in range(3)]
    for r in runs[1:]:
        for k in runs[0]:
            np.testing.assert_array_equal(runs[0][k].view(np.uint8), r[k].view(np.uint8), err_msg=k)
    check_all(cfg, layer, x, runs[0])


def _grouped_case(sizes, d, F, dtype, identity=False):
    rng = np.random.default_rng(len(sizes) * 7 + d)
    G = len(sizes)
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    rows = int(offs[-1])
    cfg = mi.small_config(n_tokens=max(rows, 1) if identity else 50, d_model=d, d_ff=F,
                          n_experts=G, top_k=1, dtype=dtype, layer_id=710, x_id=710)
    lay, x = mi.make_layer(cfg), mi.make_x(cfg)
    perm = None if identity else rng.integers(0, cfg.n_tokens * 3, size=rows).astype(np.int32)
    return cfg, lay, x, offs, perm


def _run_grouped(cfg, lay, x, offs, perm, rpt, max_rows, extra_ws=0):
    shape = moe.shape_for(cfg)
    F = cfg.d_ff
    esz = 2 if cfg.dtype == "bf16" else 4
    ws = torch.empty(max(256, ((max_rows * F * esz + 255) // 256) * 256) + extra_ws, dtype=torch.uint8, device=DEV)
    out = torch.full((max(1, max_rows), cfg.d_model), float("nan"), dtype=torch.float32, device=DEV)
    dv = lambda a: to_device(a, DEV)
    moe.moe_grouped_swiglu(shape, len(offs) - 1, F, dv(x), dv(perm) if perm is not None else None,
                           rpt, dv(offs), max_rows, dv(lay.w_gate), dv(lay.w_up), dv(lay.w_down),
                           out, ws)
    torch.cuda.synchronize()
    return P.to_host(out)


@pytest.mark.parametrize("dtype,sizes,extra_ws,slack", [
    ("bf16", [0, 1, 255, 256, 257, 0, 513, 2, 300], 0, 0),          # mean >= 128 rows: 256-row tiles
    ("bf16", [0, 1, 63, 64, 65, 0, 3, 127, 0, 0], 0, 0),            # small mean: 64-row tiles
    ("bf16", [0, 1, 255, 256, 257, 0, 513, 2, 300], 64 << 20, 0),   # the same, with split workspace
    ("bf16", [0, 1, 63, 64, 65, 0, 3, 127, 0, 0], 1 << 20, 0),      # tail tiles split along K (grid 2x the
                                                                    # tiles), workspace for a few parts only
    ("f32", [0, 1, 31, 32, 33, 0, 65], 1 << 20, 0),                 # fp32: never split
    ("bf16", [1030, 1052, 1041, 1049], 0, 0),                       # tall segments: 320-row gate|up tiles
    ("bf16", [1279, 0, 1100, 33, 1250, 1270], 0, 0),                # the same class, ragged, empty, tiny
    ("bf16", [1279, 0, 1100, 33, 1250, 1270], 64 << 20, 3 * 4932),  # max_rows 4x the rows: a grid 4x the
                                                                    # tiles, so both phases split along K
    # 256-row tiles with segments of 1, 2, 31..33 and 63..65 rows among them
    ("bf16", [1, 2, 31, 32, 33, 63, 64, 65, 600, 700, 800, 0, 900], 0, 0),
    ("bf16", [1, 2, 31, 32, 33, 63, 64, 65, 600, 700, 800, 0, 900], 64 << 20, 0),
])
def test_grouped_segment_edges(dtype, sizes, extra_ws, slack):
    _segment_edges(dtype, sizes, extra_ws, slack, 128, 256)


@pytest.mark.parametrize("sizes,extra_ws", [
    ([0, 1, 63, 64, 65, 0, 150, 191, 192, 100], 0),       # 64 to 191 mean rows: 64 x 512 gate|up tiles,
    ([0, 1, 63, 64, 65, 0, 150, 191, 192, 100], 1 << 20),  # a partial second n-tile (F = 320), split tails
])
def test_grouped_wide_gate_up_edges(sizes, extra_ws):
    _segment_edges("bf16", sizes, extra_ws, 0, 192, 320)


def _segment_edges(dtype, sizes, extra_ws, slack, d, F):
    cfg, lay, x, offs, perm = _grouped_case(sizes, d, F, dtype)
    rpt = 3
    out = _run_grouped(cfg, lay, x, offs, perm, rpt, int(offs[-1]) + slack, extra_ws)
    x64 = mi.to_f64(x)
    ref = np.zeros((int(offs[-1]), d))
    for g in range(len(sizes)):
        a, b = offs[g], offs[g + 1]
        if a == b:
            continue
        ref[a:b] = O.swiglu_expert(x64[perm[a:b] // rpt], mi.to_f64(lay.w_gate[g]), mi.to_f64(lay.w_up[g]),
                                   mi.to_f64(lay.w_down[g]), round_h=(dtype == "bf16"))
    P.check_y(out[: int(offs[-1])], ref)


def test_grouped_identity_rows_and_row_limit():
    # perm = NULL: row r reads x[r - segment start]; rows at or past max_rows are not computed
    d, F = 128, 128
    cfg, lay, x, offs, _ = _grouped_case([70, 70], d, F, "bf16", identity=True)
    max_rows = 100
    out = _run_grouped(cfg, lay, x, offs, None, 1, max_rows)
    x64 = mi.to_f64(x)
    for g in range(2):
        a, b = offs[g], min(offs[g + 1], max_rows)
        ref = O.swiglu_expert(x64[: b - a], mi.to_f64(lay.w_gate[g]), mi.to_f64(lay.w_up[g]),
                              mi.to_f64(lay.w_down[g]), round_h=True)
        P.check_y(out[a:b], ref)


def test_staged_entry_points_match_forward():
    cfg = small("staged", n_tokens=200, n_experts=16, top_k=4, n_shared=1, d_ff_shared=128,
                capacity=60, select_bias=0.05)
    layer, x = mi.make_layer(cfg), mi.make_x(cfg)
    fused = run_gpu(cfg, layer, x)
    shape = moe.shape_for(cfg)
    dv = lambda a: to_device(a, DEV)
    N, k, E, d = cfg.n_tokens, cfg.top_k, cfg.n_experts, cfg.d_model
    xd = dv(x)
    ws = torch.empty(moe.workspace_bytes(shape), dtype=torch.uint8, device=DEV)
    i32, f32, f64 = torch.int32, torch.float32, torch.float64
    idx = torch.empty(N, k, dtype=i32, device=DEV)
    w = torch.empty(N, k, dtype=f32, device=DEV)
    ps = torch.empty(E, dtype=f64, device=DEV)
    moe.moe_route(shape, xd, dv(layer.w_router), dv(layer.logit_bias), dv(layer.select_bias), idx, w, ps, ws)
    counts = torch.empty(E, dtype=i32, device=DEV)
    offs = torch.empty(E + 1, dtype=i32, device=DEV)
    perm = torch.empty(N * k, dtype=i32, device=DEV)
    slot = torch.empty(N * k, dtype=i32, device=DEV)
    stat = torch.empty(1, dtype=f64, device=DEV)
    moe.moe_permute(shape, idx, ps, counts, offs, perm, slot, stat, ws)
    O_r = torch.empty(N * k, d, dtype=f32, device=DEV)
    moe.moe_grouped_swiglu(shape, E, cfg.d_ff, xd, perm, k, offs, N * k, dv(layer.w_gate),
                           dv(layer.w_up), dv(layer.w_down), O_r, ws)
    O_s = torch.empty(N, d, dtype=f32, device=DEV)
    ws2 = torch.empty(N * cfg.d_ff_shared * 2 + 256, dtype=torch.uint8, device=DEV)
    moe.moe_grouped_swiglu(shape, 1, cfg.d_ff_shared, xd, None, 1,
                           torch.tensor([0, N], dtype=i32, device=DEV), N, dv(layer.s_gate),
                           dv(layer.s_up), dv(layer.s_down), O_s, ws2)
    y = torch.empty(N, d, dtype=f32, device=DEV)
    moe.moe_combine(shape, O_r, slot, w, O_s, y)
    torch.cuda.synchronize()
    staged = dict(topk_idx=idx, topk_w=w, prob_sum=ps, counts=counts, offsets=offs, slot_pos=slot,
                  balance_stat=stat)
    for key, t in staged.items():
        np.testing.assert_array_equal(P.to_host(t), fused[key], err_msg=key)
    P.check_y(P.to_host(y), fused["y"].astype(np.float64), tol=1e-6)


def _random_layers(n=16, seed=77):
    """Seeded random small layers: every knob of the forward drawn at once (both dtypes)."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        E = int(rng.choice([1, 3, 8, 16, 64, 128]))
        k = int(rng.integers(1, min(E, 8) + 1))
        N = int(rng.choice([1, 5, 64, 200, 333, 1000]))
        kw = dict(n_tokens=N, n_experts=E, top_k=k, d_model=int(rng.choice([64, 128, 192, 320])),
                  d_ff=int(rng.choice([64, 128, 192, 384])), renormalize=bool(rng.integers(0, 2)) or k == 1,
                  dtype="f32" if rng.random() < 0.25 else "bf16", layer_id=1000 + i, x_id=1000 + i)
        if rng.random() < 0.4:
            kw.update(n_shared=int(rng.integers(1, 3)), d_ff_shared=int(rng.choice([64, 128])))
        if rng.random() < 0.4:
            kw["capacity"] = int(rng.integers(1, max(2, 2 * N * k // E)))
        if rng.random() < 0.3:
            kw["select_bias"] = 0.05
        if rng.random() < 0.3:
            kw["logit_skew"] = 1.0
        cases.append((i, kw))
    return cases


@pytest.mark.parametrize("i,kw", _random_layers(), ids=lambda v: str(v) if isinstance(v, int) else None)
def test_random_small_layers(i, kw):
    cfg = small(f"rand{i}", **kw)
    layer, x = mi.make_layer(cfg), mi.make_x(cfg)
    gpu = run_gpu(cfg, layer, x)
    check_all(cfg, layer, x, gpu, per_token_rows=np.arange(min(cfg.n_tokens, 8)))
