"""moe_forward and moe_forward_noalloc captured in a HIP graph.

A serving loop captures the layer once and replays it. Every kernel of the
forward clears what it needs with its own stores (no memset nodes), so each
replay must give the eager call's outputs bit for bit. Each test captures the
call on a side stream, then replays it three times. Before each replay it
runs an eager forward of another input through the same buffers and poisons
every output.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import sparse_mixture_experts_44_amd as moe
from sparse_mixture_experts_44_amd import _native as N
from sparse_mixture_experts_44_amd.layer import MoELayer, to_device

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
FIELDS = ("y", "topk_idx", "topk_w", "counts", "offsets", "perm", "slot_pos", "prob_sum", "balance_stat")

CASES = {
    # decode-shaped: few tokens, many experts, a shared expert, selection bias (split tail tiles)
    "decode": dict(n_tokens=64, d_model=512, d_ff=256, n_experts=64, top_k=8, n_shared=1, d_ff_shared=256,
                   select_bias=0.05),
    # prefill-sized fused router, capacity dropping, skewed logits
    "capacity": dict(n_tokens=2048, d_model=256, d_ff=512, n_experts=64, top_k=1, capacity=40, logit_skew=1.0),
    # large-tile GEMMs (at least 192 rows per expert)
    "large": dict(n_tokens=1024, d_model=256, d_ff=256, n_experts=8, top_k=2),
}


def _poison(o):
    for f in FIELDS:
        t = getattr(o, f)
        if t.dtype.is_floating_point:
            t.fill_(float("nan"))
        else:
            t.fill_(-7)


def _call(L, x, noalloc):
    o = L.out
    args = (L.shape, x, L.w_router, L.logit_bias, L.select_bias, L.w_gate, L.w_up, L.w_down, L.s_gate,
            L.s_up, L.s_down, o.y, o.topk_idx, o.topk_w, o.counts, o.offsets, o.perm, o.slot_pos, o.prob_sum,
            o.balance_stat)
    if noalloc:
        N.moe_forward_noalloc(*args)
    else:
        N.moe_forward(*args, L.ws)


# the large-tile layer's workspace is beyond the static array of moe_forward_noalloc
@pytest.mark.parametrize("name,noalloc", [("decode", False), ("decode", True), ("capacity", False),
                                          ("capacity", True), ("large", False)])
def test_graph_replay_matches_eager(name, noalloc):
    cfg = mi.small_config(f"graph_{name}", layer_id=700, x_id=700, **CASES[name])
    layer, x = mi.make_layer(cfg), mi.make_x(cfg)
    x2 = mi.make_x(mi.with_(cfg, x_id=701))
    L = MoELayer.from_numpy(moe.shape_for(cfg), layer, DEV)
    xd, xd2 = to_device(x, DEV), to_device(x2, DEV)
    _call(L, xd, noalloc)
    torch.cuda.synchronize()
    ref = {f: getattr(L.out, f).clone() for f in FIELDS}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _call(L, xd, noalloc)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        _call(L, xd, noalloc)
    torch.cuda.synchronize()
    for rep in range(3):
        _call(L, xd2, noalloc)  # other values through the same buffers and workspace
        torch.cuda.synchronize()
        _poison(L.out)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        kept = int(ref["offsets"][-1])  # perm holds the kept copies only; entries past them are unspecified
        for f in FIELDS:
            got, want = getattr(L.out, f), ref[f]
            if f == "perm":
                got, want = got[:kept], want[:kept]
            assert torch.equal(got.view(torch.uint8) if got.dtype.is_floating_point else got,
                               want.view(torch.uint8) if want.dtype.is_floating_point else want), \
                f"{name} replay {rep}: {f} differs from the eager call"
        print(f"{name} ({'noalloc' if noalloc else 'ws'}): replay {rep} bitwise equal to eager", flush=True)
