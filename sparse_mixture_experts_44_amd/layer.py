"""A MoE layer whose weights stay resident in HBM and whose outputs are
preallocated: MoE(d, d_ff, n_experts, top_k, n_shared) of "混合专家 MoE"
(anrans ai-infra handbook), section "实现：逐 token 与按专家分组".

This is plumbing around moe_forward. torch allocates the device buffers, and
libmoe.so does every step of the computation.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import _native as N


def to_device(a: Optional[np.ndarray], device) -> Optional[torch.Tensor]:
    """numpy -> device tensor. uint16 arrays are bf16 bit patterns."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


@dataclass
class Outputs:
    y: torch.Tensor          # [N, d] fp32
    topk_idx: torch.Tensor   # [N, k] int32
    topk_w: torch.Tensor     # [N, k] fp32
    counts: torch.Tensor     # [E] int32
    offsets: torch.Tensor    # [E+1] int32
    perm: torch.Tensor       # [N*k] int32
    slot_pos: torch.Tensor   # [N*k] int32
    prob_sum: torch.Tensor   # [E] fp64
    balance_stat: torch.Tensor  # [1] fp64

    @classmethod
    def empty(cls, n, d, E, k, device):
        i32, f32, f64 = torch.int32, torch.float32, torch.float64
        return cls(torch.empty(n, d, dtype=f32, device=device),
                   torch.empty(n, k, dtype=i32, device=device),
                   torch.empty(n, k, dtype=f32, device=device),
                   torch.empty(E, dtype=i32, device=device),
                   torch.empty(E + 1, dtype=i32, device=device),
                   torch.empty(max(1, n * k), dtype=i32, device=device),
                   torch.empty(max(1, n * k), dtype=i32, device=device),
                   torch.empty(E, dtype=f64, device=device),
                   torch.empty(1, dtype=f64, device=device))


@dataclass
class Grads:
    """fp32 gradients of one moe_backward call (ds_*: None without shared experts)."""
    dx: torch.Tensor            # [N, d]
    dw_router: torch.Tensor     # [E, d]
    d_logit_bias: torch.Tensor  # [E]
    dw_gate: torch.Tensor       # [E, F, d]
    dw_up: torch.Tensor         # [E, F, d]
    dw_down: torch.Tensor       # [E, d, F]
    ds_gate: Optional[torch.Tensor] = None   # [S, Fs, d]
    ds_up: Optional[torch.Tensor] = None     # [S, Fs, d]
    ds_down: Optional[torch.Tensor] = None   # [S, d, Fs]

    @classmethod
    def empty(cls, s: N.MoEShape, device, weight_dtype=torch.float32):
        """weight_dtype: of the expert weight gradients (bf16 for MOE_GRAD_WRITE_BF16); the rest is fp32."""
        f = lambda *sh: torch.empty(sh, dtype=torch.float32, device=device)
        w = lambda *sh: torch.empty(sh, dtype=weight_dtype, device=device)
        E, d, F, S, Fs = s.n_experts, s.d_model, s.d_ff, s.n_shared, s.d_ff_shared
        g = cls(f(s.n_tokens, d), f(E, d), f(E), w(E, F, d), w(E, F, d), w(E, d, F))
        if S:
            g.ds_gate, g.ds_up, g.ds_down = w(S, Fs, d), w(S, Fs, d), w(S, d, Fs)
        return g


class MoELayer:
    """Weights on the device plus a workspace and outputs sized for n_tokens."""

    def __init__(self, shape: N.MoEShape, w_router, w_gate, w_up, w_down, s_gate=None, s_up=None,
                 s_down=None, logit_bias=None, select_bias=None, device="cuda:0"):
        self.shape = shape
        self.device = torch.device(device)
        self.w_router, self.w_gate, self.w_up, self.w_down = w_router, w_gate, w_up, w_down
        self.s_gate, self.s_up, self.s_down = s_gate, s_up, s_down
        self.logit_bias, self.select_bias = logit_bias, select_bias
        self._alloc()

    @classmethod
    def from_numpy(cls, shape: N.MoEShape, layer, device="cuda:0") -> "MoELayer":
        """From a moe_inputs.Layer (numpy, storage format)."""
        dv = lambda a: to_device(a, device)
        return cls(shape, dv(layer.w_router), dv(layer.w_gate), dv(layer.w_up), dv(layer.w_down),
                   dv(layer.s_gate), dv(layer.s_up), dv(layer.s_down), dv(layer.logit_bias),
                   dv(layer.select_bias), device)

    def _alloc(self):
        s = self.shape
        nbytes = N.workspace_bytes(s)
        if nbytes == 0:
            raise N.MoEError("moe_workspace_bytes", N.MOE_ERR_INVALID_ARG, "invalid shape")
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.out = Outputs.empty(s.n_tokens, s.d_model, s.n_experts, s.top_k, self.device)
        self.grads = self.grads_bf16 = self.bws = None
        self.gu = None          # fp32 G and U kept by a training forward (moe_forward_train)
        self.gu_valid = False   # whether self.gu belongs to the last forward

    fp8 = None   # after quantize_fp8(): codes and row scales of every expert weight
    int4 = None  # after quantize_int4(): packed codes and row scales of every expert weight

    def _quantize(self, kind: str, keep_bf16: bool):
        if self.shape.dtype != N.MOE_DTYPE_BF16:
            raise ValueError(f"{kind} expert weights need a bf16 layer")
        if self.fp8 is not None or self.int4 is not None:
            raise ValueError("the expert weights are already quantised")
        q = {}
        for name in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down"):
            w = getattr(self, name)
            if w is None:
                q[name] = q["sc_" + name] = None
                continue
            rows, cols = w.numel() // w.shape[-1], w.shape[-1]
            scales = torch.empty(w.shape[:-1], dtype=torch.float32, device=self.device)
            if kind == "fp8":
                codes = torch.empty(w.shape, dtype=torch.uint8, device=self.device)
                N.moe_quantize_fp8(rows, cols, w, codes, scales)
            else:
                codes = torch.empty(tuple(w.shape[:-1]) + (cols // 2,), dtype=torch.uint8, device=self.device)
                N.moe_quantize_int4(rows, cols, w, codes, scales)
            q[name], q["sc_" + name] = codes, scales
            if not keep_bf16:
                setattr(self, name, None)
        return q

    def quantize_fp8(self, keep_bf16: bool = False):
        """Quantise every expert weight (routed and shared) to FP8 E4M3 codes with
        per-row fp32 scales on the device (moe_quantize_fp8); forward then runs
        moe_forward_fp8. The bf16 expert weights are dropped unless keep_bf16."""
        self.fp8 = self._quantize("fp8", keep_bf16)
        return self.fp8

    def quantize_int4(self, keep_bf16: bool = False):
        """Quantise every expert weight (routed and shared) to packed int4 codes with
        per-row fp32 scales on the device (moe_quantize_int4); forward then runs
        moe_forward_int4. The bf16 expert weights are dropped unless keep_bf16."""
        self.int4 = self._quantize("int4", keep_bf16)
        return self.int4

    def _check_x(self, x: torch.Tensor):
        """x must be [n, d_model], on this layer's device, in the layer's dtype."""
        want = torch.bfloat16 if self.shape.dtype == N.MOE_DTYPE_BF16 else torch.float32
        if not getattr(x, "is_cuda", False) or x.device != self.w_router.device:
            raise ValueError(f"x must be a tensor on {self.w_router.device}")
        if x.dtype != want:
            raise ValueError(f"x must be {want} for this layer, not {x.dtype}")
        if x.dim() != 2 or x.shape[1] != self.shape.d_model:
            raise ValueError(f"x must be [n, {self.shape.d_model}], not {list(x.shape)}")

    def forward(self, x: torch.Tensor, stage_events=None, stream=None, save_for_backward: bool = False) -> Outputs:
        """save_for_backward (bf16 layers): run moe_forward_train, which also keeps the fp32 gate and up
        values for backward() (which then skips recomputing them)."""
        self._check_x(x)
        if x.shape[0] != self.shape.n_tokens:
            self.shape.n_tokens = x.shape[0]
            self._alloc()
        o = self.out
        self.gu_valid = False
        if save_for_backward:
            if self.fp8 is not None or self.int4 is not None:
                raise ValueError("save_for_backward needs the bf16 expert weights")
            if self.gu is None:
                self.gu = torch.empty(max(1, N.train_save_floats(self.shape)), dtype=torch.float32,
                                      device=self.device)
            N.moe_forward_train(self.shape, x, self.w_router, self.logit_bias, self.select_bias, self.w_gate,
                                self.w_up, self.w_down, self.s_gate, self.s_up, self.s_down, o.y, o.topk_idx,
                                o.topk_w, o.counts, o.offsets, o.perm, o.slot_pos, o.prob_sum, o.balance_stat,
                                self.gu, self.ws, stage_events=stage_events, stream=stream)
            self.gu_valid = True
            return o
        if self.fp8 is not None or self.int4 is not None:
            q = self.fp8 if self.fp8 is not None else self.int4
            fwd = N.moe_forward_fp8 if self.fp8 is not None else N.moe_forward_int4
            sc = N.weight_scales(q["sc_w_gate"], q["sc_w_up"], q["sc_w_down"], q["sc_s_gate"],
                                 q["sc_s_up"], q["sc_s_down"])
            fwd(self.shape, x, self.w_router, self.logit_bias, self.select_bias,
                q["w_gate"], q["w_up"], q["w_down"], q["s_gate"], q["s_up"],
                q["s_down"], sc, o.y, o.topk_idx, o.topk_w, o.counts, o.offsets,
                o.perm, o.slot_pos, o.prob_sum, o.balance_stat, self.ws,
                stage_events=stage_events, stream=stream)
            return o
        N.moe_forward(self.shape, x, self.w_router, self.logit_bias, self.select_bias, self.w_gate,
                      self.w_up, self.w_down, self.s_gate, self.s_up, self.s_down, o.y, o.topk_idx,
                      o.topk_w, o.counts, o.offsets, o.perm, o.slot_pos, o.prob_sum,
                      o.balance_stat, self.ws, stage_events=stage_events, stream=stream)
        return o

    def backward(self, x: torch.Tensor, dy: torch.Tensor, aux_coef: float = 0.0, accumulate: bool = False,
                 bf16_weight_grads: bool = False, stream=None) -> Grads:
        """Gradients (moe_backward) of sum(dy * y) + aux_coef * balance statistic for the last
        forward(x) of this bf16 layer, whose routing in self.out it reuses (and its saved gate and up
        values, after forward(..., save_for_backward=True)). The gradient buffers and the backward
        workspace are allocated on first use and reused. accumulate: add the weight gradients to the
        buffers (which start as zeros) instead of overwriting them; dx is always overwritten.
        bf16_weight_grads: the expert weight gradients as bf16 (separate buffers; not with accumulate)."""
        if accumulate and bf16_weight_grads:
            raise ValueError("bf16 weight gradients are written, not accumulated")
        if self.fp8 is not None or self.int4 is not None:
            raise ValueError("the backward pass needs the bf16 expert weights")
        self._check_x(x)
        if x.shape[0] != self.shape.n_tokens or tuple(dy.shape) != (self.shape.n_tokens, self.shape.d_model):
            raise ValueError("x and dy must match the last forward's tokens")
        if not dy.is_cuda or dy.device != x.device or dy.dtype != torch.float32:
            raise ValueError(f"dy must be a float32 tensor on {x.device}")
        if self.bws is None:
            self.bws = torch.empty(max(1, N.backward_workspace_bytes(self.shape)), dtype=torch.uint8,
                                   device=self.device)
        if bf16_weight_grads:
            if self.grads_bf16 is None:
                self.grads_bf16 = Grads.empty(self.shape, self.device, torch.bfloat16)
            g, mode = self.grads_bf16, N.MOE_GRAD_WRITE_BF16
        else:
            if self.grads is None:
                self.grads = Grads.empty(self.shape, self.device)
                for t in vars(self.grads).values():
                    if t is not None:
                        t.zero_()
            g, mode = self.grads, (N.MOE_GRAD_ACCUMULATE if accumulate else N.MOE_GRAD_WRITE)
        o = self.out
        N.moe_backward(self.shape, x, self.w_router, self.logit_bias, self.w_gate, self.w_up, self.w_down,
                       self.s_gate, self.s_up, self.s_down, o.topk_idx, o.topk_w, o.counts, o.offsets, o.perm,
                       o.slot_pos, dy, self.gu if self.gu_valid else None, aux_coef, mode, g.dx,
                       g.dw_router, g.d_logit_bias, g.dw_gate, g.dw_up, g.dw_down, g.ds_gate, g.ds_up, g.ds_down,
                       self.bws, stream=stream)
        return g
