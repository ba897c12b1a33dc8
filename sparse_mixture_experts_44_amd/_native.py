"""ctypes binding of libmoe.so (include/moe.h).

The functions here have the C names and only marshal arguments: torch tensors
become device pointers, and the current torch stream becomes the hipStream_t.
Every computation happens in the library's HIP kernels. If the library is
missing, loading fails with an error: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_DTYPE_F32, MOE_DTYPE_BF16 = 0, 1
MOE_STAGE_EVENTS = 6
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20
STAGES = ("route", "permute", "gate_up", "down", "combine")


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: {text} ({status})")
        self.status = status


class MoEShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_tokens", "d_model", "d_ff", "n_experts", "top_k", "n_shared", "d_ff_shared",
        "capacity", "renormalize", "dtype")]

    @classmethod
    def make(cls, n_tokens, d_model, d_ff, n_experts, top_k, n_shared=0, d_ff_shared=0,
             capacity=0, renormalize=True, dtype=MOE_DTYPE_BF16) -> "MoEShape":
        return cls(n_tokens, d_model, d_ff, n_experts, top_k, n_shared, d_ff_shared, capacity,
                   int(bool(renormalize)), dtype)


class MoEWeightScales(ctypes.Structure):
    """moe_weight_scales (alias moe_fp8_scales): device pointers to the fp32 row scales of the
    quantised (FP8 or int4) expert weights."""
    _fields_ = [(n, ctypes.c_void_p) for n in ("gate", "up", "down", "s_gate", "s_up", "s_down")]


MoEFp8Scales = MoEWeightScales


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32
_SZ = ctypes.c_size_t
_SHP = ctypes.POINTER(MoEShape)

_SIGS = {
    "moe_workspace_bytes": (_SZ, [_SHP]),
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_route": (ctypes.c_int, [_SHP, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_permute": (ctypes.c_int, [_SHP, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_grouped_swiglu": (ctypes.c_int, [_SHP, _I, _I, _P, _P, _I, _P, _I, _P, _P, _P, _P, _P,
                                          _SZ, _P]),
    "moe_combine": (ctypes.c_int, [_SHP, _P, _P, _P, _P, _P, _P]),
    "moe_forward": (ctypes.c_int, [_SHP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                   _P, _P, _P, _P, _P, _P, _SZ, _P, _P]),
    "moe_quantize_fp8": (ctypes.c_int, [ctypes.c_int64, _I, _P, _P, _P, _P]),
    "moe_dequantize_fp8": (ctypes.c_int, [ctypes.c_int64, _I, _P, _P, _P, _P]),
    "moe_forward_noalloc": (ctypes.c_int, [_SHP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                           _P, _P, _P, _P, _P, _P, _P]),
    "moe_train_save_floats": (_SZ, [_SHP]),
    "moe_forward_train": (ctypes.c_int, [_SHP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                         _P, _P, _P, _P, _P, _P, _P, _SZ, _P, _P]),
    "moe_router_aux": (ctypes.c_int, [_SHP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_update_select_bias": (ctypes.c_int, [_SHP, _P, ctypes.c_float, _P, _P]),
    "moe_grouped_swiglu_fp8": (ctypes.c_int, [_SHP, _I, _I, _P, _P, _I, _P, _I, _P, _P, _P, _P, _P,
                                              _P, _P, _P, _SZ, _P]),
    "moe_forward_fp8": (ctypes.c_int, [_SHP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                       ctypes.POINTER(MoEWeightScales), _P, _P, _P, _P, _P, _P, _P,
                                       _P, _P, _P, _SZ, _P, _P]),
    "moe_quantize_int4": (ctypes.c_int, [ctypes.c_int64, _I, _P, _P, _P, _P]),
    "moe_backward_workspace_bytes": (_SZ, [_SHP]),
    "moe_backward": (ctypes.c_int, [_SHP] + [_P] * 17 + [ctypes.c_double, _I] + [_P] * 10 + [_SZ, _P]),
    "moe_grouped_swiglu_int4": (ctypes.c_int, [_SHP, _I, _I, _P, _P, _I, _P, _I, _P, _P, _P, _P, _P,
                                               _P, _P, _P, _SZ, _P]),
    "moe_forward_int4": (ctypes.c_int, [_SHP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                        ctypes.POINTER(MoEWeightScales), _P, _P, _P, _P, _P, _P, _P,
                                        _P, _P, _P, _SZ, _P, _P]),
}


def lib() -> ctypes.CDLL:
    """The loaded libmoe.so (loaded once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m sparse_mixture_experts_44_amd.build`")
        import torch  # noqa: F401  (load torch's HIP runtime first, so libmoe.so shares it)
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def _check(fn: str, status: int):
    if status != MOE_OK:
        raise MoEError(fn, status, status_string(status))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not getattr(t, "is_cuda", False):
        raise ValueError("tensors passed to libmoe must be device (CUDA) tensors")
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoe must be contiguous")
    return t.data_ptr()


def _guard(fn: str, spec):
    """Host-side checks before a call: every given tensor is a contiguous device tensor, all on
    one device, and each holds at least the elements (of the dtype) the call will touch.
    spec: iterable of (name, tensor or None, minimum numel, torch dtype or None)."""
    dev = None
    for name, t, n, dt in spec:
        if t is None:
            continue
        if not getattr(t, "is_cuda", False):
            raise ValueError(f"{fn}: {name} must be a device (CUDA) tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{fn}: {name} is on {t.device}, the other tensors on {dev}")
        if dt is not None and t.dtype != dt:
            raise ValueError(f"{fn}: {name} must be {dt}, not {t.dtype}")
        if t.numel() < n:
            raise ValueError(f"{fn}: {name} holds {t.numel()} elements, the call needs {n}")


def _dims(shape):
    import torch
    act = torch.bfloat16 if shape.dtype == MOE_DTYPE_BF16 else torch.float32
    return (shape.n_tokens, shape.d_model, shape.d_ff, shape.n_experts, shape.top_k, shape.n_shared,
            shape.d_ff_shared if shape.n_shared > 0 else 0, act)


def _router_spec(shape, x, w_router, logit_bias, select_bias):
    import torch
    N, d, F, E, k, S, Fs, act = _dims(shape)
    return [("x", x, N * d, act), ("w_router", w_router, E * d, act),
            ("logit_bias", logit_bias, E, torch.float32), ("select_bias", select_bias, E, torch.float32)]


def _layer_spec(shape, x, w_router, logit_bias, select_bias, w_gate, w_up, w_down, s_gate, s_up, s_down,
                y, topk_idx, topk_w, counts, offsets, perm, slot_pos, prob_sum, balance_stat, weights="act"):
    """weights: "act" (x's dtype), "fp8" (one byte per weight) or "int4" (half a byte)."""
    import torch
    N, d, F, E, k, S, Fs, act = _dims(shape)
    wdt, per = {"act": (act, 1.0), "fp8": (torch.uint8, 1.0), "int4": (torch.uint8, 0.5)}[weights]
    i32, f32, f64 = torch.int32, torch.float32, torch.float64
    return _router_spec(shape, x, w_router, logit_bias, select_bias) + [
        ("w_gate", w_gate, int(E * F * d * per), wdt), ("w_up", w_up, int(E * F * d * per), wdt),
        ("w_down", w_down, int(E * d * F * per), wdt), ("s_gate", s_gate, int(S * Fs * d * per), wdt),
        ("s_up", s_up, int(S * Fs * d * per), wdt), ("s_down", s_down, int(S * d * Fs * per), wdt),
        ("y", y, N * d, f32), ("topk_idx", topk_idx, N * k, i32), ("topk_w", topk_w, N * k, f32),
        ("counts", counts, E, i32), ("offsets", offsets, E + 1, i32), ("perm", perm, N * k, i32),
        ("slot_pos", slot_pos, N * k, i32), ("prob_sum", prob_sum, E, f64),
        ("balance_stat", balance_stat, 1, f64)]


def _grouped_spec(shape, n_groups, d_ff, x, perm, offsets, max_rows, w_gate, w_up, w_down, out, weights="act"):
    import torch
    N, d, _, _, _, _, _, act = _dims(shape)
    wdt, per = {"act": (act, 1.0), "fp8": (torch.uint8, 1.0), "int4": (torch.uint8, 0.5)}[weights]
    G = int(n_groups)
    # perm is read for the rows below offsets[G] only, which the host does not see: dtype only
    return [("x", x, N * d, act), ("perm", perm, 0, torch.int32),
            ("offsets", offsets, G + 1, torch.int32), ("w_gate", w_gate, int(G * d_ff * d * per), wdt),
            ("w_up", w_up, int(G * d_ff * d * per), wdt), ("w_down", w_down, int(G * d * d_ff * per), wdt),
            ("out", out, int(max_rows) * d, torch.float32)]


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def workspace_bytes(shape: MoEShape) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(shape)))


def moe_route(shape, x, w_router, logit_bias, select_bias, topk_idx, topk_w, prob_sum, ws,
              stream=None):
    _guard("moe_route", _router_spec(shape, x, w_router, logit_bias, select_bias) + [
        ("topk_idx", topk_idx, shape.n_tokens * shape.top_k, None),
        ("topk_w", topk_w, shape.n_tokens * shape.top_k, None), ("prob_sum", prob_sum, shape.n_experts, None),
        ("ws", ws, 0, None)])
    _check("moe_route", lib().moe_route(
        ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(logit_bias), _ptr(select_bias),
        _ptr(topk_idx), _ptr(topk_w), _ptr(prob_sum), _ptr(ws),
        ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream)))


def moe_permute(shape, topk_idx, prob_sum, counts, offsets, perm, slot_pos, balance_stat, ws,
                stream=None):
    NK, E = shape.n_tokens * shape.top_k, shape.n_experts
    _guard("moe_permute", [("topk_idx", topk_idx, NK, None), ("prob_sum", prob_sum, E, None),
                           ("counts", counts, E, None), ("offsets", offsets, E + 1, None), ("perm", perm, NK, None),
                           ("slot_pos", slot_pos, NK, None), ("balance_stat", balance_stat, 1, None),
                           ("ws", ws, 0, None)])
    _check("moe_permute", lib().moe_permute(
        ctypes.byref(shape), _ptr(topk_idx), _ptr(prob_sum), _ptr(counts), _ptr(offsets),
        _ptr(perm), _ptr(slot_pos), _ptr(balance_stat), _ptr(ws),
        ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream)))


def moe_grouped_swiglu(shape, n_groups, d_ff, x, perm, rows_per_token, offsets, max_rows,
                       w_gate, w_up, w_down, out, ws, stream=None):
    _guard("moe_grouped_swiglu", _grouped_spec(shape, n_groups, d_ff, x, perm, offsets, max_rows, w_gate, w_up,
                                               w_down, out) + [("ws", ws, 0, None)])
    _check("moe_grouped_swiglu", lib().moe_grouped_swiglu(
        ctypes.byref(shape), int(n_groups), int(d_ff), _ptr(x), _ptr(perm), int(rows_per_token),
        _ptr(offsets), int(max_rows), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(out), _ptr(ws),
        ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream)))


def moe_combine(shape, expert_out, slot_pos, topk_w, shared_out, y, stream=None):
    N, d, k, S = shape.n_tokens, shape.d_model, shape.top_k, shape.n_shared
    _guard("moe_combine", [("expert_out", expert_out, 0, None), ("slot_pos", slot_pos, N * k, None),
                           ("topk_w", topk_w, N * k, None), ("shared_out", shared_out, S * N * d, None),
                           ("y", y, N * d, None)])
    _check("moe_combine", lib().moe_combine(
        ctypes.byref(shape), _ptr(expert_out), _ptr(slot_pos), _ptr(topk_w), _ptr(shared_out),
        _ptr(y), _stream(stream)))


def moe_forward(shape, x, w_router, logit_bias, select_bias, w_gate, w_up, w_down, s_gate, s_up,
                s_down, y, topk_idx, topk_w, counts, offsets, perm, slot_pos, prob_sum,
                balance_stat, ws, stage_events: Optional[Sequence[int]] = None, stream=None):
    ev = None
    if stage_events is not None:
        if len(stage_events) != MOE_STAGE_EVENTS:
            raise ValueError(f"stage_events needs {MOE_STAGE_EVENTS} hipEvent_t handles")
        ev = (ctypes.c_void_p * MOE_STAGE_EVENTS)(*stage_events)
    _guard("moe_forward", _layer_spec(shape, x, w_router, logit_bias, select_bias, w_gate, w_up, w_down, s_gate,
                                      s_up, s_down, y, topk_idx, topk_w, counts, offsets, perm, slot_pos,
                                      prob_sum, balance_stat) + [("ws", ws, 0, None)])
    _check("moe_forward", lib().moe_forward(
        ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(logit_bias), _ptr(select_bias),
        _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(s_gate), _ptr(s_up), _ptr(s_down), _ptr(y),
        _ptr(topk_idx), _ptr(topk_w), _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(slot_pos),
        _ptr(prob_sum), _ptr(balance_stat), _ptr(ws),
        ws.numel() * ws.element_size() if ws is not None else 0,
        ctypes.cast(ev, ctypes.c_void_p) if ev is not None else None, _stream(stream)))


def moe_forward_noalloc(shape, x, w_router, logit_bias, select_bias, w_gate, w_up, w_down, s_gate, s_up,
                        s_down, y, topk_idx, topk_w, counts, offsets, perm, slot_pos, prob_sum,
                        balance_stat, stage_events: Optional[Sequence[int]] = None, stream=None):
    """moe_forward with the library's static device workspace (no ws argument)."""
    _guard("moe_forward_noalloc", _layer_spec(shape, x, w_router, logit_bias, select_bias, w_gate, w_up, w_down,
                                              s_gate, s_up, s_down, y, topk_idx, topk_w, counts, offsets, perm,
                                              slot_pos, prob_sum, balance_stat))
    ev = None
    if stage_events is not None:
        if len(stage_events) != MOE_STAGE_EVENTS:
            raise ValueError(f"stage_events needs {MOE_STAGE_EVENTS} hipEvent_t handles")
        ev = (ctypes.c_void_p * MOE_STAGE_EVENTS)(*stage_events)
    _check("moe_forward_noalloc", lib().moe_forward_noalloc(
        ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(logit_bias), _ptr(select_bias),
        _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(s_gate), _ptr(s_up), _ptr(s_down), _ptr(y),
        _ptr(topk_idx), _ptr(topk_w), _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(slot_pos),
        _ptr(prob_sum), _ptr(balance_stat),
        ctypes.cast(ev, ctypes.c_void_p) if ev is not None else None, _stream(stream)))


def train_save_floats(shape: MoEShape) -> int:
    return int(lib().moe_train_save_floats(ctypes.byref(shape)))


def moe_forward_train(shape, x, w_router, logit_bias, select_bias, w_gate, w_up, w_down, s_gate, s_up,
                      s_down, y, topk_idx, topk_w, counts, offsets, perm, slot_pos, prob_sum,
                      balance_stat, gu_save, ws, stage_events: Optional[Sequence[int]] = None, stream=None):
    ev = None
    if stage_events is not None:
        if len(stage_events) != MOE_STAGE_EVENTS:
            raise ValueError(f"stage_events needs {MOE_STAGE_EVENTS} hipEvent_t handles")
        ev = (ctypes.c_void_p * MOE_STAGE_EVENTS)(*stage_events)
    _guard("moe_forward_train", _layer_spec(shape, x, w_router, logit_bias, select_bias, w_gate, w_up, w_down,
                                            s_gate, s_up, s_down, y, topk_idx, topk_w, counts, offsets, perm,
                                            slot_pos, prob_sum, balance_stat) +
           [("gu_save", gu_save, train_save_floats(shape), None), ("ws", ws, 0, None)])
    _check("moe_forward_train", lib().moe_forward_train(
        ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(logit_bias), _ptr(select_bias),
        _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(s_gate), _ptr(s_up), _ptr(s_down), _ptr(y),
        _ptr(topk_idx), _ptr(topk_w), _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(slot_pos),
        _ptr(prob_sum), _ptr(balance_stat), _ptr(gu_save), _ptr(ws),
        ws.numel() * ws.element_size() if ws is not None else 0,
        ctypes.cast(ev, ctypes.c_void_p) if ev is not None else None, _stream(stream)))


def moe_quantize_fp8(rows, cols, w_bf16, codes, scales, stream=None):
    _check("moe_quantize_fp8", lib().moe_quantize_fp8(
        int(rows), int(cols), _ptr(w_bf16), _ptr(codes), _ptr(scales), _stream(stream)))


def moe_dequantize_fp8(rows, cols, codes, scales, out, stream=None):
    _check("moe_dequantize_fp8", lib().moe_dequantize_fp8(
        int(rows), int(cols), _ptr(codes), _ptr(scales), _ptr(out), _stream(stream)))


def moe_grouped_swiglu_fp8(shape, n_groups, d_ff, x, perm, rows_per_token, offsets, max_rows,
                           w_gate, w_up, w_down, sc_gate, sc_up, sc_down, out, ws, stream=None):
    _guard("moe_grouped_swiglu_fp8", _grouped_spec(shape, n_groups, d_ff, x, perm, offsets, max_rows, w_gate,
                                                   w_up, w_down, out, "fp8") + [("ws", ws, 0, None)])
    _check("moe_grouped_swiglu_fp8", lib().moe_grouped_swiglu_fp8(
        ctypes.byref(shape), int(n_groups), int(d_ff), _ptr(x), _ptr(perm), int(rows_per_token),
        _ptr(offsets), int(max_rows), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(sc_gate),
        _ptr(sc_up), _ptr(sc_down), _ptr(out), _ptr(ws),
        ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream)))


def weight_scales(gate, up, down, s_gate=None, s_up=None, s_down=None) -> MoEWeightScales:
    return MoEWeightScales(*[_ptr(t) for t in (gate, up, down, s_gate, s_up, s_down)])


fp8_scales = weight_scales


def moe_quantize_int4(rows, cols, w_bf16, packed, scales, stream=None):
    _check("moe_quantize_int4", lib().moe_quantize_int4(
        int(rows), int(cols), _ptr(w_bf16), _ptr(packed), _ptr(scales), _stream(stream)))


def moe_grouped_swiglu_int4(shape, n_groups, d_ff, x, perm, rows_per_token, offsets, max_rows,
                            w_gate, w_up, w_down, sc_gate, sc_up, sc_down, out, ws, stream=None):
    _guard("moe_grouped_swiglu_int4", _grouped_spec(shape, n_groups, d_ff, x, perm, offsets, max_rows, w_gate,
                                                    w_up, w_down, out, "int4") + [("ws", ws, 0, None)])
    _check("moe_grouped_swiglu_int4", lib().moe_grouped_swiglu_int4(
        ctypes.byref(shape), int(n_groups), int(d_ff), _ptr(x), _ptr(perm), int(rows_per_token),
        _ptr(offsets), int(max_rows), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(sc_gate),
        _ptr(sc_up), _ptr(sc_down), _ptr(out), _ptr(ws),
        ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream)))


def _forward_quantised(name, shape, x, w_router, logit_bias, select_bias, w_gate, w_up, w_down,
                       s_gate, s_up, s_down, scales, y, topk_idx, topk_w, counts, offsets, perm,
                       slot_pos, prob_sum, balance_stat, ws, stage_events, stream):
    ev = None
    if stage_events is not None:
        if len(stage_events) != MOE_STAGE_EVENTS:
            raise ValueError(f"stage_events needs {MOE_STAGE_EVENTS} hipEvent_t handles")
        ev = (ctypes.c_void_p * MOE_STAGE_EVENTS)(*stage_events)
    _guard(name, _layer_spec(shape, x, w_router, logit_bias, select_bias, w_gate, w_up, w_down, s_gate, s_up,
                             s_down, y, topk_idx, topk_w, counts, offsets, perm, slot_pos, prob_sum,
                             balance_stat, "fp8" if name.endswith("fp8") else "int4") + [("ws", ws, 0, None)])
    _check(name, getattr(lib(), name)(
        ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(logit_bias), _ptr(select_bias),
        _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(s_gate), _ptr(s_up), _ptr(s_down),
        ctypes.byref(scales) if scales is not None else None, _ptr(y),
        _ptr(topk_idx), _ptr(topk_w), _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(slot_pos),
        _ptr(prob_sum), _ptr(balance_stat), _ptr(ws),
        ws.numel() * ws.element_size() if ws is not None else 0,
        ctypes.cast(ev, ctypes.c_void_p) if ev is not None else None, _stream(stream)))


def moe_forward_fp8(shape, x, w_router, logit_bias, select_bias, w_gate, w_up, w_down, s_gate,
                    s_up, s_down, scales: MoEWeightScales, y, topk_idx, topk_w, counts, offsets, perm,
                    slot_pos, prob_sum, balance_stat, ws,
                    stage_events: Optional[Sequence[int]] = None, stream=None):
    _forward_quantised("moe_forward_fp8", shape, x, w_router, logit_bias, select_bias, w_gate, w_up,
                       w_down, s_gate, s_up, s_down, scales, y, topk_idx, topk_w, counts, offsets, perm,
                       slot_pos, prob_sum, balance_stat, ws, stage_events, stream)


def moe_forward_int4(shape, x, w_router, logit_bias, select_bias, w_gate, w_up, w_down, s_gate,
                     s_up, s_down, scales: MoEWeightScales, y, topk_idx, topk_w, counts, offsets, perm,
                     slot_pos, prob_sum, balance_stat, ws,
                     stage_events: Optional[Sequence[int]] = None, stream=None):
    _forward_quantised("moe_forward_int4", shape, x, w_router, logit_bias, select_bias, w_gate, w_up,
                       w_down, s_gate, s_up, s_down, scales, y, topk_idx, topk_w, counts, offsets, perm,
                       slot_pos, prob_sum, balance_stat, ws, stage_events, stream)


def moe_router_aux(shape, x, w_router, logit_bias, topk_idx, topk_w, z_loss, importance,
                   importance_cv2, ws, stream=None):
    _check("moe_router_aux", lib().moe_router_aux(
        ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(logit_bias), _ptr(topk_idx), _ptr(topk_w),
        _ptr(z_loss), _ptr(importance), _ptr(importance_cv2), _ptr(ws),
        ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream)))


def moe_update_select_bias(shape, counts, gamma, select_bias, stream=None):
    _check("moe_update_select_bias", lib().moe_update_select_bias(
        ctypes.byref(shape), _ptr(counts), float(gamma), _ptr(select_bias), _stream(stream)))


def backward_workspace_bytes(shape: MoEShape) -> int:
    return int(lib().moe_backward_workspace_bytes(ctypes.byref(shape)))


MOE_GRAD_WRITE, MOE_GRAD_ACCUMULATE, MOE_GRAD_WRITE_BF16 = 0, 1, 2  # moe_backward's grad_mode


def moe_backward(shape, x, w_router, logit_bias, w_gate, w_up, w_down, s_gate, s_up, s_down, topk_idx, topk_w,
                 counts, offsets, perm, slot_pos, dy, gu_saved, aux_coef, grad_mode, dx, dw_router, d_logit_bias,
                 dw_gate, dw_up, dw_down, ds_gate, ds_up, ds_down, ws, stream=None):
    import torch
    N, d, F, E, k, S, Fs, act = _dims(shape)
    gdt = torch.bfloat16 if int(grad_mode) == MOE_GRAD_WRITE_BF16 else torch.float32
    _guard("moe_backward", _layer_spec(shape, x, w_router, logit_bias, None, w_gate, w_up, w_down, s_gate, s_up,
                                       s_down, None, topk_idx, topk_w, counts, offsets, perm, slot_pos, None,
                                       None) + [
        ("dy", dy, N * d, torch.float32), ("gu_saved", gu_saved, train_save_floats(shape), torch.float32),
        ("dx", dx, N * d, torch.float32), ("dw_router", dw_router, E * d, torch.float32),
        ("d_logit_bias", d_logit_bias, E, torch.float32), ("dw_gate", dw_gate, E * F * d, gdt),
        ("dw_up", dw_up, E * F * d, gdt), ("dw_down", dw_down, E * d * F, gdt),
        ("ds_gate", ds_gate, S * Fs * d, gdt), ("ds_up", ds_up, S * Fs * d, gdt),
        ("ds_down", ds_down, S * d * Fs, gdt), ("ws", ws, 0, None)])
    _check("moe_backward", lib().moe_backward(
        ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(logit_bias), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
        _ptr(s_gate), _ptr(s_up), _ptr(s_down), _ptr(topk_idx), _ptr(topk_w), _ptr(counts), _ptr(offsets),
        _ptr(perm), _ptr(slot_pos), _ptr(dy), _ptr(gu_saved), float(aux_coef), int(grad_mode), _ptr(dx),
        _ptr(dw_router),
        _ptr(d_logit_bias),
        _ptr(dw_gate), _ptr(dw_up), _ptr(dw_down), _ptr(ds_gate), _ptr(ds_up), _ptr(ds_down), _ptr(ws),
        ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream)))
