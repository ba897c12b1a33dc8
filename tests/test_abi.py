"""The C ABI without a GPU: the library loads, exports every function
include/moe.h declares, and rejects bad arguments with the documented status
before anything reaches the HIP runtime."""
import ctypes
import os
import re

import pytest

import moe_inputs as mi
import sparse_mixture_experts_44_amd as moe
from sparse_mixture_experts_44_amd import _native as N

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:[A-Za-z_][\w\s\*]*?[\s\*])(moe_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert set(names) >= {"moe_route", "moe_permute", "moe_grouped_swiglu", "moe_combine",
                          "moe_forward", "moe_workspace_bytes", "moe_status_string"}
    lib = ctypes.CDLL(N.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for st in (0, -1, -2, -3, -4, 99):
        assert isinstance(moe.status_string(st), str) and moe.status_string(st)


def shp(**kw):
    base = dict(n_tokens=64, d_model=128, d_ff=256, n_experts=8, top_k=2)
    base.update(kw)
    return N.MoEShape.make(**base)


FAKE = 0x1000  # never dereferenced: every case below fails validation first


def route(shape, ws_bytes=1 << 30, **ptrs):
    p = dict(x=FAKE, w=FAKE, idx=FAKE, tw=FAKE, ps=FAKE, ws=FAKE)
    p.update(ptrs)
    return moe.lib().moe_route(ctypes.byref(shape), p["x"], p["w"], None, None, p["idx"], p["tw"],
                               p["ps"], p["ws"], ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(top_k=0), N.MOE_ERR_INVALID_ARG),
    (dict(top_k=9), N.MOE_ERR_INVALID_ARG),
    (dict(n_tokens=-1), N.MOE_ERR_INVALID_ARG),
    (dict(d_model=0), N.MOE_ERR_INVALID_ARG),
    (dict(dtype=7), N.MOE_ERR_INVALID_ARG),
    (dict(n_shared=1, d_ff_shared=0), N.MOE_ERR_INVALID_ARG),
    (dict(d_model=100), N.MOE_ERR_UNSUPPORTED),
    (dict(d_ff=96), N.MOE_ERR_UNSUPPORTED),
    (dict(n_experts=1024, top_k=2), N.MOE_ERR_UNSUPPORTED),
    (dict(n_experts=64, top_k=33), N.MOE_ERR_UNSUPPORTED),
    # 32-bit row offsets: N * d, and N * (k + S) * max(d, F, Fs), must stay below 2^31
    (dict(n_tokens=300_000, d_model=7168, d_ff=2048, n_experts=256, top_k=1), N.MOE_ERR_UNSUPPORTED),
    (dict(n_tokens=40_000, d_model=7168, d_ff=2048, n_experts=256, top_k=8, n_shared=1, d_ff_shared=2048),
     N.MOE_ERR_UNSUPPORTED),
    (dict(n_tokens=160_000, d_model=4096, d_ff=14336, n_experts=8, top_k=2), N.MOE_ERR_UNSUPPORTED),
])
def test_shape_validation(kw, status):
    s = shp(**kw)
    assert route(s) == status
    assert moe.lib().moe_workspace_bytes(ctypes.byref(s)) == 0


def test_null_pointers_and_workspace():
    s = shp()
    assert route(s, x=None) == N.MOE_ERR_INVALID_ARG
    assert route(s, ps=None) == N.MOE_ERR_INVALID_ARG
    assert route(s, ws_bytes=16) == N.MOE_ERR_WORKSPACE
    assert moe.lib().moe_route(None, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                               None) == N.MOE_ERR_INVALID_ARG
    L = moe.lib()
    # permute: a statistic needs the probability sums
    assert L.moe_permute(ctypes.byref(s), FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                         None) == N.MOE_ERR_INVALID_ARG
    assert L.moe_permute(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8,
                         None) == N.MOE_ERR_WORKSPACE
    # grouped: bad group count, unsupported width, small workspace
    args = lambda G, F, ws: (ctypes.byref(s), G, F, FAKE, FAKE, 2, FAKE, 100, FAKE, FAKE, FAKE,
                             FAKE, FAKE, ws, None)
    assert L.moe_grouped_swiglu(*args(0, 256, 1 << 30)) == N.MOE_ERR_INVALID_ARG
    assert L.moe_grouped_swiglu(*args(4, 200, 1 << 30)) == N.MOE_ERR_UNSUPPORTED
    assert L.moe_grouped_swiglu(*args(4, 256, 1000)) == N.MOE_ERR_WORKSPACE
    # grouped: rows whose 32-bit element offsets would overflow
    big = (ctypes.byref(s), 4, 14336, FAKE, FAKE, 2, FAKE, 160_000, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert L.moe_grouped_swiglu(*big) == N.MOE_ERR_UNSUPPORTED
    # combine: shared experts need their output
    s2 = shp(n_shared=1, d_ff_shared=128)
    assert L.moe_combine(ctypes.byref(s2), FAKE, FAKE, FAKE, None, FAKE, None) == N.MOE_ERR_INVALID_ARG
    # forward: workspace below moe_workspace_bytes
    need = L.moe_workspace_bytes(ctypes.byref(s2))
    fwd = [ctypes.byref(s2)] + [FAKE] * 20 + [need - 1, None, None]
    assert L.moe_forward(*fwd) == N.MOE_ERR_WORKSPACE
    fwd[9] = None  # s_up missing with a shared expert
    assert L.moe_forward(*fwd) == N.MOE_ERR_INVALID_ARG


def test_workspace_sizes_of_the_layers():
    for name, cfg in mi.CONFIGS.items():
        s = moe.shape_for(cfg)
        nb = moe.workspace_bytes(s)
        NK, S = cfg.n_tokens * cfg.top_k, cfg.n_shared
        o_bytes = (NK + S * cfg.n_tokens) * cfg.d_model * 4
        assert nb >= o_bytes, name
        assert nb < 2 * o_bytes + (64 << 20) + NK * cfg.d_ff * 4, name


def test_fp8_entry_points_validate():
    L = moe.lib()
    # quantize: bad sizes, missing pointers, columns not a multiple of 64
    assert L.moe_quantize_fp8(-1, 64, FAKE, FAKE, FAKE, None) == N.MOE_ERR_INVALID_ARG
    assert L.moe_quantize_fp8(4, 0, FAKE, FAKE, FAKE, None) == N.MOE_ERR_INVALID_ARG
    assert L.moe_quantize_fp8(4, 64, None, FAKE, FAKE, None) == N.MOE_ERR_INVALID_ARG
    assert L.moe_quantize_fp8(4, 96, FAKE, FAKE, FAKE, None) == N.MOE_ERR_UNSUPPORTED
    assert L.moe_quantize_fp8(0, 64, None, None, None, None) == N.MOE_OK  # nothing to do
    assert L.moe_dequantize_fp8(-1, 64, FAKE, FAKE, FAKE, None) == N.MOE_ERR_INVALID_ARG
    assert L.moe_dequantize_fp8(4, 0, FAKE, FAKE, FAKE, None) == N.MOE_ERR_INVALID_ARG
    assert L.moe_dequantize_fp8(4, 64, FAKE, None, FAKE, None) == N.MOE_ERR_INVALID_ARG
    assert L.moe_dequantize_fp8(4, 12, FAKE, FAKE, FAKE, None) == N.MOE_ERR_UNSUPPORTED
    assert L.moe_dequantize_fp8(0, 64, None, None, None, None) == N.MOE_OK  # nothing to do
    # grouped: scales required, bf16 layers only
    s = shp()
    args = (64, 256, FAKE, FAKE, 2, FAKE, 128, FAKE, FAKE, FAKE)
    assert L.moe_grouped_swiglu_fp8(ctypes.byref(s), *args, None, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                                    None) == N.MOE_ERR_INVALID_ARG
    s32 = shp(dtype=N.MOE_DTYPE_F32)
    assert L.moe_grouped_swiglu_fp8(ctypes.byref(s32), *args, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                                    None) == N.MOE_ERR_UNSUPPORTED
    # forward: a scales struct with every routed pointer, and the shared ones when S > 0
    sc = N.MoEFp8Scales(FAKE, FAKE, FAKE, None, None, None)
    fw = lambda shape, scales: L.moe_forward_fp8(
        ctypes.byref(shape), FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None, None, None, scales,
        FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None, None)
    assert fw(s, None) == N.MOE_ERR_INVALID_ARG
    assert fw(s, ctypes.byref(N.MoEFp8Scales(FAKE, None, FAKE, None, None, None))) == N.MOE_ERR_INVALID_ARG
    assert fw(shp(n_shared=1, d_ff_shared=128), ctypes.byref(sc)) == N.MOE_ERR_INVALID_ARG
    assert fw(s32, ctypes.byref(sc)) == N.MOE_ERR_UNSUPPORTED
    assert fw(s, ctypes.byref(sc)) == N.MOE_ERR_WORKSPACE  # 16 bytes: validation reaches the workspace check


def test_int4_entry_points_validate():
    L = moe.lib()
    assert L.moe_quantize_int4(-1, 64, FAKE, FAKE, FAKE, None) == N.MOE_ERR_INVALID_ARG
    assert L.moe_quantize_int4(4, 0, FAKE, FAKE, FAKE, None) == N.MOE_ERR_INVALID_ARG
    assert L.moe_quantize_int4(4, 64, FAKE, None, FAKE, None) == N.MOE_ERR_INVALID_ARG
    assert L.moe_quantize_int4(4, 96, FAKE, FAKE, FAKE, None) == N.MOE_ERR_UNSUPPORTED
    assert L.moe_quantize_int4(1 << 31, 64, FAKE, FAKE, FAKE, None) == N.MOE_ERR_UNSUPPORTED
    assert L.moe_quantize_int4(0, 64, None, None, None, None) == N.MOE_OK
    s = shp()
    args = (64, 256, FAKE, FAKE, 2, FAKE, 128, FAKE, FAKE, FAKE)
    assert L.moe_grouped_swiglu_int4(ctypes.byref(s), *args, FAKE, None, FAKE, FAKE, FAKE, 1 << 30,
                                     None) == N.MOE_ERR_INVALID_ARG
    s32 = shp(dtype=N.MOE_DTYPE_F32)
    assert L.moe_grouped_swiglu_int4(ctypes.byref(s32), *args, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                                     None) == N.MOE_ERR_UNSUPPORTED
    sc = N.MoEWeightScales(FAKE, FAKE, FAKE, None, None, None)
    fw = lambda shape, scales: L.moe_forward_int4(
        ctypes.byref(shape), FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None, None, None, scales,
        FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None, None)
    assert fw(s, None) == N.MOE_ERR_INVALID_ARG
    assert fw(s, ctypes.byref(N.MoEWeightScales(FAKE, FAKE, None, None, None, None))) == N.MOE_ERR_INVALID_ARG
    assert fw(shp(n_shared=1, d_ff_shared=128), ctypes.byref(sc)) == N.MOE_ERR_INVALID_ARG
    assert fw(s32, ctypes.byref(sc)) == N.MOE_ERR_UNSUPPORTED
    assert fw(s, ctypes.byref(sc)) == N.MOE_ERR_WORKSPACE


def test_backward_entry_point_validates():
    L = moe.lib()
    s = shp()
    assert moe.backward_workspace_bytes(s) > moe.workspace_bytes(s)
    s32 = shp(dtype=N.MOE_DTYPE_F32)
    bw = lambda shape, aux=0.0, ws_bytes=1 << 40, ptr=FAKE, acc=0: L.moe_backward(
        ctypes.byref(shape), FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None, None, FAKE, FAKE, FAKE, FAKE, FAKE,
        FAKE, FAKE, None, ctypes.c_double(aux), acc, ptr, FAKE, None, FAKE, FAKE, FAKE, None, None, None, FAKE,
        ws_bytes, None)
    assert bw(s32) == N.MOE_ERR_UNSUPPORTED
    assert bw(s, aux=float("nan")) == N.MOE_ERR_INVALID_ARG
    assert bw(s, acc=3) == N.MOE_ERR_INVALID_ARG                       # unknown grad_mode
    assert bw(s, acc=-1) == N.MOE_ERR_INVALID_ARG
    assert bw(s, ptr=None) == N.MOE_ERR_INVALID_ARG                    # dx missing
    assert bw(shp(n_shared=1, d_ff_shared=128)) == N.MOE_ERR_INVALID_ARG  # shared gradients missing
    assert bw(s, ws_bytes=16) == N.MOE_ERR_WORKSPACE


def test_router_aux_entry_points_validate():
    L = moe.lib()
    s = shp()
    big = 1 << 30
    aux = lambda shape, z, imp, cv2, ws_bytes=big, x=FAKE: L.moe_router_aux(
        ctypes.byref(shape), x, FAKE, None, FAKE, FAKE, z, imp, cv2, FAKE, ws_bytes, None)
    assert aux(s, None, None, None) == N.MOE_ERR_INVALID_ARG          # nothing asked for
    assert aux(s, FAKE, None, None, ws_bytes=16) == N.MOE_ERR_WORKSPACE
    assert aux(s, FAKE, None, None, x=None) == N.MOE_ERR_INVALID_ARG   # z-loss needs x
    assert aux(shp(top_k=0), FAKE, None, None) == N.MOE_ERR_INVALID_ARG
    up = lambda shape, counts, g, b: L.moe_update_select_bias(ctypes.byref(shape), counts, g, b, None)
    assert up(s, None, 1e-3, FAKE) == N.MOE_ERR_INVALID_ARG
    assert up(s, FAKE, -1.0, FAKE) == N.MOE_ERR_INVALID_ARG
    assert up(s, FAKE, float("nan"), FAKE) == N.MOE_ERR_INVALID_ARG
    assert up(s, FAKE, float("inf"), FAKE) == N.MOE_ERR_INVALID_ARG


def test_train_forward_entry_point_validates():
    L = moe.lib()
    s = shp(n_shared=1, d_ff_shared=128)
    assert moe.train_save_floats(s) == 2 * (s.n_tokens * s.top_k * s.d_ff + s.n_tokens * s.d_ff_shared)
    assert moe.train_save_floats(shp(top_k=0)) == 0                   # invalid shape
    ft = lambda shape, gu=FAKE, ws_bytes=1 << 40: L.moe_forward_train(
        ctypes.byref(shape), FAKE, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
        FAKE, FAKE, FAKE, FAKE, FAKE, gu, FAKE, ws_bytes, None, None)
    assert ft(shp(dtype=N.MOE_DTYPE_F32)) == N.MOE_ERR_UNSUPPORTED     # bf16 layers only
    assert ft(s, gu=None) == N.MOE_ERR_INVALID_ARG                      # nowhere to keep G and U
    assert ft(s, ws_bytes=16) == N.MOE_ERR_WORKSPACE


# ------------------------------------------------------------------ host-side checks of the binding

class FakeDev:
    """Stands in for a device tensor on a host without a GPU: only what the binding's checks read."""

    def __init__(self, numel, dtype, device="cuda:0", shape=None):
        import torch
        self.is_cuda = True
        self._n = numel
        self.dtype = dtype
        self.device = torch.device(device)
        self.shape = tuple(shape) if shape is not None else (numel,)

    def numel(self):
        return self._n

    def dim(self):
        return len(self.shape)


def _layer_tensors(s, **over):
    import torch
    Nt, d, F, E, k = s.n_tokens, s.d_model, s.d_ff, s.n_experts, s.top_k
    bf, f32, i32, f64 = torch.bfloat16, torch.float32, torch.int32, torch.float64
    t = dict(x=FakeDev(Nt * d, bf), w_router=FakeDev(E * d, bf), logit_bias=None, select_bias=None,
             w_gate=FakeDev(E * F * d, bf), w_up=FakeDev(E * F * d, bf), w_down=FakeDev(E * d * F, bf),
             s_gate=None, s_up=None, s_down=None, y=FakeDev(Nt * d, f32), topk_idx=FakeDev(Nt * k, i32),
             topk_w=FakeDev(Nt * k, f32), counts=FakeDev(E, i32), offsets=FakeDev(E + 1, i32),
             perm=FakeDev(Nt * k, i32), slot_pos=FakeDev(Nt * k, i32), prob_sum=FakeDev(E, f64),
             balance_stat=FakeDev(1, f64))
    t.update(over)
    return t


def test_binding_rejects_host_tensors():
    import torch
    s = shp()
    with pytest.raises(ValueError, match="device"):
        N.moe_route(s, torch.zeros(64, 128, dtype=torch.bfloat16), None, None, None, None, None, None, None)
    with pytest.raises(ValueError, match="device"):
        N._ptr(torch.zeros(4))


@pytest.mark.parametrize("name,bad,match", [
    ("x", dict(numel=64 * 128 - 1), "elements"),            # too small
    ("x", dict(dtype="float32"), "must be"),                 # fp32 x on a bf16 layer
    ("y", dict(numel=10), "elements"),
    ("topk_idx", dict(dtype="int64"), "must be"),
    ("w_down", dict(numel=5), "elements"),
    ("perm", dict(device="cuda:1"), "is on"),               # a second device
    ("prob_sum", dict(dtype="float32"), "must be"),
])
def test_binding_checks_buffers(name, bad, match):
    import torch
    s = shp()
    t = _layer_tensors(s)
    spec = N._layer_spec(s, **t)
    N._guard("moe_forward", spec)  # the good set passes
    ref = t[name]
    kw = dict(numel=ref.numel(), dtype=ref.dtype, device="cuda:0")
    kw.update({k: (getattr(torch, v) if k == "dtype" else v) for k, v in bad.items()})
    t[name] = FakeDev(kw["numel"], kw["dtype"], kw["device"])
    with pytest.raises(ValueError, match=match):
        N._guard("moe_forward", N._layer_spec(s, **t))


def test_layer_checks_x():
    import torch
    from sparse_mixture_experts_44_amd.layer import MoELayer

    class Fake:
        shape = shp()
        w_router = FakeDev(8 * 128, torch.bfloat16)
    MoELayer._check_x(Fake, FakeDev(64 * 128, torch.bfloat16, shape=(64, 128)))
    for x, match in ((FakeDev(64 * 128, torch.float32, shape=(64, 128)), "must be torch.bfloat16"),
                     (FakeDev(64 * 256, torch.bfloat16, shape=(64, 256)), r"must be \[n, 128\]"),
                     (FakeDev(64 * 128, torch.bfloat16, device="cuda:1", shape=(64, 128)), "tensor on")):
        with pytest.raises(ValueError, match=match):
            MoELayer._check_x(Fake, x)
    with pytest.raises(ValueError, match="tensor on"):
        MoELayer._check_x(Fake, torch.zeros(64, 128, dtype=torch.bfloat16))


def test_noalloc_rejects_shapes_beyond_its_array_before_any_launch():
    # moe_forward_noalloc checks the shape's workspace against its static array first
    L = moe.lib()
    big = N.MoEShape.make(4096, 4096, 14336, 8, 2)
    assert L.moe_workspace_bytes(ctypes.byref(big)) > N.MOE_NOALLOC_SCRATCH_BYTES
    assert L.moe_forward_noalloc(ctypes.byref(big), *([FAKE] * 19), None, None) == N.MOE_ERR_UNSUPPORTED
    assert L.moe_forward_noalloc(ctypes.byref(shp(top_k=0)), *([FAKE] * 19), None, None) == N.MOE_ERR_INVALID_ARG
    assert L.moe_forward_noalloc(None, *([FAKE] * 19), None, None) == N.MOE_ERR_INVALID_ARG
