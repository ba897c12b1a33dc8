"""Benchmark: the forward pass of the MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dsv3_prefill]

One step is one moe_forward over the whole layer: route, permute, the gate|up
and down grouped GEMMs, and combine. Inputs are seeded synthetic tensors
(moe_inputs), already resident in HBM when the timed region starts. The
timed region is K back-to-back steps, with a device synchronisation on each
side; in it, HIP events around the gate|up kernel give that kernel's time.
K more steps with an event at every stage boundary give the per-stage
times.

It prints one JSON line:
* value: tokens per second;
* roofline: the dominant kernel (the gate|up grouped GEMM) against the
  bf16 MFMA peak;
* cpu_baseline: the CPU oracle timed on a bounded sample of the same
  workload, on this host's cores;
* extras: layer TFLOP/s and algorithmic GB/s, and cold-cache reps (each
  after a 1 GiB write that evicts L2 and the Infinity Cache; median, min,
  max), outside the timed region;
* backward (bf16 workloads, unless --no-backward): moe_backward timed by
  HIP events, writing or accumulating the gradients, and the training
  forward with the backward that reads its kept gate and up values.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + TFLOP/s (%MFMA peak); decode HBM GB/s (%peak)"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PROFILE_DIR = os.path.join(ROOT, "profiles")


def expert_params(d_model: int, d_ff: int) -> int:
    """Parameters of one SwiGLU expert (gate, up, down; no biases): 3 * d * d_ff."""
    return 3 * d_model * d_ff


WORKLOADS = {
    # name -> (moe_inputs config, description, expert weight format, roofline bound of the gate|up kernel)
    "mixtral": ("mixtral", "Mixtral-shaped prefill: N=4096 d=4096 d_ff=14336 E=8 k=2, bf16", "bf16", "mfma"),
    "dsv3_prefill": ("dsv3_prefill", "DeepSeek-V3-shaped prefill: N=8192 d=7168 d_ff=2048 E=256 k=8 +1 shared, bf16",
                     "bf16", "mfma"),
    "dsv3_decode": ("dsv3_decode", "DeepSeek-V3-shaped decode: N=64 d=7168 d_ff=2048 E=256 k=8 +1 shared, bf16",
                    "bf16", "hbm"),
    "dsv3_decode_fp8": ("dsv3_decode", "DeepSeek-V3-shaped decode with FP8 (E4M3, per-row scale) expert weights: "
                        "N=64 d=7168 d_ff=2048 E=256 k=8 +1 shared, bf16 activations", "fp8", "hbm"),
    "dsv3_decode_int4": ("dsv3_decode", "DeepSeek-V3-shaped decode with int4 (per-row scale, W4A16) expert "
                         "weights: N=64 d=7168 d_ff=2048 E=256 k=8 +1 shared, bf16 activations", "int4", "hbm"),
    "switch_cap": ("switch_cap", "Switch-style top-1 with capacity 160: N=16384 d=2048 d_ff=8192 E=128, bf16",
                   "bf16", "hbm"),
}


def algorithmic_work(cfg, counts, kept, weights="bf16"):
    """Work the method must do, from the real routing.

    The returned dict holds:
    * flops_gate_up: 2 * d * 2F per kept copy, plus per token per shared expert;
    * flops_down: 2 * F * d per kept copy, plus the shared experts;
    * bytes: x once, W_r, every expert with at least one kept copy (3 d F
      weights each), the shared experts, fp32 y, and idx/w (8 bytes per copy);
    * bytes_gate_up: what the gate|up kernel must move: x, the gate and up
      weights of the touched experts (and the shared ones), and bf16 h out.
    FP8 expert weights count 1 byte per weight plus a 4-byte scale per row,
    int4 weights half a byte per weight plus the same scale.
    """
    import numpy as np
    d, F, E, N, k = cfg.d_model, cfg.d_ff, cfg.n_experts, cfg.n_tokens, cfg.top_k
    S, Fs = cfg.n_shared, cfg.d_ff_shared
    b = 2 if cfg.dtype == "bf16" else 4
    n_kept = int(np.sum(kept))
    touched = int(np.sum(np.asarray(kept) > 0))
    fl_gu = 2 * d * 2 * F * n_kept + S * N * 2 * d * 2 * Fs
    fl_dn = 2 * F * d * n_kept + S * N * 2 * Fs * d
    bw = {"fp8": 1, "int4": 0.5}.get(weights, b)              # bytes per expert weight
    rs = 4 if weights in ("fp8", "int4") else 0               # bytes per weight row (its scale)
    w_bytes = (touched * (expert_params(d, F) * bw + (2 * F + d) * rs)
               + S * (expert_params(d, Fs) * bw + (2 * Fs + d) * rs))
    byts = N * d * b + E * d * b + w_bytes + N * d * 4 + N * k * 8
    by_gu = (N * d * b + (touched * 2 * F * d + S * 2 * Fs * d) * bw + (touched * 2 * F + S * 2 * Fs) * rs
             + (n_kept * F + S * N * Fs) * b)
    return dict(flops_gate_up=fl_gu, flops_down=fl_dn, flops=fl_gu + fl_dn, bytes=byts,
                bytes_gate_up=by_gu, touched=touched, kept=n_kept)


def backward_work(cfg, kept):
    """FLOPs of the backward pass from the real routing (moe_backward).

    * algorithmic: what the backward must compute given the forward's
      activations: per kept copy dH' = dy Wd (2 d F), dX = [dG|dU] [Wg;Wu]
      (4 d F), dWd (2 d F), dWg and dWu (4 d F): 12 d F; the same per token per
      shared expert; the router: dW_r and dl W_r (4 N E d);
    * executed: moe_backward also recomputes G and U (4 d F per copy) and the
      router logits (2 N E d) instead of keeping them from the forward pass.

    And the bytes it must move at least (bf16 layer):
    * read: x, dy (fp32), W_r, the weights of every touched expert and of the
      shared experts;
    * written: dx (fp32), dW_r and the logit-bias gradient (fp32), and the
      expert weight gradients: every expert's in fp32 when writing them (the
      experts no copy reached get zeros), the touched and shared experts' read
      and written back when accumulating, every expert's in bf16 for bf16
      weight gradients.
    """
    import numpy as np
    d, F, E, N = cfg.d_model, cfg.d_ff, cfg.n_experts, cfg.n_tokens
    S, Fs = cfg.n_shared, cfg.d_ff_shared
    n_kept = int(np.sum(kept))
    touched = int(np.sum(np.asarray(kept) > 0))
    alg = 12 * d * F * n_kept + S * N * 12 * d * Fs + 4 * N * E * d
    exe = alg + 4 * d * F * n_kept + S * N * 4 * d * Fs + 2 * N * E * d
    common = N * d * 2 + N * d * 4 + E * d * 2 + (touched * expert_params(d, F) + S * expert_params(d, Fs)) * 2 \
        + N * d * 4 + E * d * 4 + E * 4
    grads_all = E * expert_params(d, F) + S * expert_params(d, Fs)
    grads_touched = touched * expert_params(d, F) + S * expert_params(d, Fs)
    return dict(flops_algorithmic=alg, flops_executed=exe,
                bytes_write=common + grads_all * 4, bytes_accumulate=common + grads_touched * 8,
                bytes_bf16_weight_grads=common + grads_all * 2)


def backward_roofline(flops, byts, ms):
    """The roofline a backward time is closest to: MFMA (bf16 peak) or HBM, whichever takes longer at peak."""
    t_mfma = flops / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = byts / (PEAK_HBM_GBS * 1e9)
    bound = "mfma" if t_mfma >= t_hbm else "hbm"
    return {"bound": bound, "frac": (t_mfma if bound == "mfma" else t_hbm) / (ms * 1e-3),
            "mfma_frac": t_mfma / (ms * 1e-3), "hbm_frac": t_hbm / (ms * 1e-3)}


def time_backward(L, xd, cfg, steps, warmup, kept):
    """K moe_backward calls on the last forward's routing, bracketed by HIP events on the stream
    they run on; dy is a seeded bf16-valued N(0, 1) tensor, aux_coef 0.01."""
    import torch
    g = torch.Generator(device=xd.device).manual_seed(1234)
    dy = torch.randn(cfg.n_tokens, cfg.d_model, generator=g, device=xd.device).bfloat16().float()
    stream = torch.cuda.current_stream().cuda_stream

    def timed(accumulate, bf16=False):
        for _ in range(warmup):
            L.backward(xd, dy, 0.01, accumulate=accumulate, bf16_weight_grads=bf16)
        ev = HipEvents(2)
        torch.cuda.synchronize()
        ev.record(0, stream)
        for _ in range(steps):
            L.backward(xd, dy, 0.01, accumulate=accumulate, bf16_weight_grads=bf16)
        ev.record(1, stream)
        torch.cuda.synchronize()
        return ev.elapsed_ms(0, 1) / steps

    ms, ms_acc, ms_bf16 = timed(False), timed(True), timed(False, bf16=True)
    # training forward (keeps G and U), then the backward that reads them
    for _ in range(max(1, warmup)):  # the first call also allocates the G, U buffer
        L.forward(xd, save_for_backward=True)
    ev = HipEvents(2)
    torch.cuda.synchronize()
    ev.record(0, stream)
    for _ in range(steps):
        L.forward(xd, save_for_backward=True)
    ev.record(1, stream)
    torch.cuda.synchronize()
    ms_fwd_train = ev.elapsed_ms(0, 1) / steps
    ms_saved = timed(False)
    w = backward_work(cfg, kept)
    tf = w["flops_algorithmic"] / (ms * 1e-3) / 1e12
    fl = w["flops_algorithmic"]
    return {"ms": ms, "steps": steps, "tflops_algorithmic": tf, "mfma_frac": tf / PEAK_BF16_TFLOPS,
            "tflops_executed": w["flops_executed"] / (ms * 1e-3) / 1e12, **w,
            "roofline": {"write": backward_roofline(fl, w["bytes_write"], ms),
                         "accumulate": backward_roofline(fl, w["bytes_accumulate"], ms_acc),
                         "bf16_weight_grads": backward_roofline(fl, w["bytes_bf16_weight_grads"], ms_bf16)},
            "ms_accumulate": ms_acc, "ms_bf16_weight_grads": ms_bf16, "forward_train_ms": ms_fwd_train,
            "ms_with_saved_gate_up": ms_saved,
            "note": "moe_backward alone (gradients of x, W_r, logit bias, every expert weight), writing the "
                    "gradients (ms), adding them to fp32 buffers (ms_accumulate) or writing the expert weight "
                    "gradients as bf16 (ms_bf16_weight_grads); forward_train_ms: "
                    "moe_forward_train, which keeps G and U; ms_with_saved_gate_up: the backward reading them; "
                    "algorithmic FLOPs exclude the G, U and logit recompute"}


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch has loaded."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(h.value)

    def record(self, i, stream):
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        if self.hip.hipEventRecord(self.ev[i], stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.ev[a]), ctypes.c_void_p(self.ev[b])) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_mixture_experts_44_amd", "csrc")
    for f in ("grouped_swiglu.hip", "moe_common.h"):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per gate|up launch from the committed rocprofv3 counter summary, or None.

    The summary is used only when it was taken on the current kernel source."""
    path = os.path.join(PROFILE_DIR, f"gate_up_{workload}_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_backward_baseline(cfg, layer, x, n_sample=256):
    """The backward oracle as it stands (oracle/moe_backward.layer_backward, fp64) on the first
    n_sample tokens of the workload: routing of the sample, then the gradients of every parameter
    for a seeded bf16-valued dy, including the fp64 upcast of every expert. Skipped when those
    fp64 weights would not fit comfortably in host memory (the DeepSeek-shaped layers)."""
    import numpy as np
    from threadpoolctl import threadpool_info
    import moe_inputs as mi
    from oracle import moe_backward as B
    from oracle import moe_oracle as O

    fp64_bytes = 8 * 3 * (cfg.n_experts * cfg.d_model * cfg.d_ff + cfg.n_shared * cfg.d_model * cfg.d_ff_shared)
    if fp64_bytes > 24e9:
        return {"skipped": f"the oracle's fp64 expert weights ({fp64_bytes / 1e9:.0f} GB) exceed the host budget"}
    n = min(cfg.n_tokens, n_sample)
    dy = O.bf16_round(np.random.default_rng(1234).standard_normal((n, cfg.d_model)))

    class View:
        def __init__(self, a):
            self.a = a

        def __getitem__(self, e):
            return mi.to_f64(self.a[e])

        def __len__(self):
            return len(self.a)

    t = time.perf_counter()
    x64 = mi.to_f64(x[:n])
    wr = mi.to_f64(layer.w_router)
    r = O.route(x64, wr, cfg.top_k, layer.logit_bias, layer.select_bias, cfg.renormalize)
    shared = None
    if layer.s_gate is not None:
        shared = (View(layer.s_gate), View(layer.s_up), View(layer.s_down))
    B.layer_backward(x64, wr, View(layer.w_gate), View(layer.w_up), View(layer.w_down), r.idx, dy, shared=shared,
                     logit_bias=layer.logit_bias, capacity=cfg.capacity, renormalize=cfg.renormalize, round_h=True,
                     aux_coef=0.01)
    dt = time.perf_counter() - t
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("internal_api") == "openblas"] or [1])
    return {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of {cfg.n_tokens} tokens of the same layer: route, then layer_backward in fp64 "
                      f"(every expert upcast), {dt:.1f} s"}


def cpu_baseline(cfg, layer, x, budget_s=20.0, weights="bf16"):
    """The oracle as it stands (grouped fp64 form) on the first rows of the workload.

    The sample grows from 16 rows, doubling, until one run takes about a
    tenth of the budget. It is then scaled to fill about the budget. The time
    covers routing of the sample, grouping, the fp64 upcast of each touched
    expert, the expert products and the combine. Input generation is left out.
    With FP8 weights each touched expert is quantised and dequantised by the
    oracle on the way (its form of the FP8 layer).
    """
    import numpy as np
    from threadpoolctl import threadpool_info
    import moe_inputs as mi
    from oracle import moe_oracle as O

    def run(n):
        xs = x[:n]
        t = time.perf_counter()
        r = O.route(mi.to_f64(xs), mi.to_f64(layer.w_router), cfg.top_k, layer.logit_bias,
                    layer.select_bias, cfg.renormalize)
        g = O.group(r.idx, cfg.n_experts, cfg.capacity)

        class View:
            def __init__(self, a):
                self.a = a

            def __getitem__(self, e):
                if weights == "fp8":
                    return O.dequantize_fp8_rows(*O.quantize_fp8_rows(mi.bf16_bits_to_f32(self.a[e])))
                if weights == "int4":
                    return O.dequantize_int4_rows(*O.quantize_int4_rows(mi.bf16_bits_to_f32(self.a[e])))
                return mi.to_f64(self.a[e])

            def __len__(self):
                return len(self.a)

        shared = None
        if layer.s_gate is not None:
            shared = (View(layer.s_gate), View(layer.s_up), View(layer.s_down))
        O.forward_grouped(mi.to_f64(xs), r.idx, r.w, g, View(layer.w_gate), View(layer.w_up),
                          View(layer.w_down), shared=shared, round_h=(cfg.dtype == "bf16"))
        return time.perf_counter() - t

    n = 16
    dt = run(n)
    while dt < budget_s / 10 and n * 2 <= cfg.n_tokens:
        n *= 2
        dt = run(n)
    # scale toward the budget; the time grows less than linearly in n where the fp64 upcast of
    # the touched experts dominates, so a few rounds may be needed
    for _ in range(3):
        if dt >= budget_s / 2 or n >= cfg.n_tokens:
            break
        n = int(min(cfg.n_tokens, max(n + 1, n * (budget_s / max(dt, 1e-3)) * 0.8)))
        dt = run(n)
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("internal_api") == "openblas"] or [1])
    return {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of {cfg.n_tokens} tokens of the same layer, full route+group+"
                      f"grouped fp64 experts+combine, {dt:.1f} s"}


def library_reference(cfg, kept, ours_ms, dev, reps=5):
    """The grouped forward as a per-expert loop of vendor GEMMs, for context beside our kernels.

    The pages' grouped form runs one dense product per expert over that
    expert's rows. Here each product is torch.mm (hipBLASLt on this GPU) on
    bf16 operands of the layer's shapes and value scale (rows ~ N(0, 1),
    weights ~ N(0, 1/K)), one weight matrix per segment, over the same segment
    sizes as the layer's last forward (kept rows per routed expert, then the
    shared experts' N rows). The gather of x, the SwiGLU and the combine are
    left out, which favours the loop. The same phases as one dense GEMM over
    all rows with a single weight give the library's own rate on this data.
    """
    import numpy as np
    import torch

    d, F, Fs = cfg.d_model, cfg.d_ff, cfg.d_ff_shared or cfg.d_ff
    segs = [(int(r), F) for r in kept if r > 0] + [(cfg.n_tokens, Fs)] * cfg.n_shared
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    bf = torch.bfloat16

    def rnd(*shape, scale=1.0):
        return torch.randn(*shape, device=dev, dtype=bf, generator=g) * scale

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    out = {"kind": "per-expert loop of torch.mm (hipBLASLt) over the layer's segments; random bf16 operands of "
                   "the same shapes and scale; gather, SwiGLU and combine not included",
           "segments": len(segs)}
    for phase, name in ((1, "gate_up"), (2, "down")):
        if phase == 1:
            ops = [(rnd(r, d), rnd(d, 2 * f, scale=d ** -0.5)) for r, f in segs]
        else:
            ops = [(rnd(r, f), rnd(f, d, scale=f ** -0.5)) for r, f in segs]
        ms = timed(lambda: [torch.mm(a, w) for a, w in ops])
        flops = sum(2 * a.shape[0] * a.shape[1] * w.shape[1] for a, w in ops)
        rows = sum(a.shape[0] for a, _ in ops)
        a_all, w0 = rnd(rows, ops[0][0].shape[1]), ops[0][1]
        del ops
        dense_ms = timed(lambda: torch.mm(a_all, w0))
        dense_flops = 2 * rows * a_all.shape[1] * w0.shape[1]
        del a_all, w0
        torch.cuda.empty_cache()
        out[name] = {"loop_ms": ms, "loop_tflops": flops / ms / 1e9, "ours_ms": ours_ms[name],
                     "ours_speedup": ms / ours_ms[name], "dense_one_weight_ms": dense_ms,
                     "dense_one_weight_tflops": dense_flops / dense_ms / 1e9,
                     "dense_one_weight_frac": dense_flops / dense_ms / 1e9 / PEAK_BF16_TFLOPS}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3_prefill", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--cold-reps", type=int, default=20,
                    help="extra untimed-region reps, each after a 1 GiB write that evicts L2 and the "
                         "Infinity Cache; reported as layer.cold (median/min/max)")
    ap.add_argument("--no-backward", dest="backward", action="store_false",
                    help="skip timing moe_backward and the training forward (bf16 workloads; reported as "
                         "backward, outside the headline value)")
    ap.add_argument("--backward", dest="backward", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--no-library-reference", dest="library_reference", action="store_false",
                    help="skip the per-expert vendor-GEMM loop timed for context (bf16 workloads)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device-to-device copy 3 times (calibrates the HBM byte counters)")
    args = ap.parse_args()

    if args.copy_calibration:
        import torch
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0").fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 1 << 30, "reps": 3}))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this MoE layer library has no multi-GPU path "
              "(expert-parallel sharding is a design note, not code). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import moe_inputs as mi
    import sparse_mixture_experts_44_amd as moe
    from sparse_mixture_experts_44_amd.layer import MoELayer, to_device

    cfg_name, desc, weights, bound = WORKLOADS[args.workload]
    cfg = mi.CONFIGS[cfg_name]
    t = time.time()
    layer, x = mi.make_layer(cfg), mi.make_x(cfg)
    print(f"# inputs generated in {time.time() - t:.1f}s", file=sys.stderr, flush=True)
    dev = "cuda:0"
    L = MoELayer.from_numpy(moe.shape_for(cfg), layer, dev)
    if weights == "fp8":
        L.quantize_fp8()  # one-off conversion on the device, before any timing
    elif weights == "int4":
        L.quantize_int4()
    xd = to_device(x, dev)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        L.forward(xd)
    torch.cuda.synchronize()
    K = args.steps
    # Timed region: K steps. Each step records only the two events around
    # the gate|up kernel (every recorded event adds a few microseconds of
    # stream time, so the full per-stage breakdown is taken after it).
    gu = HipEvents(2 * K)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        L.forward(xd, stage_events=[None, None, gu.ev[2 * i], gu.ev[2 * i + 1], None, None])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gate_up_ms = float(np.mean([gu.elapsed_ms(2 * i, 2 * i + 1) for i in range(K)]))

    # Per-stage breakdown: K more steps, every stage boundary recorded.
    ev = HipEvents(6 * K)
    for i in range(K):
        L.forward(xd, stage_events=ev.ev[6 * i: 6 * i + 6])
    torch.cuda.synchronize()
    stage_ms = {s: [] for s in moe.STAGES}
    step_ms = []
    for i in range(K):
        for j, s in enumerate(moe.STAGES):
            stage_ms[s].append(ev.elapsed_ms(6 * i + j, 6 * i + j + 1))
        step_ms.append(ev.elapsed_ms(6 * i, 6 * i + 5))
    avg = {s: float(np.mean(v)) for s, v in stage_ms.items()}

    # Cold-cache reps: a 1 GiB write before each rep leaves no weights in L2 or
    # the 256 MB Infinity Cache; each rep is timed by its own stage events.
    cold = None
    if args.cold_reps > 0:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        cev = HipEvents(6 * args.cold_reps)
        for i in range(args.cold_reps):
            flush.fill_(i & 0xFF)
            L.forward(xd, stage_events=cev.ev[6 * i: 6 * i + 6])
        torch.cuda.synchronize()
        rep_ms = [cev.elapsed_ms(6 * i, 6 * i + 5) for i in range(args.cold_reps)]
        cstage = {s: float(np.median([cev.elapsed_ms(6 * i + j, 6 * i + j + 1) for i in range(args.cold_reps)]))
                  for j, s in enumerate(moe.STAGES)}
        cold = {"reps": args.cold_reps, "flush_bytes": 1 << 30, "ms_median": float(np.median(rep_ms)),
                "ms_min": float(np.min(rep_ms)), "ms_max": float(np.max(rep_ms)), "stage_ms_median": cstage,
                "tokens_per_s_median": cfg.n_tokens / (float(np.median(rep_ms)) * 1e-3)}
        del flush

    counts = L.out.counts.cpu().numpy()
    offs = L.out.offsets.cpu().numpy()
    kept = np.diff(offs)
    work = algorithmic_work(cfg, counts, kept, weights)
    ms_step = wall / K * 1e3
    tok_s = cfg.n_tokens * K / wall
    gu_s = gate_up_ms * 1e-3
    if bound == "mfma":
        achieved, peak, unit, per_launch = work["flops_gate_up"] / gu_s / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s", \
            {"algorithmic_flops_per_launch": work["flops_gate_up"]}
    else:
        achieved, peak, unit, per_launch = work["bytes_gate_up"] / gu_s / 1e9, PEAK_HBM_GBS, "GB/s", \
            {"algorithmic_bytes_per_launch": work["bytes_gate_up"]}
    traffic = measured_traffic(args.workload)

    out = {
        "metric": METRIC, "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic (seeded, shapes of the pages' models)",
        "config": {"workload": desc, "tokens": cfg.n_tokens, "d_model": cfg.d_model,
                   "d_ff": cfg.d_ff, "experts": cfg.n_experts, "top_k": cfg.top_k,
                   "shared": cfg.n_shared, "capacity": cfg.capacity, "expert_weights": weights},
        "roofline": {"kernel": "grouped gate|up (phase 1)", "bound": bound, "achieved": achieved,
                     "peak": peak, "unit": unit, "frac": achieved / peak,
                     "traffic": traffic, "avg_launch_ms": gate_up_ms, **per_launch},
        "layer": {"tflops": work["flops"] / (ms_step * 1e-3) / 1e12,
                  "mfma_frac": work["flops"] / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                  "algorithmic_GBs": work["bytes"] / (ms_step * 1e-3) / 1e9,
                  "hbm_frac": work["bytes"] / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
                  "event_ms_per_step": float(np.mean(step_ms)), "stage_ms": avg,
                  "stage_ms_note": "from K extra steps after the timed region, all 6 stage events recorded",
                  "touched_experts": work["touched"], "kept_copies": work["kept"],
                  "balance_stat": float(L.out.balance_stat.item()), "cold": cold},
    }
    if args.library_reference and weights == "bf16" and cfg.dtype == "bf16":
        try:
            out["library_reference"] = library_reference(cfg, kept, avg, dev)
        except Exception as e:  # context only: never hides the forward line
            out["library_reference"] = {"error": f"{type(e).__name__}: {e}"}
    if args.backward and weights == "bf16":
        try:
            out["backward"] = time_backward(L, xd, cfg, K, args.warmup, kept)
        except Exception as e:  # the training-path timing never hides the forward line
            out["backward"] = {"error": f"{type(e).__name__}: {e}"}
    if not args.no_cpu_baseline:
        del L, xd
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline(cfg, layer, x, args.cpu_budget, weights)
        if isinstance(out.get("backward"), dict) and "ms" in out["backward"]:
            out["backward"]["cpu_baseline"] = cpu_backward_baseline(cfg, layer, x)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
