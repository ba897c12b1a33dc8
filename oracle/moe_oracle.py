"""Plain CPU oracle for the forward pass of a top-k routed MoE layer.

This is test infrastructure only. The tests, the smoke check and the
benchmark's CPU-baseline leg may use it. The GPU path never imports or calls
it, and it imports nothing from the GPU path.

Everything is computed in numpy float64. Inputs that are bf16 or fp32 in
storage are upcast exactly by the caller. Each function states the passage
it follows. The main source is the layer in "混合专家 MoE" (anrans
ai-infra handbook):

* section "结构": structure and the output formula;
* section "实现：逐 token 与按专家分组": ``moe.py``, with ``route``,
  ``forward_naive`` and ``forward_grouped``;
* section "负载均衡": ``aux_loss`` and the bias used only for selection.

Capacity dropping follows the notes "混合专家模型 (MoE)：大规模稀疏条件计算的
架构与工程实践", section 三.1 "容量因子 (Capacity Factor) 与 Token 丢弃策略".

Readings where the pages are silent:

* top-k order: larger score first; equal scores go to the lower expert index;
* capacity: copies compete in copy order c = t*k + j;
* the bf16 rounding point: only the SwiGLU intermediate h, and only for bf16
  layers.

What pins each function (in tests/test_oracle_*.py):

* softmax: row sums, the E=1 and equal-logit closed forms, and
  scipy.special.softmax;
* top-k: brute force from the counting definition on small inputs with
  planted ties;
* renormalise: sums to 1, k=1 gives 1, k=E gives p, and the printed
  0.62/0.38 figure;
* grouping: bincount and numpy's stable sort; a per-copy brute force of
  capacity; the C >= N*k and C = 0 special cases;
* experts: the per-token form equals the grouped form; E=1, k=1 equals a
  dense SwiGLU FFN built from torch.nn.functional;
* balance statistic: uniform gives 1, one-hot gives E, and the handbook's
  skewed case gives exactly 4;
* bf16_round: nearest-value brute force over every bf16 pattern, and torch's
  fp32 -> bf16 cast;
* FP8 expert weights: decode against torch's float8_e4m3fn for all 256 codes;
  encode against a nearest-code brute force and torch's cast; per-row
  quantisation against its invariants (the row maximum maps to 448, the
  dequantised error is within half a code step) and a dense layer rebuilt
  from the dequantised weights.

FP8 expert weights (a W8A16 variant for decode) follow the remark in section
"推理视角" of the handbook that DeepSeek-V3 ships its weights in FP8. The page
names no format and no scale granularity. The readings: OCP FP8 E4M3
(e4m3fn: bias 7, largest 448, no infinities), one fp32 scale per output row
of each weight matrix (scale = row max |w| / 448), codes by round-to-nearest-
even of w / scale, both divisions in fp32. The quantised layer is the bf16
layer with every expert weight replaced by scale * decode(code).

Int4 expert weights (W4A16) follow the notes "混合专家模型 (MoE)：大规模稀疏条件
计算的架构与工程实践", section 五.1: INT4 weights for the expert layers only,
activations in 16 bits, the product taken on the dequantised weights. No
granularity or rounding is given. The readings: one fp32 scale per output row
(scale = row max |w| / 7), codes q = nearest integer, ties to even, of the
fp32 quotient w / scale, in [-7, 7]. The quantised layer is the bf16 layer
with every expert weight replaced by scale * q. The packed storage
(pack_int4_rows) is the library's layout, not the pages'. Pins: the
quantisation against a nearest-integer brute force and its invariants (the
row maximum maps to 7, the error is within half a step), the packing against
a block worked out by hand (tests/golden/int4_block.txt) and a round trip, and
a dense layer rebuilt from the dequantised weights.

Training-side router statistics (z-loss, importance, the selection-bias
update) are readings of passages whose formulas were lost; each function
states its reading. Pins: closed forms (equal logits, one-hot and uniform
routing), scipy's logsumexp, numpy's bincount, an element-wise brute force.

Two correct roundings of h: the layer rounds h = silu(g) * u to bf16 at the
same point on the GPU (from fp32 sums) and here (from fp64). Where h lies
within an fp32 evaluation's error of a bf16 midpoint, every bf16 value in
[bf16(h - bound), bf16(h + bound)] is a correct rounding (h_rounding_band,
with the probabilistic fp32 error bound of fp32_dot_bound), and
y_rounding_flips gives how each such element moves y. Pins: a planted
midpoint (both neighbours, and only they), the bf16 roundings of h -+ bound
by brute force over the bf16 grid, fp32 evaluations in the modelled orders
staying inside the bound, and y with one element rounded otherwise by brute
force.

The near-tie gap of route() is the k-th minus the (k+1)-th largest selection
score (with the selection bias), pinned by planted scores and by the set
margin min(chosen) - max(others).

No page prints a value of y. On general inputs (any E, k, capacity, both
biases, shared experts) y is pinned by properties that hold for every input:
it is the sum of its single-expert shares (the layer with every other
expert's down projection zeroed, which leaves the routing as it is), each
share being w times torch's dense SwiGLU FFN on the tokens whose kept copy
chose that expert and zero elsewhere; it does not change when the experts
are relabelled; and without a capacity its rows follow the token order.
The per-token and grouped forms agree.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Optional, Sequence

import numpy as np

F64 = np.float64


# ---------------------------------------------------------------- rounding

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127

# ---------------------------------------------------------------- FP8 (E4M3) weights

FP8_MAX = 448.0          # largest finite e4m3fn value: 1.75 * 2**8
_FP8_MIN_NORMAL = 2.0 ** -6
_FP8_SUB_STEP = 2.0 ** -9  # code step below the smallest normal


def fp8_e4m3_decode(codes) -> np.ndarray:
    """Values of e4m3fn codes (fp64): sign bit 7, exponent bits 6..3 with bias
    7, mantissa bits 2..0; exponent 0 is subnormal (m * 2**-9); 0x7F and 0xFF
    are NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * _FP8_SUB_STEP, (1.0 + m / 8.0) * np.exp2(e.astype(F64) - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def fp8_e4m3_encode(v) -> np.ndarray:
    """Round float values to the nearest e4m3fn code, ties to the even code,
    the sign bit copied from the input;
    magnitudes that round above 448 saturate to 448 (this quantisation never
    produces them: |w / scale| <= 448 up to one fp32 rounding)."""
    a = np.abs(np.asarray(v, dtype=F64))
    neg = np.signbit(np.asarray(v, dtype=F64))
    # code step: 2**(exponent - 3) for normal magnitudes, 2**-9 below 2**-6
    _, ex = np.frexp(np.where(a > 0, a, 1.0))          # a = f * 2**ex, f in [0.5, 1)
    step = np.where(a >= _FP8_MIN_NORMAL, np.exp2((ex - 1 - 3).astype(F64)), _FP8_SUB_STEP)
    q = np.rint(a / step) * step                       # exact: a / step is a scaled binary value
    q = np.minimum(q, FP8_MAX)
    # value -> code
    sub = q < _FP8_MIN_NORMAL
    m_sub = np.rint(q / _FP8_SUB_STEP).astype(np.int64)   # 0..8 (8 is the smallest normal)
    _, qe = np.frexp(np.where(q > 0, q, 1.0))
    e_field = (qe - 1 + 7).astype(np.int64)
    m_norm = np.rint((q / np.exp2((qe - 1).astype(F64)) - 1.0) * 8.0).astype(np.int64)
    code = np.where(sub, m_sub, (e_field << 3) | m_norm)
    code = np.where(neg, code | 0x80, code)  # the sign bit follows the input's (-0 and tiny negatives: 0x80)
    return code.astype(np.uint8)


def quantize_fp8_rows(w) -> tuple:
    """Per-output-row FP8 quantisation of one weight matrix [rows, cols]:
    scale_r = fp32(max_c |w[r, c]|) / 448 in fp32; code = e4m3(fp32(w / scale_r));
    an all-zero row has scale 0 and codes 0. Returns (codes uint8, scales fp32)."""
    w32 = np.asarray(w, dtype=np.float32)
    amax = np.max(np.abs(w32), axis=1)
    scale = (amax / np.float32(FP8_MAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    ratio = (w32 / safe[:, None]).astype(np.float32)
    codes = fp8_e4m3_encode(ratio)
    codes[scale == 0] = 0
    return codes, scale


def dequantize_fp8_rows(codes, scales) -> np.ndarray:
    """scale_r * decode(code) in fp64 (exact)."""
    return fp8_e4m3_decode(codes) * np.asarray(scales, dtype=F64)[:, None]


# ---------------------------------------------------------------- int4 weights (W4A16)

INT4_MAX = 7
_INT4_SHIFT = np.array([8 * (j % 4) + 4 * (j // 4) for j in range(8)])  # bit position of code j in its word


def _int4_field(q):
    """The 4-bit sign and magnitude field of int4 codes: 8 + |q| for q < 0, else q."""
    q = np.asarray(q, dtype=np.int64)
    return np.where(q < 0, 8 - q, q)


def quantize_int4_rows(w) -> tuple:
    """Per-output-row int4 quantisation of one weight matrix [rows, cols]:
    scale_r = fp32(max_c |w[r, c]|) / 7 in fp32; q = the nearest integer to
    fp32(w / scale_r), ties to even, clamped to [-7, 7]; an all-zero row has
    scale 0 and codes 0. Returns (codes int8, scales fp32)."""
    w32 = np.asarray(w, dtype=np.float32)
    amax = np.max(np.abs(w32), axis=1)
    scale = (amax / np.float32(INT4_MAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    ratio = (w32 / safe[:, None]).astype(np.float32)
    q = np.clip(np.rint(ratio.astype(F64)), -INT4_MAX, INT4_MAX).astype(np.int8)
    q[scale == 0] = 0
    return q, scale


def dequantize_int4_rows(codes, scales) -> np.ndarray:
    """scale_r * q in fp64 (exact)."""
    return np.asarray(codes, dtype=F64) * np.asarray(scales, dtype=F64)[:, None]


def pack_int4_rows(codes) -> np.ndarray:
    """The packed storage of int4 codes [rows, cols] (cols a multiple of 64):
    per block of 64 codes, the little-endian 32-bit word at byte 16 h + 4 s
    holds codes 16 s + 8 h + j (j = 0..7), each as a 4-bit sign and
    magnitude field (8 + |q| for q < 0, else q), code j in byte j % 4 of the
    word, low nibble for j < 4 and high nibble for j >= 4. Returns uint8
    [rows, cols / 2]."""
    q = np.asarray(codes, dtype=np.int64)
    rows, cols = q.shape
    f = _int4_field(q).reshape(rows, cols // 64, 4, 2, 8).astype(np.uint64)   # [row, block, s, h, j]
    words = np.zeros((rows, cols // 64, 4, 2), dtype=np.uint64)
    for j in range(8):
        words |= f[..., j] << np.uint64(_INT4_SHIFT[j])
    words = words.transpose(0, 1, 3, 2)                                                   # [row, block, h, s]
    return np.ascontiguousarray(words.astype("<u4")).view(np.uint8).reshape(rows, cols // 2)


def unpack_int4_rows(packed, cols: int) -> np.ndarray:
    """Codes [rows, cols] (int8) from their packed storage (inverse of pack_int4_rows)."""
    b = np.ascontiguousarray(np.asarray(packed, dtype=np.uint8))
    rows = b.shape[0]
    words = b.reshape(rows, cols // 2).view("<u4").reshape(rows, cols // 64, 2, 4)  # [row, block, h, s]
    words = words.transpose(0, 1, 3, 2).astype(np.int64)                           # [row, block, s, h]
    q = np.zeros((rows, cols // 64, 4, 2, 8), dtype=np.int64)
    for j in range(8):
        f = (words >> int(_INT4_SHIFT[j])) & 0xF
        q[..., j] = np.where(f & 8, -(f & 7), f & 7)
    return q.reshape(rows, cols).astype(np.int8)



def bf16_round(a) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits. The smallest normal is 2^-126, and
    below it the spacing is fixed at 2^-133. Values that round past the
    largest finite bf16 become +-inf. The result is returned as float64.
    """
    a = np.asarray(a, dtype=F64)
    _, e = np.frexp(a)                  # a = m * 2^e with 0.5 <= |m| < 1
    e = np.maximum(e, -125)             # fixed spacing in the subnormal range
    q = np.rint(np.ldexp(a, 8 - e))     # integer count of spacings; rint ties to even
    r = np.ldexp(q, e - 8)
    big = np.abs(r) > _BF16_MAX
    if np.any(big):
        r = np.where(big, np.copysign(np.inf, a), r)
    return r


# ---------------------------------------------------------------- router

def softmax(logits: np.ndarray) -> np.ndarray:
    """Row softmax in float64: p_e = exp(l_e - max) / sum_e' exp(l_e' - max).

    The router's probabilities in ``route`` ("实现" section) are the softmax
    of its linear layer's output over the experts. Subtracting the row
    maximum changes no value mathematically.
    """
    l = np.asarray(logits, dtype=F64)
    z = np.exp(l - l.max(axis=-1, keepdims=True))
    return z / z.sum(axis=-1, keepdims=True)


def router_logits(x: np.ndarray, w_router: np.ndarray,
                  logit_bias: Optional[np.ndarray] = None) -> np.ndarray:
    """l[t, e] = x[t] . W_r[e] (+ logit_bias[e]).

    The router is ``nn.Linear(d, E, bias=False)``, so y = x W_r^T. The
    optional additive bias is the gate ``nn.Linear(input_dim, num_experts)``
    (with bias) in MoEGating on the cloud.baidu.com overview of MoE. It also
    carries the Zipf-like skew of the capacity workload.
    """
    l = np.asarray(x, dtype=F64) @ np.asarray(w_router, dtype=F64).T
    if logit_bias is not None:
        l = l + np.asarray(logit_bias, dtype=F64)[None, :]
    return l


def topk_order(scores: np.ndarray, k: int) -> np.ndarray:
    """idx[t, :k]: the k largest scores of row t, largest first.

    Order: a larger score ranks first, and equal scores rank the lower expert
    index first. A stable sort of -s gives exactly this order (library sort
    as one step).
    """
    s = np.asarray(scores, dtype=F64)
    order = np.argsort(-s, axis=-1, kind="stable")
    return order[..., :k].astype(np.int64)


@dataclass
class Routing:
    idx: np.ndarray       # [N, k] int64, expert ids, best first
    w: np.ndarray         # [N, k] float64 combine weights
    probs: np.ndarray     # [N, E] float64 softmax (without the selection bias)
    gap: np.ndarray       # [N] float64: s_(k) - s_(k+1) (inf when k == E)


def route(x, w_router, k: int, logit_bias=None, select_bias=None,
          renormalize: bool = True) -> Routing:
    """Router of the layer: linear, softmax, (selection bias), top-k, renormalise.

    Follows ``route`` ("实现" section): the probabilities are the softmax of
    the router's logits; the k largest give the chosen experts and their
    weights; the weights are then divided by their sum.

    The selection-only bias comes from the aux-loss-free balancing bullet of
    the "负载均衡" section: the bias is added to the scores used to choose the
    top-k and does not change the weights. So the weights are always taken
    from the unbiased p.
    """
    p = softmax(router_logits(x, w_router, logit_bias))
    s = p if select_bias is None else p + np.asarray(select_bias, dtype=F64)[None, :]
    idx = topk_order(s, k)
    w = combine_weights(p, idx, renormalize)
    E = p.shape[1]
    if k < E:
        # the near-tie measure: the k-th largest selection score minus the
        # (k+1)-th, on s (the scores that choose), not on p
        srt = -np.sort(-s, axis=1)
        gap = srt[:, k - 1] - srt[:, k]
    else:
        gap = np.full(p.shape[0], np.inf)
    return Routing(idx=idx, w=w, probs=p, gap=gap)


def combine_weights(probs, idx, renormalize: bool = True) -> np.ndarray:
    """w[t, j] = p[t, idx[t, j]], divided by the sum over the token's k
    chosen experts when renormalising ("实现" section, ``route``). Always the
    unbiased p: the selection bias only chooses ("负载均衡" section)."""
    w = np.take_along_axis(np.asarray(probs, dtype=F64), np.asarray(idx, dtype=np.int64), axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return w


def forced_routing(r: "Routing", idx, renormalize: bool = True) -> "Routing":
    """The routing with the expert choice replaced by a given idx: p and the
    near-tie gaps stay those of ``r``; the weights are p at the given experts,
    renormalised the same way. Each later step of the layer can then be
    checked on that choice of experts."""
    idx = np.asarray(idx, dtype=np.int64)
    return Routing(idx=idx, w=combine_weights(r.probs, idx, renormalize), probs=r.probs, gap=r.gap)


# ---------------------------------------------------------------- grouping

def expert_counts(idx: np.ndarray, n_experts: int) -> np.ndarray:
    """counts[e] = number of (token, slot) copies routed to e, before capacity.

    ``forward_grouped`` ("实现" section) counts the flattened expert ids per
    expert, empty experts included.
    """
    counts = np.zeros(n_experts, dtype=np.int64)
    for e in np.asarray(idx).reshape(-1):
        counts[int(e)] += 1
    return counts


def capacity_keep(idx: np.ndarray, n_experts: int, capacity: int) -> np.ndarray:
    """keep[c] for every copy c = t*k + j: does it fit in its expert's buffer?

    Follows the token-dropping rule in section 三.1 of the notes: each expert
    has a static buffer of ``capacity`` rows, and the copies beyond it skip
    every expert branch. The pages do not say which copies overflow. Here
    copies take their places in copy order, so a copy is kept iff fewer than
    C earlier copies went to the same expert. capacity <= 0 means no limit.
    """
    flat = np.asarray(idx).reshape(-1)
    keep = np.ones(flat.shape[0], dtype=bool)
    if capacity <= 0:
        return keep
    fill = np.zeros(n_experts, dtype=np.int64)
    for c, e in enumerate(flat):
        e = int(e)
        if fill[e] < capacity:
            fill[e] += 1
        else:
            keep[c] = False
    return keep


@dataclass
class Grouping:
    counts: np.ndarray    # [E] routed copies per expert (before capacity)
    kept: np.ndarray      # [E] copies that fit the capacity
    offsets: np.ndarray   # [E+1] exclusive prefix sum of kept
    perm: np.ndarray      # [sum kept] copy ids grouped by expert, increasing within a group
    slot_pos: np.ndarray  # [N*k] row of each copy in perm, -1 if dropped


def group(idx: np.ndarray, n_experts: int, capacity: int = 0) -> Grouping:
    """Sort the token copies by expert: count, capacity, prefix sum, permutation.

    ``forward_grouped`` ("实现" section) flattens idx, takes a stable argsort
    by expert, and walks the segments with a running start. That section
    also names the histogram and the prefix sum of starts. Dropped copies are
    left out of their segment.
    """
    flat = np.asarray(idx).reshape(-1).astype(np.int64)
    counts = expert_counts(idx, n_experts)
    keep = capacity_keep(idx, n_experts, capacity)
    order = np.argsort(flat, kind="stable")           # copies sorted by (expert, copy id)
    perm = order[keep[order]]
    kept = np.zeros(n_experts, dtype=np.int64)
    for c in perm:
        kept[flat[c]] += 1
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(kept)
    slot_pos = np.full(flat.shape[0], -1, dtype=np.int64)
    slot_pos[perm] = np.arange(perm.shape[0])
    return Grouping(counts=counts, kept=kept, offsets=offsets, perm=perm, slot_pos=slot_pos)


# ---------------------------------------------------------------- experts

def silu(z) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z)) (``F.silu`` in the Expert module)."""
    z = np.asarray(z, dtype=F64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_expert(X, w_gate, w_up, w_down, round_h: bool) -> np.ndarray:
    """Expert(x) = down(silu(gate(x)) * up(x)) for the rows of X.

    This is ``Expert.forward`` ("实现" section). gate_proj and up_proj are
    ``nn.Linear(d, d_ff)``, so their weights are [d_ff, d]. down_proj is
    ``nn.Linear(d_ff, d)``, with weight [d, d_ff]. In bf16 layers the
    intermediate h is rounded to bf16 before the down projection.
    """
    X = np.atleast_2d(np.asarray(X, dtype=F64))
    g = X @ np.asarray(w_gate, dtype=F64).T
    u = X @ np.asarray(w_up, dtype=F64).T
    h = silu(g) * u
    if round_h:
        h = bf16_round(h)
    return h @ np.asarray(w_down, dtype=F64).T


WeightSet = Sequence  # indexable by expert id -> 2-D array (converted to float64 on use)


# ---------------------------------------------------------------- where two roundings of h are correct
#
# The layer rounds h = silu(g) * u to bf16 before the down projection, and the
# fp32 GPU path and this fp64 oracle round it at the same point. A value of h
# that lies very close to the midpoint between two bf16 neighbours may round
# either way, depending only on the last bits of an fp32 evaluation of g and
# u. Reading: such an element has two correct roundings. The functions below
# find these elements, under a stated error bound of an fp32 evaluation, and
# give the change of y for each alternative rounding.

U32 = 2.0 ** -24   # unit roundoff of fp32


@dataclass
class HBand:
    h: np.ndarray      # [R, F] silu(g) * u in fp64, before rounding
    ref: np.ndarray    # bf16_round(h)
    lo: np.ndarray     # the smallest correct bf16 rounding: bf16_round(h - bound)
    hi: np.ndarray     # the largest: bf16_round(h + bound)
    bound: np.ndarray  # error bound of an fp32 evaluation of h (absolute)
    amb: np.ndarray    # lo < hi: more than one rounding is correct


LAMBDA = 8.0       # confidence of the probabilistic bound: P(exceeded) <= 2 exp(-LAMBDA^2 / 2) ~ 2.5e-14


def fp32_dot_bound(X, W, chunk: int = 16, parts: int = 8, lam: float = LAMBDA) -> np.ndarray:
    """Probabilistic error bound of an fp32 evaluation of X @ W^T (rows of bf16 values).

    The evaluation model: products of bf16 values are exact in fp32; groups
    of at most ``chunk`` consecutive products along K are summed (each sum
    that rounds is within 4 u of its sum of |terms|, u = 2^-24) and added to
    an fp32 accumulator in K order; K may be cut into at most ``parts``
    contiguous pieces whose accumulators are added at the end. The bound
    follows the probabilistic rounding error analysis of Higham and Mary ("A
    New Approach to Probabilistic Rounding Error Analysis", SIAM J. Sci.
    Comput. 41(5), 2019): the rounding errors are independent and mean zero,
    each at most u times the value it rounds, so by the Azuma-Hoeffding
    inequality their sum exceeds lam * u * sqrt(sum of the squared values)
    with probability at most 2 exp(-lam^2 / 2). The rounded values are:
      * the accumulators: the partial sums S_i (sums of the first i groups)
        of their piece, S_i - S_c for a piece starting at group c, whose
        squares are at most 2 S_i^2 + 2 M^2 (M = max_i |S_i|); plus at most
        ``parts`` additions of pieces, each at most 2 M;
      * the group sums, at most 4 times their sum of |terms| A_c each.
    Hence, per output element, with n groups,
        |fp32 - exact| <= lam * u * (sqrt(2 sum_i S_i^2 + (2 n + 4 parts) M^2) + 4 sqrt(sum_c A_c^2)).
    A worst-case bound (every error at its maximum with the same sign) would
    be n / sqrt(n) times larger and would mark most elements of a long K.
    """
    X = np.atleast_2d(np.asarray(X, dtype=F64))
    W = np.atleast_2d(np.asarray(W, dtype=F64))
    R, K = X.shape
    n = -(-K // chunk)
    pad = n * chunk - K
    if pad:
        X = np.pad(X, ((0, 0), (0, pad)))
        W = np.pad(W, ((0, 0), (0, pad)))
    Xc = X.reshape(R, n, chunk)
    Wc = W.reshape(W.shape[0], n, chunk)
    S = np.cumsum(np.einsum("rci,fci->rfc", Xc, Wc), axis=2)
    M = np.max(np.abs(S), axis=2)
    A = np.einsum("rci,fci->rfc", np.abs(Xc), np.abs(Wc))
    acc = np.sqrt(2.0 * np.sum(S * S, axis=2) + (2.0 * n + 4.0 * parts) * M * M)
    grp = 4.0 * np.sqrt(np.sum(A * A, axis=2))
    return lam * U32 * (acc + grp)


def h_rounding_band(X, w_gate, w_up, *, chunk: int = 16, parts: int = 8, scaled: bool = False) -> HBand:
    """For the rows of X through one expert: h, its bf16 rounding, the range
    of correct bf16 roundings, and the error bound of an fp32 evaluation.

    An fp32 evaluation lands in [h - bound, h + bound], and rounding to bf16
    is monotone, so every bf16 value from bf16_round(h - bound) to
    bf16_round(h + bound) is a correct rounding. Next to a midpoint that is
    the two neighbours; where the bound exceeds a bf16 step (h near zero
    after cancellation in g or u) it is more.

    The bound of h combines the bounds of g and u (fp32_dot_bound) through
    h = silu(g) * u, with a factor 2 for the linearisation, plus 8 units of
    fp32 roundoff of |h| for the SiLU and the product themselves (exp, a
    reciprocal, two products and a sum, each within about one unit, taken at
    their worst).
    ``scaled``: the weights carry per-row scales applied after the sum
    (quantised weights), one more fp32 rounding of g and of u.
    """
    X = np.atleast_2d(np.asarray(X, dtype=F64))
    Wg = np.asarray(w_gate, dtype=F64)
    Wu = np.asarray(w_up, dtype=F64)
    g = X @ Wg.T
    u = X @ Wu.T
    eg = fp32_dot_bound(X, Wg, chunk, parts)
    eu = fp32_dot_bound(X, Wu, chunk, parts)
    if scaled:
        eg = eg + U32 * np.abs(g)
        eu = eu + U32 * np.abs(u)
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))
    s = g * sig
    ds = sig * (1.0 + g * (1.0 - sig))      # d silu / d g
    h = s * u
    bound = 2.0 * (np.abs(ds * u) * eg + np.abs(s) * eu) + 8.0 * U32 * np.abs(h) + 2.0 ** -140
    return HBand(h=h, ref=bf16_round(h), lo=bf16_round(h - bound), hi=bf16_round(h + bound), bound=bound,
                 amb=bf16_round(h - bound) < bf16_round(h + bound))


@dataclass
class YFlips:
    """The outputs y_t that other correct roundings of h allow:
    y_t(choice) = y_t + sum_i V[i] * (h_i - ref[i]) for bf16 values h_i in [lo[i], hi[i]]."""
    V: np.ndarray      # [m, d]: weight * W_down[:, f] of each ambiguous element
    ref: np.ndarray    # [m] the oracle's rounding of each
    lo: np.ndarray     # [m] smallest correct rounding
    hi: np.ndarray     # [m] largest correct rounding


def y_rounding_flips(x_t, experts, shared=None, *, scaled: bool = False) -> YFlips:
    """The ambiguous h elements of one token's row (h_rounding_band) and how
    each moves y_t.

    ``experts`` lists the token's kept copies as (weight, w_gate, w_up,
    w_down); ``shared`` is None or a tuple (s_gate, s_up, s_down) of weight
    sets (weight 1). Row i of V is weight * W_down[:, f] for one ambiguous
    element f of one copy: y_t with that element rounded to h instead of ref
    is y_t + V[i] * (h - ref).
    """
    x_t = np.atleast_2d(np.asarray(x_t, dtype=F64))
    items = list(experts)
    if shared is not None:
        sg, su, sd = shared
        items += [(1.0, sg[s], su[s], sd[s]) for s in range(len(sg))]
    V, ref, lo, hi = [], [], [], []
    for wt, wg, wu, wd in items:
        b = h_rounding_band(x_t, wg, wu, scaled=scaled)
        f = np.nonzero(b.amb[0])[0]
        if f.size:
            V.append(float(wt) * np.asarray(wd, dtype=F64)[:, f].T)
            ref.append(b.ref[0, f])
            lo.append(b.lo[0, f])
            hi.append(b.hi[0, f])
    if not V:
        z = np.zeros(0)
        return YFlips(V=np.zeros((0, x_t.shape[1])), ref=z, lo=z, hi=z)
    return YFlips(V=np.concatenate(V), ref=np.concatenate(ref), lo=np.concatenate(lo), hi=np.concatenate(hi))


def forward_per_token(x, idx, w, keep, w_gate: WeightSet, w_up: WeightSet, w_down: WeightSet,
                      shared=None, round_h: bool = False, rows=None) -> np.ndarray:
    """The per-token form: y_t = sum_j w[t,j] Expert_{idx[t,j]}(x_t) + sum_s Shared_s(x_t).

    Follows ``forward_naive`` ("实现" section) and the output formula in
    section "结构". Each kept copy is one matrix-vector expert application on
    one token row. A dropped copy adds nothing. The layer returns no residual:
    section 三.1 of the notes sends dropped tokens through the residual path,
    which lies outside the layer. Shared experts have no gate and weight 1 on
    every token ("结构", DeepSeekMoE's second point).

    ``shared`` is None or a tuple (s_gate, s_up, s_down) of weight sets.
    ``rows`` restricts the output to those token rows (all rows if None).
    """
    x = np.asarray(x, dtype=F64)
    N = x.shape[0]
    k = idx.shape[1]
    rows = np.arange(N) if rows is None else np.asarray(rows)
    keep = np.asarray(keep).reshape(N, k)
    cache = {}

    def weights(e):
        if e not in cache:
            cache[e] = (np.asarray(w_gate[e], dtype=F64), np.asarray(w_up[e], dtype=F64),
                        np.asarray(w_down[e], dtype=F64))
        return cache[e]

    out = np.zeros((rows.shape[0], x.shape[1]), dtype=F64)
    for i, t in enumerate(rows):
        for j in range(k):
            if not keep[t, j]:
                continue
            e = int(idx[t, j])
            out[i] += w[t, j] * swiglu_expert(x[t], *weights(e), round_h=round_h)[0]
        if shared is not None:
            sg, su, sd = shared
            for s in range(len(sg)):
                out[i] += swiglu_expert(x[t], sg[s], su[s], sd[s], round_h=round_h)[0]
    return out


def forward_grouped(x, idx, w, grouping: Grouping, w_gate: WeightSet, w_up: WeightSet,
                    w_down: WeightSet, shared=None, round_h: bool = False, rows=None) -> np.ndarray:
    """The grouped form: one matrix product per expert over its segment.

    Follows ``forward_grouped`` ("实现" section). The segment of expert e is
    ``perm[offsets[e]:offsets[e+1]]``, and its token ids are c // k. Each
    segment with at least one row runs the expert once over all of its rows.
    The result is added back at the tokens, scaled by their weights. Empty
    segments are skipped, as that section's second exercise requires.

    ``rows`` keeps only those token rows, in the order given (all if None).
    Each segment then holds only the copies of those tokens.
    """
    x = np.asarray(x, dtype=F64)
    N, k = idx.shape
    rows = np.arange(N) if rows is None else np.asarray(rows)
    where = np.full(N, -1, dtype=np.int64)   # token -> output row, -1 if not kept
    where[rows] = np.arange(rows.shape[0])
    out = np.zeros((rows.shape[0], x.shape[1]), dtype=F64)
    wf = np.asarray(w, dtype=F64).reshape(-1)
    E = grouping.offsets.shape[0] - 1
    for e in range(E):
        a, b = int(grouping.offsets[e]), int(grouping.offsets[e + 1])
        sel = grouping.perm[a:b]
        sel = sel[where[sel // k] >= 0]
        if sel.shape[0] == 0:
            continue
        tok = sel // k
        y = swiglu_expert(x[tok], w_gate[e], w_up[e], w_down[e], round_h=round_h)
        np.add.at(out, where[tok], y * wf[sel][:, None])
    if shared is not None:
        sg, su, sd = shared
        for s in range(len(sg)):
            out += swiglu_expert(x[rows], sg[s], su[s], sd[s], round_h=round_h)
    return out


# ---------------------------------------------------------------- statistic

def balance_stat(counts, prob_sum, n_tokens: int, top_k: int) -> float:
    """E * sum_e f_e P_e, the load-balancing statistic.

    This is ``aux_loss`` ("负载均衡" section), written there as
    E * sum_i f_i P_i:

    * f_e = counts_e / (N*k), the share of the copies: the page divides the
      counts by the number of entries of idx, which is N*k;
    * P_e = prob_sum_e / N, the mean router probability.

    counts are the routed copies before capacity.
    """
    counts = np.asarray(counts, dtype=F64)
    prob_sum = np.asarray(prob_sum, dtype=F64)
    E = counts.shape[0]
    f = counts / float(n_tokens * top_k)
    P = prob_sum / float(n_tokens)
    return float(E * np.sum(f * P))



# ---------------------------------------------------------------- training-side router statistics
#
# Side outputs for training, next to the forward pass. The formulas on the
# pages are lost in extraction, so each is a reading (stated per function).

def z_loss(logits) -> float:
    """Router z-loss: the mean over tokens of logsumexp(logits)^2.

    The notes (section 三.3 "路由策略稳定性与 Z-Loss") apply it to the raw gate
    logits before top-k, to bound their magnitude. Reading: the ST-MoE form
    (1/N) sum_t (log sum_e exp l[t, e])^2 on the logits that enter the
    softmax (with the logit bias). An empty batch gives 0.
    """
    l = np.asarray(logits, dtype=F64)
    if l.shape[0] == 0:
        return 0.0
    m = l.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(l - m).sum(axis=1))
    return float(np.mean(lse * lse))


def importance(idx, w, n_experts: int) -> np.ndarray:
    """Importance of each expert: the sum of the gate weights it was given.

    The notes (section 二, "Importance Loss") penalise the spread of the gate
    weights over experts. Reading: importance_e = sum over copies routed to e
    (before capacity) of their weight w.
    """
    idx = np.asarray(idx, dtype=np.int64).reshape(-1)
    w = np.asarray(w, dtype=F64).reshape(-1)
    return np.bincount(idx, weights=w, minlength=n_experts).astype(F64)


def importance_cv2(imp) -> float:
    """The importance loss: squared coefficient of variation of importance over
    experts, Var/Mean^2 with the population variance (0 if the mean is 0)."""
    imp = np.asarray(imp, dtype=F64)
    mean = imp.mean()
    if mean == 0:
        return 0.0
    return float(((imp - mean) ** 2).mean() / (mean * mean))


def update_select_bias(bias, counts, n_tokens: int, top_k: int, gamma: float) -> np.ndarray:
    """One step of the aux-loss-free balancing of section "负载均衡" (handbook):
    the selection bias of an overloaded expert goes down and that of an idle
    one goes up. Reading (no step size or rule on the page): with the mean load
    N*k/E, b_e <- b_e - gamma * sign(counts_e - N*k/E), in fp32 (the bias's
    storage type); counts before capacity."""
    b = np.asarray(bias, dtype=np.float32)
    E = b.shape[0]
    c = np.asarray(counts, dtype=F64)
    s = np.sign(c - float(n_tokens) * float(top_k) / float(E)).astype(np.float32)
    return (b - np.float32(gamma) * s).astype(np.float32)

# ---------------------------------------------------------------- whole layer

@dataclass
class LayerResult:
    routing: Routing
    grouping: Grouping
    prob_sum: np.ndarray
    stat: float
    y: Optional[np.ndarray]


def moe_layer(x, w_router, w_gate, w_up, w_down, k: int, *, shared=None, logit_bias=None,
              select_bias=None, capacity: int = 0, renormalize: bool = True,
              round_h: bool = False, form: str = "per_token", rows=None,
              forced_idx: Optional[np.ndarray] = None) -> LayerResult:
    """Route, group, run the experts and combine, in the pages' order.

    With ``forced_idx`` set, routing still computes p, but the expert choice
    comes from the given idx. The weights are then p at those experts,
    renormalised the same way. This forced-routing mode lets each later step
    be checked on a given choice of experts. ``form`` is "per_token" (the
    authority), "grouped", or "none" to skip the experts.
    """
    r = route(x, w_router, k, logit_bias, select_bias, renormalize)
    if forced_idx is not None:
        r = forced_routing(r, forced_idx, renormalize)
    E = r.probs.shape[1]
    g = group(r.idx, E, capacity)
    prob_sum = r.probs.sum(axis=0)
    stat = balance_stat(g.counts, prob_sum, r.idx.shape[0], k)
    y = None
    if form == "per_token":
        y = forward_per_token(x, r.idx, r.w, g.slot_pos >= 0, w_gate, w_up, w_down,
                              shared=shared, round_h=round_h, rows=rows)
    elif form == "grouped":
        y = forward_grouped(x, r.idx, r.w, g, w_gate, w_up, w_down, shared=shared,
                            round_h=round_h, rows=rows)
    return LayerResult(routing=r, grouping=g, prob_sum=prob_sum, stat=stat, y=y)
