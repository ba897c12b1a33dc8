// C ABI of libmoe.so (declared in include/moe.h): argument validation,
// workspace layout and launch order. Nothing here allocates, synchronises
// or keeps state between calls.
#include <math.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <utility>

#include "moe_common.h"

namespace moe {
namespace {

__global__ void fill_f64_kernel(double* p, int n, double v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

size_t esize(const moe_shape& s) { return s.dtype == MOE_DTYPE_BF16 ? 2 : 4; }

int check_shape(const moe_shape* sp) {
  if (!sp) return MOE_ERR_INVALID_ARG;
  const moe_shape& s = *sp;
  if (s.n_tokens < 0 || s.d_model <= 0 || s.d_ff <= 0 || s.n_experts <= 0) return MOE_ERR_INVALID_ARG;
  if (s.top_k < 1 || s.top_k > s.n_experts) return MOE_ERR_INVALID_ARG;
  if (s.n_shared < 0 || (s.n_shared > 0 && s.d_ff_shared <= 0)) return MOE_ERR_INVALID_ARG;
  if (s.dtype != MOE_DTYPE_F32 && s.dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;
  if (s.renormalize != 0 && s.renormalize != 1) return MOE_ERR_INVALID_ARG;
  if (s.d_model % 64 || s.d_ff % 64 || (s.n_shared > 0 && s.d_ff_shared % 64)) return MOE_ERR_UNSUPPORTED;
  if (s.n_experts > kMaxExperts || s.top_k > kMaxTopK) return MOE_ERR_UNSUPPORTED;
  if (s.n_shared > kMaxShared) return MOE_ERR_UNSUPPORTED;
  const long long N = s.n_tokens;
  if (N * s.top_k >= (1LL << 31) || N * (s.top_k + s.n_shared) >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  // the kernels index rows of x, h and the expert outputs with 32-bit element offsets
  const long long F = std::max(s.d_ff, s.n_shared > 0 ? s.d_ff_shared : 0);
  if (N * s.d_model >= (1LL << 31) || N * (s.top_k + s.n_shared) * std::max<long long>(F, s.d_model) >= (1LL << 31))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Workspace layout shared by the entry points (byte offsets, 256-aligned).
struct Layout {
  size_t partials, logits, hist, base, aux, split, h_routed, h_shared, o, total;
};

Layout layout(const moe_shape& s) {
  Layout L;
  const size_t N = (size_t)s.n_tokens, NK = N * s.top_k, E = (size_t)s.n_experts;
  const size_t S = (size_t)s.n_shared;
  size_t off = 0;
  L.partials = off;
  off += align256(route_partials_bytes(s));
  L.logits = off;
  off += align256(route_logits_floats(s) * sizeof(float));
  L.hist = off;
  off += align256((size_t)permute_chunks(s) * E * sizeof(int32_t));
  L.base = off;
  off += align256((size_t)permute_chunks(s) * E * sizeof(int32_t));
  L.aux = off;  // router statistics: importance when the caller does not keep it
  off += align256(E * sizeof(double));
  L.split = off;  // K-parts of the grouped GEMMs' split tail tiles (bf16 layers)
  off += align256(s.dtype == MOE_DTYPE_BF16 && N > 0 ? grouped_split_bytes((long long)NK, s.n_experts) : 0);
  L.h_routed = off;
  off += align256(NK * s.d_ff * esize(s));
  L.h_shared = off;
  off += align256(S * N * (S ? s.d_ff_shared : 0) * esize(s));
  L.o = off;
  off += align256((NK + S * N) * s.d_model * sizeof(float));
  L.total = off;
  return L;
}

inline uint8_t* at(void* ws, size_t off) { return static_cast<uint8_t*>(ws) + off; }

int zero_f64(double* p, int n, hipStream_t st) {
  if (n <= 0) return MOE_OK;
  hipLaunchKernelGGL(fill_f64_kernel, dim3((n + 255) / 256), dim3(256), 0, st, p, n, 0.0);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// defer_nb: see launch_route (the forward hands the last step to the permutation)
int do_route(const moe_shape& s, const void* x, const void* w_router, const float* lb, const float* sb,
             int32_t* idx, float* tw, double* prob_sum, void* ws, hipStream_t st, int* defer_nb = nullptr) {
  if (defer_nb) *defer_nb = 0;
  if (s.n_tokens == 0) return zero_f64(prob_sum, s.n_experts, st);
  const Layout L = layout(s);
  // the grouped GEMMs' split region is idle while routing: a large router's GEMM uses it
  return launch_route(s, x, w_router, lb, sb, idx, tw, prob_sum,
                      reinterpret_cast<double*>(at(ws, L.partials)),
                      reinterpret_cast<float*>(at(ws, L.logits)), reinterpret_cast<float*>(at(ws, L.split)),
                      L.h_routed - L.split, st, defer_nb);
}

int do_permute(const moe_shape& s, const int32_t* idx, const double* prob_sum, int32_t* counts,
               int32_t* offsets, int32_t* perm, int32_t* slot_pos, double* stat, void* ws,
               hipStream_t st, int nb = 0, double* sum_out = nullptr) {
  const Layout L = layout(s);
  return launch_permute(s, idx, prob_sum, counts, offsets, perm, slot_pos, stat,
                        reinterpret_cast<int32_t*>(at(ws, L.hist)),
                        reinterpret_cast<int32_t*>(at(ws, L.base)), st,
                        nb > 0 ? reinterpret_cast<const double*>(at(ws, L.partials)) : nullptr, nb, sum_out);
}

// wq: expert weight format (0 bf16/fp32, 8 FP8 codes, 4 packed int4 codes; the last two with row scales)
int grouped_impl(const moe_shape* shape, int32_t n_groups, int32_t d_ff, const void* x,
                 const int32_t* perm, int32_t rows_per_token, const int32_t* offsets, int32_t max_rows,
                 const void* w_gate, const void* w_up, const void* w_down, int wq, const float* sc_gate,
                 const float* sc_up, const float* sc_down, float* out, void* ws, size_t ws_bytes,
                 hipStream_t stream) {
  if (!shape) return MOE_ERR_INVALID_ARG;
  const moe_shape& s = *shape;
  if (s.n_tokens < 0 || s.d_model <= 0 || d_ff <= 0 || n_groups < 1 || max_rows < 0 || rows_per_token < 1)
    return MOE_ERR_INVALID_ARG;
  if (s.dtype != MOE_DTYPE_F32 && s.dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;
  if (!offsets || !w_gate || !w_up || !w_down || (max_rows > 0 && (!x || !out || !ws)))
    return MOE_ERR_INVALID_ARG;
  if (s.d_model % 64 || d_ff % 64 || n_groups > kMaxTileEntries) return MOE_ERR_UNSUPPORTED;
  // 32-bit element offsets into x and h rows
  if ((long long)s.n_tokens * s.d_model >= (1LL << 31) ||
      (long long)max_rows * std::max(d_ff, s.d_model) >= (1LL << 31))
    return MOE_ERR_UNSUPPORTED;
  const size_t need = align256((size_t)max_rows * d_ff * esize(s));
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (max_rows == 0 || s.n_tokens == 0) return MOE_OK;
  GroupedParams p{};
  p.n_sets = 1;
  p.x = x;
  p.n_tokens = s.n_tokens;
  p.d_model = s.d_model;
  p.dtype = s.dtype;
  p.wq = wq;
  if (s.dtype == MOE_DTYPE_BF16 && ws_bytes >= need + 256) {  // workspace past h: tail-tile K-parts
    p.split_ws = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + need);
    p.split_cap = (long long)((ws_bytes - need) / sizeof(float));
  }
  SegSet& S = p.set[0];
  S.offsets = offsets;
  S.perm = perm;
  S.n_groups = n_groups;
  S.uniform_rows = 0;
  S.rows_per_token = rows_per_token;
  S.max_rows = max_rows;
  S.d_ff = d_ff;
  S.w_gate = w_gate;
  S.w_up = w_up;
  S.w_down = w_down;
  S.sc_gate = sc_gate;
  S.sc_up = sc_up;
  S.sc_down = sc_down;
  S.h = ws;
  S.out = out;
  int st = launch_grouped(p, 1, stream);
  if (st != MOE_OK) return st;
  return launch_grouped(p, 2, stream);
}

// ------------------------------------------------------------------ backward
// Workspace of moe_backward (byte offsets, 256-aligned). R = N*k rows (the
// kept copies occupy the first offsets[E]), Kmax = R rounded up to 64 plus 64
// per expert (each expert's rows padded to 64 in the transposed layout).
struct BwLayout {
  size_t logits, dl, rpart, dlh, dlT, rterm, dw, kofs, kofs_s, Xg, dYg, dO, G, U, dHp, h, dGU, dXr, dOT, hT, dGT, dUT, XT, split;
  size_t Xs, dYs, Gs, Us, dHs, hs, dGUs, dXs, dOsT, hsT, dGsT, dUsT, XsT, total;
  long long R, Kmax, Npad, KSmax;
};

BwLayout bw_layout(const moe_shape& s) {
  BwLayout L{};
  const long long N = s.n_tokens, k = s.top_k, E = s.n_experts, d = s.d_model, F = s.d_ff;
  const long long S = s.n_shared, Fs = S ? s.d_ff_shared : 0;
  L.R = N * k;
  L.Kmax = (L.R + 63) / 64 * 64 + 64 * E;
  L.Npad = (N + 63) / 64 * 64;
  L.KSmax = S * L.Npad;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += align256(bytes); return o; };
  L.logits = take(route_logits_floats(s) * 4);
  L.dl = take(N * E * 4);
  L.rpart = take(router_wgrad_part_floats((int)N, (int)E, (int)d) * 4);
  L.dlh = take(N * 2 * E * 2);   // dl as bf16 hi | lo parts, and its transpose (router products as GEMMs)
  L.dlT = take(E * 2 * N * 2);
  L.rterm = take(N * d * 4);     // dl W_r
  L.dw = take(N * k * 4);
  L.kofs = take((E + 1) * 4);
  L.kofs_s = take((S + 1) * 4);
  L.Xg = take(L.R * d * 2);
  L.dYg = take(L.R * d * 2);
  L.dO = take(L.R * d * 2);
  L.G = take(L.R * F * 4);
  L.U = take(L.R * F * 4);
  L.dHp = take(L.R * F * 4);
  L.h = take(L.R * F * 2);
  L.dGU = take(L.R * 2 * F * 2);
  L.dXr = take(L.R * d * 4);
  L.dOT = take(d * L.Kmax * 2);
  L.hT = take(F * L.Kmax * 2);
  L.dGT = take(F * L.Kmax * 2);
  L.dUT = take(F * L.Kmax * 2);
  L.XT = take(d * L.Kmax * 2);
  L.split = take(std::max(grouped_split_bytes(L.R, (int)E), grouped_split_bytes(E * std::max(d, F), (int)E)));
  L.Xs = take(S * N * d * 2);
  L.dYs = take(S * N * d * 2);
  L.Gs = take(S * N * Fs * 4);
  L.Us = take(S * N * Fs * 4);
  L.dHs = take(S * N * Fs * 4);
  L.hs = take(S * N * Fs * 2);
  L.dGUs = take(S * N * 2 * Fs * 2);
  L.dXs = take(S * N * d * 4);
  L.dOsT = take(d * L.KSmax * 2);
  L.hsT = take(Fs * L.KSmax * 2);
  L.dGsT = take(Fs * L.KSmax * 2);
  L.dUsT = take(Fs * L.KSmax * 2);
  L.XsT = take(d * L.KSmax * 2);
  L.total = off;
  return L;
}

// One plain grouped product out[r, n] = sum_k A[r, k] B_g[n, k] over groups of rows
// (offsets, or `uniform` rows per group), or, with kofs, the weight-gradient form
// out[g*M + m, n] = sum over group g's K range of A[m, k] B[n, k].
int grouped_gemm(int n_groups, const int32_t* offsets, int uniform, long long max_rows, int K_or_stride, int ncols,
                 const void* A, const void* B, float* out, const int32_t* kofs, float* split_ws, size_t split_bytes,
                 hipStream_t st, int accumulate = 0, int out_bf16 = 0, int skip_empty_k = 0) {
  GroupedParams p{};
  p.n_sets = 1;
  p.x = A;
  p.n_tokens = 1;
  p.d_model = ncols;
  p.dtype = MOE_DTYPE_BF16;
  p.split_ws = split_ws;
  p.split_cap = split_ws ? (long long)(split_bytes / sizeof(float)) : 0;
  SegSet& S = p.set[0];
  S.offsets = offsets;
  S.n_groups = n_groups;
  S.uniform_rows = uniform;
  S.rows_per_token = 1;
  S.max_rows = (int32_t)max_rows;
  S.d_ff = K_or_stride;
  S.w_gate = S.w_up = S.w_down = B;
  S.h = const_cast<void*>(A);
  S.out = out;
  S.k_offsets = kofs;
  S.skip_empty_k = skip_empty_k;
  S.accumulate = accumulate;
  S.out_bf16 = out_bf16;
  return launch_grouped(p, 2, st);
}

// out[r, n] = sum_k A[r, k] B_g[k, n] with the weights in their stored, N-major
// orientation: B_g's rows k < b_split (all K rows when b_split == 0) are rows of
// B_lo + g * b_split * ncols (g * K * ncols), the others rows k - b_split of
// B_hi + g * b_split * ncols.
int grouped_gemm_nmajor(int n_groups, const int32_t* offsets, int uniform, long long max_rows, int K, int ncols,
                        const void* A, const void* B_lo, const void* B_hi, int b_split, float* out, float* split_ws,
                        size_t split_bytes, hipStream_t st, int accumulate = 0) {
  // each 64-row K stage must lie within one of the two matrices
  if (K % 64 || b_split % 64 || b_split < 0 || (b_split > 0 && K - b_split > b_split)) return MOE_ERR_UNSUPPORTED;
  GroupedParams p{};
  p.n_sets = 1;
  p.x = A;
  p.n_tokens = 1;
  p.d_model = ncols;
  p.dtype = MOE_DTYPE_BF16;
  p.split_ws = split_ws;
  p.split_cap = split_ws ? (long long)(split_bytes / sizeof(float)) : 0;
  SegSet& S = p.set[0];
  S.offsets = offsets;
  S.n_groups = n_groups;
  S.uniform_rows = uniform;
  S.rows_per_token = 1;
  S.max_rows = (int32_t)max_rows;
  S.d_ff = K;
  S.w_gate = S.w_down = B_lo;
  S.w_up = B_hi;
  S.h = const_cast<void*>(A);
  S.out = out;
  S.b_nmajor = 1;
  S.b_split = b_split;
  S.accumulate = accumulate;
  return launch_grouped(p, 2, st);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_workspace_bytes(const moe_shape* shape) {
  if (check_shape(shape) != MOE_OK) return 0;
  return std::max<size_t>(layout(*shape).total, 256);  // never 0 for a valid shape
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported size or option";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int moe_route(const moe_shape* shape, const void* x, const void* w_router, const float* logit_bias,
              const float* select_bias, int32_t* topk_idx, float* topk_w, double* prob_sum, void* ws,
              size_t ws_bytes, hipStream_t stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape& s = *shape;
  if (!prob_sum || (s.n_tokens > 0 && (!x || !w_router || !topk_idx || !topk_w || !ws)))
    return MOE_ERR_INVALID_ARG;
  if (ws_bytes < layout(s).hist) return MOE_ERR_WORKSPACE;
  return do_route(s, x, w_router, logit_bias, select_bias, topk_idx, topk_w, prob_sum, ws, stream);
}

int moe_permute(const moe_shape* shape, const int32_t* topk_idx, const double* prob_sum,
                int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* slot_pos,
                double* balance_stat, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape& s = *shape;
  if (!counts || !offsets || (balance_stat && !prob_sum)) return MOE_ERR_INVALID_ARG;
  if (s.n_tokens > 0 && (!topk_idx || !perm || !slot_pos || !ws)) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < layout(s).h_routed) return MOE_ERR_WORKSPACE;
  return do_permute(s, topk_idx, prob_sum, counts, offsets, perm, slot_pos, balance_stat, ws, stream);
}

int moe_grouped_swiglu(const moe_shape* shape, int32_t n_groups, int32_t d_ff, const void* x,
                       const int32_t* perm, int32_t rows_per_token, const int32_t* offsets,
                       int32_t max_rows, const void* w_gate, const void* w_up, const void* w_down,
                       float* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  return grouped_impl(shape, n_groups, d_ff, x, perm, rows_per_token, offsets, max_rows, w_gate, w_up,
                      w_down, 0, nullptr, nullptr, nullptr, out, ws, ws_bytes, stream);
}

int moe_grouped_swiglu_fp8(const moe_shape* shape, int32_t n_groups, int32_t d_ff, const void* x,
                           const int32_t* perm, int32_t rows_per_token, const int32_t* offsets,
                           int32_t max_rows, const uint8_t* w_gate, const uint8_t* w_up,
                           const uint8_t* w_down, const float* sc_gate, const float* sc_up,
                           const float* sc_down, float* out, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  if (!shape) return MOE_ERR_INVALID_ARG;
  if (!sc_gate || !sc_up || !sc_down) return MOE_ERR_INVALID_ARG;
  if (shape->dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
  return grouped_impl(shape, n_groups, d_ff, x, perm, rows_per_token, offsets, max_rows, w_gate, w_up,
                      w_down, 8, sc_gate, sc_up, sc_down, out, ws, ws_bytes, stream);
}

int moe_grouped_swiglu_int4(const moe_shape* shape, int32_t n_groups, int32_t d_ff, const void* x,
                            const int32_t* perm, int32_t rows_per_token, const int32_t* offsets,
                            int32_t max_rows, const uint8_t* w_gate, const uint8_t* w_up,
                            const uint8_t* w_down, const float* sc_gate, const float* sc_up,
                            const float* sc_down, float* out, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  if (!shape) return MOE_ERR_INVALID_ARG;
  if (!sc_gate || !sc_up || !sc_down) return MOE_ERR_INVALID_ARG;
  if (shape->dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
  return grouped_impl(shape, n_groups, d_ff, x, perm, rows_per_token, offsets, max_rows, w_gate, w_up,
                      w_down, 4, sc_gate, sc_up, sc_down, out, ws, ws_bytes, stream);
}

int moe_quantize_int4(int64_t rows, int32_t cols, const void* w_bf16, uint8_t* packed, float* scales,
                      hipStream_t stream) {
  if (rows < 0 || cols <= 0) return MOE_ERR_INVALID_ARG;
  if (rows > 0 && (!w_bf16 || !packed || !scales)) return MOE_ERR_INVALID_ARG;
  if (cols % 64 || rows >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  return launch_quantize_int4(rows, cols, w_bf16, packed, scales, stream);
}

int moe_quantize_fp8(int64_t rows, int32_t cols, const void* w_bf16, uint8_t* codes, float* scales,
                     hipStream_t stream) {
  if (rows < 0 || cols <= 0) return MOE_ERR_INVALID_ARG;
  if (rows > 0 && (!w_bf16 || !codes || !scales)) return MOE_ERR_INVALID_ARG;
  if (cols % 64 || rows >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  return launch_quantize_fp8(rows, cols, w_bf16, codes, scales, stream);
}

int moe_dequantize_fp8(int64_t rows, int32_t cols, const uint8_t* codes, const float* scales, float* out,
                       hipStream_t stream) {
  if (rows < 0 || cols <= 0) return MOE_ERR_INVALID_ARG;
  if (rows > 0 && (!codes || !scales || !out)) return MOE_ERR_INVALID_ARG;
  if (cols % 8) return MOE_ERR_UNSUPPORTED;
  return launch_dequantize_fp8(rows, cols, codes, scales, out, stream);
}

int moe_combine(const moe_shape* shape, const float* expert_out, const int32_t* slot_pos,
                const float* topk_w, const float* shared_out, float* y, hipStream_t stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape& s = *shape;
  if (s.n_tokens > 0 && (!expert_out || !slot_pos || !topk_w || !y)) return MOE_ERR_INVALID_ARG;
  if (s.n_shared > 0 && s.n_tokens > 0 && !shared_out) return MOE_ERR_INVALID_ARG;
  return launch_combine(s, expert_out, slot_pos, topk_w, s.n_shared > 0 ? shared_out : nullptr, y,
                        stream);
}

static int forward_impl(const moe_shape* shape, const void* x, const void* w_router,
                        const float* logit_bias, const float* select_bias, const void* w_gate,
                        const void* w_up, const void* w_down, const void* s_gate, const void* s_up,
                        const void* s_down, int wq, const moe_weight_scales* sc, float* y, int32_t* topk_idx,
                        float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                        int32_t* slot_pos, double* prob_sum, double* balance_stat, void* ws,
                        size_t ws_bytes, hipEvent_t* stage_events, hipStream_t stream,
                        float* gu_save = nullptr) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape& s = *shape;
  if (!counts || !offsets || !prob_sum || !balance_stat || !w_gate || !w_up || !w_down)
    return MOE_ERR_INVALID_ARG;
  if (s.n_tokens > 0 && (!x || !w_router || !y || !topk_idx || !topk_w || !perm || !slot_pos || !ws))
    return MOE_ERR_INVALID_ARG;
  if (s.n_shared > 0 && (!s_gate || !s_up || !s_down)) return MOE_ERR_INVALID_ARG;
  const Layout L = layout(s);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;

  auto mark = [&](int i) {
    if (stage_events && stage_events[i]) hipEventRecord(stage_events[i], stream);
  };
  mark(0);
  // The router's last step (adding its per-workgroup probability sums) rides in
  // the permutation's column scan when that kernel runs (more than one chunk).
  int pnb = 0;
  if ((st = do_route(s, x, w_router, logit_bias, select_bias, topk_idx, topk_w, prob_sum, ws, stream, &pnb)))
    return st;
  const bool fold_in_scan = pnb > 0 && permute_chunks(s) > 1;
  if (pnb > 0 && !fold_in_scan &&
      (st = launch_prob_sum(reinterpret_cast<const double*>(at(ws, L.partials)), pnb, s.n_experts, prob_sum,
                            stream)))
    return st;
  mark(1);
  if ((st = do_permute(s, topk_idx, prob_sum, counts, offsets, perm, slot_pos, balance_stat, ws, stream,
                       fold_in_scan ? pnb : 0, prob_sum)))
    return st;
  mark(2);
  const size_t NK = (size_t)s.n_tokens * s.top_k;
  float* O = reinterpret_cast<float*>(at(ws, L.o));
  float* O_shared = O + NK * s.d_model;
  GroupedParams p{};
  if (s.n_tokens > 0) {
    p.x = x;
    p.n_tokens = s.n_tokens;
    p.d_model = s.d_model;
    p.dtype = s.dtype;
    p.n_sets = s.n_shared > 0 ? 2 : 1;
    if (s.dtype == MOE_DTYPE_BF16 && L.h_routed > L.split) {
      p.split_ws = reinterpret_cast<float*>(at(ws, L.split));
      p.split_cap = (long long)((L.h_routed - L.split) / sizeof(float));
    }
    SegSet& R = p.set[0];
    R.offsets = offsets;
    R.perm = perm;
    R.n_groups = s.n_experts;
    R.rows_per_token = s.top_k;
    R.max_rows = (int32_t)NK;
    // a token takes k distinct experts, so no expert gets more than N rows (C with a capacity)
    R.group_rows_max = s.capacity > 0 ? std::min(s.capacity, s.n_tokens) : s.n_tokens;
    R.d_ff = s.d_ff;
    R.w_gate = w_gate;
    R.w_up = w_up;
    R.w_down = w_down;
    if (sc) {
      p.wq = wq;
      R.sc_gate = sc->gate;
      R.sc_up = sc->up;
      R.sc_down = sc->down;
    }
    R.h = at(ws, L.h_routed);
    R.out = O;
    if (gu_save) {  // [NK, F] gate, [NK, F] up, then the shared experts' [S N, Fs] each
      R.g_save = gu_save;
      R.u_save = gu_save + NK * s.d_ff;
    }
    if (s.n_shared > 0) {
      SegSet& Sh = p.set[1];
      Sh.offsets = nullptr;
      Sh.perm = nullptr;
      Sh.n_groups = s.n_shared;
      Sh.uniform_rows = s.n_tokens;
      Sh.rows_per_token = 1;
      Sh.max_rows = s.n_shared * s.n_tokens;
      Sh.d_ff = s.d_ff_shared;
      Sh.w_gate = s_gate;
      Sh.w_up = s_up;
      Sh.w_down = s_down;
      if (sc) {
        Sh.sc_gate = sc->s_gate;
        Sh.sc_up = sc->s_up;
        Sh.sc_down = sc->s_down;
      }
      Sh.h = at(ws, L.h_shared);
      Sh.out = O_shared;
      if (gu_save) {
        const size_t SN = (size_t)s.n_shared * s.n_tokens;
        Sh.g_save = gu_save + 2 * NK * s.d_ff;
        Sh.u_save = Sh.g_save + SN * s.d_ff_shared;
      }
    }
    if ((st = launch_grouped(p, 1, stream))) return st;
  }
  mark(3);
  if (s.n_tokens > 0 && (st = launch_grouped(p, 2, stream))) return st;
  mark(4);
  if ((st = launch_combine(s, O, slot_pos, topk_w, s.n_shared > 0 ? O_shared : nullptr, y, stream)))
    return st;
  mark(5);
  return MOE_OK;
}

int moe_forward(const moe_shape* shape, const void* x, const void* w_router, const float* logit_bias,
                const float* select_bias, const void* w_gate, const void* w_up, const void* w_down,
                const void* s_gate, const void* s_up, const void* s_down, float* y,
                int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                int32_t* slot_pos, double* prob_sum, double* balance_stat, void* ws,
                size_t ws_bytes, hipEvent_t* stage_events, hipStream_t stream) {
  return forward_impl(shape, x, w_router, logit_bias, select_bias, w_gate, w_up, w_down, s_gate, s_up,
                      s_down, 0, nullptr, y, topk_idx, topk_w, counts, offsets, perm, slot_pos, prob_sum,
                      balance_stat, ws, ws_bytes, stage_events, stream);
}

size_t moe_train_save_floats(const moe_shape* shape) {
  if (check_shape(shape) != MOE_OK) return 0;
  const moe_shape& s = *shape;
  return 2 * ((size_t)s.n_tokens * s.top_k * s.d_ff + (size_t)s.n_shared * s.n_tokens * (s.n_shared ? s.d_ff_shared : 0));
}

int moe_forward_train(const moe_shape* shape, const void* x, const void* w_router, const float* logit_bias,
                      const float* select_bias, const void* w_gate, const void* w_up, const void* w_down,
                      const void* s_gate, const void* s_up, const void* s_down, float* y,
                      int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                      int32_t* slot_pos, double* prob_sum, double* balance_stat, float* gu_save, void* ws,
                      size_t ws_bytes, hipEvent_t* stage_events, hipStream_t stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (shape->dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
  if (shape->n_tokens > 0 && !gu_save) return MOE_ERR_INVALID_ARG;
  return forward_impl(shape, x, w_router, logit_bias, select_bias, w_gate, w_up, w_down, s_gate, s_up,
                      s_down, 0, nullptr, y, topk_idx, topk_w, counts, offsets, perm, slot_pos, prob_sum,
                      balance_stat, ws, ws_bytes, stage_events, stream, shape->n_tokens > 0 ? gu_save : nullptr);
}

static int forward_quantised(int wq, const moe_shape* shape, const void* x, const void* w_router,
                             const float* logit_bias, const float* select_bias, const uint8_t* w_gate,
                             const uint8_t* w_up, const uint8_t* w_down, const uint8_t* s_gate,
                             const uint8_t* s_up, const uint8_t* s_down, const moe_weight_scales* scales,
                             float* y, int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                             int32_t* perm, int32_t* slot_pos, double* prob_sum, double* balance_stat,
                             void* ws, size_t ws_bytes, hipEvent_t* stage_events, hipStream_t stream) {
  if (!shape || !scales) return MOE_ERR_INVALID_ARG;
  if (!scales->gate || !scales->up || !scales->down) return MOE_ERR_INVALID_ARG;
  if (shape->n_shared > 0 && (!scales->s_gate || !scales->s_up || !scales->s_down)) return MOE_ERR_INVALID_ARG;
  if (shape->dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
  return forward_impl(shape, x, w_router, logit_bias, select_bias, w_gate, w_up, w_down, s_gate, s_up,
                      s_down, wq, scales, y, topk_idx, topk_w, counts, offsets, perm, slot_pos, prob_sum,
                      balance_stat, ws, ws_bytes, stage_events, stream);
}

int moe_forward_fp8(const moe_shape* shape, const void* x, const void* w_router,
                    const float* logit_bias, const float* select_bias, const uint8_t* w_gate,
                    const uint8_t* w_up, const uint8_t* w_down, const uint8_t* s_gate,
                    const uint8_t* s_up, const uint8_t* s_down, const moe_fp8_scales* scales,
                    float* y, int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                    int32_t* perm, int32_t* slot_pos, double* prob_sum, double* balance_stat,
                    void* ws, size_t ws_bytes, hipEvent_t* stage_events, hipStream_t stream) {
  return forward_quantised(8, shape, x, w_router, logit_bias, select_bias, w_gate, w_up, w_down, s_gate, s_up,
                           s_down, scales, y, topk_idx, topk_w, counts, offsets, perm, slot_pos, prob_sum,
                           balance_stat, ws, ws_bytes, stage_events, stream);
}

int moe_forward_int4(const moe_shape* shape, const void* x, const void* w_router,
                     const float* logit_bias, const float* select_bias, const uint8_t* w_gate,
                     const uint8_t* w_up, const uint8_t* w_down, const uint8_t* s_gate,
                     const uint8_t* s_up, const uint8_t* s_down, const moe_weight_scales* scales,
                     float* y, int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                     int32_t* perm, int32_t* slot_pos, double* prob_sum, double* balance_stat,
                     void* ws, size_t ws_bytes, hipEvent_t* stage_events, hipStream_t stream) {
  return forward_quantised(4, shape, x, w_router, logit_bias, select_bias, w_gate, w_up, w_down, s_gate, s_up,
                           s_down, scales, y, topk_idx, topk_w, counts, offsets, perm, slot_pos, prob_sum,
                           balance_stat, ws, ws_bytes, stage_events, stream);
}

int moe_router_aux(const moe_shape* shape, const void* x, const void* w_router, const float* logit_bias,
                   const int32_t* topk_idx, const float* topk_w, double* z_loss, double* importance,
                   double* importance_cv2, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape& s = *shape;
  if (!z_loss && !importance && !importance_cv2) return MOE_ERR_INVALID_ARG;
  if (!ws) return MOE_ERR_INVALID_ARG;
  const Layout L = layout(s);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (s.n_tokens > 0) {
    if (z_loss && (!x || !w_router)) return MOE_ERR_INVALID_ARG;
    if ((importance || importance_cv2) && (!topk_idx || !topk_w)) return MOE_ERR_INVALID_ARG;
  }
  if (s.n_tokens == 0) {  // no tokens: every statistic is 0
    if (z_loss && (st = zero_f64(z_loss, 1, stream))) return st;
    if (importance && (st = zero_f64(importance, s.n_experts, stream))) return st;
    if (importance_cv2 && (st = zero_f64(importance_cv2, 1, stream))) return st;
    return MOE_OK;
  }
  double* imp = importance ? importance : (importance_cv2 ? reinterpret_cast<double*>(at(ws, L.aux)) : nullptr);
  return launch_router_aux(s, x, w_router, logit_bias, topk_idx, topk_w, z_loss, imp, importance_cv2,
                           reinterpret_cast<double*>(at(ws, L.partials)),
                           reinterpret_cast<float*>(at(ws, L.logits)), reinterpret_cast<float*>(at(ws, L.split)),
                           L.h_routed - L.split, stream);
}

int moe_update_select_bias(const moe_shape* shape, const int32_t* counts, float gamma, float* select_bias,
                           hipStream_t stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!counts || !select_bias || !(gamma >= 0.0f) || gamma == INFINITY) return MOE_ERR_INVALID_ARG;
  return launch_bias_update(*shape, counts, gamma, select_bias, stream);
}

size_t moe_backward_workspace_bytes(const moe_shape* shape) {
  if (check_shape(shape) != MOE_OK) return 0;
  return std::max<size_t>(bw_layout(*shape).total, 256);
}

int moe_backward(const moe_shape* shape, const void* x, const void* w_router, const float* logit_bias,
                 const void* w_gate, const void* w_up, const void* w_down, const void* s_gate, const void* s_up,
                 const void* s_down, const int32_t* topk_idx, const float* topk_w, const int32_t* counts,
                 const int32_t* offsets, const int32_t* perm, const int32_t* slot_pos, const float* dy,
                 const float* gu_saved, double aux_coef, int32_t grad_mode, float* dx, float* dw_router,
                 float* d_logit_bias, void* dw_gate_, void* dw_up_, void* dw_down_, void* ds_gate_, void* ds_up_,
                 void* ds_down_, void* ws, size_t ws_bytes, hipStream_t stream) {
  // expert weight gradients: fp32, or bf16 under MOE_GRAD_WRITE_BF16 (the GEMM's out pointer either way)
  float* dw_gate = static_cast<float*>(dw_gate_);
  float* dw_up = static_cast<float*>(dw_up_);
  float* dw_down = static_cast<float*>(dw_down_);
  float* ds_gate = static_cast<float*>(ds_gate_);
  float* ds_up = static_cast<float*>(ds_up_);
  float* ds_down = static_cast<float*>(ds_down_);
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape& s = *shape;
  if (s.dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
  if (!std::isfinite(aux_coef) || grad_mode < MOE_GRAD_WRITE || grad_mode > MOE_GRAD_WRITE_BF16)
    return MOE_ERR_INVALID_ARG;
  const int accumulate = grad_mode == MOE_GRAD_ACCUMULATE;
  const int wbf16 = grad_mode == MOE_GRAD_WRITE_BF16;  // expert weight gradients stored as bf16
  if (!dw_router || !dw_gate || !dw_up || !dw_down || !w_gate || !w_up || !w_down || !w_router || !ws)
    return MOE_ERR_INVALID_ARG;
  if (s.n_shared > 0 && (!s_gate || !s_up || !s_down || !ds_gate || !ds_up || !ds_down)) return MOE_ERR_INVALID_ARG;
  if (s.n_tokens > 0 && (!x || !topk_idx || !topk_w || !counts || !offsets || !perm || !slot_pos || !dy || !dx))
    return MOE_ERR_INVALID_ARG;
  const BwLayout L = bw_layout(s);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  const int N = s.n_tokens, k = s.top_k, E = s.n_experts, d = s.d_model, F = s.d_ff;
  const int S = s.n_shared, Fs = S ? s.d_ff_shared : 0;
  if (N == 0) {  // no tokens: every gradient is 0 (nothing to add when accumulating)
    if (accumulate) return MOE_OK;
    // zero bytes (+0 in fp32 and in bf16): expert weight gradients take 2 bytes each in bf16 mode
    const size_t wb = wbf16 ? 2 : 4;
    for (auto pr : {std::make_pair(dw_router, (size_t)E * d * 4), std::make_pair(dw_gate, (size_t)E * F * d * wb),
                    std::make_pair(dw_up, (size_t)E * F * d * wb), std::make_pair(dw_down, (size_t)E * d * F * wb),
                    std::make_pair(d_logit_bias, (size_t)E * 4), std::make_pair(ds_gate, (size_t)S * Fs * d * wb),
                    std::make_pair(ds_up, (size_t)S * Fs * d * wb), std::make_pair(ds_down, (size_t)S * d * Fs * wb)})
      if (pr.first && (st = launch_fill_f32(pr.first, pr.second / 4, 0.f, stream))) return st;
    return MOE_OK;
  }
  auto P = [&](size_t o) { return static_cast<void*>(at(ws, o)); };
  auto Pf = [&](size_t o) { return reinterpret_cast<float*>(at(ws, o)); };
  auto Pi = [&](size_t o) { return reinterpret_cast<int32_t*>(at(ws, o)); };
  float* split = Pf(L.split);
  const size_t split_bytes = L.Xs - L.split;
  const int R = (int)L.R, Kmax = (int)L.Kmax;
  const int32_t* n_kept = offsets + E;
#define MOE_TRY(call) \
  if ((st = (call)) != MOE_OK) return st
  // ---- routed experts
  MOE_TRY(launch_fill_f32(Pf(L.dw), (size_t)N * k, 0.f, stream));  // dropped copies keep 0
  MOE_TRY(launch_gather_rows(x, dy, topk_w, perm, n_kept, k, d, R, P(L.Xg), P(L.dYg), P(L.dO), stream));
  // G and U: kept by the training forward, or recomputed
  const float* G = gu_saved ? gu_saved : Pf(L.G);
  const float* U = gu_saved ? gu_saved + (size_t)R * F : Pf(L.U);
  if (!gu_saved) {
    MOE_TRY(grouped_gemm(E, offsets, 0, R, d, F, P(L.Xg), w_gate, Pf(L.G), nullptr, split, split_bytes, stream));
    MOE_TRY(grouped_gemm(E, offsets, 0, R, d, F, P(L.Xg), w_up, Pf(L.U), nullptr, split, split_bytes, stream));
  }
  // dH' = dy Wd: w_down [E, d, F] is read as d rows of F values
  MOE_TRY(grouped_gemm_nmajor(E, offsets, 0, R, d, F, P(L.dYg), w_down, nullptr, 0, Pf(L.dHp), split, split_bytes,
                              stream));
  MOE_TRY(launch_swiglu_backward(G, U, Pf(L.dHp), topk_w, perm, n_kept, R, F, P(L.h), P(L.dGU),
                                 Pf(L.dw), stream));
  // dX = [dG | dU] [Wg ; Wu]: rows k < F of the operand are w_gate's, the rest w_up's
  MOE_TRY(grouped_gemm_nmajor(E, offsets, 0, R, 2 * F, d, P(L.dGU), w_gate, w_up, F, Pf(L.dXr), split, split_bytes,
                              stream));
  MOE_TRY(launch_k_offsets(offsets, E, 0, Pi(L.kofs), stream));
  MOE_TRY(launch_transpose_padded(P(L.dO), d, 0, d, offsets, 0, 0, Pi(L.kofs), E, P(L.dOT), Kmax, stream));
  MOE_TRY(launch_transpose_padded(P(L.h), F, 0, F, offsets, 0, 0, Pi(L.kofs), E, P(L.hT), Kmax, stream));
  MOE_TRY(launch_transpose_padded(P(L.dGU), 2 * F, 0, F, offsets, 0, 0, Pi(L.kofs), E, P(L.dGT), Kmax, stream));
  MOE_TRY(launch_transpose_padded(P(L.dGU), 2 * F, F, F, offsets, 0, 0, Pi(L.kofs), E, P(L.dUT), Kmax, stream));
  MOE_TRY(launch_transpose_padded(P(L.Xg), d, 0, d, offsets, 0, 0, Pi(L.kofs), E, P(L.XT), Kmax, stream));
  // experts with no kept copy get no GEMM tiles: their gradient blocks are zeroed by a fill
  // (or, when accumulating, left as they are)
  if (!accumulate) {
    const size_t blk = (size_t)d * F * (wbf16 ? 2 : 4);
    MOE_TRY(launch_zero_empty_groups(dw_down, Pi(L.kofs), E, blk, stream));
    MOE_TRY(launch_zero_empty_groups(dw_gate, Pi(L.kofs), E, blk, stream));
    MOE_TRY(launch_zero_empty_groups(dw_up, Pi(L.kofs), E, blk, stream));
  }
  MOE_TRY(grouped_gemm(E, nullptr, d, (long long)E * d, Kmax, F, P(L.dOT), P(L.hT), dw_down, Pi(L.kofs), split,
                       split_bytes, stream, accumulate, wbf16, 1));
  MOE_TRY(grouped_gemm(E, nullptr, F, (long long)E * F, Kmax, d, P(L.dGT), P(L.XT), dw_gate, Pi(L.kofs), split,
                       split_bytes, stream, accumulate, wbf16, 1));
  MOE_TRY(grouped_gemm(E, nullptr, F, (long long)E * F, Kmax, d, P(L.dUT), P(L.XT), dw_up, Pi(L.kofs), split,
                       split_bytes, stream, accumulate, wbf16, 1));
  // ---- shared experts: every token, weight 1
  if (S > 0) {
    const int RS = S * N, KS = (int)L.KSmax;
    for (int q = 0; q < S; ++q)
      MOE_TRY(launch_gather_rows(x, dy, nullptr, nullptr, nullptr, 1, d, N,
                                 static_cast<uint8_t*>(P(L.Xs)) + (size_t)q * N * d * 2,
                                 static_cast<uint8_t*>(P(L.dYs)) + (size_t)q * N * d * 2, nullptr, stream));
    const float* Gs = gu_saved ? gu_saved + 2 * (size_t)R * F : Pf(L.Gs);
    const float* Us = gu_saved ? Gs + (size_t)RS * Fs : Pf(L.Us);
    if (!gu_saved) {
      MOE_TRY(grouped_gemm(S, nullptr, N, RS, d, Fs, P(L.Xs), s_gate, Pf(L.Gs), nullptr, split, split_bytes,
                           stream));
      MOE_TRY(grouped_gemm(S, nullptr, N, RS, d, Fs, P(L.Xs), s_up, Pf(L.Us), nullptr, split, split_bytes, stream));
    }
    MOE_TRY(grouped_gemm_nmajor(S, nullptr, N, RS, d, Fs, P(L.dYs), s_down, nullptr, 0, Pf(L.dHs), split,
                                split_bytes, stream));
    MOE_TRY(launch_swiglu_backward(Gs, Us, Pf(L.dHs), nullptr, nullptr, nullptr, RS, Fs, P(L.hs),
                                   P(L.dGUs), nullptr, stream));
    MOE_TRY(grouped_gemm_nmajor(S, nullptr, N, RS, 2 * Fs, d, P(L.dGUs), s_gate, s_up, Fs, Pf(L.dXs), split,
                                split_bytes, stream));
    MOE_TRY(launch_k_offsets(nullptr, S, N, Pi(L.kofs_s), stream));
    MOE_TRY(launch_transpose_padded(P(L.dYs), d, 0, d, nullptr, N, 0, Pi(L.kofs_s), S, P(L.dOsT), KS, stream));
    MOE_TRY(launch_transpose_padded(P(L.hs), Fs, 0, Fs, nullptr, N, 0, Pi(L.kofs_s), S, P(L.hsT), KS, stream));
    MOE_TRY(launch_transpose_padded(P(L.dGUs), 2 * Fs, 0, Fs, nullptr, N, 0, Pi(L.kofs_s), S, P(L.dGsT), KS, stream));
    MOE_TRY(launch_transpose_padded(P(L.dGUs), 2 * Fs, Fs, Fs, nullptr, N, 0, Pi(L.kofs_s), S, P(L.dUsT), KS, stream));
    MOE_TRY(launch_transpose_padded(P(L.Xs), d, 0, d, nullptr, N, 0, Pi(L.kofs_s), S, P(L.XsT), KS, stream));
    MOE_TRY(grouped_gemm(S, nullptr, d, (long long)S * d, KS, Fs, P(L.dOsT), P(L.hsT), ds_down, Pi(L.kofs_s), split,
                         split_bytes, stream, accumulate, wbf16));
    MOE_TRY(grouped_gemm(S, nullptr, Fs, (long long)S * Fs, KS, d, P(L.dGsT), P(L.XsT), ds_gate, Pi(L.kofs_s), split,
                         split_bytes, stream, accumulate, wbf16));
    MOE_TRY(grouped_gemm(S, nullptr, Fs, (long long)S * Fs, KS, d, P(L.dUsT), P(L.XsT), ds_up, Pi(L.kofs_s), split,
                         split_bytes, stream, accumulate, wbf16));
  }
  // ---- router and dx
  int splits = 1;
  MOE_TRY(launch_router_logits(s, x, w_router, Pf(L.logits), &splits, split, split_bytes, stream));
  MOE_TRY(launch_router_backward(s, Pf(L.logits), splits, logit_bias, topk_idx, topk_w, Pf(L.dw), counts, aux_coef,
                                 Pf(L.dl), stream));
  // dW_r = dl^T x and the router term dl W_r of dx: with dl split into bf16 hi + lo parts
  // (2^-16 relative), both are bf16 GEMMs reading W_r and x in their stored orientation
  // (K = 2E and 2N, rows from the same matrix twice: each half a whole number of 64-row K stages)
  float* rterm = nullptr;
  if (E % 64 == 0 && N % 64 == 0) {
    MOE_TRY(launch_split_hilo(Pf(L.dl), N, E, P(L.dlh), P(L.dlT), stream));
    rterm = Pf(L.rterm);
    MOE_TRY(grouped_gemm_nmajor(1, nullptr, N, N, 2 * E, d, P(L.dlh), w_router, w_router, E, rterm, split,
                                split_bytes, stream));
    MOE_TRY(grouped_gemm_nmajor(1, nullptr, E, E, 2 * N, d, P(L.dlT), x, x, N, dw_router, split, split_bytes,
                                stream, accumulate));
    MOE_TRY(launch_logit_bias_grad(Pf(L.dl), N, E, d_logit_bias, accumulate, stream));
  } else {
    MOE_TRY(launch_router_wgrad(Pf(L.dl), x, N, E, d, Pf(L.rpart), dw_router, d_logit_bias, accumulate, stream));
  }
  MOE_TRY(launch_dx(Pf(L.dXr), slot_pos, S > 0 ? Pf(L.dXs) : nullptr, S, Pf(L.dl), w_router, rterm, N, E, k, d, dx,
                    stream));
#undef MOE_TRY
  return MOE_OK;
}


// ---------------------------------------------------------------------
// moe_forward without a workspace argument: the workspace is a static device
// array of this file, one per device, held until the process ends.

// The scratch array. Its host-side name only stands in for the symbol:
// kernels and copies use the device address that hipGetSymbolAddress returns
// for the current device (scratch_address below), never the name.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up

// Device address of `scratch` on the current device, looked up on the first
// call on that device (with that device current) and kept.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace

int moe_forward_noalloc(const moe_shape* shape, const void* x, const void* w_router, const float* logit_bias,
                        const float* select_bias, const void* w_gate, const void* w_up, const void* w_down,
                        const void* s_gate, const void* s_up, const void* s_down, float* y,
                        int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                        int32_t* slot_pos, double* prob_sum, double* balance_stat, hipEvent_t* stage_events,
                        hipStream_t stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  // the same workspace layout as moe_forward, so the kernels and their results are the same
  const size_t need = layout(*shape).total;
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if ((st = scratch_address(&ws))) return st;
  return forward_impl(shape, x, w_router, logit_bias, select_bias, w_gate, w_up, w_down, s_gate, s_up,
                      s_down, 0, nullptr, y, topk_idx, topk_w, counts, offsets, perm, slot_pos, prob_sum,
                      balance_stat, ws, need, stage_events, stream);
}

}  // extern "C"
