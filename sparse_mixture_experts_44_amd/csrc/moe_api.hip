// C ABI of libmoe.so (declared in include/moe.h): argument validation,
// workspace layout and launch order. Nothing here allocates, synchronises
// or keeps state between calls.
#include <math.h>

#include <algorithm>

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
  off += align256((size_t)route_blocks(s) * E * sizeof(double));
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

int do_route(const moe_shape& s, const void* x, const void* w_router, const float* lb, const float* sb,
             int32_t* idx, float* tw, double* prob_sum, void* ws, hipStream_t st) {
  if (s.n_tokens == 0) return zero_f64(prob_sum, s.n_experts, st);
  const Layout L = layout(s);
  return launch_route(s, x, w_router, lb, sb, idx, tw, prob_sum,
                      reinterpret_cast<double*>(at(ws, L.partials)),
                      reinterpret_cast<float*>(at(ws, L.logits)), st);
}

int do_permute(const moe_shape& s, const int32_t* idx, const double* prob_sum, int32_t* counts,
               int32_t* offsets, int32_t* perm, int32_t* slot_pos, double* stat, void* ws,
               hipStream_t st) {
  const Layout L = layout(s);
  return launch_permute(s, idx, prob_sum, counts, offsets, perm, slot_pos, stat,
                        reinterpret_cast<int32_t*>(at(ws, L.hist)),
                        reinterpret_cast<int32_t*>(at(ws, L.base)), st);
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
                        size_t ws_bytes, hipEvent_t* stage_events, hipStream_t stream) {
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
  if ((st = do_route(s, x, w_router, logit_bias, select_bias, topk_idx, topk_w, prob_sum, ws, stream)))
    return st;
  mark(1);
  if ((st = do_permute(s, topk_idx, prob_sum, counts, offsets, perm, slot_pos, balance_stat, ws,
                       stream)))
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
                           reinterpret_cast<float*>(at(ws, L.logits)), stream);
}

int moe_update_select_bias(const moe_shape* shape, const int32_t* counts, float gamma, float* select_bias,
                           hipStream_t stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!counts || !select_bias || !(gamma >= 0.0f) || gamma == INFINITY) return MOE_ERR_INVALID_ARG;
  return launch_bias_update(*shape, counts, gamma, select_bias, stream);
}

}  // extern "C"
