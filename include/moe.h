/*
 * moe.h - C ABI of libmoe.so: the forward pass of a top-k routed
 * Mixture-of-Experts layer on one AMD MI355X (gfx950).
 *
 * The layer is the MoE module of "混合专家 MoE" (anrans ai-infra
 * handbook), section "实现：逐 token 与按专家分组". It is
 * MoE(d, d_ff, n_experts, top_k, n_shared), built from:
 *   route(x)              -> (weights, idx, probs)
 *   forward_grouped(x)    -> y
 *   aux_loss(probs, idx)  -> the balance statistic (section "负载均衡")
 * It has two options from the other pages:
 *   - an additive router bias: MoEGating's nn.Linear(input_dim,
 *     num_experts) on the cloud.baidu.com overview;
 *   - a per-expert capacity: the notes "混合专家模型 (MoE)：大规模稀疏条件计算的
 *     架构与工程实践", section 三.1.
 *
 * Conventions, for every entry point:
 *   - Every pointer is a DEVICE pointer, except `shape` (host) and
 *     `stage_events` (a host array of event handles).
 *   - Tensors are dense and row-major, with exactly the shapes given. Data
 *     pointers are 16-byte aligned. Inputs are read-only.
 *   - The caller owns every buffer, including the workspace. The library
 *     allocates nothing, keeps no state between calls, and never
 *     synchronises the host. Work is queued on `stream`; outputs are valid
 *     once the stream reaches the end of the call. Two calls may run at the
 *     same time if their output and workspace buffers do not overlap.
 *   - Every argument is validated before anything is launched. On an error
 *     nothing is queued and a negative moe_status is returned. A launch
 *     failure reported by the runtime returns MOE_ERR_HIP; earlier work of
 *     the same call may already be queued.
 *   - Supported sizes:
 *       d_model and every d_ff a multiple of 64;
 *       1 <= top_k <= min(n_experts, 32);
 *       n_experts <= 512; n_shared <= 16; grouped_swiglu n_groups <= 528;
 *       n_tokens * top_k < 2^31;
 *       n_tokens * d_model < 2^31 and n_tokens * (top_k + n_shared) *
 *       max(d_model, d_ff, d_ff_shared) < 2^31 (grouped_swiglu: max_rows *
 *       max(d_model, d_ff) < 2^31), because the kernels address rows of x,
 *       h and the expert outputs with 32-bit element offsets.
 *     Other sizes return MOE_ERR_UNSUPPORTED.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null required pointer, bad dimension, k outside [1, E] */
  MOE_ERR_UNSUPPORTED = -2, /* valid, but outside the sizes the kernels handle */
  MOE_ERR_WORKSPACE = -3,   /* ws_bytes smaller than required */
  MOE_ERR_HIP = -4          /* the runtime reported a launch error */
} moe_status;

typedef enum {
  MOE_DTYPE_F32 = 0,  /* x and all weights fp32; h stays fp32 */
  MOE_DTYPE_BF16 = 1  /* x and all weights bf16; fp32 accumulation; h rounded to bf16 */
} moe_dtype;

/* The layer's sizes and options. Tensor shapes below use these names:
 * N = n_tokens, d = d_model, F = d_ff, E = n_experts, k = top_k,
 * S = n_shared, Fs = d_ff_shared. */
typedef struct {
  int32_t n_tokens;
  int32_t d_model;
  int32_t d_ff;
  int32_t n_experts;
  int32_t top_k;
  int32_t n_shared;     /* always-on shared experts (0 = none) */
  int32_t d_ff_shared;  /* their hidden size (ignored when n_shared == 0) */
  int32_t capacity;     /* rows per expert buffer C; <= 0 means unlimited */
  int32_t renormalize;  /* 1: w = p / sum of the k selected p; 0: w = p */
  int32_t dtype;        /* moe_dtype */
} moe_shape;

/* Number of hipEvent_t handles moe_forward records when given stage_events. */
#define MOE_STAGE_EVENTS 6

/* Workspace bytes that suffice for every entry point called with this shape
 * (route, permute, grouped_swiglu with max_rows <= N*k + S*N, forward).
 * At least 256 for a valid shape (also when N = 0); 0 for an invalid shape. */
size_t moe_workspace_bytes(const moe_shape* shape);

/* Static text for a status code; never NULL. */
const char* moe_status_string(int status);

/* Router: linear d -> E, softmax, selection-only bias, top-k, renormalise.
 * ("实现" section: route; "负载均衡" section: the bias for selection only.)
 *   x           [N, d]  (dtype)
 *   w_router    [E, d]  (dtype); logits l = x W_r^T
 *   logit_bias  [E] fp32 or NULL: added to the logits before the softmax
 *   select_bias [E] fp32 or NULL: s = p + select_bias chooses the top-k;
 *               the weights always come from the unbiased p
 *   topk_idx    [N, k] int32 out: the k largest s, best first; an equal
 *               score ranks the lower expert index first
 *   topk_w      [N, k] fp32 out: p at topk_idx, divided by their sum if
 *               renormalize
 *   prob_sum    [E] fp64 out: sum over tokens of p[t, e], summed in a fixed
 *               order, so it is reproducible bit for bit
 *   ws          >= moe_workspace_bytes(shape) bytes */
int moe_route(const moe_shape* shape, const void* x, const void* w_router,
              const float* logit_bias, const float* select_bias,
              int32_t* topk_idx, float* topk_w, double* prob_sum,
              void* ws, size_t ws_bytes, hipStream_t stream);

/* Grouping of the N*k token copies by expert: histogram, capacity, prefix
 * sum, stable permutation. This is forward_grouped's flatten, stable
 * argsort and bincount ("实现" section). Copy c = t*k + j is slot j of token
 * t. A copy is kept iff fewer than C earlier copies (in c order) went to the
 * same expert (capacity, notes section 三.1).
 *   topk_idx     [N, k] int32 in, values in [0, E) (other values: undefined result)
 *   prob_sum     [E] fp64 in, or NULL (then balance_stat must be NULL)
 *   counts       [E] int32 out: routed copies per expert, before capacity
 *   offsets      [E+1] int32 out: exclusive prefix sum of min(counts, C)
 *   perm         [N*k] int32 out: kept copy ids grouped by expert, and
 *                increasing within each expert; entries past offsets[E]
 *                are left untouched
 *   slot_pos     [N*k] int32 out: row of copy c in perm, or -1 if dropped
 *   balance_stat [1] fp64 out or NULL: E * sum_e (counts_e/(N*k)) * (prob_sum_e/N)
 *                (aux_loss, "负载均衡" section) */
int moe_permute(const moe_shape* shape, const int32_t* topk_idx, const double* prob_sum,
                int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* slot_pos,
                double* balance_stat, void* ws, size_t ws_bytes, hipStream_t stream);

/* Grouped SwiGLU experts: for every group g and every row r of its segment
 * [offsets[g], offsets[g+1]):
 *   out[r] = W_down[g] (silu(W_gate[g] x_r) * (W_up[g] x_r))
 * This is Expert.forward ("实现" section), one matrix product per group.
 * In bf16 layers h = silu(.)*(.) is rounded to bf16 before the down
 * projection, and accumulation is fp32.
 *   shape       n_tokens, d_model and dtype are read; nothing else
 *   n_groups    G >= 1;  d_ff: F of these experts
 *   x           [N, d] (dtype)
 *   perm        [max_rows] int32, or NULL. Row r's input is
 *               x[perm[r] / rows_per_token]; with NULL it is
 *               x[r - offsets[g]] (identity rows, as for a shared expert
 *               with offsets {0, N})
 *   offsets     [G+1] int32: non-decreasing, offsets[0] = 0,
 *               offsets[G] <= max_rows. Rows past max_rows are not
 *               computed, and input rows past N read as zero
 *   w_gate/w_up [G, F, d] (dtype);  w_down [G, d, F] (dtype)
 *   out         [max_rows, d] fp32 out, in grouped order; rows past
 *               offsets[G] are left untouched
 *   ws          >= max_rows * F * sizeof(dtype) + 256 bytes. Workspace past
 *               max_rows * F * sizeof(dtype) (rounded up to 256) is used, when
 *               there is some, to split the last partial round of tiles
 *               along K (bf16 layers); results stay deterministic for a
 *               given device and workspace size. On return, the first
 *               max_rows * F elements of ws hold h, row r of the grouped
 *               order at element r * F (bf16 in bf16 layers, the value the
 *               down projection read; fp32 in fp32 layers), for the rows
 *               below offsets[G]; the rest of ws is unspecified */
int moe_grouped_swiglu(const moe_shape* shape, int32_t n_groups, int32_t d_ff,
                       const void* x, const int32_t* perm, int32_t rows_per_token,
                       const int32_t* offsets, int32_t max_rows,
                       const void* w_gate, const void* w_up, const void* w_down,
                       float* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* Weighted combine in token order, with no atomics and a fixed summation
 * order:
 *   y[t] = sum_{j=0..k-1, slot_pos[t*k+j] >= 0} topk_w[t,j] * expert_out[slot_pos[t*k+j]]
 *          + sum_{s<S} shared_out[s, t]
 * This is the output formula of section "结构", and forward_grouped's
 * index_add_. A dropped copy adds nothing. The residual is the caller's.
 *   expert_out [rows, d] fp32 (rows >= max slot_pos + 1)
 *   slot_pos   [N*k] int32;  topk_w [N, k] fp32
 *   shared_out [S, N, d] fp32, or NULL (required when S > 0)
 *   y          [N, d] fp32 out */
int moe_combine(const moe_shape* shape, const float* expert_out, const int32_t* slot_pos,
                const float* topk_w, const float* shared_out, float* y, hipStream_t stream);

/* The whole layer: route, permute, the grouped experts (routed and shared
 * in one launch per projection), then combine. Outputs are as in the
 * calls above. s_gate/s_up [S, Fs, d] and s_down [S, d, Fs] may be NULL
 * only when S == 0.
 * stage_events: NULL, or MOE_STAGE_EVENTS events created by the caller. It
 * records event i before stage i (route, permute, gate|up, down, combine)
 * and the last event after combine, all on `stream`. A NULL entry is
 * skipped (each recorded event costs the stream a few microseconds).
 * The call may be captured in a HIP graph (stage_events NULL): it issues
 * kernels only, with no memset or copy nodes, every kernel writing what a
 * later one reads, so each replay gives the eager call's results bit for
 * bit while ws and the buffers stay allocated. */
int moe_forward(const moe_shape* shape, const void* x, const void* w_router,
                const float* logit_bias, const float* select_bias,
                const void* w_gate, const void* w_up, const void* w_down,
                const void* s_gate, const void* s_up, const void* s_down,
                float* y, int32_t* topk_idx, float* topk_w,
                int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* slot_pos,
                double* prob_sum, double* balance_stat,
                void* ws, size_t ws_bytes, hipEvent_t* stage_events, hipStream_t stream);

/* moe_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same arguments as moe_forward without ws and ws_bytes, and the same
 * kernels and results (bit for bit, on the same device). The workspace is a
 * static device array inside the library, MOE_NOALLOC_SCRATCH_BYTES bytes on
 * each device the entry point runs on, held until the process ends; its
 * address is looked up on the first call on a device. The call allocates
 * nothing and needs no zeroed memory (every kernel writes what it later
 * reads). Every call on a device shares that device's array: calls that can
 * overlap on one device (other streams, other host threads) race and must
 * be serialised by the caller.
 * Errors: as moe_forward; MOE_ERR_UNSUPPORTED when moe_workspace_bytes(shape)
 * exceeds MOE_NOALLOC_SCRATCH_BYTES (decode-sized layers fit: the
 * DeepSeek-V3-shaped layer at 64 tokens needs about 51 MiB); MOE_ERR_HIP
 * when the device or the array's address cannot be obtained. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_forward_noalloc(const moe_shape* shape, const void* x, const void* w_router,
                        const float* logit_bias, const float* select_bias,
                        const void* w_gate, const void* w_up, const void* w_down,
                        const void* s_gate, const void* s_up, const void* s_down,
                        float* y, int32_t* topk_idx, float* topk_w,
                        int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* slot_pos,
                        double* prob_sum, double* balance_stat, hipEvent_t* stage_events,
                        hipStream_t stream);

/* Training forward: moe_forward (bf16 layers) that also keeps, in the
 * caller's gu_save, the fp32 gate and up values G = x W_gate^T and
 * U = x W_up^T of every computed row, for moe_backward (which then skips
 * recomputing them). gu_save holds moe_train_save_floats(shape) floats:
 * routed G [N*k, F] then routed U [N*k, F], rows in the grouped order of
 * perm (rows at or past offsets[E] are not written); then each shared
 * expert's G [S*N, Fs] then U [S*N, Fs] (shared expert s at rows s*N..).
 * Everything else as in moe_forward. Errors: MOE_ERR_UNSUPPORTED unless the
 * dtype is MOE_DTYPE_BF16; MOE_ERR_INVALID_ARG when gu_save is NULL and N > 0. */
size_t moe_train_save_floats(const moe_shape* shape);
int moe_forward_train(const moe_shape* shape, const void* x, const void* w_router,
                      const float* logit_bias, const float* select_bias,
                      const void* w_gate, const void* w_up, const void* w_down,
                      const void* s_gate, const void* s_up, const void* s_down,
                      float* y, int32_t* topk_idx, float* topk_w,
                      int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* slot_pos,
                      double* prob_sum, double* balance_stat, float* gu_save,
                      void* ws, size_t ws_bytes, hipEvent_t* stage_events, hipStream_t stream);

/* ---------------------------------------------------------------------
 * Training-side router statistics (side outputs; the forward needs none).
 * The pages' formulas for these were lost in extraction; each call states
 * the reading it computes.
 * --------------------------------------------------------------------- */

/* z-loss, importance and the importance loss, from the router of shape:
 *   z_loss[0]         = (1/N) sum_t (log sum_e exp l[t,e])^2, l = x W_r^T (+ logit_bias):
 *                       the ST-MoE form of the z-loss on the raw gate logits
 *                       (notes "混合专家模型 (MoE)...", section 三.3); the logits
 *                       are recomputed here
 *   importance[e]     = sum of topk_w[t,j] over the copies with topk_idx[t,j] = e,
 *                       before capacity (notes, section 二, importance loss)
 *   importance_cv2[0] = Var_e(importance) / Mean_e(importance)^2, population
 *                       variance; 0 when the mean is 0
 * Each output is fp64 and may be NULL (not computed); at least one is given.
 * topk_idx/topk_w are moe_route's outputs (needed for the importance terms),
 * x/w_router/logit_bias as in moe_route (needed for z_loss). Sums run in a
 * fixed order. N = 0 gives zeros. ws >= moe_workspace_bytes(shape). */
int moe_router_aux(const moe_shape* shape, const void* x, const void* w_router, const float* logit_bias,
                   const int32_t* topk_idx, const float* topk_w, double* z_loss, double* importance,
                   double* importance_cv2, void* ws, size_t ws_bytes, hipStream_t stream);

/* One step of the aux-loss-free balancing of section "负载均衡": the
 * selection bias of an overloaded expert goes down, an idle one's goes up.
 * The page gives no rule or step size; this computes, in place and in fp32,
 *   select_bias[e] -= gamma * sign(counts[e] - N*k/E)
 * with the sign taken exactly (counts[e]*E against N*k) and counts the
 * routed copies before capacity (moe_permute's counts). gamma >= 0, finite. */
int moe_update_select_bias(const moe_shape* shape, const int32_t* counts, float gamma, float* select_bias,
                           hipStream_t stream);

/* ---------------------------------------------------------------------
 * FP8 expert weights (W8A16), for decode, whose time is the time to read
 * the touched experts' weights ("推理视角" section: DeepSeek-V3 ships FP8
 * weights). The page names no format or scale granularity; these calls use
 * OCP FP8 E4M3 codes (e4m3fn: exponent bias 7, largest 448, no infinities)
 * with one fp32 scale per output row of each weight matrix. The layer they
 * compute is the bf16 layer with every expert weight replaced by
 * scale[row] * decode(code). x, the router and h stay bf16; the shape's
 * dtype must be MOE_DTYPE_BF16 (else MOE_ERR_UNSUPPORTED).
 * --------------------------------------------------------------------- */

/* Row scales of quantised expert weights, FP8 or int4 (device pointers, fp32). */
typedef struct {
  const float* gate;    /* [E, F]: scale of w_gate row (e, f) */
  const float* up;      /* [E, F] */
  const float* down;    /* [E, d] */
  const float* s_gate;  /* [S, Fs]; NULL allowed only when S == 0 */
  const float* s_up;    /* [S, Fs] */
  const float* s_down;  /* [S, d] */
} moe_weight_scales;
typedef moe_weight_scales moe_fp8_scales;

/* Quantise a bf16 matrix [rows, cols], row by row:
 *   scales[r]   = max_c |w[r, c]| / 448                     (fp32 division)
 *   codes[r, c] = E4M3 round-to-nearest-even of w[r, c] / scales[r]
 *                 (fp32 division; the sign bit follows the quotient's)
 * An all-zero row gets scale 0 and codes 0. A stacked [E, F, d] weight is
 * rows = E*F, cols = d.
 *   w_bf16 [rows, cols] bf16 in;  codes [rows, cols] uint8 out;  scales [rows] fp32 out
 * cols must be a multiple of 64 and rows < 2^31 (else MOE_ERR_UNSUPPORTED). */
int moe_quantize_fp8(int64_t rows, int32_t cols, const void* w_bf16, uint8_t* codes, float* scales,
                     hipStream_t stream);

/* The weights that FP8 codes stand for, as the FP8 grouped GEMM reads them
 * (the same section of the handbook; E4M3 as in moe_quantize_fp8):
 *   out[r, c] = scales[r] * value(codes[r, c])     (one fp32 product)
 * value() widens each code to bf16 exactly, with the routine the FP8 grouped
 * GEMM applies to its weight fragments; the codes 0x7F and 0xFF give NaN.
 *   codes [rows, cols] uint8 in;  scales [rows] fp32 in;  out [rows, cols] fp32 out
 * All device pointers, caller-owned. rows < 0, cols <= 0 or a NULL pointer
 * with rows > 0: MOE_ERR_INVALID_ARG; cols not a multiple of 8:
 * MOE_ERR_UNSUPPORTED. rows == 0 does nothing. */
int moe_dequantize_fp8(int64_t rows, int32_t cols, const uint8_t* codes, const float* scales, float* out,
                       hipStream_t stream);

/* moe_grouped_swiglu with FP8 weights: w_gate/w_up [G, F, d] and w_down
 * [G, d, F] are E4M3 codes; sc_gate/sc_up [G, F] and sc_down [G, d] their
 * row scales. Everything else as in moe_grouped_swiglu (bf16 x and h). */
int moe_grouped_swiglu_fp8(const moe_shape* shape, int32_t n_groups, int32_t d_ff, const void* x,
                           const int32_t* perm, int32_t rows_per_token, const int32_t* offsets,
                           int32_t max_rows, const uint8_t* w_gate, const uint8_t* w_up,
                           const uint8_t* w_down, const float* sc_gate, const float* sc_up,
                           const float* sc_down, float* out, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/* moe_forward with FP8 routed and shared expert weights (codes) and their
 * row scales. The router weights stay bf16. Outputs, workspace and events
 * as in moe_forward. */
int moe_forward_fp8(const moe_shape* shape, const void* x, const void* w_router,
                    const float* logit_bias, const float* select_bias, const uint8_t* w_gate,
                    const uint8_t* w_up, const uint8_t* w_down, const uint8_t* s_gate,
                    const uint8_t* s_up, const uint8_t* s_down, const moe_fp8_scales* scales,
                    float* y, int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                    int32_t* perm, int32_t* slot_pos, double* prob_sum, double* balance_stat,
                    void* ws, size_t ws_bytes, hipEvent_t* stage_events, hipStream_t stream);

/* ---------------------------------------------------------------------
 * Int4 expert weights (W4A16). The notes "混合专家模型 (MoE)：大规模稀疏条件
 * 计算的架构与工程实践", section 五.1 (the memory wall of inference), suggest
 * INT4 weights with FP16/BF16 activations for the expert layers only, the
 * product taken on the dequantised weights. They give no scale granularity
 * or rounding; these calls use one fp32 scale per output row of each weight
 * matrix and symmetric codes q in [-7, 7]. The layer they compute is the
 * bf16 layer with every expert weight replaced by scale[row] * q. x, the
 * router and h stay bf16; the shape's dtype must be MOE_DTYPE_BF16 (else
 * MOE_ERR_UNSUPPORTED).
 *
 * Packed format: a row of K codes is K/2 bytes, in blocks of 64 codes (32
 * bytes). In the block of codes [k0, k0 + 64), the little-endian 32-bit
 * word at byte 16*h + 4*s (h = 0, 1; s = 0..3) holds codes
 * k0 + 16*s + 8*h + j, j = 0..7, each in a 4-bit sign and magnitude field
 * (bit 3 set for q < 0, bits 0..2 = |q|): code j in byte j % 4 of the word,
 * its low nibble for j < 4 and its high nibble for j >= 4. K must be a
 * multiple of 64.
 * --------------------------------------------------------------------- */

/* Quantise a bf16 matrix [rows, cols], row by row:
 *   scales[r] = max_c |w[r, c]| / 7                             (fp32 division)
 *   q[r, c]   = w[r, c] / scales[r] rounded to the nearest integer, ties to
 *               even (fp32 division), clamped to [-7, 7]
 * An all-zero row gets scale 0 and codes 0 (bytes 0x00).
 *   w_bf16 [rows, cols] bf16 in;  packed [rows, cols/2] uint8 out (format
 *   above);  scales [rows] fp32 out
 * cols must be a multiple of 64 and rows < 2^31 (else MOE_ERR_UNSUPPORTED). */
int moe_quantize_int4(int64_t rows, int32_t cols, const void* w_bf16, uint8_t* packed, float* scales,
                      hipStream_t stream);

/* moe_grouped_swiglu with int4 weights: w_gate/w_up [G, F, d/2] and w_down
 * [G, d, F/2] packed as above; sc_gate/sc_up [G, F] and sc_down [G, d] their
 * row scales. Everything else as in moe_grouped_swiglu (bf16 x and h). */
int moe_grouped_swiglu_int4(const moe_shape* shape, int32_t n_groups, int32_t d_ff, const void* x,
                            const int32_t* perm, int32_t rows_per_token, const int32_t* offsets,
                            int32_t max_rows, const uint8_t* w_gate, const uint8_t* w_up,
                            const uint8_t* w_down, const float* sc_gate, const float* sc_up,
                            const float* sc_down, float* out, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/* moe_forward with int4 routed and shared expert weights (packed) and their
 * row scales. The router weights stay bf16. Outputs, workspace and events
 * as in moe_forward. */
int moe_forward_int4(const moe_shape* shape, const void* x, const void* w_router,
                     const float* logit_bias, const float* select_bias, const uint8_t* w_gate,
                     const uint8_t* w_up, const uint8_t* w_down, const uint8_t* s_gate,
                     const uint8_t* s_up, const uint8_t* s_down, const moe_weight_scales* scales,
                     float* y, int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                     int32_t* perm, int32_t* slot_pos, double* prob_sum, double* balance_stat,
                     void* ws, size_t ws_bytes, hipEvent_t* stage_events, hipStream_t stream);

/* ---------------------------------------------------------------------
 * Backward pass (training). The gradients of
 *   L = sum_{t,c} dy[t, c] * y[t, c] + aux_coef * stat
 * for the bf16 layer of moe_forward, with the forward's top-k selection and
 * dropped set frozen (they are piecewise constant); stat is the balance
 * statistic of "混合专家 MoE" (anrans ai-infra handbook), section "负载均衡",
 * with the counts held constant. The layer differentiated is that of the
 * same handbook, section "实现：逐 token 与按专家分组". Readings: the bf16
 * rounding of h passes the gradient unchanged; a dropped copy (capacity, the
 * notes "混合专家模型 (MoE)：大规模稀疏条件计算的架构与工程实践", section 三.1)
 * sends no gradient into its expert and its combine weight gets none, but it
 * stays in its token's renormalisation; the selection-only bias gets none.
 * The product operands (dy, w * dy, h, and the SwiGLU input gradients) are
 * rounded to bf16 for the matrix cores, with fp32 accumulation; every other
 * step and every reduction is fp32 in a fixed order (deterministic).
 * --------------------------------------------------------------------- */

/* Workspace bytes of moe_backward for a shape (0 for an invalid shape). */
size_t moe_backward_workspace_bytes(const moe_shape* shape);

/* How moe_backward delivers the gradients (grad_mode). */
enum moe_grad_mode {
  MOE_GRAD_WRITE = 0,       /* every output written, fp32 */
  MOE_GRAD_ACCUMULATE = 1,  /* dx written; every other gradient added to the fp32 buffer's contents */
  MOE_GRAD_WRITE_BF16 = 2   /* as MOE_GRAD_WRITE, but the expert weight gradients (dw_gate, dw_up,
                               dw_down, ds_*) are stored as bf16: the round-to-nearest-even of the
                               fp32 values MOE_GRAD_WRITE stores */
};

/* Inputs: the layer's bf16 weights as passed to moe_forward; the forward's
 * outputs topk_idx [N, k], topk_w [N, k], counts [E], offsets [E+1], perm
 * [N*k], slot_pos [N*k] (unchanged since that call); gu_saved: the gu_save
 * buffer of a moe_forward_train call with the same inputs (NULL: G and U are
 * recomputed); dy [N, d] fp32, read at
 * bf16 precision (every use goes through its round-to-nearest-even bf16
 * value, so bf16-valued dy loses nothing); aux_coef (finite; 0 drops the
 * balance term); grad_mode (enum moe_grad_mode).
 * Outputs: dx [N, d] fp32; dw_router [E, d] fp32; d_logit_bias [E] fp32
 * (NULL: not computed); dw_gate, dw_up [E, F, d]; dw_down [E, d, F]; ds_gate,
 * ds_up [S, Fs, d] and ds_down [S, d, Fs] (may be NULL when S == 0): fp32, or
 * bf16 under MOE_GRAD_WRITE_BF16.
 * MOE_GRAD_WRITE(_BF16): every entry is written (an expert with no kept copy
 * gets zeros). MOE_GRAD_ACCUMULATE: dx is written, every other output gets
 * the gradient added to its contents (an expert with no kept copy is not
 * touched): the form for summing gradients over micro-batches into fp32
 * buffers, which also skips writing the zero gradients of idle experts.
 * MOE_GRAD_WRITE_BF16 halves the bytes of the weight-gradient stores, which
 * bound those products when experts receive few rows.
 * Errors: MOE_ERR_UNSUPPORTED unless the shape's dtype is MOE_DTYPE_BF16;
 * MOE_ERR_INVALID_ARG for a missing pointer, a non-finite aux_coef or an
 * unknown grad_mode;
 * MOE_ERR_WORKSPACE when ws_bytes < moe_backward_workspace_bytes(shape). */
int moe_backward(const moe_shape* shape, const void* x, const void* w_router, const float* logit_bias,
                 const void* w_gate, const void* w_up, const void* w_down, const void* s_gate, const void* s_up,
                 const void* s_down, const int32_t* topk_idx, const float* topk_w, const int32_t* counts,
                 const int32_t* offsets, const int32_t* perm, const int32_t* slot_pos, const float* dy,
                 const float* gu_saved, double aux_coef, int32_t grad_mode, float* dx, float* dw_router,
                 float* d_logit_bias, void* dw_gate, void* dw_up, void* dw_down, void* ds_gate, void* ds_up,
                 void* ds_down, void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
