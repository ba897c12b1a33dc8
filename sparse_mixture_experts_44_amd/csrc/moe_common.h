// Shared device helpers and the internal launch interfaces of libmoe.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef uint16_t bf16_t;  // raw bfloat16 bits
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));  // 16-byte piece (a native vector, not HIP's uint4 struct)

constexpr int kWave = 64;
constexpr int kMaxExperts = 512;
constexpr int kMaxTopK = 32;
constexpr int kMaxShared = 16;
constexpr int kMaxTileEntries = kMaxExperts + kMaxShared;  // routed + shared groups in one grouped launch

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// fp32 -> bf16 bits, round to nearest, ties to even (NaN stays a quiet NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);
  return (bf16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

// FP8 E4M3 -> bf16 for 8 codes (bytes of lo, then hi), two per instruction
// (v_cvt_scalef32_pk_bf16_fp8 with scale 1): exact, since every e4m3 value
// (4 significant bits, exponents 2^-9 .. 2^8) is a bf16 value.
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, false);
  const bf16x2_t e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, true);
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  const bf16x4_t ab = __builtin_shufflevector(a, b, 0, 1, 2, 3), ce = __builtin_shufflevector(c, e, 0, 1, 2, 3);
  return __builtin_shufflevector(ab, ce, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ------------------------------------------------------------------ LDS staging (grouped GEMM, router)

// LDS tile rows hold BK bf16 of K: PPR = BK/8 pieces of 16 bytes, stored at
// piece ^ swz(row). A wave's MFMA operand read has lanes 0..31 on 32
// consecutive rows at the same logical piece. These XOR patterns spread every
// group of 8 lanes (128 bytes per clock) and every group of 16 lanes (256
// bytes per clock) over distinct banks:
//   PPR = 8 (128-byte rows): g(r) = (r & 7) ^ ((r >> 3) & 1)
//   PPR = 4 (64-byte rows):  g(r) = ((r >> 1) & 3) ^ ((r >> 3) & 1)
//   PPR = 2 (32-byte rows of int4 weights, read 16 bytes per lane per step):
//                            g(r) = ((r >> 2) ^ (r >> 3)) & 1
//   PPR = 16, 32 (256- and 512-byte rows, which all start on bank 0):
//                            g(r) = r & 15 (16 rows on 16 distinct 16-byte bank groups)
template <int PPR>
__device__ __forceinline__ int swz(int row) {
  if constexpr (PPR >= 16) return row & 15;
  else if constexpr (PPR == 8) return (row & 7) ^ ((row >> 3) & 1);
  else if constexpr (PPR == 4) return ((row >> 1) & 3) ^ ((row >> 3) & 1);
  else return ((row >> 2) ^ (row >> 3)) & 1;
}

// Copy 16 bytes per lane from global memory straight into LDS at
// lds_addr + 16 * lane (global_load_lds_dwordx4; no VGPR staging, counted by
// vmcnt). It is written as an instruction rather than the builtin: the
// compiler treats the builtin's LDS write as aliasing every LDS read and
// would drain all copies in flight (vmcnt(0)) before each fragment read,
// which defeats the multi-stage prefetch. The instruction has no output
// registers; the explicit vmcnt waits below order the reads after the copies.
// On gfx9 an LDS copy needs one wait state after a scalar write of M0 (the
// compiler inserts it for the builtin, not inside inline asm): hence the nop.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g),
               "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Wait until at most N of this wave's vector-memory operations are
// outstanding, then a workgroup barrier. The barrier is written out (not
// __syncthreads) so that the compiler does not also wait for the LDS copies
// of later stages that are still in flight.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// wait_vm_barrier<n> for a wave-uniform n in [0, MAXN] known only at run time
// (a chain of scalar compares; anything out of range waits for everything).
template <int MAXN>
__device__ __forceinline__ void wait_vm_barrier_rt(int n) {
  if constexpr (MAXN == 0) {
    wait_vm_barrier<0>();
  } else {
    if (n == MAXN) wait_vm_barrier<MAXN>();
    else wait_vm_barrier_rt<MAXN - 1>(n);
  }
}

// ------------------------------------------------------------------ router

// prob_sum[e] from the router's nb per-workgroup sums (rows of E doubles), by
// one wavefront: lane-strided sums, then a fixed butterfly. The router's own
// launch and the permute's column scan (which takes this step over when the
// forward defers it) both use it, so prob_sum is the same bits either way.
__device__ __forceinline__ double prob_sum_wave(const double* __restrict__ partials, int nb, int E, int e,
                                                int lane) {
  double a = 0.0;
  for (int b = lane; b < nb; b += kWave) a += partials[(size_t)b * E + e];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) a += __shfl_xor(a, o, kWave);
  return a;
}
// `partials`: route_partials_bytes(s) bytes; `logits`: route_logits_floats(s) floats (workspace).
// defer_nb != NULL: where the last step would be a launch of its own that adds
// the per-workgroup sums into prob_sum, it is left out and *defer_nb is their
// count (the partials rows), for the caller to take over (else *defer_nb = 0).
int launch_route(const moe_shape& s, const void* x, const void* w_router, const float* logit_bias,
                 const float* select_bias, int32_t* topk_idx, float* topk_w, double* prob_sum,
                 double* partials, float* logits, float* split_ws, size_t split_bytes, hipStream_t stream,
                 int* defer_nb = nullptr);
int launch_prob_sum(const double* partials, int nb, int E, double* prob_sum, hipStream_t stream);
int route_blocks(const moe_shape& s);
size_t route_partials_bytes(const moe_shape& s);  // the partials region: route_blocks(s) x E doubles + a counter
// Training-side statistics: z-loss (recomputes the logits), importance and its CV^2; any output may be NULL.
int launch_router_aux(const moe_shape& s, const void* x, const void* w_router, const float* logit_bias,
                      const int32_t* topk_idx, const float* topk_w, double* z_loss, double* imp,
                      double* imp_cv2, double* partials, float* logits, float* split_ws, size_t split_bytes,
                      hipStream_t stream);
int launch_bias_update(const moe_shape& s, const int32_t* counts, float gamma, float* bias,
                       hipStream_t stream);
size_t route_logits_floats(const moe_shape& s);
// The router logits' K-split partial sums ([splits, N, E] floats; their sum in split order is x W_r^T).
// Large bf16 routers (E >= 64, N >= 256) are one grouped GEMM on the matrix cores (splits = 1), whose
// split tail tiles use split_ws (split_bytes; the grouped GEMMs' region, idle while the router runs).
int launch_router_logits(const moe_shape& s, const void* x, const void* w_router, float* logits, int* splits,
                         float* split_ws, size_t split_bytes, hipStream_t stream);

// ------------------------------------------------------------------ permute
int permute_chunks(const moe_shape& s);
// partials, nb > 0: the router's deferred per-workgroup sums; the column scan
// adds them into sum_out (the same E doubles as prob_sum) before the scatter
// reads prob_sum. Needs more than one chunk (permute_chunks(s) > 1).
int launch_permute(const moe_shape& s, const int32_t* topk_idx, const double* prob_sum,
                   int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* slot_pos,
                   double* balance_stat, int32_t* hist, int32_t* base, hipStream_t stream,
                   const double* partials = nullptr, int nb = 0, double* sum_out = nullptr);

// ------------------------------------------------------------------ grouped SwiGLU
// One set of segments (the routed experts, or the shared experts).
struct SegSet {
  const int32_t* offsets;  // [n_groups+1] on the device; NULL: group g = rows [g*uniform_rows, (g+1)*uniform_rows)
  const int32_t* perm;     // row r reads x[perm[r] / rows_per_token]; NULL: x[r - seg_start]
  int32_t n_groups;
  int32_t uniform_rows;
  int32_t rows_per_token;
  int32_t max_rows;        // rows at or past this are never computed
  int32_t group_rows_max;  // a bound on every group's rows known on the host (a capacity), or 0
  int32_t d_ff;
  const void* w_gate;      // [G, d_ff, d]  (bf16, fp32, FP8 E4M3 codes, or [G, d_ff, d/2] packed int4)
  const void* w_up;        // [G, d_ff, d]
  const void* w_down;      // [G, d, d_ff]
  const float* sc_gate;    // quantised weights only: [G, d_ff] row scales of w_gate
  const float* sc_up;      // [G, d_ff]
  const float* sc_down;    // [G, d]
  void* h;                 // [max_rows, d_ff]: gate|up output, down input
  float* g_save;           // phase 1, bf16 weights, optional: [max_rows, d_ff] fp32 gate values (x W_gate^T)
  float* u_save;           //   and up values, beside h, for the backward pass
  float* out;              // [max_rows, d]
  // Weight-gradient mode (phase 2 only, bf16): when set, group g (uniform_rows
  // = M rows) multiplies the K_g = k_offsets[g+1] - k_offsets[g] columns
  // (multiples of 64; K_g = 0: zero output) of its own blocks of h and w_down:
  // h + M * k_offsets[g] holds [M, K_g] and w_down + d_model * k_offsets[g]
  // holds [d_model, K_g], each row-major: out[g*M + m, n] = sum_k h_g[m, k] * w_g[n, k].
  const int32_t* k_offsets;
  // With k_offsets: groups with K_g = 0 get no tiles, and their output is left
  // as it is (the caller zeroes it, or leaves it when accumulating).
  int32_t skip_empty_k;
  // N-major weights (phase 2 only, bf16, not with k_offsets): when b_nmajor is
  // set, group g's operand is read as K rows of d_model values each (the
  // weight in its stored orientation: out[r, n] = sum_k h[r, k] * B_g[k, n]).
  // Rows k < b_split (all rows when b_split == 0) come from w_down + g*b_split*d
  // (g*K*d without a split), rows k >= b_split from w_up + g*b_split*d at row
  // k - b_split. b_split is a multiple of 64.
  int32_t b_nmajor;
  int32_t b_split;
  // Phase 2, set 0 (one set per launch): add the products to out instead of writing them; with k_offsets,
  // a group whose K range is empty then leaves its rows untouched.
  int32_t accumulate;
  // Phase 2, not with accumulate: out holds bf16 (round to nearest even of the fp32 sums).
  int32_t out_bf16;
};

struct GroupedParams {
  SegSet set[2];
  int32_t n_sets;
  const void* x;           // [n_tokens, d]
  int32_t n_tokens;
  int32_t d_model;
  int32_t dtype;
  int32_t balance_m;       // 1: split each segment into equal m-tiles (else BM rows and a short last tile)
  int32_t wq;              // expert weights: 0 bf16/fp32, 8 FP8 E4M3 codes, 4 packed int4 codes (both with
                           // per-row scales; x and h bf16)
  float* split_ws;         // workspace for the K-parts of split tail tiles (bf16 path), or NULL
  long long split_cap;     // its size in floats (0: no split)
};

// Workspace bytes that let every launch split its tail tiles (grouped_split_bytes(rows, groups) for
// a launch whose routed set has `rows` rows over `groups` groups).
size_t grouped_split_bytes(long long rows, int groups);

// Phase 1: h = silu(x Wg^T) * (x Wu^T) per segment; phase 2: out = h Wd^T.
int launch_grouped(const GroupedParams& p, int phase, hipStream_t stream);

// ------------------------------------------------------------------ FP8 weights
// codes[r, c] = e4m3(w[r, c] / scales[r]), scales[r] = max_c |w[r, c]| / 448 (fp32).
int launch_quantize_fp8(long long rows, int cols, const void* w_bf16, uint8_t* codes, float* scales,
                        hipStream_t stream);
// out[r, c] = scales[r] * decode(codes[r, c]) in fp32, decoding with fp8x8_to_bf16 (cols a multiple of 8).
int launch_dequantize_fp8(long long rows, int cols, const uint8_t* codes, const float* scales, float* out,
                          hipStream_t stream);
// ------------------------------------------------------------------ int4 weights
// q[r, c] = clamp(rint(w[r, c] / scales[r]), -7, 7), scales[r] = max_c |w[r, c]| / 7 (fp32), packed as
// the grouped GEMM reads it (quant_int4.hip states the layout).
int launch_quantize_int4(long long rows, int cols, const void* w_bf16, uint8_t* packed, float* scales,
                         hipStream_t stream);

// ------------------------------------------------------------------ backward (backward.hip)
int launch_gather_rows(const void* x, const float* dy, const float* topk_w, const int32_t* perm,
                       const int32_t* n_valid, int k, int d, int rows, void* Xg, void* dYg, void* dO, hipStream_t st);
int launch_swiglu_backward(const float* G, const float* U, const float* dHp, const float* topk_w,
                           const int32_t* perm, const int32_t* n_valid, int rows, int F, void* h, void* dGU,
                           float* dw, hipStream_t st);
int launch_k_offsets(const int32_t* offsets, int G, int uniform, int32_t* kofs, hipStream_t st);
int launch_transpose_padded(const void* in, int in_stride, int col_off, int C, const int32_t* offsets, int uniform,
                            int replicate, const int32_t* kofs, int G, void* out, int kmax, hipStream_t st);
int launch_router_backward(const moe_shape& s, const float* logits, int splits, const float* logit_bias,
                           const int32_t* topk_idx, const float* topk_w, const float* dw, const int32_t* counts,
                           double aux_coef, float* dl, hipStream_t st);
// The router weight gradient sums token chunks into part (router_wgrad_part_floats
// floats), then the chunks in order into dwr; dlb (optional) gets sum_t dl.
int router_wgrad_splits(int N);
size_t router_wgrad_part_floats(int N, int E, int d);
int launch_router_wgrad(const float* dl, const void* x, int N, int E, int d, float* part, float* dwr, float* dlb,
                        int accumulate, hipStream_t st);
int launch_dx(const float* dXr, const int32_t* slot_pos, const float* dXs, int S, const float* dl, const void* wr,
              const float* rterm, int N, int E, int k, int d, float* dx, hipStream_t st);
// dl [N, E] fp32 -> bf16 parts: dlh [N, 2E] (hi | lo per row) and dlT [E, 2N] (its transpose)
int launch_split_hilo(const float* dl, int N, int E, void* dlh, void* dlT, hipStream_t st);
// d_logit_bias[e] = sum_t dl[t][e] (added to d_logit_bias when accumulating)
int launch_logit_bias_grad(const float* dl, int N, int E, float* dlb, int accumulate, hipStream_t st);
int launch_fill_f32(float* p, size_t n, float v, hipStream_t st);
// Zeroes block g (block_bytes at out + g * block_bytes, a multiple of 16) of every group g < G
// with K_g = kofs[g + 1] - kofs[g] = 0.
int launch_zero_empty_groups(void* out, const int32_t* kofs, int G, size_t block_bytes, hipStream_t st);

// ------------------------------------------------------------------ combine
int launch_combine(const moe_shape& s, const float* expert_out, const int32_t* slot_pos,
                   const float* topk_w, const float* shared_out, float* y, hipStream_t stream);

}  // namespace moe
