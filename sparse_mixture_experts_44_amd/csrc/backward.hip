// Backward pass of the MoE layer: the element-wise, gather, transpose and
// router kernels around the grouped GEMMs (which grouped_swiglu.hip runs).
//
// The function differentiated is the forward layer of "混合专家 MoE" (anrans
// ai-infra handbook), section "实现：逐 token 与按专家分组", with the top-k
// selection and the dropped set of the forward frozen, and the scalar
//   L = sum(dy * y) + aux_coef * E * sum_e f_e P_e
// (the balance statistic of section "负载均衡", counts held constant). For one
// expert over its rows X (SwiGLU, h = silu(G) * U, G = X Wg^T, U = X Wu^T,
// O = h Wd^T, output scaled by the combine weight w):
//   dH' = dy Wd            (per row, before the weight)
//   dw  = sum_f h * dH'    (the combine weight's gradient: dy . O)
//   dH  = w dH';  dG = dH * U * silu'(G);  dU = dH * silu(G)
//   dX  = dG Wg + dU Wu;   dWd = (w dy)^T h;  dWg = dG^T X;  dWu = dU^T X
// and for the router, per token: the renormalisation w_j = p_j / sum_i p_i,
// the balance term's dp[e] += aux_coef * E * f_e / N, and the softmax
// dl = p * (dp - sum(dp * p)); then dW_r = dl^T x, d(logit bias) = sum_t dl,
// dx += dl W_r. The rounding of h to bf16 passes the gradient unchanged.
//
// Rounding points (bf16 operands of the MFMA GEMMs, fp32 accumulation): dy,
// w * dy, h, dG and dU are rounded to bf16 where they feed a GEMM; dl feeds the
// router products as two bf16 parts (hi + lo, about 2^-16 relative) when those
// run as GEMMs. The element-wise steps and every reduction here run in fp32, in
// a fixed order.
#include <math.h>

#include <algorithm>

#include "moe_common.h"

namespace moe {
namespace {

constexpr int kT = 256;

__device__ __forceinline__ float bf(bf16_t b) { return bf16_to_f32(b); }

// Rows of the kept copies in grouped order: Xg[r] = x[t], dYg[r] = bf16(dy[t]),
// dO[r] = bf16(w[t, j] * dYg[r]), for copy c = perm[r] = t * k + j.
// Shared experts (perm == nullptr): row r is token r, w = 1 (dO is not written).
// Rows at or past *n_valid (when given) are not kept copies and are skipped.
// Eight columns (16 bytes of bf16) per thread; d is a multiple of 8.
__global__ __launch_bounds__(kT) void gather_rows_kernel(const bf16_t* __restrict__ x, const float* __restrict__ dy,
                                                         const float* __restrict__ topk_w,
                                                         const int32_t* __restrict__ perm,
                                                         const int32_t* __restrict__ n_valid, int k, int d,
                                                         bf16_t* __restrict__ Xg, bf16_t* __restrict__ dYg,
                                                         bf16_t* __restrict__ dO) {
  const int r = blockIdx.x;
  if (n_valid && r >= *n_valid) return;
  const int c = perm ? perm[r] : r;
  const int t = perm ? c / k : r;
  const float w = perm ? topk_w[c] : 1.f;
  const int d8 = d / 8;
  const u32x4_t* xs = reinterpret_cast<const u32x4_t*>(x + (size_t)t * d);
  const float4* ys = reinterpret_cast<const float4*>(dy + (size_t)t * d);
  u32x4_t* xo = reinterpret_cast<u32x4_t*>(Xg + (size_t)r * d);
  u32x4_t* yo = reinterpret_cast<u32x4_t*>(dYg + (size_t)r * d);
  u32x4_t* oo = reinterpret_cast<u32x4_t*>(dO + (size_t)r * d);
  for (int i = threadIdx.x; i < d8; i += kT) {
    if (Xg) xo[i] = xs[i];
    const float4 a = ys[2 * i], b = ys[2 * i + 1];
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    u32x4_t yb, ob;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf16_t y0 = f32_to_bf16(v[2 * q]), y1 = f32_to_bf16(v[2 * q + 1]);
      yb[q] = (uint32_t)y0 | ((uint32_t)y1 << 16);
      ob[q] = (uint32_t)f32_to_bf16(w * bf(y0)) | ((uint32_t)f32_to_bf16(w * bf(y1)) << 16);
    }
    yo[i] = yb;
    if (dO) oo[i] = ob;
  }
}

// A 64 x 64 bf16 tile in LDS: rows of 66 halves (33 words), so that the
// column reads of the transposed store hit at most two lanes per bank.
constexpr int kTP = 66;

// Packs the 8 column entries tile[a0 .. a0+7][b] into 16 bytes.
__device__ __forceinline__ u32x4_t tile_column8(const uint16_t (*tile)[kTP], int a0, int b) {
  u32x4_t v;
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = (uint32_t)tile[a0 + 2 * q][b] | ((uint32_t)tile[a0 + 2 * q + 1][b] << 16);
  return v;
}

// Stores 16 bytes (8 halves) into row a of the tile at column b0 (b0 a multiple of 8).
__device__ __forceinline__ void tile_row8(uint16_t (*tile)[kTP], int a, int b0, u32x4_t v) {
  uint32_t* p = reinterpret_cast<uint32_t*>(&tile[a][b0]);  // 4-byte aligned: 66 a + b0 is even
#pragma unroll
  for (int q = 0; q < 4; ++q) p[q] = v[q];
}

// One row per workgroup: from G, U (fp32 [rows, F]), dH' = dy Wd (fp32) and the
// row's combine weight w: h = bf16(silu(G) U) (written when h != nullptr),
// dw = sum_f h dH' (fixed tree order; written to dw[perm[r]] when dw != nullptr),
// dGU[r] = [bf16(w dH' U silu'(G)) | bf16(w dH' silu(G))].
__global__ __launch_bounds__(kT) void swiglu_backward_kernel(const float* __restrict__ G, const float* __restrict__ U,
                                                             const float* __restrict__ dHp, const float* __restrict__ topk_w,
                                                             const int32_t* __restrict__ perm,
                                                             const int32_t* __restrict__ n_valid, int F,
                                                             bf16_t* __restrict__ h, bf16_t* __restrict__ dGU,
                                                             float* __restrict__ dw) {
  __shared__ float s_part[kT];
  const int r = blockIdx.x;
  if (n_valid && r >= *n_valid) return;  // whole workgroup, before any barrier
  const float w = perm ? topk_w[perm[r]] : 1.f;
  const size_t o = (size_t)r * F;
  float acc = 0.f;
  for (int f = threadIdx.x; f < F; f += kT) {
    const float g = G[o + f], u = U[o + f], dp = dHp[o + f];
    const float s = 1.f / (1.f + expf(-g));
    const float silu = g * s;
    const bf16_t hb = f32_to_bf16(silu * u);
    if (h) h[o + f] = hb;
    acc += bf(hb) * dp;
    const float dh = w * dp;
    dGU[(size_t)r * 2 * F + f] = f32_to_bf16(dh * u * s * (1.f + g * (1.f - s)));
    dGU[(size_t)r * 2 * F + F + f] = f32_to_bf16(dh * silu);
  }
  s_part[threadIdx.x] = acc;
  __syncthreads();
  for (int st = kT / 2; st > 0; st >>= 1) {
    if (threadIdx.x < st) s_part[threadIdx.x] += s_part[threadIdx.x + st];
    __syncthreads();
  }
  if (dw && threadIdx.x == 0) dw[perm[r]] = s_part[0];
}

// kofs[g] = start of group g's K range in the padded transposed layout: the
// groups' row counts, each rounded up to a multiple of 64, summed in order.
// offsets == nullptr: every group has `uniform` rows.
__global__ void k_offsets_kernel(const int32_t* __restrict__ offsets, int G, int uniform, int32_t* __restrict__ kofs) {
  if (threadIdx.x != 0) return;
  int run = 0;
  for (int g = 0; g < G; ++g) {
    kofs[g] = run;
    const int rows = offsets ? offsets[g + 1] - offsets[g] : uniform;
    run += (rows + 63) / 64 * 64;
  }
  kofs[G] = run;
}

// Transposes grouped rows into the blocks the weight-gradient GEMMs read: group g
// (rows_g rows, padded to K_g = kofs[g + 1] - kofs[g]) becomes the row-major
// [C, K_g] block at out + C * kofs[g]: block[c][i] = in[row_g(i)][col_off + c] for
// i < rows_g, and 0 on the pad columns; row_g(i) = offsets[g] + i (or
// g * uniform + i, or, with replicate, i: every group reads rows [0, uniform)).
// One 64 x 64 tile per workgroup (tile k0 of the concatenated K ranges; tiles
// past kofs[G] do nothing), 16-byte loads and stores (in_stride, col_off and C
// multiples of 8). Each group's rows stay a few KB long, however many groups.
__global__ __launch_bounds__(kT) void transpose_padded_kernel(const bf16_t* __restrict__ in, int in_stride, int col_off,
                                                              int C, const int32_t* __restrict__ offsets, int uniform,
                                                              int replicate, const int32_t* __restrict__ kofs, int G,
                                                              bf16_t* __restrict__ out) {
  __shared__ uint16_t tile[64][kTP];
  __shared__ int s_g;
  const int c0 = blockIdx.y * 64, k0 = blockIdx.x * 64;
  if (threadIdx.x == 0) {
    int g = -1;
    if (k0 < kofs[G]) {
      int lo = 0, hi = G;  // kofs[lo] <= k0 < kofs[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (kofs[mid] <= k0) lo = mid;
        else hi = mid;
      }
      g = lo;
    }
    s_g = g;
  }
  __syncthreads();
  const int g = s_g;
  if (g < 0) return;  // whole workgroup
  const int rows = offsets ? offsets[g + 1] - offsets[g] : uniform;
  const int first = replicate ? 0 : (offsets ? offsets[g] : g * uniform);
  const int i0 = k0 - kofs[g];  // row index within the group of column k0
  const int Kg = kofs[g + 1] - kofs[g];
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int q = threadIdx.x + it * kT, i = q >> 3, ch = q & 7;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (i0 + i < rows && c0 + ch * 8 < C)
      v = *reinterpret_cast<const u32x4_t*>(in + (size_t)(first + i0 + i) * in_stride + col_off + c0 + ch * 8);
    tile_row8(tile, i, ch * 8, v);
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int q = threadIdx.x + it * kT, c = q >> 3, ch = q & 7;
    if (c0 + c < C)
      *reinterpret_cast<u32x4_t*>(out + (size_t)C * kofs[g] + (size_t)(c0 + c) * Kg + i0 + ch * 8) =
          tile_column8(tile, ch * 8, c);
  }
}

// Router backward, one wave per token: p = softmax(l + logit_bias) from the
// summed logit splits; w_j = topk_w (the forward's combine weights), sum_i p_i
// over the selected; dsel_j = (dw_j - sum_i dw_i w_i) / sum_i p_i (renormalised)
// or dw_j; dp[e] = dsel at the selected experts + aux_coef * E * f_e / N;
// dl = p * (dp - sum(dp * p)).
template <int EL>
__global__ __launch_bounds__(kT) void router_backward_kernel(const float* __restrict__ part, int splits,
                                                             const float* __restrict__ logit_bias,
                                                             const int32_t* __restrict__ topk_idx,
                                                             const float* __restrict__ topk_w,
                                                             const float* __restrict__ dw,
                                                             const int32_t* __restrict__ counts, float aux_scale,
                                                             int N, int E, int k, int renorm,
                                                             float* __restrict__ dl) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kT / kWave) + (threadIdx.x >> 6);
  if (t >= N) return;  // whole wave
  const size_t split_stride = (size_t)N * E;
  float l[EL], pe[EL];
  float mx = -INFINITY;
#pragma unroll
  for (int m = 0; m < EL; ++m) {
    const int e = lane + kWave * m;
    float v = -INFINITY;
    if (e < E) {
      v = 0.f;
      for (int q = 0; q < splits; ++q) v += part[(size_t)q * split_stride + (size_t)t * E + e];
      if (logit_bias) v += logit_bias[e];
    }
    l[m] = v;
    mx = fmaxf(mx, v);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
  float sum = 0.f;
#pragma unroll
  for (int m = 0; m < EL; ++m) {
    pe[m] = (lane + kWave * m < E) ? expf(l[m] - mx) : 0.f;
    sum += pe[m];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, kWave);
#pragma unroll
  for (int m = 0; m < EL; ++m) pe[m] /= sum;
  // the selected experts' p (each lane looks its own experts up), sum_i p_i and sum_i dw_i w_i
  float ssum = 0.f, dww = 0.f;
  for (int j = 0; j < k; ++j) {
    const int e = topk_idx[(size_t)t * k + j];
    float pj = 0.f;
#pragma unroll
    for (int m = 0; m < EL; ++m)
      if (lane + kWave * m == e) pj = pe[m];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) pj += __shfl_xor(pj, o, kWave);
    ssum += pj;
    dww += dw[(size_t)t * k + j] * topk_w[(size_t)t * k + j];
  }
  float dp[EL];
#pragma unroll
  for (int m = 0; m < EL; ++m) {
    const int e = lane + kWave * m;
    dp[m] = (e < E && counts) ? aux_scale * (float)counts[e] : 0.f;
  }
  for (int j = 0; j < k; ++j) {
    const int e = topk_idx[(size_t)t * k + j];
    const float dwj = dw[(size_t)t * k + j];
    const float ds = renorm ? (dwj - dww) / ssum : dwj;
#pragma unroll
    for (int m = 0; m < EL; ++m)
      if (lane + kWave * m == e) dp[m] += ds;
  }
  float dot = 0.f;
#pragma unroll
  for (int m = 0; m < EL; ++m) dot += dp[m] * pe[m];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) dot += __shfl_xor(dot, o, kWave);
#pragma unroll
  for (int m = 0; m < EL; ++m) {
    const int e = lane + kWave * m;
    if (e < E) dl[(size_t)t * E + e] = pe[m] * (dp[m] - dot);
  }
}

// Router weight gradient, first pass: part[z][e][c] = sum over the tokens t of
// chunk z (in order) of dl[t][e] x[t][c]. A workgroup takes EB experts and kT
// columns (one per thread, EB fp32 accumulators) over one chunk, staging 64
// tokens of dl at a time in LDS (read back as broadcasts).
constexpr int kRT = 64;  // tokens per LDS stage
template <int EB>
__global__ __launch_bounds__(kT) void router_wgrad_part_kernel(const float* __restrict__ dl,
                                                               const bf16_t* __restrict__ x, int N, int E, int d,
                                                               int chunk, float* __restrict__ part) {
  __shared__ __align__(16) float s_dl[kRT][EB];
  const int c = blockIdx.x * kT + threadIdx.x;
  const int e0 = blockIdx.y * EB;
  const int t0 = blockIdx.z * chunk, t1 = min(N, t0 + chunk);
  float acc[EB];
#pragma unroll
  for (int q = 0; q < EB; ++q) acc[q] = 0.f;
  for (int tb = t0; tb < t1; tb += kRT) {
    const int nt = min(kRT, t1 - tb);
    for (int i = threadIdx.x; i < kRT * EB; i += kT) {
      const int tt = i / EB, ee = i % EB;
      s_dl[tt][ee] = (tt < nt && e0 + ee < E) ? dl[(size_t)(tb + tt) * E + e0 + ee] : 0.f;
    }
    __syncthreads();
    if (c < d) {
      for (int tt = 0; tt < nt; ++tt) {
        const float xv = bf(x[(size_t)(tb + tt) * d + c]);
#pragma unroll
        for (int q = 0; q < EB; q += 4) {
          const float4 g = *reinterpret_cast<const float4*>(&s_dl[tt][q]);
          acc[q] += g.x * xv;
          acc[q + 1] += g.y * xv;
          acc[q + 2] += g.z * xv;
          acc[q + 3] += g.w * xv;
        }
      }
    }
    __syncthreads();
  }
  if (c >= d) return;
#pragma unroll
  for (int q = 0; q < EB; ++q)
    if (e0 + q < E) part[((size_t)blockIdx.z * E + e0 + q) * d + c] = acc[q];
}

// Second pass: dW_r[e][c] = sum_z part[z][e][c], z in order (added to dW_r when accumulating).
__global__ __launch_bounds__(kT) void router_wgrad_reduce_kernel(const float* __restrict__ part, int Z, size_t n,
                                                                 int accumulate, float* __restrict__ dwr) {
  const size_t i = (size_t)blockIdx.x * kT + threadIdx.x;
  if (i >= n) return;
  float acc = 0.f;
  for (int z = 0; z < Z; ++z) acc += part[(size_t)z * n + i];
  dwr[i] = accumulate ? dwr[i] + acc : acc;
}

// d_logit_bias[e] = sum_t dl[t][e]: one workgroup per expert, a strided sum per
// thread and a fixed tree over the threads.
__global__ __launch_bounds__(kT) void logit_bias_grad_kernel(const float* __restrict__ dl, int N, int E,
                                                             int accumulate, float* __restrict__ dlb) {
  __shared__ float s_part[kT];
  const int e = blockIdx.x;
  float acc = 0.f;
  for (int t = threadIdx.x; t < N; t += kT) acc += dl[(size_t)t * E + e];
  s_part[threadIdx.x] = acc;
  __syncthreads();
  for (int st = kT / 2; st > 0; st >>= 1) {
    if (threadIdx.x < st) s_part[threadIdx.x] += s_part[threadIdx.x + st];
    __syncthreads();
  }
  if (threadIdx.x == 0) dlb[e] = accumulate ? dlb[e] + s_part[0] : s_part[0];
}

// dx[t][c] = (sum_j dXr[slot_pos[t*k + j]][c] over the kept copies, j in order,
//             + sum_s dXs[s*N + t][c]) + sum_e dl[t][e] W_r[e][c] (e in order).
// A workgroup takes 64 tokens and kT columns (one per thread, 64 fp32 router
// accumulators); dl is staged 64 experts at a time in LDS, transposed, and read
// back as broadcasts.
constexpr int kXT = 64;   // tokens per workgroup
constexpr int kXE = 64;   // experts per LDS stage
constexpr int kXP = kXT + 4;  // LDS row pitch (floats): 16-byte aligned rows
// With rterm (the router term dl W_r already computed, [N, d]), the expert loop is skipped.
__global__ __launch_bounds__(kT) void dx_kernel(const float* __restrict__ dXr, const int32_t* __restrict__ slot_pos,
                                                const float* __restrict__ dXs, int S, const float* __restrict__ dl,
                                                const bf16_t* __restrict__ wr, const float* __restrict__ rterm,
                                                int N, int E, int k, int d, float* __restrict__ dx) {
  __shared__ __align__(16) float s_dl[kXE][kXP];
  const int c = blockIdx.x * kT + threadIdx.x;
  const int t0 = blockIdx.y * kXT;
  const int nt = min(kXT, N - t0);
  float acc[kXT];
#pragma unroll
  for (int q = 0; q < kXT; ++q) acc[q] = 0.f;
  for (int e0 = 0; e0 < (rterm ? 0 : E); e0 += kXE) {
    const int ne = min(kXE, E - e0);
    for (int i = threadIdx.x; i < kXT * kXE; i += kT) {
      const int tt = i / kXE, ee = i % kXE;
      s_dl[ee][tt] = (tt < nt && ee < ne) ? dl[(size_t)(t0 + tt) * E + e0 + ee] : 0.f;
    }
    __syncthreads();
    if (c < d) {
      for (int ee = 0; ee < ne; ++ee) {
        const float w = bf(wr[(size_t)(e0 + ee) * d + c]);
#pragma unroll
        for (int q = 0; q < kXT; q += 4) {
          const float4 g = *reinterpret_cast<const float4*>(&s_dl[ee][q]);
          acc[q] += g.x * w;
          acc[q + 1] += g.y * w;
          acc[q + 2] += g.z * w;
          acc[q + 3] += g.w * w;
        }
      }
    }
    __syncthreads();
  }
  if (c >= d) return;
#pragma unroll
  for (int q = 0; q < kXT; ++q) {
    if (q < nt) {
      const int t = t0 + q;
      float sum = 0.f;
      for (int j = 0; j < k; ++j) {
        const int r = slot_pos[(size_t)t * k + j];
        if (r >= 0) sum += dXr[(size_t)r * d + c];
      }
      for (int s2 = 0; s2 < S; ++s2) sum += dXs[((size_t)s2 * N + t) * d + c];
      dx[(size_t)t * d + c] = sum + (rterm ? rterm[(size_t)t * d + c] : acc[q]);
    }
  }
}

// Splits dl [N, E] (fp32) into bf16 parts hi = bf16(dl), lo = bf16(dl - hi), so that
// hi + lo equals dl to about 2^-16 relative: the router products then run as bf16
// matrix-core GEMMs on exact bf16 W_r and x. Writes dlh [N, 2E] (row t: hi | lo) and
// its transpose dlT [E, 2N] (row e: hi | lo). One 64 x 64 tile per workgroup through
// LDS (partial edge tiles are checked element by element).
__global__ __launch_bounds__(kT) void split_hilo_kernel(const float* __restrict__ dl, int N, int E,
                                                        bf16_t* __restrict__ dlh, bf16_t* __restrict__ dlT) {
  __shared__ uint16_t th[64][kTP], tl[64][kTP];
  const int t0 = blockIdx.y * 64, e0 = blockIdx.x * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += kT) {
    const int tt = i / 64, ee = i % 64, t = t0 + tt, e = e0 + ee;
    if (t < N && e < E) {
      const float v = dl[(size_t)t * E + e];
      const bf16_t h = f32_to_bf16(v), l = f32_to_bf16(v - bf(h));
      dlh[(size_t)t * 2 * E + e] = h;
      dlh[(size_t)t * 2 * E + E + e] = l;
      th[tt][ee] = h;
      tl[tt][ee] = l;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += kT) {
    const int ee = i / 64, tt = i % 64, t = t0 + tt, e = e0 + ee;
    if (t < N && e < E) {
      dlT[(size_t)e * 2 * N + t] = th[tt][ee];
      dlT[(size_t)e * 2 * N + N + t] = tl[tt][ee];
    }
  }
}

// dx[t][c] = (sum_j dXr[slot_pos[t*k + j]][c] over the kept copies, j in order
//            + sum_s dXs[s*N + t][c]) + rterm[t][c], the router term already computed:
// the same sums as dx_kernel, four columns per thread (d is a multiple of 4).
__global__ __launch_bounds__(kT) void dx_gather_kernel(const float* __restrict__ dXr,
                                                       const int32_t* __restrict__ slot_pos,
                                                       const float* __restrict__ dXs, int S,
                                                       const float* __restrict__ rterm, int N, int k, int d,
                                                       float* __restrict__ dx) {
  const int t = blockIdx.y;
  const int c = (blockIdx.x * kT + threadIdx.x) * 4;
  if (c >= d) return;
  float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const int r = slot_pos[(size_t)t * k + j];
    if (r >= 0) {
      const float4 v = *reinterpret_cast<const float4*>(dXr + (size_t)r * d + c);
      sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
    }
  }
  for (int s2 = 0; s2 < S; ++s2) {
    const float4 v = *reinterpret_cast<const float4*>(dXs + ((size_t)s2 * N + t) * d + c);
    sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
  }
  const float4 rr = *reinterpret_cast<const float4*>(rterm + (size_t)t * d + c);
  *reinterpret_cast<float4*>(dx + (size_t)t * d + c) = make_float4(sum.x + rr.x, sum.y + rr.y, sum.z + rr.z,
                                                                  sum.w + rr.w);
}

__global__ void fill_f32_kernel(float* p, size_t n, float v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

// Workgroup (b, g): slice b of group g's output block, when K_g = 0.
__global__ void zero_empty_groups_kernel(uint4* out, const int32_t* __restrict__ kofs, size_t n16) {
  const int g = blockIdx.y;
  if (kofs[g + 1] != kofs[g]) return;
  uint4* p = out + (size_t)g * n16;
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x) p[i] = z;
}

}  // namespace

int launch_gather_rows(const void* x, const float* dy, const float* topk_w, const int32_t* perm,
                       const int32_t* n_valid, int k, int d, int rows, void* Xg, void* dYg, void* dO, hipStream_t st) {
  if (rows <= 0) return MOE_OK;
  if (d % 8) return MOE_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(rows), dim3(kT), 0, st, static_cast<const bf16_t*>(x), dy, topk_w,
                     perm, n_valid, k, d, static_cast<bf16_t*>(Xg), static_cast<bf16_t*>(dYg),
                     static_cast<bf16_t*>(dO));
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int launch_swiglu_backward(const float* G, const float* U, const float* dHp, const float* topk_w,
                           const int32_t* perm, const int32_t* n_valid, int rows, int F, void* h, void* dGU,
                           float* dw, hipStream_t st) {
  if (rows <= 0) return MOE_OK;
  hipLaunchKernelGGL(swiglu_backward_kernel, dim3(rows), dim3(kT), 0, st, G, U, dHp, topk_w, perm, n_valid, F,
                     static_cast<bf16_t*>(h), static_cast<bf16_t*>(dGU), dw);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int launch_k_offsets(const int32_t* offsets, int G, int uniform, int32_t* kofs, hipStream_t st) {
  hipLaunchKernelGGL(k_offsets_kernel, dim3(1), dim3(kWave), 0, st, offsets, G, uniform, kofs);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int launch_transpose_padded(const void* in, int in_stride, int col_off, int C, const int32_t* offsets, int uniform,
                            int replicate, const int32_t* kofs, int G, void* out, int kmax, hipStream_t st) {
  if (C <= 0 || kmax <= 0) return MOE_OK;
  if (in_stride % 8 || col_off % 8 || C % 8 || kmax % 64) return MOE_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(transpose_padded_kernel, dim3(kmax / 64, (C + 63) / 64), dim3(kT), 0, st,
                     static_cast<const bf16_t*>(in), in_stride, col_off, C, offsets, uniform, replicate, kofs, G,
                     static_cast<bf16_t*>(out));
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int launch_router_backward(const moe_shape& s, const float* logits, int splits, const float* logit_bias,
                           const int32_t* topk_idx, const float* topk_w, const float* dw, const int32_t* counts,
                           double aux_coef, float* dl, hipStream_t st) {
  const int N = s.n_tokens, E = s.n_experts, k = s.top_k;
  // aux_coef * E * f_e / N with f_e = counts_e / (N k)
  const float aux_scale = (float)(aux_coef * E / ((double)N * k * N));
  const int el = (E + kWave - 1) / kWave;
  const dim3 grid((N + kT / kWave - 1) / (kT / kWave));
#define MOE_RB(EL_)                                                                                          \
  hipLaunchKernelGGL(router_backward_kernel<EL_>, grid, dim3(kT), 0, st, logits, splits, logit_bias, topk_idx, \
                     topk_w, dw, aux_coef != 0.0 ? counts : nullptr, aux_scale, N, E, k, s.renormalize, dl)
  if (el <= 1) MOE_RB(1);
  else if (el <= 2) MOE_RB(2);
  else if (el <= 4) MOE_RB(4);
  else MOE_RB(8);
#undef MOE_RB
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int router_wgrad_splits(int N) { return std::max(1, std::min(64, N / 256)); }

size_t router_wgrad_part_floats(int N, int E, int d) { return (size_t)router_wgrad_splits(N) * E * d; }

int launch_router_wgrad(const float* dl, const void* x, int N, int E, int d, float* part, float* dwr, float* dlb,
                        int accumulate, hipStream_t st) {
  const int Z = router_wgrad_splits(N);
  const int chunk = (N + Z - 1) / Z;
  const int eb = E <= 8 ? 8 : E <= 16 ? 16 : E <= 32 ? 32 : 64;
  const dim3 grid((d + kT - 1) / kT, (E + eb - 1) / eb, Z);
#define MOE_RW(EB_)                                                                                              \
  hipLaunchKernelGGL(router_wgrad_part_kernel<EB_>, grid, dim3(kT), 0, st, dl, static_cast<const bf16_t*>(x), N, E, \
                     d, chunk, part)
  if (eb == 8) MOE_RW(8);
  else if (eb == 16) MOE_RW(16);
  else if (eb == 32) MOE_RW(32);
  else MOE_RW(64);
#undef MOE_RW
  const size_t n = (size_t)E * d;
  hipLaunchKernelGGL(router_wgrad_reduce_kernel, dim3((unsigned)((n + kT - 1) / kT)), dim3(kT), 0, st, part, Z, n,
                     accumulate, dwr);
  if (dlb) hipLaunchKernelGGL(logit_bias_grad_kernel, dim3(E), dim3(kT), 0, st, dl, N, E, accumulate, dlb);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int launch_dx(const float* dXr, const int32_t* slot_pos, const float* dXs, int S, const float* dl, const void* wr,
              const float* rterm, int N, int E, int k, int d, float* dx, hipStream_t st) {
  if (N <= 0) return MOE_OK;
  if (rterm && d % 4 == 0) {
    hipLaunchKernelGGL(dx_gather_kernel, dim3((d / 4 + kT - 1) / kT, N), dim3(kT), 0, st, dXr, slot_pos, dXs, S,
                       rterm, N, k, d, dx);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
  }
  hipLaunchKernelGGL(dx_kernel, dim3((d + kT - 1) / kT, (N + kXT - 1) / kXT), dim3(kT), 0, st, dXr, slot_pos, dXs, S,
                     dl, static_cast<const bf16_t*>(wr), rterm, N, E, k, d, dx);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int launch_logit_bias_grad(const float* dl, int N, int E, float* dlb, int accumulate, hipStream_t st) {
  if (!dlb || E <= 0) return MOE_OK;
  hipLaunchKernelGGL(logit_bias_grad_kernel, dim3(E), dim3(kT), 0, st, dl, N, E, accumulate, dlb);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int launch_split_hilo(const float* dl, int N, int E, void* dlh, void* dlT, hipStream_t st) {
  if (N <= 0 || E <= 0) return MOE_OK;
  hipLaunchKernelGGL(split_hilo_kernel, dim3((E + 63) / 64, (N + 63) / 64), dim3(kT), 0, st, dl, N, E,
                     static_cast<bf16_t*>(dlh), static_cast<bf16_t*>(dlT));
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int launch_zero_empty_groups(void* out, const int32_t* kofs, int G, size_t block_bytes, hipStream_t st) {
  if (G <= 0 || block_bytes == 0) return MOE_OK;
  if (block_bytes % 16) return MOE_ERR_UNSUPPORTED;
  const size_t n16 = block_bytes / 16;
  const int nb = (int)std::min<size_t>(64, (n16 + kT - 1) / kT);
  hipLaunchKernelGGL(zero_empty_groups_kernel, dim3(nb, G), dim3(kT), 0, st, static_cast<uint4*>(out), kofs, n16);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int launch_fill_f32(float* p, size_t n, float v, hipStream_t st) {
  if (n == 0) return MOE_OK;
  hipLaunchKernelGGL(fill_f32_kernel, dim3(1024), dim3(kT), 0, st, p, n, v);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
