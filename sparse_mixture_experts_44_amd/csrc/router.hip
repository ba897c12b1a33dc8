// Router of the MoE layer: logits = x W_r^T (+ logit bias), softmax, the
// selection-only bias, top-k, renormalisation, and per-expert probability
// sums. This is route() of "混合专家 MoE" (anrans ai-infra handbook), section
// "实现：逐 token 与按专家分组". The bias for selection only is the
// aux-loss-free balancing of its section "负载均衡".
//
// One workgroup takes 32 tokens and every expert.
//
// Logits: a VALU GEMM. The matrix cores are kept for the expert GEMMs.
//   - The K dimension is staged through LDS in chunks of 128 bytes per row.
//     Rows are padded to 144 bytes, so 16-byte reads from consecutive rows
//     fall in different banks.
//   - Each thread owns 4 tokens x EPT experts. bf16 uses v_dot2_f32_bf16,
//     two products per instruction with fp32 accumulation.
//   - Each chunk is summed into a fresh partial, which is then added to the
//     running sum. This keeps the fp32 rounding of long rows small.
//
// Softmax and top-k: one wavefront per token.
//   - Each lane holds E/64 scores.
//   - Max and sum use butterfly reductions, whose order is fixed.
//   - Top-k runs k rounds of a wave arg-max. A larger score wins; on equal
//     scores the lower expert index wins.
//
// Probability sums: p is added into fp64 per-wave partials, then the waves
// are combined in a fixed order. A second kernel adds the workgroup rows in
// workgroup order. So prob_sum is bit-reproducible.
#include <math.h>

#include "moe_common.h"

namespace moe {
namespace {

constexpr int kTok = 32;          // tokens per workgroup
constexpr int kThreads = 256;
constexpr int kChunk = 32;        // dwords per row chunk: 64 bf16 or 32 fp32
constexpr int kRow = kChunk + 4;  // padded LDS row stride in dwords

template <bool BF16>
__device__ __forceinline__ float mac(uint32_t a, uint32_t b, float c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
  } else {
    return fmaf(__uint_as_float(a), __uint_as_float(b), c);
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

template <bool BF16, int EPT>
__global__ __launch_bounds__(kThreads) void router_kernel(
    const uint32_t* __restrict__ x, const uint32_t* __restrict__ w,
    const float* __restrict__ logit_bias, const float* __restrict__ select_bias, int N,
    int dw, int E, int k, int renorm, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, double* __restrict__ partials) {
  constexpr int EROWS = 32 * EPT;                 // expert rows covered by the thread grid
  constexpr int EL = (EROWS + kWave - 1) / kWave;  // experts per lane in the softmax phase
  constexpr int LROW = EROWS + 1;                 // logits row stride (floats)
  static_assert(kTok * LROW <= EROWS * kRow, "logits must fit in the W staging area");
  __shared__ uint32_t s_w[EROWS * kRow];
  __shared__ uint32_t s_x[kTok * kRow];
  __shared__ double s_part[kThreads / kWave][EROWS];

  const int tid = threadIdx.x;
  const int eg = tid & 31;   // expert group: experts eg + 32 j
  const int tg = tid >> 5;   // token group: tokens tg + 8 i
  const int t0 = blockIdx.x * kTok;

  float acc[4][EPT];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < EPT; ++j) acc[i][j] = 0.f;

  u32x4_t px;
  u32x4_t pw[EPT];
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  auto load_chunk = [&](int kc) {
    const int r = tid >> 3, pc = tid & 7;
    const int t = t0 + r;
    px = (t < N) ? *reinterpret_cast<const u32x4_t*>(x + (size_t)t * dw + kc + pc * 4) : zero;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int piece = tid + kThreads * j;
      const int er = piece >> 3, epc = piece & 7;
      pw[j] = (er < E) ? *reinterpret_cast<const u32x4_t*>(w + (size_t)er * dw + kc + epc * 4) : zero;
    }
  };

  load_chunk(0);
  for (int kc = 0; kc < dw; kc += kChunk) {
    __syncthreads();  // everyone finished reading the previous chunk
    *reinterpret_cast<u32x4_t*>(s_x + (tid >> 3) * kRow + (tid & 7) * 4) = px;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int piece = tid + kThreads * j;
      *reinterpret_cast<u32x4_t*>(s_w + (piece >> 3) * kRow + (piece & 7) * 4) = pw[j];
    }
    __syncthreads();
    if (kc + kChunk < dw) load_chunk(kc + kChunk);
    float part[4][EPT];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < EPT; ++j) part[i][j] = 0.f;
#pragma unroll
    for (int q = 0; q < kChunk / 4; ++q) {
      u32x4_t xv[4], wv[EPT];
#pragma unroll
      for (int i = 0; i < 4; ++i) xv[i] = *reinterpret_cast<const u32x4_t*>(s_x + (tg + 8 * i) * kRow + q * 4);
#pragma unroll
      for (int j = 0; j < EPT; ++j) wv[j] = *reinterpret_cast<const u32x4_t*>(s_w + (eg + 32 * j) * kRow + q * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
          float a = part[i][j];
          a = mac<BF16>(xv[i].x, wv[j].x, a);
          a = mac<BF16>(xv[i].y, wv[j].y, a);
          a = mac<BF16>(xv[i].z, wv[j].z, a);
          a = mac<BF16>(xv[i].w, wv[j].w, a);
          part[i][j] = a;
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < EPT; ++j) acc[i][j] += part[i][j];
  }

  // ---- logits to LDS (reusing the W staging area)
  __syncthreads();
  float* s_log = reinterpret_cast<float*>(s_w);
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = eg + 32 * j;
    if (e < E) {
      const float lb = logit_bias ? logit_bias[e] : 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) s_log[(tg + 8 * i) * LROW + e] = acc[i][j] + lb;
    }
  }
  __syncthreads();

  // ---- softmax, selection score, top-k, renormalise: one wavefront per token
  const int wv = tid >> 6, lane = tid & 63;
  double pacc[EL];
  float sb[EL];
#pragma unroll
  for (int m = 0; m < EL; ++m) {
    const int e = lane + kWave * m;
    pacc[m] = 0.0;
    sb[m] = (select_bias && e < E) ? select_bias[e] : 0.f;
  }
  for (int tt = wv; tt < kTok; tt += kThreads / kWave) {
    const int t = t0 + tt;
    if (t >= N) break;
    float v[EL], p[EL], s[EL];
    float mx = -INFINITY;
#pragma unroll
    for (int m = 0; m < EL; ++m) {
      const int e = lane + kWave * m;
      v[m] = (e < E) ? s_log[tt * LROW + e] : -INFINITY;
      mx = fmaxf(mx, v[m]);
    }
    mx = wave_max(mx);
    float sum = 0.f;
#pragma unroll
    for (int m = 0; m < EL; ++m) {
      const int e = lane + kWave * m;
      v[m] = (e < E) ? expf(v[m] - mx) : 0.f;
      sum += v[m];
    }
    sum = wave_sum(sum);
#pragma unroll
    for (int m = 0; m < EL; ++m) {
      p[m] = v[m] / sum;
      pacc[m] += (double)p[m];
      s[m] = p[m] + sb[m];
    }
    uint32_t taken = 0;
    float sel_sum = 0.f, mine_p = 0.f;
    int mine_idx = -1;
    for (int j = 0; j < k; ++j) {
      float bv = -INFINITY, bp = 0.f;
      int bi = 0x7fffffff;
#pragma unroll
      for (int m = 0; m < EL; ++m) {
        const int e = lane + kWave * m;
        if (e < E && !((taken >> m) & 1u) && (s[m] > bv || (s[m] == bv && e < bi))) {
          bv = s[m];
          bi = e;
          bp = p[m];
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, kWave);
        const int oi = __shfl_xor(bi, o, kWave);
        const float op = __shfl_xor(bp, o, kWave);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
          bp = op;
        }
      }
      if (bi < E && (bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
      if (lane == j) {
        mine_idx = bi < E ? bi : -1;
        mine_p = bp;
      }
      sel_sum += bp;
    }
    if (lane < k) {
      topk_idx[(size_t)t * k + lane] = mine_idx;
      topk_w[(size_t)t * k + lane] = renorm ? mine_p / sel_sum : mine_p;
    }
  }

  // ---- per-workgroup probability sums, waves combined in a fixed order
#pragma unroll
  for (int m = 0; m < EL; ++m) {
    const int e = lane + kWave * m;
    if (e < EROWS) s_part[wv][e] = pacc[m];
  }
  __syncthreads();
  for (int e = tid; e < E; e += kThreads) {
    double a = s_part[0][e];
#pragma unroll
    for (int q = 1; q < kThreads / kWave; ++q) a += s_part[q][e];
    partials[(size_t)blockIdx.x * E + e] = a;
  }
}

// prob_sum[e] = sum over workgroups b (in order) of partials[b][e].
__global__ __launch_bounds__(256) void prob_sum_kernel(const double* __restrict__ partials, int nb,
                                                       int E, double* __restrict__ prob_sum) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  double a = 0.0;
  for (int b = 0; b < nb; ++b) a += partials[(size_t)b * E + e];
  prob_sum[e] = a;
}

template <bool BF16, int EPT>
void launch_router_t(const moe_shape& s, const void* x, const void* w, const float* lb,
                     const float* sb, int32_t* idx, float* tw, double* partials, hipStream_t st) {
  const int nb = route_blocks(s);
  const int dw = BF16 ? s.d_model / 2 : s.d_model;
  hipLaunchKernelGGL((router_kernel<BF16, EPT>), dim3(nb), dim3(kThreads), 0, st,
                     static_cast<const uint32_t*>(x), static_cast<const uint32_t*>(w), lb, sb,
                     s.n_tokens, dw, s.n_experts, s.top_k, s.renormalize, idx, tw, partials);
}

template <bool BF16>
void launch_router_e(const moe_shape& s, const void* x, const void* w, const float* lb,
                     const float* sb, int32_t* idx, float* tw, double* partials, hipStream_t st) {
  const int need = (s.n_experts + 31) / 32;
  if (need <= 1) launch_router_t<BF16, 1>(s, x, w, lb, sb, idx, tw, partials, st);
  else if (need <= 2) launch_router_t<BF16, 2>(s, x, w, lb, sb, idx, tw, partials, st);
  else if (need <= 4) launch_router_t<BF16, 4>(s, x, w, lb, sb, idx, tw, partials, st);
  else if (need <= 8) launch_router_t<BF16, 8>(s, x, w, lb, sb, idx, tw, partials, st);
  else launch_router_t<BF16, 16>(s, x, w, lb, sb, idx, tw, partials, st);
}

}  // namespace

int route_blocks(const moe_shape& s) { return (s.n_tokens + kTok - 1) / kTok; }

int launch_route(const moe_shape& s, const void* x, const void* w_router, const float* logit_bias,
                 const float* select_bias, int32_t* topk_idx, float* topk_w, double* prob_sum,
                 double* partials, hipStream_t stream) {
  if (s.dtype == MOE_DTYPE_BF16)
    launch_router_e<true>(s, x, w_router, logit_bias, select_bias, topk_idx, topk_w, partials, stream);
  else
    launch_router_e<false>(s, x, w_router, logit_bias, select_bias, topk_idx, topk_w, partials, stream);
  hipLaunchKernelGGL(prob_sum_kernel, dim3((s.n_experts + 255) / 256), dim3(256), 0, stream,
                     partials, route_blocks(s), s.n_experts, prob_sum);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
