// Weighted combine back to token order: the output formula of section "结构"
// of "混合专家 MoE" (anrans ai-infra handbook), which forward_grouped
// computes with index_add_.
//
// This is a gather instead of atomics. A workgroup sums a 1024-column slice
// of one token (or of four, one after another, for large top-1 layers): its
// k expert rows (through slot_pos), then its shared-expert rows. They are
// added in a fixed order (slot 0 .. k-1, then shared 0 .. S-1) and y is
// written once with 16-byte stores. The result is
// bit-reproducible. A dropped copy (slot_pos -1) adds nothing, and a row with
// nothing to add is exactly +0. The rows of one batch of slots, and the first
// shared-expert row, are loaded together before they are added, so the loads
// overlap; every row is read once, with non-temporal loads.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kBatch = 8;  // slots loaded together

typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 load_nt(const float4* p) {
  const f32x4v v = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

// Workgroup (b, c): tokens TPW*b .. TPW*b + TPW-1, one after another, over
// column slice c. Several tokens per workgroup amortise its set-up over more
// rows when there are many tokens.
template <int TPW>
__global__ __launch_bounds__(kThreads) void combine_kernel(const float4* __restrict__ O,
                                                           const int32_t* __restrict__ slot_pos,
                                                           const float* __restrict__ w,
                                                           const float4* __restrict__ shared, int S,
                                                           int N, int d4, int k, float4* __restrict__ y) {
  __shared__ int32_t s_slot[TPW][kMaxTopK];
  __shared__ float s_w[TPW][kMaxTopK];
  const int t0 = blockIdx.x * TPW;
  for (int i = threadIdx.x; i < TPW * k; i += kThreads) {
    const int u = i / k, j = i - u * k;
    const bool in = t0 + u < N;
    s_slot[u][j] = in ? slot_pos[(size_t)(t0 + u) * k + j] : -1;
    s_w[u][j] = in ? w[(size_t)(t0 + u) * k + j] : 0.f;
  }
  __syncthreads();
  const int c = blockIdx.y * kThreads + threadIdx.x;
  if (c >= d4) return;
  for (int tu = 0; tu < TPW; ++tu) {
    const int t = t0 + tu;
    if (t >= N) break;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 sh0 = S > 0 ? load_nt(&shared[(size_t)t * d4 + c]) : a;
    for (int j0 = 0; j0 < k; j0 += kBatch) {
      float4 o[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int sp = j0 + u < k ? s_slot[tu][j0 + u] : -1;
        o[u] = sp >= 0 ? load_nt(&O[(size_t)sp * d4 + c]) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (j0 + u >= k || s_slot[tu][j0 + u] < 0) continue;
        const float wj = s_w[tu][j0 + u];
        a.x = fmaf(wj, o[u].x, a.x);
        a.y = fmaf(wj, o[u].y, a.y);
        a.z = fmaf(wj, o[u].z, a.z);
        a.w = fmaf(wj, o[u].w, a.w);
      }
    }
    for (int s = 0; s < S; ++s) {
      const float4 o = s == 0 ? sh0 : load_nt(&shared[((size_t)s * N + t) * d4 + c]);
      a.x += o.x;
      a.y += o.y;
      a.z += o.z;
      a.w += o.w;
    }
    y[(size_t)t * d4 + c] = a;
  }
}

}  // namespace

int launch_combine(const moe_shape& s, const float* expert_out, const int32_t* slot_pos,
                   const float* topk_w, const float* shared_out, float* y, hipStream_t stream) {
  if (s.n_tokens == 0) return MOE_OK;
  const int d4 = s.d_model / 4;
  const int gy = (d4 + kThreads - 1) / kThreads;  // column slices
  const float4* O4 = reinterpret_cast<const float4*>(expert_out);
  const float4* sh4 = reinterpret_cast<const float4*>(shared_out);
  const int S = shared_out ? s.n_shared : 0;
  float4* y4 = reinterpret_cast<float4*>(y);
  // four tokens per workgroup where a token has at most two rows to add (a top-1 layer):
  // Switch-shaped combine 36 -> 34 us; with more rows per token one token per workgroup
  // keeps more loads in flight (DeepSeek-shaped: 0.41 against 0.42 ms)
  if (s.n_tokens >= 4096 && s.top_k + S <= 2)
    hipLaunchKernelGGL(combine_kernel<4>, dim3((s.n_tokens + 3) / 4, gy), dim3(kThreads), 0, stream, O4,
                       slot_pos, topk_w, sh4, S, s.n_tokens, d4, s.top_k, y4);
  else
    hipLaunchKernelGGL(combine_kernel<1>, dim3(s.n_tokens, gy), dim3(kThreads), 0, stream, O4, slot_pos,
                       topk_w, sh4, S, s.n_tokens, d4, s.top_k, y4);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
