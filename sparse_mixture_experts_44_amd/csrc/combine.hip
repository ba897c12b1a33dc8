// Weighted combine back to token order: the output formula of section "结构"
// of "混合专家 MoE" (anrans ai-infra handbook), which forward_grouped
// computes with index_add_.
//
// This is a gather instead of atomics. Workgroup (t, c) sums a 1024-column
// slice of token t: its k expert rows (through slot_pos), then its
// shared-expert rows. They are added in a fixed order (slot 0 .. k-1, then
// shared 0 .. S-1) and y is written once with 16-byte stores. The result is
// bit-reproducible. A dropped copy (slot_pos -1) adds nothing, and a row with
// nothing to add is exactly +0. The rows of one batch of slots are loaded
// together before they are added, so the loads overlap.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kBatch = 8;  // slots loaded together

__global__ __launch_bounds__(kThreads) void combine_kernel(const float4* __restrict__ O,
                                                           const int32_t* __restrict__ slot_pos,
                                                           const float* __restrict__ w,
                                                           const float4* __restrict__ shared, int S,
                                                           int N, int d4, int k, float4* __restrict__ y) {
  __shared__ int32_t s_slot[kMaxTopK];
  __shared__ float s_w[kMaxTopK];
  const int t = blockIdx.x;
  if (threadIdx.x < k) {
    s_slot[threadIdx.x] = slot_pos[(size_t)t * k + threadIdx.x];
    s_w[threadIdx.x] = w[(size_t)t * k + threadIdx.x];
  }
  __syncthreads();
  const int c = blockIdx.y * kThreads + threadIdx.x;
  if (c >= d4) return;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j0 = 0; j0 < k; j0 += kBatch) {
    float4 o[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int sp = j0 + u < k ? s_slot[j0 + u] : -1;
      o[u] = sp >= 0 ? O[(size_t)sp * d4 + c] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (j0 + u >= k || s_slot[j0 + u] < 0) continue;
      const float wj = s_w[j0 + u];
      a.x = fmaf(wj, o[u].x, a.x);
      a.y = fmaf(wj, o[u].y, a.y);
      a.z = fmaf(wj, o[u].z, a.z);
      a.w = fmaf(wj, o[u].w, a.w);
    }
  }
  for (int s = 0; s < S; ++s) {
    const float4 o = shared[((size_t)s * N + t) * d4 + c];
    a.x += o.x;
    a.y += o.y;
    a.z += o.z;
    a.w += o.w;
  }
  y[(size_t)t * d4 + c] = a;
}

}  // namespace

int launch_combine(const moe_shape& s, const float* expert_out, const int32_t* slot_pos,
                   const float* topk_w, const float* shared_out, float* y, hipStream_t stream) {
  if (s.n_tokens == 0) return MOE_OK;
  const int d4 = s.d_model / 4;
  hipLaunchKernelGGL(combine_kernel, dim3(s.n_tokens, (d4 + kThreads - 1) / kThreads), dim3(kThreads), 0, stream,
                     reinterpret_cast<const float4*>(expert_out), slot_pos, topk_w,
                     reinterpret_cast<const float4*>(shared_out), shared_out ? s.n_shared : 0,
                     s.n_tokens, s.d_model / 4, s.top_k, reinterpret_cast<float4*>(y));
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
