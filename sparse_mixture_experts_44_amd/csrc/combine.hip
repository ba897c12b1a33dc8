// Weighted combine back to token order: the output formula of section "结构"
// of "混合专家 MoE" (anrans ai-infra handbook), which forward_grouped
// computes with index_add_.
//
// This is a gather instead of atomics. One workgroup per token reads its k
// expert rows (through slot_pos) and its shared-expert rows. It adds them in
// a fixed order (slot 0 .. k-1, then shared 0 .. S-1) and writes y once with
// 16-byte stores. The result is bit-reproducible. A dropped copy
// (slot_pos -1) adds nothing, and a row with nothing to add is exactly +0.
#include "moe_common.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void combine_kernel(const float4* __restrict__ O,
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
  for (int c = threadIdx.x; c < d4; c += blockDim.x) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const int sp = s_slot[j];
      if (sp < 0) continue;
      const float4 o = O[(size_t)sp * d4 + c];
      const float wj = s_w[j];
      a.x = fmaf(wj, o.x, a.x);
      a.y = fmaf(wj, o.y, a.y);
      a.z = fmaf(wj, o.z, a.z);
      a.w = fmaf(wj, o.w, a.w);
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
}

}  // namespace

int launch_combine(const moe_shape& s, const float* expert_out, const int32_t* slot_pos,
                   const float* topk_w, const float* shared_out, float* y, hipStream_t stream) {
  if (s.n_tokens == 0) return MOE_OK;
  hipLaunchKernelGGL(combine_kernel, dim3(s.n_tokens), dim3(256), 0, stream,
                     reinterpret_cast<const float4*>(expert_out), slot_pos, topk_w,
                     reinterpret_cast<const float4*>(shared_out), shared_out ? s.n_shared : 0,
                     s.n_tokens, s.d_model / 4, s.top_k, reinterpret_cast<float4*>(y));
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
