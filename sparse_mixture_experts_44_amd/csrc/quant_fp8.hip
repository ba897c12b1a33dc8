// FP8 (E4M3) expert weights for the W8A16 variant of the grouped SwiGLU.
//
// The handbook "混合专家 MoE" (anrans ai-infra handbook), section "推理视角",
// notes that DeepSeek-V3 ships its weights in FP8 and that decode time is
// the time to read the touched experts' weights. It names no format and no
// scale granularity. This library reads them as: OCP E4M3 (e4m3fn, exponent
// bias 7, largest value 448, no infinities), with one fp32 scale per output
// row of each weight matrix:
//   scale_r   = (max_c |w[r, c]|) / 448            (fp32 division)
//   code[r,c] = E4M3 nearest-even of (w[r, c] / scale_r)   (fp32 division)
// An all-zero row gets scale 0 and codes 0. The grouped GEMM multiplies each
// output column by its row's scale, so the dequantised weight is exactly
// scale_r * decode(code).
#include <math.h>

#include <algorithm>

#include "moe_common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// fp32 -> E4M3 code, round to nearest even, the sign bit copied from v.
// Magnitudes from 2^-6 up are normal: keep 3 mantissa bits (the carry moves
// into the exponent), re-bias the exponent from 127 to 7, and saturate at
// 448 (0x7E). Below 2^-6 the codes are multiples of 2^-9 (code 8 is 2^-6).
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  uint32_t code;
  if (a >= 0x3c800000u) {  // 2^-6
    const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;  // (exponent << 3) | mantissa, rounded
    code = min(r - ((127u - 7u) << 3), 0x7eu);
  } else {
    code = (uint32_t)rintf(__uint_as_float(a) * 512.0f);
  }
  return sign | code;
}

// One workgroup per weight row: the row maximum, then the codes, 8 per thread per pass.
__global__ __launch_bounds__(kThreads) void quantize_fp8_kernel(const u32x4_t* __restrict__ w, int cols,
                                                                 u32x2_t* __restrict__ q,
                                                                 float* __restrict__ scales) {
  __shared__ float s_max[kThreads / kWave];
  const size_t row = blockIdx.x;
  const int c8 = cols / 8;  // 8 values per 16-byte piece
  const u32x4_t* src = w + row * c8;
  float m = 0.f;
  for (int i = threadIdx.x; i < c8; i += kThreads) {
    const u32x4_t v = src[i];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const uint32_t two = v[h];
      m = fmaxf(m, fabsf(__uint_as_float(two << 16)));
      m = fmaxf(m, fabsf(__uint_as_float(two & 0xffff0000u)));
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
  if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = m;
  __syncthreads();
  float amax = s_max[0];
#pragma unroll
  for (int i = 1; i < kThreads / kWave; ++i) amax = fmaxf(amax, s_max[i]);
  const float scale = amax / 448.0f;
  if (threadIdx.x == 0) scales[row] = scale;
  u32x2_t* dst = q + row * c8;
  for (int i = threadIdx.x; i < c8; i += kThreads) {
    const u32x4_t v = src[i];
    uint32_t out[2] = {0u, 0u};
    if (scale > 0.f) {
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const uint32_t lo = e4m3_code(__uint_as_float(v[h] << 16) / scale);
        const uint32_t hi = e4m3_code(__uint_as_float(v[h] & 0xffff0000u) / scale);
        out[h >> 1] |= (lo | (hi << 8)) << (16 * (h & 1));
      }
    }
    u32x2_t o;
    o.x = out[0];
    o.y = out[1];
    dst[i] = o;
  }
}

// out[r, c] = scales[r] * value(codes[r, c]): 8 codes per thread, widened with
// the grouped GEMM's own fp8x8_to_bf16, then one fp32 product each.
__global__ __launch_bounds__(kThreads) void dequantize_fp8_kernel(const u32x2_t* __restrict__ codes, long long n8,
                                                                  int c8, const float* __restrict__ scales,
                                                                  float* __restrict__ out) {
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < n8; i += (long long)gridDim.x * kThreads) {
    const u32x2_t q = codes[i];
    const float sc = scales[i / c8];
    const bf16x8_t v = fp8x8_to_bf16(q.x, q.y);
    float* o = out + i * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (float)v[e] * sc;
  }
}

}  // namespace

int launch_dequantize_fp8(long long rows, int cols, const uint8_t* codes, const float* scales, float* out,
                          hipStream_t stream) {
  const long long n8 = rows * (cols / 8);
  if (n8 == 0) return MOE_OK;
  const long long blocks = std::min<long long>((n8 + kThreads - 1) / kThreads, 4096);
  hipLaunchKernelGGL(dequantize_fp8_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     reinterpret_cast<const u32x2_t*>(codes), n8, cols / 8, scales, out);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int launch_quantize_fp8(long long rows, int cols, const void* w_bf16, uint8_t* codes, float* scales,
                        hipStream_t stream) {
  if (rows == 0) return MOE_OK;
  hipLaunchKernelGGL(quantize_fp8_kernel, dim3((unsigned)rows), dim3(kThreads), 0, stream,
                     static_cast<const u32x4_t*>(w_bf16), cols, reinterpret_cast<u32x2_t*>(codes), scales);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
