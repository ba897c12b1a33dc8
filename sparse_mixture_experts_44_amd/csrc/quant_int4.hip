// Int4 expert weights for the W4A16 variant of the grouped SwiGLU.
//
// The notes "混合专家模型 (MoE)：大规模稀疏条件计算的架构与工程实践", section
// 五.1 (the memory wall of inference), suggest W4A16 for the expert layers
// only: INT4 weights, FP16/BF16 activations, and the product taken on the
// dequantised weights. They give no scale granularity and no rounding. The
// readings here, as for the FP8 weights:
//   scale_r = (max_c |w[r, c]|) / 7                          (fp32 division)
//   q[r, c] = w[r, c] / scale_r rounded to the nearest integer, ties to even
//             (fp32 division), clamped to [-7, 7]
// An all-zero row gets scale 0 and codes 0. The dequantised weight is
// scale_r * q[r, c].
//
// Packed layout (what the grouped GEMM reads): a row of K codes takes K / 2
// bytes, in blocks of 64 codes (32 bytes). In the block of codes
// [k0, k0 + 64), the 32-bit word at byte 16 h + 4 s (h = 0, 1; s = 0..3)
// holds the 8 codes k0 + 16 s + 8 h + j (j = 0..7), each as 4-bit sign and
// magnitude (bit 3 set for q < 0, bits 0..2 = |q|): code j in byte j % 4 of
// the word, in its low nibble for j < 4 and its high nibble for j >= 4. That
// is the order in which the GEMM widens a word into the 8 bf16 operands of
// one lane's k16 step.
#include <math.h>

#include "moe_common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// bit position of code j (0..7) within its 32-bit word: byte j % 4, high nibble for j >= 4
__device__ __forceinline__ int shift_of(int j) { return 8 * (j & 3) + 4 * (j >> 2); }

// One workgroup per weight row: the row maximum, then one 64-code block per thread per pass.
__global__ __launch_bounds__(kThreads) void quantize_int4_kernel(const u32x4_t* __restrict__ w, int cols,
                                                                  u32x4_t* __restrict__ packed,
                                                                  float* __restrict__ scales) {
  __shared__ float s_max[kThreads / kWave];
  const size_t row = blockIdx.x;
  const int c8 = cols / 8;      // 16-byte pieces of 8 bf16 per row
  const int nblk = cols / 64;   // 64-code blocks per row
  const u32x4_t* src = w + row * c8;
  float m = 0.f;
  for (int i = threadIdx.x; i < c8; i += kThreads) {
    const u32x4_t v = src[i];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      m = fmaxf(m, fabsf(__uint_as_float(v[h] << 16)));
      m = fmaxf(m, fabsf(__uint_as_float(v[h] & 0xffff0000u)));
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
  if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = m;
  __syncthreads();
  float amax = s_max[0];
#pragma unroll
  for (int i = 1; i < kThreads / kWave; ++i) amax = fmaxf(amax, s_max[i]);
  const float scale = amax / 7.0f;
  if (threadIdx.x == 0) scales[row] = scale;
  u32x4_t* dst = packed + row * (size_t)(nblk * 2);  // 32 bytes per block
  for (int b = threadIdx.x; b < nblk; b += kThreads) {
    uint32_t word[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};  // word index h * 4 + s
    // the block's 64 codes, 8 per 16-byte piece: piece i holds codes 8 i .. 8 i + 7 = (s, h) = (i / 2, i % 2)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4_t v = src[b * 8 + i];
      const int s = i >> 1, h = i & 1;
      uint32_t acc = 0u;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t two = v[j >> 1];
        const float x = __uint_as_float((j & 1) ? (two & 0xffff0000u) : (two << 16));
        int q = 0;
        if (scale > 0.f) q = (int)fminf(fmaxf(rintf(x / scale), -7.f), 7.f);
        acc |= (uint32_t)(q < 0 ? 8 - q : q) << shift_of(j);  // sign and magnitude
      }
      word[h * 4 + s] = acc;
    }
    u32x4_t lo, hi;
    lo.x = word[0]; lo.y = word[1]; lo.z = word[2]; lo.w = word[3];
    hi.x = word[4]; hi.y = word[5]; hi.z = word[6]; hi.w = word[7];
    dst[b * 2] = lo;
    dst[b * 2 + 1] = hi;
  }
}

}  // namespace

int launch_quantize_int4(long long rows, int cols, const void* w_bf16, uint8_t* packed, float* scales,
                         hipStream_t stream) {
  if (rows == 0) return MOE_OK;
  hipLaunchKernelGGL(quantize_int4_kernel, dim3((unsigned)rows), dim3(kThreads), 0, stream,
                     static_cast<const u32x4_t*>(w_bf16), cols, reinterpret_cast<u32x4_t*>(packed), scales);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
