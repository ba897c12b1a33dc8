// Grouping of token copies by expert: histogram, capacity, prefix sum, and a
// stable permutation.
//
// forward_grouped in "混合专家 MoE" (anrans ai-infra handbook), section
// "实现：逐 token 与按专家分组", flattens idx, sorts it stably by expert,
// counts with bincount, and walks the segments from a running start. The
// same section describes the count as a histogram and the start of each
// expert as a prefix sum. Capacity is the static per-expert buffer of the
// notes "混合专家模型 (MoE)：大规模稀疏条件计算的架构与工程实践", section 三.1.
// Copies take their places in copy order c = t*k + j.
//
// The work runs in three kernels, over chunks of kChunk consecutive copies:
//   1. hist:    a per-chunk expert histogram from LDS atomics. Counting
//               does not depend on the order of the atomics.
//   2. scan:    one workgroup.
//               - For each expert, an exclusive scan over the chunks gives
//                 the rank of each chunk's first copy within the expert.
//               - counts = the totals; kept = min(counts, C).
//               - offsets = exclusive scan of kept.
//               - The balance statistic, summed in expert order.
//   3. scatter: one wavefront per chunk, 64 copies at a time, in copy order.
//               - A copy's rank within its expert = the chunk base
//                 + the copies of that expert already seen in this chunk
//                 + the lower lanes of this step with the same expert.
//               - Lanes with equal experts are matched with ballots.
//               - Rank < C keeps the copy at offsets[e] + rank.
// Every output is a pure function of topk_idx: there are no races and no
// order-dependent atomics.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kChunk = 512;

__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ idx, int NK, int E,
                                                   int32_t* __restrict__ hist) {
  __shared__ int32_t s_h[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += blockDim.x) s_h[e] = 0;
  __syncthreads();
  const int c0 = blockIdx.x * kChunk;
  const int c1 = min(NK, c0 + kChunk);
  for (int c = c0 + threadIdx.x; c < c1; c += blockDim.x) {
    const int e = idx[c];
    if ((unsigned)e < (unsigned)E) atomicAdd(&s_h[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[(size_t)blockIdx.x * E + e] = s_h[e];
}

__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ hist, int nchunks,
                                                    int E, int C, int N, int k,
                                                    int32_t* __restrict__ base,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets,
                                                    const double* __restrict__ prob_sum,
                                                    double* __restrict__ stat) {
  __shared__ int32_t s_kept[kMaxExperts];
  __shared__ int32_t s_cnt[kMaxExperts];
  __shared__ int32_t s_scan[1024];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += blockDim.x) {
    int run = 0;
    for (int b = 0; b < nchunks; ++b) {
      base[(size_t)b * E + e] = run;
      run += hist[(size_t)b * E + e];
    }
    counts[e] = run;
    s_cnt[e] = run;
    s_kept[e] = (C > 0 && run > C) ? C : run;
  }
  __syncthreads();
  // inclusive Hillis-Steele scan of kept over e (E <= 1024 = blockDim)
  int v = tid < E ? s_kept[tid] : 0;
  s_scan[tid] = v;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int add = tid >= o ? s_scan[tid - o] : 0;
    __syncthreads();
    s_scan[tid] += add;
    __syncthreads();
  }
  if (tid < E) offsets[tid] = s_scan[tid] - v;
  if (tid == 0) offsets[E] = E > 0 ? s_scan[E - 1] : 0;
  if (tid == 0 && stat) {
    // E * sum_e (counts_e / (N k)) (prob_sum_e / N), summed in expert order
    // (no copies: the statistic is defined as 0)
    const double nk = (double)N * (double)k, n = (double)N;
    double a = 0.0;
    if (N > 0)
      for (int e = 0; e < E; ++e) a += ((double)s_cnt[e] / nk) * (prob_sum[e] / n);
    *stat = (double)E * a;
  }
}

__global__ __launch_bounds__(64) void scatter_kernel(const int32_t* __restrict__ idx, int NK, int E,
                                                     int C, const int32_t* __restrict__ base,
                                                     const int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ perm,
                                                     int32_t* __restrict__ slot_pos) {
  __shared__ int32_t s_run[kMaxExperts];
  __shared__ int32_t s_off[kMaxExperts];
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += kWave) {
    s_run[e] = base[(size_t)blockIdx.x * E + e];
    s_off[e] = offsets[e];
  }
  __syncthreads();
  const int c0 = blockIdx.x * kChunk;
  const int c1 = min(NK, c0 + kChunk);
  const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));  // lanes below this one
  for (int cs = c0; cs < c1; cs += kWave) {
    const int c = cs + lane;
    const bool in = c < c1;
    int e = in ? idx[c] : -1;
    const bool valid = in && (unsigned)e < (unsigned)E;
    if (!valid) e = -1;
    int rank = 0;
    uint64_t todo = __ballot(valid);
    while (todo) {
      const int leader = __ffsll((unsigned long long)todo) - 1;
      const int el = __shfl(e, leader, kWave);
      const uint64_t same = __ballot(e == el) & todo;
      if (e == el) rank = s_run[el] + __popcll(same & lower);
      __syncthreads();  // every lane has read s_run[el] before the leader moves it
      if (lane == leader) s_run[el] += __popcll(same);
      __syncthreads();
      todo &= ~same;
    }
    if (in) {
      if (!valid) {
        slot_pos[c] = -1;
      } else if (C > 0 && rank >= C) {
        slot_pos[c] = -1;
      } else {
        const int pos = s_off[e] + rank;
        perm[pos] = c;
        slot_pos[c] = pos;
      }
    }
  }
}

}  // namespace

int permute_chunks(const moe_shape& s) {
  const long long nk = (long long)s.n_tokens * s.top_k;
  return (int)((nk + kChunk - 1) / kChunk);
}

int launch_permute(const moe_shape& s, const int32_t* topk_idx, const double* prob_sum,
                   int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* slot_pos,
                   double* balance_stat, int32_t* hist, int32_t* base, hipStream_t stream) {
  const int NK = s.n_tokens * s.top_k;
  const int nch = permute_chunks(s);
  const int C = s.capacity > 0 ? s.capacity : 0;
  if (nch > 0)
    hipLaunchKernelGGL(hist_kernel, dim3(nch), dim3(256), 0, stream, topk_idx, NK, s.n_experts, hist);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, stream, hist, nch, s.n_experts, C,
                     s.n_tokens, s.top_k, base, counts, offsets, prob_sum, balance_stat);
  if (nch > 0)
    hipLaunchKernelGGL(scatter_kernel, dim3(nch), dim3(kWave), 0, stream, topk_idx, NK,
                       s.n_experts, C, base, offsets, perm, slot_pos);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
