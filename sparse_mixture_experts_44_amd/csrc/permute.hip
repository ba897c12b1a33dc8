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
// The work runs in three kernels, over chunks of kChunk consecutive copies
// (one kernel, scatter, when a single chunk holds every copy):
//   1. hist:    a per-chunk expert histogram from LDS atomics. Counting
//               does not depend on the order of the atomics.
//   2. colscan: one wavefront per expert scans the chunk histograms, giving
//               each chunk's base rank within the expert and the expert's
//               total count (integer sums, so exact in any order).
//   3. scatter: one wavefront per chunk.
//               - It loads the counts and forms kept = min(count, C) and
//                 offsets = exclusive scan of kept in LDS. Workgroup 0 also
//                 writes offsets and the balance statistic.
//               - It then walks its copies 64 at a time, in copy order. A
//                 copy's rank within its expert = the chunk base + the copies
//                 of that expert already seen in this chunk + the lower lanes
//                 of this step with the same expert. Each lane counts those
//                 by scanning the step's 64 experts in LDS.
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

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  return v;
}

// One wavefront per expert: base[b][e] = sum_{b' < b} hist[b'][e]; counts[e] = total.
__global__ __launch_bounds__(256) void colscan_kernel(const int32_t* __restrict__ hist, int nchunks,
                                                      int E, int32_t* __restrict__ base,
                                                      int32_t* __restrict__ counts) {
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (e >= E) return;
  int run = 0;
  for (int b0 = 0; b0 < nchunks; b0 += kWave) {
    const int b = b0 + lane;
    const int v = b < nchunks ? hist[(size_t)b * E + e] : 0;
    const int incl = wave_incl_scan(v, lane);
    if (b < nchunks) base[(size_t)b * E + e] = run + incl - v;
    run += __shfl(incl, kWave - 1, kWave);
  }
  if (lane == 0) counts[e] = run;
}

// The workgroup is one wavefront, whose LDS accesses complete in issue order.
// Between the steps it only waits for its own LDS accesses: __syncthreads
// would also wait for the perm and slot_pos stores of the step before.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// base == nullptr: a single chunk holds every copy. Then this kernel also
// counts (the chunk's histogram is the expert counts, and every base is 0),
// in place of hist_kernel and colscan_kernel.
__global__ __launch_bounds__(64) void scatter_kernel(const int32_t* __restrict__ idx, int NK, int E,
                                                     int C, int N, int k,
                                                     const int32_t* __restrict__ base,
                                                     int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ perm,
                                                     int32_t* __restrict__ slot_pos,
                                                     const double* __restrict__ prob_sum,
                                                     double* __restrict__ stat) {
  constexpr int kSteps = kChunk / kWave;
  __shared__ int32_t s_run[kMaxExperts];
  __shared__ int32_t s_cnt[kMaxExperts];
  __shared__ int32_t s_off[kMaxExperts + 1];
  __shared__ __attribute__((aligned(16))) int32_t s_step[kWave];
  const int lane = threadIdx.x;
  const bool single = base == nullptr;
  const int c0 = blockIdx.x * kChunk;
  const int c1 = min(NK, c0 + kChunk);
  // this chunk's experts, all loaded up front (-1: past the end or out of range)
  int ev[kSteps];
#pragma unroll
  for (int q = 0; q < kSteps; ++q) {
    const int c = c0 + q * kWave + lane;
    const int e = c < c1 ? idx[c] : -1;
    ev[q] = (unsigned)e < (unsigned)E ? e : -1;
  }
  if (single) {
    for (int e = lane; e < E; e += kWave) s_cnt[e] = 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kSteps; ++q)
      if (ev[q] >= 0) atomicAdd(&s_cnt[ev[q]], 1);
    __syncthreads();
    for (int e = lane; e < E; e += kWave) {
      counts[e] = s_cnt[e];
      s_run[e] = 0;
    }
  } else {
    for (int e = lane; e < E; e += kWave) {
      s_cnt[e] = counts[e];
      s_run[e] = base[(size_t)blockIdx.x * E + e];
    }
  }
  __syncthreads();
  // offsets = exclusive scan of kept = min(counts, C), lane l owning experts [l*per, (l+1)*per)
  const int per = (E + kWave - 1) / kWave;
  int sum = 0;
  for (int q = 0; q < per; ++q) {
    const int e = lane * per + q;
    if (e < E) {
      const int c = s_cnt[e];
      const int kept = (C > 0 && c > C) ? C : c;
      s_off[e] = kept;
      sum += kept;
    }
  }
  const int incl = wave_incl_scan(sum, lane);
  int run = incl - sum;
  for (int q = 0; q < per; ++q) {
    const int e = lane * per + q;
    if (e < E) {
      const int kept = s_off[e];
      s_off[e] = run;
      run += kept;
    }
  }
  if (lane == kWave - 1) s_off[E] = incl;
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int e = lane; e <= E; e += kWave) offsets[e] = s_off[e];
    if (stat) {
      // E * sum_e (counts_e / (N k)) (prob_sum_e / N): lane-strided sums, then a fixed butterfly
      // (no copies: the statistic is defined as 0)
      const double nk = (double)N * (double)k, n = (double)N;
      double a = 0.0;
      if (N > 0)
        for (int e = lane; e < E; e += kWave) a += ((double)s_cnt[e] / nk) * (prob_sum[e] / n);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) a += __shfl_xor(a, o, kWave);
      if (lane == 0) *stat = (double)E * a;
    }
  }
#pragma unroll
  for (int q = 0; q < kSteps; ++q) {
    const int c = c0 + q * kWave + lane;
    if (c0 + q * kWave >= c1) break;  // uniform: the chunk's last step is done
    const bool in = c < c1;
    const int e = ev[q];
    const bool valid = e >= 0;
    // rank among this step's copies: lanes below with the same expert (and
    // how many lanes of the step share it), from one pass over the step's
    // experts in LDS
    s_step[lane] = e;
    wave_lds_sync();
    int below = 0, same = 0;
#pragma unroll 4
    for (int j = 0; j < kWave; j += 4) {
      const int4 v = *reinterpret_cast<const int4*>(&s_step[j]);
      below += (v.x == e && j < lane) + (v.y == e && j + 1 < lane) + (v.z == e && j + 2 < lane) +
               (v.w == e && j + 3 < lane);
      same += (v.x == e) + (v.y == e) + (v.z == e) + (v.w == e);
    }
    const int rank = valid ? s_run[e] + below : 0;
    wave_lds_sync();  // every lane has read s_run and s_step before they change
    if (valid && below == same - 1) s_run[e] += same;  // the step's last copy of e
    wave_lds_sync();
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

__global__ void empty_kernel(int E, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                             double* __restrict__ stat) {
  for (int e = threadIdx.x; e <= E; e += blockDim.x) {
    if (e < E) counts[e] = 0;
    offsets[e] = 0;
  }
  if (threadIdx.x == 0 && stat) *stat = 0.0;
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
  const int E = s.n_experts;
  if (nch == 0) {  // no copies
    hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(256), 0, stream, E, counts, offsets, balance_stat);
  } else {
    if (nch > 1) {
      hipLaunchKernelGGL(hist_kernel, dim3(nch), dim3(256), 0, stream, topk_idx, NK, E, hist);
      hipLaunchKernelGGL(colscan_kernel, dim3((E + 3) / 4), dim3(256), 0, stream, hist, nch, E, base, counts);
    }
    hipLaunchKernelGGL(scatter_kernel, dim3(nch), dim3(kWave), 0, stream, topk_idx, NK, E, C,
                       s.n_tokens, s.top_k, nch > 1 ? base : nullptr, counts, offsets, perm, slot_pos,
                       prob_sum, balance_stat);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
