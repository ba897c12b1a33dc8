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
//   3. scatter: one workgroup per chunk, one thread per copy.
//               - It loads the counts and forms kept = min(count, C) and
//                 offsets = exclusive scan of kept in LDS. Workgroup 0 also
//                 writes offsets and the balance statistic.
//               - A copy's rank within its expert = the chunk base + the
//                 earlier copies of the chunk with that expert: those of
//                 earlier waves from per-wave histograms in LDS, those of its
//                 own wave by a scan of the wave's experts.
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
// With the router's per-workgroup sums (partials, nb > 0) it also adds them
// into prob_sum[e]: the router's last step, which the forward can defer to here.
__global__ __launch_bounds__(256) void colscan_kernel(const int32_t* __restrict__ hist, int nchunks,
                                                      int E, int32_t* __restrict__ base,
                                                      int32_t* __restrict__ counts,
                                                      const double* __restrict__ partials, int nb,
                                                      double* __restrict__ prob_sum) {
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (e >= E) return;
  if (nb > 0) {
    const double a = prob_sum_wave(partials, nb, E, e, lane);
    if (lane == 0) prob_sum[e] = a;
  }
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

// One workgroup per chunk, one thread per copy (kChunk threads).
// base == nullptr: a single chunk holds every copy. Then this kernel also
// counts (the chunk's histogram is the expert counts, and every base is 0),
// in place of hist_kernel and colscan_kernel.
constexpr int kScatterThreads = kChunk;
constexpr int kScatterWaves = kScatterThreads / kWave;

__global__ __launch_bounds__(kScatterThreads) void scatter_kernel(const int32_t* __restrict__ idx, int NK,
                                                                  int E, int C, int N, int k,
                                                                  const int32_t* __restrict__ base,
                                                                  int32_t* __restrict__ counts,
                                                                  int32_t* __restrict__ offsets,
                                                                  int32_t* __restrict__ perm,
                                                                  int32_t* __restrict__ slot_pos,
                                                                  const double* __restrict__ prob_sum,
                                                                  double* __restrict__ stat) {
  __shared__ int32_t s_run[kMaxExperts];
  __shared__ int32_t s_cnt[kMaxExperts];
  __shared__ int32_t s_off[kMaxExperts + 1];
  __shared__ __attribute__((aligned(16))) int32_t s_e[kChunk];
  __shared__ int32_t s_wh[kScatterWaves][kMaxExperts];  // per-wave expert histograms of the chunk
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const bool single = base == nullptr;
  const int c0 = blockIdx.x * kChunk;
  const int c = c0 + tid;
  const bool in = c < NK;
  int e = in ? idx[c] : -1;
  if ((unsigned)e >= (unsigned)E) e = -1;  // past the end, or out of range: no expert
  s_e[tid] = e;
  // the balance statistic's prob_sum terms, loaded now so that their latency
  // overlaps the counting (wave 0 of workgroup 0; lane l holds experts l + 64 q)
  constexpr int kPs = kMaxExperts / kWave;
  double ps[kPs];
  const bool do_stat = blockIdx.x == 0 && stat && wave == 0;
#pragma unroll
  for (int q = 0; q < kPs; ++q) {
    const int x = lane + kWave * q;
    ps[q] = (do_stat && x < E) ? prob_sum[x] : 0.0;
  }
  for (int x = tid; x < E; x += kScatterThreads) {
    s_cnt[x] = single ? 0 : counts[x];
    s_run[x] = single ? 0 : base[(size_t)blockIdx.x * E + x];
  }
  for (int x = tid; x < kScatterWaves * E; x += kScatterThreads) s_wh[x / E][x % E] = 0;
  __syncthreads();
  if (e >= 0) {  // the order of the additions does not matter
    atomicAdd(&s_wh[wave][e], 1);
    if (single) atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();
  if (single)
    for (int x = tid; x < E; x += kScatterThreads) counts[x] = s_cnt[x];
  // offsets = exclusive scan of kept = min(counts, C): wave 0, lane l owning experts [l*per, (l+1)*per)
  if (wave == 0) {
    const int per = (E + kWave - 1) / kWave;
    int sum = 0;
    for (int q = 0; q < per; ++q) {
      const int x = lane * per + q;
      if (x < E) {
        const int cnt = s_cnt[x];
        const int kept = (C > 0 && cnt > C) ? C : cnt;
        s_off[x] = kept;
        sum += kept;
      }
    }
    const int incl = wave_incl_scan(sum, lane);
    int run = incl - sum;
    for (int q = 0; q < per; ++q) {
      const int x = lane * per + q;
      if (x < E) {
        const int kept = s_off[x];
        s_off[x] = run;
        run += kept;
      }
    }
    if (lane == kWave - 1) s_off[E] = incl;
    if (do_stat) {
      // E * sum_e (counts_e / (N k)) (prob_sum_e / N): lane-strided sums, then a fixed butterfly
      // (no copies: the statistic is defined as 0)
      const double nk = (double)N * (double)k, n = (double)N;
      double a = 0.0;
      if (N > 0)
#pragma unroll
        for (int q = 0; q < kPs; ++q) {
          const int x = lane + kWave * q;
          if (x < E) a += ((double)s_cnt[x] / nk) * (ps[q] / n);
        }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) a += __shfl_xor(a, o, kWave);
      if (lane == 0) *stat = (double)E * a;
    }
  }
  __syncthreads();
  if (blockIdx.x == 0)
    for (int x = tid; x <= E; x += kScatterThreads) offsets[x] = s_off[x];
  if (!in) return;  // no barrier follows
  if (e < 0) {
    slot_pos[c] = -1;
    return;
  }
  // rank within the expert: the chunk's base, plus the copies of earlier waves
  // with the same expert (their histograms), plus the earlier copies of this
  // wave with the same expert (a scan of at most 63 entries in LDS)
  int rank = s_run[e];
  for (int w = 0; w < wave; ++w) rank += s_wh[w][e];
  const int full = tid & ~3;
  for (int j = wave * kWave; j < full; j += 4) {
    const int4 v = *reinterpret_cast<const int4*>(&s_e[j]);
    rank += (v.x == e) + (v.y == e) + (v.z == e) + (v.w == e);
  }
  for (int j = full; j < tid; ++j) rank += s_e[j] == e;
  if (C > 0 && rank >= C) {
    slot_pos[c] = -1;
  } else {
    const int pos = s_off[e] + rank;
    perm[pos] = c;
    slot_pos[c] = pos;
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
                   double* balance_stat, int32_t* hist, int32_t* base, hipStream_t stream,
                   const double* partials, int nb, double* sum_out) {
  const int NK = s.n_tokens * s.top_k;
  const int nch = permute_chunks(s);
  const int C = s.capacity > 0 ? s.capacity : 0;
  const int E = s.n_experts;
  if (nch == 0) {  // no copies
    hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(256), 0, stream, E, counts, offsets, balance_stat);
  } else {
    if (nch > 1) {
      hipLaunchKernelGGL(hist_kernel, dim3(nch), dim3(256), 0, stream, topk_idx, NK, E, hist);
      hipLaunchKernelGGL(colscan_kernel, dim3((E + 3) / 4), dim3(256), 0, stream, hist, nch, E, base, counts,
                         partials, nb, sum_out);
    }
    hipLaunchKernelGGL(scatter_kernel, dim3(nch), dim3(kScatterThreads), 0, stream, topk_idx, NK, E, C,
                       s.n_tokens, s.top_k, nch > 1 ? base : nullptr, counts, offsets, perm, slot_pos,
                       prob_sum, balance_stat);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
