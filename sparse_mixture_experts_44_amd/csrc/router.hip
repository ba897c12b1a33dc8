// Router of the MoE layer: logits = x W_r^T (+ logit bias), softmax, the
// selection-only bias, top-k, renormalisation, and per-expert probability
// sums. This is route() of "混合专家 MoE" (anrans ai-infra handbook), section
// "实现：逐 token 与按专家分组". The bias for selection only is the
// aux-loss-free balancing of its section "负载均衡".
//
// Two forms:
//   Fused (bf16 layers with 64 <= E <= 256 and at least 1024 tokens):
//     route_fused_kernel does the whole route() of a tile of tokens in one
//     kernel: the logits against every expert on the matrix cores (the
//     logits are a dense contraction of K = d; on the VALU they would take
//     several times longer), the softmax, selection and renormalisation of
//     each token by one wavefront from LDS (select_token), and the tile's
//     fp64 probability sums. prob_sum_kernel then adds the tiles' sums.
//   Otherwise (small batches, fp32 layers, other E):
//   1. logits_kernel: a VALU GEMM.
//      - Grid: (token tile) x (K split) x (expert tile), sized to give every
//        CU more than one workgroup also at decode sizes (N = 64). At most 8
//        K splits; few tokens get one output per thread and expert tiles.
//      - K is staged through LDS 128 bytes per row at a time. Rows are padded
//        to 144 bytes, so 16-byte reads from consecutive rows use distinct
//        banks.
//      - Each thread owns TPT tokens x EPT experts. bf16 uses v_dot2_f32_bf16
//        (two products per instruction, fp32 accumulation).
//      - Each chunk is summed into a fresh partial before it is added to the
//        running sum.
//      - Output: fp32 partial logits [split][N][E].
//   2. select_kernel: one wavefront per token (select_token).
//      - Sums the splits in split order, adds the logit bias, then softmax
//        with wave reductions in a fixed order (on the DPP lane network),
//        the selection score, and k rounds of a wave arg-max. A larger
//        score wins; on equal scores the lower expert index wins.
//      - Renormalises the k weights.
//      - Adds p into fp64 per-workgroup sums in a fixed order.
//      - With at most 64 workgroups, the last one to finish (a counter that
//        the logits kernel cleared) adds the workgroup sums into prob_sum,
//        workgroup by workgroup in index order.
//   3. prob_sum_kernel (more select workgroups, the fused form, or logits
//      from the matrix cores): one wavefront per expert adds the workgroup
//      sums with a fixed tree. Either way prob_sum is bit-reproducible.
// The router z-loss and the backward pass recompute the logits alone; large
// bf16 routers run that as one grouped GEMM on the matrix cores
// (compute_logits).
#include <math.h>

#include "moe_common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 32;         // dwords per row chunk: 64 bf16 or 32 fp32
constexpr int kRow = kChunk + 4;   // padded LDS row stride in dwords
constexpr int kSelTokMax = 8;      // tokens per select workgroup, at most (2 per wave)
constexpr int kTargetBlocks = 512; // logits workgroups to aim for
constexpr int kMaxSplits = 8;      // K splits of the logits, at most
constexpr int kFewTiles = 64;      // fewer token tiles than this: split the experts over workgroups

template <bool BF16>
__device__ __forceinline__ float mac(uint32_t a, uint32_t b, float c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
  } else {
    return fmaf(__uint_as_float(a), __uint_as_float(b), c);
  }
}

// Workgroup barrier after this wave's LDS accesses have completed. Unlike
// __syncthreads it does not wait for global loads in flight (the prefetched
// chunks).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Wave reductions on the DPP lane network: two quad permutations, the
// half-row mirror and the row mirror leave every lane of each 16-lane row
// with the row's reduction (the two operands of every step are the same pair
// in every lane of the row, so the rows agree bit for bit); the four row
// values are then read into scalars and combined in a fixed order. Each DPP
// step is a VALU operand modifier, with no LDS round trip as a cross-lane
// shuffle takes.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppQuad1032 = 0xB1;       // quad_perm [1, 0, 3, 2]
constexpr int kDppQuad2301 = 0x4E;       // quad_perm [2, 3, 0, 1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

__device__ __forceinline__ float rows_of(float v, int r) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16 * r));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<kDppQuad1032>(v));
  v = fmaxf(v, dpp<kDppQuad2301>(v));
  v = fmaxf(v, dpp<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp<kDppRowMirror>(v));
  return fmaxf(fmaxf(rows_of(v, 0), rows_of(v, 1)), fmaxf(rows_of(v, 2), rows_of(v, 3)));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<kDppQuad1032>(v);
  v += dpp<kDppQuad2301>(v);
  v += dpp<kDppRowHalfMirror>(v);
  v += dpp<kDppRowMirror>(v);
  return (rows_of(v, 0) + rows_of(v, 1)) + (rows_of(v, 2) + rows_of(v, 3));
}

// ---------------------------------------------------------------- 1. logits

// Thread grid: EG expert groups x (256/EG) token groups. Thread (tg, eg) owns
// tokens tg + TG*i (i < TPT) and experts eg + EG*j (j < EPT).
template <bool BF16, int EG, int EPT, int TPT, int PD>
__global__ __launch_bounds__(kThreads) void logits_kernel(const uint32_t* __restrict__ x,
                                                          const uint32_t* __restrict__ w, int N,
                                                          int dw, int E, int chunks_per_split,
                                                          float* __restrict__ part,
                                                          unsigned int* __restrict__ clear) {
  constexpr int TG = kThreads / EG;
  constexpr int TT = TG * TPT;        // tokens per workgroup
  constexpr int EROWS = EG * EPT;     // expert rows covered
  constexpr int XP = (TT * 8 + kThreads - 1) / kThreads;     // x pieces (16 B) per thread per chunk
  constexpr int WP = (EROWS * 8 + kThreads - 1) / kThreads;  // W pieces per thread per chunk
  __shared__ uint32_t s_w[EROWS * kRow];
  __shared__ uint32_t s_x[TT * kRow];

  const int tid = threadIdx.x;
  if (clear && (blockIdx.x | blockIdx.y | blockIdx.z | tid) == 0) *clear = 0u;  // the select kernel's counter
  const int eg = tid % EG, tg = tid / EG;
  const int t0 = blockIdx.x * TT;
  const int split = blockIdx.y;
  const int e0 = blockIdx.z * EROWS;  // first expert of this workgroup's expert tile
  const int nchunks = dw / kChunk;
  const int c0 = split * chunks_per_split;
  const int c1 = min(nchunks, c0 + chunks_per_split);

  float acc[TPT][EPT];
#pragma unroll
  for (int i = 0; i < TPT; ++i)
#pragma unroll
    for (int j = 0; j < EPT; ++j) acc[i][j] = 0.f;

  // PD chunks in flight per thread: slot u of the ring holds chunk c0 + PD*i + u
  u32x4_t px[PD][XP], pw[PD][WP];
  const u32x4_t zero = {0u, 0u, 0u, 0u};
#define MOE_LOAD_CHUNK(C, U)                                                              \
  {                                                                                       \
    const int kc_ = (C) * kChunk;                                                         \
    _Pragma("unroll") for (int q = 0; q < XP; ++q) {                                      \
      const int piece = tid + kThreads * q, r = piece >> 3, pc = piece & 7;               \
      const int t = t0 + r;                                                               \
      px[U][q] = (r < TT && t < N) ? *reinterpret_cast<const u32x4_t*>(x + (size_t)t * dw + kc_ + pc * 4) : zero; \
    }                                                                                     \
    _Pragma("unroll") for (int q = 0; q < WP; ++q) {                                      \
      const int piece = tid + kThreads * q, er = piece >> 3, pc = piece & 7;              \
      pw[U][q] = (er < EROWS && e0 + er < E) ? *reinterpret_cast<const u32x4_t*>(w + (size_t)(e0 + er) * dw + kc_ + pc * 4) : zero; \
    }                                                                                     \
  }

#pragma unroll
  for (int u = 0; u < PD; ++u)
    if (c0 + u < c1) MOE_LOAD_CHUNK(c0 + u, u);
  for (int cb = c0; cb < c1; cb += PD) {
#pragma unroll
    for (int u = 0; u < PD; ++u) {
      const int c = cb + u;
      if (c >= c1) break;
      lds_barrier();  // everyone finished reading the previous chunk
#pragma unroll
      for (int q = 0; q < XP; ++q) {
        const int piece = tid + kThreads * q;
        if (piece < TT * 8) *reinterpret_cast<u32x4_t*>(s_x + (piece >> 3) * kRow + (piece & 7) * 4) = px[u][q];
      }
#pragma unroll
      for (int q = 0; q < WP; ++q) {
        const int piece = tid + kThreads * q;
        if (piece < EROWS * 8) *reinterpret_cast<u32x4_t*>(s_w + (piece >> 3) * kRow + (piece & 7) * 4) = pw[u][q];
      }
      lds_barrier();
      if (c + PD < c1) MOE_LOAD_CHUNK(c + PD, u);
      float pt[TPT][EPT];
#pragma unroll
      for (int i = 0; i < TPT; ++i)
#pragma unroll
        for (int j = 0; j < EPT; ++j) pt[i][j] = 0.f;
#pragma unroll
      for (int q = 0; q < kChunk / 4; ++q) {
        u32x4_t xv[TPT], wv[EPT];
#pragma unroll
        for (int i = 0; i < TPT; ++i) xv[i] = *reinterpret_cast<const u32x4_t*>(s_x + (tg + TG * i) * kRow + q * 4);
#pragma unroll
        for (int j = 0; j < EPT; ++j) wv[j] = *reinterpret_cast<const u32x4_t*>(s_w + (eg + EG * j) * kRow + q * 4);
#pragma unroll
        for (int i = 0; i < TPT; ++i)
#pragma unroll
          for (int j = 0; j < EPT; ++j) {
            float a = pt[i][j];
            a = mac<BF16>(xv[i].x, wv[j].x, a);
            a = mac<BF16>(xv[i].y, wv[j].y, a);
            a = mac<BF16>(xv[i].z, wv[j].z, a);
            a = mac<BF16>(xv[i].w, wv[j].w, a);
            pt[i][j] = a;
          }
      }
#pragma unroll
      for (int i = 0; i < TPT; ++i)
#pragma unroll
        for (int j = 0; j < EPT; ++j) acc[i][j] += pt[i][j];
    }
  }
#undef MOE_LOAD_CHUNK

  float* out = part + (size_t)split * N * E;
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int t = t0 + tg + TG * i;
    if (t >= N) continue;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int e = e0 + eg + EG * j;
      if (e < E) out[(size_t)t * E + e] = acc[i][j];
    }
  }
}

// ---------------------------------------------------------------- 2. select

// One token's selection, by one wavefront. v holds the token's logits (with
// the logit bias), EL per lane: expert e = lane + 64 m, -inf past E. Softmax
// with butterfly reductions in a fixed order, the selection score s = p +
// select bias, k rounds of a wave arg-max (a larger score wins; on equal
// scores the lower expert index), the k weights (renormalised or not), and p
// added into pacc.
template <int EL>
__device__ __forceinline__ void select_token(float (&v)[EL], const float (&sb)[EL], int lane, int E, int k,
                                             int renorm, int32_t* __restrict__ idx_row,
                                             float* __restrict__ w_row, double (&pacc)[EL]) {
  float mx = -INFINITY;
#pragma unroll
  for (int m = 0; m < EL; ++m) mx = fmaxf(mx, v[m]);
  mx = wave_max(mx);
  float sum = 0.f;
#pragma unroll
  for (int m = 0; m < EL; ++m) {
    const int e = lane + kWave * m;
    v[m] = (e < E) ? expf(v[m] - mx) : 0.f;
    sum += v[m];
  }
  sum = wave_sum(sum);
  float p[EL], s[EL];
#pragma unroll
  for (int m = 0; m < EL; ++m) {
    p[m] = v[m] / sum;
    pacc[m] += (double)p[m];
    s[m] = p[m] + sb[m];
  }
  // k rounds. Each takes the largest remaining score (a wave max), then the
  // lowest expert index that holds it: expert e = lane + 64 m, so that is the
  // lowest lane of the first m whose ballot is not empty. Its p is read from
  // the owner lane, which then drops the expert from its candidates.
  uint32_t avail = 0;  // bit m: expert lane + 64 m is still a candidate
#pragma unroll
  for (int m = 0; m < EL; ++m)
    if (lane + kWave * m < E) avail |= 1u << m;
  float sel_sum = 0.f, mine_p = 0.f;
  int mine_idx = -1;
  for (int j = 0; j < k; ++j) {
    float lm = -INFINITY;
#pragma unroll
    for (int m = 0; m < EL; ++m)
      if ((avail >> m) & 1u) lm = fmaxf(lm, s[m]);
    const float top = wave_max(lm);
    int bm = -1, bl = 0;
#pragma unroll
    for (int m = 0; m < EL; ++m) {
      const unsigned long long b = __ballot(((avail >> m) & 1u) && s[m] == top);
      if (bm < 0 && b != 0ull) {
        bm = m;
        bl = __builtin_ctzll(b);
      }
    }
    float bp = 0.f;
#pragma unroll
    for (int m = 0; m < EL; ++m)
      if (m == bm) bp = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p[m]), bl));
    if (bm >= 0 && lane == bl) avail &= ~(1u << bm);
    if (lane == j) {
      mine_idx = bm >= 0 ? kWave * bm + bl : -1;
      mine_p = bp;
    }
    sel_sum += bp;
  }
  if (lane < k) {
    idx_row[lane] = mine_idx;
    w_row[lane] = renorm ? mine_p / sel_sum : mine_p;
  }
}

// prob_sum[e] for e = threadIdx.x + kThreads * i, by the select kernel's last
// workgroup when there are at most kFoldBlocks workgroup sums: added in
// workgroup order, their loads issued in batches of 16 so that they overlap.
constexpr int kFoldBlocks = 64;

__device__ __forceinline__ void add_prob_sums(const double* __restrict__ partials, int nb, int E,
                                              double* __restrict__ prob_sum) {
  for (int e = (int)threadIdx.x; e < E; e += kThreads) {
    double a = 0.0;
    for (int b0 = 0; b0 < nb; b0 += 16) {
      double v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = b0 + u < nb ? partials[(size_t)(b0 + u) * E + e] : 0.0;
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (b0 + u < nb) a += v[u];
    }
    prob_sum[e] = a;
  }
}

template <int EL>  // experts per lane: E <= 64 * EL
__global__ __launch_bounds__(kThreads) void select_kernel(
    const float* __restrict__ part, int splits, const float* __restrict__ logit_bias,
    const float* __restrict__ select_bias, int N, int E, int k, int renorm, int tpb,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, double* __restrict__ partials,
    unsigned int* __restrict__ done, double* __restrict__ prob_sum) {
  __shared__ double s_part[kThreads / kWave][64 * EL];
  __shared__ unsigned int s_ticket;
  const int tid = threadIdx.x;
  const int wv = tid >> 6, lane = tid & 63;
  const int t0 = blockIdx.x * tpb;
  double pacc[EL];
  float lb[EL], sb[EL];
#pragma unroll
  for (int m = 0; m < EL; ++m) {
    const int e = lane + kWave * m;
    pacc[m] = 0.0;
    lb[m] = (logit_bias && e < E) ? logit_bias[e] : 0.f;
    sb[m] = (select_bias && e < E) ? select_bias[e] : 0.f;
  }
  const size_t split_stride = (size_t)N * E;
  for (int tt = wv; tt < tpb; tt += kThreads / kWave) {
    const int t = t0 + tt;
    if (t >= N) break;
    float v[EL];
#pragma unroll
    for (int m = 0; m < EL; ++m) {
      const int e = lane + kWave * m;
      float l = -INFINITY;
      if (e < E) {
        // splits added in split order; loaded 8 at a time so the loads overlap
        const float* src = part + (size_t)t * E + e;
        l = 0.f;
        for (int q0 = 0; q0 < splits; q0 += 8) {
          float b[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) b[u] = (q0 + u < splits) ? src[(size_t)(q0 + u) * split_stride] : 0.f;
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (q0 + u < splits) l += b[u];
        }
        l += lb[m];
      }
      v[m] = l;
    }
    select_token<EL>(v, sb, lane, E, k, renorm, topk_idx + (size_t)t * k, topk_w + (size_t)t * k, pacc);
  }
  // per-workgroup probability sums, waves combined in a fixed order
#pragma unroll
  for (int m = 0; m < EL; ++m) s_part[wv][lane + kWave * m] = pacc[m];
  __syncthreads();
  for (int e = tid; e < E; e += kThreads) {
    double a = s_part[0][e];
#pragma unroll
    for (int q = 1; q < kThreads / kWave; ++q) a += s_part[q][e];
    partials[(size_t)blockIdx.x * E + e] = a;
  }
  if (!done) return;  // prob_sum_kernel follows
  // the last workgroup to get here adds every workgroup's sums: release this
  // workgroup's sums before taking a ticket, acquire the others' after
  __threadfence();
  __syncthreads();
  if (tid == 0) s_ticket = atomicAdd(done, 1u);
  __syncthreads();
  if (s_ticket != gridDim.x - 1) return;
  __threadfence();
  add_prob_sums(partials, gridDim.x, E, prob_sum);
  if (tid == 0) *done = 0u;
}

// ---------------------------------------------------------------- 2b. fused router (bf16, prefill)

// The whole route() for a tile of TM tokens in one kernel: the logits against
// all experts on the matrix cores, then the selection of 2. from LDS, then
// the tile's probability sums.
// - 8 waves as WT x WE; wave (wt, we) computes tokens 32 wt .. + 32 of the
//   tile against experts 32 we .. + 32 (v_mfma_f32_32x32x16_bf16, fp32 sums of
//   exact bf16 products). TM = 32 WT, and the tile spans EP = 32 WE >= E
//   experts.
// - K runs in steps of 64 through NS LDS stages. A stage holds the TM x rows,
//   then the EP W_r rows, 128 bytes each, filled by direct global->LDS copies
//   of 8 rows per instruction (coalesced 128-byte row pieces), 16-byte pieces
//   XOR-swizzled by row so that the MFMA operand reads hit distinct banks.
//   W_r is read by every workgroup and stays in L2.
// - Rows past N or E re-read the last row; their results are never used.
template <int WT, int NS, bool ROT>
__global__ __launch_bounds__(512, 1) void route_fused_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ w, const float* __restrict__ logit_bias,
    const float* __restrict__ select_bias, int N, int d, int E, int k, int renorm,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, double* __restrict__ partials) {
  constexpr int NW = 8, NT = NW * kWave;
  constexpr int WE = NW / WT;
  constexpr int TM = 32 * WT, EP = 32 * WE;
  constexpr int EL = (EP + kWave - 1) / kWave;  // experts per lane in the selection
  constexpr int ROWS = TM + EP;                 // stage rows: x, then W_r
  constexpr int STAGE = ROWS * 128;
  constexpr int INS = ROWS / 8;                 // 1 KB copy instructions per stage
  constexpr int PER = (INS + NW - 1) / NW;      // per wave, at most
  constexpr int LS = EP + 4;                    // row stride of the logits tile (floats)
  static_assert(INS * 8 == ROWS && NS * STAGE >= TM * LS * 4 + NW * kWave * EL * 8, "tile shape");
  __shared__ __attribute__((aligned(1024))) uint8_t s_tile[NS * STAGE];  // later: logits tile, then sums
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wt = wave / WE, we = wave % WE;
  const int t0 = blockIdx.x * TM;

  // copy i of this wave: instruction c = wave + NW i fills rows 8c .. 8c + 7; the lane writes
  // piece lane % 8 of row 8c + lane / 8, which holds the logical piece (lane % 8) ^ swz(row)
  const int cnt = (INS - wave + NW - 1) / NW;  // this wave's copies per stage (wave-uniform)
  const bf16_t* src[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = min(wave + NW * i, INS - 1);
    const int r = 8 * c + (lane >> 3);
    const int pc = ((lane & 7) ^ swz<8>(r)) * 8;
    src[i] = r < TM ? x + (size_t)min(t0 + r, N - 1) * d + pc : w + (size_t)min(r - TM, E - 1) * d + pc;
  }
  const uint32_t lds0 = lds_addr(&s_tile[0]);
  const int nk = d / 64;
  // ROT: workgroup b walks K from step b mod nk on, wrapping, so that the
  // workgroups do not all read the same W_r lines at once
  const int rot = ROT ? (int)(blockIdx.x % (unsigned)nk) : 0;
  auto issue = [&](int kt) {
    const uint32_t st = lds0 + (kt % NS) * STAGE;
    int ks = kt + rot;
    ks -= ks >= nk ? nk : 0;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (i < cnt) dma16(src[i] + ks * 64, st + (wave + NW * i) * 1024);
  };

  f32x16_t acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
  for (int s2 = 0; s2 < NS - 1; ++s2)
    if (s2 < nk) issue(s2);
  const int ra = wt * 32 + (lane & 31), rb = TM + we * 32 + (lane & 31);
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt has landed once at most (stages issued after it) * cnt copies of this wave are
    // outstanding (loads complete in order); the barrier covers the other waves' copies
    const int later = min(NS - 2, nk - 1 - kt);  // stages issued after stage kt
    if (cnt == PER) wait_vm_barrier_rt<(NS - 2) * PER>(later * PER);
    else wait_vm_barrier_rt<(NS - 2) * (PER - 1)>(later * (PER - 1));
    if (kt + NS - 1 < nk) issue(kt + NS - 1);  // the buffer of stage kt - 1, read by every wave already
    const uint8_t* sa = &s_tile[(kt % NS) * STAGE];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int chunk = ks * 2 + (lane >> 5);
      const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(sa + ra * 128 + ((chunk ^ swz<8>(ra)) << 4));
      const bf16x8_t bf = *reinterpret_cast<const bf16x8_t*>(sa + rb * 128 + ((chunk ^ swz<8>(rb)) << 4));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, acc, 0, 0, 0);
    }
  }
  __syncthreads();  // every wave is done with the stages: the logits tile reuses them
  float* s_l = reinterpret_cast<float*>(s_tile);
  // acc[v]: token 8 (v / 4) + 4 (lane / 32) + (v % 4) of the wave's 32, expert lane % 32 of its 32
#pragma unroll
  for (int v = 0; v < 16; ++v)
    s_l[(wt * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)) * LS + we * 32 + (lane & 31)] = acc[v];
  __syncthreads();

  double pacc[EL];
  float lb[EL], sb[EL];
#pragma unroll
  for (int m = 0; m < EL; ++m) {
    const int e = lane + kWave * m;
    pacc[m] = 0.0;
    lb[m] = (logit_bias && e < E) ? logit_bias[e] : 0.f;
    sb[m] = (select_bias && e < E) ? select_bias[e] : 0.f;
  }
  for (int tt = wave; tt < TM; tt += NW) {
    const int t = t0 + tt;
    if (t >= N) break;
    float v[EL];
#pragma unroll
    for (int m = 0; m < EL; ++m) {
      const int e = lane + kWave * m;
      v[m] = (e < E) ? s_l[tt * LS + e] + lb[m] : -INFINITY;
    }
    select_token<EL>(v, sb, lane, E, k, renorm, topk_idx + (size_t)t * k, topk_w + (size_t)t * k, pacc);
  }
  double* s_part = reinterpret_cast<double*>(s_tile + TM * LS * 4);  // past the logits tile
#pragma unroll
  for (int m = 0; m < EL; ++m) s_part[wave * kWave * EL + lane + kWave * m] = pacc[m];
  __syncthreads();
  for (int e = tid; e < E; e += NT) {
    double a = s_part[e];
#pragma unroll
    for (int q = 1; q < NW; ++q) a += s_part[q * kWave * EL + e];
    partials[(size_t)blockIdx.x * E + e] = a;
  }
}

// ---------------------------------------------------------------- 3. prob_sum

// prob_sum[e] = sum over select workgroups b of partials[b][e]: lane l adds
// b = l, l+64, ... in order, then a butterfly adds the 64 lane sums.
__global__ __launch_bounds__(kThreads) void prob_sum_kernel(const double* __restrict__ partials,
                                                           int nb, int E, double* __restrict__ prob_sum) {
  const int e = blockIdx.x * (kThreads / kWave) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (e >= E) return;
  const double a = prob_sum_wave(partials, nb, E, e, lane);
  if (lane == 0) prob_sum[e] = a;
}

// ---------------------------------------------------------------- 4. training-side statistics
//
// Side outputs for training (the forward does not use them). Readings of the
// pages, whose formulas were lost in extraction:
//   z-loss (notes, section 三.3): (1/N) sum_t logsumexp(l[t, :])^2 on the
//     logits that enter the softmax;
//   importance (notes, section 二): per expert, the sum of the gate weights
//     w of the copies routed to it, and its squared coefficient of variation;
//   aux-loss-free balancing (handbook, "负载均衡"): b_e -= gamma *
//     sign(counts_e - N k / E).
// Every sum runs in a fixed order, so the results are reproducible bit for bit.

// One wavefront per token: splits added in split order, then the logit bias,
// logsumexp in fp32; each workgroup adds its tokens' squares in fp64 in a
// fixed order.
template <int EL>
__global__ __launch_bounds__(kThreads) void lse_sq_kernel(const float* __restrict__ part, int splits,
                                                          const float* __restrict__ logit_bias, int N,
                                                          int E, int tpb, double* __restrict__ partials) {
  __shared__ double s_sq[kThreads / kWave];
  const int tid = threadIdx.x;
  const int wv = tid >> 6, lane = tid & 63;
  const size_t split_stride = (size_t)N * E;
  double acc = 0.0;
  for (int tt = wv; tt < tpb; tt += kThreads / kWave) {
    const int t = blockIdx.x * tpb + tt;
    if (t >= N) break;
    float v[EL];
    float mx = -INFINITY;
#pragma unroll
    for (int m = 0; m < EL; ++m) {
      const int e = lane + kWave * m;
      float l = -INFINITY;
      if (e < E) {
        const float* src = part + (size_t)t * E + e;
        l = 0.f;
        for (int q = 0; q < splits; ++q) l += src[(size_t)q * split_stride];
        if (logit_bias) l += logit_bias[e];
      }
      v[m] = l;
      mx = fmaxf(mx, l);
    }
    mx = wave_max(mx);
    float sum = 0.f;
#pragma unroll
    for (int m = 0; m < EL; ++m) sum += (lane + kWave * m < E) ? expf(v[m] - mx) : 0.f;
    sum = wave_sum(sum);
    const double lse = (double)(mx + logf(sum));
    acc += lse * lse;  // the same value in every lane
  }
  if (lane == 0) s_sq[wv] = acc;
  __syncthreads();
  if (tid == 0) {
    double a = s_sq[0];
#pragma unroll
    for (int q = 1; q < kThreads / kWave; ++q) a += s_sq[q];
    partials[blockIdx.x] = a;
  }
}

// One wavefront: out = scale * sum of v[0..n): lane-strided sums, then a fixed butterfly.
__global__ __launch_bounds__(kWave) void sum_f64_kernel(const double* __restrict__ v, int n, double scale,
                                                        double* __restrict__ out) {
  const int lane = threadIdx.x;
  double a = 0.0;
  for (int i = lane; i < n; i += kWave) a += v[i];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) a += __shfl_xor(a, o, kWave);
  if (lane == 0) *out = a * scale;
}

// One wavefront per expert: the gate weights of the copies routed to it.
__global__ __launch_bounds__(kThreads) void importance_kernel(const int32_t* __restrict__ idx,
                                                              const float* __restrict__ w, int NK, int E,
                                                              double* __restrict__ imp) {
  const int e = blockIdx.x * (kThreads / kWave) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (e >= E) return;
  double a = 0.0;
  for (int c = lane; c < NK; c += kWave)
    if (idx[c] == e) a += (double)w[c];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) a += __shfl_xor(a, o, kWave);
  if (lane == 0) imp[e] = a;
}

// One wavefront: Var/Mean^2 of imp[0..E) (population variance; 0 when the mean is 0).
__global__ __launch_bounds__(kWave) void cv2_kernel(const double* __restrict__ imp, int E,
                                                    double* __restrict__ out) {
  const int lane = threadIdx.x;
  double a = 0.0;
  for (int e = lane; e < E; e += kWave) a += imp[e];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) a += __shfl_xor(a, o, kWave);
  const double mean = a / E;
  double v = 0.0;
  for (int e = lane; e < E; e += kWave) v += (imp[e] - mean) * (imp[e] - mean);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  if (lane == 0) *out = mean == 0.0 ? 0.0 : (v / E) / (mean * mean);
}

// b_e -= gamma * sign(counts_e - N k / E), the sign taken exactly on integers (counts_e * E vs N k).
__global__ void bias_update_kernel(const int32_t* __restrict__ counts, long long nk, int E, float gamma,
                                   float* __restrict__ bias) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const long long c = (long long)counts[e] * E;
  if (c > nk) bias[e] = bias[e] - gamma;
  else if (c < nk) bias[e] = bias[e] + gamma;
}

// ---------------------------------------------------------------- launch

struct LogitsPlan {
  int eg, ept, tpt, tt, tiles, etiles, splits, chunks_per_split;
};

LogitsPlan plan_logits(const moe_shape& s) {
  LogitsPlan L;
  const int E = s.n_experts;
  if (E <= 8) { L.eg = 8; L.ept = 1; L.tpt = 4; }
  else if (E <= 32) { L.eg = 32; L.ept = 1; L.tpt = 4; }
  else if (E <= 64) { L.eg = 32; L.ept = 2; L.tpt = 4; }
  else if (E <= 128) { L.eg = 32; L.ept = 4; L.tpt = s.n_tokens >= 8192 ? 8 : 4; }  // 8 tokens: fewer LDS reads per dot
  else if (E <= 256) { L.eg = 32; L.ept = 8; L.tpt = 4; }
  else { L.eg = 32; L.ept = 16; L.tpt = 2; }
  L.tt = (kThreads / L.eg) * L.tpt;
  L.tiles = (s.n_tokens + L.tt - 1) / L.tt;
  L.etiles = 1;
  if (L.tiles < kFewTiles) {
    // few tokens: one expert (or 8) per thread and one token per thread, and
    // the experts split over workgroups, so that the chip fills with few K
    // splits (the select kernel adds the splits one by one)
    L.eg = E <= 8 ? 8 : 32;
    L.ept = 1;
    L.tpt = 1;
    L.tt = kThreads / L.eg;
    L.tiles = (s.n_tokens + L.tt - 1) / L.tt;
    L.etiles = (E + L.eg - 1) / L.eg;
  }
  const int dw = s.dtype == MOE_DTYPE_BF16 ? s.d_model / 2 : s.d_model;
  const int nchunks = dw / kChunk;
  // enough workgroups to fill the chip, each with at least two chunks of K
  const int tiles = std::max(1, L.tiles * L.etiles);
  int splits = (kTargetBlocks + tiles - 1) / tiles;
  splits = std::max(1, std::min({splits, kMaxSplits, nchunks / 2}));
  L.chunks_per_split = (nchunks + splits - 1) / splits;
  L.splits = (nchunks + L.chunks_per_split - 1) / L.chunks_per_split;
  return L;
}

template <bool BF16, int EG, int EPT, int TPT>
void launch_logits_t(const moe_shape& s, const LogitsPlan& L, const void* x, const void* w,
                     float* part, unsigned int* clear, hipStream_t st) {
  const int dw = BF16 ? s.d_model / 2 : s.d_model;
  // one output per thread: registers to spare for a deep prefetch ring (a split of up to 16
  // chunks then has every load in flight at once)
  constexpr int PD = TPT == 1 ? 16 : 1;
  hipLaunchKernelGGL((logits_kernel<BF16, EG, EPT, TPT, PD>), dim3(L.tiles, L.splits, L.etiles), dim3(kThreads), 0, st,
                     static_cast<const uint32_t*>(x), static_cast<const uint32_t*>(w), s.n_tokens, dw,
                     s.n_experts, L.chunks_per_split, part, clear);
}

template <bool BF16>
void launch_logits(const moe_shape& s, const LogitsPlan& L, const void* x, const void* w, float* part,
                   unsigned int* clear, hipStream_t st) {
  if (L.tpt == 1) {
    if (L.eg == 8) launch_logits_t<BF16, 8, 1, 1>(s, L, x, w, part, clear, st);
    else launch_logits_t<BF16, 32, 1, 1>(s, L, x, w, part, clear, st);
  } else if (L.eg == 8) launch_logits_t<BF16, 8, 1, 4>(s, L, x, w, part, clear, st);
  else if (L.ept == 1) launch_logits_t<BF16, 32, 1, 4>(s, L, x, w, part, clear, st);
  else if (L.ept == 2) launch_logits_t<BF16, 32, 2, 4>(s, L, x, w, part, clear, st);
  else if (L.ept == 4 && L.tpt == 8) launch_logits_t<BF16, 32, 4, 8>(s, L, x, w, part, clear, st);
  else if (L.ept == 4) launch_logits_t<BF16, 32, 4, 4>(s, L, x, w, part, clear, st);
  else if (L.ept == 8) launch_logits_t<BF16, 32, 8, 4>(s, L, x, w, part, clear, st);
  else launch_logits_t<BF16, 32, 16, 2>(s, L, x, w, part, clear, st);
}

}  // namespace

// tokens per select workgroup: enough workgroups (>= 256) at small N, 32 at most
int select_tpb(const moe_shape& s) {
  return std::max(4, std::min(kSelTokMax, (s.n_tokens / 256) / 4 * 4));
}

int route_blocks(const moe_shape& s) {
  const int tpb = select_tpb(s);
  return (s.n_tokens + tpb - 1) / tpb;
}

size_t route_partials_bytes(const moe_shape& s) {
  return (size_t)route_blocks(s) * s.n_experts * sizeof(double) + 64;  // the sums, then the select counter
}

unsigned int* route_counter(const moe_shape& s, double* partials) {
  return reinterpret_cast<unsigned int*>(partials + (size_t)route_blocks(s) * s.n_experts);
}

// Large bf16 routers go to the matrix cores: logits = x W_r^T is then one grouped
// GEMM (one segment of N rows, K = d, W_r as the [E, d] weight), fp32 sums of exact
// bf16 products as on the VALU path, in another order.
bool logits_by_mfma(const moe_shape& s) {
  return s.dtype == MOE_DTYPE_BF16 && s.n_experts >= 64 && s.n_tokens >= 256;
}

// clear: a counter for the select kernel, zeroed by the VALU logits kernel
// (nothing is written to it when the logits run on the matrix cores).
int compute_logits(const moe_shape& s, const void* x, const void* w_router, float* logits, float* split_ws,
                   size_t split_bytes, int* splits, hipStream_t st, unsigned int* clear = nullptr) {
  if (logits_by_mfma(s)) {
    GroupedParams p{};
    p.n_sets = 1;
    p.x = x;
    p.n_tokens = s.n_tokens;
    p.d_model = s.n_experts;  // output columns
    p.dtype = MOE_DTYPE_BF16;
    p.split_ws = split_ws;
    p.split_cap = split_ws ? (long long)(split_bytes / sizeof(float)) : 0;
    SegSet& S = p.set[0];
    S.n_groups = 1;
    S.uniform_rows = s.n_tokens;
    S.rows_per_token = 1;
    S.max_rows = s.n_tokens;
    S.d_ff = s.d_model;  // K
    S.w_gate = S.w_up = S.w_down = w_router;
    S.h = const_cast<void*>(x);
    S.out = logits;
    *splits = 1;
    return launch_grouped(p, 2, st);
  }
  const LogitsPlan L = plan_logits(s);
  if (s.dtype == MOE_DTYPE_BF16) launch_logits<true>(s, L, x, w_router, logits, clear, st);
  else launch_logits<false>(s, L, x, w_router, logits, clear, st);
  *splits = L.splits;
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

size_t route_logits_floats(const moe_shape& s) {
  if (logits_by_mfma(s)) return (size_t)s.n_tokens * s.n_experts;
  const LogitsPlan L = plan_logits(s);
  return (size_t)L.splits * s.n_tokens * s.n_experts;
}

// The fused router (2b) serves bf16 layers with 64 <= E <= 256 and enough tokens
// to give the chip a workgroup per CU or so; the others take logits + select.
bool route_fused(const moe_shape& s) {
  return s.dtype == MOE_DTYPE_BF16 && s.n_experts >= 64 && s.n_experts <= 256 && s.n_tokens >= 1024;
}

template <int WT, int NS, bool ROT>
void launch_route_fused_t(const moe_shape& s, const void* x, const void* w_router, const float* logit_bias,
                          const float* select_bias, int32_t* topk_idx, float* topk_w, double* partials, int* nb,
                          hipStream_t st) {
  constexpr int TM = 32 * WT;
  *nb = (s.n_tokens + TM - 1) / TM;
  hipLaunchKernelGGL((route_fused_kernel<WT, NS, ROT>), dim3(*nb), dim3(512), 0, st, static_cast<const bf16_t*>(x),
                     static_cast<const bf16_t*>(w_router), logit_bias, select_bias, s.n_tokens, s.d_model,
                     s.n_experts, s.top_k, s.renormalize, topk_idx, topk_w, partials);
}

int launch_prob_sum(const double* partials, int nb, int E, double* prob_sum, hipStream_t stream) {
  hipLaunchKernelGGL(prob_sum_kernel, dim3((E + 3) / 4), dim3(kThreads), 0, stream, partials, nb, E, prob_sum);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int launch_route(const moe_shape& s, const void* x, const void* w_router, const float* logit_bias,
                 const float* select_bias, int32_t* topk_idx, float* topk_w, double* prob_sum,
                 double* partials, float* logits, float* split_ws, size_t split_bytes, hipStream_t stream,
                 int* defer_nb) {
  if (defer_nb) *defer_nb = 0;
  if (route_fused(s)) {
    int nb = 0;
    if (s.n_experts <= 64)        // 128 tokens x 64 experts per workgroup
      launch_route_fused_t<4, 4, true>(s, x, w_router, logit_bias, select_bias, topk_idx, topk_w, partials, &nb, stream);
    else if (s.n_experts <= 128)  // 64 x 128
      launch_route_fused_t<2, 4, true>(s, x, w_router, logit_bias, select_bias, topk_idx, topk_w, partials, &nb, stream);
    else                          // 32 x 256
      launch_route_fused_t<1, 4, true>(s, x, w_router, logit_bias, select_bias, topk_idx, topk_w, partials, &nb, stream);
    if (defer_nb) {
      *defer_nb = nb;
      return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
    }
    return launch_prob_sum(partials, nb, s.n_experts, prob_sum, stream);
  }
  const int nb = route_blocks(s);
  // the select kernel's counter sits after the workgroup sums; the VALU logits
  // kernel clears it, and then the last select workgroup adds the sums
  unsigned int* done = logits_by_mfma(s) || nb > kFoldBlocks ? nullptr : route_counter(s, partials);
  int splits = 1;
  if (const int st = compute_logits(s, x, w_router, logits, split_ws, split_bytes, &splits, stream, done)) return st;
  const int el = (s.n_experts + kWave - 1) / kWave;
#define MOE_SELECT(EL_)                                                                          \
  hipLaunchKernelGGL(select_kernel<EL_>, dim3(nb), dim3(kThreads), 0, stream, logits, splits, \
                     logit_bias, select_bias, s.n_tokens, s.n_experts, s.top_k, s.renormalize,   \
                     select_tpb(s), topk_idx, topk_w, partials, done, prob_sum)
  if (el <= 1) MOE_SELECT(1);
  else if (el <= 2) MOE_SELECT(2);
  else if (el <= 4) MOE_SELECT(4);
  else MOE_SELECT(8);
#undef MOE_SELECT
  if (done) return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
  if (defer_nb) {
    *defer_nb = nb;
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
  }
  return launch_prob_sum(partials, nb, s.n_experts, prob_sum, stream);
}

int launch_router_logits(const moe_shape& s, const void* x, const void* w_router, float* logits, int* splits,
                         float* split_ws, size_t split_bytes, hipStream_t stream) {
  return compute_logits(s, x, w_router, logits, split_ws, split_bytes, splits, stream);
}

int launch_router_aux(const moe_shape& s, const void* x, const void* w_router, const float* logit_bias,
                      const int32_t* topk_idx, const float* topk_w, double* z_loss, double* imp,
                      double* imp_cv2, double* partials, float* logits, float* split_ws, size_t split_bytes,
                      hipStream_t stream) {
  const int N = s.n_tokens, E = s.n_experts;
  if (z_loss) {
    int splits = 1;
    if (const int st = compute_logits(s, x, w_router, logits, split_ws, split_bytes, &splits, stream)) return st;
    const int nb = route_blocks(s);
    const int el = (E + kWave - 1) / kWave;
#define MOE_LSE(EL_)                                                                                \
  hipLaunchKernelGGL(lse_sq_kernel<EL_>, dim3(nb), dim3(kThreads), 0, stream, logits, splits, logit_bias, \
                     N, E, select_tpb(s), partials)
    if (el <= 1) MOE_LSE(1);
    else if (el <= 2) MOE_LSE(2);
    else if (el <= 4) MOE_LSE(4);
    else MOE_LSE(8);
#undef MOE_LSE
    hipLaunchKernelGGL(sum_f64_kernel, dim3(1), dim3(kWave), 0, stream, partials, nb, 1.0 / N, z_loss);
  }
  if (imp) {
    hipLaunchKernelGGL(importance_kernel, dim3((E + 3) / 4), dim3(kThreads), 0, stream, topk_idx, topk_w,
                       N * s.top_k, E, imp);
    if (imp_cv2) hipLaunchKernelGGL(cv2_kernel, dim3(1), dim3(kWave), 0, stream, imp, E, imp_cv2);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int launch_bias_update(const moe_shape& s, const int32_t* counts, float gamma, float* bias,
                       hipStream_t stream) {
  hipLaunchKernelGGL(bias_update_kernel, dim3((s.n_experts + 255) / 256), dim3(256), 0, stream, counts,
                     (long long)s.n_tokens * s.top_k, s.n_experts, gamma, bias);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
