// Grouped SwiGLU experts: one GEMM per expert segment, for all segments in
// one launch per projection.
//
// Expert.forward in "混合专家 MoE" (anrans ai-infra handbook), section
// "实现：逐 token 与按专家分组", is down(silu(gate(x)) * up(x)).
// forward_grouped runs it once per expert over that expert's rows. The same
// section describes grouping plus one grouped GEMM over all experts as the
// skeleton of a fused MoE kernel. Two phases:
//   phase 1  H[r, :] = bf16( silu(x_r Wg^T) * (x_r Wu^T) ).
//            Gate and up tiles are computed side by side, so the SiLU*up
//            epilogue stays in registers.
//   phase 2  O[r, :] = H[r, :] Wd^T, written in fp32.
//
// bf16 path (gfx950 matrix cores):
//   - v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
//   - Both operands are K-contiguous: x rows, and weights stored
//     [out, in] like nn.Linear. Each lane's MFMA operand is one 16-byte
//     piece of a row.
//   - Tiles are BM x BN x 64, double buffered in LDS. Each 128-byte LDS row
//     stores its eight 16-byte pieces XOR-swizzled by (row & 7) ^ ((row >> 3)
//     & 1). The MFMA reads then hit distinct banks whether the LDS serves
//     128 or 256 bytes per clock.
//   - A persistent grid walks a tile list built on the device from the
//     segment offsets, so no host round trip is needed.
//       * Tiles go (segment, n-tile, m-tile), with the m-tile fastest, so
//         that neighbouring tiles share a weight tile.
//       * Workgroup ids are remapped so that each XCD (and its L2) works on
//         a contiguous run of tiles.
//       * Empty segments produce no tiles.
// fp32 path: a plain LDS-tiled SIMT kernel for fp32 layers.
#include <math.h>

#include "moe_common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kXcds = 8;

struct SetView {  // the fields of one SegSet, picked with selects rather than a dynamic index
  const int32_t* perm;
  int32_t rpt;
  int32_t d_ff;
  const void* wg;
  const void* wu;
  const void* wd;
  void* h;
  float* out;
};

__device__ __forceinline__ SetView pick(const GroupedParams& p, int si) {
  SetView v;
  v.perm = si ? p.set[1].perm : p.set[0].perm;
  v.rpt = si ? p.set[1].rows_per_token : p.set[0].rows_per_token;
  v.d_ff = si ? p.set[1].d_ff : p.set[0].d_ff;
  v.wg = si ? p.set[1].w_gate : p.set[0].w_gate;
  v.wu = si ? p.set[1].w_up : p.set[0].w_up;
  v.wd = si ? p.set[1].w_down : p.set[0].w_down;
  v.h = si ? p.set[1].h : p.set[0].h;
  v.out = si ? p.set[1].out : p.set[0].out;
  return v;
}

__device__ __forceinline__ void seg_bounds(const SegSet& S, int g, int& start, int& rows) {
  int a, b;
  if (S.offsets) {
    a = S.offsets[g];
    b = S.offsets[g + 1];
  } else {
    a = g * S.uniform_rows;
    b = a + S.uniform_rows;
  }
  a = max(0, min(a, S.max_rows));
  b = max(a, min(b, S.max_rows));
  start = a;
  rows = b - a;
}

// LDS tile table: entry i (routed groups, then shared groups) owns tiles
// [cum[i], cum[i+1]). Built by every workgroup from the device offsets.
struct TableLds {
  int cum[kMaxTileEntries + 1];
  int start[kMaxTileEntries];
  int rows[kMaxTileEntries];
  int tmp[kThreads];
};

template <int BM>
__device__ int build_table(const GroupedParams& p, int nt0, int nt1, TableLds& t) {
  const int G0 = p.set[0].n_groups;
  const int G1 = p.n_sets > 1 ? p.set[1].n_groups : 0;
  const int n = G0 + G1;
  const int tid = threadIdx.x;
  const int per = (n + kThreads - 1) / kThreads;  // <= 4
  int local[kMaxTileEntries / kThreads];
  int sum = 0;
#pragma unroll
  for (int q = 0; q < kMaxTileEntries / kThreads; ++q) {
    local[q] = 0;
    const int i = tid * per + q;
    if (q < per && i < n) {
      int start, rows;
      if (i < G0) seg_bounds(p.set[0], i, start, rows);
      else seg_bounds(p.set[1], i - G0, start, rows);
      t.start[i] = start;
      t.rows[i] = rows;
      local[q] = ((rows + BM - 1) / BM) * (i < G0 ? nt0 : nt1);
      sum += local[q];
    }
  }
  t.tmp[tid] = sum;
  __syncthreads();
  for (int o = 1; o < kThreads; o <<= 1) {
    const int add = tid >= o ? t.tmp[tid - o] : 0;
    __syncthreads();
    t.tmp[tid] += add;
    __syncthreads();
  }
  int run = tid ? t.tmp[tid - 1] : 0;
#pragma unroll
  for (int q = 0; q < kMaxTileEntries / kThreads; ++q) {
    const int i = tid * per + q;
    if (q < per && i < n) {
      t.cum[i] = run;
      run += local[q];
    }
  }
  if (tid == kThreads - 1) t.cum[n] = t.tmp[kThreads - 1];
  __syncthreads();
  return t.cum[n];
}

__device__ __forceinline__ int find_entry(const int* cum, int n, int T) {
  int lo = 0, hi = n;  // cum[lo] <= T < cum[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cum[mid] <= T) lo = mid;
    else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ int xcd_block() {
  // hardware places workgroup b on XCD b % 8; give each XCD a contiguous run
  const int G = gridDim.x;  // a multiple of kXcds
  const int b = blockIdx.x;
  return (b % kXcds) * (G / kXcds) + b / kXcds;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.f + expf(-g)) * u; }

// =====================================================================  bf16 MFMA

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

template <int BM, int BN, int WGM, int WGN, bool P1>
__global__ __launch_bounds__(kThreads, 1) void grouped_mfma_kernel(GroupedParams p) {
  constexpr int BK = 64;              // bf16 per K step
  constexpr int ROWB = BK * 2;        // LDS bytes per tile row
  constexpr int TM = BM / WGM;        // rows per wave
  constexpr int FM = TM / 32;
  constexpr int BH = P1 ? BN / 2 : BN;  // output columns per tile
  constexpr int TN = BH / WGN;          // output columns per wave
  constexpr int FN = TN / 32;
  constexpr int NB = P1 ? 2 * FN : FN;  // B fragments per k-step
  constexpr int A_PER = BM * 8 / kThreads;
  constexpr int B_PER = BN * 8 / kThreads;
  static_assert(A_PER >= 1 && B_PER >= 2 && FM >= 1 && FN >= 1, "tile shape");

  __shared__ __attribute__((aligned(16))) uint8_t s_a[2][BM * ROWB];
  __shared__ __attribute__((aligned(16))) uint8_t s_b[2][BN * ROWB];
  __shared__ TableLds tab;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int d = p.d_model;
  // output columns per set (h columns in phase 1, d in phase 2); the last n-tile may be partial
  const int nt0 = ((P1 ? p.set[0].d_ff : d) + BH - 1) / BH;
  const int nt1 = p.n_sets > 1 ? ((P1 ? p.set[1].d_ff : d) + BH - 1) / BH : 0;
  const int G0 = p.set[0].n_groups;
  const int nent = G0 + (p.n_sets > 1 ? p.set[1].n_groups : 0);
  const int total = build_table<BM>(p, nt0, nt1, tab);
  const bf16_t* __restrict__ xg = static_cast<const bf16_t*>(p.x);

  // this thread's load slots: row (tid >> 3) + 32 q, 16-byte piece (tid & 7)
  const int lrow = tid >> 3, lpc = tid & 7;

  for (int T = xcd_block(); T < total; T += gridDim.x) {
    const int ent = find_entry(tab.cum, nent, T);
    const int si = ent < G0 ? 0 : 1;
    const int g = si ? ent - G0 : ent;
    const SetView S = pick(p, si);
    const int start = tab.start[ent], rows = tab.rows[ent];
    const int mt = (rows + BM - 1) / BM;
    const int local = T - tab.cum[ent];
    const int ntile = local / mt, mtile = local - ntile * mt;
    const int m0 = mtile * BM;
    const int mvalid = min(BM, rows - m0);
    const int n0 = ntile * BH;
    const int F = S.d_ff;
    const int K = P1 ? d : F;
    const int nk = K / BK;

    // ---- global sources: 32-bit element offsets of this thread's 16-byte pieces.
    // Rows past the segment (or tokens out of range) load row 0 of the
    // source and are zeroed after the load.
    const bf16_t* a_base = P1 ? xg : static_cast<const bf16_t*>(S.h);
    uint32_t a_off[A_PER];
    uint32_t a_ok = 0;
#pragma unroll
    for (int q = 0; q < A_PER; ++q) {
      const int r = lrow + 32 * q;
      uint32_t off = 0;
      if (r < mvalid) {
        const int row = start + m0 + r;
        if constexpr (P1) {
          const int tok = S.perm ? S.perm[row] / S.rpt : row - start;
          if ((unsigned)tok < (unsigned)p.n_tokens) {
            off = (uint32_t)tok * (uint32_t)d + lpc * 8;
            a_ok |= 1u << q;
          }
        } else {
          off = (uint32_t)row * (uint32_t)F + lpc * 8;
          a_ok |= 1u << q;
        }
      }
      a_off[q] = off;
    }
    // B rows: weight rows n0 + lrow + 32 q. Rows past the last output column
    // (a partial n-tile; columns come in multiples of 64) re-read an in-range
    // row, and their results are never stored.
    const int ncols = P1 ? F : d;
    const int qmax = (min(BH, ncols - n0) + 31) / 32 - 1;
    constexpr int BQ = P1 ? B_PER / 2 : B_PER;  // B pieces per weight matrix
    const bf16_t* b_base0;  // gate (phase 1) or down (phase 2) weights of group g
    const bf16_t* b_base1;  // up weights of group g (phase 1)
    if constexpr (P1) {
      b_base0 = static_cast<const bf16_t*>(S.wg) + (size_t)g * F * d;
      b_base1 = static_cast<const bf16_t*>(S.wu) + (size_t)g * F * d;
    } else {
      b_base0 = static_cast<const bf16_t*>(S.wd) + (size_t)g * d * F;
      b_base1 = b_base0;
    }
    uint32_t b_off[BQ];
#pragma unroll
    for (int q = 0; q < BQ; ++q) b_off[q] = (uint32_t)(n0 + lrow + 32 * min(q, qmax)) * (uint32_t)K + lpc * 8;
    // LDS byte offsets of this thread's pieces (same for both buffers)
    uint32_t a_lds[A_PER], b_lds[B_PER];
#pragma unroll
    for (int q = 0; q < A_PER; ++q) {
      const int r = lrow + 32 * q;
      a_lds[q] = r * ROWB + ((lpc ^ swz(r)) << 4);
    }
#pragma unroll
    for (int q = 0; q < B_PER; ++q) {
      // phase 1: pieces [0, BQ) are gate rows (tile rows [0, BN/2)), [BQ, 2 BQ) up rows
      const int r = lrow + 32 * (q % BQ) + (q / BQ) * (BN / 2);
      b_lds[q] = r * ROWB + ((lpc ^ swz(r)) << 4);
    }

    u32x4_t ra[A_PER], rb[B_PER];
#define MOE_GLOAD(KT)                                                                      \
  {                                                                                        \
    const int ko_ = (KT) * BK;                                                             \
    _Pragma("unroll") for (int q = 0; q < A_PER; ++q) {                                    \
      ra[q] = *reinterpret_cast<const u32x4_t*>(a_base + a_off[q] + ko_);                    \
    }                                                                                      \
    _Pragma("unroll") for (int q = 0; q < BQ; ++q) {                                       \
      rb[q] = *reinterpret_cast<const u32x4_t*>(b_base0 + b_off[q] + ko_);                 \
      if constexpr (P1) rb[q + BQ] = *reinterpret_cast<const u32x4_t*>(b_base1 + b_off[q] + ko_); \
    }                                                                                      \
  }
#define MOE_LSTORE(BUF)                                                                    \
  {                                                                                        \
    _Pragma("unroll") for (int q = 0; q < A_PER; ++q) {                                    \
      u32x4_t v_ = ra[q];                                                                    \
      if (!((a_ok >> q) & 1u)) v_ = u32x4_t{0u, 0u, 0u, 0u};                                \
      *reinterpret_cast<u32x4_t*>(&s_a[BUF][a_lds[q]]) = v_;                                 \
    }                                                                                      \
    _Pragma("unroll") for (int q = 0; q < B_PER; ++q) {                                    \
      *reinterpret_cast<u32x4_t*>(&s_b[BUF][b_lds[q]]) = rb[q];                              \
    }                                                                                      \
  }

    f32x16_t acc[FM][NB];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    __syncthreads();  // previous tile's LDS reads are done
    MOE_GLOAD(0);
    MOE_LSTORE(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < nk) MOE_GLOAD(kt + 1);
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int chunk = ks * 2 + (lane >> 5);
        bf16x8_t af[FM], bfr[NB];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int r = wm * TM + i * 32 + (lane & 31);
          af[i] = *reinterpret_cast<const bf16x8_t*>(&s_a[buf][r * ROWB + ((chunk ^ swz(r)) << 4)]);
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          // phase 1: fragments [0, FN) are gate rows, [FN, 2 FN) the matching up rows
          const int jj = P1 ? (j % FN) : j;
          const int half = P1 ? (j / FN) * (BN / 2) : 0;
          const int r = half + wn * TN + jj * 32 + (lane & 31);
          bfr[j] = *reinterpret_cast<const bf16x8_t*>(&s_b[buf][r * ROWB + ((chunk ^ swz(r)) << 4)]);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < nk) MOE_LSTORE(buf ^ 1);
      __syncthreads();
    }
#undef MOE_GLOAD
#undef MOE_LSTORE

    // ---- epilogue. acc[i][j][v]: column (lane & 31), row 8 (v / 4) + 4 (lane / 32) + (v % 4)
    const int col_l = lane & 31;
    const int col0 = n0 + wn * TN + col_l;  // this lane's first output column
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * TM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (r >= mvalid) continue;
        const size_t row = (size_t)(start + m0 + r);
        if constexpr (P1) {
          bf16_t* hrow = static_cast<bf16_t*>(S.h) + row * F + col0;
#pragma unroll
          for (int j = 0; j < FN; ++j)
            if (col0 + j * 32 < ncols) hrow[j * 32] = f32_to_bf16(silu_mul(acc[i][j][v], acc[i][j + FN][v]));
        } else {
          float* orow = S.out + row * d + col0;
#pragma unroll
          for (int j = 0; j < FN; ++j)
            if (col0 + j * 32 < ncols) orow[j * 32] = acc[i][j][v];
        }
      }
    }
  }
}

// =====================================================================  fp32 SIMT

template <bool P1>
__global__ __launch_bounds__(kThreads) void grouped_f32_kernel(GroupedParams p) {
  constexpr int BM = 32, BC = 32, BK = 32;
  __shared__ float s_a[BM][BK + 1];
  __shared__ float s_b0[BC][BK + 1];
  __shared__ float s_b1[BC][BK + 1];
  __shared__ TableLds tab;
  const int tid = threadIdx.x;
  const int tx = tid & 31, ty = tid >> 5;
  const int d = p.d_model;
  const int nt0 = (P1 ? p.set[0].d_ff : d) / BC;
  const int nt1 = p.n_sets > 1 ? (P1 ? p.set[1].d_ff : d) / BC : 0;
  const int G0 = p.set[0].n_groups;
  const int nent = G0 + (p.n_sets > 1 ? p.set[1].n_groups : 0);
  const int total = build_table<BM>(p, nt0, nt1, tab);
  const float* __restrict__ xg = static_cast<const float*>(p.x);

  for (int T = xcd_block(); T < total; T += gridDim.x) {
    const int ent = find_entry(tab.cum, nent, T);
    const int si = ent < G0 ? 0 : 1;
    const int g = si ? ent - G0 : ent;
    const SetView S = pick(p, si);
    const int start = tab.start[ent], rows = tab.rows[ent];
    const int mt = (rows + BM - 1) / BM;
    const int local = T - tab.cum[ent];
    const int ntile = local / mt, mtile = local - ntile * mt;
    const int m0 = mtile * BM, n0 = ntile * BC;
    const int mvalid = min(BM, rows - m0);
    const int F = S.d_ff;
    const int K = P1 ? d : F;
    float acc0[4] = {0.f, 0.f, 0.f, 0.f}, acc1[4] = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < K; k0 += BK) {
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = tid + kThreads * q;
        const int r = e >> 5, kk = e & 31;
        float a = 0.f;
        if (r < mvalid) {
          const int row = start + m0 + r;
          if constexpr (P1) {
            const int tok = S.perm ? S.perm[row] / S.rpt : row - start;
            if ((unsigned)tok < (unsigned)p.n_tokens) a = xg[(size_t)tok * d + k0 + kk];
          } else {
            a = static_cast<const float*>(S.h)[(size_t)row * F + k0 + kk];
          }
        }
        s_a[r][kk] = a;
        if constexpr (P1) {
          s_b0[r][kk] = static_cast<const float*>(S.wg)[((size_t)g * F + n0 + r) * d + k0 + kk];
          s_b1[r][kk] = static_cast<const float*>(S.wu)[((size_t)g * F + n0 + r) * d + k0 + kk];
        } else {
          s_b0[r][kk] = static_cast<const float*>(S.wd)[((size_t)g * d + n0 + r) * F + k0 + kk];
        }
      }
      __syncthreads();
#pragma unroll 8
      for (int kk = 0; kk < BK; ++kk) {
        const float b0 = s_b0[tx][kk];
        const float b1 = P1 ? s_b1[tx][kk] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = s_a[ty + 8 * i][kk];
          acc0[i] = fmaf(a, b0, acc0[i]);
          if (P1) acc1[i] = fmaf(a, b1, acc1[i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = ty + 8 * i;
      if (r >= mvalid) continue;
      const size_t row = (size_t)(start + m0 + r);
      if constexpr (P1) static_cast<float*>(S.h)[row * F + n0 + tx] = silu_mul(acc0[i], acc1[i]);
      else S.out[row * d + n0 + tx] = acc0[i];
    }
  }
}

int num_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

long long tiles_upper_bound(const GroupedParams& p, int phase, int BM, int BH) {
  long long ub = 0;
  for (int s = 0; s < p.n_sets; ++s) {
    const SegSet& S = p.set[s];
    const int nt = ((phase == 1 ? S.d_ff : p.d_model) + BH - 1) / BH;
    ub += ((long long)S.max_rows / BM + S.n_groups) * nt;
  }
  return ub;
}

int grid_for(long long ub, int per_cu) {
  long long g = std::min<long long>(ub, (long long)num_cus() * per_cu);
  g = std::max<long long>(g, 1);
  return (int)((g + kXcds - 1) / kXcds * kXcds);
}

template <int BM, int BN, int WGM, int WGN>
void launch_mfma(const GroupedParams& p, int phase, hipStream_t st) {
  const int BH = phase == 1 ? BN / 2 : BN;
  const int grid = grid_for(tiles_upper_bound(p, phase, BM, BH), 1);
  if (phase == 1)
    hipLaunchKernelGGL((grouped_mfma_kernel<BM, BN, WGM, WGN, true>), dim3(grid), dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL((grouped_mfma_kernel<BM, BN, WGM, WGN, false>), dim3(grid), dim3(kThreads), 0, st, p);
}

}  // namespace

int launch_grouped(const GroupedParams& p, int phase, hipStream_t stream) {
  if (p.dtype == MOE_DTYPE_F32) {
    const int grid = grid_for(tiles_upper_bound(p, phase, 32, 32), 4);
    if (phase == 1)
      hipLaunchKernelGGL(grouped_f32_kernel<true>, dim3(grid), dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL(grouped_f32_kernel<false>, dim3(grid), dim3(kThreads), 0, stream, p);
  } else {
    // tile height from the mean routed rows per expert segment
    const long long avg = (long long)p.set[0].max_rows / std::max(1, p.set[0].n_groups);
    if (avg >= 128) launch_mfma<256, 256, 2, 2>(p, phase, stream);
    else launch_mfma<64, 256, 1, 4>(p, phase, stream);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
