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
//       * Tiles go (segment, band of 8 m-tiles, n-tile, m-tile), with the
//         m-tile fastest, so that neighbouring tiles share a weight tile and
//         a run of them shares a few row tiles.
//       * Workgroup ids are remapped so that each XCD (and its L2) works on
//         a contiguous run of tiles.
//       * Empty segments produce no tiles.
// fp32 path: a plain LDS-tiled SIMT kernel for fp32 layers.
#include <math.h>

#include <type_traits>

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
  const float* sg;  // FP8 weights: row scales
  const float* su;
  const float* sd;
  void* h;
  float* out;
  const int32_t* kofs;  // weight-gradient mode (phase 2): per-group K ranges
  int32_t bsplit;       // N-major weights: rows >= bsplit come from wu (0: none)
  int32_t urows;        // rows per group of a uniform set
  float* gsave;         // phase 1: fp32 gate and up values (optional)
  float* usave;
};

__device__ __forceinline__ SetView pick(const GroupedParams& p, int si) {
  SetView v;
  v.perm = si ? p.set[1].perm : p.set[0].perm;
  v.rpt = si ? p.set[1].rows_per_token : p.set[0].rows_per_token;
  v.d_ff = si ? p.set[1].d_ff : p.set[0].d_ff;
  v.wg = si ? p.set[1].w_gate : p.set[0].w_gate;
  v.wu = si ? p.set[1].w_up : p.set[0].w_up;
  v.wd = si ? p.set[1].w_down : p.set[0].w_down;
  v.sg = si ? p.set[1].sc_gate : p.set[0].sc_gate;
  v.su = si ? p.set[1].sc_up : p.set[0].sc_up;
  v.sd = si ? p.set[1].sc_down : p.set[0].sc_down;
  v.h = si ? p.set[1].h : p.set[0].h;
  v.out = si ? p.set[1].out : p.set[0].out;
  v.kofs = si ? p.set[1].k_offsets : p.set[0].k_offsets;
  v.bsplit = si ? p.set[1].b_split : p.set[0].b_split;
  v.urows = si ? p.set[1].uniform_rows : p.set[0].uniform_rows;
  v.gsave = si ? p.set[1].g_save : p.set[0].g_save;
  v.usave = si ? p.set[1].u_save : p.set[0].u_save;
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
  if (S.k_offsets && S.skip_empty_k && S.k_offsets[g + 1] == S.k_offsets[g]) b = a;  // K_g = 0: no tiles
  start = a;
  rows = b - a;
}

// LDS tile table: entry i (routed groups, then shared groups) owns tiles
// [cum[i], cum[i+1]). Built by every workgroup from the device offsets.
struct TableLds {
  int cum[kMaxTileEntries + 1];
  int start[kMaxTileEntries];
  int rows[kMaxTileEntries];
};

// `scratch` holds NT ints of LDS that are free while the table is built.
template <int BM, int NT>
__device__ int build_table(const GroupedParams& p, int nt0, int nt1, TableLds& t, int* scratch) {
  constexpr int PER = (kMaxTileEntries + NT - 1) / NT;
  const int G0 = p.set[0].n_groups;
  const int G1 = p.n_sets > 1 ? p.set[1].n_groups : 0;
  const int n = G0 + G1;
  const int tid = threadIdx.x;
  const int per = (n + NT - 1) / NT;  // <= PER
  int local[PER];
  int sum = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
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
  scratch[tid] = sum;
  __syncthreads();
  for (int o = 1; o < NT; o <<= 1) {
    const int add = tid >= o ? scratch[tid - o] : 0;
    __syncthreads();
    scratch[tid] += add;
    __syncthreads();
  }
  int run = tid ? scratch[tid - 1] : 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int i = tid * per + q;
    if (q < per && i < n) {
      t.cum[i] = run;
      run += local[q];
    }
  }
  if (tid == NT - 1) t.cum[n] = scratch[NT - 1];
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

// bf16(silu(g) * u) for the bf16 epilogue: exp(-g) as the hardware exp2 of -g log2(e) and the
// hardware reciprocal (about 1 ulp of fp32 each, against 2^16 ulp per bf16 step), then the hardware
// round-to-nearest-even conversion. Large |g| gives the limits: e = inf -> -0, e = 0 -> g * u.
__device__ __forceinline__ bf16_t silu_mul_bf16(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(g * -1.44269504088896341f);
  const float s = g * __builtin_amdgcn_rcpf(1.f + e) * u;
  return __builtin_bit_cast(bf16_t, (__bf16)s);
}

// =====================================================================  bf16 MFMA

// N-major B tiles (the weight read in its stored orientation). The LDS tile
// holds BK k-rows of BN bf16 (n contiguous); 64-byte unit u of row k is stored
// at unit u ^ (k & 3). ds_read_b64_tr_b16 works on groups of 16 lanes: lane i
// of a group receives, as element j, element (i % 4) of the 8 bytes addressed
// by lane 4 j + i / 4 of the group. Each lane here addresses 4 consecutive n
// of one k-row: lane s reads row 8 (s / 32) + (s / 4) % 4 (+ 4 for the second
// read) at column 16 ((s / 16) % 2) + 4 (s % 4) of its 32-column block, so that
// lane L ends up with B[8 (L / 32) + t][L % 32], t = 0..7: the MFMA B fragment,
// in the same k order as the A fragment.
typedef short i16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i16x4_t lds_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(p));
}

template <int ROW>
__device__ __forceinline__ int nmajor_offset(int k, int n) {
  return k * ROW + ((((n >> 5) ^ (k & 3)) << 6) | ((n & 31) << 1));
}

constexpr int kBandM = 8;  // m-tiles per band of the tile order

// Int4 weights: a 32-bit word holds 8 codes q in [-7, 7] as 4-bit sign and
// magnitude (bit 3 the sign, bits 0..2 |q|); code j sits in byte j % 4, in
// its low nibble for j < 4 and its high nibble for j >= 4. Moving the sign
// bit to bit 7 of its byte makes each code the E4M3 byte whose value is
// q * 2^-9 (exponent field 0: a subnormal with mantissa |q|), which the FP8
// widening turns into bf16 exactly: the 8 operands of one k16 step, in code
// order. The MFMA then sums x * q * 2^-9 exactly product by product, and the
// epilogue multiplies by 2^9 times the row scale.
__device__ __forceinline__ bf16x8_t int4x8_to_bf16(uint32_t w) {
  const uint32_t lo = ((w << 4) & 0x80808080u) | (w & 0x07070707u);  // codes 0..3
  const uint32_t hi = (w & 0x80808080u) | ((w >> 4) & 0x07070707u);  // codes 4..7
  return fp8x8_to_bf16(lo, hi);
}
constexpr float kInt4Unit = 512.f;  // 2^9: the widened int4 operands are q * 2^-9

// Where tile T lies: its entry (group of a set), rows and columns.
struct TileGeom {
  int si, g;          // set and group
  int start;          // first row of the segment
  int m0, mvalid;     // tile rows [m0, m0 + mvalid) of the segment
  int n0;             // first output column
};

template <int BM, int BH>
__device__ __forceinline__ TileGeom tile_geom(const GroupedParams& p, const TableLds& tab, int nent, int G0,
                                              int T) {
  TileGeom t;
  const int ent = find_entry(tab.cum, nent, T);
  t.si = ent < G0 ? 0 : 1;
  t.g = t.si ? ent - G0 : ent;
  t.start = tab.start[ent];
  const int rows = tab.rows[ent];
  const int mt = (rows + BM - 1) / BM;
  const int nt = (tab.cum[ent + 1] - tab.cum[ent]) / max(mt, 1);
  const int local = T - tab.cum[ent];
  // Tiles go m-fastest within bands of kBandM m-tiles, then n, then band: a
  // run of consecutive tiles (one XCD's share of a round) then covers a few
  // m-tiles times a few n-tiles, so its L2 holds both operands' slices,
  // instead of one n-tile times every m-tile of a tall segment (which makes
  // every XCD stream all of that segment's rows for each n-tile).
  const int full_bands = mt / kBandM;
  const int in_full = full_bands * kBandM * nt;
  int ntile, mtile;
  if (local < in_full) {
    const int band = local / (kBandM * nt), in = local - band * (kBandM * nt);
    ntile = in / kBandM;
    mtile = band * kBandM + (in - ntile * kBandM);
  } else {
    const int rem = mt - full_bands * kBandM, in = local - in_full;
    ntile = in / rem;
    mtile = full_bands * kBandM + (in - ntile * rem);
  }
  // A segment of `rows` rows takes mt = ceil(rows / BM) m-tiles: either BM
  // rows each and a short last one, or (balance_m) an even split, so that the
  // tiles sharing a weight tile take about the same time. The 256-row class
  // splits the segment's 32-row MFMA blocks evenly, so that only its last
  // block holds empty rows (DeepSeek-shaped prefill 1% faster). The tall
  // class, for a few segments of ~4 m-tiles each, splits the rows evenly:
  // every tile then has the same number of blocks, and the tiles of a weight
  // tile stay in step (split by blocks, 8 + 8 + 8 + 9 blocks, the Mixtral-
  // shaped gate|up fetched twice the bytes from beyond L2).
  if (p.balance_m && BM == 320) {
    t.m0 = (int)((long long)mtile * rows / mt);
    t.mvalid = (int)((long long)(mtile + 1) * rows / mt) - t.m0;
  } else if (p.balance_m) {
    const int nb = (rows + 31) / 32;  // mt <= nb, and no tile gets more than BM / 32 blocks
    const int b0 = (int)((long long)mtile * nb / mt), b1 = (int)((long long)(mtile + 1) * nb / mt);
    t.m0 = 32 * b0;
    t.mvalid = min(32 * b1, rows) - t.m0;
  } else {
    t.m0 = mtile * BM;
    t.mvalid = min(BM, rows - t.m0);
  }
  t.n0 = ntile * BH;
  return t;
}

// Tail split. With G workgroups, tiles [base, total) form a last, partial
// round. When workspace is given, each of those `tail` tiles is split along
// K into S parts (S <= G / tail), so the last round keeps every CU busy.
// Each part writes its fp32 accumulators to the workspace, and the launch
// after it (split_finish_kernel) adds the S parts in part order and applies
// the epilogue.
constexpr int kMaxSplit = 8;
// Split workspace: a header ([0] tail tiles, [1] K-parts S, int32), then one
// geometry record per tail tile (the tail is shorter than the grid, which is
// at most kSplitRecords workgroups), then the parts.
constexpr int kSplitRecords = 512;
constexpr int kSplitRecInts = 8;
constexpr int kSplitHeader = 64 + kSplitRecords * kSplitRecInts;  // floats before the parts
struct SplitPlan {
  int base, tail, S;
};

__device__ __forceinline__ SplitPlan split_plan(int total, int G, long long cap_floats, int tile_floats) {
  SplitPlan sp;
  sp.base = (total / G) * G;
  sp.tail = total - sp.base;
  sp.S = 1;
  // with four or more full rounds the idle part of the last one costs less
  // than writing and adding the parts
  if (sp.tail > 0 && sp.tail <= kSplitRecords && cap_floats > 0 && total < 4 * G) {
    int S = min(kMaxSplit, G / sp.tail);
    while (S > 1 && (long long)sp.tail * S * tile_floats > cap_floats) --S;
    sp.S = max(S, 1);
  }
  return sp;
}

// The epilogue of one tile from its accumulators. acc[i][j][v] holds column
// (lane & 31) and row 8 (v / 4) + 4 (lane / 32) + (v % 4) of 32x32 block
// (i, j). Phase 1 writes h = bf16(silu(g) * u), phase 2 writes fp32 O;
// with quantised weights (WQ = 8: FP8, 4: int4) each column is first
// multiplied by its weight row's scale (int4: times 2^9, the unit of the
// widened codes).
template <int BM, int BN, int WGM, int WGN, int WQ, bool P1, bool SAVE, int FM, int NB, bool OBF = false,
          bool ACC = false>
__device__ __forceinline__ void store_tile(f32x16_t (&acc)[FM][NB], const SetView& S, const TileGeom& t,
                                           int d, int lane, int wm, int wn) {
  constexpr bool WS = WQ != 0;
  constexpr float unit = WQ == 4 ? kInt4Unit : 1.f;
  constexpr int TM = BM / WGM;
  constexpr int BH = P1 ? BN / 2 : BN;
  constexpr int TN = BH / WGN;
  constexpr int FN = TN / 32;
  const int F = S.d_ff;
  const int ncols = P1 ? F : d;
  const int g = t.g;
  const int col0 = t.n0 + wn * TN + (lane & 31);  // this lane's first output column
  float sc0[FN], sc1[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    sc0[j] = sc1[j] = 1.f;
    if constexpr (WS) {
      const int c = min(col0 + j * 32, ncols - 1);
      if constexpr (P1) {
        sc0[j] = S.sg[(size_t)g * F + c] * unit;
        sc1[j] = S.su[(size_t)g * F + c] * unit;
      } else {
        sc0[j] = S.sd[(size_t)g * d + c] * unit;
      }
    }
  }
  int rbase = wm * TM + 4 * (lane >> 5);
  asm volatile("" : "+v"(rbase));  // per tile: keeps the 64 row offsets from being hoisted (and spilled)
  auto rows = [&](auto check) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if constexpr (!P1 && !WS && ACC) {
        // out += product: the block's old values are all loaded before the first
        // store (a load after a store to another row would wait for that store)
        float old[16][FN];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = rbase + i * 32 + 8 * (v >> 2) + (v & 3);
          const bool ok = !decltype(check)::value || r < t.mvalid;
          const float* orow = S.out + (size_t)(t.start + t.m0 + r) * d + col0;
#pragma unroll
          for (int j = 0; j < FN; ++j) old[v][j] = (ok && col0 + j * 32 < ncols) ? orow[j * 32] : 0.f;
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = rbase + i * 32 + 8 * (v >> 2) + (v & 3);
          if (decltype(check)::value && r >= t.mvalid) continue;
          float* orow = S.out + (size_t)(t.start + t.m0 + r) * d + col0;
#pragma unroll
          for (int j = 0; j < FN; ++j)
            if (col0 + j * 32 < ncols) orow[j * 32] = old[v][j] + acc[i][j][v];
        }
        continue;
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = rbase + i * 32 + 8 * (v >> 2) + (v & 3);
        if (decltype(check)::value && r >= t.mvalid) continue;
        const size_t row = (size_t)(t.start + t.m0 + r);
        if constexpr (P1) {
          bf16_t* hrow = static_cast<bf16_t*>(S.h) + row * F + col0;
          if constexpr (SAVE) {  // training: keep the gate and up values for the backward pass
#pragma unroll
            for (int j = 0; j < FN; ++j)
              if (col0 + j * 32 < ncols) {
                S.gsave[row * F + col0 + j * 32] = acc[i][j][v];
                S.usave[row * F + col0 + j * 32] = acc[i][j + FN][v];
              }
          }
#pragma unroll
          for (int j = 0; j < FN; ++j)
            if (col0 + j * 32 < ncols)
              hrow[j * 32] = WS ? silu_mul_bf16(acc[i][j][v] * sc0[j], acc[i][j + FN][v] * sc1[j])
                                : silu_mul_bf16(acc[i][j][v], acc[i][j + FN][v]);
        } else if constexpr (OBF) {  // bf16 output (round to nearest even)
          bf16_t* orow = reinterpret_cast<bf16_t*>(S.out) + row * d + col0;
#pragma unroll
          for (int j = 0; j < FN; ++j)
            if (col0 + j * 32 < ncols) orow[j * 32] = __builtin_bit_cast(bf16_t, (__bf16)acc[i][j][v]);
        } else {
          float* orow = S.out + row * d + col0;
#pragma unroll
          for (int j = 0; j < FN; ++j)
            if (col0 + j * 32 < ncols) orow[j * 32] = WS ? acc[i][j][v] * sc0[j] : acc[i][j][v];
        }
      }
    }
  };
  // a wave whose rows all lie in the segment stores without the per-row test
  if ((wm + 1) * TM <= t.mvalid) rows(std::false_type{});
  else rows(std::true_type{});
}

// One grouped GEMM launch (phase 1: gate|up + SiLU*up -> H; phase 2: down -> O).
// Workgroup tile BM x BN x BK with NS LDS stages, filled by direct global->LDS
// copies issued NS-1 steps ahead. WGM x WGN waves; wave tile (BM/WGM) x
// (BN/WGN) of v_mfma_f32_32x32x16_bf16 blocks with fp32 accumulators.
// WQ = 8: the weights (B) are FP8 E4M3 codes. They are copied to LDS as
// codes (half the bytes), widened to bf16 exactly as each fragment is read,
// and each output column is multiplied by its weight row's scale in the
// epilogue. WQ = 4: int4 codes, two per byte (a quarter of the bytes). Each
// lane reads its 16 bytes of a B row once per step (the 4 words of its 4
// k16 steps) and widens a word per k16 step to q * 2^-9 exactly
// (int4x8_to_bf16).
// SPREAD: the copies that refill a stage go out in equal pieces, one before
// each k16 step of the first half of the step, instead of all at its start,
// so that fewer copies queue at once behind the barrier (3-5% faster on
// 256 x 256 tiles; the second half of the step still covers their latency).
template <int BM, int BN, int BK, int WGM, int WGN, int NS, int MINB, int WQ, bool P1, bool SPREAD,
          bool NMAJ = false, bool SAVE = false, bool OBF = false, bool ACC = false>
__global__ __launch_bounds__(WGM * WGN * 64, MINB) void grouped_mfma_kernel(GroupedParams p) {
  constexpr bool W8 = WQ == 8, W4 = WQ == 4, WS = WQ != 0;
  using BT = typename std::conditional<WS, uint8_t, bf16_t>::type;  // weight storage unit
  constexpr int KDIV = W4 ? 2 : 1;            // K values per BT unit of a weight row
  constexpr int ROWA = BK * 2;                // LDS bytes per A row (bf16)
  constexpr int ROWB = BK * (int)sizeof(BT) / KDIV;  // LDS bytes per B row
  constexpr int PPA = ROWA / 16, PPB = ROWB / 16;        // 16-byte pieces per row
  constexpr int RPIA = kWave / PPA, RPIB = kWave / PPB;  // rows per 1 KB copy instruction
  constexpr int EPP = 16 / (int)sizeof(BT);   // B elements per 16-byte piece
  constexpr int TM = BM / WGM;        // rows per wave
  constexpr int FM = TM / 32;
  constexpr int BH = P1 ? BN / 2 : BN;  // output columns per tile
  constexpr int TN = BH / WGN;          // output columns per wave
  constexpr int FN = TN / 32;
  constexpr int NB = P1 ? 2 * FN : FN;  // B fragments per k16 step
  constexpr int WAVES = WGM * WGN;
  constexpr int NT = WAVES * kWave;
  // copy instructions per wave per stage; with BM / RPIA not a multiple of the
  // wave count the last waves have fewer A copies (a_act below never counts a
  // copy past BM, since mvalid <= BM)
  constexpr int A_INS = (BM / RPIA + WAVES - 1) / WAVES;
  constexpr int B_INS = BN / RPIB / WAVES;
  constexpr int L = A_INS + B_INS;          // vector-memory ops per wave per stage
  constexpr int STAGE_A = BM * ROWA, STAGE = STAGE_A + BN * ROWB;
  static_assert(WS ? (BK == 64 || BK == 128 || BK == 256) : (BK == 32 || BK == 64), "K step");
  constexpr int QB = BK / 64;  // int4: 64-code blocks (32 bytes) per B row per stage
  static_assert(A_INS >= 1 && B_INS >= 1 && FM >= 1 && FN >= 1 && NS >= 2 && NS <= 6, "tile shape");
  static_assert(BM % RPIA == 0 && A_INS * RPIA * WAVES >= BM && B_INS * RPIB * WAVES == BN,
                "copy slots cover the tile");
  static_assert(!P1 || (BN / 2) % (RPIB * B_INS) == 0, "a wave's B rows come from one matrix");
  // N-major B: a 1 KB copy fills 1024 / (2 BN) k-rows
  constexpr int ROWBN = BN * 2;
  static_assert(!NMAJ || (!P1 && !WS && BK == 64 && ROWBN == 512 && B_INS * 2 * WAVES == BK),
                "N-major weights: phase 2, bf16, 64 x 256 B tiles");

  __shared__ __attribute__((aligned(1024))) uint8_t s_tile[NS][STAGE];
  __shared__ TableLds tab;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave / WGN, wn = wave % WGN;
  const int d = p.d_model;
  // output columns per set (h columns in phase 1, d in phase 2); the last n-tile may be partial
  const int nt0 = ((P1 ? p.set[0].d_ff : d) + BH - 1) / BH;
  const int nt1 = p.n_sets > 1 ? ((P1 ? p.set[1].d_ff : d) + BH - 1) / BH : 0;
  const int G0 = p.set[0].n_groups;
  const int nent = G0 + (p.n_sets > 1 ? p.set[1].n_groups : 0);
  static_assert(NS * STAGE >= NT * 4, "table scan scratch fits in the stage buffers");
  const int total = build_table<BM, NT>(p, nt0, nt1, tab, reinterpret_cast<int*>(&s_tile[0][0]));
  const bf16_t* __restrict__ xg = static_cast<const bf16_t*>(p.x);

  // Copy slots: instruction i of this wave fills tile rows (wave*INS + i)*RPI + lane/PP;
  // lane writes LDS piece (lane % PP), so it fetches logical piece (lane % PP) ^ swz(row).
  const int crowA = lane / PPA, cpcA = lane % PPA;
  const int crowB = lane / PPB, cpcB = lane % PPB;

  const SplitPlan sp = split_plan(total, gridDim.x, p.split_cap - kSplitHeader, BM * BN);
  const int units = sp.base + sp.tail * sp.S;
  if (p.split_ws && blockIdx.x == 0 && tid == 0) {  // for the finishing kernel
    reinterpret_cast<int*>(p.split_ws)[0] = sp.S > 1 ? sp.tail : 0;
    reinterpret_cast<int*>(p.split_ws)[1] = sp.S;
  }
  for (int u = xcd_block(); u < units; u += gridDim.x) {
    int T = u, part = -1;  // part >= 0: this unit is K-part `part` of a split tail tile
    if (sp.S > 1 && u >= sp.base) {
      T = sp.base + (u - sp.base) / sp.S;
      part = (u - sp.base) % sp.S;
    }
    const TileGeom tg = tile_geom<BM, BH>(p, tab, nent, G0, T);
    const int si = tg.si, g = tg.g;
    const SetView S = pick(p, si);
    const int start = tg.start, m0 = tg.m0, mvalid = tg.mvalid, n0 = tg.n0;
    const int F = S.d_ff;
    // K values per row of A (phase 2) and of the weight rows; a weight-gradient
    // group takes K = kofs[g + 1] - kofs[g] from its own blocks at kofs[g] (below)
    const int kstride = P1 ? d : F;
    int K = kstride, kbase = 0;
    if constexpr (!P1) {
      if (S.kofs) {
        kbase = S.kofs[g];
        K = S.kofs[g + 1] - kbase;
      }
    }
    const int nk_all = K / BK;
    // accumulating weight gradients: a group with no rows adds nothing (a K-part
    // of a split tile still writes its zero sum for the part-sum kernel)
    if (ACC && nk_all == 0 && part < 0) continue;
    // this unit's K steps: all of them, or part `part` of sp.S
    const int k_lo = part < 0 ? 0 : (int)((long long)part * nk_all / sp.S);
    const int nk = part < 0 ? nk_all : (int)((long long)(part + 1) * nk_all / sp.S) - k_lo;
    const int ncols = P1 ? F : d;

    // ---- A sources: rows past the segment (or with a token out of range)
    // re-read the segment's first row; their outputs are never stored.
    const bf16_t* a_base = P1 ? xg : static_cast<const bf16_t*>(S.h);
    if constexpr (!P1) {
      if (S.kofs) a_base += (size_t)S.urows * kbase;  // this group's [M, K] block
    }
    uint32_t a_off[A_INS];
#pragma unroll
    for (int i = 0; i < A_INS; ++i) {
      const int r = (wave * A_INS + i) * RPIA + crowA;
      const int rr = r < mvalid ? r : 0;
      const int row = start + m0 + rr;
      uint32_t src;
      if constexpr (P1) {
        const int tok = S.perm ? S.perm[row] / S.rpt : row - start;
        src = (unsigned)tok < (unsigned)p.n_tokens ? (uint32_t)tok : 0u;
        src *= (uint32_t)d;
      } else {
        src = S.kofs ? (uint32_t)(row - start) * (uint32_t)K : (uint32_t)row * (uint32_t)F;
      }
      a_off[i] = src + ((cpcA ^ swz<PPA>(r)) << 3);
    }
    // ---- B sources: weight rows n0 + (tile row within its matrix); rows past
    // the last output column (partial n-tile) re-read an in-range row.
    // N-major weights: k-rows (wave*B_INS + i)*2 + lane/32, lane%32 the 16-byte
    // piece, fetched from the swizzled column; columns past the last output
    // column re-read an in-range piece.
    const int lastq = min(BH, ncols - n0) - 1;
    const BT* b_base;
    const BT* b_hi = nullptr;
    const int bsplit = NMAJ ? (S.bsplit ? S.bsplit : K) : 0;
    if constexpr (P1) {
      const bool up = wave * B_INS * RPIB >= BN / 2;
      b_base = static_cast<const BT*>(up ? S.wu : S.wg) + (size_t)g * F * d / KDIV;
    } else if constexpr (NMAJ) {
      b_base = static_cast<const BT*>(S.wd) + (size_t)g * bsplit * d;
      b_hi = static_cast<const BT*>(S.wu) + (size_t)g * bsplit * d;
    } else {
      b_base = static_cast<const BT*>(S.wd) + (S.kofs ? (size_t)d * kbase : (size_t)g * d * F / KDIV);
    }
    uint32_t b_off[B_INS];
#pragma unroll
    for (int i = 0; i < B_INS; ++i) {
      if constexpr (NMAJ) {
        const int kr = (wave * B_INS + i) * 2 + (lane >> 5);
        const int pl = lane & 31;
        const int pg = (((pl >> 2) ^ (kr & 3)) << 2) | (pl & 3);
        b_off[i] = (uint32_t)kr * (uint32_t)d + (uint32_t)min(n0 + pg * 8, ncols - 8);
      } else {
        const int r = (wave * B_INS + i) * RPIB + crowB;    // tile row
        const int mr = P1 ? (r % (BN / 2)) : r;              // row within its weight matrix tile
        // a weight-gradient group reads its own [d, K] block (rows K apart)
        const int bstride = (!P1 && S.kofs) ? K : kstride;
        b_off[i] = (uint32_t)(n0 + min(mr, lastq)) * (uint32_t)(bstride / KDIV) +
                   (uint32_t)((cpcB ^ swz<PPB>(r)) * EPP);
      }
    }
    // the source of this wave's B copies for the stage at K offset ko
    auto b_src = [&](int ko) -> const BT* {
      if constexpr (NMAJ) return ko < bsplit ? b_base + (size_t)ko * d : b_hi + (size_t)(ko - bsplit) * d;
      else return b_base + ko / KDIV;
    };
    const uint32_t a_lds0 = lds_addr(&s_tile[0][(wave * A_INS) * 1024]);
    const uint32_t b_lds0 = lds_addr(&s_tile[0][STAGE_A + (wave * B_INS) * 1024]);

    // A copies whose RPI rows all lie past the segment are skipped: those LDS
    // rows keep stale data, which only reaches output rows that are never
    // stored (an MFMA output row depends on its own A row alone). Each wave
    // then issues lw = a_act + B_INS copies per stage (fixed for the tile),
    // and the waits count in units of lw.
    const int a_act = min(A_INS, max(0, (mvalid + RPIA - 1) / RPIA - wave * A_INS));
    const int lw = a_act + B_INS;

    // Down projections on the small classes walk K from one start per XCD (the
    // XCD's workgroups together, 1/8 of K apart between XCDs): their weight rows
    // are d_ff apart, and in step on every XCD they load the same row offsets at
    // once (DeepSeek-shaped decode down 0.205 -> 0.195 ms). Gate|up keeps the
    // natural K order, in which the rounding of h to bf16 is checked, and so do
    // the balanced large tiles, whose m-tiles share operand panels in L2.
    const int rot = (!P1 && !NMAJ && !S.kofs && !p.balance_m) ? (int)(blockIdx.x % kXcds) * nk / kXcds : 0;
    auto kstep = [&](int kt) {
      const int kk = kt + rot;
      return kk >= nk ? kk - nk : kk;
    };
    auto issue = [&](int kt) {
      const int st = kt % NS;
      const int ko = (k_lo + kstep(kt)) * BK;
#pragma unroll
      for (int i = 0; i < A_INS; ++i)
        if (i < a_act) dma16(a_base + a_off[i] + ko, a_lds0 + st * STAGE + i * 1024);
      const BT* bsrc = b_src(ko);
#pragma unroll
      for (int i = 0; i < B_INS; ++i) dma16(bsrc + b_off[i], b_lds0 + st * STAGE + i * 1024);
    };
    // copies [c0, c1) of stage kt, in the order A (active ones) then B
    auto issue_part = [&](int kt, int c0, int c1) {
      const int st = kt % NS;
      const int ko = (k_lo + kstep(kt)) * BK;
#pragma unroll
      for (int c = 0; c < L; ++c) {
        if (c < c0 || c >= c1) continue;
        if (c < A_INS) {
          if (c < a_act) dma16(a_base + a_off[c] + ko, a_lds0 + st * STAGE + c * 1024);
        } else {
          dma16(b_src(ko) + b_off[c - A_INS], b_lds0 + st * STAGE + (c - A_INS) * 1024);
        }
      }
    };

    f32x16_t acc[FM][NB];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // 32-row MFMA blocks of this wave that hold segment rows: a segment's last
    // tile is often short, and its empty blocks skip their reads and MFMAs.
    const int nact = max(0, min(FM, (mvalid - wm * TM + 31) / 32));

#define MOE_K_LOOP(ACTIVE)                                                                       \
    for (int kt = 0; kt < nk; ++kt) {                                                            \
      /* stage kt has landed once at most (stages issued after it) * lw copies are outstanding */ \
      /* (loads complete in issue order) */                                                      \
      const int later = min(NS - 2, nk - 1 - kt);                                                \
      if constexpr (NS == 2) wait_vm_barrier<0>();                                               \
      else wait_vm_barrier_rt<(NS - 2) * L>(later * lw);                                         \
      if (!SPREAD && kt + NS - 1 < nk) issue(kt + NS - 1); /* refills the stage read in step kt-1 */ \
      const uint8_t* sa = &s_tile[kt % NS][0];                                                   \
      const uint8_t* sb = sa + STAGE_A;                                                          \
      /* int4: this lane's 4 words (one per k16 step) of each 64-code block of each B row */    \
      u32x4_t wq[W4 ? NB : 1][W4 ? QB : 1];                                                     \
      if constexpr (W4) {                                                                        \
        _Pragma("unroll") for (int j = 0; j < NB; ++j) {                                         \
          const int jj = P1 ? (j % FN) : j;                                                      \
          const int half = P1 ? (j / FN) * (BN / 2) : 0;                                         \
          const int r = half + wn * TN + jj * 32 + (lane & 31);                                  \
          _Pragma("unroll") for (int b = 0; b < QB; ++b)                                         \
            wq[j][b] = *reinterpret_cast<const u32x4_t*>(sb + r * ROWB + (((2 * b + (lane >> 5)) ^ swz<PPB>(r)) << 4)); \
        }                                                                                        \
      }                                                                                          \
      _Pragma("unroll") for (int ks = 0; ks < BK / 16; ++ks) {                                   \
        if constexpr (SPREAD) {                                                                  \
          /* the refill's copies, spread over the first half of the k16 steps */                 \
          constexpr int KSP = (BK / 16 + 1) / 2;                                                 \
          constexpr int PER = (L + KSP - 1) / KSP;                                               \
          if (ks < KSP && kt + NS - 1 < nk) issue_part(kt + NS - 1, ks * PER, ks * PER + PER);  \
        }                                                                                        \
        const int chunk = ks * 2 + (lane >> 5);                                                  \
        bf16x8_t af[FM], bfr[NB];                                                                \
        _Pragma("unroll") for (int i = 0; i < FM; ++i) {                                         \
          if (!(ACTIVE(i))) continue;                                                            \
          const int r = wm * TM + i * 32 + (lane & 31);                                          \
          af[i] = *reinterpret_cast<const bf16x8_t*>(sa + r * ROWA + ((chunk ^ swz<PPA>(r)) << 4)); \
        }                                                                                        \
        _Pragma("unroll") for (int j = 0; j < NB; ++j) {                                         \
          /* phase 1: fragments [0, FN) are gate rows, [FN, 2 FN) the matching up rows */        \
          const int jj = P1 ? (j % FN) : j;                                                      \
          const int half = P1 ? (j / FN) * (BN / 2) : 0;                                         \
          const int r = half + wn * TN + jj * 32 + (lane & 31);                                  \
          if constexpr (NMAJ) {                                                                  \
            const int kr = ks * 16 + 8 * (lane >> 5) + ((lane >> 2) & 3);                        \
            const int nc = wn * TN + jj * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);          \
            const uint8_t* pt = sb + nmajor_offset<ROWBN>(kr, nc);                               \
            const i16x4_t lo = lds_read_tr16(pt), hi = lds_read_tr16(pt + 4 * ROWBN);            \
            bfr[j] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7)); \
          } else if constexpr (W4) {                                                             \
            bfr[j] = int4x8_to_bf16(wq[j][ks / 4][ks % 4]);                                      \
          } else if constexpr (W8) {                                                             \
            /* piece ks holds the 16 codes of this k16 step; lanes 32-63 take its upper 8 */     \
            const u32x2_t q = *reinterpret_cast<const u32x2_t*>(sb + r * ROWB + ((ks ^ swz<PPB>(r)) << 4) + ((lane >> 5) << 3)); \
            bfr[j] = fp8x8_to_bf16(q.x, q.y);                                                    \
          } else {                                                                               \
            bfr[j] = *reinterpret_cast<const bf16x8_t*>(sb + r * ROWB + ((chunk ^ swz<PPB>(r)) << 4)); \
          }                                                                                      \
        }                                                                                        \
        _Pragma("unroll") for (int i = 0; i < FM; ++i) {                                         \
          if (!(ACTIVE(i))) continue;                                                            \
          _Pragma("unroll") for (int j = 0; j < NB; ++j)                                         \
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0); \
        }                                                                                        \
      }                                                                                          \
    }
#define MOE_ALL(i) true
#define MOE_SOME(i) ((i) < nact)
    __syncthreads();  // every wave is done with the previous tile's stages
#pragma unroll
    for (int s2 = 0; s2 < NS - 1; ++s2)
      if (s2 < nk) issue(s2);
    if (nact == FM) {
      MOE_K_LOOP(MOE_ALL)
    } else {
      MOE_K_LOOP(MOE_SOME)
    }
#undef MOE_ALL
#undef MOE_SOME
#undef MOE_K_LOOP

    // ---- epilogue
    if (part >= 0) {
      // a K-part of a split tail tile: raw accumulators, thread-major, for the finishing
      // kernel; part 0 also records the tile's geometry
      if (part == 0 && tid == 0) {
        int* rec = reinterpret_cast<int*>(p.split_ws) + 64 + (T - sp.base) * kSplitRecInts;
        rec[0] = tg.si;
        rec[1] = tg.g;
        rec[2] = tg.start;
        rec[3] = tg.m0;
        rec[4] = tg.mvalid;
        rec[5] = tg.n0;
      }
      float* dst = p.split_ws + kSplitHeader + ((size_t)(T - sp.base) * sp.S + part) * (BM * BN);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            dst[((i * NB + j) * 16 + v) * NT + tid] = acc[i][j][v];
      continue;
    }
    store_tile<BM, BN, WGM, WGN, WQ, P1, SAVE, FM, NB, OBF, ACC>(acc, S, tg, d, lane, wm, wn);
  }
}

// Finishes the split tail tiles of the launch before it (same parameters),
// one wave per workgroup: workgroup b takes wave b % NW of tail tile b / NW,
// adds that wave's accumulators over the S K-parts in part order and runs the
// wave's share of the tile epilogue. The tail, S and each tail tile's
// geometry come from the header and records the launch wrote; workgroups
// past the tail exit at once.
template <int BM, int BN, int WGM, int WGN, int WQ, bool P1, bool SAVE = false, bool OBF = false, bool ACC = false>
__global__ __launch_bounds__(kWave) void split_finish_kernel(GroupedParams p) {
  constexpr int NW = WGM * WGN;
  constexpr int TM = BM / WGM, FM = TM / 32;
  constexpr int BH = P1 ? BN / 2 : BN;
  constexpr int TN = BH / WGN, FN = TN / 32;
  constexpr int NB = P1 ? 2 * FN : FN;
  constexpr int NT = NW * kWave;  // threads of the GEMM workgroup that wrote the parts
  const int* hdr = reinterpret_cast<const int*>(p.split_ws);
  const int tail = hdr[0], S = hdr[1];
  const int tt = blockIdx.x / NW, w = blockIdx.x % NW;
  if (S <= 1 || tt >= tail) return;
  const int lane = threadIdx.x;
  const int wm = w / WGN, wn = w % WGN;
  const int d = p.d_model;
  const int* rec = hdr + 64 + tt * kSplitRecInts;
  TileGeom tg;
  tg.si = rec[0];
  tg.g = rec[1];
  tg.start = rec[2];
  tg.m0 = rec[3];
  tg.mvalid = rec[4];
  tg.n0 = rec[5];
  const SetView Sv = pick(p, tg.si);
  f32x16_t acc[FM][NB];
  const float* src = p.split_ws + kSplitHeader + (size_t)tt * S * (BM * BN) + w * kWave + lane;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = src[((size_t)(i * NB + j) * 16 + v) * NT];
  for (int q = 1; q < S; ++q) {
    // the whole part is loaded before any of it is added, so that its loads are in flight together
    const float* sq = src + (size_t)q * (BM * BN);
    float t[FM][NB][16];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) t[i][j][v] = __builtin_nontemporal_load(&sq[((size_t)(i * NB + j) * 16 + v) * NT]);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] += t[i][j][v];
  }
  store_tile<BM, BN, WGM, WGN, WQ, P1, SAVE, FM, NB, OBF, ACC>(acc, Sv, tg, d, lane, wm, wn);
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
  __shared__ int s_scan[kThreads];
  const int total = build_table<BM, kThreads>(p, nt0, nt1, tab, s_scan);
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

// A tile shape that can run gate|up: each wave takes whole 32-column blocks of
// the tile's BN / 2 gate (and as many up) rows. Launchers instantiate the
// gate|up kernels only for these (a class used only for the down projection
// may be narrower).
template <int BN, int WGN>
constexpr bool kGateUpShape = BN / 2 / WGN >= 32;

// per_cu: workgroups launched per CU at most. 1 is a persistent grid (each
// workgroup walks the tile list with stride gridDim.x); a large value
// launches about one workgroup per tile.
template <int BM, int BN, int BK, int WGM, int WGN, int NS, int WQ, bool SPREAD = false, int MINB = 1,
          bool NMAJ = false>
void launch_mfma(const GroupedParams& p, int phase, int per_cu, hipStream_t st) {
  const int BH = phase == 1 ? BN / 2 : BN;
  long long ub = tiles_upper_bound(p, phase, BM, BH);
  // Fewer tiles than CUs, each with a long K loop (a router product: one
  // segment of N rows times E or d columns): launch up to kMaxSplit workgroups
  // per tile so that the tail split spreads the K loops over the idle CUs.
  const int K = phase == 1 ? p.d_model : p.set[0].d_ff;
  if (p.split_ws && p.split_cap > kSplitHeader && ub < num_cus() && K >= 16 * BK)
    ub = std::min<long long>(ub * kMaxSplit, num_cus());
  const int grid = grid_for(ub, per_cu);
  // the training forward (bf16 phase 1 with g_save) runs its own instantiation: the
  // inference kernels keep their code unchanged
  const bool save = WQ == 0 && phase == 1 && p.set[0].g_save;
  const bool obf = WQ == 0 && phase == 2 && !NMAJ && p.set[0].out_bf16;
  // accumulating gradients (bf16, phase 2): instantiations of their own, so that
  // the other kernels carry no accumulate epilogue
  const bool accum = WQ == 0 && phase == 2 && p.set[0].accumulate;
  if constexpr (NMAJ) {
    if (accum)
      hipLaunchKernelGGL((grouped_mfma_kernel<BM, BN, BK, WGM, WGN, NS, MINB, WQ, false, SPREAD, true, false, false,
                                              WQ == 0>),
                         dim3(grid), dim3(WGM * WGN * 64), 0, st, p);
    else
      hipLaunchKernelGGL((grouped_mfma_kernel<BM, BN, BK, WGM, WGN, NS, MINB, WQ, false, SPREAD, true>), dim3(grid),
                         dim3(WGM * WGN * 64), 0, st, p);
  } else if (phase == 1) {
    if constexpr (kGateUpShape<BN, WGN>) {
      if (save)
        hipLaunchKernelGGL((grouped_mfma_kernel<BM, BN, BK, WGM, WGN, NS, MINB, WQ, true, SPREAD, false, WQ == 0>),
                           dim3(grid), dim3(WGM * WGN * 64), 0, st, p);
      else
        hipLaunchKernelGGL((grouped_mfma_kernel<BM, BN, BK, WGM, WGN, NS, MINB, WQ, true, SPREAD>), dim3(grid),
                           dim3(WGM * WGN * 64), 0, st, p);
    }
  } else if (obf) {
    hipLaunchKernelGGL((grouped_mfma_kernel<BM, BN, BK, WGM, WGN, NS, MINB, WQ, false, SPREAD, false, false, WQ == 0>),
                       dim3(grid), dim3(WGM * WGN * 64), 0, st, p);
  } else if (accum) {
    hipLaunchKernelGGL((grouped_mfma_kernel<BM, BN, BK, WGM, WGN, NS, MINB, WQ, false, SPREAD, false, false, false,
                                            WQ == 0>),
                       dim3(grid), dim3(WGM * WGN * 64), 0, st, p);
  } else {
    hipLaunchKernelGGL((grouped_mfma_kernel<BM, BN, BK, WGM, WGN, NS, MINB, WQ, false, SPREAD>), dim3(grid),
                       dim3(WGM * WGN * 64), 0, st, p);
  }
  if (p.split_ws && p.split_cap > kSplitHeader) {
    // one wave per workgroup; the tail holds fewer tiles than the grid has workgroups
    const dim3 fg(grid * WGM * WGN), fb(kWave);
    if (phase == 1) {
      if constexpr (kGateUpShape<BN, WGN>) {
        if (save)
          hipLaunchKernelGGL((split_finish_kernel<BM, BN, WGM, WGN, WQ, true, WQ == 0>), fg, fb, 0, st, p);
        else
          hipLaunchKernelGGL((split_finish_kernel<BM, BN, WGM, WGN, WQ, true>), fg, fb, 0, st, p);
      }
    } else if (obf)
      hipLaunchKernelGGL((split_finish_kernel<BM, BN, WGM, WGN, WQ, false, false, WQ == 0>), fg, fb, 0, st, p);
    else if (accum)
      hipLaunchKernelGGL((split_finish_kernel<BM, BN, WGM, WGN, WQ, false, false, false, WQ == 0>), fg, fb, 0, st,
                         p);
    else
      hipLaunchKernelGGL((split_finish_kernel<BM, BN, WGM, WGN, WQ, false>), fg, fb, 0, st, p);
  }
}

// tile height from the mean routed rows per expert segment (an upper bound: N k / E).
// At 128 rows per expert (the Switch-shaped capacity layer, where capacity and
// skew leave ~50 rows per touched expert) the 64-row tiles are faster: the same
// gate|up time and 30% less down time than 256-row tiles.
bool large_tiles(long long rows, int groups) { return rows / std::max(1, groups) >= 192; }

// Gate|up of layers with 64 to 191 mean rows per segment: 64 x 512 tiles. With fewer
// rows (decode) the 64 x 256 tiles, twice as many, stream the weights faster.
bool wide_gate_up(long long rows, int groups) {
  const long long m = rows / std::max(1, groups);
  return m >= 64 && m < 192;
}

// Segments that a capacity bounds at 65-160 rows fit one 160-row tile.
bool one_tall_tile(int group_rows_max) { return group_rows_max > 64 && group_rows_max <= 160; }

// Few, tall segments (bf16 layers): 320-row tiles when they need at least 20%
// fewer m-tiles than 256-row ones. Tile time there scales with the tile count
// more than with the rows: the Mixtral-shaped segments of 1030-1052 rows take
// five 208-row tiles or four 260-row ones, and the four are faster in all (gate|up
// 1-5%, down 2-3%; a 260-row tile costs ~1.2x a 208-row one). The counts are
// estimated from the mean rows per segment plus 2% (the segments' spread under
// random routing). The weight-gradient GEMMs keep 256-row tiles.
bool tall_tiles(long long rows, int groups) {
  const long long m100 = rows * 102 / std::max(1, groups);  // mean rows + 2%, in hundredths
  if (m100 < 76800) return false;
  const long long t256 = (m100 + 25599) / 25600, t320 = (m100 + 31999) / 32000;
  return t320 * 5 <= t256 * 4;
}

template <int WQ>
void launch_class(const GroupedParams& p, int phase, hipStream_t stream) {
  if constexpr (WQ == 4) {
    // int4 weights (a decode format). Gate|up (K = d, a multiple of 256): 32 x 512
    // tiles, 8 waves, 128 K values per stage, three stages (40 KB each). Each
    // weight row piece a copy fetches is 64 bytes (32 at 64 K values per stage),
    // and each token row is read once per 256 columns of h instead of 128: at 4
    // bits per weight the activation rows are a large share of a tile's copies.
    // DeepSeek-shaped decode gate|up 0.157 ms (64 x 256, 64-K stages) -> 0.142 ms
    // (32 x 256, 256-K stages) -> 0.133 ms. Down (K = d_ff, 2048 on that layer: few K steps per tile) and
    // other K: 64 x 256 tiles, 64 K values per stage, two workgroups per CU.
    if (phase == 1 && p.d_model % 256 == 0)
      launch_mfma<32, 512, 128, 1, 8, 3, 4, false, 1>(p, phase, 1, stream);
    else
      launch_mfma<64, 256, 64, 1, 4, 4, 4, false, 2>(p, phase, 2, stream);
  } else if (large_tiles(p.set[0].max_rows, p.set[0].n_groups)) {
    // persistent grid with even m-tiles: the workgroups that share a weight
    // tile run in step, so their copies of it hit in L2
    GroupedParams q = p;
    q.balance_m = 1;
    if (WQ == 0 && phase == 2 && p.set[0].b_nmajor) {
      launch_mfma<256, 256, 64, 2, 4, 2, 0, true, 1, true>(q, 2, 1, stream);
    } else if (WQ == 0 && !p.set[0].k_offsets && !p.set[0].accumulate &&
               tall_tiles(p.set[0].max_rows, p.set[0].n_groups)) {
      if constexpr (WQ == 0) launch_mfma<320, 256, 64, 2, 4, 2, 0, true>(q, phase, 1, stream);
    } else {
      launch_mfma<256, 256, 64, 2, 4, 2, WQ, true>(q, phase, 1, stream);
    }
  } else if (WQ == 0 && phase == 2 && p.set[0].b_nmajor) {
    launch_mfma<64, 256, 64, 1, 4, 3, 0, false, 1, true>(p, 2, 1, stream);
  } else if (WQ == 0 && phase == 1 && !p.set[0].g_save && wide_gate_up(p.set[0].max_rows, p.set[0].n_groups)) {
    if (one_tall_tile(p.set[0].group_rows_max)) {
      // a capacity of 65-160 rows: one 160 x 512 tile per segment and weight tile,
      // so each weight panel is read once (with 64-row tiles, up to three times);
      // 32 K values per stage leave room for three stages. Switch-shaped capacity
      // layer gate|up 0.366 -> 0.342 ms, the same bits
      launch_mfma<160, 512, 32, 1, 8, 3, 0, false>(p, phase, 1, stream);
    } else {
      // 64 x 512 tiles, 8 waves, two stages: half the tiles of 64 x 256 (half the x-row
      // re-reads and per-tile starts); Switch-shaped capacity layer gate|up 0.38 -> 0.37 ms
      launch_mfma<64, 512, 64, 1, 8, 2, 0, false>(p, phase, 1, stream);
    }
  } else if (WQ == 8 && phase == 1 && p.d_model % 128 == 0) {
    // FP8 gate|up: 128 K values per stage, whole 128-byte weight row pieces
    // (DeepSeek-shaped decode gate|up 0.221 -> 0.205 ms; the down projection's
    // short K loops run faster on the 64-K stages below)
    launch_mfma<64, 256, 128, 1, 4, 3, 8, false, 1>(p, phase, 1, stream);
  } else {
    // FP8 weights halve the B stages (80 KB of LDS in all), so two workgroups share a CU
    launch_mfma<64, 256, 64, 1, 4, 3, WQ>(p, phase, WQ == 8 ? 2 : 1, stream);
  }
}

}  // namespace

size_t grouped_split_bytes(long long rows, int groups) {
  // the parts of one launch fill at most one tile per workgroup: G = CUs x workgroups per CU
  // (the tallest large tile has 320 rows), after the header and the tail tile records
  const bool large = large_tiles(rows, groups);
  const size_t G = (size_t)num_cus() * (large ? 1 : 2);
  return (kSplitHeader + G * (large ? 320 * 256 : 64 * 256)) * sizeof(float);
}

int launch_grouped(const GroupedParams& p, int phase, hipStream_t stream) {
  if (p.dtype == MOE_DTYPE_F32) {
    const int grid = grid_for(tiles_upper_bound(p, phase, 32, 32), 4);
    if (phase == 1)
      hipLaunchKernelGGL(grouped_f32_kernel<true>, dim3(grid), dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL(grouped_f32_kernel<false>, dim3(grid), dim3(kThreads), 0, stream, p);
  } else if (p.wq == 8) {
    launch_class<8>(p, phase, stream);
  } else if (p.wq == 4) {
    launch_class<4>(p, phase, stream);
  } else {
    launch_class<0>(p, phase, stream);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
