// fox_fwd.hip -- K2: fused causal FoX attention forward on gfx950 MFMA.
//
// Definition (FoX module page, ForgettingAttention.forward, decoder mode;
// foxwindow README, opening paragraph):
//   s_ij = scale * q_i.k_j + sum_{t=j+1..i} log f_t  (j <= i),  softmax over j,  O_i = sum_j p_ij v_j.
//
// Work decomposition
//   * One workgroup of NW waves (4 or 8) per (query block of 32*NW rows, batch*head).
//     Wave w owns 32 query rows; the 8-wave form halves the K/V staging traffic per flop.  Grid x = batch*head (fastest, so the workgroups of one
//     head land on one XCD when batch*head is a multiple of 8 and share its L2),
//     grid y = query block, heaviest (last) blocks dispatched first.
//   * Key tiles of 64 keys are visited from the diagonal tile DOWN to tile 0; tiles
//     above the diagonal are never touched (their weights are exactly 0).  Walking
//     backwards makes the first tile a row sees hold its largest gate bias, so the
//     running max rarely moves and the lazy rescale below almost never fires.
//   * Gate bias without a prefix-sum buffer: while walking backwards the loader keeps
//     the fp64 suffix sum R_j = sum_{t=j+1..ref} log f_t (ref = the block's last row).
//     Then c_i - c_j = R_j - R_i; the per-row constant R_i drops out of the softmax and
//     is added back to lse only.  Each score costs one FMA: s2 = acc*scale*log2e + R_j*log2e.
//     The block's own c_i = c_ref - R_i is written as the `c` output.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (keys = M, queries = N), so a lane holds
//     one query row and 16 keys per 32x32 block: the row max / sum are in-lane plus
//     one permlane32 swap.  The S^T accumulator registers are, after rounding to bf16,
//     directly the B operand of O^T = V^T P^T (the V operand follows the same key order).
//   * K and V are staged row-major in LDS (padded rows).  The PV operand, which needs 8
//     keys of one dim per lane, comes from gfx950's transposing LDS read
//     (ds_read_b64_tr_b16), so no transposed stores.  Global loads of the next tile are
//     issued before the current tile's MFMAs (register prefetch).
//   * Online softmax in base 2 with lazy rescaling: the running max is only raised when
//     a row's tile max exceeds it by more than kTau (exact: the final normalisation uses
//     the same stale max; p stays <= 2^kTau).
//
// fp32 inputs use the same schedule with v_mfma_f32_32x32x2f32 and fp32 P; there the
// bias R_j - R_i is formed per score in fp64 (kept in LDS), so no fp32 rounding of a
// block-relative gate sum enters the scores.
#include <math.h>

#include "fox_device.h"
#include "fox_internal.h"

namespace fox {
namespace {

#ifndef FOX_EXP_TREE
#define FOX_EXP_TREE 0
#endif
#ifndef FOX_EXP_PRIO
#define FOX_EXP_PRIO 0
#endif

constexpr int kThreads = 256;  // fp32 kernel; the bf16 kernel runs 64 * NW threads
constexpr int kBR = 128;       // query rows per workgroup of the fp32 kernel (32 per wave)
constexpr int kMaxBR = 256;    // largest query block (bf16, 8 waves)
constexpr int kBC = 64;       // keys per tile
constexpr float kTau = 8.0f;  // lazy-rescale threshold, log2 units
constexpr float kNegInf = -INFINITY;

struct GateRows {      // per workgroup
  double rowR[kMaxBR]; // R_i for the block's own rows
  double cref;         // c at the block's reference row (sum of log f over 0..ref)
};

// Wave 0: gate sums for tile kt.  Lane t holds log f of key 63-t of the tile (0 beyond
// ref), so the lane-order exclusive prefix is the key-order exclusive suffix
// sum_{u > j} log f_u inside the tile.  `carry` (fp64) is the sum of log f over
// (tile end, ref] and is advanced by the tile total.  Writes R_j = carry + suffix for
// the tile (r2 = R_j * log2 e in fp32; r64 = R_j, when given), R_i for the block's own
// rows and, after tile 0, c at the reference row.  Everything is fp64 until the single
// rounding to fp32.
__device__ __forceinline__ void gate_tile(float* r2, double* r64, GateRows& rows, int lane, int kt, int row0,
                                          int ref, float lf_rev, double& carry) {
  const double incl = wave_incl_scan((double)lf_rev);
  const double excl = wave_shr1(incl);
  const int jl = 63 - lane;
  const double rj = carry + excl;
  r2[jl] = (float)(rj * kLog2ed);
  if (r64) r64[jl] = rj;
  const int j = kt * kBC + jl;
  if (j >= row0 && j <= ref) rows.rowR[j - row0] = rj;
  carry += wave_last(incl);
  if (kt == 0 && lane == 0) rows.cref = carry;
}

// ------------------------------------------------------------------------------------------
// bf16
// ------------------------------------------------------------------------------------------
template <int D, int NW>
struct Bf16Tile {
  static constexpr int KS = D + 8;  // K row stride in LDS (bf16): 16-byte pad, b128 row reads hit distinct banks
  // V row stride in LDS (bf16): the transposed b64 reads of one half-wave touch 4 rows x 64
  // bytes; a stride of 16 dwords (mod 64 banks) puts those rows on disjoint banks.
  static constexpr int VS = (D == 32) ? D : D + 32;
  static constexpr int THREADS = 64 * NW;
  static constexpr int GROUPS = D / 8;                 // 16-byte chunks per key row
  static constexpr int KPT = kBC * GROUPS / THREADS;   // keys per thread in the tile loader
  static_assert(KPT >= 1 && KPT * THREADS == kBC * GROUPS, "loader mapping");
  u32x4 k[KPT];
  u32x4 v[KPT];
};

template <int D>
struct Bf16Stage {  // one staged key tile
  bf16 k[kBC * (D + 8)];
  bf16 v[kBC * ((D == 32) ? D : D + 32)];
  float r2[kBC];  // R_j * log2(e)
};

template <int D>
struct Bf16Lds {
  Bf16Stage<D> st[2];  // double buffer: tile t is computed while tile t-1 is staged
  GateRows rows;
};

template <int D, int NW>
__device__ __forceinline__ void bf16_load_tile(Bf16Tile<D, NW>& t, const bf16* kb, const bf16* vb, int kt, int n,
                                               int tid) {
  constexpr int G = Bf16Tile<D, NW>::GROUPS, KPT = Bf16Tile<D, NW>::KPT;
  const int c = tid % G, a = tid / G;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int key = kt * kBC + a * KPT + i;
    if (key < n) {
      t.k[i] = *reinterpret_cast<const u32x4*>(kb + (size_t)key * D + 8 * c);
      t.v[i] = *reinterpret_cast<const u32x4*>(vb + (size_t)key * D + 8 * c);
    } else {
      t.k[i] = u32x4{0u, 0u, 0u, 0u};
      t.v[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// A complete tile (every key < n): no bounds checks.
template <int D, int NW>
__device__ __forceinline__ void bf16_load_full_tile(Bf16Tile<D, NW>& t, const bf16* kb, const bf16* vb, int kt,
                                                    int tid) {
  constexpr int G = Bf16Tile<D, NW>::GROUPS, KPT = Bf16Tile<D, NW>::KPT;
  const int c = tid % G, a = tid / G;
  const size_t off = (size_t)(kt * kBC + a * KPT) * D + 8 * c;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    t.k[i] = *reinterpret_cast<const u32x4*>(kb + off + (size_t)i * D);
    t.v[i] = *reinterpret_cast<const u32x4*>(vb + off + (size_t)i * D);
  }
}

template <int D, int NW>
__device__ __forceinline__ void bf16_store_tile(const Bf16Tile<D, NW>& t, Bf16Stage<D>& s, int tid) {
  constexpr int G = Bf16Tile<D, NW>::GROUPS, KPT = Bf16Tile<D, NW>::KPT, KS = Bf16Tile<D, NW>::KS,
                VS = Bf16Tile<D, NW>::VS;
  const int c = tid % G, a = tid / G;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    *reinterpret_cast<u32x4*>(&s.k[(a * KPT + i) * KS + 8 * c]) = t.k[i];
    *reinterpret_cast<u32x4*>(&s.v[(a * KPT + i) * VS + 8 * c]) = t.v[i];
  }
}

// ds_read_b64_tr_b16: within each 16-lane group, output lane j element e is element j%4
// of the 8 bytes addressed by lane 4e + j/4 of the group (transpose of a 16x4 block).
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;
__device__ __forceinline__ bf16x4 lds_read_tr16(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p));
}

// Softmax and P.V for one 32-key block b of a tile, given its S^T accumulator: bias,
// (causal mask), lazy rescale of the running state, p = exp2(s - m), O^T += V^T P^T.
template <int D, bool DIAG>
__device__ __forceinline__ void bf16_block_softmax_pv(const Bf16Stage<D>& st, f32x16 sacc, int b,
                                                      f32x16 (&oacc)[D / 32], float& m, float& lsum, int key0,
                                                      int my_row, int lane, float scale_log2) {
  constexpr int VS = Bf16Tile<D, 4>::VS, DB = D / 32;
  const int hi = lane >> 5, li = lane & 15;
#if FOX_EXP_TREE
  float gm[4];
#else
  float mx = kNegInf;
#endif
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int kl = 32 * b + 8 * g + 4 * hi;
    const f32x4 r2 = *reinterpret_cast<const f32x4*>(&st.r2[kl]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float sv = fmaf(sacc[4 * g + e], scale_log2, r2[e]);
      if constexpr (DIAG) {
        if (key0 + kl + e > my_row) sv = kNegInf;
      }
      sacc[4 * g + e] = sv;
#if !FOX_EXP_TREE
      mx = fmaxf(mx, sv);
#endif
    }
#if FOX_EXP_TREE
    gm[g] = fmaxf(fmaxf(sacc[4 * g], sacc[4 * g + 1]), fmaxf(sacc[4 * g + 2], sacc[4 * g + 3]));
#endif
  }
#if FOX_EXP_TREE
  float mx = fmaxf(fmaxf(gm[0], gm[1]), fmaxf(gm[2], gm[3]));
#endif
  mx = pair32_max(mx);

  const float mcand = fmaxf(m, mx);
  const bool need = mcand > m + kTau;
  if (wave_any(need)) {
    const float mn = need ? mcand : m;
    const float alpha = exp2_hw(m - mn);
    lsum *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
    m = mn;
  }
  const float msub = (m == kNegInf) ? 0.0f : m;

  // A operand of O^T += V^T P^T: lane (l32, hi) needs V[key][32db + l32] for the 8 keys
  // 16u + {4hi .. 4hi+3, 8+4hi .. 8+4hi+3} of block b (the key order of the S^T registers
  // in pb).  Two transposed reads of 4 keys each: lane i of a 16-lane group points at
  // V[key0 + i/4][dim0 + 4(i%4)].
  const bf16* vlane = &st.v[(32 * b + 4 * hi + (li >> 2)) * VS + 16 * ((lane >> 4) & 1) + 4 * (li & 3)];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    bf16x8 pb;
#if FOX_EXP_TREE
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pv[e] = exp2_hw(sacc[8 * u + e] - msub);
      pb[e] = (bf16)pv[e];
    }
    lsum += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
#else
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pv = exp2_hw(sacc[8 * u + e] - msub);
      lsum += pv;
      pb[e] = (bf16)pv;
    }
#endif
    const bf16* vrow = vlane + 16 * u * VS;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16x4 lo = lds_read_tr16(vrow + 32 * db);
      const bf16x4 hi4 = lds_read_tr16(vrow + 32 * db + 8 * VS);
      const bf16x8 a = __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[db], 0, 0, 0);
    }
  }
}

// One 64-key tile for one wave: both S^T blocks on MFMA first, then block 0's softmax
// (overlapping block 1's MFMAs) and P.V, then block 1's.
template <int D, bool DIAG>
__device__ __forceinline__ void bf16_tile_compute(const Bf16Stage<D>& st, const bf16x8 (&qreg)[D / 16],
                                                  f32x16 (&oacc)[D / 32], float& m, float& lsum, int key0,
                                                  int my_row, int lane, float scale_log2) {
  constexpr int KS = Bf16Tile<D, 4>::KS, KK = D / 16;
  const int l32 = lane & 31, hi = lane >> 5;
  f32x16 s0 = f32x16{}, s1 = f32x16{};
  const bf16* k0 = &st.k[l32 * KS + 8 * hi];
#if FOX_EXP_PRIO
  __builtin_amdgcn_s_setprio(1);
#endif
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(k0 + 16 * kk), qreg[kk], s0, 0,
                                                 0, 0);
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(k0 + 32 * KS + 16 * kk),
                                                 qreg[kk], s1, 0, 0, 0);
#if FOX_EXP_PRIO
  __builtin_amdgcn_s_setprio(0);
#endif
  bf16_block_softmax_pv<D, DIAG>(st, s0, 0, oacc, m, lsum, key0, my_row, lane, scale_log2);
  bf16_block_softmax_pv<D, DIAG>(st, s1, 1, oacc, m, lsum, key0, my_row, lane, scale_log2);
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ logf, bf16* __restrict__ o, float* __restrict__ lse, float* __restrict__ c_out, int n,
    float scale_log2) {
  constexpr int KK = D / 16, DB = D / 32, BR = 32 * NW;
  __shared__ Bf16Lds<D> lds;

  const int bh = blockIdx.x;
  const int qb = gridDim.y - 1 - blockIdx.y;
  const int row0 = qb * BR;
  const int ref = min(row0 + BR - 1, n - 1);
  const int kt_hi = ref / kBC;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const size_t base = (size_t)bh * n * D;
  const bf16* kb = k + base;
  const bf16* vb = v + base;
  const float* lfb = logf + (size_t)bh * n;

  const int wrow0 = row0 + wave * 32;
  const bool active = wrow0 < n;
  const int kt_first = active ? min(wrow0 + 31, n - 1) / kBC : -1;
  const int my_row = wrow0 + l32;

  bf16x8 qreg[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    if (my_row < n)
      qreg[kk] = *reinterpret_cast<const bf16x8*>(q + base + (size_t)my_row * D + 16 * kk + 8 * hi);
    else
      qreg[kk] = bf16x8{};
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m = kNegInf, lsum = 0.0f;
  double carry = 0.0;

  // Prologue: stage the top tile (the only one that may run past n) into buffer 0 and
  // start loading the next one.
  Bf16Tile<D, NW> tile;
  bf16_load_tile<D, NW>(tile, kb, vb, kt_hi, n, tid);
  float lf = 0.0f;  // wave 0: log f of key 63-lane of the tile being staged
  if (wave == 0) {
    const int j = kt_hi * kBC + 63 - lane;
    lf = (j <= ref) ? lfb[j] : 0.0f;
  }
  bf16_store_tile<D, NW>(tile, lds.st[0], tid);
  if (wave == 0) gate_tile(lds.st[0].r2, nullptr, lds.rows, lane, kt_hi, row0, ref, lf, carry);
  if (kt_hi > 0) {
    bf16_load_full_tile<D, NW>(tile, kb, vb, kt_hi - 1, tid);
    if (wave == 0) lf = lfb[(kt_hi - 1) * kBC + 63 - lane];
  }

  for (int kt = kt_hi; kt >= 0; --kt) {
    const int cur = (kt_hi - kt) & 1;
    // One barrier per tile: buffer `cur` is fully staged, and every wave is done with
    // buffer cur^1 (tile kt+1), which is staged next.
    __syncthreads();
    if (kt > 0) {
      bf16_store_tile<D, NW>(tile, lds.st[cur ^ 1], tid);
      if (wave == 0) gate_tile(lds.st[cur ^ 1].r2, nullptr, lds.rows, lane, kt - 1, row0, ref, lf, carry);
      if (kt > 1) {
        bf16_load_full_tile<D, NW>(tile, kb, vb, kt - 2, tid);
        if (wave == 0) lf = lfb[(kt - 2) * kBC + 63 - lane];
      }
    }
    if (!active || kt > kt_first) continue;
    const int key0 = kt * kBC;
    if (key0 + kBC - 1 > wrow0)
      bf16_tile_compute<D, true>(lds.st[cur], qreg, oacc, m, lsum, key0, my_row, lane, scale_log2);
    else
      bf16_tile_compute<D, false>(lds.st[cur], qreg, oacc, m, lsum, key0, my_row, lane, scale_log2);
  }

  // ---- epilogue: O = acc / l, lse, c ---------------------------------------------------
  __syncthreads();  // rows / cref written by wave 0 are visible (also when no tile was computed)
  if (!active) return;
  const float ltot = pair32_sum(lsum);
  if (my_row >= n) return;
  const float inv = 1.0f / ltot;
  bf16* orow = o + base + (size_t)my_row * D;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w;
      w[0] = pack_bf16x2(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv);
      w[1] = pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
      *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * g + 4 * hi) = w;
    }
  }
  if (hi == 0) {
    const double ri = lds.rows.rowR[my_row - row0];
    const size_t idx = (size_t)bh * n + my_row;
    if (lse) lse[idx] = (float)(((double)m + (double)log2_hw(ltot)) * kLn2d - ri);
    if (c_out) c_out[idx] = (float)(lds.rows.cref - ri);
  }
}

// ------------------------------------------------------------------------------------------
// fp32
// ------------------------------------------------------------------------------------------
template <int D>
struct F32Tile {
  static constexpr int KS = D + 1;  // K row stride (floats): odd, so column reads spread over banks
  static constexpr int VS = D + 8;  // V row stride (floats)
  static constexpr int GROUPS = D / 4;
  static constexpr int KPT = kBC * GROUPS / kThreads;
  static_assert(KPT >= 1 && KPT * kThreads == kBC * GROUPS, "loader mapping");
  f32x4 k[KPT];
  f32x4 v[KPT];
};

template <int D>
struct F32Lds {
  float k[kBC * F32Tile<D>::KS];
  float v[kBC * F32Tile<D>::VS];
  float r2[kBC];
  double r64[kBC];  // R_j in fp64: the fp32-input kernel forms R_j - R_i exactly from these
  GateRows rows;
};

template <int D>
__device__ __forceinline__ void f32_load_tile(F32Tile<D>& t, const float* kb, const float* vb, int kt, int n,
                                              int tid) {
  constexpr int G = F32Tile<D>::GROUPS, KPT = F32Tile<D>::KPT;
  const int c = tid % G, a = tid / G;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int key = kt * kBC + a * KPT + i;
    if (key < n) {
      t.k[i] = *reinterpret_cast<const f32x4*>(kb + (size_t)key * D + 4 * c);
      t.v[i] = *reinterpret_cast<const f32x4*>(vb + (size_t)key * D + 4 * c);
    } else {
      t.k[i] = f32x4{};
      t.v[i] = f32x4{};
    }
  }
}

template <int D>
__device__ __forceinline__ void f32_store_tile(const F32Tile<D>& t, F32Lds<D>& s, int tid) {
  constexpr int G = F32Tile<D>::GROUPS, KPT = F32Tile<D>::KPT, KS = F32Tile<D>::KS, VS = F32Tile<D>::VS;
  const int c = tid % G, a = tid / G;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int key = a * KPT + i;
#pragma unroll
    for (int e = 0; e < 4; ++e) s.k[key * KS + 4 * c + e] = t.k[i][e];
    *reinterpret_cast<f32x4*>(&s.v[key * VS + 4 * c]) = t.v[i];
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                          const float* __restrict__ v,
                                                          const float* __restrict__ logf, float* __restrict__ o,
                                                          float* __restrict__ lse, float* __restrict__ c_out, int n,
                                                          float scale_log2) {
  constexpr int KS = F32Tile<D>::KS, VS = F32Tile<D>::VS, KK = D / 2, DB = D / 32;
  __shared__ F32Lds<D> lds;

  const int bh = blockIdx.x;
  const int qb = gridDim.y - 1 - blockIdx.y;
  const int row0 = qb * kBR;
  const int ref = min(row0 + kBR - 1, n - 1);
  const int kt_hi = ref / kBC;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const size_t base = (size_t)bh * n * D;
  const float* kb = k + base;
  const float* vb = v + base;
  const float* lfb = logf + (size_t)bh * n;

  const int wrow0 = row0 + wave * 32;
  const bool active = wrow0 < n;
  const int kt_first = active ? min(wrow0 + 31, n - 1) / kBC : -1;
  const int my_row = wrow0 + l32;

  float qf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) qf[kk] = (my_row < n) ? q[base + (size_t)my_row * D + 2 * kk + hi] : 0.0f;

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m = kNegInf, lsum = 0.0f;
  double carry = 0.0, ri_row = 0.0;

  F32Tile<D> tile;
  f32_load_tile<D>(tile, kb, vb, kt_hi, n, tid);
  float lf = 0.0f;  // wave 0: log f of key 63-lane of the next tile
  if (wave == 0) {
    const int j = kt_hi * kBC + 63 - lane;
    lf = (j <= ref) ? lfb[j] : 0.0f;
  }

  for (int kt = kt_hi; kt >= 0; --kt) {
    __syncthreads();
    f32_store_tile<D>(tile, lds, tid);
    if (wave == 0) gate_tile(lds.r2, lds.r64, lds.rows, lane, kt, row0, ref, lf, carry);
    __syncthreads();
    if (kt > 0) {
      f32_load_tile<D>(tile, kb, vb, kt - 1, n, tid);
      if (wave == 0) lf = lfb[(kt - 1) * kBC + 63 - lane];
    }
    if (!active || kt > kt_first) continue;

    f32x16 sacc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      sacc[b] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        sacc[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(lds.k[(32 * b + l32) * KS + 2 * kk + hi], qf[kk], sacc[b],
                                                       0, 0, 0);
    }

    // This row's R_i is in the gate LDS from the wave's first (diagonal) tile on.
    if (kt == kt_first) ri_row = (my_row < n) ? lds.rows.rowR[my_row - row0] : 0.0;
    const bool diag = kt * kBC + kBC - 1 > wrow0;
    float mx = kNegInf;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int kl = 32 * b + 8 * g + 4 * hi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // full bias sum_{t=j+1..i} log f_t = R_j - R_i, formed in fp64 and rounded once
          const float bias2 = (float)((lds.r64[kl + e] - ri_row) * kLog2ed);
          float s = fmaf(sacc[b][4 * g + e], scale_log2, bias2);
          if (diag && kt * kBC + kl + e > my_row) s = kNegInf;
          sacc[b][4 * g + e] = s;
          mx = fmaxf(mx, s);
        }
      }
    }
    mx = pair32_max(mx);

    const float mcand = fmaxf(m, mx);
    const bool need = mcand > m + kTau;
    if (wave_any(need)) {
      const float mn = need ? mcand : m;
      const float alpha = exp2_hw(m - mn);
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      m = mn;
    }
    const float msub = (m == kNegInf) ? 0.0f : m;

#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2_hw(sacc[b][r] - msub);
        lsum += p;
        const int key = 32 * b + 8 * (r / 4) + 4 * hi + (r % 4);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(lds.v[key * VS + 32 * db + l32], p, oacc[db], 0, 0, 0);
      }
    }
  }

  if (!active) return;
  const float ltot = pair32_sum(lsum);
  if (my_row >= n) return;
  const float inv = 1.0f / ltot;
  float* orow = o + base + (size_t)my_row * D;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = oacc[db][4 * g + e] * inv;
      *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * g + 4 * hi) = w;
    }
  }
  if (hi == 0) {
    const double ri = lds.rows.rowR[my_row - row0];
    const size_t idx = (size_t)bh * n + my_row;
    if (lse) lse[idx] = (float)(((double)m + (double)log2f(ltot)) * kLn2d);  // scores already carry -R_i
    if (c_out) c_out[idx] = (float)(lds.rows.cref - ri);
  }
}

template <typename T, int D>
hipError_t launch_fwd_t(const void* q, const void* k, const void* v, const float* logf, void* o, float* lse,
                        float* c, int64_t bh, int n, float scale_log2, hipStream_t stream) {
  if constexpr (sizeof(T) == 2) {
    // 256-row blocks (8 waves) stage each K/V tile for twice the compute of 128-row
    // blocks, halving the L2 -> LDS traffic per flop; used when there are enough blocks
    // to keep every CU busy for two rounds.
    int cus = 256, dev = 0;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const int64_t blocks256 = bh * (int64_t)((n + 255) / 256);
    bool big = false;
    if constexpr (D >= 64) {
      if (blocks256 >= 2 * (int64_t)cus) {
        big = true;
        const dim3 grid((unsigned)bh, (unsigned)((n + 255) / 256));
        hipLaunchKernelGGL((fwd_bf16_kernel<D, 8>), grid, dim3(512), 0, stream, (const bf16*)q, (const bf16*)k,
                           (const bf16*)v, logf, (bf16*)o, lse, c, n, scale_log2);
      }
    }
    if (!big) {
      const dim3 grid((unsigned)bh, (unsigned)((n + 127) / 128));
      hipLaunchKernelGGL((fwd_bf16_kernel<D, 4>), grid, dim3(256), 0, stream, (const bf16*)q, (const bf16*)k,
                         (const bf16*)v, logf, (bf16*)o, lse, c, n, scale_log2);
    }
  } else {
    const dim3 grid((unsigned)bh, (unsigned)((n + kBR - 1) / kBR));
    hipLaunchKernelGGL(fwd_f32_kernel<D>, grid, dim3(kThreads), 0, stream, (const float*)q, (const float*)k,
                       (const float*)v, logf, (float*)o, lse, c, n, scale_log2);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const void* q, const void* k, const void* v, const float* logf, void* o, float* lse,
                           float* c, int64_t bh, int n, int d, float scale, bool is_bf16, hipStream_t stream) {
  const float scale_log2 = (float)((double)scale * kLog2ed);
  if (is_bf16) {
    switch (d) {
      case 32: return launch_fwd_t<bf16, 32>(q, k, v, logf, o, lse, c, bh, n, scale_log2, stream);
      case 64: return launch_fwd_t<bf16, 64>(q, k, v, logf, o, lse, c, bh, n, scale_log2, stream);
      case 128: return launch_fwd_t<bf16, 128>(q, k, v, logf, o, lse, c, bh, n, scale_log2, stream);
    }
  } else {
    switch (d) {
      case 32: return launch_fwd_t<float, 32>(q, k, v, logf, o, lse, c, bh, n, scale_log2, stream);
      case 64: return launch_fwd_t<float, 64>(q, k, v, logf, o, lse, c, bh, n, scale_log2, stream);
      case 128: return launch_fwd_t<float, 128>(q, k, v, logf, o, lse, c, bh, n, scale_log2, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace fox
