// fox_fwd_f32.hip -- the FoX forward on fp32 tensors (both modes, both layouts).
//
// Definition as in fox_fwd.hip (FoX module page, ForgettingAttention.forward; foxwindow README,
// opening paragraph).  A non-pipelined schedule on v_mfma_f32_32x32x2f32 with fp32 P: 128 query rows
// per workgroup (32 per wave), 64-key tiles staged through LDS from registers, the gate sums of each
// tile scanned in fp64 by wave 0 (fox_fwd_gates.h).  The bias R_j - R_i is formed per score in fp64
// from LDS copies of R_j, so no fp32 rounding of a block-relative gate sum enters the scores.
//
// This file is compiled apart from the bf16 kernels: it keeps the compiler's default MFMA form,
// which at d = 128 (one wave per SIMD) holds O in AGPRs.
#include <math.h>

#include "fox_device.h"
#include "fox_fwd_gates.h"

namespace fox {
namespace {

constexpr int kThreads = 256;  // threads per workgroup
constexpr int kBR = 128;       // query rows per workgroup (32 per wave)

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
                                              int tid, int rs) {
  constexpr int G = F32Tile<D>::GROUPS, KPT = F32Tile<D>::KPT;
  const int c = tid % G, a = tid / G;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int key = kt * kBC + a * KPT + i;
    if (key < n) {
      t.k[i] = *reinterpret_cast<const f32x4*>(kb + (size_t)key * rs + 4 * c);
      t.v[i] = *reinterpret_cast<const f32x4*>(vb + (size_t)key * rs + 4 * c);
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

template <int D, bool CAUSAL, bool TM>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                          const float* __restrict__ v,
                                                          const float* __restrict__ logf, float* __restrict__ o,
                                                          float* __restrict__ lse, float* __restrict__ c_out, int n,
                                                          float scale_log2, const FwdLayout lay) {
  constexpr int KS = F32Tile<D>::KS, VS = F32Tile<D>::VS, KK = D / 2, DB = D / 32;
  __shared__ F32Lds<D> lds;

  const int bh = blockIdx.x;
  const int qb = gridDim.y - 1 - blockIdx.y;
  const int row0 = qb * kBR;
  const int ref = min(row0 + kBR - 1, n - 1);  // the block's last row
  const int fref = CAUSAL ? ref : n - 1;       // frame row of the gate sums
  const int kt_hi = fref / kBC;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int bb = bh / lay.nh, hh = bh - bb * lay.nh;
  const size_t base = TM ? (size_t)bb * lay.bs + (size_t)hh * lay.hs : (size_t)bh * n * D;  // q/k/v/o
  const size_t gbase = TM ? (size_t)bb * lay.gbs + (size_t)hh * lay.ghs : (size_t)bh * n;  // gates/lse/c
  const int rs = TM ? lay.rs : D, gs = TM ? lay.gs : 1;
  const float* kb = k + base;
  const float* vb = v + base;
  const float* lfb = logf + gbase;

  const int wrow0 = row0 + wave * 32;
  const bool active = wrow0 < n;
  const int kt_first = !active ? -1 : (CAUSAL ? min(wrow0 + 31, n - 1) / kBC : kt_hi);
  const int my_row = wrow0 + l32;

  float qf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) qf[kk] = (my_row < n) ? q[base + (size_t)my_row * rs + 2 * kk + hi] : 0.0f;

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  // The row sum runs in fp64 over per-tile fp32 partial sums of 32 terms (a single fp32 running
  // sum over thousands of keys drifts by more than the 1e-5 that lse must meet), and lse takes
  // an fp64 logarithm.
  float m = kNegInf;
  double lsum = 0.0;
  double carry = 0.0, ri_row = 0.0;
  // Unmasked mode: the biases stay relative to the frame row n-1 (R_j - 0), where every row's
  // heaviest keys lie, so those scores are small and exactly rounded; R_i comes off in lse.
  F32Tile<D> tile;
  f32_load_tile<D>(tile, kb, vb, kt_hi, n, tid, rs);
  float lf = 0.0f;  // wave 0: log f of key 63-lane of the next tile
  if (wave == 0) {
    const int j = kt_hi * kBC + 63 - lane;
    lf = (j <= fref) ? lfb[(size_t)j * gs] : 0.0f;
  }

  for (int kt = kt_hi; kt >= 0; --kt) {
    __syncthreads();
    f32_store_tile<D>(tile, lds, tid);
    if (wave == 0) gate_tile(lds.r2, lds.r64, lds.rows, lane, kt, row0, ref, lf, carry, kLog2ed);
    __syncthreads();
    if (kt > 0) {
      f32_load_tile<D>(tile, kb, vb, kt - 1, n, tid, rs);
      if (wave == 0) lf = lfb[(size_t)((kt - 1) * kBC + 63 - lane) * gs];
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
    if (CAUSAL && kt == kt_first) ri_row = (my_row < n) ? lds.rows.rowR[my_row - row0] : 0.0;
    // causal: keys past the row; otherwise only keys past the end of the sequence
    const int last_key = CAUSAL ? my_row : n - 1;
    const bool diag = CAUSAL ? kt * kBC + kBC - 1 > wrow0 : kt * kBC + kBC > n;
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
          if (diag && kt * kBC + kl + e > last_key) s = kNegInf;
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

    float tsum[2] = {0.0f, 0.0f};
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2_hw(sacc[b][r] - msub);
        tsum[r & 1] += p;
        const int key = 32 * b + 8 * (r / 4) + 4 * hi + (r % 4);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(lds.v[key * VS + 32 * db + l32], p, oacc[db], 0, 0, 0);
      }
    }
    lsum += (double)tsum[0] + (double)tsum[1];
  }

  if (!active) return;
  const double ltot = lsum + __shfl_xor(lsum, 32);
  if (my_row >= n) return;
  const float inv = (float)(1.0 / ltot);
  float* orow = o + base + (size_t)my_row * rs;
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
    const size_t idx = gbase + (size_t)my_row * gs;
    // causal scores already carry -R_i
    if (lse) lse[idx] = (float)(((double)m + log2(ltot)) * kLn2d - (CAUSAL ? 0.0 : ri));
    if (c_out) c_out[idx] = (float)(lds.rows.cref - ri);
  }
}

template <int D, bool CAUSAL, bool TM>
hipError_t launch_f32_t(const float* q, const float* k, const float* v, const float* logf, float* o, float* lse,
                        float* c, int64_t bh, int n, float scale_log2, const FwdLayout& lay, hipStream_t stream) {
  const dim3 grid((unsigned)bh, (unsigned)((n + kBR - 1) / kBR));
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL, TM>), grid, dim3(kThreads), 0, stream, q, k, v, logf, o, lse, c, n,
                     scale_log2, lay);
  return hipGetLastError();
}

template <bool CAUSAL, bool TM>
hipError_t launch_f32_m(const float* q, const float* k, const float* v, const float* logf, float* o, float* lse,
                        float* c, int64_t bh, int n, int d, float scale_log2, const FwdLayout& lay,
                        hipStream_t stream) {
  switch (d) {
    case 32: return launch_f32_t<32, CAUSAL, TM>(q, k, v, logf, o, lse, c, bh, n, scale_log2, lay, stream);
    case 64: return launch_f32_t<64, CAUSAL, TM>(q, k, v, logf, o, lse, c, bh, n, scale_log2, lay, stream);
    case 128: return launch_f32_t<128, CAUSAL, TM>(q, k, v, logf, o, lse, c, bh, n, scale_log2, lay, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, const float* logf, float* o, float* lse,
                          float* c, int64_t bh, int n, int d, float scale_log2, bool causal, bool token_major,
                          const FwdLayout& lay, hipStream_t stream) {
  if (causal)
    return token_major ? launch_f32_m<true, true>(q, k, v, logf, o, lse, c, bh, n, d, scale_log2, lay, stream)
                       : launch_f32_m<true, false>(q, k, v, logf, o, lse, c, bh, n, d, scale_log2, lay, stream);
  return token_major ? launch_f32_m<false, true>(q, k, v, logf, o, lse, c, bh, n, d, scale_log2, lay, stream)
                     : launch_f32_m<false, false>(q, k, v, logf, o, lse, c, bh, n, d, scale_log2, lay, stream);
}

}  // namespace fox
