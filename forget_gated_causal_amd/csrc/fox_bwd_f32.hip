// fox_bwd_f32.hip -- backward pass of FoX attention on fp32 tensors (the fp32 forward's gradients).
//
// The same chain rule as the bf16 backward (fox_bwd.hip), through the forward definition of the
// FoX module page (ForgettingAttention.forward), in fp32 throughout (no bf16 rounding of P or dS):
//   P_ij = exp(s_ij - lse_i) with s_ij = scale q_i.k_j + c_i - c_j (j <= i when causal)
//   dv = P^T dO;  dP = dO v^T;  dS = P * (dP - D_i), D_i = dO_i . O_i
//   dq = scale dS k;  dk = scale dS^T q;  dlog f_t = sum_{i >= t} (rowsum(dS)_i - colsum(dS)_i)
// The fp32 path serves the fp32 forward's (small, correctness-sized) workloads, so it runs on the
// vector ALU in plain tiles rather than on MFMA:
//  * The gate-rows kernel (fox_bwd.hip) writes the fp64 block starts C_b of the gate prefix sums
//    (as for the bf16 path); these kernels form the in-block parts cq_i = c_i - C_b(i) themselves,
//    in fp64, from log f (f32_inblock: one wave scan per 64 positions).  Each score's exponent is
//    scale q.k log2 e plus one fp32 rounding of its whole bias, formed in fp64 per (row, key) as
//    [(cq_i - lse_i) log2 e - corr_i + (C_b(i) - C_b(j)) log2 e] - cq_j log2 e, the bracket once
//    per (row, key block).  The bias is as small as the exponents of the scores that carry weight,
//    while c_i and lse_i alone can be thousands (without the mask, where later keys are weighted
//    up, lse_i follows c_i of the heaviest keys) and cq_i and cq_j up to 32 |log f| each, which
//    with strong gates (|log f| of 4 and more) is far above the bias of a weighted pair.
//  * In the unmasked mode the lse the backward is given (fp32, |lse| possibly in the thousands) is
//    itself only good to half an ulp of that size: a normalisation pass (bwd_f32_dq_kernel with
//    ZPASS) sums P_ij over each row with it and keeps corr_i = log2 sum_j P_ij, which the main
//    kernels subtract, so each row of P sums to 1 to fp64 rounding of the fp32 terms.  The same
//    pass forms D_i = sum_j P_ij dP_ij (P so normalised) rather than dO_i . O_i: without the mask
//    dlog f is a difference of cross-block sums of dS over every row, and with D_i formed from the
//    same fp32 P and dP as dS, each row of dS sums to zero up to the rounding of its own terms,
//    where the rounding of O and of its dot product with dO would add up over the rows.
//  * bwd_f32_pre_kernel (with the mask): D_i = dO_i . O_i into the row vectors.
//  * bwd_f32_kv_kernel<D, CAUSAL>: one 256-thread workgroup per (64-key block, head); the block's K
//    and V rows sit in LDS, 32-query tiles of q and dO stream through it.  Per tile, thread t forms
//    P and dS for key t % 64 and queries 8 (t / 64) .. +7 (phase A, into LDS), then accumulates
//    dV and dK for key t % 64 over dims D/4 (t / 64) .. +D/4 (phase B).  Writes dk, dv and the
//    column sums of dS.
//  * bwd_f32_dq_kernel<D, CAUSAL>: one workgroup per (64-query block, head), 32-key tiles; the same
//    two phases with queries and keys exchanged.  Writes dq and the row sums of dS.
//  * The reversed gate scan (fox_scan.hip) turns row sums - column sums into dlog f.
// Every output element has one writer.  LDS rows are padded by one float, so the per-thread row
// reads (stride D + 1 words) fall in distinct banks.
#include <math.h>

#include "fox_device.h"
#include "fox_internal.h"

namespace fox {
namespace {

constexpr int kF32Threads = 256;
constexpr int kF32Blk = 64;   // keys (kv kernel) or queries (dq kernel) per workgroup
constexpr int kF32Tile = 32;  // queries (kv kernel) or keys (dq kernel) per streamed tile
constexpr int kF32Pad = 64;   // per-head row vectors are padded to a multiple of this

// Strides of one backward call (elements): tensors (bs, hs, rs), gate-sized vectors (gbs, ghs, gs).
struct F32Layout {
  int64_t bs, hs;
  int rs;
  int64_t gbs, ghs;
  int gs;
  int nh;
  __device__ __forceinline__ int64_t tbase(int bh) const { return (int64_t)(bh / nh) * bs + (bh % nh) * hs; }
  __device__ __forceinline__ int64_t gbase(int bh) const { return (int64_t)(bh / nh) * gbs + (bh % nh) * ghs; }
};

int f32_npad(int n) { return (n + kF32Pad - 1) / kF32Pad * kF32Pad; }

// One thread per (head, row): D_i = dO_i . O_i into the row vectors' D slot (the gate-rows kernel
// writes the rest, padding included).
template <int D>
__global__ __launch_bounds__(kF32Threads) void bwd_f32_pre_kernel(const float* __restrict__ o,
                                                                  const float* __restrict__ dout,
                                                                  float* __restrict__ rowv, int64_t bh_count, int n,
                                                                  int npad, F32Layout lay) {
  const int64_t prow = (int64_t)blockIdx.x * kF32Threads + threadIdx.x;
  const int64_t bh = prow / npad;
  if (bh >= bh_count) return;
  const int i = (int)(prow - bh * npad);
  float* blk = rowv + bh * 3 * npad;
  if (i >= n) return;
  const float* orow = o + lay.tbase((int)bh) + (int64_t)i * lay.rs;
  const float* drow = dout + lay.tbase((int)bh) + (int64_t)i * lay.rs;
  float s = 0.0f;
#pragma unroll 8
  for (int e = 0; e < D; ++e) s = fmaf(orow[e], drow[e], s);
  blk[npad + i] = s;
}

// In-block parts of the gate prefix sums for the 64 positions p0 .. p0 + 63 (p0 a multiple of 32,
// so two whole gate blocks), fp64 in log2 units: lane l of the calling wave (all 64 lanes active)
// gets cq_{p0+l} log2 e, cq_i = sum_{32 b(i) <= t <= i} log f_t, or +inf at or past n.
__device__ __forceinline__ double f32_inblock(const float* __restrict__ logf, int64_t gb, int gs, int p0, int n,
                                              int lane) {
  const int p = p0 + lane;
  const double incl = wave_incl_scan(p < n ? (double)logf[gb + (int64_t)p * gs] : 0.0);
  const u32x2 w = __builtin_bit_cast(u32x2, incl);
  u32x2 r;
  r[0] = (uint32_t)__builtin_amdgcn_readlane((int)w[0], 31);
  r[1] = (uint32_t)__builtin_amdgcn_readlane((int)w[1], 31);
  const double first = __builtin_bit_cast(double, r);  // the sum over the first block
  return p < n ? (lane < 32 ? incl : incl - first) * kLog2ed : INFINITY;
}

// Lane src's value of x (every lane of the wave active).
__device__ __forceinline__ double lane_value(double x, int src) {
  const u32x2 w = __builtin_bit_cast(u32x2, x);
  u32x2 r;
  r[0] = (uint32_t)__shfl((int)w[0], src);
  r[1] = (uint32_t)__shfl((int)w[1], src);
  return __builtin_bit_cast(double, r);
}

// Copy `rows` rows of D floats (global row stride rs) into an LDS tile of row stride D + 1;
// rows at or past `valid` read as zeros.
template <int D>
__device__ __forceinline__ void f32_stage(float* lds, const float* src, int rows, int valid, int rs) {
  for (int x = threadIdx.x; x < rows * D; x += kF32Threads) {
    const int r = x / D, e = x - r * D;
    lds[r * (D + 1) + e] = r < valid ? src[(int64_t)r * rs + e] : 0.0f;
  }
}

// Four interleaved partial sums (dims e mod 4), so the FMA chain is a quarter as long.
template <int D>
__device__ __forceinline__ float f32_dot(const float* a, const float* b) {
  float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll 8
  for (int e = 0; e < D; e += 4) {
    s0 = fmaf(a[e], b[e], s0);
    s1 = fmaf(a[e + 1], b[e + 1], s1);
    s2 = fmaf(a[e + 2], b[e + 2], s2);
    s3 = fmaf(a[e + 3], b[e + 3], s3);
  }
  return (s0 + s1) + (s2 + s3);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kF32Threads) void bwd_f32_kv_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dout, const float* __restrict__ rowv, const double* __restrict__ cb,
    const float* __restrict__ logf, const float* __restrict__ lse, const float* __restrict__ corr,
    float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ colsum_out, int n, int npad, int ncb,
    float scale, F32Layout lay) {
  constexpr int DP = D + 1, DC = D / 4;
  static_assert(kF32Blk == 2 * kF32Tile && kF32Tile == 32, "two 32-position gate blocks of keys per workgroup");
  __shared__ float ks[kF32Blk * DP], vs[kF32Blk * DP];
  __shared__ float qs[kF32Tile * DP], ds_[kF32Tile * DP];
  __shared__ float pt[kF32Blk * (kF32Tile + 1)], st[kF32Blk * (kF32Tile + 1)];
  __shared__ double arow[2][kF32Tile];
  __shared__ float drow[kF32Tile], csum[4][kF32Blk];
  const int bh = blockIdx.x, key0 = blockIdx.y * kF32Blk;
  const int tid = threadIdx.x, jl = tid & 63, g = tid >> 6;
  const int j = key0 + jl;
  const int64_t tb = lay.tbase(bh);
  const float* blk = rowv + (int64_t)bh * 3 * npad;
  const float scale_log2 = scale * kLog2e;
  f32_stage<D>(ks, k + tb + (int64_t)key0 * lay.rs, kF32Blk, n - key0, lay.rs);
  f32_stage<D>(vs, v + tb + (int64_t)key0 * lay.rs, kF32Blk, n - key0, lay.rs);
  const int64_t gb = lay.gbase(bh);
  const double clj = f32_inblock(logf, gb, lay.gs, key0, n, jl);  // this thread's key; +inf past n
  const double* cbh = cb + (int64_t)bh * ncb;
  float accv[DC], acck[DC];
#pragma unroll
  for (int x = 0; x < DC; ++x) accv[x] = acck[x] = 0.0f;
  float cs = 0.0f;
  const int qfirst = CAUSAL ? key0 : 0;  // earlier queries see none of these keys
  for (int q0 = qfirst - qfirst % kF32Tile; q0 < n; q0 += kF32Tile) {
    __syncthreads();  // the previous tile's phase B is done with qs, ds_, pt, st
    f32_stage<D>(qs, q + tb + (int64_t)q0 * lay.rs, kF32Tile, n - q0, lay.rs);
    f32_stage<D>(ds_, dout + tb + (int64_t)q0 * lay.rs, kF32Tile, n - q0, lay.rs);
    const double cqt = f32_inblock(logf, gb, lay.gs, q0, n, jl);  // lanes 0..31: the tile's queries
    if (tid < 2 * kF32Tile) {
      // row term of query i against key block kb: (c_i - C_kb - lse_i) log2 e - corr_i, in fp64
      const int kb = tid / kF32Tile, il = tid % kF32Tile, i = q0 + il;
      const double cqi = lane_value(cqt, il);
      double a = -INFINITY;
      if (i < n)
        a = cqi - (double)lse[gb + (int64_t)i * lay.gs] * kLog2ed - (corr ? (double)corr[(int64_t)bh * n + i] : 0.0) +
            (cbh[q0 >> 5] - cbh[(key0 >> 5) + kb]) * kLog2ed;
      arow[kb][il] = a;
    } else if (tid < 3 * kF32Tile) {
      const int il = tid - 2 * kF32Tile;
      drow[il] = q0 + il < n ? blk[npad + q0 + il] : 0.0f;
    }
    __syncthreads();
    const double* arw = arow[jl / kF32Tile];  // this key's block
    // phase A: P and dS for key j and queries q0 + 8g .. + 7
#pragma unroll 1
    for (int u = 0; u < 8; ++u) {
      const int il = 8 * g + u, i = q0 + il;
      float p = 0.0f, dsv = 0.0f;
      if (j < n && i < n && (!CAUSAL || j <= i)) {
        const float s = f32_dot<D>(&ks[jl * DP], &qs[il * DP]);
        const float dp = f32_dot<D>(&vs[jl * DP], &ds_[il * DP]);
        p = exp2_hw(fmaf(s, scale_log2, (float)(arw[il] - clj)));
        dsv = p * (dp - drow[il]);
      }
      pt[jl * (kF32Tile + 1) + il] = p;
      st[jl * (kF32Tile + 1) + il] = dsv;
      cs += dsv;
    }
    __syncthreads();
    // phase B: dV_j += P_j. dO, dK_j += dS_j. Q over dims DC g .. DC g + DC - 1
#pragma unroll 1
    for (int il = 0; il < kF32Tile; ++il) {
      const float p = pt[jl * (kF32Tile + 1) + il], dsv = st[jl * (kF32Tile + 1) + il];
#pragma unroll
      for (int x = 0; x < DC; ++x) {
        accv[x] = fmaf(p, ds_[il * DP + DC * g + x], accv[x]);
        acck[x] = fmaf(dsv, qs[il * DP + DC * g + x], acck[x]);
      }
    }
  }
  csum[g][jl] = cs;
  __syncthreads();
  if (j < n) {
    float* dkr = dk + tb + (int64_t)j * lay.rs + DC * g;
    float* dvr = dv + tb + (int64_t)j * lay.rs + DC * g;
#pragma unroll
    for (int x = 0; x < DC; ++x) {
      dkr[x] = acck[x] * scale;
      dvr[x] = accv[x];
    }
    if (g == 0) colsum_out[(int64_t)bh * n + j] = (csum[0][jl] + csum[1][jl]) + (csum[2][jl] + csum[3][jl]);
  }
}

// ZPASS: the normalisation pass instead -- per row, with the given lse, Z_i = sum_j P_ij and
// sum_j P_ij dP_ij (fp64 sums of the fp32 terms); writes corr_i = log2 Z_i to corr_out and
// D_i = sum_j P_ij dP_ij / Z_i to dslot_out (the row vectors' D slot, which this pass does not
// read); no dQ.
template <int D, bool CAUSAL, bool ZPASS = false>
__global__ __launch_bounds__(kF32Threads) void bwd_f32_dq_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dout, const float* __restrict__ rowv, const double* __restrict__ cb,
    const float* __restrict__ logf, const float* __restrict__ lse, const float* __restrict__ corr,
    float* __restrict__ dq,
    float* __restrict__ rowsum_out, float* __restrict__ corr_out, float* __restrict__ dslot_out, int n, int npad,
    int ncb, float scale, F32Layout lay) {
  constexpr int DP = D + 1, DC = D / 4;
  __shared__ float qs[kF32Blk * DP], ds_[kF32Blk * DP];
  __shared__ float ks[kF32Tile * DP], vs[kF32Tile * DP];
  __shared__ float st[kF32Blk * (kF32Tile + 1)];
  __shared__ double clt[kF32Tile];
  __shared__ float rsum[4][kF32Blk];
  __shared__ double zsum[ZPASS ? 4 : 1][kF32Blk], wsum[ZPASS ? 4 : 1][kF32Blk];
  const int bh = blockIdx.x, qblk0 = blockIdx.y * kF32Blk;
  const int tid = threadIdx.x, il = tid & 63, g = tid >> 6;
  const int i = qblk0 + il;
  const int64_t tb = lay.tbase(bh);
  const float* blk = rowv + (int64_t)bh * 3 * npad;
  const float scale_log2 = scale * kLog2e;
  f32_stage<D>(qs, q + tb + (int64_t)qblk0 * lay.rs, kF32Blk, n - qblk0, lay.rs);
  f32_stage<D>(ds_, dout + tb + (int64_t)qblk0 * lay.rs, kF32Blk, n - qblk0, lay.rs);
  const float di = (i < n && !ZPASS) ? blk[npad + i] : 0.0f;
  const double* cbh = cb + (int64_t)bh * ncb;
  const double cqi = cbh[i >> 5];  // start of the query's 32-position block
  const int64_t gb = lay.gbase(bh);
  const double cqd = f32_inblock(logf, gb, lay.gs, qblk0, n, il);  // this thread's query
  // row term (c_i - C_b(i) - lse_i) log2 e - corr_i in fp64; each key tile adds its block difference
  const double ri = i < n ? cqd - (double)lse[gb + (int64_t)i * lay.gs] * kLog2ed -
                                (corr ? (double)corr[(int64_t)bh * n + i] : 0.0)
                          : 0.0;
  double zs = 0.0, wsp = 0.0;
  float acc[DC];
#pragma unroll
  for (int x = 0; x < DC; ++x) acc[x] = 0.0f;
  float rs = 0.0f;
  const int kend = CAUSAL ? min(n, qblk0 + kF32Blk) : n;  // later keys are masked for every row
  for (int k0 = 0; k0 < kend; k0 += kF32Tile) {
    __syncthreads();  // the previous tile's phase B is done with ks, vs, st
    f32_stage<D>(ks, k + tb + (int64_t)k0 * lay.rs, kF32Tile, n - k0, lay.rs);
    f32_stage<D>(vs, v + tb + (int64_t)k0 * lay.rs, kF32Tile, n - k0, lay.rs);
    const double ckt = f32_inblock(logf, gb, lay.gs, k0, n, il);  // lanes 0..31: the tile's keys
    if (tid < kF32Tile) clt[tid] = ckt;
    __syncthreads();
    // the row term with the tile's block difference (the tile is one 32-position block)
    const double ait = i < n ? ri + (cqi - cbh[k0 >> 5]) * kLog2ed : -INFINITY;
#pragma unroll 1
    for (int u = 0; u < 8; ++u) {
      const int jl = 8 * g + u, j = k0 + jl;
      float dsv = 0.0f;
      if (j < n && i < n && (!CAUSAL || j <= i)) {
        const float s = f32_dot<D>(&qs[il * DP], &ks[jl * DP]);
        const float p = exp2_hw(fmaf(s, scale_log2, (float)(ait - clt[jl])));
        const float dp = f32_dot<D>(&ds_[il * DP], &vs[jl * DP]);
        if constexpr (ZPASS) {
          zs += (double)p;
          wsp += (double)p * (double)dp;
        } else {
          dsv = p * (dp - di);
        }
      }
      if constexpr (!ZPASS) {
        st[il * (kF32Tile + 1) + jl] = dsv;
        rs += dsv;
      }
    }
    __syncthreads();
    if constexpr (ZPASS) continue;
#pragma unroll 1
    for (int jl = 0; jl < kF32Tile; ++jl) {
      const float dsv = st[il * (kF32Tile + 1) + jl];
#pragma unroll
      for (int x = 0; x < DC; ++x) acc[x] = fmaf(dsv, ks[jl * DP + DC * g + x], acc[x]);
    }
  }
  if constexpr (ZPASS) {
    zsum[g][il] = zs;
    wsum[g][il] = wsp;
    __syncthreads();
    if (i < n && g == 0) {
      double z = (zsum[0][il] + zsum[1][il]) + (zsum[2][il] + zsum[3][il]);
      if (!(z > 0.0 && z < INFINITY)) z = 1.0;  // an lse that does not belong to these scores
      corr_out[(int64_t)bh * n + i] = (float)log2(z);
      dslot_out[(int64_t)bh * 3 * npad + npad + i] = (float)(((wsum[0][il] + wsum[1][il]) + (wsum[2][il] + wsum[3][il])) / z);
    }
    return;
  }
  rsum[g][il] = rs;
  __syncthreads();
  if (i < n) {
    float* dqr = dq + tb + (int64_t)i * lay.rs + DC * g;
#pragma unroll
    for (int x = 0; x < DC; ++x) dqr[x] = acc[x] * scale;
    if (g == 0) rowsum_out[(int64_t)bh * n + i] = (rsum[0][il] + rsum[1][il]) + (rsum[2][il] + rsum[3][il]);
  }
}

template <int D>
hipError_t launch_bwd_f32_t(const float* q, const float* k, const float* v, const float* o, const float* dout,
                            const float* lse, const float* logf, float* dq, float* dk, float* dv, float* dlogf,
                            void* ws, int64_t b, int64_t h, int n, float scale, bool causal, bool token_major,
                            hipStream_t stream) {
  const int64_t bh = b * h;
  const int npad = f32_npad(n);
  const int ncb = bwd_gate_blocks(n);
  // {bs, hs, rs, gbs, ghs, gs, nh}
  const F32Layout lay = token_major
                            ? F32Layout{(int64_t)n * h * D, (int64_t)D, (int)(h * D), (int64_t)n * h, 1, (int)h, (int)h}
                            : F32Layout{h * n * (int64_t)D, (int64_t)n * D, D, h * (int64_t)n, (int64_t)n, 1, (int)h};
  const BwdWorkspace w = bwd_workspace(ws, bh, n, npad);
  hipError_t e = launch_bwd_gate_rows(logf, lse, w.rowv, w.cb, bh, n, npad, (int)h, token_major, stream);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)bh, (unsigned)((n + kF32Blk - 1) / kF32Blk));
  const float* rowv = w.rowv;
  const double* cb = w.cb;
  if (causal) {  // |lse| stays small with the mask: the given lse is used as it is
    hipLaunchKernelGGL((bwd_f32_pre_kernel<D>), dim3((unsigned)((bh * npad + kF32Threads - 1) / kF32Threads)),
                       dim3(kF32Threads), 0, stream, o, dout, w.rowv, bh, n, npad, lay);
    hipLaunchKernelGGL((bwd_f32_kv_kernel<D, true>), grid, dim3(kF32Threads), 0, stream, q, k, v, dout, rowv, cb,
                       logf, lse, (const float*)nullptr, dk, dv, w.csum, n, npad, ncb, scale, lay);
    hipLaunchKernelGGL((bwd_f32_dq_kernel<D, true>), grid, dim3(kF32Threads), 0, stream, q, k, v, dout, rowv, cb,
                       logf, lse, (const float*)nullptr, dq, w.rsum, (float*)nullptr, (float*)nullptr, n, npad, ncb,
                       scale, lay);
  } else {
    hipLaunchKernelGGL((bwd_f32_dq_kernel<D, false, true>), grid, dim3(kF32Threads), 0, stream, q, k, v, dout, rowv,
                       cb, logf, lse, (const float*)nullptr, (float*)nullptr, (float*)nullptr, w.corr, w.rowv, n,
                       npad, ncb, scale, lay);
    hipLaunchKernelGGL((bwd_f32_kv_kernel<D, false>), grid, dim3(kF32Threads), 0, stream, q, k, v, dout, rowv, cb,
                       logf, lse, (const float*)w.corr, dk, dv, w.csum, n, npad, ncb, scale, lay);
    hipLaunchKernelGGL((bwd_f32_dq_kernel<D, false>), grid, dim3(kF32Threads), 0, stream, q, k, v, dout, rowv, cb,
                       logf, lse, (const float*)w.corr, dq, w.rsum, (float*)nullptr, (float*)nullptr, n, npad, ncb,
                       scale, lay);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // dlog f_t = sum_{i >= t} (rowsum_i - colsum_i), written in the gates' layout
  return launch_suffix_sum(w.rsum, w.csum, dlogf, bh, n, (int)h, token_major, stream);
}

}  // namespace

hipError_t launch_attn_bwd_f32(const float* q, const float* k, const float* v, const float* o, const float* dout,
                               const float* lse, const float* logf, float* dq, float* dk, float* dv, float* dlogf,
                               void* workspace, int64_t b, int64_t h, int n, int d, float scale, bool causal,
                               bool token_major, hipStream_t stream) {
  switch (d) {
    case 32:
      return launch_bwd_f32_t<32>(q, k, v, o, dout, lse, logf, dq, dk, dv, dlogf, workspace, b, h, n, scale, causal,
                                  token_major, stream);
    case 64:
      return launch_bwd_f32_t<64>(q, k, v, o, dout, lse, logf, dq, dk, dv, dlogf, workspace, b, h, n, scale, causal,
                                  token_major, stream);
    case 128:
      return launch_bwd_f32_t<128>(q, k, v, o, dout, lse, logf, dq, dk, dv, dlogf, workspace, b, h, n, scale, causal,
                                   token_major, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fox
