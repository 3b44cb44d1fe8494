// fox_bwd.hip -- backward pass of FoX attention (bf16 q/k/v/o/dO, fp32 accumulation).
//
// The pages derive no backward pass; this is the chain rule through the forward definition
// (FoX module page, ForgettingAttention.forward):
//   S = scale q k^T + (c_i - c_j) (masked),  P = softmax_rows(S),  O = P v
//   dv = P^T dO;  dP = dO v^T;  dS = P * (dP - D_i) with D_i = dO_i . O_i
//   dq = scale dS k;  dk = scale dS^T q
//   dc_j = rowsum(dS)_j - colsum(dS)_j;  dlog f_t = sum_{i >= t} dc_i
// The row sums of dS vanish in exact arithmetic (sum_j P_ij dP_ij = dO_i . O_i = D_i) but not in
// rounded arithmetic, and dlog f_t = sum_{i>=t} dc_i then adds up the rounding of every row
// i >= t.  With both sums taken over the same bf16-rounded dS, the terms of the block i, j >= t
// cancel and dlog f_t reduces to the cross block (i >= t > j) as it does exactly.  The
// forward's lse and c (its outputs) give P without a second softmax.
//
// Kernels (one call of fox_attn_bwd runs them in this order on the caller's stream):
//  * bwd_pre_kernel: D_i = dO_i . O_i per row, and zeroes the fp32 dq and dc accumulators.
//  * bwd_main_kernel<D, CAUSAL>: one workgroup of 4 waves per (128-key block, batch*head); wave w
//    owns keys 32w..32w+31 of the block.  K and V of the block stay in LDS; 32-query tiles of q
//    and dO stream through LDS.  Per tile, on v_mfma_f32_32x32x16_bf16 with queries as M and
//    keys as N (so every accumulator lane holds one key and 16 queries):
//      S = Q K^T, dP = dO V^T (A = row-major q / dO, B = row-major K / V),
//      P and dS elementwise in registers,
//      dV^T += dO^T P and dK^T += Q^T dS (A = transposed LDS reads of dO / q, B = the bf16 P /
//      dS registers, whose query order the transposed reads follow, as in the forward's P.V),
//      dS^T goes to LDS, and dQ^T = K^T dS^T over the block's 128 keys is added to a global
//      fp32 accumulator with atomics (each query tile is shared by every key block); the same
//      B operands against an all-ones A give the row sums of dS, added to dc with atomics.
//    dK, dV and -colsum(dS) (into dc) are written once per key after the last tile.
//  * bwd_post_kernel: dq = fp32 accumulator rounded to bf16;
//  * the suffix-sum scan (fox_scan.hip): dlog f from dc.
#include <math.h>

#include <algorithm>

#include "fox_device.h"
#include "fox_internal.h"

namespace fox {
namespace {

constexpr int kBK = 128;  // keys per workgroup
constexpr int kBQ = 32;   // queries per tile
constexpr int kBwdThreads = 256;
constexpr float kNegInfB = -INFINITY;

template <int D>
struct alignas(16) BwdLds {
  static constexpr int RS = D + 8;    // row stride of the K / V / q / dO tiles (16-byte pad: no bank conflicts
                                      // for 16-byte row reads)
  static constexpr int QS = kBQ + 8;  // row stride of dS^T [key][query]
  bf16 k[kBK * RS];
  bf16 v[kBK * RS];
  bf16 q[kBQ * RS];
  bf16 dout[kBQ * RS];
  bf16 dst[kBK * QS];
  float arow[kBQ];  // (c_i - lse_i) * log2 e of the tile's queries; -inf past n
  float drow[kBQ];  // D_i of the tile's queries; 0 past n
};

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_b;

// ds_read_b64_tr_b16: within each 16-lane group, output lane j element e is element j%4 of the
// 8 bytes addressed by lane 4e + j/4 of the group.
__device__ __forceinline__ bf16x4 tr16(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_b*)(p));
}

// A operand of an MFMA whose M is a dim block and whose K runs over 16 rows of a row-major
// [row][dim] LDS tile: lane (l32, hi) gets column dim0 + l32 of rows
// {row0 + 4hi .. +3, row0 + 8 + 4hi .. +3}, the row order of the accumulator registers 8u..8u+7.
__device__ __forceinline__ bf16x8 transposed_operand(const bf16* tile, int stride, int row0, int dim0, int lane) {
  const int li = lane & 15, half = (lane >> 4) & 1, hi = lane >> 5;
  const bf16* p = tile + (size_t)(row0 + 4 * hi + (li >> 2)) * stride + dim0 + 16 * half + 4 * (li & 3);
  const bf16x4 lo = tr16(p);
  const bf16x4 up = tr16(p + 8 * stride);
  return __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x8 row_operand(const bf16* tile, int stride, int row, int col) {
  return *reinterpret_cast<const bf16x8*>(tile + (size_t)row * stride + col);
}

// Registers 8u..8u+7 of an accumulator as a bf16 B operand (round to nearest even).
__device__ __forceinline__ bf16x8 acc_operand(const f32x16& a, int u) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16)a[8 * u + e];
  return r;
}

// Cooperative copy of `rows` rows of d bf16 (global row stride d) into an LDS tile of row
// stride RS; rows at or past `valid` are zero-filled.
template <int D>
__device__ __forceinline__ void stage_rows(bf16* lds, const bf16* src, int rows, int valid, int tid) {
  constexpr int CH = D / 8;
  for (int i = tid; i < rows * CH; i += kBwdThreads) {
    const int r = i / CH, ch = i - r * CH;
    bf16x8 x = bf16x8{};
    if (r < valid) x = *reinterpret_cast<const bf16x8*>(src + (size_t)r * D + 8 * ch);
    *reinterpret_cast<bf16x8*>(lds + r * BwdLds<D>::RS + 8 * ch) = x;
  }
}

template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const bf16* __restrict__ o, const bf16* __restrict__ dout,
                                                      float* __restrict__ dvec, float* __restrict__ dq_acc,
                                                      float* __restrict__ dc, int64_t rows) {
  constexpr int G = D / 8;  // lanes per row, 8 elements each
  const int64_t row = (int64_t)blockIdx.x * (kBwdThreads / G) + threadIdx.x / G;
  const int g = threadIdx.x % G;
  float s = 0.0f;
  if (row < rows) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(o + row * D + 8 * g);
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(dout + row * D + 8 * g);
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf((float)a[e], (float)b[e], s);
    float4* z = reinterpret_cast<float4*>(dq_acc + row * D + 8 * g);
    z[0] = float4{0.0f, 0.0f, 0.0f, 0.0f};
    z[1] = float4{0.0f, 0.0f, 0.0f, 0.0f};
  }
#pragma unroll
  for (int off = G / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if (row < rows && g == 0) {
    dvec[row] = s;
    dc[row] = 0.0f;
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads) void bwd_main_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v, const bf16* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ c, const float* __restrict__ dvec,
    float* __restrict__ dq_acc, bf16* __restrict__ dk, bf16* __restrict__ dv, float* __restrict__ dc, int n,
    float scale) {
  using L = BwdLds<D>;
  constexpr int RS = L::RS, QS = L::QS, KK = D / 16, DB = D / 32;
  __shared__ L lds;

  const size_t bh = blockIdx.x;  // heads fastest: the key blocks of one head share its q / dO in L2
  const int kb = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int key0 = kb * kBK;
  const int key = key0 + 32 * wave + l32;  // this lane's key (accumulator column)
  const size_t base = bh * (size_t)n;
  const float scale_log2 = scale * kLog2e;

  stage_rows<D>(lds.k, k + (base + key0) * D, kBK, n - key0, tid);
  stage_rows<D>(lds.v, v + (base + key0) * D, kBK, n - key0, tid);
  // keys past n: +inf here makes every score -inf, so P and dS are 0 for them
  const float bkey = key < n ? c[base + key] * kLog2e : INFINITY;

  f32x16 dkt[DB], dvt[DB];  // dK^T, dV^T: lane = key, 16 dims per 32-dim block
#pragma unroll
  for (int db = 0; db < DB; ++db) dkt[db] = dvt[db] = f32x16{};
  float colsum = 0.0f;

  // The next query tile's q / dO rows, (c - lse) log2 e and D_i are loaded into registers while
  // the current tile computes, and written to LDS at the top of the next iteration.
  constexpr int CH = D / 8, NCH = kBQ * CH;
  constexpr int PF = (NCH + kBwdThreads - 1) / kBwdThreads;
  bf16x8 nq[PF], nd[PF];
  float na = kNegInfB, ndr = 0.0f;
  auto fetch = [&](int q0) {
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int i = tid + j * kBwdThreads, r = i / CH, ch = i - r * CH;
      nq[j] = nd[j] = bf16x8{};
      if ((NCH % kBwdThreads == 0 || i < NCH) && q0 + r < n) {
        nq[j] = *reinterpret_cast<const bf16x8*>(q + (base + q0 + r) * D + 8 * ch);
        nd[j] = *reinterpret_cast<const bf16x8*>(dout + (base + q0 + r) * D + 8 * ch);
      }
    }
    if (tid < kBQ) {
      const int i = q0 + tid;
      na = i < n ? (c[base + i] - lse[base + i]) * kLog2e : kNegInfB;
      ndr = i < n ? dvec[base + i] : 0.0f;
    }
  };

  const int nqt = (n + kBQ - 1) / kBQ;
  const int qt0 = CAUSAL ? key0 / kBQ : 0;  // earlier query tiles see none of these keys
  if (qt0 < nqt) fetch(qt0 * kBQ);
  for (int qt = qt0; qt < nqt; ++qt) {
    const int q0 = qt * kBQ;
    __syncthreads();  // the previous tile's q / dO / dS^T are no longer read
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int i = tid + j * kBwdThreads, r = i / CH, ch = i - r * CH;
      if (NCH % kBwdThreads == 0 || i < NCH) {
        *reinterpret_cast<bf16x8*>(lds.q + r * RS + 8 * ch) = nq[j];
        *reinterpret_cast<bf16x8*>(lds.dout + r * RS + 8 * ch) = nd[j];
      }
    }
    if (tid < kBQ) {
      lds.arow[tid] = na;
      lds.drow[tid] = ndr;
    }
    __syncthreads();
    if (qt + 1 < nqt) fetch(q0 + kBQ);

    // S = Q K^T and dP = dO V^T for this wave's 32 keys
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int col = 16 * kk + 8 * hi;
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_operand(lds.q, RS, l32, col),
                                                  row_operand(lds.k, RS, 32 * wave + l32, col), s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_operand(lds.dout, RS, l32, col),
                                                   row_operand(lds.v, RS, 32 * wave + l32, col), dp, 0, 0, 0);
    }
    // P and dS: register r holds query m = 8(r/4) + 4hi + r%4 of the tile
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 a4 = *reinterpret_cast<const f32x4*>(&lds.arow[8 * g + 4 * hi]);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(&lds.drow[8 * g + 4 * hi]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        float p = exp2_hw(fmaf(s[r], scale_log2, a4[e]) - bkey);
        if (CAUSAL && key > q0 + 8 * g + 4 * hi + e) p = 0.0f;
        // dS as the bf16 value the products and the row sums use
        const float dsv = (float)(bf16)(p * (dp[r] - d4[e]));
        s[r] = p;
        dp[r] = dsv;
        colsum += dsv;
      }
    }
    // dV^T += dO^T P, dK^T += Q^T dS (K of these MFMAs runs over the tile's 32 queries)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const bf16x8 pb = acc_operand(s, u), sb = acc_operand(dp, u);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        dvt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(transposed_operand(lds.dout, RS, 16 * u, 32 * db, lane), pb,
                                                          dvt[db], 0, 0, 0);
        dkt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(transposed_operand(lds.q, RS, 16 * u, 32 * db, lane), sb,
                                                          dkt[db], 0, 0, 0);
      }
    }
    // dS^T to LDS: four runs of 4 consecutive queries per lane, 8 bytes each
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 w4;
#pragma unroll
      for (int e = 0; e < 4; ++e) w4[e] = (bf16)dp[4 * g + e];
      *reinterpret_cast<bf16x4*>(&lds.dst[(32 * wave + l32) * QS + 8 * g + 4 * hi]) = w4;
    }
    __syncthreads();
    // dQ (queries x dims) = dS K over the block's keys; DB output blocks of 32 dims shared by
    // the 4 waves (a wave takes block wave % DB and its share of the 8 key steps)
    {
      constexpr int PER = 4 / DB;  // waves per output block
      constexpr int KS = 8 / PER;  // key steps per wave
      const int db = wave % DB, part = wave / DB;
      f32x16 acc = f32x16{}, rsum = f32x16{};
      const bf16x2 one2 = {(bf16)1.0f, (bf16)1.0f};
      const bf16x8 ones = __builtin_shufflevector(one2, one2, 0, 1, 0, 1, 0, 1, 0, 1);
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        const int ks = part * KS + j;
        const bf16x8 aop = transposed_operand(lds.dst, QS, 16 * ks, 0, lane);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, transposed_operand(lds.k, RS, 16 * ks, 32 * db, lane), acc,
                                                      0, 0, 0);
        if (db == 0) rsum = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, ones, rsum, 0, 0, 0);
      }
      // lane: dim 32db + l32; register r: query q0 + 8(r/4) + 4hi + r%4.  One atomic instruction
      // covers 32 consecutive dims of two queries (two full 128-byte lines).
      float* dst = dq_acc + (base + q0 + 4 * hi) * D + 32 * db + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = 8 * (r >> 2) + (r & 3);
        if (q0 + 4 * hi + m < n) atomicAdd(dst + (size_t)m * D, acc[r] * scale);
      }
      // every lane of rsum holds the row sums of its 16 queries; lane l32 < 16 adds register l32
      if (db == 0) {
        float rs = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) rs = l32 == r ? rsum[r] : rs;
        const int qi = q0 + 8 * (l32 >> 2) + 4 * hi + (l32 & 3);
        if (l32 < 16 && qi < n) atomicAdd(dc + base + qi, rs);
      }
    }
  }

  // dK = scale dK^T, dV = dV^T: lane = key, dims 32db + 8(r/4) + 4hi + r%4 (runs of 4)
  colsum = pair32_sum(colsum);
  if (key < n) {
    bf16* dkr = dk + (base + key) * D;
    bf16* dvr = dv + (base + key) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = (bf16)(dkt[db][4 * g + e] * scale);
          b[e] = (bf16)dvt[db][4 * g + e];
        }
        *reinterpret_cast<bf16x4*>(dkr + 32 * db + 8 * g + 4 * hi) = a;
        *reinterpret_cast<bf16x4*>(dvr + 32 * db + 8 * g + 4 * hi) = b;
      }
    }
    if (hi == 0) atomicAdd(dc + base + key, -colsum);
  }
}

__global__ __launch_bounds__(256) void bwd_post_kernel(const float* __restrict__ dq_acc, bf16* __restrict__ dq,
                                                       int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += (int64_t)gridDim.x * 256)
    dq[i] = (bf16)dq_acc[i];
}

template <int D>
hipError_t launch_bwd_t(const void* q, const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, const float* c, void* dq, void* dk, void* dv, float* dlogf, float* ws,
                        int64_t bh, int n, float scale, bool causal, hipStream_t stream) {
  const int64_t rows = bh * n;
  float* dq_acc = ws;
  float* dvec = dq_acc + rows * D;
  float* dc = dvec + rows;
  constexpr int RPB = kBwdThreads / (D / 8);
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(kBwdThreads), 0, stream,
                     (const bf16*)o, (const bf16*)dout, dvec, dq_acc, dc, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)bh, (unsigned)((n + kBK - 1) / kBK));
  if (causal)
    hipLaunchKernelGGL((bwd_main_kernel<D, true>), grid, dim3(kBwdThreads), 0, stream, (const bf16*)q, (const bf16*)k,
                       (const bf16*)v, (const bf16*)dout, lse, c, (const float*)dvec, dq_acc, (bf16*)dk, (bf16*)dv,
                       dc, n, scale);
  else
    hipLaunchKernelGGL((bwd_main_kernel<D, false>), grid, dim3(kBwdThreads), 0, stream, (const bf16*)q,
                       (const bf16*)k, (const bf16*)v, (const bf16*)dout, lse, c, (const float*)dvec, dq_acc,
                       (bf16*)dk, (bf16*)dv, dc, n, scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t cnt = rows * D;
  const unsigned pg = (unsigned)std::min<int64_t>((cnt + 255) / 256, 65536);
  hipLaunchKernelGGL(bwd_post_kernel, dim3(pg), dim3(256), 0, stream, (const float*)dq_acc, (bf16*)dq, cnt);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_suffix_sum(dc, dlogf, bh, n, stream);
}

}  // namespace

size_t attn_bwd_workspace_bytes(int64_t bh, int n, int d) {
  return (size_t)bh * (size_t)n * ((size_t)d + 2) * sizeof(float);
}

hipError_t launch_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, const float* c, void* dq, void* dk, void* dv, float* dlogf,
                           float* workspace, int64_t bh, int n, int d, float scale, bool causal, hipStream_t stream) {
  switch (d) {
    case 32: return launch_bwd_t<32>(q, k, v, o, dout, lse, c, dq, dk, dv, dlogf, workspace, bh, n, scale, causal, stream);
    case 64: return launch_bwd_t<64>(q, k, v, o, dout, lse, c, dq, dk, dv, dlogf, workspace, bh, n, scale, causal, stream);
    case 128:
      return launch_bwd_t<128>(q, k, v, o, dout, lse, c, dq, dk, dv, dlogf, workspace, bh, n, scale, causal, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fox
