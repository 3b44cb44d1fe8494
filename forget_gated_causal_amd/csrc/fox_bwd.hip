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
constexpr int kRawBufferCfg = 0x00020000;  // dword 3 of a raw (unswizzled, byte-offset) buffer resource
// vector-memory instructions every wave issues between a tile's direct-to-LDS loads and the
// wait for them (from the second tile on): the 16 dQ atomics of the tile before (wave 0 may
// issue one more, which only makes the wait stronger)
constexpr int kAtomicsPerTile = 16;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) void*)p);
}
// Direct-to-LDS buffer loads (lane l's bytes land at LDS byte address m0v + l * size).  Issued
// through inline assembly, so the compiler does not wait for them; the kernel waits itself.
// Raw buffer resource in SGPRs for the assembly below (the same fields the compiler builds for
// __builtin_amdgcn_make_buffer_rsrc).
__device__ __forceinline__ u32x4 sgpr_rsrc(const void* p, uint32_t num_bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  u32x4 r;
  r[0] = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
  r[2] = (uint32_t)__builtin_amdgcn_readfirstlane((int)num_bytes);
  r[3] = (uint32_t)kRawBufferCfg;
  return r;
}
__device__ __forceinline__ void lds_load16(uint32_t m0v, u32x4 rsrc, uint32_t voff) {
  __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   :
                   : "s"(m0v), "v"(voff), "s"(rsrc)
                   : "memory", "m0");
}
__device__ __forceinline__ void lds_load4(uint32_t m0v, u32x4 rsrc, uint32_t voff) {
  __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                   :
                   : "s"(m0v), "v"(voff), "s"(rsrc)
                   : "memory", "m0");
}
// s_waitcnt vmcnt(N), expcnt and lgkmcnt not waited on
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// LDS tiles are row-major with W bf16 per row and no padding; the 16-byte chunk ch of row r
// sits at chunk position ch ^ swz<W>(r).  The LDS serves 16 lanes of a 16-byte read, or 32 lanes
// of an 8-byte read, per cycle from 64 four-byte banks.  The swizzle keeps both access shapes
// used here conflict-free: 16-byte reads of one chunk column over 16 consecutive rows, and the
// transposed 8-byte reads, whose 32 lanes cover 64 contiguous bytes of 4 consecutive rows
// (rows 4m..4m+3).
template <int W>
__device__ __forceinline__ int swz(int r) {
  if constexpr (W >= 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else if constexpr (W == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  else return (r >> 2) & 3;
}
// element offset of (row r, element e) in a swizzled tile of W bf16 per row
template <int W>
__device__ __forceinline__ int sw_off(int r, int e) {
  return r * W + 8 * ((e >> 3) ^ swz<W>(r)) + (e & 7);
}

// K and V rows as register-resident B operands (else read from LDS on every query tile)
template <int D>
constexpr bool kv_in_regs() {
#ifdef FOX_BWD_KVREG_MIN_D
  return D >= FOX_BWD_KVREG_MIN_D;
#else
  return D >= 128;
#endif
}

template <int D>
struct alignas(16) BwdLds {
  bf16 k[kBK * D];  // the block's keys (swizzled rows); read transposed for dQ
  bf16 v[kv_in_regs<D>() ? 8 : kBK * D];
  bf16 q[2][kBQ * D];     // query tiles, double-buffered, filled by direct-to-LDS loads
  bf16 dout[2][kBQ * D];  // dO tiles, likewise
  bf16 dst[2][kBK * kBQ];  // dS^T [key][query], double-buffered (written for tile t, read for it one tile later)
  float rowv[2][2 * kBQ];  // per buffer: a_i = (c_i - lse_i) log2 e of the tile's queries, then D_i
  float rpart[2][4][kBQ];  // per tile parity and wave: partial row sums of dS over its two key steps
};

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_b;

// ds_read_b64_tr_b16: within each 16-lane group, output lane j element e is element j%4 of the
// 8 bytes addressed by lane 4e + j/4 of the group.
__device__ __forceinline__ bf16x4 tr16(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_b*)(p));
}

// Operand of an MFMA whose M (or N) is a block of 32 columns and whose K runs over 16 rows of a
// swizzled row-major [row][column] LDS tile: lane (l32, hi) gets column dim0 + l32 of rows
// {row0 + 4hi .. +3, row0 + 8 + 4hi .. +3}, the row order of the accumulator registers 8u..8u+7.
template <int W>
__device__ __forceinline__ bf16x8 transposed_operand(const bf16* tile, int row0, int dim0, int lane) {
  const int li = lane & 15, half = (lane >> 4) & 1, hi = lane >> 5;
  const int r = row0 + 4 * hi + (li >> 2), e = dim0 + 16 * half + 4 * (li & 3);
  const bf16x4 lo = tr16(tile + sw_off<W>(r, e));
  const bf16x4 up = tr16(tile + sw_off<W>(r + 8, e));
  return __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int W>
__device__ __forceinline__ bf16x8 row_operand(const bf16* tile, int row, int col) {
  return *reinterpret_cast<const bf16x8*>(tile + sw_off<W>(row, col));
}

// Registers 8u..8u+7 of an accumulator as a bf16 B operand (round to nearest even).
__device__ __forceinline__ bf16x8 acc_operand(const f32x16& a, int u) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16)a[8 * u + e];
  return r;
}

// Cooperative copy of `rows` rows of d bf16 (global row stride d) into a swizzled LDS tile;
// rows at or past `valid` are zero-filled.
template <int D>
__device__ __forceinline__ void stage_rows(bf16* lds, const bf16* src, int rows, int valid, int tid) {
  constexpr int CH = D / 8;
  for (int i = tid; i < rows * CH; i += kBwdThreads) {
    const int r = i / CH, ch = i - r * CH;
    bf16x8 x = bf16x8{};
    if (r < valid) x = *reinterpret_cast<const bf16x8*>(src + (size_t)r * D + 8 * ch);
    *reinterpret_cast<bf16x8*>(lds + sw_off<D>(r, 8 * ch)) = x;
  }
}

// Per query row: zero its dq accumulator row and dc entry; per head, the row vector block
// [a_0 .. a_{npad-1} | D_0 .. D_{npad-1}] with a_i = (c_i - lse_i) log2 e and D_i = dO_i . O_i,
// padded past n with a = -inf (no key weight) and D = 0.  Grid: one thread group of D/8 lanes per
// (head, padded row).
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const bf16* __restrict__ o, const bf16* __restrict__ dout,
                                                      const float* __restrict__ lse, const float* __restrict__ c,
                                                      float* __restrict__ rowv, float* __restrict__ dq_acc,
                                                      float* __restrict__ dc, int64_t bh_count, int n, int npad) {
  constexpr int G = D / 8;  // lanes per row, 8 elements each
  const int64_t prow = (int64_t)blockIdx.x * (kBwdThreads / G) + threadIdx.x / G;
  const int g = threadIdx.x % G;
  const int64_t bh = prow / npad;
  const int i = (int)(prow - bh * npad);
  const bool live = bh < bh_count && i < n;
  const int64_t row = bh * n + i;
  float s = 0.0f;
  if (live) {
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
  if (bh < bh_count && g == 0) {
    float* blk = rowv + bh * 2 * npad;
    blk[i] = live ? (c[row] - lse[row]) * kLog2e : kNegInfB;
    blk[npad + i] = live ? s : 0.0f;
    if (live) dc[row] = 0.0f;
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(D <= 64 ? 2 : 1))) void bwd_main_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v, const bf16* __restrict__ dout,
    const float* __restrict__ rowv, float* __restrict__ dq_acc, bf16* __restrict__ dk, bf16* __restrict__ dv,
    const float* __restrict__ c, float* __restrict__ dc, int n, int npad, float scale) {
  using L = BwdLds<D>;
  constexpr int KK = D / 16, DB = D / 32;
  __shared__ L lds;

  const size_t bh = blockIdx.x;  // heads fastest: the key blocks of one head share its q / dO in L2
  const int kb = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int key0 = kb * kBK;
  const int key = key0 + 32 * wave + l32;  // this lane's key (accumulator column)
  const size_t base = bh * (size_t)n;
  const float scale_log2 = scale * kLog2e;

  // Buffer resources over this head's rows: loads past row n return zeros and atomics past it
  // are dropped, so the ragged last query tile needs no branches.
  const u32x4 rq = sgpr_rsrc(q + base * D, (uint32_t)(n * D * 2));
  const u32x4 rdo = sgpr_rsrc(dout + base * D, (uint32_t)(n * D * 2));
  const u32x4 rrow = sgpr_rsrc(rowv + bh * 2 * npad, (uint32_t)(2 * npad * 4));
  const auto rdq = __builtin_amdgcn_make_buffer_rsrc((void*)(dq_acc + base * D), 0, n * D * 4, kRawBufferCfg);
  const auto rdc = __builtin_amdgcn_make_buffer_rsrc((void*)(dc + base), 0, n * 4, kRawBufferCfg);

  stage_rows<D>(lds.k, k + (base + key0) * D, kBK, n - key0, tid);
  if constexpr (!kv_in_regs<D>()) stage_rows<D>(lds.v, v + (base + key0) * D, kBK, n - key0, tid);
  // this lane's key row of K and V as the B operands of S = Q K^T and dP = dO V^T (k-elements
  // 16kk + 8hi .. +7), held in registers for the whole query loop where they fit
  constexpr int KR = kv_in_regs<D>() ? KK : 1;
  bf16x8 kreg[KR], vreg[KR];
#pragma unroll
  for (int kk = 0; kk < KR; ++kk) {
    kreg[kk] = vreg[kk] = bf16x8{};
    if (kv_in_regs<D>() && key < n) {
      kreg[kk] = *reinterpret_cast<const bf16x8*>(k + (base + key) * D + 16 * kk + 8 * hi);
      vreg[kk] = *reinterpret_cast<const bf16x8*>(v + (base + key) * D + 16 * kk + 8 * hi);
    }
  }
  // keys past n: +inf here makes every score -inf, so P and dS are 0 for them
  const float bkey = key < n ? c[base + key] * kLog2e : INFINITY;

  // Direct-to-LDS loads of one query tile: the q and dO tiles are 2 * 32 * D / 8 chunks of 16
  // bytes, IPW wave instructions of 64 chunks per wave; instruction g of the tile fills LDS chunks
  // 64(g % TB) .. +63 of tile g / TB (q, then dO).  LDS chunk P = r * CH + pc holds global chunk
  // (r, pc ^ swz(r)), which realises the swizzled layout with linear LDS writes.  Wave 0 also
  // loads the tile's 32 a_i (lanes 0..31) and 32 D_i (lanes 32..63).
  constexpr int CH = D / 8, TB = kBQ * CH / 64, IPW = 2 * TB / 4;
  static_assert(2 * TB % 4 == 0, "tile instructions per wave");
  uint32_t toff[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int g = wave * IPW + j, P = 64 * (g % TB) + lane, r = P / CH, pc = P % CH;
    toff[j] = (uint32_t)((r * D + 8 * (pc ^ swz<D>(r))) * 2);
  }
  const uint32_t roff = (uint32_t)((hi ? npad : 0) + l32) * 4u;
  auto load_tile = [&](int q0, int buf) {
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int g = wave * IPW + j;
      const bool is_q = g < TB;  // wave-uniform
      const uint32_t m0v = (uint32_t)__builtin_amdgcn_readfirstlane(
          (int)lds_addr(is_q ? &lds.q[buf][64 * 8 * (g % TB)] : &lds.dout[buf][64 * 8 * (g % TB)]));
      lds_load16(m0v, is_q ? rq : rdo, toff[j] + (uint32_t)(q0 * D * 2));
    }
    if (wave == 0)
      lds_load4((uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(&lds.rowv[buf][0])), rrow,
                roff + (uint32_t)q0 * 4u);
  };

  // wave 0: dc[q0 + l] += the four waves' partial row sums of query tile q0 (lanes 0..31)
  auto add_row_sums = [&](int q0, int par) {
    const float t = lds.rpart[par][0][l32] + lds.rpart[par][1][l32] + lds.rpart[par][2][l32] + lds.rpart[par][3][l32];
    if (hi == 0) __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(t, rdc, (q0 + l32) * 4, 0, 0);
  };
  const bf16x2 one2 = {(bf16)1.0f, (bf16)1.0f};
  const bf16x8 ones = __builtin_shufflevector(one2, one2, 0, 1, 0, 1, 0, 1, 0, 1);
  // dQ (queries x dims) = dS K over the block's keys for query tile q0, from dS^T in LDS; DB
  // output blocks of 32 dims shared by the 4 waves (a wave takes block wave % DB and its share of
  // the 8 key steps).  Also this wave's partial row sums of dS, into rpart[par].
  auto dq_tile = [&](int q0, const bf16* dsrc, int par) {
    constexpr int PER = 4 / DB;  // waves per output block
    constexpr int KS = 8 / PER;  // key steps per wave
    const int db = wave % DB, part = wave / DB;
    f32x16 acc = f32x16{}, rsum = f32x16{};
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      const int ks = part * KS + j;
      const bf16x8 aop = transposed_operand<kBQ>(dsrc, 16 * ks, 0, lane);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, transposed_operand<D>(lds.k, 16 * ks, 32 * db, lane), acc, 0, 0,
                                                    0);
    }
    // row sums over key steps 2 wave, 2 wave + 1: an all-ones A against dS as B (N = queries)
    // leaves query l32's partial sum in every register of lane l32
#pragma unroll
    for (int j = 0; j < 2; ++j)
      rsum = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, transposed_operand<kBQ>(dsrc, 16 * (2 * wave + j), 0, lane),
                                                     rsum, 0, 0, 0);
    if (hi == 0) lds.rpart[par][wave][l32] = rsum[0];
    // lane: dim 32db + l32; register r: query q0 + 8(r/4) + 4hi + r%4.  One atomic instruction
    // covers 32 consecutive dims of two queries (two full 128-byte lines).
    const int off = ((q0 + 4 * hi) * D + 32 * db + l32) * 4;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(acc[r] * scale, rdq, off + (8 * (r >> 2) + (r & 3)) * D * 4, 0, 0);
  };

  f32x16 dkt[DB], dvt[DB];  // dK^T, dV^T: lane = key, 16 dims per 32-dim block
#pragma unroll
  for (int db = 0; db < DB; ++db) dkt[db] = dvt[db] = f32x16{};
  float colsum = 0.0f;

  const int nqt = (n + kBQ - 1) / kBQ;
  const int qt0 = CAUSAL ? key0 / kBQ : 0;  // earlier query tiles see none of these keys
  load_tile(qt0 * kBQ, 0);
  wait_vmem<0>();  // K, V and the first tile
  // Iteration t: S, dP, P, dS, dV^T and dK^T of query tile t (dS^T into dst[t & 1]), and dQ of
  // tile t - 1 from dst[(t - 1) & 1]: one barrier per tile, and the dQ atomics of a tile are
  // issued a whole iteration before the loads queued behind them are waited for.
  for (int qt = qt0; qt < nqt; ++qt) {
    const int q0 = qt * kBQ, it = qt - qt0, buf = it & 1;
    // this wave's loads of tile qt were issued before the dQ atomics of tile qt - 2; after the
    // barrier every wave's loads are visible, dS^T of tile qt - 1 is complete, and the reads of
    // tile qt - 1's q / dO buffer and of tile qt - 2's dS^T buffer are done
    if (it == 1)
      wait_vmem<0>();
    else if (it > 1)
      wait_vmem<kAtomicsPerTile>();
    __syncthreads();
    if (qt + 1 < nqt) load_tile(q0 + kBQ, buf ^ 1);
    if (it >= 2 && wave == 0) add_row_sums(q0 - 2 * kBQ, buf);
    if (it >= 1) dq_tile(q0 - kBQ, lds.dst[buf ^ 1], buf ^ 1);
    const bf16* tq = lds.q[buf];
    const bf16* tdo = lds.dout[buf];
    const float* arow = &lds.rowv[buf][0];
    const float* drow = &lds.rowv[buf][kBQ];

    // S = Q K^T and dP = dO V^T for this wave's 32 keys
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int col = 16 * kk + 8 * hi;
      bf16x8 kb, vb;
      if constexpr (kv_in_regs<D>()) {
        kb = kreg[kk];
        vb = vreg[kk];
      } else {
        kb = row_operand<D>(lds.k, 32 * wave + l32, col);
        vb = row_operand<D>(lds.v, 32 * wave + l32, col);
      }
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_operand<D>(tq, l32, col), kb, s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_operand<D>(tdo, l32, col), vb, dp, 0, 0, 0);
    }
    // P and dS: register r holds query m = 8(r/4) + 4hi + r%4 of the tile
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 a4 = *reinterpret_cast<const f32x4*>(&arow[8 * g + 4 * hi]);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(&drow[8 * g + 4 * hi]);
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
        dvt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(transposed_operand<D>(tdo, 16 * u, 32 * db, lane), pb, dvt[db],
                                                          0, 0, 0);
        dkt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(transposed_operand<D>(tq, 16 * u, 32 * db, lane), sb, dkt[db],
                                                          0, 0, 0);
      }
    }
    // dS^T to LDS: four runs of 4 consecutive queries per lane, 8 bytes each
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 w4;
#pragma unroll
      for (int e = 0; e < 4; ++e) w4[e] = (bf16)dp[4 * g + e];
      *reinterpret_cast<bf16x4*>(&lds.dst[buf][sw_off<kBQ>(32 * wave + l32, 8 * g + 4 * hi)]) = w4;
    }
  }
  // the last tile's dQ, and the row sums of the last two tiles
  {
    const int nt = nqt - qt0, lb = (nt - 1) & 1;
    __syncthreads();
    if (nt >= 2 && wave == 0) add_row_sums((nqt - 2) * kBQ, lb ^ 1);
    dq_tile((nqt - 1) * kBQ, lds.dst[lb], lb);
    __syncthreads();
    if (wave == 0) add_row_sums((nqt - 1) * kBQ, lb);
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

int bwd_npad(int n) { return (n + kBQ - 1) / kBQ * kBQ; }

template <int D>
hipError_t launch_bwd_t(const void* q, const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, const float* c, void* dq, void* dk, void* dv, float* dlogf, float* ws,
                        int64_t bh, int n, float scale, bool causal, hipStream_t stream) {
  const int64_t rows = bh * n;
  const int npad = bwd_npad(n);
  // workspace: dq accumulator [bh][n][D], row vectors [bh][2][npad], dc [bh][n] (fp32)
  float* dq_acc = ws;
  float* rowv = dq_acc + rows * D;
  float* dc = rowv + bh * 2 * npad;
  constexpr int RPB = kBwdThreads / (D / 8);
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((bh * npad + RPB - 1) / RPB)), dim3(kBwdThreads), 0, stream,
                     (const bf16*)o, (const bf16*)dout, lse, c, rowv, dq_acc, dc, bh, n, npad);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)bh, (unsigned)((n + kBK - 1) / kBK));
  if (causal)
    hipLaunchKernelGGL((bwd_main_kernel<D, true>), grid, dim3(kBwdThreads), 0, stream, (const bf16*)q, (const bf16*)k,
                       (const bf16*)v, (const bf16*)dout, (const float*)rowv, dq_acc, (bf16*)dk, (bf16*)dv, c, dc, n,
                       npad, scale);
  else
    hipLaunchKernelGGL((bwd_main_kernel<D, false>), grid, dim3(kBwdThreads), 0, stream, (const bf16*)q,
                       (const bf16*)k, (const bf16*)v, (const bf16*)dout, (const float*)rowv, dq_acc, (bf16*)dk,
                       (bf16*)dv, c, dc, n, npad, scale);
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
  return (size_t)bh * ((size_t)n * ((size_t)d + 1) + 2 * (size_t)bwd_npad(n)) * sizeof(float);
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
