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
// i >= t.  With both sums taken over the same dS values, the terms of the block i, j >= t cancel
// and dlog f_t reduces to the cross blocks (i >= t > j, and i < t <= j without the mask) as it
// does exactly.  With the mask the sums use the bf16 dS the MFMAs use (the one cross block is
// short: its rows see keys before t only within their window); without it the two cross blocks
// can be far larger than dlog f_t, and the sums use the fp32 dS before rounding (those kernels
// then need more registers than two waves per SIMD allow, and run one).  The forward's lse
// gives P without a second softmax (rescaled to unit row sums without the mask: the D pass).
//
// Gate bias.  The prefix sums c grow with the sequence (|c| ~ 10^5 at a million tokens), so fp32
// values of c_i and c_j carry errors far larger than the bias c_i - c_j of nearby pairs.  The
// gate rows (gate_rows_block below) split c at 32-position blocks instead: C_b in fp64 per block,
// and the in-block part cq_i = c_i - C_b(i) in the row vectors.  A score's bias is then
// (cq_i - cq_j) + (C_b(i) - C_b(j)); the block difference is one fp64 subtraction per (tile,
// wave), and every fp32 rounding is of a term bounded by 32 |log f| rather than by |c|.  (With
// strong gates that bound still exceeds the bias of a weighted pair -- 10^-5 relative in P at
// |log f| = 4.5, well inside bf16 bounds; the fp32 backward forms each bias in fp64 instead.)
//
// D_i.  dO_i . O_i uses the forward's O, rounded to bf16.  Without the mask, dlog f_t is the
// difference of two cross-block sums that can be far larger than it, and the rounding of O
// (through D_i, in every dS of row i) no longer cancels: the unmasked mode therefore first runs
// the query-stationary part in a D pass, D_i = sum_j P_ij dP_ij in fp32 from the same P and dP.
//
// Two parts split the work so that every output has one writer (no atomics, and the results are
// the same from run to run).  Large grids run them as two kernels, small grids as one
// (bwd_main_kernel, which alternates key and query blocks); both use an explicit slot schedule
// that overlaps the next tile's score MFMAs with the current tile's elementwise work:
//  * bwd_kv_block / bwd_kv_kernel<D, CAUSAL>: key-stationary.  One workgroup of 4 waves per (128-key block,
//    head); wave w owns keys 32w..32w+31.  32-query tiles of q and dO stream through LDS.  Per
//    tile, on v_mfma_f32_32x32x16_bf16 with queries as M and keys as N (every accumulator lane
//    holds one key and 16 queries): S = Q K^T, dP = dO V^T; P and dS in registers; dV^T += dO^T P
//    and dK^T += Q^T dS (A = transposed LDS reads of dO / q, B = the bf16 P / dS registers).
//    Writes dk, dv and the column sums of dS.
//  * bwd_dq_block / bwd_dq_kernel<D, CAUSAL>: query-stationary.  One workgroup of 4 waves per (128-query block,
//    head); wave w owns queries 32w..32w+31, whose q and dO rows stay in registers.  64-key tiles
//    of K, V and c stream through LDS.  Per 32-key block, with keys as M and queries as N (every
//    lane holds one query): S^T = K Q^T, dP^T = V dO^T, P^T and dS^T in registers, and
//    dQ += dS K with the dS^T accumulators as the A operand (queries as M) and K read transposed.
//    Writes dq and the row sums of dS.
//  * before them: the gate rows (gate_rows_block: the padded row vectors and the fp64 block sums
//    C_b that both parts load) and D_i = dO_i . O_i in one launch (bwd_rows_kernel) with the
//    mask; without it the gate rows, then bwd_dpass_kernel (D_i = sum_j P_ij dP_ij in fp32, and
//    the row terms rescaled so that each row of P sums to 1 in fp32).
//    After them the reversed prefix scan (fox_scan.hip): dlog f from row sums - column sums.
//  * staged dS (fox_attn_bwd_staged; causal, d = 128): the key-stationary kernel also
//    stores the bf16 dS it packed for its own dK^T MFMAs into the workspace, and
//    bwd_dq_staged_kernel contracts dQ = dS K and the row sums from it in place of bwd_dq_kernel,
//    which would form S and dP a second time (about n^2 bytes of workspace per head instead).
// Tensors are head-major [B,H,N,d] or token-major [B,N,H,d] (BwdLayout: row strides d or H d,
// gate-vector strides 1 or H); the workspace is head-major either way.
#include <math.h>

#include <type_traits>

#include "fox_device.h"
#include "fox_internal.h"

namespace fox {
namespace {

constexpr int kBK = 128;  // keys per workgroup of the key-stationary kernel
constexpr int kBQ = 32;   // queries per tile of the key-stationary kernel
constexpr int kQB = 128;  // queries per workgroup of the query-stationary kernel
constexpr int kKT = 64;   // keys per tile of the query-stationary kernel
constexpr int kBwdThreads = 256;
constexpr int kPad = 64;  // per-head row vectors are padded to a multiple of this
constexpr int64_t kFuseMaxBlocks = 1024;  // grids up to this many blocks run both parts in one launch

// Staged dS (fox_attn_bwd_staged): per head, key block kb holds the query tiles 4 kb .. nqt - 1
// (those at or below its diagonal), each a [128 keys][32 queries] bf16 tile; the blocks follow
// one another, so block kb starts at tile kb nqt - 2 kb (kb - 1).
__host__ __device__ __forceinline__ int64_t staged_tile0(int kb, int nqt) {
  return (int64_t)kb * nqt - 2 * (int64_t)kb * (kb - 1);
}
__host__ __device__ __forceinline__ int64_t staged_tiles(int n) {
  const int nqt = (n + kBQ - 1) / kBQ, nkb = (n + kBK - 1) / kBK;
  return staged_tile0(nkb, nqt);
}
constexpr float kNegInfB = -INFINITY;
constexpr int kRawBufferCfg = 0x00020000;  // dword 3 of a raw (unswizzled, byte-offset) buffer resource

// Where a head's rows live: q, k, v, o, dO and the gradients share (bs, hs, rs); lse, c and dlog f
// share (gbs, ghs, gs).  Head-major [B,H,N,d]: rs = d; token-major [B,N,H,d]: rs = H d.
struct BwdLayout {
  int64_t bs, hs;    // tensors: batch and head strides (elements)
  int rs;            // tensors: row (token) stride
  int64_t gbs, ghs;  // vectors: batch and head strides
  int gs;            // vectors: row stride
  int nh;            // heads per batch entry
  __device__ __forceinline__ int64_t tbase(int bh) const { return (int64_t)(bh / nh) * bs + (bh % nh) * hs; }
  __device__ __forceinline__ int64_t gbase(int bh) const { return (int64_t)(bh / nh) * gbs + (bh % nh) * ghs; }
};

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) void*)p);
}
// Raw buffer resource in SGPRs for the direct-to-LDS loads below: loads at or past num_bytes
// return zeros.
__device__ __forceinline__ u32x4 sgpr_rsrc(const void* p, uint32_t num_bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  u32x4 r;
  r[0] = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
  r[2] = (uint32_t)__builtin_amdgcn_readfirstlane((int)num_bytes);
  r[3] = (uint32_t)kRawBufferCfg;
  return r;
}
// Direct-to-LDS buffer loads (lane l's bytes land at LDS byte address m0v + l * size).  Issued
// through inline assembly, so the compiler does not wait for them; the kernel waits itself.  M0
// is an input operand the compiler writes before each load; the s_nop is the wait state an M0
// write needs before an LDS-DMA instruction reads it.
__device__ __forceinline__ void lds_load16(uint32_t m0v, u32x4 rsrc, uint32_t voff) {
  __asm__ volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                   :
                   : "v"(voff), "s"(rsrc), "{m0}"(m0v)
                   : "memory");
}
// ... with the streaming hint, for data read once (the staged dS)
__device__ __forceinline__ void lds_load16_nt(uint32_t m0v, u32x4 rsrc, uint32_t voff) {
  __asm__ volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
                   :
                   : "v"(voff), "s"(rsrc), "{m0}"(m0v)
                   : "memory");
}
__device__ __forceinline__ void lds_load4(uint32_t m0v, u32x4 rsrc, uint32_t voff) {
  __asm__ volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
                   :
                   : "v"(voff), "s"(rsrc), "{m0}"(m0v)
                   : "memory");
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

// K and V rows as register-resident B operands of the key-stationary kernel (else read from
// LDS on every query tile)
template <int D>
constexpr bool kv_in_regs() {
  return D >= 128;
}

template <int D>
struct alignas(16) KvLds {
  bf16 k[kv_in_regs<D>() ? 8 : kBK * D];  // the block's keys and values (swizzled rows)
  bf16 v[kv_in_regs<D>() ? 8 : kBK * D];
  bf16 q[3][kBQ * D];      // query tiles, three buffers, filled by direct-to-LDS loads
  bf16 dout[3][kBQ * D];   // dO tiles, likewise
  float rowv[3][2 * kBQ];  // per buffer: a_i = (c_i - lse_i) log2 e of the tile's queries, then D_i
};

template <int D>
struct alignas(16) DqLds {
  bf16 k[3][kKT * D];  // key tiles, three buffers, filled by direct-to-LDS loads
  bf16 v[3][kKT * D];  // value tiles, likewise
  float cl[3][kKT];    // c_j log2 e of the tile's keys (+inf past n)
};

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_b;

// ds_read_b64_tr_b16: within each 16-lane group, output lane j element e is element j%4 of the
// 8 bytes addressed by lane 4e + j/4 of the group.
__device__ __forceinline__ bf16x4 tr16(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_b*)(p));
}

// Accumulating MFMAs of the d = 128 kernels (one wave per SIMD, 512 registers): dK^T and dV^T
// (key side) and dQ (query side) stay in AGPRs, written only by these inline-assembly MFMAs, while
// the score MFMAs (builtins; this file is compiled with the MFMA VGPR form forced) write VGPRs
// that the VALU reads directly, with no AGPR-to-VGPR copies.  The compiler does not see an MFMA
// here: the _nop form keeps the 2 wait states an XDL MFMA needs after a VALU write of its A or
// B operand (first use of each freshly packed P or dS), and agpr_fence the 11 an XDL result
// needs before the VALU reads it (16 here; the AGPRs are operands, so no access moves across).
__device__ __forceinline__ void mfma_acc(f32x16& c, const bf16x8& a, const bf16x8& b) {
  __asm__ volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_acc_nop(f32x16& c, const bf16x8& a, const bf16x8& b) {
  __asm__ volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
template <int N>
__device__ __forceinline__ void agpr_fence(f32x16 (&c)[N]) {
  static_assert(N == 4, "d = 128 accumulators");
  __asm__ volatile("s_nop 15" : "+a"(c[0]), "+a"(c[1]), "+a"(c[2]), "+a"(c[3]));
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

// Sum of the 16 registers of an accumulator (pairwise).
__device__ __forceinline__ float tree_sum16(const f32x16& a) {
  float t[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) t[e] = a[e] + a[e + 8];
#pragma unroll
  for (int e = 0; e < 4; ++e) t[e] += t[e + 4];
  return (t[0] + t[2]) + (t[1] + t[3]);
}

// Registers 8u..8u+7 of an accumulator as a bf16 B operand (round to nearest even).
__device__ __forceinline__ bf16x8 acc_operand(const f32x16& a, int u) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16)a[8 * u + e];
  return r;
}

// Cooperative copy of `rows` rows of d bf16 (global row stride rs) into a swizzled LDS tile;
// rows at or past `valid` are zero-filled.
template <int D>
__device__ __forceinline__ void stage_rows(bf16* lds, const bf16* src, int rows, int valid, int rs, int tid) {
  constexpr int CH = D / 8;
  for (int i = tid; i < rows * CH; i += kBwdThreads) {
    const int r = i / CH, ch = i - r * CH;
    bf16x8 x = bf16x8{};
    if (r < valid) x = *reinterpret_cast<const bf16x8*>(src + (size_t)r * rs + 8 * ch);
    *reinterpret_cast<bf16x8*>(lds + sw_off<D>(r, 8 * ch)) = x;
  }
}

// The backward's gate terms of one (batch, head) row.  The prefix sums are split at blocks of
// kGateBlock positions: C_b = sum_{t < 32b} log f_t (fp64, one per block) and the in-block part
// cq_i = sum_{32b(i) <= t <= i} log f_t, so that c_i - c_j = (cq_i - cq_j) + (C_b(i) - C_b(j)).
// Every term the backward kernels round to fp32 is then bounded by 32 |log f|, not by |c| (which
// grows with the sequence).  Written into the head's row-vector block
// [a | D | cl] of 3 * npad floats: a_i = (cq_i - lse_i) log2 e, cl_i = cq_i log2 e, and D_i = 0
// past n (a = -inf, cl = +inf there, so padded rows and keys carry no weight); C_b for the ncb
// blocks into cb.  One 256-thread workgroup per row, chunks of 1024 positions, each thread 4 of them, fp64 scan
// (a wave DPP scan and a 4-entry LDS scan per chunk, a carry between chunks).
constexpr int kGateBlock = 32;
struct GateRowsIn {  // logf / lse of row r: (r / nh) gbs + (r % nh) ghs + t gs
  int nh;
  int64_t gbs, ghs;
  int gs;
};
GateRowsIn gate_rows_in(int nh, int n, bool token_major) {
  return token_major ? GateRowsIn{nh, (int64_t)n * nh, 1, nh} : GateRowsIn{1, (int64_t)n, 0, 1};
}
constexpr int kScanThreads = 256;
constexpr int kScanPerThread = 4;
constexpr int kScanChunk = kScanThreads * kScanPerThread;
__device__ __forceinline__ void gate_rows_block(const float* __restrict__ logf, const float* __restrict__ lse,
                                                float* __restrict__ rowv, double* __restrict__ cb, int n, int npad,
                                                int ncb, const GateRowsIn& gi, int64_t row) {
  static_assert(kGateBlock % kScanPerThread == 0 && 64 % (kGateBlock / kScanPerThread) == 0, "block lanes");
  constexpr int LPB = kGateBlock / kScanPerThread;  // lanes per block
  __shared__ double wave_tot[2][kScanThreads / 64];
  const int64_t g0 = (row / gi.nh) * gi.gbs + (row % gi.nh) * gi.ghs;
  float* blk = rowv + row * 3 * (int64_t)npad;
  double* cbr = cb + row * (int64_t)ncb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int span = ncb * kGateBlock;  // >= npad
  double carry = 0.0;
  // A chunk's log f and lse are loaded one chunk ahead, so the loads of the next chunk are in
  // flight while this one is scanned and written.
  float lfv[kScanPerThread], lsv[kScanPerThread];
  auto load_chunk = [&](int base, float (&lf)[kScanPerThread], float (&ls)[kScanPerThread]) {
#pragma unroll
    for (int e = 0; e < kScanPerThread; ++e) {
      const int i = base + tid * kScanPerThread + e;
      lf[e] = i < n ? logf[g0 + (int64_t)i * gi.gs] : 0.0f;
      ls[e] = i < n ? lse[g0 + (int64_t)i * gi.gs] : 0.0f;
    }
  };
  load_chunk(0, lfv, lsv);
  for (int base = 0, it = 0; base < span; base += kScanChunk, ++it) {
    const int i0 = base + tid * kScanPerThread;
    float nlf[kScanPerThread] = {}, nls[kScanPerThread] = {};
    if (base + kScanChunk < span) load_chunk(base + kScanChunk, nlf, nls);
    double x[kScanPerThread];
#pragma unroll
    for (int e = 0; e < kScanPerThread; ++e) x[e] = (double)lfv[e];
#pragma unroll
    for (int e = 1; e < kScanPerThread; ++e) x[e] += x[e - 1];
    const double t = wave_incl_scan(x[kScanPerThread - 1]);
    const double excl = wave_shr1(t);
    if (lane == 63) wave_tot[it & 1][wave] = t;
    __syncthreads();
    double before = carry, chunk = 0.0;
#pragma unroll
    for (int w = 0; w < kScanThreads / 64; ++w) {
      if (w < wave) before += wave_tot[it & 1][w];
      chunk += wave_tot[it & 1][w];
    }
    const double pre = before + excl;  // sum of log f before position i0
    // C_b: the prefix before the block's first position, held by the block's first lane
    const int src = lane & ~(LPB - 1);
    const u32x2 pw = __builtin_bit_cast(u32x2, pre);
    u32x2 cw;
    cw[0] = (uint32_t)__shfl((int)pw[0], src);
    cw[1] = (uint32_t)__shfl((int)pw[1], src);
    const double cblk = __builtin_bit_cast(double, cw);
#pragma unroll
    for (int e = 0; e < kScanPerThread; ++e) {
      const int i = i0 + e;
      if (i < npad) {
        const double cq = (pre + x[e]) - cblk;
        const bool live = i < n;
        blk[i] = live ? (float)((cq - (double)lsv[e]) * kLog2ed) : -INFINITY;
        blk[2 * npad + i] = live ? (float)(cq * kLog2ed) : INFINITY;
        if (!live) blk[npad + i] = 0.0f;
      }
    }
    if ((lane & (LPB - 1)) == 0 && i0 < span) cbr[i0 / kGateBlock] = cblk;
    carry += chunk;
#pragma unroll
    for (int e = 0; e < kScanPerThread; ++e) {
      lfv[e] = nlf[e];
      lsv[e] = nls[e];
    }
  }
}

__global__ __launch_bounds__(kScanThreads) void bwd_gate_rows_kernel(const float* __restrict__ logf,
                                                                     const float* __restrict__ lse,
                                                                     float* __restrict__ rowv, double* __restrict__ cb,
                                                                     int n, int npad, int ncb, GateRowsIn gi) {
  gate_rows_block(logf, lse, rowv, cb, n, npad, ncb, gi, blockIdx.x);
}

// D_i = dO_i . O_i into the D slot of each head's row-vector block [a | D | cl] (the gate-rows
// kernel writes a, cl and the padding).  One group of D/8 lanes per (head, padded row).
template <int D>
__device__ __forceinline__ void pre_block(const bf16* __restrict__ o, const bf16* __restrict__ dout,
                                          float* __restrict__ rowv, int64_t bh_count, int n, int npad,
                                          const BwdLayout& lay, int64_t blk) {
  constexpr int G = D / 8;  // lanes per row, 8 elements each
  const int64_t prow = blk * (kBwdThreads / G) + threadIdx.x / G;
  const int g = threadIdx.x % G;
  const int64_t bh = prow / npad;
  const int i = (int)(prow - bh * npad);
  const bool live = bh < bh_count && i < n;
  const int64_t trow = live ? lay.tbase((int)bh) + (int64_t)i * lay.rs : 0;
  float s = 0.0f;
  if (live) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(o + trow + 8 * g);
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(dout + trow + 8 * g);
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf((float)a[e], (float)b[e], s);
  }
#pragma unroll
  for (int off = G / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if (live && g == 0) rowv[bh * 3 * npad + npad + i] = s;
}

// With the mask, one launch runs both: workgroups below `rows` build the gate terms of one head's
// row (gate_rows_block), the rest take D_i for kBwdThreads / (D / 8) padded rows each.  The two
// write disjoint parts of the row vectors.
template <int D>
__global__ __launch_bounds__(256) void bwd_rows_kernel(const float* __restrict__ logf, const float* __restrict__ lse,
                                                       const bf16* __restrict__ o, const bf16* __restrict__ dout,
                                                       float* __restrict__ rowv, double* __restrict__ cb,
                                                       int64_t rows, int n, int npad, int ncb, GateRowsIn gi,
                                                       BwdLayout lay) {
  static_assert(kScanThreads == kBwdThreads, "one block size for both parts");
  if ((int64_t)blockIdx.x < rows) gate_rows_block(logf, lse, rowv, cb, n, npad, ncb, gi, blockIdx.x);
  else pre_block<D>(o, dout, rowv, rows, n, npad, lay, (int64_t)blockIdx.x - rows);
}

// Direct-to-LDS loads of a tile of ROWS rows of D bf16 (global rows from `row0` of the head) into
// a swizzled LDS tile: 64 chunks of 16 bytes per wave instruction; LDS chunk P = r * CH + pc holds
// global chunk (r, pc ^ swz(r)), which realises the swizzle with linear LDS writes.  The NI =
// ROWS * CH / 64 instructions are spread over the 4 waves (instruction g = wave * IPW + j; with
// fewer than 4, waves 0 .. NI-1 issue one each); toff holds a lane's byte offsets.
template <int D, int ROWS>
struct TileLoader {
  static constexpr int CH = D / 8, NI = ROWS * CH / 64, IPW = NI >= 4 ? NI / 4 : 1;
  static_assert(NI >= 1 && (NI < 4 || NI % 4 == 0), "tile instructions per wave");
  uint32_t toff[IPW];
  int rs;  // global row stride (elements)
  __device__ __forceinline__ TileLoader(int wave, int lane, int rs_) : rs(rs_) {
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int P = 64 * ((wave * IPW + j) % NI) + lane, r = P / CH, pc = P % CH;
      toff[j] = (uint32_t)((r * rs + 8 * (pc ^ swz<D>(r))) * 2);
    }
  }
  __device__ __forceinline__ void load(bf16* tile, u32x4 rsrc, int row0, int wave) const {
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int g = wave * IPW + j;  // wave-uniform
      if (NI >= 4 || g < NI) {
        const uint32_t m0v = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(tile + 64 * 8 * g));
        lds_load16(m0v, rsrc, toff[j] + (uint32_t)row0 * (uint32_t)(rs * 2));
      }
    }
  }
};

// Key-stationary part (dK, dV, column sums of dS) for key block kb of head bh.  STAGE: also write
// the bf16 dS of every query tile to ds_stage (the block's first staged tile; see bwd_dq_staged_kernel).
template <int D, bool CAUSAL, bool STAGE = false>
__device__ __forceinline__ void bwd_kv_block(KvLds<D>& lds, size_t bh, int kb, const bf16* __restrict__ q,
                                             const bf16* __restrict__ k, const bf16* __restrict__ v,
                                             const bf16* __restrict__ dout, const float* __restrict__ rowv,
                                             const double* __restrict__ cb, bf16* __restrict__ dk,
                                             bf16* __restrict__ dv, float* __restrict__ colsum_out, int n, int npad,
                                             int ncb, float scale, const BwdLayout& lay,
                                             bf16* __restrict__ ds_stage = nullptr) {
  constexpr int KK = D / 16, DB = D / 32;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int key0 = kb * kBK;
  const int key = key0 + 32 * wave + l32;  // this lane's key (accumulator column)
  const size_t base = bh * (size_t)n;  // this head's rows of the column-sum workspace
  const int64_t tb = lay.tbase((int)bh);
  const int rs = lay.rs;
  const float scale_log2 = scale * kLog2e;
  const float* blk = rowv + bh * 3 * npad;

  // buffer resources over this head's rows: loads past row n return zeros
  const uint32_t span = (uint32_t)(((int64_t)(n - 1) * rs + D) * 2);
  const u32x4 rq = sgpr_rsrc(q + tb, span);
  const u32x4 rdo = sgpr_rsrc(dout + tb, span);
  const u32x4 rrow = sgpr_rsrc(blk, (uint32_t)(2 * npad * 4));

  if constexpr (!kv_in_regs<D>()) {
    stage_rows<D>(lds.k, k + tb + (int64_t)key0 * rs, kBK, n - key0, rs, tid);
    stage_rows<D>(lds.v, v + tb + (int64_t)key0 * rs, kBK, n - key0, rs, tid);
  }
  // this lane's key row of K and V as the B operands of S = Q K^T and dP = dO V^T (k-elements
  // 16kk + 8hi .. +7), held in registers for the whole query loop where they fit
  constexpr int KR = kv_in_regs<D>() ? KK : 1;
  bf16x8 kreg[KR], vreg[KR];
#pragma unroll
  for (int kk = 0; kk < KR; ++kk) {
    kreg[kk] = vreg[kk] = bf16x8{};
    if (kv_in_regs<D>() && key < n) {
      kreg[kk] = *reinterpret_cast<const bf16x8*>(k + tb + (int64_t)key * rs + 16 * kk + 8 * hi);
      vreg[kk] = *reinterpret_cast<const bf16x8*>(v + tb + (int64_t)key * rs + 16 * kk + 8 * hi);
    }
  }
  // cq_j log2 e (+inf past n: every score of the key is then -inf, so P and dS are 0), and the
  // start C of the wave's 32-key block; each query tile adds its own block difference
  const float bkey = key < n ? blk[2 * npad + key] : INFINITY;
  const double* cbh = cb + bh * (size_t)ncb;
  const double ckey = cbh[(key0 >> 5) + wave];

  // q and dO tiles (and the tile's 32 a_i, lanes 0..31 of wave 0, and 32 D_i, lanes 32..63)
  const TileLoader<D, kBQ> tl(wave, lane, rs);
  const uint32_t roff = (uint32_t)((hi ? npad : 0) + l32) * 4u;
  auto load_tile = [&](int q0, int buf) {
    tl.load(lds.q[buf], rq, q0, wave);
    tl.load(lds.dout[buf], rdo, q0, wave);
    if (wave == 0)
      lds_load4((uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(&lds.rowv[buf][0])), rrow,
                roff + (uint32_t)q0 * 4u);
  };

  f32x16 dkt[DB], dvt[DB];  // dK^T, dV^T: lane = key, 16 dims per 32-dim block
#pragma unroll
  for (int db = 0; db < DB; ++db) dkt[db] = dvt[db] = f32x16{};
  float colsum = 0.0f;

  // S = Q K^T and dP = dO V^T of one query tile for this wave's 32 keys
  auto scores = [&](int buf, f32x16& s, f32x16& dp) {
    const bf16* tq = lds.q[buf];
    const bf16* tdo = lds.dout[buf];
    s = dp = f32x16{};
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
  };

  // Software pipeline over the query tiles: step t issues the score MFMAs of tile t + 1 and does
  // the elementwise work and the dV^T / dK^T MFMAs of tile t.  Three LDS buffers: tile t (read
  // transposed), t + 1 (scores), t + 2 (loading).  The schedule is explicit, as in the forward:
  // each slot holds one MFMA and a share of the VALU work that does not depend on it, with the
  // LDS operands read a few slots ahead; sched_barrier keeps the compiler from regrouping slots.
  constexpr int NQ = 2 * KK;   // score MFMAs per tile (S and dP alternate)
  constexpr int EQ = 16 / NQ;  // accumulator elements of the previous tile per score slot
  constexpr int PFQ = NQ >= 8 ? 4 : NQ;  // score operands in flight
  constexpr int NP = 4 * DB;   // dV^T / dK^T MFMAs per tile
  constexpr int PFP = NP >= 8 ? 4 : NP;  // their operands in flight
  static_assert(16 % NQ == 0, "elements per slot");
  const int nqt = (n + kBQ - 1) / kBQ;
  const int qt0 = CAUSAL ? key0 / kBQ : 0;  // earlier query tiles see none of these keys
  const int nt = nqt - qt0;

  const bf16x2 one2 = {(bf16)1.0f, (bf16)1.0f};
  float colsum1 = 0.0f;
  double cq_t = cbh[qt0];  // block start of the query tile being processed (32 queries = one block)
  // One step.  HN: there is a next tile; MASK: the tile may hold keys past its queries (causal);
  // BC: the tile's LDS buffer when known at compile time (t % 3), else -1.
  auto step = [&](auto hn, auto mk, auto bc, int t, f32x16& s, f32x16& dp) {
    constexpr bool HN = decltype(hn)::value, MASK = CAUSAL && decltype(mk)::value;
    constexpr int BC = decltype(bc)::value;
    const int q0 = (qt0 + t) * kBQ;
    const int buf = BC >= 0 ? BC : t % 3, nb = BC >= 0 ? (BC + 1) % 3 : (t + 1) % 3;
    if constexpr (HN) {
      // this wave's loads of tile t + 1 are the only vector-memory instructions in flight (with
      // STAGE, besides the 2 stores of tile t - 1's dS issued after them); after the barrier every
      // wave's loads are visible and tile t - 1's buffer is no longer read
      if (STAGE && t > 0)
        wait_vmem<2>();
      else
        wait_vmem<0>();
      __syncthreads();
      if (t + 2 < nt) load_tile(q0 + 2 * kBQ, BC >= 0 ? (BC + 2) % 3 : (t + 2) % 3);
    }
    const bf16* tq = lds.q[buf];
    const bf16* tdo = lds.dout[buf];
    // the key's bias term with this tile's block difference: c_i - c_j = a-part + (C_q - C_k) - cq_j
    const float bkt = bkey - (float)((cq_t - ckey) * kLog2ed);
    if constexpr (HN) cq_t = cbh[qt0 + t + 1];
    const float* arow = &lds.rowv[buf][0];
    const float* drow = &lds.rowv[buf][kBQ];
    // score operands of tile t + 1: slot i is S (i even) or dP (i odd) for k-step i / 2
    auto qread = [&](int i) -> bf16x8 {
      return row_operand<D>(i & 1 ? lds.dout[nb] : lds.q[nb], l32, 16 * (i >> 1) + 8 * hi);
    };
    auto kvread = [&](int i) -> bf16x8 {
      if constexpr (kv_in_regs<D>()) return i & 1 ? vreg[i >> 1] : kreg[i >> 1];
      else return row_operand<D>(i & 1 ? lds.v : lds.k, 32 * wave + l32, 16 * (i >> 1) + 8 * hi);
    };
    bf16x8 aop[NQ], bop[NQ];
    f32x4 a4[4], d4[4];
    f32x16 s2 = f32x16{}, dp2 = f32x16{};
    a4[0] = *reinterpret_cast<const f32x4*>(&arow[4 * hi]);
    d4[0] = *reinterpret_cast<const f32x4*>(&drow[4 * hi]);
    if constexpr (HN) {
#pragma unroll
      for (int i = 0; i < PFQ; ++i) {
        aop[i] = qread(i);
        bop[i] = kvread(i);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      // the row vectors of query group g, two slots before their first use
#pragma unroll
      for (int g = 1; g < 4; ++g) {
        if (i == (4 * g / EQ >= 2 ? 4 * g / EQ - 2 : 0)) {
          a4[g] = *reinterpret_cast<const f32x4*>(&arow[8 * g + 4 * hi]);
          d4[g] = *reinterpret_cast<const f32x4*>(&drow[8 * g + 4 * hi]);
        }
      }
      // P and dS of tile t (fp32; rounded to bf16 once, as MFMA operands): register r holds
      // query m = 8(r/4) + 4hi + r%4
#pragma unroll
      for (int r = i * EQ; r < (i + 1) * EQ; ++r) {
        const int g = r >> 2, e = r & 3;
        float p = exp2_hw(fmaf(s[r], scale_log2, a4[g][e]) - bkt);
        if (MASK && key > q0 + 8 * g + 4 * hi + e) p = 0.0f;
        s[r] = p;
        dp[r] = p * (dp[r] - d4[g][e]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (HN) {
        if (i & 1) dp2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[i], bop[i], dp2, 0, 0, 0);
        else s2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[i], bop[i], s2, 0, 0, 0);
        if (i + PFQ < NQ) {
          aop[i + PFQ] = qread(i + PFQ);
          bop[i + PFQ] = kvread(i + PFQ);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // dV^T += dO^T P, dK^T += Q^T dS (K of these MFMAs runs over the tile's 32 queries); slot j:
    // query half u = j / (2 DB), dim block db, dV (even) or dK (odd).  The column sums of dS are
    // taken over the fp32 values without the mask, over the bf16 values the MFMAs use with it.
    if constexpr (!CAUSAL) colsum += tree_sum16(dp);
    const bf16x8 pb[2] = {acc_operand(s, 0), acc_operand(s, 1)};
    const bf16x8 sb[2] = {acc_operand(dp, 0), acc_operand(dp, 1)};
    if constexpr (STAGE) {
      // tile t of dS in two halves u of [128 keys][2 lane halves] x 8 bf16: sb[u] of this lane
      // (queries 16u + 4hi + 0..3 and 16u + 8 + 4hi + 0..3 of its key), so that each store
      // instruction writes 1 KiB in one piece; streaming stores, read once by the dQ kernel
      bf16* tile = ds_stage + (size_t)t * (kBK * kBQ) + (32 * wave + l32) * 16 + 8 * hi;
#pragma unroll
      for (int u = 0; u < 2; ++u)
        __builtin_nontemporal_store(sb[u], reinterpret_cast<bf16x8*>(tile + u * (kBK * 16)));
    }
    if constexpr (CAUSAL) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const bf16x2 pr = {sb[u][2 * w], sb[u][2 * w + 1]};
          if (w & 1) colsum1 = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, colsum1, false);
          else colsum = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, colsum, false);
        }
      }
    }
    auto tread = [&](int j) -> bf16x8 {
      const int u = j / (2 * DB), db = (j >> 1) % DB;
      return transposed_operand<D>(j & 1 ? tq : tdo, 16 * u, 32 * db, lane);
    };
    bf16x8 top[NP];
#pragma unroll
    for (int j = 0; j < PFP; ++j) top[j] = tread(j);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int u = j / (2 * DB), db = (j >> 1) % DB;
      if constexpr (D == 128) {  // P and dS were packed just before: first reads with the wait states
        if (j & 1) (j < 2 ? mfma_acc_nop : mfma_acc)(dkt[db], top[j], sb[u]);
        else (j < 2 ? mfma_acc_nop : mfma_acc)(dvt[db], top[j], pb[u]);
      } else {
        if (j & 1) dkt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(top[j], sb[u], dkt[db], 0, 0, 0);
        else dvt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(top[j], pb[u], dvt[db], 0, 0, 0);
      }
      if (j + PFP < NP) top[j + PFP] = tread(j + PFP);
      __builtin_amdgcn_sched_barrier(0);
    }
    s = s2;
    dp = dp2;
  };
  using T_ = std::integral_constant<bool, true>;
  using F_ = std::integral_constant<bool, false>;
  using DYN = std::integral_constant<int, -1>;

  load_tile(qt0 * kBQ, 0);
  if (nt > 1) load_tile((qt0 + 1) * kBQ, 1);
  wait_vmem<0>();
  __syncthreads();
  f32x16 s, dp;
  scores(0, s, dp);
  // the first 6 tiles (the 4 that hold the block's diagonal, rounded up to a multiple of 3) with
  // the mask; then groups of 3 with the LDS buffers known at compile time; the rest, and the last
  // tile (no next), with the mask (harmless where every key precedes every query)
  const int nm = CAUSAL ? min(nt - 1, 6) : 0;
  int t = 0;
  for (; t < nm; ++t) step(T_{}, T_{}, DYN{}, t, s, dp);
  if (t % 3 == 0) {
    for (; t + 3 < nt; t += 3) {
      step(T_{}, F_{}, std::integral_constant<int, 0>{}, t, s, dp);
      step(T_{}, F_{}, std::integral_constant<int, 1>{}, t + 1, s, dp);
      step(T_{}, F_{}, std::integral_constant<int, 2>{}, t + 2, s, dp);
    }
  }
  for (; t + 1 < nt; ++t) step(T_{}, T_{}, DYN{}, t, s, dp);
  step(F_{}, T_{}, DYN{}, nt - 1, s, dp);
  colsum += colsum1;

  // dK = scale dK^T, dV = dV^T: lane = key, dims 32db + 8(r/4) + 4hi + r%4 (runs of 4)
  if constexpr (D == 128) {
    agpr_fence(dkt);
    agpr_fence(dvt);
  }
  colsum = pair32_sum(colsum);
  if (key < n) {
    bf16* dkr = dk + tb + (int64_t)key * rs;
    bf16* dvr = dv + tb + (int64_t)key * rs;
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
    if (hi == 0) colsum_out[base + key] = colsum;
  }
}

// Query-stationary part (dQ, row sums of dS) for query block qb of head bh.  DPASS: the D pass
// instead, no dQ.  With D_i = 0 the row sums of dS are sum_j P_ij dP_ij; the pass also sums
// Z_i = sum_j P_ij.  The lse it is given normalised the forward's bf16-rounded probabilities,
// so these fp32 ones sum to Z_i = 1 + O(2^-9), and that excess, taken once per row, adds up in
// the suffix sums of dlog f over every row.  The pass divides it out: it writes D_i / Z_i to the
// D slot and a_i - log2 Z_i to the row term slot (dout_d: the row vectors, whose row term slot of
// its own rows it reads and rewrites only through dout_d), so the main parts see P with unit row
// sums.
template <int D, bool CAUSAL, bool DPASS = false>
__device__ __forceinline__ void bwd_dq_block(DqLds<D>& lds, size_t bh, int qb, const bf16* __restrict__ q,
                                             const bf16* __restrict__ k, const bf16* __restrict__ v,
                                             const bf16* __restrict__ dout, const float* __restrict__ rowv,
                                             const double* __restrict__ cb, bf16* __restrict__ dq,
                                             float* __restrict__ rowsum_out, float* __restrict__ dout_d, int n,
                                             int npad, int ncb, float scale, const BwdLayout& lay) {
  constexpr int KK = D / 16, DB = D / 32;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int qw0 = qb * kQB + 32 * wave;  // this wave's first query
  const int qi = qw0 + l32;               // this lane's query (accumulator column of S^T)
  const size_t base = bh * (size_t)n;  // this head's rows of the row-sum workspace
  const int64_t tb = lay.tbase((int)bh);
  const int rs = lay.rs;
  const float scale_log2 = scale * kLog2e;
  const float* blk = rowv + bh * 3 * npad;

  const uint32_t span = (uint32_t)(((int64_t)(n - 1) * rs + D) * 2);
  const u32x4 rk = sgpr_rsrc(k + tb, span);
  const u32x4 rv = sgpr_rsrc(v + tb, span);
  const u32x4 rcl = sgpr_rsrc(blk + 2 * npad, (uint32_t)(npad * 4));

  // this lane's q and dO rows as the B operands of S^T = K Q^T and dP^T = V dO^T
  bf16x8 qreg[KK], dreg[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    qreg[kk] = dreg[kk] = bf16x8{};
    if (qi < n) {
      qreg[kk] = *reinterpret_cast<const bf16x8*>(q + tb + (int64_t)qi * rs + 16 * kk + 8 * hi);
      dreg[kk] = *reinterpret_cast<const bf16x8*>(dout + tb + (int64_t)qi * rs + 16 * kk + 8 * hi);
    }
  }
  // (cq_i - lse_i) log2 e; no weight past n
  const float aq = qi >= n ? kNegInfB : DPASS ? dout_d[bh * 3 * (size_t)npad + qi] : blk[qi];
  const float dq_i = (qi < n && !DPASS) ? blk[npad + qi] : 0.0f;  // D_i
  // start C of the wave's 32-query block; each 32-key block adds its own block difference
  const double* cbh = cb + bh * (size_t)ncb;
  const double cqw = cbh[qw0 >> 5];
  double ck_b = cbh[0];  // block start of the 32-key block being processed

  const TileLoader<D, kKT> tl(wave, lane, rs);
  auto load_tile = [&](int k0, int buf) {
    tl.load(lds.k[buf], rk, k0, wave);
    tl.load(lds.v[buf], rv, k0, wave);
    if (wave == 0)
      lds_load4((uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(&lds.cl[buf][0])), rcl,
                (uint32_t)(k0 + lane) * 4u);
  };

  f32x16 acc[DB];  // dQ: lane = dim 32db + l32, register r = query 8(r/4) + 4hi + r%4
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  float rsum0 = 0.0f, rsum1 = 0.0f, zsum = 0.0f;
  const bf16x2 one2 = {(bf16)1.0f, (bf16)1.0f};

  const int kend = CAUSAL ? min(n, (qb + 1) * kQB) : n;  // keys this block sees
  const int nkt = (kend + kKT - 1) / kKT;
  const int nblk = 2 * nkt;  // 32-key blocks (the last may lie past kend: zero weight)

  // S^T = K Q^T and dP^T = V dO^T of one 32-key block: register r holds key 8(r/4) + 4hi + r%4
  constexpr int NQ = 2 * KK;   // score MFMAs per block (S and dP alternate)
  constexpr int EQ = 16 / NQ;  // accumulator elements of the previous block per score slot
  constexpr int PFQ = NQ >= 8 ? 4 : NQ;
  constexpr int NP = 2 * DB;   // dQ MFMAs per block
  constexpr int PFP = NP >= 4 ? 4 : NP;
  auto kvrow = [&](int buf, int kb, int i) -> bf16x8 {
    return row_operand<D>(i & 1 ? lds.v[buf] : lds.k[buf], 32 * kb + l32, 16 * (i >> 1) + 8 * hi);
  };
  auto scores = [&](int buf, int kb, f32x16& s, f32x16& dp) {
    s = dp = f32x16{};
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      if (i & 1) dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kvrow(buf, kb, i), dreg[i >> 1], dp, 0, 0, 0);
      else s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kvrow(buf, kb, i), qreg[i >> 1], s, 0, 0, 0);
    }
  };

  // One step per 32-key block b (tile b / 2, half b % 2), pipelined like the key-stationary
  // kernel: the score MFMAs of block b + 1 share slots with the elementwise work of block b, then
  // dQ += dS K for block b.  Three LDS buffers: the tile of block b, the next, and one loading.
  // HN: a next block exists; MASK: causal mask needed (the block may hold keys past queries);
  // BC: block b's index modulo 6 when known at compile time (its buffer (b / 2) % 3), else -1.
  auto step = [&](auto hn, auto mk, auto bc, int b, f32x16& s, f32x16& dp) {
    constexpr bool HN = decltype(hn)::value, MASK = CAUSAL && decltype(mk)::value;
    constexpr int BC = decltype(bc)::value;
    const int kt = b >> 1, kb = BC >= 0 ? (BC & 1) : (b & 1);
    const int buf = BC >= 0 ? (BC >> 1) : kt % 3;
    const int nbuf = BC >= 0 ? (((BC + 1) % 6) >> 1) : ((b + 1) >> 1) % 3, nkb = kb ^ 1;
    if constexpr (HN) {
      if (kb == 1) {
        // block b + 1 opens tile kt + 1: this wave's loads of it are the only vector-memory
        // instructions in flight; after the barrier every wave's loads are visible and tile
        // kt - 1's buffer is no longer read
        wait_vmem<0>();
        __syncthreads();
        if (kt + 2 < nkt) load_tile((kt + 2) * kKT, BC >= 0 ? ((BC >> 1) + 2) % 3 : (kt + 2) % 3);
      }
    }
    const int key0 = b * 32;
    const float aqb = aq + (float)((cqw - ck_b) * kLog2ed);  // the row term with this block's difference
    if constexpr (HN) ck_b = cbh[b + 1];
    const float* clb = &lds.cl[buf][32 * kb];
    bf16x8 aop[NQ];
    f32x4 c4[4];
    f32x16 s2 = f32x16{}, dp2 = f32x16{}, pz;
    c4[0] = *reinterpret_cast<const f32x4*>(&clb[4 * hi]);
    if constexpr (HN) {
#pragma unroll
      for (int i = 0; i < PFQ; ++i) aop[i] = kvrow(nbuf, nkb, i);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
#pragma unroll
      for (int g = 1; g < 4; ++g)
        if (i == (4 * g / EQ >= 2 ? 4 * g / EQ - 2 : 0)) c4[g] = *reinterpret_cast<const f32x4*>(&clb[8 * g + 4 * hi]);
      // P^T and dS^T of block b (fp32; rounded to bf16 once, as the dQ operand)
#pragma unroll
      for (int r = i * EQ; r < (i + 1) * EQ; ++r) {
        const int g = r >> 2, e = r & 3;
        float p = exp2_hw(fmaf(s[r], scale_log2, aqb) - c4[g][e]);
        if (MASK && key0 + 8 * g + 4 * hi + e > qi) p = 0.0f;
        if constexpr (DPASS) pz[r] = p;
        s[r] = p * (dp[r] - dq_i);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (HN) {
        if (i & 1) dp2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[i], dreg[i >> 1], dp2, 0, 0, 0);
        else s2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[i], qreg[i >> 1], s2, 0, 0, 0);
        if (i + PFQ < NQ) aop[i + PFQ] = kvrow(nbuf, nkb, i + PFQ);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // dQ += dS K: A = dS^T (queries as M, keys as K), B = K read transposed.  The row sums of dS
    // are taken over the fp32 values without the mask, over the bf16 values the MFMAs use with it.
    if constexpr (!CAUSAL) rsum0 += tree_sum16(s);
    if constexpr (DPASS) zsum += tree_sum16(pz);
    if constexpr (!DPASS) {
      const bf16x8 sb[2] = {acc_operand(s, 0), acc_operand(s, 1)};
      if constexpr (CAUSAL) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const bf16x2 pr = {sb[u][2 * w], sb[u][2 * w + 1]};
            if (w & 1) rsum1 = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, rsum1, false);
            else rsum0 = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, rsum0, false);
          }
        }
      }
      const bf16* tk = lds.k[buf];
      auto tread = [&](int j) -> bf16x8 {
        return transposed_operand<D>(tk, 32 * kb + 16 * (j / DB), 32 * (j % DB), lane);
      };
      bf16x8 top[NP];
#pragma unroll
      for (int j = 0; j < PFP; ++j) top[j] = tread(j);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        if constexpr (D == 128)  // dS was packed just before: first reads with the wait states
          (j % DB == 0 ? mfma_acc_nop : mfma_acc)(acc[j % DB], sb[j / DB], top[j]);
        else
          acc[j % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sb[j / DB], top[j], acc[j % DB], 0, 0, 0);
        if (j + PFP < NP) top[j + PFP] = tread(j + PFP);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    s = s2;
    dp = dp2;
  };
  using T_ = std::integral_constant<bool, true>;
  using F_ = std::integral_constant<bool, false>;
  using DYN = std::integral_constant<int, -1>;

  load_tile(0, 0);
  if (nkt > 1) load_tile(kKT, 1);
  wait_vmem<0>();
  __syncthreads();
  f32x16 s, dp;
  scores(0, 0, s, dp);
  // groups of 6 blocks (3 tiles) with the buffers known at compile time, unmasked; then the
  // rest one by one, with the causal mask on the blocks of the last tile... all blocks from
  // nblk - 4 on (the 128 keys of the diagonal)
  const int nfree = CAUSAL ? nblk - 4 : nblk - 1;  // blocks before the masked tail (with a next)
  int b = 0;
  for (; b + 6 <= nfree; b += 6) {
    step(T_{}, F_{}, std::integral_constant<int, 0>{}, b, s, dp);
    step(T_{}, F_{}, std::integral_constant<int, 1>{}, b + 1, s, dp);
    step(T_{}, F_{}, std::integral_constant<int, 2>{}, b + 2, s, dp);
    step(T_{}, F_{}, std::integral_constant<int, 3>{}, b + 3, s, dp);
    step(T_{}, F_{}, std::integral_constant<int, 4>{}, b + 4, s, dp);
    step(T_{}, F_{}, std::integral_constant<int, 5>{}, b + 5, s, dp);
  }
  for (; b + 1 < nblk; ++b) step(T_{}, T_{}, DYN{}, b, s, dp);
  step(F_{}, T_{}, DYN{}, nblk - 1, s, dp);

  // the two lane halves hold the two halves of each 32-key block
  const float rsum = pair32_sum(rsum0 + rsum1);
  if constexpr (DPASS) {
    float z = pair32_sum(zsum);
    if (!(z > 0.0f && z < INFINITY)) z = 1.0f;  // an lse that does not belong to these scores
    if (hi == 0 && qi < n) {
      float* row = dout_d + bh * 3 * (size_t)npad;
      row[qi] = aq - log2f(z);
      row[npad + qi] = rsum / z;
    }
    return;
  }
  // dq = scale dQ: lane = dim 32db + l32, register r = query qw0 + 8(r/4) + 4hi + r%4
  if constexpr (D == 128) agpr_fence(acc);
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qr = qw0 + 8 * (r >> 2) + 4 * hi + (r & 3);
      if (qr < n) dq[tb + (int64_t)qr * rs + 32 * db + l32] = (bf16)(acc[db][r] * scale);
    }
  }
  if (hi == 0 && qi < n) rowsum_out[base + qi] = rsum;
}

// The two parts as kernels of their own (large grids) ...
template <int D, bool CAUSAL, bool STAGE = false>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(D <= 64 && CAUSAL ? 2 : 1))) void bwd_kv_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v, const bf16* __restrict__ dout,
    const float* __restrict__ rowv, const double* __restrict__ cb, bf16* __restrict__ dk, bf16* __restrict__ dv,
    float* __restrict__ colsum_out, int n, int npad, int ncb, float scale, BwdLayout lay, bf16* __restrict__ ds = nullptr,
    int64_t ds_head = 0) {
  __shared__ KvLds<D> lds;
  // heads fastest: the key blocks of one head share its q / dO in L2; causal work falls with kb
  const int kb = (int)blockIdx.y;
  bf16* ds_stage = nullptr;
  if constexpr (STAGE) ds_stage = ds + blockIdx.x * ds_head + staged_tile0(kb, (n + kBQ - 1) / kBQ) * (kBK * kBQ);
  bwd_kv_block<D, CAUSAL, STAGE>(lds, blockIdx.x, kb, q, k, v, dout, rowv, cb, dk, dv, colsum_out, n, npad, ncb, scale,
                                 lay, ds_stage);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(D <= 64 && CAUSAL ? 2 : 1))) void bwd_dq_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v, const bf16* __restrict__ dout,
    const float* __restrict__ rowv, const double* __restrict__ cb, bf16* __restrict__ dq,
    float* __restrict__ rowsum_out, int n, int npad, int ncb, float scale, BwdLayout lay) {
  __shared__ DqLds<D> lds;
  // the longest causal blocks (the last queries) start first
  bwd_dq_block<D, CAUSAL>(lds, blockIdx.x, (int)(gridDim.y - 1 - blockIdx.y), q, k, v, dout, rowv, cb, dq, rowsum_out,
                          nullptr, n, npad, ncb, scale, lay);
}

// dQ and the row sums of dS from the staged dS (fox_attn_bwd_staged: causal, d = 128).  One
// workgroup of 4 waves per (128-query block, head); wave w owns query tile 4 qb + w.  Stage s is
// half s % 2 of key block s / 2: 64 keys of K and the matching 64 rows of the 4 waves' dS tiles,
// brought in by direct-to-LDS loads into a ring of kStageSlots stages, the next kStageSlots - 1 in
// flight while one is read.  Two slots (64 KiB) let two workgroups share a CU, each one stage ahead;
// that ran 2-3 % faster than one workgroup with three or four stages in flight.  dQ^T = K^T dS^T on
// v_mfma_f32_32x32x16_bf16 with dims as M and queries as N (A: K read transposed, B: the dS tile
// read transposed), so every accumulator lane holds one query; the row sums add the same bf16 dS
// values that the key-stationary kernel summed into the column sums.
constexpr int kStageKeys = 64;
constexpr int kStageSlots = 2;

template <int D>
struct alignas(16) StagedLds {
  bf16 k[kStageSlots][kStageKeys * D];        // K rows of each stage (swizzled, W = D)
  bf16 ds[kStageSlots][4][kStageKeys * kBQ];  // per stage and wave: dS rows [key][32 queries] (W = 32)
};

template <int D>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(kStageSlots <= 2 ? 2 : 1))) void bwd_dq_staged_kernel(
    const bf16* __restrict__ k, const bf16* __restrict__ ds, bf16* __restrict__ dq, float* __restrict__ rowsum_out,
    int n, int64_t ds_head, float scale, BwdLayout lay) {
  constexpr int DB = D / 32;
  __shared__ StagedLds<D> lds;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const size_t bh = blockIdx.x;
  const int qb = (int)(gridDim.y - 1 - blockIdx.y);  // the longest blocks first
  const int nqt = (n + kBQ - 1) / kBQ;
  const int qt = 4 * qb + wave;   // this wave's query tile (past the last one: loads and barriers only)
  // this lane's query: column l32 of the LDS dS rows (staged order, above)
  const int qi = qt * kBQ + 16 * (l32 >> 4) + 4 * ((l32 >> 3) & 1) + (l32 & 3) + 8 * ((l32 >> 2) & 1);
  const int64_t tb = lay.tbase((int)bh);
  const int rs = lay.rs;
  const int ns = 2 * (qb + 1);  // stages: key blocks 0..qb, two halves each

  // buffer resources: K rows past n and dS past the head's staged tiles read as zeros
  const u32x4 rk = sgpr_rsrc(k + tb, (uint32_t)(((int64_t)(n - 1) * rs + D) * 2));
  const u32x4 rds = sgpr_rsrc(ds + bh * ds_head, (uint32_t)(ds_head * 2));
  const TileLoader<D, kStageKeys> tl(wave, lane, rs);
  // this wave's 64 dS rows in LDS as [key][32 queries] with the queries in the staged order: chunk c
  // of a row is the 16 bytes a lane half c % 2 stored from register block c / 2, i.e. queries
  // 16 (c/2) + 4 (c%2) + {0..3, 8..11}.  4 loads of 16 rows: lane l of load j lands at chunk
  // position 4 (16 j + l / 4) + l % 4 of the stage, which holds chunk (l % 4) ^ swz<32>(row).
  uint32_t dsoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 16 * j + (lane >> 2), c = (lane & 3) ^ swz<kBQ>(r);
    dsoff[j] = (uint32_t)(((c >> 1) * (kBK * 16) + r * 16 + 8 * (c & 1)) * 2);
  }
  auto issue = [&](int st) {  // 8 vector-memory instructions per wave
    const int slot = st % kStageSlots, kbk = st >> 1, half = st & 1;
    tl.load(lds.k[slot], rk, kbk * kBK + half * kStageKeys, wave);
    const int64_t tile = staged_tile0(kbk, nqt) + (qt - 4 * kbk);
    const uint32_t base = (uint32_t)((tile * (kBK * kBQ) + half * (kStageKeys * 16)) * 2);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      lds_load16_nt((uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(&lds.ds[slot][wave][64 * 8 * j])), rds,
                    base + dsoff[j]);
  };

  f32x16 acc[DB];  // dQ^T: lane = query, register r = dim 32mb + 8(r/4) + 4hi + r%4
#pragma unroll
  for (int mb = 0; mb < DB; ++mb) acc[mb] = f32x16{};
  float rs0 = 0.0f, rs1 = 0.0f;
  const bf16x2 one2 = {(bf16)1.0f, (bf16)1.0f};

  static_assert(kStageSlots >= 2 && kStageSlots <= 5, "the waits below allow up to 3 later stages in flight");
  for (int st = 0; st < kStageSlots - 1 && st < ns; ++st) issue(st);
  for (int st = 0; st < ns; ++st) {
    // stage st has landed once at most the stages issued after it are in flight
    const int after = min(ns - 1, st + kStageSlots - 2) - st;
    if (after >= 3)
      wait_vmem<24>();
    else if (after == 2)
      wait_vmem<16>();
    else if (after == 1)
      wait_vmem<8>();
    else
      wait_vmem<0>();
    __syncthreads();  // every wave's loads of stage st are visible; stage st - 1's slot is free
    if (st + kStageSlots - 1 < ns) issue(st + kStageSlots - 1);
    const int slot = st % kStageSlots;
    const bf16* kt = lds.k[slot];
    const bf16* dt = lds.ds[slot][wave];
#pragma unroll
    for (int ks = 0; ks < kStageKeys / 16; ++ks) {
      const bf16x8 bop = transposed_operand<kBQ>(dt, 16 * ks, 0, lane);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const bf16x2 pr = {bop[2 * w], bop[2 * w + 1]};
        if (w & 1) rs1 = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, rs1, false);
        else rs0 = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, rs0, false);
      }
#pragma unroll
      for (int mb = 0; mb < DB; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(transposed_operand<D>(kt, 16 * ks, 32 * mb, lane), bop,
                                                          acc[mb], 0, 0, 0);
    }
  }
  const float rsum = pair32_sum(rs0 + rs1);
  if (qt < nqt && qi < n) {
    bf16* dqr = dq + tb + (int64_t)qi * rs;
#pragma unroll
    for (int mb = 0; mb < DB; ++mb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 a;
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = (bf16)(acc[mb][4 * g + e] * scale);
        *reinterpret_cast<bf16x4*>(dqr + 32 * mb + 8 * g + 4 * hi) = a;
      }
    }
    if (hi == 0) rowsum_out[bh * (size_t)n + qi] = rsum;
  }
}

// The D pass of the unmasked mode: D_i = sum_j P_ij dP_ij into the row vectors' D slot, with P
// rescaled to unit row sums (the row term slot takes the rescaling).
template <int D>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(1))) void bwd_dpass_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v, const bf16* __restrict__ dout,
    float* __restrict__ rowv, const double* __restrict__ cb, int n, int npad, int ncb, float scale, BwdLayout lay) {
  __shared__ DqLds<D> lds;
  bwd_dq_block<D, false, true>(lds, blockIdx.x, (int)blockIdx.y, q, k, v, dout, rowv, cb, nullptr, nullptr, rowv, n,
                               npad, ncb, scale, lay);
}

// ... and both in one launch for small grids, where each fills the other's tail.  blockIdx.x is the head (the
// blocks of one head are adjacent and share its tensors in L2); blockIdx.y = 2j is key block j and
// 2j + 1 is query block nb - 1 - j, so both kinds are issued heaviest first (causal work falls
// with the key block and grows with the query block).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(D <= 64 && CAUSAL ? 2 : 1))) void bwd_main_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v, const bf16* __restrict__ dout,
    const float* __restrict__ rowv, const double* __restrict__ cb, bf16* __restrict__ dq, bf16* __restrict__ dk,
    bf16* __restrict__ dv, float* __restrict__ rowsum_out, float* __restrict__ colsum_out, int n, int npad, int ncb,
    float scale, BwdLayout lay) {
  __shared__ union {
    KvLds<D> kv;
    DqLds<D> dq;
  } lds;
  const size_t bh = blockIdx.x;
  const int j = (int)(blockIdx.y >> 1);
  if ((blockIdx.y & 1) == 0)
    bwd_kv_block<D, CAUSAL>(lds.kv, bh, j, q, k, v, dout, rowv, cb, dk, dv, colsum_out, n, npad, ncb, scale, lay);
  else
    bwd_dq_block<D, CAUSAL>(lds.dq, bh, (int)(gridDim.y >> 1) - 1 - j, q, k, v, dout, rowv, cb, dq, rowsum_out,
                            nullptr, n, npad, ncb, scale, lay);
}

int bwd_npad(int n) { return (n + kPad - 1) / kPad * kPad; }

template <int D, bool CAUSAL>
hipError_t launch_bwd_c(const void* q, const void* k, const void* v, const void* dout, const float* rowv,
                        const double* cb, void* dq, void* dk, void* dv, float* rsum, float* csum, int64_t bh, int n,
                        int npad, int ncb, float scale, const BwdLayout& lay, hipStream_t stream, bf16* ds,
                        int64_t ds_head) {
  static_assert(kBK == kQB, "one key block and one query block per block pair");
  const int nb = (n + kBK - 1) / kBK;
  if constexpr (D == 128 && CAUSAL) {
    if (ds) {  // staged dS: the key-stationary kernel writes it, a contraction with K gives dQ
      const dim3 grid((unsigned)bh, (unsigned)nb);
      hipLaunchKernelGGL((bwd_kv_kernel<D, true, true>), grid, dim3(kBwdThreads), 0, stream, (const bf16*)q,
                         (const bf16*)k, (const bf16*)v, (const bf16*)dout, rowv, cb, (bf16*)dk, (bf16*)dv, csum, n,
                         npad, ncb, scale, lay, ds, ds_head);
      hipLaunchKernelGGL((bwd_dq_staged_kernel<D>), grid, dim3(kBwdThreads), 0, stream, (const bf16*)k,
                         (const bf16*)ds, (bf16*)dq, rsum, n, ds_head, scale, lay);
      return hipGetLastError();
    }
  }
  if (2 * bh * nb <= kFuseMaxBlocks) {
    hipLaunchKernelGGL((bwd_main_kernel<D, CAUSAL>), dim3((unsigned)bh, (unsigned)(2 * nb)), dim3(kBwdThreads), 0,
                       stream, (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)dout, rowv, cb, (bf16*)dq,
                       (bf16*)dk, (bf16*)dv, rsum, csum, n, npad, ncb, scale, lay);
  } else {
    const dim3 grid((unsigned)bh, (unsigned)nb);
    hipLaunchKernelGGL((bwd_kv_kernel<D, CAUSAL>), grid, dim3(kBwdThreads), 0, stream, (const bf16*)q,
                       (const bf16*)k, (const bf16*)v, (const bf16*)dout, rowv, cb, (bf16*)dk, (bf16*)dv, csum, n,
                       npad, ncb, scale, lay);
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), grid, dim3(kBwdThreads), 0, stream, (const bf16*)q,
                       (const bf16*)k, (const bf16*)v, (const bf16*)dout, rowv, cb, (bf16*)dq, rsum, n, npad, ncb,
                       scale, lay);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_t(const void* q, const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, const float* logf, void* dq, void* dk, void* dv, float* dlogf, void* ws,
                        int64_t b, int64_t h, int n, float scale, bool causal, bool token_major,
                        hipStream_t stream, bf16* ds = nullptr, int64_t ds_head = 0) {
  const int64_t bh = b * h;
  const int npad = bwd_npad(n);
  const int ncb = bwd_gate_blocks(n);
  // {bs, hs, rs, gbs, ghs, gs, nh}
  const BwdLayout lay = token_major
                            ? BwdLayout{(int64_t)n * h * D, (int64_t)D, (int)(h * D), (int64_t)n * h, 1, (int)h, (int)h}
                            : BwdLayout{h * n * (int64_t)D, (int64_t)n * D, D, h * (int64_t)n, (int64_t)n, 1, (int)h};
  const BwdWorkspace w = bwd_workspace(ws, bh, n, npad);
  hipError_t e = hipSuccess;
  if (causal) {
    constexpr int RPB = kBwdThreads / (D / 8);
    const int64_t pre_blocks = (bh * npad + RPB - 1) / RPB;
    hipLaunchKernelGGL((bwd_rows_kernel<D>), dim3((unsigned)(bh + pre_blocks)), dim3(kBwdThreads), 0, stream, logf,
                       lse, (const bf16*)o, (const bf16*)dout, w.rowv, w.cb, bh, n, npad, ncb,
                       gate_rows_in((int)h, n, token_major), lay);
  } else {
    e = launch_bwd_gate_rows(logf, lse, w.rowv, w.cb, bh, n, npad, (int)h, token_major, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dpass_kernel<D>), dim3((unsigned)bh, (unsigned)((n + kQB - 1) / kQB)), dim3(kBwdThreads),
                       0, stream, (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)dout, w.rowv,
                       (const double*)w.cb, n, npad, ncb, scale, lay);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = causal ? launch_bwd_c<D, true>(q, k, v, dout, w.rowv, w.cb, dq, dk, dv, w.rsum, w.csum, bh, n, npad, ncb, scale,
                                     lay, stream, ds, ds_head)
             : launch_bwd_c<D, false>(q, k, v, dout, w.rowv, w.cb, dq, dk, dv, w.rsum, w.csum, bh, n, npad, ncb, scale,
                                      lay, stream, nullptr, 0);
  if (e != hipSuccess) return e;
  // dlog f_t = sum_{i >= t} (rowsum_i - colsum_i), written in the gates' layout
  return launch_suffix_sum(w.rsum, w.csum, dlogf, bh, n, (int)h, token_major, stream);
}

}  // namespace

int bwd_gate_blocks(int n) { return (n + 127) / 128 * (128 / kGateBlock); }

hipError_t launch_bwd_gate_rows(const float* logf, const float* lse, float* rowv, double* cb, int64_t rows, int n,
                                int npad, int nh, bool token_major, hipStream_t stream) {
  hipLaunchKernelGGL(bwd_gate_rows_kernel, dim3((unsigned)rows), dim3(kScanThreads), 0, stream, logf, lse, rowv, cb,
                     n, npad, bwd_gate_blocks(n), gate_rows_in(nh, n, token_major));
  return hipGetLastError();
}

// workspace: row vectors [bh][3][npad] (fp32), gate block starts [bh][ncb] (fp64), row sums and
// column sums of dS and the fp32 path's lse normalisation [bh][n] each (fp32)
BwdWorkspace bwd_workspace(void* ws, int64_t bh, int n, int npad) {
  BwdWorkspace w;
  w.rowv = static_cast<float*>(ws);
  w.cb = reinterpret_cast<double*>(w.rowv + bh * 3 * (int64_t)npad);
  w.rsum = reinterpret_cast<float*>(w.cb + bh * (int64_t)bwd_gate_blocks(n));
  w.csum = w.rsum + bh * (int64_t)n;
  w.corr = w.csum + bh * (int64_t)n;
  return w;
}

size_t attn_bwd_workspace_bytes(int64_t bh, int n, int d) {
  (void)d;
  return (size_t)bh * ((3 * (size_t)bwd_npad(n) + 3 * (size_t)n) * sizeof(float) +
                       (size_t)bwd_gate_blocks(n) * sizeof(double));
}

hipError_t launch_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, const float* logf, void* dq, void* dk, void* dv, float* dlogf,
                           void* workspace, int64_t b, int64_t h, int n, int d, float scale, bool causal,
                           bool token_major, hipStream_t stream) {
  switch (d) {
    case 32:
      return launch_bwd_t<32>(q, k, v, o, dout, lse, logf, dq, dk, dv, dlogf, workspace, b, h, n, scale, causal,
                              token_major, stream);
    case 64:
      return launch_bwd_t<64>(q, k, v, o, dout, lse, logf, dq, dk, dv, dlogf, workspace, b, h, n, scale, causal,
                              token_major, stream);
    case 128:
      return launch_bwd_t<128>(q, k, v, o, dout, lse, logf, dq, dk, dv, dlogf, workspace, b, h, n, scale, causal,
                               token_major, stream);
  }
  return hipErrorInvalidValue;
}

// Staged backward: the workspace of attn_bwd_workspace_bytes, then (256-byte aligned) the staged dS
// of every head, staged_tiles(n) tiles of 128 x 32 bf16 each.
size_t attn_bwd_staged_workspace_bytes(int64_t bh, int n) {
  const size_t base = (attn_bwd_workspace_bytes(bh, n, 128) + 255) / 256 * 256;
  return base + (size_t)bh * (size_t)staged_tiles(n) * (kBK * kBQ) * sizeof(bf16);
}

int64_t attn_bwd_staged_head_bytes(int n) { return staged_tiles(n) * (kBK * kBQ) * (int64_t)sizeof(bf16); }

hipError_t launch_attn_bwd_staged(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                  const float* lse, const float* logf, void* dq, void* dk, void* dv, float* dlogf,
                                  void* workspace, int64_t b, int64_t h, int n, float scale, bool token_major,
                                  hipStream_t stream) {
  const size_t base = (attn_bwd_workspace_bytes(b * h, n, 128) + 255) / 256 * 256;
  bf16* ds = reinterpret_cast<bf16*>(static_cast<char*>(workspace) + base);
  return launch_bwd_t<128>(q, k, v, o, dout, lse, logf, dq, dk, dv, dlogf, workspace, b, h, n, scale, true,
                           token_major, stream, ds, staged_tiles(n) * (kBK * kBQ));
}

}  // namespace fox
