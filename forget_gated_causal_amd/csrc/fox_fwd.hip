// fox_fwd.hip -- fused causal FoX attention forward on gfx950 MFMA.
//
// Definition (FoX module page, ForgettingAttention.forward, decoder mode;
// foxwindow README, opening paragraph):
//   s_ij = scale * q_i.k_j + sum_{t=j+1..i} log f_t  (j <= i),  softmax over j,  O_i = sum_j p_ij v_j.
//
// Work decomposition (bf16)
//   * One workgroup of NW waves (4 or 8) per (query block of 32*NW rows, batch*head); wave w
//     owns 32 query rows.  Grid x = batch*head (fastest, so the workgroups of one head land
//     on one XCD when batch*head is a multiple of 8 and share its L2), grid y = query block,
//     heaviest (last) blocks dispatched first.  8-wave blocks stage each K/V tile for twice
//     the rows; they are used when the grid still has two blocks per CU.
//   * Key tiles of 64 keys are visited from the diagonal tile DOWN to tile 0; tiles above
//     the diagonal are never touched (their weights are exactly 0).  Walking backwards makes
//     the first tile a row sees hold its largest gate bias, so the running max rarely moves
//     and the lazy rescale below almost never fires.
//   * Gate bias without a prefix-sum buffer: while walking backwards one wave keeps the fp64
//     suffix sum R_j = sum_{t=j+1..ref} log f_t (ref = the block's last row).  Then
//     c_i - c_j = R_j - R_i; the per-row constant R_i drops out of the softmax and is added
//     back to lse only.  The biases enter as the initial value of the S accumulators (R_j /
//     scale per key), so a score costs one FMA into its exponential:
//     p = exp2(acc * scale * log2e - m).  The block's own c_i = c_ref - R_i is written as the
//     `c` output.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (keys = M, queries = N), so a lane holds one
//     query row and 16 keys per 32x32 block: the row max / sum are in-lane plus one
//     permlane32 swap.  The S^T accumulator registers are, after rounding to bf16, directly
//     the B operand of O^T = V^T P^T (the V operand follows the same key order).
//   * K and V tiles move global -> LDS with direct-to-LDS buffer loads into a ring of four
//     stages (XOR-swizzled rows, no padding).  The PV operand, which needs 8 keys of one dim
//     per lane, comes from gfx950's transposing LDS read (ds_read_b64_tr_b16).
//   * Each wave software-pipelines its tiles: the MFMAs of S for tile t run beside the
//     exponentials of tile t+1, the MFMAs of O += V^T P^T for tile t+1 beside the row max of
//     tile t (a two-wave split of MFMA and VALU roles measured slower on this chip).
//   * Online softmax in base 2 with lazy rescaling: the running max is only raised when a
//     row's tile max exceeds it by more than kTau (exact: the final normalisation uses the
//     same stale max; p stays <= 2^kTau).  The row sum adds the bf16-rounded p, the same
//     weights the P.V products use.
//
// fp32 inputs run the kernel of fox_fwd_f32.hip (launch_fwd_f32); the gate-sum scan and the tile
// constants both use are in fox_fwd_gates.h.
#include <math.h>

#include <type_traits>

#include "fox_device.h"
#include "fox_fwd_gates.h"
#include "fox_internal.h"

namespace fox {
namespace {

// ------------------------------------------------------------------------------------------
// bf16
// ------------------------------------------------------------------------------------------
// Staging geometry of the bf16 kernel.  Key tiles move global -> LDS with direct-to-LDS
// buffer loads (buffer_load_dwordx4 ... lds): one wave instruction writes 1 KB of LDS, 16
// bytes per lane, contiguously.  Rows are therefore unpadded, and bank spreading comes from an XOR
// swizzle of the 16-byte chunks of each row, applied by choosing which global chunk each
// lane fetches.
template <int D, int NW>
struct Bf16Geom {
  static constexpr int BR = 32 * NW;         // query rows per workgroup
  static constexpr int ROWB = 2 * D;         // bytes per key row
  static constexpr int CH = D / 8;           // 16-byte chunks per row
  static constexpr int RPO = 1024 / ROWB;    // key rows per 1 KB wave instruction
  static constexpr int OPS = kBC * ROWB / 1024 / NW;  // wave instructions per wave for K (and for V)
  static_assert(OPS >= 1 && OPS * NW * 1024 == kBC * ROWB, "staging mapping");
};

// Chunk swizzles.  K is read 16 bytes per lane by 16 consecutive rows at one logical
// chunk: the swizzle gives those rows 16 distinct chunks of the 64 banks.  V is read by
// the transposed b64 loads, 4 consecutive rows x 64 bytes per half-wave: the swizzle moves
// the 4 rows onto disjoint 64-byte bank groups.
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  if constexpr (D == 128) return row & 15;
  else if constexpr (D == 64) return (row >> 1) & 7;
  else return (row >> 2) & 3;
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  if constexpr (D == 128) return 4 * (row & 3);
  else if constexpr (D == 64) return 4 * ((row >> 1) & 1);
  else return 0;
}

template <int D>
struct alignas(1024) Bf16Stage {  // one staged key tile; 1 KB aligned so swizzled offsets XOR into the address
  bf16 k[kBC * D];
  bf16 v[kBC * D];
  float lf[kBC];  // the tile's log gates, as loaded
};

typedef __attribute__((address_space(3))) void lds_void_t;

// LDS byte address of a __shared__ object (address space 3 offset).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) void*)p);
}

// Raw buffer resource (byte offsets, no stride) over num_bytes at p: loads at or past
// num_bytes return zeros, which is how keys past n in the top tile are zero-filled.
__device__ __forceinline__ u32x4 raw_rsrc(const void* p, uint32_t num_bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  u32x4 r;
  r[0] = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
  r[2] = (uint32_t)__builtin_amdgcn_readfirstlane((int)num_bytes);
  r[3] = 0x00020000u;
  return r;
}

// Direct-to-LDS buffer loads: lane l's bytes land at LDS address m0v + l * size.  Issued
// through inline assembly so the compiler does not track them: the kernel waits for them
// itself (s_waitcnt vmcnt with counts derived from its own issue order), which lets the
// next tiles stay in flight across barriers and LDS reads of other stages.  M0 is an input
// operand: the compiler writes it (and knows it holds m0v) before each load; the s_nop is the
// wait state an M0 write needs before an LDS-DMA instruction reads it.
__device__ __forceinline__ void lds_dma16(uint32_t m0v, u32x4 rsrc, uint32_t voff) {
  __asm__ volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                   :
                   : "v"(voff), "s"(rsrc), "{m0}"(m0v)
                   : "memory");
}
__device__ __forceinline__ void lds_dma4(uint32_t m0v, u32x4 rsrc, uint32_t voff) {
  __asm__ volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
                   :
                   : "v"(voff), "s"(rsrc), "{m0}"(m0v)
                   : "memory");
}

// Per-lane byte offsets, inside a tile, of the 16-byte chunks this lane stages for K and V.
template <int D, int NW>
struct StageOffsets {
  int k[Bf16Geom<D, NW>::OPS];
  int v[Bf16Geom<D, NW>::OPS];
};

template <int D, int NW>
__device__ __forceinline__ StageOffsets<D, NW> stage_offsets(int wave, int lane, int rs) {
  using G = Bf16Geom<D, NW>;
  StageOffsets<D, NW> so;
#pragma unroll
  for (int o = 0; o < G::OPS; ++o) {
    const int g = wave * G::OPS + o;           // 1 KB slice of the tile
    const int row = g * G::RPO + lane / G::CH;  // key row inside the tile
    const int pc = lane % G::CH;                // physical chunk this lane fills
    so.k[o] = (row * rs + 8 * (pc ^ swz_k<D>(row))) * (int)sizeof(bf16);
    so.v[o] = (row * rs + 8 * (pc ^ swz_v<D>(row))) * (int)sizeof(bf16);
  }
  return so;
}

// One load instruction of the gate wave: tile t's 64 log gates into lf.
__device__ __forceinline__ void bf16_stage_gates(float* lf, u32x4 rl, int t, int gs) {
  // lane index recomputed here (volatile, so not hoisted) rather than kept live across the tile loop
  uint32_t ln;
  __asm__ volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
  lds_dma4(lds_addr(lf), rl, ((uint32_t)(t * kBC) + ln) * (uint32_t)(gs * (int)sizeof(float)));
}

// Issue this wave's loads of key tile t into stage `s`: (the gate wave, when asked) one for the
// tile's 64 log gates, then 2 * OPS for K and V.  Number of instructions issued, per wave, is what
// the vmcnt waits below count.
template <int D, int NW>
__device__ __forceinline__ void bf16_stage_tile(Bf16Stage<D>& s, float* lf, u32x4 rk, u32x4 rv, u32x4 rl,
                                                const StageOffsets<D, NW>& so, int t, int wave, int lane,
                                                bool gate_wave, int rs, int gs) {
  using G = Bf16Geom<D, NW>;
  const uint32_t tile_off = (uint32_t)t * (uint32_t)(kBC * rs * (int)sizeof(bf16));
  const int wv = __builtin_amdgcn_readfirstlane(wave);  // LDS destinations are wave-uniform (M0)
  if (gate_wave) bf16_stage_gates(lf, rl, t, gs);
#pragma unroll
  for (int o = 0; o < G::OPS; ++o) {
    const int g = wv * G::OPS + o;
    lds_dma16(lds_addr(&s.k[g * 512]), rk, tile_off + (uint32_t)so.k[o]);
    lds_dma16(lds_addr(&s.v[g * 512]), rv, tile_off + (uint32_t)so.v[o]);
  }
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt not waited on).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that does not drain outstanding global loads (a __syncthreads() would
// wait for the in-flight prefetches); callers wait for exactly the loads they need first.
__device__ __forceinline__ void barrier_lds() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0): gate / LDS writes done
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// ds_read_b64_tr_b16: within each 16-lane group, output lane j element e is element j%4
// of the 8 bytes addressed by lane 4e + j/4 of the group (transpose of a 16x4 block).
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;
__device__ __forceinline__ bf16x4 lds_read_tr16(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p));
}

// Byte-offset access into a stage array, keeping the pointer's provenance (the compiler
// needs to see which __shared__ object is read to not order it after unrelated loads).
__device__ __forceinline__ bf16x8 lds_read_b128(const bf16* base, uint32_t byte_off) {
  return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(base) + byte_off);
}
__device__ __forceinline__ bf16x4 lds_read_tr16_at(const bf16* base, uint32_t byte_off) {
  return lds_read_tr16(reinterpret_cast<const bf16*>(reinterpret_cast<const char*>(base) + byte_off));
}

// Per-lane LDS byte offsets inside a stage.  The swizzles only touch bits 5-7 (K) and 6-7
// (V) of these offsets, so the operand of chunk step kk is at k ^ (kk << 5) and that of dim
// block db at v ^ (db << 6); row offsets of later blocks / steps are multiples of 512 bytes
// and are added on top.
template <int D>
struct LaneOffsets {
  uint32_t k;  // K operand, chunk step 0, key row l32
  uint32_t v;  // V operand, dim block 0, the lane's transposed-read row
};

template <int D>
__device__ __forceinline__ LaneOffsets<D> lane_offsets(int lane) {
  LaneOffsets<D> off;
  const int l32 = lane & 31, hi = lane >> 5, li = lane & 15, half = (lane >> 4) & 1;
  off.k = (uint32_t)(2 * (l32 * D + 8 * (hi ^ swz_k<D>(l32))));
  const int vrow = 4 * hi + (li >> 2);
  const int dim = 16 * half + 4 * (li & 3);
  off.v = (uint32_t)(2 * (vrow * D + 8 * ((dim >> 3) ^ swz_v<D>(vrow)) + (dim & 7)));
  return off;
}

// ------------------------------------------------------------------------------------------
// bf16, software-pipelined form
// ------------------------------------------------------------------------------------------
// Each wave runs its own two-stage pipeline over key tiles: while the MFMAs of S(t) = K_t Q^T
// execute, the wave computes the probabilities of tile t+1 (the previous tile in visiting
// order); while the MFMAs of O += V_{t+1}^T P^T execute, it takes the row max of tile t.  A
// wave issues at most about one VALU instruction per 8 clocks, so its VALU work sits between
// its own MFMAs, and the two waves of a SIMD overlap each other's MFMAs as well (a split of
// the two roles between the waves, switching at barriers, measured slower).  Four LDS stages
// hold tile t+1 (V still read), tile t, and the two tiles in flight.

template <int D>
struct PipeGeom {
  static constexpr int KK = D / 16;  // MFMA k-steps of S (16 dims each)
  static constexpr int DB = D / 32;  // 32-dim output blocks of O
};

// The gate biases of a tile enter the scores as the S accumulators' initial value: the lead
// wave stores R_j / (scale log2 e) * log2 e = R_j / scale per key, so a finished accumulator
// holds a_ij = q_i.k_j + R_j / scale, and the base-2 score is a_ij * scale * log2 e.  Per
// score that leaves one FMA, exp2(a * scale * log2 e - m), and a max on the raw a (the
// scale is positive, so the max commutes with it).
//
// Bias tuple of block b in the accumulator layout of S^T: register 4g+e of lane (l32, hi)
// is key 32b + 8g + 4hi + e.
__device__ __forceinline__ f32x16 pipe_bias(const float* r2s, int b, int hi) {
  f32x16 c;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const f32x4 r = *reinterpret_cast<const f32x4*>(&r2s[32 * b + 8 * g + 4 * hi]);
#pragma unroll
    for (int e = 0; e < 4; ++e) c[4 * g + e] = r[e];
  }
  return c;
}

// S^T of one tile: s[b] = K[32b .. 32b+31] Q^T + bias (32 keys x 32 queries per block).
template <int D>
__device__ __forceinline__ void pipe_qk(const Bf16Stage<D>& st, uint32_t koff, const bf16x8 (&qreg)[D / 16],
                                        const float* r2s, int hi, f32x16 (&s)[2]) {
  constexpr int KK = PipeGeom<D>::KK;
  s[0] = pipe_bias(r2s, 0, hi);
  s[1] = pipe_bias(r2s, 1, hi);
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const uint32_t a = koff ^ (uint32_t)(kk << 5);
    s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read_b128(st.k, a), qreg[kk], s[0], 0, 0, 0);
    s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read_b128(st.k, a + 64 * D), qreg[kk], s[1], 0, 0, 0);
  }
}

// Causal mask of the first tile (keys past `my_row` -> -inf, in place) and the tile's row
// max in base-2 units (both lanes of a row).
template <bool DIAG>
__device__ __forceinline__ float pipe_scores(f32x16 (&s)[2], int key0, int my_row, int hi, float scale_log2) {
  float mx = kNegInf;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float sv = s[b][r];
      if constexpr (DIAG) {
        if (key0 + 32 * b + 8 * (r >> 2) + 4 * hi + (r & 3) > my_row) sv = kNegInf;
      }
      s[b][r] = sv;
      mx = fmaxf(mx, sv);
    }
  }
  return pair32_max(mx) * scale_log2;
}

// Lazy rescale (mx = the tile's row max, base 2): raise m only when the tile max exceeds it
// by more than kTau, and scale O and l to the new max.
template <int DB>
__device__ __forceinline__ void pipe_rescale(float mx, float& m, float& lsum, f32x16 (&oacc)[DB]) {
  const float rel = mx - m;
  const bool need = rel > kTau;
  if (wave_any(need)) {
    const float delta = need ? rel : 0.0f;
    const float alpha = exp2_hw(-delta);
    lsum *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
    m += delta;
  }
}

// p = exp2(a * scale * log2 e - m) rounded to bf16, in the key order of the S^T registers:
// p[2b+u] holds keys 32b + 16u + {4hi .. 4hi+3, 8+4hi .. 8+4hi+3}, the B operand of
// O^T += V^T P^T.
__device__ __forceinline__ void pipe_probs(const f32x16 (&s)[2], float m, float scale_log2, bf16x8 (&p)[4]) {
#pragma unroll
  for (int b = 0; b < 2; ++b) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int e = 0; e < 8; ++e) p[2 * b + u][e] = (bf16)exp2_hw(fmaf(s[b][8 * u + e], scale_log2, -m));
    }
  }
}

// Row-sum of the rounded probabilities (the weights the P.V products actually use).
__device__ __forceinline__ float pipe_psum(const bf16x8 (&p)[4], float acc) {
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
  float a0 = acc, a1 = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const bf16x2 pr = {p[i][2 * w], p[i][2 * w + 1]};
      if (w & 1) a1 = __builtin_amdgcn_fdot2_f32_bf16(pr, one, a1, false);
      else a0 = __builtin_amdgcn_fdot2_f32_bf16(pr, one, a0, false);
    }
  }
  return a0 + a1;
}

// O^T += V^T P^T over one tile.  The V operand of lane (l32, hi) is V[key][32db + l32] for
// the 8 keys of p[2b+u]: two transposed reads of 4 keys each (lane i of a 16-lane group
// points at V[key0 + i/4][dim0 + 4(i%4)]).
template <int D>
__device__ __forceinline__ void pipe_pv(const Bf16Stage<D>& st, uint32_t voff, const bf16x8 (&p)[4],
                                        f32x16 (&oacc)[D / 32]) {
  constexpr int DB = PipeGeom<D>::DB;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint32_t va = (voff ^ (uint32_t)(db << 6)) + (uint32_t)(2 * (32 * b + 16 * u) * D);
        const bf16x4 lo = lds_read_tr16_at(st.v, va);
        const bf16x4 hi4 = lds_read_tr16_at(st.v, va + 16 * D);
        const bf16x8 a = __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p[2 * b + u], oacc[db], 0, 0, 0);
      }
    }
  }
}

// Steady state, one tile: S(cur) = K_cur Q^T and O += V_prev^T P(prev)^T on MFMA, with the
// softmax of both tiles between them.  The schedule is explicit: each slot holds one MFMA,
// the LDS reads a few slots ahead of their use, and a share of the VALU work that does
// not depend on in-flight MFMAs; sched_barrier keeps the compiler from regrouping slots.
//   S slots (2*KK):  MFMA of S(cur); sc arrives holding cur's gate-bias tuples, the initial
//                    value of its accumulators; p = exp2(a * scale log2 e - m) for 32/(2*KK)
//                    scores of prev.
//   PV slots (4*DB): MFMA of O += V^T P^T; bf16 packing and row sum of P(prev); row max of
//                    cur (block 0 first: its MFMAs finished earlier); once a block of prev is
//                    packed, its registers take the next tile's bias tuple (r2next): they are
//                    the next step's accumulators.
// With GATE the wave also runs the gate scan of a later tile (GateJob) in the P.V slots, so
// the wave that owns the scan does not hold the others up at the next barrier.
template <int D, bool GATE>
__device__ __forceinline__ void pipe_steady(const Bf16Stage<D>& cur, const float* r2next, const Bf16Stage<D>& prev,
                                            const LaneOffsets<D>& off, const bf16x8 (&qreg)[D / 16],
                                            f32x16 (&sp)[2], f32x16 (&sc)[2], f32x16 (&oacc)[D / 32], float& m,
                                            float& lsum, int lane, float scale_log2, const GateJob& gj) {
  const int hi = lane >> 5;
  constexpr int KK = PipeGeom<D>::KK, DB = PipeGeom<D>::DB;
  constexpr int NQ = 2 * KK;   // S MFMAs
  constexpr int NP = 4 * DB;   // P.V MFMAs
  constexpr int PFK = NQ >= 6 ? 4 : NQ - 2;  // K operands in flight
  constexpr int PFV = NP >= 4 ? 4 : NP;      // V operands in flight
  constexpr int EQ = 32 / NQ;  // exponentials per S slot
  constexpr int EP = 32 / NP;  // scores per P.V slot
  static_assert(NQ >= PFK + 2 && NQ >= PFV && NP >= PFV && 32 % NQ == 0 && 32 % NP == 0, "slot shares");

  bf16x8 kop[NQ];
  bf16x8 vop[NP];
  bf16x8 p[4];
  auto kread = [&](int i) -> bf16x8 {
    return lds_read_b128(cur.k, (off.k ^ (uint32_t)((i >> 1) << 5)) + (uint32_t)((i & 1) * 64 * D));
  };
  auto vread = [&](int i) -> bf16x8 {
    const int pi = i / DB, db = i % DB, b = pi >> 1, u = pi & 1;
    const uint32_t va = (off.v ^ (uint32_t)(db << 6)) + (uint32_t)(2 * (32 * b + 16 * u) * D);
    const bf16x4 lo = lds_read_tr16_at(prev.v, va);
    const bf16x4 hi4 = lds_read_tr16_at(prev.v, va + 16 * D);
    return __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto pack = [&](int pi) {
    const int b = pi >> 1, u = pi & 1;
#pragma unroll
    for (int e = 0; e < 8; ++e) p[pi][e] = (bf16)sp[b][8 * u + e];
  };
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
  const float negm = -m;
  float ls0 = lsum, ls1 = 0.0f;
  float mx0 = kNegInf, mx1 = kNegInf;
  double gx = 0.0, gy = 0.0;  // gate value of key 63-lane of the next tile, its running scan

  // The step runs one of two instances of this schedule (with and without the gate job).  Their
  // exponentials are identical, so the compiler would hoist them above the branch, out of the
  // S slots they are meant to overlap; an opaque, instance-specific copy of their inputs keeps
  // them here.
  if constexpr (GATE) __asm__ volatile("; gate" : "+v"(sp[0]), "+v"(sp[1]));
  else __asm__ volatile("; nogate" : "+v"(sp[0]), "+v"(sp[1]));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < PFK; ++i) kop[i] = kread(i);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int b = i & 1, kk = i >> 1;
    // The slot's exponentials go ahead of its MFMA: at the start of a tile they run while the
    // first K operands are still in flight.
#pragma unroll
    for (int e = i * EQ; e < (i + 1) * EQ; ++e) sp[e >> 4][e & 15] = exp2_hw(fmaf(sp[e >> 4][e & 15], scale_log2, negm));
    __builtin_amdgcn_sched_barrier(0);
    sc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[i], qreg[kk], sc[b], 0, 0, 0);
    if (i + PFK < NQ) kop[i + PFK] = kread(i + PFK);
    if (i >= NQ - PFV) vop[i - (NQ - PFV)] = vread(i - (NQ - PFV));  // first V operands of the P.V slots
    if (i == NQ - 1) pack(0);
    if (GATE && i == 0) gx = (double)((gj.kt * kBC + 63 - lane <= gj.fref) ? gj.lf[63 - lane] : 0.0f);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int pi = i / DB, db = i % DB;
    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[i], p[pi], oacc[db], 0, 0, 0);
    if (i + PFV < NP) vop[i + PFV] = vread(i + PFV);
    if (db == DB - 1 && pi < 3) pack(pi + 1);
    // row sum: the 4 words of p[pi] over the DB slots of pi
#pragma unroll
    for (int w = db * 4 / DB; w < (db + 1) * 4 / DB; ++w) {
      const bf16x2 pr = {p[pi][2 * w], p[pi][2 * w + 1]};
      if (w & 1) ls1 = __builtin_amdgcn_fdot2_f32_bf16(pr, one, ls1, false);
      else ls0 = __builtin_amdgcn_fdot2_f32_bf16(pr, one, ls0, false);
    }
#pragma unroll
    for (int e = i * EP; e < (i + 1) * EP; ++e) {
      const float sv = sc[e >> 4][e & 15];
      if (e & 1) mx1 = fmaxf(mx1, sv);
      else mx0 = fmaxf(mx0, sv);
    }
    // next tile's bias quads: block 0 once pack(1) has consumed sp[0], block 1 after pack(3)
#pragma unroll
    for (int qd = 0; qd < 8; ++qd) {
      const int b = qd >> 2, g = qd & 3;
      if ((b == 0 ? DB + (2 * DB * g) / 4 : 3 * DB + (DB * g) / 4) == i) {
        const f32x4 r = *reinterpret_cast<const f32x4*>(&r2next[32 * b + 8 * g + 4 * hi]);
#pragma unroll
        for (int e = 0; e < 4; ++e) sp[b][4 * g + e] = r[e];
      }
    }
    if constexpr (GATE) {  // scan steps 1..7 and the finish, spread evenly over the slots
#pragma unroll
      for (int k = 1; k <= 8; ++k) {
        if ((k - 1) * NP / 8 == i) {
          if (k <= 7) wave_scan_step(k, gx, gy);
          else gate_finish(gy, gj.r2, nullptr, *gj.rows, lane, gj.kt, gj.row0, gj.ref, *gj.carry, gj.unit);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  lsum = ls0 + ls1;
  pipe_rescale<DB>(pair32_max(fmaxf(mx0, mx1)) * scale_log2, m, lsum, oacc);
}

// Kernel body.  NWR waves of 32 rows each share a block of 32*NWR query rows; with SP == 2
// a second set of NWR waves takes the lower half of the block's key tiles (an in-workgroup
// key split, for grids too small to fill the chip: it halves the longest chain of tiles) and
// the two partial softmax states are merged through LDS at the end.  Each split has its own
// copy of every LDS stage.
//
// PRUNE (gate-aware tile skipping, SP == 1 only): knorm holds the largest key norm of every
// 64-key tile.  Walking down from the diagonal, a wave stops once, for each of its rows,
//   scale * |q_i| * max_j |k_j| * log2 e + R_{j1} * log2 e < m_i - (25 + log2 n),
// where j1 is the highest key of the tile: every remaining score is then below the running
// max by more than that, so all remaining keys together weigh less than 2^-24 of the row sum
// (Cauchy-Schwarz on q.k; R_j grows with j).  The workgroup leaves the loop when all its
// waves have stopped.  Results then equal the full computation to fp32 rounding.
//
// CAUSAL == false (the module's default, unmasked mode): every row attends to every key; the
// gate sums are taken relative to the last row of the sequence (R_j = sum_{t=j+1..n-1} log f_t,
// so c_i - c_j = R_j - R_i still holds, with R_j >= 0 past the row), the walk starts at the
// last key tile, where each row's largest bias lies, and only keys past n are masked.
template <int D, int NWR, int SP, bool PRUNE, bool CAUSAL, bool TM>
__device__ __forceinline__ void fwd_pipe_body(Bf16Stage<D>* s0, Bf16Stage<D>* s1, Bf16Stage<D>* s2,
                                              Bf16Stage<D>* s3, float (*g0)[kBC], float (*g1)[kBC],
                                              float (*g2)[kBC], float (*g3)[kBC], GateRows& rows,
                                              const bf16* __restrict__ q, const bf16* __restrict__ k,
                                              const bf16* __restrict__ v, const float* __restrict__ logf,
                                              bf16* __restrict__ o, float* __restrict__ lse,
                                              float* __restrict__ c_out, int n, float scale_log2,
                                              const float* __restrict__ knorm, const FwdLayout& lay) {
  constexpr int NS = 4;  // LDS stages: tile t+1 (V still read), tile t, two tiles in flight
  using G = Bf16Geom<D, NWR>;
  constexpr int KK = D / 16, DB = D / 32, BR = G::BR;
  static_assert(SP == 1 || SP == 2, "key splits");
  static_assert(!PRUNE || SP == 1, "pruning runs without the key split");
  static_assert(!PRUNE || CAUSAL, "pruning bounds the keys below the diagonal");

  const int bh = blockIdx.x;
  const int qb = gridDim.y - 1 - blockIdx.y;
  const int row0 = qb * BR;
  const int ref = min(row0 + BR - 1, n - 1);  // the block's last row
  const int fref = CAUSAL ? ref : n - 1;      // frame row of the gate sums
  const int kt_hi = fref / kBC;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rw = wave % NWR;                                    // row-wave
  const int sp = __builtin_amdgcn_readfirstlane(wave / NWR);  // key split (wave-uniform: LDS DMA bases)
  const int l32 = lane & 31, hi = lane >> 5;
  // TM: token-major strides from `lay`; otherwise the head-major ones as compile-time constants
  const int bb = bh / lay.nh, hh = bh - bb * lay.nh;
  const size_t base = TM ? (size_t)bb * lay.bs + (size_t)hh * lay.hs : (size_t)bh * n * D;  // q/k/v/o
  const size_t gbase = TM ? (size_t)bb * lay.gbs + (size_t)hh * lay.ghs : (size_t)bh * n;  // gates/lse/c
  const int rs = TM ? lay.rs : D, gs = TM ? lay.gs : 1;
  const bf16* kb = k + base;
  const bf16* vb = v + base;
  const float* lfb = logf + gbase;

  // Key tiles of this wave's split: [bot, top].  Split 0 keeps the diagonal tiles (at least
  // the top two, which hold every row's diagonal) and the upper half of the rest.
  const int ntiles = kt_hi + 1;
  const int n0 = (SP == 1 || ntiles <= 2) ? ntiles : max(2, (ntiles + 1) / 2);
  const int top = sp == 0 ? kt_hi : kt_hi - n0;
  const int bot = sp == 0 ? kt_hi - n0 + 1 : 0;
  const bool lead = rw == sp;  // loads the split's gates and runs its gate scan (on distinct SIMDs)

  const int wrow0 = row0 + rw * 32;
  const bool active = wrow0 < n;
  int kt_first = !active ? -1 : (sp == 0 && CAUSAL ? min(wrow0 + 31, n - 1) / kBC : top);
  // Opaque to the optimiser: with every wave starting at the split's top tile (unmasked mode)
  // it would otherwise specialise the first unrolled step and run out of registers.
  __asm__ volatile("" : "+v"(kt_first));
  const int my_row = wrow0 + l32;
  LaneOffsets<D> off = lane_offsets<D>(lane);
  off.k += (uint32_t)(sp * sizeof(Bf16Stage<D>));  // 1 KB multiple: the XOR swizzles still apply
  off.v += (uint32_t)(sp * sizeof(Bf16Stage<D>));
  const StageOffsets<D, NWR> so = stage_offsets<D, NWR>(rw, lane, rs);
  // The resources end at the last row's last byte: rows at or past n read as zeros.
  const uint32_t kv_bytes = (uint32_t)(((size_t)(n - 1) * rs + D) * sizeof(bf16));
  const u32x4 rk = raw_rsrc(kb, kv_bytes);
  const u32x4 rv = raw_rsrc(vb, kv_bytes);
  const u32x4 rl = raw_rsrc(lfb, (uint32_t)(((size_t)(n - 1) * gs + 1) * sizeof(float)));

  auto stage = [&](auto J) -> Bf16Stage<D>* {
    constexpr int j = decltype(J)::value % NS;
    if constexpr (j == 0) return s0;
    else if constexpr (j == 1) return s1;
    else if constexpr (j == 2) return s2;
    else return s3;
  };
  auto gates = [&](auto J) -> float* {
    constexpr int j = decltype(J)::value % NS;
    if constexpr (j == 0) return g0[sp];
    else if constexpr (j == 1) return g1[sp];
    else if constexpr (j == 2) return g2[sp];
    else return g3[sp];
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  bf16x8 qreg[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    if (my_row < n)
      qreg[kk] = *reinterpret_cast<const bf16x8*>(q + base + (size_t)my_row * rs + 16 * kk + 8 * hi);
    else
      qreg[kk] = bf16x8{};
  }

  // Pruning: scale log2 e |q_i| of the lane's row (kept in LDS: the d = 128 schedule has
  // no VGPR to spare), the largest key norm below the block, the margin, stop markers.
  __shared__ float qn_lds[PRUNE ? 64 * NWR * SP : 1];
  if constexpr (PRUNE) {
    float qn = 0.0f;
    float ss = 0.0f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf((float)qreg[kk][e], (float)qreg[kk][e], ss);
    qn = scale_log2 * sqrtf(pair32_sum(ss));  // scale * log2 e * |q_i|
    qn_lds[tid] = qn;
    if (wave == 0) {
      const int nt = (n + kBC - 1) / kBC;
      float km = 0.0f;
      for (int t = lane; t <= kt_hi; t += 64) km = fmaxf(km, knorm[(size_t)bh * nt + t]);
#pragma unroll
      for (int o2 = 32; o2 >= 1; o2 >>= 1) km = fmaxf(km, __shfl_xor(km, o2));
      if (lane == 0) {
        rows.kmax = km;
        rows.prune_t = 25.0f + log2_hw((float)n);
      }
    }
    if (tid < 16) rows.done_it[tid] = (tid >= NWR || row0 + 32 * tid >= n) ? -1 : 0x7FFFFFFF;
  }
  bool wdone = false;

  // Gate sums start at 0 above each split's first tile.  For split 0 that tile holds ref, so
  // its frame is the true one; split 1's sums miss the gates of split 0's keys, a constant
  // that shifts all of split 1's scores alike and is added back to its max at the merge.
  double carry = 0.0;

  // Prologue: the log gates of tiles top, top-1 and top-2, then the K/V of tiles top and top-1 (the
  // i-th tile of the split lives in stage i % 4; the loop issues the K/V of tile kt-2 and the gates
  // of tile kt-3 while computing tile kt, whose lead wave scans the gates of tile kt-2).  The lead
  // wave scans the first two tiles' gates as soon as those have landed, while the K/V loads are
  // still in flight.
  using I2 = std::integral_constant<int, 2>;
  if (lead) {
    if (top >= bot) bf16_stage_gates(stage(I0{})[sp].lf, rl, top, gs);
    if (top - 1 >= bot) bf16_stage_gates(stage(I1{})[sp].lf, rl, top - 1, gs);
    if (top - 2 >= bot) bf16_stage_gates(stage(I2{})[sp].lf, rl, top - 2, gs);
  }
  if (top >= bot)
    bf16_stage_tile<D, NWR>(stage(I0{})[sp], stage(I0{})[sp].lf, rk, rv, rl, so, top, rw, lane, false, rs, gs);
  if (top - 1 >= bot)
    bf16_stage_tile<D, NWR>(stage(I1{})[sp], stage(I1{})[sp].lf, rk, rv, rl, so, top - 1, rw, lane, false, rs, gs);

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  f32x16 sa[2], sb[2];  // scores of the tiles at even / odd loop positions
  sa[0] = sa[1] = sb[0] = sb[1] = f32x16{};
  float m = 0.0f, lsum = 0.0f;  // m: running max of the base-2 scores
  // Stored biases R_j / scale: with an accumulator a = q.k + R_j / scale, the base-2 score is
  // a * scale_log2 (the unit is taken against the fp32 scale_log2 that multiplies it).
  const double bias_unit = kLog2ed / (double)scale_log2;
  auto gate_in = [&](const float* lf, int t, int ln) {
    return (t * kBC + 63 - ln <= fref) ? lf[63 - ln] : 0.0f;
  };
  if (lead && top >= bot) {
    // the gates of tiles top and top-1 have landed once at most the gates of top-2 and the K/V
    // loads issued after them remain
    if (top - 2 >= bot) wait_vmcnt<1 + 4 * G::OPS>();
    else if (top - 1 >= bot) wait_vmcnt<4 * G::OPS>();
    else wait_vmcnt<2 * G::OPS>();
    gate_tile(gates(I0{}), nullptr, rows, lane, top, row0, ref, gate_in(stage(I0{})[sp].lf, top, lane), carry,
              bias_unit);
    if (top - 1 >= bot)
      gate_tile(gates(I1{}), nullptr, rows, lane, top - 1, row0, ref, gate_in(stage(I1{})[sp].lf, top - 1, lane),
                carry, bias_unit);
  }
  wait_vmcnt<0>();

  // Pruning test for tile kt (and so every tile below it), wave-uniform.
  auto prune_stop = [&](int kt, const float* r2t) -> bool {
    (void)kt;
    const float bound = qn_lds[tid] * rows.kmax + r2t[kBC - 1] * scale_log2 + rows.prune_t;
    const bool ok = my_row >= n || bound < m;
    return __ballot(!ok) == 0;
  };
  // Position i of the split's tile sequence: tile kt = top - i.
  auto step = [&](auto J, int i) {
    constexpr int j = decltype(J)::value;
    using JP = std::integral_constant<int, j + NS - 1>;  // position of tile kt+1
    using JN = std::integral_constant<int, j + 2>;       // position of tiles kt+2 / kt-2
    using J1 = std::integral_constant<int, j + 1>;       // position of tile kt-1
    using J3 = std::integral_constant<int, j + 3>;       // position of tile kt-3 (stage of kt+1)
    f32x16(&sc)[2] = (j & 1) ? sb : sa;
    f32x16(&sp_)[2] = (j & 1) ? sa : sb;
    const int kt = top - i;
    const int ln = opaque_lane(lane);  // per-tile copy: keeps stage addresses out of the loop-invariant set
    // Own loads of tile kt, and the lead's gate load of tile kt-2 (issued before tile kt-1's K/V),
    // are complete once at most the K/V loads of tile kt-1 remain.
    if (kt - 1 >= bot) wait_vmcnt<2 * G::OPS>();
    else wait_vmcnt<0>();
    barrier_lds();  // tiles kt, kt-1 and their gate sums visible; every wave is done with tile kt+2's stage
    if constexpr (PRUNE) {
      // Leave when every wave stopped before this position (those marks are all visible now;
      // a mark set during this position would read as "running" to every wave alike).
      bool all = true;
#pragma unroll
      for (int w = 0; w < NWR; ++w) all = all && rows.done_it[w] < i;
      if (all) return true;
    }
    // Token-major: the lane offsets are recomputed from this step's opaque lane copy (with a
    // run-time row stride the compiler would rather keep them live, and spill them).
    // (Tile kt+1's stage holds tile kt-3's gates: its own were scanned three steps ago.)
    if (lead && kt - 3 >= bot) bf16_stage_gates(stage(J3{})[sp].lf, rl, kt - 3, gs);
    if (kt - 2 >= bot)
      bf16_stage_tile<D, NWR>(stage(JN{})[sp], stage(JN{})[sp].lf, rk, rv, rl,
                              TM ? stage_offsets<D, NWR>(rw, ln, rs) : so, kt - 2, rw, lane, false, rs, gs);
    // The lead wave's gate scan of tile kt-2 rides in its steady-state schedule when it has one
    // (tile kt-1's biases, scanned in the previous step, are what this step's P.V slots load).
    const bool gate_job = lead && kt - 2 >= bot;
    bool gate_done = false;
    const GateJob gj = {stage(JN{})[sp].lf, gates(JN{}), kt - 2, row0, ref, fref, &rows, &carry, bias_unit};
    const bool stop_here = PRUNE && active && !wdone && kt < kt_first && kt >= bot && prune_stop(kt, gates(J));
    if (active && kt >= bot && kt <= kt_first && !wdone) {
      if (kt == kt_first) {  // first tile of this wave: nothing to overlap with
        pipe_qk<D>(stage(J)[0], off.k, qreg, gates(J), ln >> 5, sc);
        // split 0's first tile holds the row's diagonal (causal) or the end of the sequence
        m = sp == 0 ? pipe_scores<true>(sc, kt * kBC, CAUSAL ? my_row : n - 1, ln >> 5, scale_log2)
                    : pipe_scores<false>(sc, 0, 0, ln >> 5, scale_log2);
        // the next tile's bias tuples into the next step's accumulators
        sp_[0] = pipe_bias(gates(J1{}), 0, ln >> 5);
        sp_[1] = pipe_bias(gates(J1{}), 1, ln >> 5);
      } else if (gate_job) {
        pipe_steady<D, true>(stage(J)[0], gates(J1{}), stage(JP{})[0], off, qreg, sp_, sc, oacc, m, lsum, ln,
                             scale_log2, gj);
        gate_done = true;
      } else {
        pipe_steady<D, false>(stage(J)[0], gates(J1{}), stage(JP{})[0], off, qreg, sp_, sc, oacc, m, lsum, ln,
                              scale_log2, gj);
      }
      // With pruning, a wave whose remaining keys (tile kt and below) are all negligible still
      // finishes tile kt (same code path) and then stops.
      if (PRUNE && kt != kt_first && stop_here) {
        wdone = true;
        if (lane == 0) rows.done_it[wave] = i;
      }
      if (kt == bot || wdone) {  // drain: probabilities and P.V of the split's last tile
        bf16x8 p[4];
        pipe_probs(sc, m, scale_log2, p);
        pipe_pv<D>(stage(J)[0], off.v, p, oacc);
        lsum = pipe_psum(p, lsum);
      }
    }
    // Otherwise the lead wave runs it here (read by everyone after the next barrier).
    if (gate_job && !gate_done)
      gate_tile(gates(JN{}), nullptr, rows, ln, kt - 2, row0, ref, gate_in(stage(JN{})[sp].lf, kt - 2, ln), carry,
                bias_unit);
    return false;
  };

  for (int i = 0; i < n0; i += NS) {
    if (step(I0{}, i) || i + 1 >= n0) break;
    if (step(I1{}, i + 1) || i + 2 >= n0) break;
    if (step(std::integral_constant<int, 2>{}, i + 2) || i + 3 >= n0) break;
    if (step(std::integral_constant<int, 3>{}, i + 3)) break;
  }
  if constexpr (PRUNE) wait_vmcnt<0>();  // an early exit leaves tile loads in flight

  // ---- epilogue: merge the splits, O = acc / l, lse, c ---------------------------------
  if (SP == 2 && sp == 0 && lead && lane == 0) rows.csplit = carry;  // split 0's gate total
  double cref_fix = 0.0;  // split 1's frame offset, when tile 0 (which sets cref) was split 1's
  if constexpr (SP == 2) {
    // Split 1 leaves (O, m, l) in LDS in its own lane layout, 16 bytes per lane and write; the
    // split-0 wave of the same rows reads the same lane's values.  The buffers sit in the two
    // stages that no wave touches after the last loop position's barrier (those of positions
    // n0 and n0 + 1, mod 4: no such tiles), so split 1 writes them without waiting for split
    // 0: row-wave r takes stage (n0 + r / 2) mod 4 of split r mod 2.
    constexpr int NQD = 4 * DB;  // float4 quads of O per lane; one more holds (m, l)
    static_assert((NQD + 1) * 64 * sizeof(f32x4) <= sizeof(Bf16Stage<D>) && NWR <= 4, "merge buffer");
    const int fs = (n0 + (rw >> 1)) & 3;
    Bf16Stage<D>* sr = (fs == 0 ? s0 : fs == 1 ? s1 : fs == 2 ? s2 : s3) + (rw & 1);
    f32x4* cb = reinterpret_cast<f32x4*>(sr);
    if (sp == 1) {
      const bool worked = active && top >= bot;
#pragma unroll
      for (int qd = 0; qd < NQD; ++qd) {
        const int db = qd >> 2, r = 4 * (qd & 3);
        cb[qd * 64 + lane] = f32x4{oacc[db][r], oacc[db][r + 1], oacc[db][r + 2], oacc[db][r + 3]};
      }
      cb[NQD * 64 + lane] = f32x4{worked ? m : kNegInf, lsum, 0.0f, 0.0f};  // split 1's frame
    }
    __syncthreads();  // partials, csplit, cref and the row sums are visible
    if (sp == 1) return;
    const double csplit = rows.csplit;
    if (kt_hi >= n0) cref_fix = csplit;  // tile 0 was split 1's: its total misses split 0's keys
    if (active) {
      const f32x4 ml = cb[NQD * 64 + lane];
      // back to the true frame: split 1's scores were high by -csplit * log2 e
      const float m1 = ml[0] + (float)(csplit * kLog2ed);
      const float mm = fmaxf(m, m1);
      const float a0 = exp2_hw(m - mm), a1 = exp2_hw(m1 - mm);
      lsum = lsum * a0 + ml[1] * a1;
#pragma unroll
      for (int qd = 0; qd < NQD; ++qd) {
        const f32x4 x = cb[qd * 64 + lane];
        const int db = qd >> 2, r = 4 * (qd & 3);
#pragma unroll
        for (int e = 0; e < 4; ++e) oacc[db][r + e] = oacc[db][r + e] * a0 + x[e] * a1;
      }
      m = mm;
    }
  } else {
    __syncthreads();  // rows / cref written by the lead wave are visible
  }
  if (!active) return;
  const float ltot = pair32_sum(lsum);
  if (my_row >= n) return;
  // The gate sums of the row are read before the output math so their latency overlaps it.
  // Rows in split 1's key range (unmasked mode only) got R_i in split 1's frame, which misses
  // the gates of split 0's keys.
  double ri = rows.rowR[my_row - row0];
  if (SP == 2 && !CAUSAL && my_row / kBC <= kt_hi - n0) ri += rows.csplit;
  const double cref = rows.cref + cref_fix;
  const float inv = 1.0f / ltot;
  // All packed words first, then the stores back to back (no store waits on a register
  // that the previous store still has to read).
  u32x2 w[DB * 4];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      w[db * 4 + g][0] = pack_bf16x2(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv);
      w[db * 4 + g][1] = pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
    }
  }
  bf16* orow = o + base + (size_t)my_row * rs;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * g + 4 * hi) = w[db * 4 + g];
  if (hi == 0) {
    const size_t idx = gbase + (size_t)my_row * gs;
    if (lse) lse[idx] = (float)(((double)m + (double)log2_hw(ltot)) * kLn2d - ri);
    if (c_out) c_out[idx] = (float)(cref - ri);
  }
}

// Waves per SIMD the register budget is set for: two, except the 4-wave blocks at d = 128, whose
// VGPR-form MFMAs need more than 256 registers (one wave per SIMD).
template <int D, int NWR>
constexpr int kFwdWavesPerSimd = D == 128 && NWR == 4 ? 1 : 2;

template <int D, int NWR, int SP, bool PRUNE, bool CAUSAL, bool TM>
__global__ __launch_bounds__(64 * NWR * SP) __attribute__((amdgpu_waves_per_eu(
    kFwdWavesPerSimd<D, NWR>, kFwdWavesPerSimd<D, NWR>))) void fwd_bf16_pipe_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ logf, bf16* __restrict__ o, float* __restrict__ lse, float* __restrict__ c_out, int n,
    float scale_log2, const float* __restrict__ knorm, const FwdLayout lay) {
  __shared__ GateRows rows;
  __shared__ Bf16Stage<D> s0[SP], s1[SP], s2[SP], s3[SP];
  __shared__ float g0[SP][kBC], g1[SP][kBC], g2[SP][kBC], g3[SP][kBC];
  fwd_pipe_body<D, NWR, SP, PRUNE, CAUSAL, TM>(s0, s1, s2, s3, g0, g1, g2, g3, rows, q, k, v, logf, o, lse, c_out,
                                               n, scale_log2, knorm, lay);
}

// Largest L2 norm of the keys of every 64-key tile (pruning bound); keys past n count as 0.
template <int D>
__global__ __launch_bounds__(256) void key_tile_norm_kernel(const bf16* __restrict__ k, float* __restrict__ kn, int n) {
  // One wave per 64-key tile.  A wave-wide load covers 64 consecutive 16-byte chunks, i.e.
  // 64/(D/8) whole keys, so every load instruction reads one contiguous 1 KiB span.
  constexpr int LPK = D / 8;        // lanes per key
  constexpr int KPL = 64 / LPK;     // keys per load
  const int nt = (n + kBC - 1) / kBC;
  const int t = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const size_t bh = blockIdx.y;
  if (t >= nt) return;
  const int sub = lane / LPK, chunk = lane % LPK;
  float nm = 0.0f;
#pragma unroll
  for (int r = 0; r < kBC / KPL; ++r) {
    const int key = t * kBC + r * KPL + sub;
    float ss = 0.0f;
    if (key < n) {
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(k + (bh * n + key) * D + 8 * chunk);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf((float)x[e], (float)x[e], ss);
    }
#pragma unroll
    for (int o2 = LPK / 2; o2 >= 1; o2 >>= 1) ss += __shfl_xor(ss, o2);
    nm = fmaxf(nm, ss);
  }
#pragma unroll
  for (int o2 = 32; o2 >= LPK; o2 >>= 1) nm = fmaxf(nm, __shfl_xor(nm, o2));
  if (lane == 0) kn[bh * nt + t] = sqrtf(nm);
}

// Kernel choice for the bf16 forward (knorm != nullptr selects the pruned, causal kernels):
//  * 256-row blocks (8 waves) stage each K/V tile for twice the compute of 128-row blocks,
//    halving the L2 -> LDS traffic per flop; used when there are enough blocks to keep every
//    CU busy for two rounds;
//  * d <= 64 with fewer than two 128-row blocks per CU: 128-row blocks whose key tiles are
//    split over two wave sets;
//  * otherwise 128-row blocks of 4 waves.
template <int D, bool CAUSAL, bool TM>
hipError_t launch_fwd_t(const void* q, const void* k, const void* v, const float* logf, void* o, float* lse,
                        float* c, int64_t bh, int n, float scale_log2, const float* knorm, const FwdLayout& lay,
                        hipStream_t stream) {
  int cus = 256, dev = 0;
  if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int64_t blocks256 = bh * (int64_t)((n + 255) / 256);
  const int64_t blocks128 = bh * (int64_t)((n + 127) / 128);
  const bf16 *qq = (const bf16*)q, *kk = (const bf16*)k, *vv = (const bf16*)v;
  bf16* oo = (bf16*)o;
  auto go = [&](auto kernel, int rows, int threads) {
    const dim3 grid((unsigned)bh, (unsigned)((n + rows - 1) / rows));
    hipLaunchKernelGGL(kernel, grid, dim3(threads), 0, stream, qq, kk, vv, logf, oo, lse, c, n, scale_log2, knorm,
                       lay);
    return hipGetLastError();
  };
  constexpr bool CAN_PRUNE = CAUSAL && !TM;
  if constexpr (D >= 64) {
    if (blocks256 >= 2 * (int64_t)cus) {
      if constexpr (CAN_PRUNE)
        if (knorm) return go(fwd_bf16_pipe_kernel<D, 8, 1, true, true, false>, 256, 512);
      return go(fwd_bf16_pipe_kernel<D, 8, 1, false, CAUSAL, TM>, 256, 512);
    }
  }
  if constexpr (D <= 64) {
    // Unmasked blocks all do the same work: once they need a second round of 8-wave workgroups,
    // 4-wave workgroups (two per CU, one round) finish first.
    if (!knorm && blocks128 < 2 * (int64_t)cus && (CAUSAL || blocks128 <= (int64_t)cus))
      return go(fwd_bf16_pipe_kernel<D, 4, 2, false, CAUSAL, TM>, 128, 512);
  }
  if constexpr (CAN_PRUNE)
    if (knorm) return go(fwd_bf16_pipe_kernel<D, 4, 1, true, true, false>, 128, 256);
  return go(fwd_bf16_pipe_kernel<D, 4, 1, false, CAUSAL, TM>, 128, 256);
}

template <bool CAUSAL, bool TM>
hipError_t launch_fwd_l(const void* q, const void* k, const void* v, const float* logf, void* o, float* lse, float* c,
                        int64_t bh, int n, int d, float scale_log2, bool is_bf16, const FwdLayout& lay,
                        const float* knorm, hipStream_t stream) {
  if (!is_bf16)
    return launch_fwd_f32((const float*)q, (const float*)k, (const float*)v, logf, (float*)o, lse, c, bh, n, d,
                          scale_log2, CAUSAL, TM, lay, stream);
  switch (d) {
    case 32: return launch_fwd_t<32, CAUSAL, TM>(q, k, v, logf, o, lse, c, bh, n, scale_log2, knorm, lay, stream);
    case 64: return launch_fwd_t<64, CAUSAL, TM>(q, k, v, logf, o, lse, c, bh, n, scale_log2, knorm, lay, stream);
    case 128: return launch_fwd_t<128, CAUSAL, TM>(q, k, v, logf, o, lse, c, bh, n, scale_log2, knorm, lay, stream);
  }
  return hipErrorInvalidValue;
}

template <bool CAUSAL>
hipError_t launch_fwd_d(const void* q, const void* k, const void* v, const float* logf, void* o, float* lse, float* c,
                        int64_t b, int64_t h, int n, int d, float scale, bool is_bf16, bool token_major,
                        const float* knorm, hipStream_t stream) {
  const float scale_log2 = (float)((double)scale * kLog2ed);
  const int64_t bh = b * h;
  // {bs, hs, rs, gbs, ghs, gs, nh}
  const FwdLayout lay = token_major
                            ? FwdLayout{(int64_t)n * h * d, (int64_t)d, (int)(h * d), (int64_t)n * h, 1, (int)h, (int)h}
                            : FwdLayout{h * n * (int64_t)d, (int64_t)n * d, d, h * (int64_t)n, (int64_t)n, 1, (int)h};
  return token_major
             ? launch_fwd_l<CAUSAL, true>(q, k, v, logf, o, lse, c, bh, n, d, scale_log2, is_bf16, lay, knorm, stream)
             : launch_fwd_l<CAUSAL, false>(q, k, v, logf, o, lse, c, bh, n, d, scale_log2, is_bf16, lay, knorm, stream);
}

template <int D>
hipError_t launch_key_norm_t(const void* k, float* kn, int64_t bh, int n, hipStream_t stream) {
  const int nt = (n + kBC - 1) / kBC;
  const dim3 grid((unsigned)((nt + 3) / 4), (unsigned)bh);
  hipLaunchKernelGGL(key_tile_norm_kernel<D>, grid, dim3(256), 0, stream, (const bf16*)k, kn, n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const void* q, const void* k, const void* v, const float* logf, void* o, float* lse,
                           float* c, int64_t b, int64_t h, int n, int d, float scale, bool is_bf16, bool causal,
                           bool token_major, hipStream_t stream) {
  return causal ? launch_fwd_d<true>(q, k, v, logf, o, lse, c, b, h, n, d, scale, is_bf16, token_major, nullptr, stream)
                : launch_fwd_d<false>(q, k, v, logf, o, lse, c, b, h, n, d, scale, is_bf16, token_major, nullptr,
                                      stream);
}

size_t attn_fwd_pruned_workspace_bytes(int64_t bh, int n) {
  return (size_t)bh * (size_t)((n + kBC - 1) / kBC) * sizeof(float);
}

hipError_t launch_attn_fwd_pruned(const void* q, const void* k, const void* v, const float* logf, void* o,
                                  float* lse, float* c, float* workspace, int64_t bh, int n, int d, float scale,
                                  bool is_bf16, hipStream_t stream) {
  if (!is_bf16)  // the fp32 path is not pruned: it computes every causal pair
    return launch_attn_fwd(q, k, v, logf, o, lse, c, bh, 1, n, d, scale, false, true, false, stream);
  hipError_t e = hipSuccess;
  switch (d) {
    case 32: e = launch_key_norm_t<32>(k, workspace, bh, n, stream); break;
    case 64: e = launch_key_norm_t<64>(k, workspace, bh, n, stream); break;
    case 128: e = launch_key_norm_t<128>(k, workspace, bh, n, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  // A pruned workgroup may stop before tile 0, where the kernel would learn c at its last
  // row; c comes from the prefix-sum kernel instead.
  if (c) {
    e = launch_logf_cumsum(logf, c, bh, n, stream);
    if (e != hipSuccess) return e;
  }
  // (batch*head, 1 head): the head-major layout of b*h independent heads
  return launch_fwd_d<true>(q, k, v, logf, o, lse, nullptr, bh, 1, n, d, scale, true, false, workspace, stream);
}

}  // namespace fox
