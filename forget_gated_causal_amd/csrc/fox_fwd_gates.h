// fox_fwd_gates.h -- pieces of the forward shared by its bf16 kernels (fox_fwd.hip) and its fp32
// kernel (fox_fwd_f32.hip): tile constants, the per-workgroup gate rows, the fp64 gate-sum scan of
// one key tile, and the tensor strides of a call.
#pragma once

#include <math.h>

#include "fox_device.h"

namespace fox {

// Element strides of one forward call.  Head-major: q/k/v/o [B,H,N,d], gates / lse / c [B,H,N]
// (rows d apart).  Token-major: q/k/v/o [B,N,H,d], gates / lse / c [B,N,H] (rows h*d apart),
// the layout the projections produce before the head permute.
struct FwdLayout {
  int64_t bs, hs;    // q/k/v/o: batch and head strides
  int rs;            // q/k/v/o: row (token) stride
  int64_t gbs, ghs;  // gates, lse, c: batch and head strides
  int gs;            // gates, lse, c: row stride
  int nh;            // heads per batch entry
};

// The fp32 forward (fox_fwd_f32.hip): d in {32, 64, 128}; scale_log2 = scale * log2 e.
hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, const float* logf, float* o, float* lse,
                          float* c, int64_t bh, int n, int d, float scale_log2, bool causal, bool token_major,
                          const FwdLayout& lay, hipStream_t stream);

namespace {

constexpr int kMaxBR = 256;    // largest query block (bf16, 8 waves)
constexpr int kBC = 64;       // keys per tile
constexpr float kTau = 8.0f;  // lazy-rescale threshold, log2 units
constexpr float kNegInf = -INFINITY;

struct GateRows {          // per workgroup
  double rowR[kMaxBR + 1]; // R_i for the block's own rows; the last slot takes discarded writes
  double cref;             // c at the frame row of the gate sums (sum of log f up to it)
  double cref_discard;     // takes the cref write of tiles other than tile 0
  double csplit;           // key split: sum of log f over split 0's keys (split 1's frame offset)
  float kmax;              // pruning: largest key norm of the block's key range
  float prune_t;           // pruning: margin 25 + log2 n (base-2 units)
  int done_it[16];         // pruning: loop position at which each wave stopped (INT_MAX: still running)
};

// Wave 0: gate sums for tile kt.  Lane t holds log f of key 63-t of the tile (0 beyond
// ref), so the lane-order exclusive prefix is the key-order exclusive suffix
// sum_{u > j} log f_u inside the tile.  `carry` (fp64) is the sum of log f over
// (tile end, ref] and is advanced by the tile total.  Writes R_j = carry + suffix for
// the tile (r2 = R_j * unit in fp32; r64 = R_j, when given), R_i for the block's own
// rows and, after tile 0, c at the reference row.  Everything is fp64 until the single
// rounding to fp32.
__device__ __forceinline__ void gate_finish(double incl, float* r2, double* r64, GateRows& rows, int lane, int kt,
                                            int row0, int ref, double& carry, double unit) {
  const double excl = wave_shr1(incl);
  const int jl = 63 - lane;
  const double rj = carry + excl;
  r2[jl] = (float)(rj * unit);
  if (r64) r64[jl] = rj;
  // Branch-free writes (this code also runs inside the MFMA schedule): rows outside the
  // block and tiles other than tile 0 write to discard slots.
  const int j = kt * kBC + jl;
  rows.rowR[(j >= row0 && j <= ref) ? j - row0 : kMaxBR] = rj;
  carry += wave_last(incl);
  *(kt == 0 ? &rows.cref : &rows.cref_discard) = carry;
}
__device__ __forceinline__ void gate_tile(float* r2, double* r64, GateRows& rows, int lane, int kt, int row0,
                                          int ref, float lf_rev, double& carry, double unit) {
  gate_finish(wave_incl_scan((double)lf_rev), r2, r64, rows, lane, kt, row0, ref, carry, unit);
}

// The gate sums of one tile as a job that a wave can spread over its MFMA schedule.
struct GateJob {
  const float* lf;  // the tile's staged log gates
  float* r2;        // its biases R_j * unit (out)
  int kt;           // tile index
  int row0, ref;    // the block's first and last rows (R_i of these rows is kept)
  int fref;         // frame row: gates past it do not enter the sums
  GateRows* rows;
  double* carry;
  double unit;      // R_j -> stored bias
};

}  // namespace
}  // namespace fox
