// fox_device.h -- device-side helpers shared by the libfox kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fox {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr double kLn2d = 0.6931471805599453;
constexpr double kLog2ed = 1.4426950408889634;

// Hardware base-2 exponential / logarithm (v_exp_f32 / v_log_f32).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// v_permlane32_swap with both operands = x: r[0] and r[1] are x of lane l and
// of lane l^32 in some order, so a symmetric op over them reduces the lane pair.
__device__ __forceinline__ float pair32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// DPP lane moves inside 16-lane rows.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// Sum over aligned groups of G consecutive lanes (G in {4, 8, 16, 32}); every lane of
// the group receives the group's sum.  Mirrors pair lanes of the two halves of the
// 8- and 16-lane rows, which for a sum is as good as an xor butterfly.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(G == 4 || G == 8 || G == 16 || G == 32, "group size");
  x += dpp_mov<kDppQuadXor1>(x);
  x += dpp_mov<kDppQuadXor2>(x);
  if constexpr (G >= 8) x += dpp_mov<kDppRowHalfMirror>(x);
  if constexpr (G >= 16) x += dpp_mov<kDppRowMirror>(x);
  if constexpr (G >= 32) x += __shfl_xor(x, 16);
  return x;
}

// Opaque copy of a per-lane value: address arithmetic derived from it cannot be hoisted out
// of the loop that makes the copy (a kernel unrolled over four LDS stages would otherwise
// keep four stages' worth of addresses live in VGPRs).
__device__ __forceinline__ int opaque_lane(int x) {
  __asm__ volatile("" : "+v"(x));
  return x;
}

// Wave-uniform "any lane" vote.
__device__ __forceinline__ bool wave_any(bool p) { return __ballot(p) != 0; }

// bf16 <-> fp32 on packed 32-bit words (low half = even element).
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 p = {(bf16)a, (bf16)b};  // v_cvt_pk_bf16_f32, round to nearest even
  return __builtin_bit_cast(uint32_t, p);
}

// Byte permute: bytes of ((uint64)hi << 32 | lo) picked by `sel` (v_perm_b32).
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}
constexpr uint32_t kSelLoLo = 0x05040100u;  // lo16(lo) | lo16(hi) << 16
constexpr uint32_t kSelHiHi = 0x07060302u;  // hi16(lo) | hi16(hi) << 16

}  // namespace fox

namespace fox {

// Inclusive prefix sum over the 64 lanes of a wave in fp64.  The lane moves are DPP
// (row shifts inside 16-lane rows, then the two row broadcasts of gfx9) applied to the
// two dwords of each double, so the moved values are exact; lanes whose row or bank is
// masked off receive 0.  Only the adds round, as fp64.
template <int CTRL, int ROW_MASK, int BANK_MASK, bool BOUND>
__device__ __forceinline__ double dpp_or_zero(double v) {
  const u32x2 w = __builtin_bit_cast(u32x2, v);
  u32x2 r;
  r[0] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)w[0], CTRL, ROW_MASK, BANK_MASK, BOUND);
  r[1] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)w[1], CTRL, ROW_MASK, BANK_MASK, BOUND);
  return __builtin_bit_cast(double, r);
}

// Step k (1..7) of the inclusive scan below, on (x, y) = (lane value, partial scan); the
// steps can be issued separately (interleaved with other work) as long as they stay in order.
__device__ __forceinline__ void wave_scan_step(int k, double x, double& y) {
  switch (k) {
    case 1: y = x + dpp_or_zero<0x111, 0xF, 0xF, true>(x); break;  // row_shr:1
    case 2: y += dpp_or_zero<0x112, 0xF, 0xF, true>(x); break;     // row_shr:2
    case 3: y += dpp_or_zero<0x113, 0xF, 0xF, true>(x); break;     // row_shr:3   -> sums of 4 within the row
    case 4: y += dpp_or_zero<0x114, 0xF, 0xE, true>(y); break;     // row_shr:4 on banks 1..3
    case 5: y += dpp_or_zero<0x118, 0xF, 0xC, true>(y); break;     // row_shr:8 on banks 2..3 -> row-local scan
    case 6: y += dpp_or_zero<0x142, 0xA, 0xF, false>(y); break;    // row_bcast:15 into rows 1 and 3
    case 7: y += dpp_or_zero<0x143, 0xC, 0xF, false>(y); break;    // row_bcast:31 into rows 2 and 3
    default: break;
  }
}

__device__ __forceinline__ double wave_incl_scan(double x) {
  double y = 0.0;
#pragma unroll
  for (int k = 1; k <= 7; ++k) wave_scan_step(k, x, y);
  return y;
}

// Value of lane l-1 (0 in lane 0): wave_shr:1.
__device__ __forceinline__ double wave_shr1(double x) { return dpp_or_zero<0x138, 0xF, 0xF, true>(x); }

// Value of lane 63, in every lane.
__device__ __forceinline__ double wave_last(double x) {
  const u32x2 w = __builtin_bit_cast(u32x2, x);
  u32x2 r;
  r[0] = (uint32_t)__builtin_amdgcn_readlane((int)w[0], 63);
  r[1] = (uint32_t)__builtin_amdgcn_readlane((int)w[1], 63);
  return __builtin_bit_cast(double, r);
}

}  // namespace fox
