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
