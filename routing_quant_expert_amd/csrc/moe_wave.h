// Cross-lane reductions of one wave64 without the LDS crossbar: the gfx950
// permlane swaps move whole 32- and 16-lane halves between two registers,
// DPP moves lanes inside a 16-lane row. A shuffle through ds_bpermute costs
// about 90 cycles per step on this chip, a permlane swap about 30 and a DPP
// operand about 14, so a 64-lane butterfly drops from about 430 cycles to
// about 110.
//
// wave_sum_xor(v) returns in every lane exactly the value of the xor
// butterfly v += shfl_xor(v, s), s = 32, 16, 8, 4, 2, 1: after each step the
// value depends only on the lane's position inside the block that step has
// summed, so a row rotation by 8 (4, 2, 1) pairs every lane with a lane that
// holds its xor partner's value, and f32 addition is commutative.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// DPP controls: quad_perm [1,0,3,2] (lane ^ 1), quad_perm [2,3,0,1] (lane ^ 2),
// row_ror:4 and row_ror:8 (inside 16-lane rows).
constexpr int kDppXor1 = 0xb1;
constexpr int kDppXor2 = 0x4e;
constexpr int kDppRor4 = 0x124;
constexpr int kDppRor8 = 0x128;

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}

// Lane l gets the values of lanes l and l ^ 32 (swap32) or l and l ^ 16
// (swap16) as (own half's, other half's) in some order; the two results are
// read into named temporaries before any bit cast (a bit cast of the
// builtin's vector element directly has been folded to the wrong element).
__device__ __forceinline__ void swap32(uint32_t x, uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  const uint32_t r0 = r[0], r1 = r[1];
  a = r0;
  b = r1;
}
__device__ __forceinline__ void swap16(uint32_t x, uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  const uint32_t r0 = r[0], r1 = r[1];
  a = r0;
  b = r1;
}

__device__ __forceinline__ float sum_xor32(float v) {
  uint32_t a, b;
  swap32(__builtin_bit_cast(uint32_t, v), a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}
__device__ __forceinline__ float sum_xor16(float v) {
  uint32_t a, b;
  swap16(__builtin_bit_cast(uint32_t, v), a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// The f32 xor butterfly over all 64 lanes (the summation order stated above).
__device__ __forceinline__ float wave_sum_xor(float v) {
  v = sum_xor32(v);
  v = sum_xor16(v);
  v = v + dpp_f32<kDppRor8>(v);
  v = v + dpp_f32<kDppRor4>(v);
  v = v + dpp_f32<kDppXor2>(v);
  v = v + dpp_f32<kDppXor1>(v);
  return v;
}

// The maximum over each aligned group of 32 lanes, in every lane of the group.
__device__ __forceinline__ float max32(float v) {
  v = fmaxf(v, dpp_f32<kDppXor1>(v));
  v = fmaxf(v, dpp_f32<kDppXor2>(v));
  v = fmaxf(v, dpp_f32<kDppRor4>(v));
  v = fmaxf(v, dpp_f32<kDppRor8>(v));
  uint32_t a, b;
  swap16(__builtin_bit_cast(uint32_t, v), a, b);
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}

// The integer sum over each aligned group of 16 lanes, in every lane of the group.
__device__ __forceinline__ int sum16(int v) {
  v += dpp_i32<kDppXor1>(v);
  v += dpp_i32<kDppXor2>(v);
  v += dpp_i32<kDppRor4>(v);
  v += dpp_i32<kDppRor8>(v);
  return v;
}

// f64 halves of the xor butterfly's lane ^ 16 and lane ^ 32 steps.
__device__ __forceinline__ double sum_xor16_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  uint32_t la, lb, ha, hb;
  swap16((uint32_t)u, la, lb);
  swap16((uint32_t)(u >> 32), ha, hb);
  return __builtin_bit_cast(double, ((uint64_t)ha << 32) | la) + __builtin_bit_cast(double, ((uint64_t)hb << 32) | lb);
}
__device__ __forceinline__ double sum_xor32_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  uint32_t la, lb, ha, hb;
  swap32((uint32_t)u, la, lb);
  swap32((uint32_t)(u >> 32), ha, hb);
  return __builtin_bit_cast(double, ((uint64_t)ha << 32) | la) + __builtin_bit_cast(double, ((uint64_t)hb << 32) | lb);
}

// acc + a.lo * b.lo + a.hi * b.hi for two pairs of packed bf16 (v_dot2_f32_bf16):
// two products of the shared expert's f32 sums per instruction, with no
// conversions (those sums are in any order).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// dot2_bf16 over the four words of two 16-byte chunks (8 bf16 each).
__device__ __forceinline__ float dot8_bf16(const uint4& a, const uint4& b, float acc) {
  acc = dot2_bf16(a.x, b.x, acc);
  acc = dot2_bf16(a.y, b.y, acc);
  acc = dot2_bf16(a.z, b.z, acc);
  return dot2_bf16(a.w, b.w, acc);
}

}  // namespace moe
