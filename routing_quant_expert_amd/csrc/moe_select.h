// Top-k selection of one token by one wave64, branch-free
// [moe_v41.rs, fn route_from_logits]:
//   key(e) = score(e) + bias(e) in f32; the k largest keys, equal keys in
//   ascending expert id (the pages' stable sort over ids 0..n-1), NaN keys
//   after every other key; weights = the unbiased scores of the picks in pick
//   order, renormalised by their f32 sum (+1e-20) and scaled by route_scale.
// Keys are compared through their bits mapped to an unsigned order (+0 and
// -0 equal, NaN lowest); the wave maximum is a DPP reduction (no LDS).
#pragma once

#include <hip/hip_runtime.h>

#include "moe_math.h"

namespace moe {

__device__ __forceinline__ uint32_t key_order_bits(float k) {
  if (isnan(k)) return 0u;
  const uint32_t u = __builtin_bit_cast(uint32_t, fadd(k, 0.0f));   // -0 -> +0
  return (u >> 31) ? ~u : (u | 0x80000000u);
}

// Maximum (minimum) of v over the 64 lanes, returned uniformly (from lane
// 63), by a DPP reduction: quad_perm [1,0,3,2], [2,3,0,1], row_shr:4,
// row_shr:8, row_bcast:15, row_bcast:31. Lanes without a source take the
// neutral value (0 for the maximum, all ones for the minimum).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xb1, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4e, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0xb1, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x4e, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x114, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x118, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x142, 0xa, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// This lane's best available key: the largest order bits, and of equal ones
// the smallest column c (expert lane + 64c); bc = -1 when none is left.
template <int KPER>
__device__ __forceinline__ void lane_best(const uint32_t (&ko)[KPER], uint32_t avail, uint32_t& bko, int& bc) {
  bko = 0u;
  bc = -1;
#pragma unroll
  for (int c = KPER - 1; c >= 0; --c) {
    const bool take = ((avail >> c) & 1u) && ko[c] >= bko;
    bko = take ? ko[c] : bko;
    bc = take ? c : bc;
  }
}

// This lane's keys' inputs: scores and bias of experts lane + 64c. Every
// load is issued before any is used (indices clamped, no branches), so a
// wave can issue the loads of several tokens before selecting any of them.
template <int KPER>
__device__ __forceinline__ void select_load(const float* __restrict__ scores, const float* __restrict__ bias,
                                            int n_routed, float (&sc)[KPER], float (&bs)[KPER]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int c = 0; c < KPER; ++c) {
    const int e = min(lane + 64 * c, n_routed - 1);
    sc[c] = scores[e];
    bs[c] = bias[e];
  }
}

// The wave selects `topk` experts from one token's scores (loaded by
// select_load) with bias. On return every lane holds the same picks[] (rank
// order); lane r < topk holds in `weight` the weight of picks[r]; nan_any
// tells whether any key was NaN. KPER = ceil(n_routed/64). Each lane keeps
// its own best available key; a round takes the wave maximum of those, then
// the smallest expert id holding it (a wave minimum over the lanes' best
// ids), which is exactly the pages' stable descending sort. Only the winning
// lane's best changes.
template <int KPER>
__device__ __forceinline__ void select_topk_from(const float (&sc)[KPER], const float (&bs)[KPER], int n_routed,
                                                 int topk, int norm, float route_scale, int (&picks)[kMaxTopk],
                                                 float& weight, bool& nan_any) {
  const int lane = threadIdx.x & 63;
  uint32_t ko[KPER];
  uint32_t avail = 0;                // bit c: expert lane + 64c still available
  bool has_nan = false;
#pragma unroll
  for (int c = 0; c < KPER; ++c) {
    const bool in = lane + 64 * c < n_routed;
    const float k = fadd(sc[c], bs[c]);
    has_nan |= in && isnan(k);
    ko[c] = key_order_bits(k);
    avail |= in ? (1u << c) : 0u;
  }
  nan_any = __any(has_nan);
  uint32_t bko;
  int bc;
  lane_best<KPER>(ko, avail, bko, bc);
  float sraw[kMaxTopk];   // the picks' unbiased scores, uniform
#pragma unroll
  for (int r = 0; r < kMaxTopk; ++r) {
    sraw[r] = 0.0f;
    picks[r] = 0;
    if (r < topk) {
      const uint32_t top = wave_max_u32(bko);
      const uint32_t id = wave_min_u32(bc >= 0 && bko == top ? (uint32_t)(lane + 64 * bc) : 0xFFFFFFFFu);
      const int wl = (int)(id & 63u);
      float s_best = sc[0];
#pragma unroll
      for (int c = 1; c < KPER; ++c) s_best = (c == bc) ? sc[c] : s_best;
      sraw[r] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s_best), wl));
      picks[r] = (int)id;
      if (lane == wl) avail &= ~(1u << bc);
      lane_best<KPER>(ko, avail, bko, bc);
    }
  }
  float w = sraw[0];
#pragma unroll
  for (int r = 1; r < kMaxTopk; ++r) w = (r == lane) ? sraw[r] : w;
  if (norm && topk > 1) {
    float sum = 0.0f;
#pragma unroll
    for (int r = 0; r < kMaxTopk; ++r)
      if (r < topk) sum = fadd(sum, sraw[r]);
    sum = fadd(sum, 1e-20f);
    w = (float)((double)w / (double)sum);
  }
  weight = fmul(w, route_scale);
}

// select_load + select_topk_from for one token's row of scores.
template <int KPER>
__device__ __forceinline__ void select_topk(const float* __restrict__ scores, const float* __restrict__ bias,
                                            int n_routed, int topk, int norm, float route_scale,
                                            int (&picks)[kMaxTopk], float& weight, bool& nan_any) {
  float sc[KPER], bs[KPER];
  select_load<KPER>(scores, bias, n_routed, sc, bs);
  select_topk_from<KPER>(sc, bs, n_routed, topk, norm, route_scale, picks, weight, nan_any);
}

}  // namespace moe
