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

// Maximum of v over the 64 lanes, returned uniformly (from lane 63), by a
// DPP reduction: quad_perm [1,0,3,2], [2,3,0,1], row_shr:4, row_shr:8,
// row_bcast:15, row_bcast:31.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xb1, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4e, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
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
// order) and weights[]; nan_any tells whether any key was NaN.
// KPER = ceil(n_routed/64). A round takes the wave maximum of the available
// keys' order bits, then the smallest id holding that maximum (one ballot per
// register column, in id order), which is exactly the pages' stable
// descending sort.
template <int KPER>
__device__ __forceinline__ void select_topk_from(const float (&sc)[KPER], const float (&bs)[KPER], int n_routed,
                                                 int topk, int norm, float route_scale, int (&picks)[kMaxTopk],
                                                 float (&weights)[kMaxTopk], bool& nan_any) {
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
#pragma unroll
  for (int r = 0; r < kMaxTopk; ++r) {
    if (r < topk) {
      uint32_t best = 0;
#pragma unroll
      for (int c = 0; c < KPER; ++c) best = ((avail >> c) & 1u) ? max(best, ko[c]) : best;
      const uint32_t top = wave_max_u32(best);
      int id = -1;
#pragma unroll
      for (int c = 0; c < KPER; ++c) {
        const unsigned long long b = __ballot(((avail >> c) & 1u) && ko[c] == top);
        if (id < 0 && b) id = 64 * c + __builtin_ctzll(b);
      }
      const int wc = id >> 6, wl = id & 63;
      float s_here = sc[0];
#pragma unroll
      for (int c = 1; c < KPER; ++c) s_here = (c == wc) ? sc[c] : s_here;
      weights[r] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s_here), wl));
      picks[r] = id;
      if (lane == wl) avail &= ~(1u << wc);
    }
  }
  if (norm && topk > 1) {
    float sum = 0.0f;
#pragma unroll
    for (int r = 0; r < kMaxTopk; ++r)
      if (r < topk) sum = fadd(sum, weights[r]);
    sum = fadd(sum, 1e-20f);
#pragma unroll
    for (int r = 0; r < kMaxTopk; ++r)
      if (r < topk) weights[r] = (float)((double)weights[r] / (double)sum);
  }
#pragma unroll
  for (int r = 0; r < kMaxTopk; ++r)
    if (r < topk) weights[r] = fmul(weights[r], route_scale);
}

// select_load + select_topk_from for one token's row of scores.
template <int KPER>
__device__ __forceinline__ void select_topk(const float* __restrict__ scores, const float* __restrict__ bias,
                                            int n_routed, int topk, int norm, float route_scale,
                                            int (&picks)[kMaxTopk], float (&weights)[kMaxTopk], bool& nan_any) {
  float sc[KPER], bs[KPER];
  select_load<KPER>(scores, bias, n_routed, sc, bs);
  select_topk_from<KPER>(sc, bs, n_routed, topk, norm, route_scale, picks, weights, nan_any);
}

}  // namespace moe
