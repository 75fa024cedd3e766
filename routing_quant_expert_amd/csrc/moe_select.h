// Top-k selection of one token by one wave64, branch-free
// [moe_v41.rs, fn route_from_logits]:
//   key(e) = score(e) + bias(e) in f32; the k largest keys, equal keys in
//   ascending expert id (the pages' stable sort over ids 0..n-1), NaN keys
//   after every other key; weights = the unbiased scores of the picks in pick
//   order, renormalised by their f32 sum (+1e-20) and scaled by route_scale.
// Each expert gets a 64-bit composite that orders exactly like that rule:
//   high word: the key's bits mapped to an unsigned order (+0 and -0 equal,
//   NaN lowest), low word: ~id. A round takes the wave maximum of the
//   not-yet-taken composites with a DPP reduction (no LDS traffic).
#pragma once

#include <hip/hip_runtime.h>

#include "moe_math.h"

namespace moe {

__device__ __forceinline__ uint32_t key_order_bits(float k) {
  if (isnan(k)) return 0u;
  const uint32_t u = __builtin_bit_cast(uint32_t, fadd(k, 0.0f));   // -0 -> +0
  return (u >> 31) ? ~u : (u | 0x80000000u);
}

// DPP move of a 32-bit value (bound_ctrl: lanes without a source read 0).
template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, BANK_MASK, false);
}

template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t v) {
  const uint32_t lo = dpp_u32<CTRL, ROW_MASK, BANK_MASK>((uint32_t)v);
  const uint32_t hi = dpp_u32<CTRL, ROW_MASK, BANK_MASK>((uint32_t)(v >> 32));
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  return o > v ? o : v;
}

// Maximum of v over the 64 lanes, returned uniformly (from lane 63).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_step<0xb1>(v);          // quad_perm [1,0,3,2]
  v = dpp_max_step<0x4e>(v);          // quad_perm [2,3,0,1]
  v = dpp_max_step<0x114>(v);         // row_shr:4
  v = dpp_max_step<0x118>(v);         // row_shr:8
  v = dpp_max_step<0x142, 0xa>(v);    // row_bcast:15
  v = dpp_max_step<0x143, 0xc>(v);    // row_bcast:31
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// The wave selects `topk` experts from scores[0..n_routed) (this token's row)
// with bias. On return every lane holds the same picks[] (rank order) and
// weights[]; nan_any tells whether any key was NaN. KPER = ceil(n_routed/64).
template <int KPER>
__device__ __forceinline__ void select_topk(const float* __restrict__ scores, const float* __restrict__ bias,
                                            int n_routed, int topk, int norm, float route_scale,
                                            int (&picks)[kMaxTopk], float (&weights)[kMaxTopk], bool& nan_any) {
  const int lane = threadIdx.x & 63;
  float sc[KPER];
  uint64_t comp[KPER];
  bool has_nan = false;
  float bs[KPER];
#pragma unroll
  for (int c = 0; c < KPER; ++c) {   // every load issued before any is used (indices clamped, no branches)
    const int e = min(lane + 64 * c, n_routed - 1);
    sc[c] = scores[e];
    bs[c] = bias[e];
  }
#pragma unroll
  for (int c = 0; c < KPER; ++c) {
    const int e = lane + 64 * c;
    const bool in = e < n_routed;
    const float k = fadd(sc[c], bs[c]);
    has_nan |= in && isnan(k);
    comp[c] = in ? (((uint64_t)key_order_bits(k) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e)) : 0ull;
  }
  nan_any = __any(has_nan);
#pragma unroll
  for (int r = 0; r < kMaxTopk; ++r) {
    if (r < topk) {
      uint64_t best = 0;
#pragma unroll
      for (int c = 0; c < KPER; ++c) best = comp[c] > best ? comp[c] : best;
      const uint64_t win = wave_max_u64(best);
      const int id = (int)(0xFFFFFFFFu - (uint32_t)win);
      const int wc = id >> 6, wl = id & 63;
      float s_here = sc[0];
#pragma unroll
      for (int c = 1; c < KPER; ++c) s_here = (c == wc) ? sc[c] : s_here;
      weights[r] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s_here), wl));
      picks[r] = id;
#pragma unroll
      for (int c = 0; c < KPER; ++c) comp[c] = (c == wc && lane == wl) ? 0ull : comp[c];
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

}  // namespace moe
