// Device parts of the layer's front, shared by the multi-token launches and
// the single-token persistent kernel: q8_1 of the input rows, the router
// GEMV rows with their scores, and the shared expert's gate/up rows.
#pragma once

#include <hip/hip_runtime.h>

#include "moe_internal.h"
#include "moe_math.h"
#include "moe_wave.h"

namespace moe {
namespace front {

__device__ inline uint16_t fp16_bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// ---------------------------------------------------------------------------
// q8_1 of bf16 rows: one thread per value, a q8_1 block = 32 consecutive
// lanes. d = amax/127, code = roundf(x/d) (half away from zero), stored scale
// fp16(d), plus the sums of 16 consecutive codes (the q8_1 sum field is not
// used; the GEMV epilogues need per-16 sums of the codes).
__device__ void quant_x_block(int blk, const uint16_t* __restrict__ x, int8_t* __restrict__ xq,
                              uint16_t* __restrict__ xd, int32_t* __restrict__ xs, double* __restrict__ xd64 = nullptr) {
  const int64_t i = (int64_t)blk * 256 + threadIdx.x;   // m*dim is a multiple of 256
  float v = bf16_f32(x[i]);
  const float a = max32(fabsf(v));
  float d = (float)((double)a / 127.0);
  int q = a == 0.0f ? 0 : q8_code(v, d);
  xq[i] = (int8_t)q;
  const int sum = sum16(q);
  const int lane32 = threadIdx.x & 31;
  if (lane32 == 0) {
    xd[i >> 5] = fp16_bits(d);
    if (xd64) xd64[i >> 5] = (double)__builtin_bit_cast(_Float16, fp16_bits(d));
  }
  if ((lane32 & 15) == 0) xs[i >> 4] = sum;
}

// ---------------------------------------------------------------------------
// Router GEMV + scores. One wave64 per expert row (three rows per workgroup
// of four waves), for the tokens [t_lo, t_hi) of the call (default: all of
// them). Lane l accumulates positions 512*i + 8*l + j (i ascending, j = 0..7) in
// f32 (product, then add: every bf16 x bf16 product is exact), then the 64
// partials combine as p += shfl_xor(p, s) for s = 32..1 (computed by
// wave_sum_xor) and lane 0 holds the logit. This per-row order is the same for every m, so a token's logits
// never depend on the batch it rides in.
// ---------------------------------------------------------------------------
constexpr int kRouterTok = 8;
constexpr int kLoadAhead = 8;   // 16-byte chunks per lane kept in flight by one wave

__device__ void router_rows(int blk, const uint16_t* __restrict__ x, int m, int dim,
                            const uint16_t* __restrict__ gate_w, int n_routed, float temp, float* __restrict__ logits,
                            float* __restrict__ scores, float* __restrict__ logits_out, const ScoreTable& st,
                            int t_lo = 0, int t_hi = -1) {
  // waves 0..2 take a row each; wave 3 runs the same code on no data at once,
  // which brings it into the instruction cache before the others need it
  const bool warm = (threadIdx.x >> 6) == 3;
  const int e = blk * 3 + (warm ? 0 : (threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  if (e >= n_routed) return;
  const uint16_t* wr = gate_w + (int64_t)e * dim;
  const int nch = (dim + 511) / 512;
  if (t_hi < 0) t_hi = m;
  for (int t0 = t_lo; t0 < t_hi; t0 += kRouterTok) {
    const int nt = min(kRouterTok, t_hi - t0);
    float p[kRouterTok];
#pragma unroll
    for (int t = 0; t < kRouterTok; ++t) p[t] = 0.0f;
    for (int c0 = 0; c0 < nch; c0 += kLoadAhead) {
      uint4 wv[kLoadAhead];
#pragma unroll
      for (int c = 0; c < kLoadAhead; ++c) {
        const int k = 512 * (c0 + c) + 8 * lane;
        wv[c] = (!warm && c0 + c < nch && k < dim) ? *reinterpret_cast<const uint4*>(wr + k) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int t = 0; t < kRouterTok; ++t) {
        if (t < nt) {
          uint4 xv[kLoadAhead];
#pragma unroll
          for (int c = 0; c < kLoadAhead; ++c) {
            const int k = 512 * (c0 + c) + 8 * lane;
            xv[c] = (!warm && c0 + c < nch && k < dim) ? *reinterpret_cast<const uint4*>(x + (int64_t)(t0 + t) * dim + k)
                                              : make_uint4(0, 0, 0, 0);
          }
          float acc = p[t];
#pragma unroll
          for (int c = 0; c < kLoadAhead; ++c) {
            const uint32_t ww[4] = {wv[c].x, wv[c].y, wv[c].z, wv[c].w};
            const uint32_t xx[4] = {xv[c].x, xv[c].y, xv[c].z, xv[c].w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const uint16_t xb = (uint16_t)(xx[j >> 1] >> (16 * (j & 1)));
              const uint16_t wb = (uint16_t)(ww[j >> 1] >> (16 * (j & 1)));
              acc = fadd(acc, fmul(bf16_f32(xb), bf16_f32(wb)));   // zero padding adds +0: exact
            }
          }
          p[t] = acc;
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kRouterTok; ++t)
      if (t < nt) p[t] = wave_sum_xor(p[t]);
    if (lane < nt) {
      float lg = 0.0f;
#pragma unroll
      for (int t = 0; t < kRouterTok; ++t)
        if (t == lane) lg = p[t];
      const int64_t o = (int64_t)(t0 + lane) * n_routed + e;
      const float sc = score_mode_of(lg, temp, st);
      if (!warm) {
        logits[o] = lg;
        if (logits_out) logits_out[o] = lg;
        scores[o] = sc;
      }
    }
  }
}

// Shared expert gate/up (m <= 8): one wave per hidden unit i: sg = W1s[i].x,
// su = W3s[i].x (f32, any order), sh = bf16(swiglu(sg, su)) [moe_v41.rs,
// module doc: the shared expert is resident bf16 on the dense GEMM/GEMV].
// A lane sums its chunks in order, two products per v_dot2_f32_bf16; then
// the lanes' partials by wave_sum_xor.
__device__ void shared_gu_rows(int blk, const uint16_t* __restrict__ x, int m, int dim, int inter,
                               const uint16_t* __restrict__ w1, const uint16_t* __restrict__ w3,
                               float* __restrict__ sg, float* __restrict__ su, uint16_t* __restrict__ sh, float L) {
  const int i = blk * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= inter) return;
  float pg[kMaxDecodeTokens], pu[kMaxDecodeTokens];
#pragma unroll
  for (int t = 0; t < kMaxDecodeTokens; ++t) pg[t] = pu[t] = 0.0f;
  const uint16_t* r1 = w1 + (int64_t)i * dim;
  const uint16_t* r3 = w3 + (int64_t)i * dim;
  const int nch = (dim + 511) / 512;
  for (int c0 = 0; c0 < nch; c0 += kLoadAhead) {
    uint4 av[kLoadAhead], bv[kLoadAhead];
#pragma unroll
    for (int c = 0; c < kLoadAhead; ++c) {
      const int k = 512 * (c0 + c) + 8 * lane;
      const bool in = c0 + c < nch && k < dim;
      av[c] = in ? load_nt16(r1 + k) : make_uint4(0, 0, 0, 0);
      bv[c] = in ? load_nt16(r3 + k) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < kMaxDecodeTokens; ++t) {
      if (t < m) {
#pragma unroll
        for (int c = 0; c < kLoadAhead; ++c) {
          const int k = 512 * (c0 + c) + 8 * lane;
          if (c0 + c < nch && k < dim) {
            const uint4 xv = *reinterpret_cast<const uint4*>(x + (int64_t)t * dim + k);
            pg[t] = dot8_bf16(av[c], xv, pg[t]);
            pu[t] = dot8_bf16(bv[c], xv, pu[t]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kMaxDecodeTokens; ++t) {
    if (t < m) {
      pg[t] = wave_sum_xor(pg[t]);
      pu[t] = wave_sum_xor(pu[t]);
    }
  }
  if (lane < m) {
    float g = 0.0f, u = 0.0f;
#pragma unroll
    for (int t = 0; t < kMaxDecodeTokens; ++t)
      if (t == lane) {
        g = pg[t];
        u = pu[t];
      }
    const int64_t o = (int64_t)lane * inter + i;
    sg[o] = g;
    su[o] = u;
    sh[o] = bf16_rne(swiglu(g, u, L));
  }
}

// Shared expert gate/up of ONE token for hidden unit `un`, by one wave: the
// same per-lane summation order and lane reduction as shared_gu_rows, so the
// values equal the multi-token ones. Every lane gets (g, u). dim <= 4096.
// In two parts, so that a caller can put other loads in flight between the
// issue of the unit's loads and their use.
struct SharedUnitLoads {
  static constexpr int kC = 8;   // 16-byte chunks per lane and row
  uint4 a[kC], b[kC], x[kC];
};

__device__ inline void shared_gu_issue(int un, const uint16_t* __restrict__ x, int dim,
                                       const uint16_t* __restrict__ w1, const uint16_t* __restrict__ w3,
                                       SharedUnitLoads& L) {
  const int lane = threadIdx.x & 63;
  const int nch = (dim + 511) / 512;
#pragma unroll
  for (int c = 0; c < SharedUnitLoads::kC; ++c) {
    const int k = 512 * c + 8 * lane;
    const bool in = c < nch && k < dim;
    L.a[c] = in ? load_nt16(w1 + (int64_t)un * dim + k) : make_uint4(0, 0, 0, 0);
    L.b[c] = in ? load_nt16(w3 + (int64_t)un * dim + k) : make_uint4(0, 0, 0, 0);
    L.x[c] = in ? *reinterpret_cast<const uint4*>(x + k) : make_uint4(0, 0, 0, 0);
  }
}

__device__ inline void shared_gu_sum(const SharedUnitLoads& L, int dim, float& g, float& u) {
  const int lane = threadIdx.x & 63;
  const int nch = (dim + 511) / 512;
  float pg = 0.0f, pu = 0.0f;
#pragma unroll
  for (int c = 0; c < SharedUnitLoads::kC; ++c) {
    const int k = 512 * c + 8 * lane;
    if (c < nch && k < dim) {
      pg = dot8_bf16(L.a[c], L.x[c], pg);
      pu = dot8_bf16(L.b[c], L.x[c], pu);
    }
  }
  g = wave_sum_xor(pg);
  u = wave_sum_xor(pu);
}

__device__ inline void shared_gu_unit(int un, const uint16_t* __restrict__ x, int dim,
                                      const uint16_t* __restrict__ w1, const uint16_t* __restrict__ w3, float& g,
                                      float& u) {
  SharedUnitLoads L;
  shared_gu_issue(un, x, dim, w1, w3, L);
  shared_gu_sum(L, dim, g, u);
}

}  // namespace front
}  // namespace moe
