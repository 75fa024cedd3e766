// Shared expert (part of A7): resident bf16 SwiGLU MLP at m <= 8 as GEMVs
// [moe_v41.rs, module doc; Kernels: gemv, "the tiled GEMM idles 15 of 16
// rows" at m = 1]. f32 accumulation, any order (compared with a tolerance);
// the SwiGLU output is rounded to bf16 for the down GEMV.
#include <hip/hip_runtime.h>

#include "moe_internal.h"
#include "moe_math.h"

namespace moe {
namespace {

__device__ inline void bf16x8(uint4 v, float (&f)[8]) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = bf16_f32((uint16_t)(w[j >> 1] >> (16 * (j & 1))));
}

// One wave per hidden unit i: sg = W1[i].x, su = W3[i].x, sh = bf16(swiglu).
__global__ __launch_bounds__(256) void k_shared_gu(const uint16_t* __restrict__ x, int m, int dim, int inter,
                                                   const uint16_t* __restrict__ w1, const uint16_t* __restrict__ w3,
                                                   float* __restrict__ sg, float* __restrict__ su,
                                                   uint16_t* __restrict__ sh, float L) {
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= inter) return;
  float pg[kMaxDecodeTokens], pu[kMaxDecodeTokens];
#pragma unroll
  for (int t = 0; t < kMaxDecodeTokens; ++t) pg[t] = pu[t] = 0.0f;
  const uint16_t* r1 = w1 + (int64_t)i * dim;
  const uint16_t* r3 = w3 + (int64_t)i * dim;
  for (int k = 8 * lane; k < dim; k += 512) {
    float a[8], b[8];
    bf16x8(load_nt16(r1 + k), a);
    bf16x8(load_nt16(r3 + k), b);
#pragma unroll
    for (int t = 0; t < kMaxDecodeTokens; ++t) {
      if (t < m) {
        float xv[8];
        bf16x8(*reinterpret_cast<const uint4*>(x + (int64_t)t * dim + k), xv);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          pg[t] = __builtin_fmaf(a[j], xv[j], pg[t]);
          pu[t] = __builtin_fmaf(b[j], xv[j], pu[t]);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kMaxDecodeTokens; ++t) {
    for (int s = 32; s >= 1; s >>= 1) {
      pg[t] += __shfl_xor(pg[t], s);
      pu[t] += __shfl_xor(pu[t], s);
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

// One wave per output row r: sd = W2[r].sh.
__global__ __launch_bounds__(256) void k_shared_down(int m, int dim, int inter, const uint16_t* __restrict__ w2,
                                                     const uint16_t* __restrict__ sh, float* __restrict__ sd) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= dim) return;
  float p[kMaxDecodeTokens];
#pragma unroll
  for (int t = 0; t < kMaxDecodeTokens; ++t) p[t] = 0.0f;
  const uint16_t* row = w2 + (int64_t)r * inter;
  for (int k = 8 * lane; k < inter; k += 512) {
    float a[8];
    bf16x8(load_nt16(row + k), a);
#pragma unroll
    for (int t = 0; t < kMaxDecodeTokens; ++t) {
      if (t < m) {
        float hv[8];
        bf16x8(*reinterpret_cast<const uint4*>(sh + (int64_t)t * inter + k), hv);
#pragma unroll
        for (int j = 0; j < 8; ++j) p[t] = __builtin_fmaf(a[j], hv[j], p[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kMaxDecodeTokens; ++t)
    for (int s = 32; s >= 1; s >>= 1) p[t] += __shfl_xor(p[t], s);
  if (lane < m) {
    float v = 0.0f;
#pragma unroll
    for (int t = 0; t < kMaxDecodeTokens; ++t)
      if (t == lane) v = p[t];
    sd[(int64_t)lane * dim + r] = v;
  }
}

}  // namespace

hipError_t launch_shared_gu(const uint16_t* x, int m, const uint16_t* w1, const uint16_t* w3, const moe_cfg& c,
                            const Ws& w, hipStream_t s) {
  hipLaunchKernelGGL(k_shared_gu, dim3((c.inter + 3) / 4), dim3(256), 0, s, x, m, c.dim, c.inter, w1, w3, w.sg, w.su,
                     w.sh, c.swiglu_limit);
  return hipGetLastError();
}

hipError_t launch_shared_down(int m, const uint16_t* w2, const moe_cfg& c, const Ws& w, hipStream_t s) {
  hipLaunchKernelGGL(k_shared_down, dim3((c.dim + 3) / 4), dim3(256), 0, s, m, c.dim, c.inter, w2, w.sh, w.sd);
  return hipGetLastError();
}

}  // namespace moe
