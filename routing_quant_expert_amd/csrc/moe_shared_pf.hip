// The shared expert for many tokens (prefill, A9): two bf16 MFMA GEMMs with
// f32 accumulation [moe_v41.rs, module doc: the shared expert is resident
// bf16 on the dense GEMM path; fn shared_side]:
//   sg = x . W1s^T, su = x . W3s^T, sh = bf16(SwiGLU(sg, su))   (k_shared_gu_pf)
//   sd = sh . W2s^T                                             (k_shared_down_pf)
//
// v_mfma_f32_32x32x16_bf16 (lane layouts checked on the GPU): lane l holds
// operand row l%32 at k offset 8*(l/32), 8 consecutive bf16; result register
// r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32. Tokens are the
// rows, weight rows the columns. Each wave streams its operands straight from
// global memory (rows of 16 contiguous bytes per lane), kU k-steps of loads
// issued before their MFMAs so that enough bytes are in flight per wave.
// Workgroup tiles are ordered so that the workgroups sharing a weight tile
// run on the same XCD (consecutive workgroups go to consecutive XCDs): the
// tile's rows are then fetched into that XCD's L2 once for all token tiles.
#include <hip/hip_runtime.h>

#include "moe_internal.h"
#include "moe_math.h"
#include "moe_prefill.h"

namespace moe {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kU = 8;        // k-steps of 16 whose loads are issued together
constexpr int kXcds = 8;

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 ld_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(p));
}

__device__ __forceinline__ int tile_tok(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Workgroup b of n_wt weight tiles x n_tt token tiles -> (weight tile, token
// tile), the token tiles of one weight tile on one XCD when the counts allow.
__device__ __forceinline__ void tile_of(int b, int n_wt, int n_tt, int& wt, int& tt) {
  if (n_wt % kXcds == 0) {
    const int x = b % kXcds, i = b / kXcds, per = n_wt / kXcds;
    wt = x * per + i / n_tt;
    tt = i % n_tt;
  } else {
    wt = b / n_tt;
    tt = b % n_tt;
  }
}

// gate/up: a wave = 32 tokens x 32 hidden units, gate and up; a workgroup =
// 4 waves over 128 units sharing the token rows; then sh = bf16(SwiGLU).
__global__ __launch_bounds__(256) void k_shared_gu_pf(const uint16_t* __restrict__ x, int m, int dim, int inter,
                                                      const uint16_t* __restrict__ w1, const uint16_t* __restrict__ w3,
                                                      float* __restrict__ sg, float* __restrict__ su,
                                                      uint16_t* __restrict__ sh, float L) {
  __shared__ float tile[2][32][128 + 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hl = lane >> 5;
  int wt, ttile;
  tile_of(blockIdx.x, inter / 128, (m + 31) / 32, wt, ttile);
  const int tok0 = 32 * ttile, unit0 = 128 * wt;
  const int ta = tok0 + (lane & 31);
  const int un = unit0 + 32 * wave + (lane & 31);
  const uint16_t* xa = x + (int64_t)min(ta, m - 1) * dim + 8 * hl;
  const uint16_t* ga = w1 + (int64_t)un * dim + 8 * hl;
  const uint16_t* ua = w3 + (int64_t)un * dim + 8 * hl;
  f32x16 cg = {}, cu = {};
  const bool arow_ok = ta < m;
  for (int k0 = 0; k0 < dim; k0 += 16 * kU) {
    bf16x8 av[kU], gv[kU], uv[kU];
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      av[i] = ld_bf16x8(xa + k0 + 16 * i);
      gv[i] = ld_bf16x8(ga + k0 + 16 * i);
      uv[i] = ld_bf16x8(ua + k0 + 16 * i);
    }
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      const bf16x8 a = arow_ok ? av[i] : bf16x8{};
      cg = mfma_bf16(a, gv[i], cg);
      cu = mfma_bf16(a, uv[i], cu);
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    tile[0][tile_tok(r, lane)][32 * wave + (lane & 31)] = cg[r];
    tile[1][tile_tok(r, lane)][32 * wave + (lane & 31)] = cu[r];
  }
  __syncthreads();
#pragma unroll 1
  for (int i = tid; i < 32 * 128; i += 256) {
    const int tt = i >> 7, uu = i & 127;
    const int t = tok0 + tt;
    if (t >= m) continue;
    const float gv = tile[0][tt][uu], uv = tile[1][tt][uu];
    const int64_t o = (int64_t)t * inter + unit0 + uu;
    sg[o] = gv;
    su[o] = uv;
    sh[o] = bf16_rne(swiglu(gv, uv, L));
  }
}

// down: sd = W2s . sh; a wave = 32 tokens x 32 output rows, a workgroup = 4
// waves over 128 rows sharing the token rows.
__global__ __launch_bounds__(256) void k_shared_down_pf(const uint16_t* __restrict__ sh, int m, int dim, int inter,
                                                        const uint16_t* __restrict__ w2, float* __restrict__ sd) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hl = lane >> 5;
  int wt, ttile;
  tile_of(blockIdx.x, dim / 128, (m + 31) / 32, wt, ttile);
  const int tok0 = 32 * ttile;
  const int ta = tok0 + (lane & 31);
  const int row = 128 * wt + 32 * wave + (lane & 31);
  const uint16_t* ha = sh + (int64_t)min(ta, m - 1) * inter + 8 * hl;
  const uint16_t* wa = w2 + (int64_t)row * inter + 8 * hl;
  const bool arow_ok = ta < m;
  f32x16 c = {};
  for (int k0 = 0; k0 < inter; k0 += 16 * kU) {
    bf16x8 av[kU], wv[kU];
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      av[i] = ld_bf16x8(ha + k0 + 16 * i);
      wv[i] = ld_bf16x8(wa + k0 + 16 * i);
    }
#pragma unroll
    for (int i = 0; i < kU; ++i) c = mfma_bf16(arow_ok ? av[i] : bf16x8{}, wv[i], c);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int t = tok0 + tile_tok(r, lane);
    if (t < m) sd[(int64_t)t * dim + row] = c[r];
  }
}

}  // namespace

hipError_t launch_shared_pf(const uint16_t* x, int m, const moe_layer& layer, const moe_cfg& c, const Ws& w,
                            hipStream_t s) {
  const int tt = (m + 31) / 32;
  MOE_LAUNCH(MOE_K_SHARED_GU, k_shared_gu_pf, dim3((c.inter / 128) * tt), dim3(256), 0, s, x, m, c.dim, c.inter,
             layer.sh_w1, layer.sh_w3, w.sg, w.su, w.sh, c.swiglu_limit);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  MOE_LAUNCH(MOE_K_SHARED_DOWN, k_shared_down_pf, dim3((c.dim / 128) * tt), dim3(256), 0, s, w.sh, m, c.dim,
             c.inter, layer.sh_w2, w.sd);
  return hipGetLastError();
}

}  // namespace moe
