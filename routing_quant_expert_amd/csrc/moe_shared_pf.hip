// The shared expert for many tokens (prefill, A9): two bf16 MFMA GEMMs with
// f32 accumulation [moe_v41.rs, module doc: the shared expert is resident
// bf16 on the dense GEMM path; fn shared_side]:
//   sg = x . W1s^T, su = x . W3s^T, sh = bf16(SwiGLU(sg, su))   (k_shared_gu_lds)
//   sd = sh . W2s^T                                             (k_shared_down_lds)
//
// v_mfma_f32_32x32x16_bf16 (lane layouts checked on the GPU): lane l holds
// operand row l%32 at k offset 8*(l/32), 8 consecutive bf16; result register
// r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32. Tokens are the
// rows, weight rows the columns. Operand tiles go HBM -> LDS by direct DMA
// through a 3-slot ring, 64 k per step, every tile row's 16-byte chunks stored
// XOR-swizzled so that an operand read spreads over all LDS banks. Workgroup
// tiles are ordered so that the workgroups sharing a weight tile run on the
// same XCD (consecutive workgroups go to consecutive XCDs): the tile's rows
// are then fetched into that XCD's L2 once for all token tiles.
#include <hip/hip_runtime.h>

#include "moe_internal.h"
#include "moe_kquant.h"
#include "moe_math.h"
#include "moe_prefill.h"

namespace moe {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kXcds = 8;

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
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

// ---------------------------------------------------------------------------
// gate/up through LDS: a workgroup = 64 tokens x 64 hidden units, gate and up
// (wave w: tokens 32*(w&1).., units 32*(w>>1)..). Each k-step of 64 stages
// the 64x64 tiles of x, W1s and W3s (8 KB each) in a 3-slot LDS ring by
// direct-to-LDS DMA (16 bytes per lane, 6 per thread and step); every tile
// row is 8 chunks of 16 bytes stored at chunk position c ^ (row & 7), so the
// 32 rows an MFMA operand read touches spread over all banks. Each output
// sums k in ascending steps of 16, one MFMA per step.
// ---------------------------------------------------------------------------
constexpr int kTk = 64;                       // k per step
constexpr int kTileB = 64 * kTk * 2;          // one 64x64 bf16 tile: 8 KB
constexpr int kGuStage = 3 * kTileB;          // x, W1s, W3s
constexpr int kGuStages = 3;
constexpr int kGuDmaPer = kGuStage / 16 / 256;   // 16-byte DMAs per thread and step (6)

// The ring's waits: step s is in once at most `after` later steps' DMAs are
// outstanding (after = 0, 1 or 2).
__device__ __forceinline__ void wait_step(int after) {
  if (after >= 2) wait_vmcnt<2 * kGuDmaPer>();
  else if (after == 1) wait_vmcnt<kGuDmaPer>();
  else wait_vmcnt<0>();
  block_sync_lds();
}
// Every wave is done reading the slot about to be refilled.
__device__ __forceinline__ void slot_free() {
  wait_lgkm0();
  block_sync_lds();
}

__global__ __launch_bounds__(256) void k_shared_gu_lds(const uint16_t* __restrict__ x, int m, int dim, int inter,
                                                       const uint16_t* __restrict__ w1,
                                                       const uint16_t* __restrict__ w3, float* __restrict__ sg,
                                                       float* __restrict__ su, uint16_t* __restrict__ sh, float L) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hl = lane >> 5;
  int wt, tt;
  tile_of(blockIdx.x, inter / 64, (m + 63) / 64, wt, tt);
  const int tok0 = 64 * tt, unit0 = 64 * wt;
  // this thread's DMA sources: position i = wave*64 + 256*k + lane of the
  // stage (x tile, then W1s, then W3s); row i'/8, stored chunk i'%8 holds
  // source chunk (i'%8) ^ (row & 7)
  const uint16_t* src[kGuDmaPer];
#pragma unroll
  for (int k = 0; k < kGuDmaPer; ++k) {
    const int i = wave * 64 + 256 * k + lane;
    const int mat = i / 512, ii = i % 512, row = ii >> 3, c = (ii & 7) ^ (row & 7);
    const uint16_t* base = mat == 0 ? x + (int64_t)min(tok0 + row, m - 1) * dim
                                    : (mat == 1 ? w1 : w3) + (int64_t)(unit0 + row) * dim;
    src[k] = base + 8 * c;
  }
  const int nk = dim / kTk;
  auto issue = [&](int s) {
    uint8_t* st = lds + (s % kGuStages) * kGuStage;
#pragma unroll
    for (int k = 0; k < kGuDmaPer; ++k)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src[k] + (int64_t)s * kTk),
                                       (__attribute__((address_space(3))) void*)(st + 16 * (wave * 64 + 256 * k)),
                                       16, 0, 0);
  };
  // operand rows of this lane: token 32*(wave&1) + l%32 of the x tile, unit 32*(wave>>1) + l%32 of the W tiles
  const int ra = 32 * (wave & 1) + (lane & 31), rb = 32 * (wave >> 1) + (lane & 31);
  f32x16 cg = {}, cu = {};
  issue(0);
  if (nk > 1) issue(1);
  if (nk > 2) issue(2);
#pragma unroll 1
  for (int s = 0; s < nk; ++s) {
    wait_step(min(s + kGuStages, nk) - s - 1);
    const uint8_t* st = lds + (s % kGuStages) * kGuStage;
    bf16x8 av[4], gv[4], uv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {   // k-substep q: chunk 2q + hl of each row
      const int c = 2 * q + hl;
      av[q] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(st + 16 * (ra * 8 + (c ^ (ra & 7)))));
      gv[q] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(st + kTileB + 16 * (rb * 8 + (c ^ (rb & 7)))));
      uv[q] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(st + 2 * kTileB + 16 * (rb * 8 + (c ^ (rb & 7)))));
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      cg = mfma_bf16(av[q], gv[q], cg);
      cu = mfma_bf16(av[q], uv[q], cu);
    }
    if (s + kGuStages < nk) {
      slot_free();
      issue(s + kGuStages);
    }
  }
  const int unit = unit0 + 32 * (wave >> 1) + (lane & 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int t = tok0 + 32 * (wave & 1) + tile_tok(r, lane);
    if (t < m) {
      const int64_t o = (int64_t)t * inter + unit;
      sg[o] = cg[r];
      su[o] = cu[r];
      sh[o] = bf16_rne(swiglu(cg[r], cu[r], L));
    }
  }
}

// down through LDS: a workgroup = 64 tokens x 128 output rows (wave w: tokens
// 32*(w&1).., rows 64*(w>>1).. as two 32-row MFMA tiles sharing the sh
// operand); each k-step of 64 stages the sh tile (8 KB) and the W2s tile
// (16 KB) in the same swizzled 3-slot ring as k_shared_gu_lds.
__global__ __launch_bounds__(256) void k_shared_down_lds(const uint16_t* __restrict__ sh, int m, int dim, int inter,
                                                         const uint16_t* __restrict__ w2, float* __restrict__ sd) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hl = lane >> 5;
  int wt, tt;
  tile_of(blockIdx.x, dim / 128, (m + 63) / 64, wt, tt);
  const int tok0 = 64 * tt, row0 = 128 * wt;
  const uint16_t* src[kGuDmaPer];
#pragma unroll
  for (int k = 0; k < kGuDmaPer; ++k) {
    const int i = wave * 64 + 256 * k + lane;
    const bool a = i < 512;
    const int ii = a ? i : i - 512, row = ii >> 3, c = (ii & 7) ^ (row & 7);
    const uint16_t* base = a ? sh + (int64_t)min(tok0 + row, m - 1) * inter : w2 + (int64_t)(row0 + row) * inter;
    src[k] = base + 8 * c;
  }
  const int nk = inter / kTk;
  auto issue = [&](int s) {
    uint8_t* st = lds + (s % kGuStages) * kGuStage;
#pragma unroll
    for (int k = 0; k < kGuDmaPer; ++k)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src[k] + (int64_t)s * kTk),
                                       (__attribute__((address_space(3))) void*)(st + 16 * (wave * 64 + 256 * k)),
                                       16, 0, 0);
  };
  const int ra = 32 * (wave & 1) + (lane & 31), rb = 64 * (wave >> 1) + (lane & 31);
  f32x16 c0 = {}, c1 = {};
  issue(0);
  if (nk > 1) issue(1);
  if (nk > 2) issue(2);
#pragma unroll 1
  for (int s = 0; s < nk; ++s) {
    wait_step(min(s + kGuStages, nk) - s - 1);
    const uint8_t* st = lds + (s % kGuStages) * kGuStage;
    bf16x8 av[4], b0[4], b1[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = 2 * q + hl;
      av[q] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(st + 16 * (ra * 8 + (c ^ (ra & 7)))));
      b0[q] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(st + kTileB + 16 * (rb * 8 + (c ^ (rb & 7)))));
      b1[q] = __builtin_bit_cast(bf16x8,
                                 *reinterpret_cast<const i32x4*>(st + kTileB + 16 * ((rb + 32) * 8 + (c ^ (rb & 7)))));
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      c0 = mfma_bf16(av[q], b0[q], c0);
      c1 = mfma_bf16(av[q], b1[q], c1);
    }
    if (s + kGuStages < nk) {
      slot_free();
      issue(s + kGuStages);
    }
  }
  const int row = row0 + rb;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int t = tok0 + 32 * (wave & 1) + tile_tok(r, lane);
    if (t < m) {
      sd[(int64_t)t * dim + row] = c0[r];
      sd[(int64_t)t * dim + row + 32] = c1[r];
    }
  }
}

}  // namespace

hipError_t launch_shared_pf(const uint16_t* x, int m, const moe_layer& layer, const moe_cfg& c, const Ws& w,
                            hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    for (const void* k : {(const void*)k_shared_gu_lds, (const void*)k_shared_down_lds}) {
      hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, kGuStages * kGuStage);
      if (e != hipSuccess) return e;
    }
    attr_set = true;
  }
  const int tt = (m + 63) / 64;
  MOE_LAUNCH(MOE_K_SHARED_GU, k_shared_gu_lds, dim3((c.inter / 64) * tt), dim3(256), kGuStages * kGuStage, s, x, m,
             c.dim, c.inter, layer.sh_w1, layer.sh_w3, w.sg, w.su, w.sh, c.swiglu_limit);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  MOE_LAUNCH(MOE_K_SHARED_DOWN, k_shared_down_lds, dim3((c.dim / 128) * tt), dim3(256), kGuStages * kGuStage, s,
             w.sh, m, c.dim, c.inter, layer.sh_w2, w.sd);
  return hipGetLastError();
}

}  // namespace moe
