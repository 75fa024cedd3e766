// Routed experts (A4-A7): K-quant GEMVs on the raw GGUF blocks against q8_1
// activations [moe_v41.rs, module doc; Kernels: mmvq_q2k_experts,
// mmvq_q3k_experts, swiglu_q8, accumulate].
//
// Numerics: a lane turns one 256-weight super-block into 16 exact integer
// sums I_s = sum(code * q8) with v_dot4 (one per 16-weight sub-block), folds
// the sub-block scales in integers per 32-weight q8_1 block, and multiplies
// by the q8_1 block scale in float64, where every such product is exact. The
// float64 partial sums of a row (one per super-block, combined across lanes
// in a fixed butterfly) are rounded once to f32: the f32 result is the
// correctly rounded exact dot product except when that lies within ~2^-47 of
// an f32 midpoint.
#include <hip/hip_runtime.h>

#include "moe_internal.h"
#include "moe_kquant.h"
#include "moe_math.h"
#include "moe_wave.h"

namespace moe {
namespace {


// ---------------------------------------------------------------------------
// Gate/up on Q2_K + clamped SwiGLU + q8_1 of h. Workgroup = (distinct expert
// u, 32-row group of the hidden units): its 32 gate rows and 32 up rows for
// every token that picked u, as four 16-row tiles (gate 0-15, up 0-15, gate
// 16-31, up 16-31) through a ring of SLOTS LDS slots, the next tiles in flight
// while one is computed. A row's NSB super-blocks go to NSB consecutive lanes
// (a lane group) and are summed by a float64 butterfly. With np tokens on the
// expert (np <= 8), the 256/NSB lane groups are split into np_pad = the power
// of two >= np token slots: group g takes token g % np_pad and, of each tile,
// the rows r with r % RG == g / np_pad (RG = groups / np_pad). Each lane
// thus loads its token's activation once and keeps it for every tile.
// ---------------------------------------------------------------------------
template <int NSB, int SLOTS>
__global__ __launch_bounds__(256) void k_gateup(XArena ex, PlanView plan, const int8_t* __restrict__ xq,
                                                const uint16_t* __restrict__ xd, const int32_t* __restrict__ xs,
                                                int dim, int inter, float* __restrict__ g_out,
                                                float* __restrict__ u_out, float* __restrict__ h_out,
                                                int8_t* __restrict__ hq, uint16_t* __restrict__ hd,
                                                int32_t* __restrict__ hs, float L) {
  using G = GateUpGeom<NSB>;
  static_assert(NSB <= 16 && kMaxDecodeTokens <= 8, "lane groups per token slot");
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ float gu[2][kMaxDecodeTokens][32];
  const int ngr = inter / 32;
  const int u = blockIdx.x / ngr, grp = blockIdx.x % ngr;
  if (u >= *plan.n_u()) return;
  const int e = plan.u_expert()[u], first = plan.u_first()[u], np = plan.u_npairs()[u];   // 1 <= np <= 8
  const int np_pad = np <= 1 ? 1 : (np <= 2 ? 2 : (np <= 4 ? 4 : 8));
  constexpr int kGroups = 256 / NSB;
  const int sb = threadIdx.x % NSB, g = threadIdx.x / NSB;
  const int j = g % np_pad, rg = g / np_pad, RG = kGroups / np_pad;
  const bool has = j < np;
  const uint8_t* gbase = ex.gate(e);
  const uint8_t* ubase = ex.up(e);
  auto tile_src = [&](int c) -> const uint8_t* {
    return ((c & 1) ? ubase : gbase) + (uint64_t)(32 * grp + 16 * (c >> 1)) * G::kRowBytes;
  };
  Act A;
  {
    const int tok = plan.pair_tok()[first + (has ? j : 0)];
    load_act(A, xq + (int64_t)tok * dim, xd + (int64_t)tok * (dim / 32), xs + (int64_t)tok * (dim / 16), sb);
  }
  __syncthreads();   // completes the activation loads: the tile DMA below is all vmcnt sees
#pragma unroll
  for (int c = 0; c < SLOTS && c < 4; ++c)
    dma_tile_exact<G::kKC>(tile_src(c), lds + c * G::kTileBytes, G::kTileChunks);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    // tiles issued after tile c and still allowed in flight
    const int issued = (c + SLOTS < 4 ? c + SLOTS : 4);
    const int after = issued - c - 1;
    if (after == 3) wait_vmcnt<3 * G::kKC>();
    else if (after == 2) wait_vmcnt<2 * G::kKC>();
    else if (after == 1) wait_vmcnt<1 * G::kKC>();
    else wait_vmcnt<0>();
    block_sync_lds();
    const uint8_t* slot = lds + (c % SLOTS) * G::kTileBytes;
    const int mat = c & 1, r0 = 16 * (c >> 1);
    for (int row = rg; row - rg < 16; row += RG) {   // the same trip count on every lane
      const bool on = has && row < 16;
      double part = on ? dot_q2k(slot + row * G::kRowBytes + kQ2KBytes * sb, A) : 0.0;
      part = seg_sum_f64<NSB>(part);
      if (on && sb == 0) gu[mat][j][r0 + row] = (float)part;
    }
    if (c + SLOTS < 4) {
      wait_lgkm0();
      block_sync_lds();
      dma_tile_exact<G::kKC>(tile_src(c + SLOTS), lds + (c % SLOTS) * G::kTileBytes, G::kTileChunks);
    }
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 31;
  for (int j = wave; j < np; j += 4) {
    const int pair = first + j;
    float gv = gu[0][j][r], uv = gu[1][j][r];
    float hv = swiglu(gv, uv, L);
    const float a = max32(fabsf(hv));
    float d = (float)((double)a / 127.0);
    int q = a == 0.0f ? 0 : q8_code(hv, d);
    const int sum = sum16(q);
    if (lane < 32) {
      const int64_t row = (int64_t)pair * inter + 32 * grp + r;
      g_out[row] = gv;
      u_out[row] = uv;
      h_out[row] = hv;
      hq[row] = (int8_t)q;
      if (r == 0) hd[(int64_t)pair * (inter / 32) + grp] = f32_to_fp16_bits(d);
      if ((r & 15) == 0) hs[(int64_t)pair * (inter / 16) + 2 * grp + (r >> 4)] = sum;
    }
  }
}

// ---------------------------------------------------------------------------
// Down on Q3_K: workgroup = (distinct expert u, 64 output rows) for every token
// that picked u (all four 16-row tiles in flight at once); y[pair][row] =
// RN32(the row's float64 sum). The lane groups (NSB lanes per row) are split
// across the expert's tokens as in the gate/up kernel, so each lane loads its
// token's q8_1(h) once. The first workgroups compute the shared expert's down
// rows (sd = W2s . sh in f32), alongside the routed ones.
// ---------------------------------------------------------------------------
constexpr int kDownRows = 64;   // output rows per routed workgroup: 16-row tiles, all in flight at once

template <int NSB>
struct DownGeom {
  static constexpr int kRowBytes = NSB * kQ3KBytes;
  static constexpr int kTileChunks = 16 * kRowBytes / 16;
  static constexpr int kKC = (kTileChunks + 255) / 256;
  static constexpr int kSlotBytes = kKC * 4096;
};

// Shared expert down rows for the m tokens: every token's sh is staged in LDS
// once per workgroup; a wave computes kRw rows with all of their weight loads
// in flight at once. Lane l sums positions 8l + 512c + (0..7) (c ascending),
// two products per v_dot2_f32_bf16, for each token, then the 64 lanes combine
// by wave_sum_xor.
template <int NSB>
struct SharedDownGeom {
  static constexpr int kCh = NSB >= 2 ? NSB / 2 : 1;    // 16-byte chunks of a row per lane (inter = 256*NSB)
  static constexpr int kRw = kCh >= 8 ? 2 : 4;          // rows per wave
  static constexpr int kRows = 4 * kRw;                 // rows per workgroup
};

template <int NSB>
__device__ void shared_down_rows(int blk, int m, int dim, int inter, const uint16_t* __restrict__ w2,
                                 const uint16_t* __restrict__ sh, float* __restrict__ sd, uint8_t* lds) {
  using S = SharedDownGeom<NSB>;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rbase = blk * S::kRows + S::kRw * wave;   // dim is a multiple of kRows
  uint4 wv[S::kRw][S::kCh];
#pragma unroll
  for (int c = 0; c < S::kCh; ++c) {
    const int k = 8 * lane + 512 * c;
#pragma unroll
    for (int r = 0; r < S::kRw; ++r)
      wv[r][c] = k < inter ? load_nt16(w2 + (int64_t)(rbase + r) * inter + k) : make_uint4(0, 0, 0, 0);
  }
  // every token's sh into LDS: each thread's pieces loaded together, then stored
  constexpr int kStage = (kMaxDecodeTokens * 256 * NSB / 8 + 255) / 256;
  uint16_t* shl = reinterpret_cast<uint16_t*>(lds);
  const int n16 = m * inter / 8;
  uint4 st[kStage];
#pragma unroll
  for (int k = 0; k < kStage; ++k) {
    const int i = threadIdx.x + 256 * k;
    st[k] = i < n16 ? *reinterpret_cast<const uint4*>(sh + 8 * i) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int k = 0; k < kStage; ++k) {
    const int i = threadIdx.x + 256 * k;
    if (i < n16) *reinterpret_cast<uint4*>(shl + 8 * i) = st[k];
  }
  __syncthreads();
  float p[S::kRw][kMaxDecodeTokens];
#pragma unroll
  for (int r = 0; r < S::kRw; ++r)
#pragma unroll
    for (int t = 0; t < kMaxDecodeTokens; ++t) p[r][t] = 0.0f;
#pragma unroll
  for (int c = 0; c < S::kCh; ++c) {
    const int k = 8 * lane + 512 * c;
    if (k < inter) {
#pragma unroll
      for (int t = 0; t < kMaxDecodeTokens; ++t) {
        if (t < m) {
          const uint4 hv = *reinterpret_cast<const uint4*>(shl + t * inter + k);
#pragma unroll
          for (int r = 0; r < S::kRw; ++r) p[r][t] = dot8_bf16(wv[r][c], hv, p[r][t]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < S::kRw; ++r) {
#pragma unroll
    for (int t = 0; t < kMaxDecodeTokens; ++t)
      if (t < m) p[r][t] = wave_sum_xor(p[r][t]);
    if (lane < m) {
      float v = 0.0f;
#pragma unroll
      for (int t = 0; t < kMaxDecodeTokens; ++t)
        if (t == lane) v = p[r][t];
      sd[(int64_t)lane * dim + rbase + r] = v;
    }
  }
}

template <int NSB>
__global__ __launch_bounds__(256) void k_down(XArena ex, PlanView plan, const int8_t* __restrict__ hq,
                                              const uint16_t* __restrict__ hd, const int32_t* __restrict__ hs,
                                              int dim, int inter, float* __restrict__ y, int shared_blocks, int m,
                                              const uint16_t* __restrict__ w2, const uint16_t* __restrict__ sh,
                                              float* __restrict__ sd) {
  using G = DownGeom<NSB>;
  static_assert(NSB <= 16 && kMaxDecodeTokens <= 8, "lane groups per token slot");
  extern __shared__ __align__(16) uint8_t lds[];
  if ((int)blockIdx.x < shared_blocks) {   // first, so that they run alongside the routed rows
    shared_down_rows<NSB>(blockIdx.x, m, dim, inter, w2, sh, sd, lds);
    return;
  }
  const int ngr = dim / kDownRows;
  const int u = (blockIdx.x - shared_blocks) / ngr, grp = (blockIdx.x - shared_blocks) % ngr;
  if (u >= *plan.n_u()) return;
  const int e = plan.u_expert()[u], first = plan.u_first()[u], np = plan.u_npairs()[u];   // 1 <= np <= 8
  const int np_pad = np <= 1 ? 1 : (np <= 2 ? 2 : (np <= 4 ? 4 : 8));
  constexpr int kGroups = 256 / NSB;
  const int sb = threadIdx.x % NSB, g = threadIdx.x / NSB;
  const int j = g % np_pad, rg = g / np_pad, RG = kGroups / np_pad;
  const bool has = j < np;
  const int pair = first + (has ? j : 0);
  const uint8_t* mbase = ex.down(e);
  Act A;
  load_act(A, hq + (int64_t)pair * inter, hd + (int64_t)pair * (inter / 32), hs + (int64_t)pair * (inter / 16), sb);
#pragma unroll
  for (int c = 0; c < kDownRows / 16; ++c)
    dma_tile<G::kKC>(mbase + (uint64_t)(kDownRows * grp + 16 * c) * G::kRowBytes, lds + c * G::kSlotBytes,
                     G::kTileChunks);
  wait_vmcnt<0>();
  block_sync_lds();
  for (int row = rg; row - rg < kDownRows; row += RG) {   // the same trip count on every lane
    const bool on = has && row < kDownRows;
    const int rr = on ? row : 0;
    double part = on ? dot_q3k(lds + (rr >> 4) * G::kSlotBytes + (rr & 15) * G::kRowBytes + kQ3KBytes * sb, A) : 0.0;
    part = seg_sum_f64<NSB>(part);
    if (on && sb == 0) y[(int64_t)pair * dim + kDownRows * grp + row] = (float)part;
  }
}

// ---------------------------------------------------------------------------
// Combine: acc = +0; over the token's picks in plan order (ascending id)
// acc = acc + w*y; then acc = acc + sd when the shared expert is present
// [moe_v41.rs, fn shared_side: added after the routed experts].
// ---------------------------------------------------------------------------
// Four consecutive output elements per thread (16-byte loads of y and sd);
// every element is summed exactly as one at a time: plan order, then sd.
__global__ __launch_bounds__(256) void k_combine(PlanView plan, const float* __restrict__ y, int dim, int topk,
                                                 const float* __restrict__ sd, LayerOut o) {
  const int t = blockIdx.y;
  const int r = 4 * (blockIdx.x * 256 + threadIdx.x);   // dim is a multiple of 256
  if (r >= dim) return;
  // the token's plan entries (its picks, then a quantised shared expert of weight 1: RN(1 * y) = y)
  int pp[kMaxSlots];
  float pw[kMaxSlots];
#pragma unroll
  for (int i = 0; i < kMaxSlots; ++i) {
    pp[i] = i <= topk ? plan.tok_pairs()[t * plan.slots() + i] : -1;
    pw[i] = pp[i] >= 0 ? plan.pair_w()[pp[i]] : 0.0f;
  }
  float4 yv[kMaxSlots];
#pragma unroll
  for (int i = 0; i < kMaxSlots; ++i)
    yv[i] = pp[i] >= 0 ? *reinterpret_cast<const float4*>(y + (int64_t)pp[i] * dim + r) : make_float4(0, 0, 0, 0);
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < kMaxSlots; ++i) {
    if (pp[i] >= 0) {
      const float v[4] = {yv[i].x, yv[i].y, yv[i].z, yv[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = fadd(acc[j], fmul(pw[i], v[j]));
    }
  }
  const int64_t i0 = (int64_t)t * dim + r;
  if (sd) {
    const float4 s4 = *reinterpret_cast<const float4*>(sd + i0);
    const float v[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = fadd(acc[j], v[j]);
  }
  const bool f32_vec = o.f32 && (((uintptr_t)o.f32 & 15) == 0);   // the caller's buffer: any 4-byte alignment
  if (f32_vec) *reinterpret_cast<float4*>(o.f32 + i0) = make_float4(acc[0], acc[1], acc[2], acc[3]);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (o.f32 && !f32_vec) o.f32[i0 + j] = acc[j];
    if (o.bf16) o.bf16[i0 + j] = bf16_rne(acc[j]);
    if (o.next) o.next[i0 + j] = bf16_rne(fadd(bf16_f32(o.resid[i0 + j]), acc[j]));
  }
}

constexpr int kGateUpSlots = 2;

template <int NSB>
hipError_t launch_gateup_t(const XArena& ex, int max_u, const moe_cfg& c, const Ws& w, hipStream_t s) {
  using G = GateUpGeom<NSB>;
  auto kern = k_gateup<NSB, kGateUpSlots>;
  const size_t shm = (size_t)kGateUpSlots * G::kTileBytes;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  MOE_LAUNCH(MOE_K_GATEUP, kern, dim3(max_u * (c.inter / 32)), dim3(256), shm, s, ex, w.plan, w.xq, w.xd, w.xs, c.dim,
             c.inter, w.g, w.u, w.h, w.hq, w.hd, w.hs, c.swiglu_limit);
  return hipGetLastError();
}

template <int NSB>
hipError_t launch_down_t(const XArena& ex, int m, int max_u, const moe_cfg& c, const Ws& w, const uint16_t* w2,
                         hipStream_t s) {
  using G = DownGeom<NSB>;
  auto kern = k_down<NSB>;
  // the two routed tiles, or (shared rows) every token's sh
  const size_t tiles = (size_t)(kDownRows / 16) * G::kSlotBytes, shs = (size_t)m * c.inter * 2;
  const size_t shm = w2 && shs > tiles ? shs : tiles;
  static bool attr_set = false;
  if (!attr_set) {
    const size_t most = (size_t)kMaxDecodeTokens * 256 * NSB * 2 > tiles ? (size_t)kMaxDecodeTokens * 256 * NSB * 2 : tiles;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)most);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int routed_blocks = max_u * (c.dim / kDownRows);
  const int shared_blocks = w2 ? c.dim / SharedDownGeom<NSB>::kRows : 0;
  MOE_LAUNCH(MOE_K_DOWN, kern, dim3(routed_blocks + shared_blocks), dim3(256), shm, s, ex, w.plan, w.hq, w.hd, w.hs,
             c.dim, c.inter, w.y, shared_blocks, m, w2, w.sh, w.sd);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gateup(const XArena& ex, int m, const moe_cfg& c, const Ws& w, hipStream_t s) {
  const int max_u = min(c.n_routed, m * c.topk) + ex.has_shared();
  hipError_t err;
  switch (c.dim / 256) {
    case 1: err = launch_gateup_t<1>(ex, max_u, c, w, s); break;
    case 2: err = launch_gateup_t<2>(ex, max_u, c, w, s); break;
    case 4: err = launch_gateup_t<4>(ex, max_u, c, w, s); break;
    case 8: err = launch_gateup_t<8>(ex, max_u, c, w, s); break;
    case 16: err = launch_gateup_t<16>(ex, max_u, c, w, s); break;
    default: err = hipErrorInvalidValue; break;
  }
  return err;
}

hipError_t launch_down(const XArena& ex, int m, const moe_cfg& c, const Ws& w, const uint16_t* w2,
                       hipStream_t s) {
  const int max_u = min(c.n_routed, m * c.topk) + ex.has_shared();
  hipError_t err;
  switch (c.inter / 256) {
    case 1: err = launch_down_t<1>(ex, m, max_u, c, w, w2, s); break;
    case 2: err = launch_down_t<2>(ex, m, max_u, c, w, w2, s); break;
    case 4: err = launch_down_t<4>(ex, m, max_u, c, w, w2, s); break;
    case 8: err = launch_down_t<8>(ex, m, max_u, c, w, w2, s); break;
    case 16: err = launch_down_t<16>(ex, m, max_u, c, w, w2, s); break;
    default: err = hipErrorInvalidValue; break;
  }
  return err;
}

hipError_t launch_combine(int m, const moe_cfg& c, const Ws& w, const float* sd, const LayerOut& o, hipStream_t s) {
  hipLaunchKernelGGL(k_combine, dim3((c.dim + 1023) / 1024, m), dim3(256), 0, s, w.plan, w.y, c.dim, c.topk, sd, o);
  return hipGetLastError();
}

}  // namespace moe
