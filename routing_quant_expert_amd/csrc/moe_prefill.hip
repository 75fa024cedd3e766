// Prefill: the layer for many tokens at once (A9) [moe_v41.rs, module doc;
// Kernels: the batched MoE path, "group by expert, int8 MFMA K-quant tiles"].
//
//  * k_router_pf: the router GEMV and scores with every (row, 8-token group)
//    pair as its own wave (the per-row summation order of the decode router,
//    so a token's logits are the same bits at any m), plus the q8_1 of x;
//  * k_group_count / k_group_fill: the (token, expert) pairs grouped by
//    expert, experts ascending, tokens ascending inside an expert (the same
//    plan the decode path builds), from the headers;
//  * k_gateup_pf: gate/up GEMMs on raw Q2_K blocks with int8 MFMA, fused
//    clamped SwiGLU and q8_1 of h;
//  * k_down_pf: down GEMMs on raw Q3_K blocks with int8 MFMA;
//  * k_shared_gu_pf / k_shared_down_pf: the bf16 shared expert as two bf16
//    MFMA GEMMs (f32 accumulation), SwiGLU fused into the first.
// The weighted combine in plan order is the decode path's k_combine.
//
// Numerics of the K-quant GEMMs (the same values as the decode GEMVs): an
// MFMA tile multiplies 32 tokens by 32 weight rows over one 32-wide q8_1
// block of k. The weight operand is the 2-bit (Q2_K) or 3-bit (Q3_K) code
// already multiplied by its 16-weight sub-block scale (still an int8), so the
// int32 result is the exact integer sum S_b = sum(sc * q * q8) of the block.
// Q2_K's sub-block minimum gives a second exact sum M_b = sum(m * q8) from a
// second MFMA whose weight operand is the minimum nibble repeated. Then per
// (row, token) in float64, exact products accumulated: over a super-block
// accS += d8_b * S_b, accM += d8_b * M_b, then y += d * accS - dmin * accM;
// y is rounded once to f32 at the end.
#include <hip/hip_runtime.h>

#include "moe_front.h"
#include "moe_internal.h"
#include "moe_kquant.h"
#include "moe_math.h"
#include "moe_prefill.h"

namespace moe {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));   // 16 bytes, 4-byte aligned
typedef uint32_t u32x4a2 __attribute__((ext_vector_type(4), aligned(2)));   // 16 bytes, 2-byte aligned
typedef uint32_t u32x2a2 __attribute__((ext_vector_type(2), aligned(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kChunk = 16;   // tokens of one expert per MFMA pass (rows 16..31 of the token operand are zero)
constexpr int kGroups = kChunk / 8;

__device__ __forceinline__ i32x16 mfma_i8(i32x4 a, i32x4 b) {
  const i32x16 z = {};
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, z, 0, 0, 0);
}

// Register r of a 32x32 MFMA result in lane l holds row 8*(r/4) + 4*(l/32) +
// r%4 (the token of the tile) and column l%32 (the weight row).
__device__ __forceinline__ int tile_tok(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// ---------------------------------------------------------------------------
// Router + q8_1 of x for m tokens. Grid (router rows / 4, ceil(m / 8)) plus
// the quantisation workgroups in the first grid row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_router_pf(const uint16_t* __restrict__ x, int m, int dim,
                                                   const uint16_t* __restrict__ gate_w, int n_routed, float temp,
                                                   int router_blocks, Ws w, float* __restrict__ logits_out) {
  const int bx = blockIdx.x;
  if (bx == 0 && blockIdx.y == 0 && threadIdx.x < 4) w.status[threadIdx.x] = 0;   // every entry point starts here
  if (bx < router_blocks) {
    const int t_lo = 8 * blockIdx.y;
    front::router_rows(bx, x, m, dim, gate_w, n_routed, temp, w.logits, w.scores, logits_out, t_lo,
                       min(m, t_lo + 8));
    return;
  }
  const int qb = (bx - router_blocks) * gridDim.y + blockIdx.y;
  if (qb < (int)((int64_t)m * dim / 256)) front::quant_x_block(qb, x, w.xq, w.xd, w.xs);
}

// ---------------------------------------------------------------------------
// Grouping by expert. Scratch `grp` (int32): tok_ok [m], e_first [n_routed],
// e_count [n_routed].
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_group_count(const int32_t* __restrict__ header, int m, int topk, int n_routed,
                                                     PlanView plan, int32_t* __restrict__ grp,
                                                     int32_t* __restrict__ status) {
  __shared__ int cnt[kMaxRouted];
  __shared__ int wtot[2][16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hw = 1 + 3 * topk;
  int32_t* tok_ok = grp;
  int32_t* e_first = grp + m;
  int32_t* e_count = e_first + n_routed;
  for (int e = tid; e < n_routed; e += 1024) cnt[e] = 0;
  __syncthreads();
  bool bad_any = false;
  for (int t = tid; t < m; t += 1024) {
    const int32_t* h = header + (int64_t)t * hw + 1;
    int p[kMaxTopk];
    bool ok = true;
#pragma unroll
    for (int r = 0; r < kMaxTopk; ++r) {
      p[r] = r < topk ? h[r] : 0;
      if (r < topk && (p[r] < 0 || p[r] >= n_routed)) ok = false;
#pragma unroll
      for (int r2 = 0; r2 < r; ++r2)
        if (r < topk && p[r2] == p[r]) ok = false;
    }
    tok_ok[t] = ok ? 1 : 0;
#pragma unroll
    for (int r = 0; r < kMaxTopk; ++r) {
      if (r < topk) {
        if (ok) atomicAdd(&cnt[p[r]], 1);
        else plan.tok_pairs()[(int64_t)t * topk + r] = -1;
      }
    }
    bad_any |= !ok;
  }
  if (bad_any) atomicOr(status, MOE_STATUS_BAD_PICK);
  __syncthreads();
  // exclusive prefix sums over the experts of the pair counts and of (count > 0)
  const int c = tid < n_routed ? cnt[tid] : 0;
  int v = c, f = c > 0 ? 1 : 0;
  for (int s = 1; s < 64; s <<= 1) {
    const int a = __shfl_up(v, s), b = __shfl_up(f, s);
    if (lane >= s) {
      v += a;
      f += b;
    }
  }
  if (lane == 63) {
    wtot[0][wave] = v;
    wtot[1][wave] = f;
  }
  __syncthreads();
  int bv = 0, bf = 0;
  for (int i = 0; i < wave; ++i) {
    bv += wtot[0][i];
    bf += wtot[1][i];
  }
  const int first = bv + v - c, uid = bf + f - (c > 0 ? 1 : 0);
  if (tid < n_routed) {
    e_first[tid] = first;
    e_count[tid] = c;
    if (c > 0) {
      plan.u_expert()[uid] = tid;
      plan.u_first()[uid] = first;
      plan.u_npairs()[uid] = c;
    }
  }
  if (tid == 1023) {   // totals over all 16 waves (threads past n_routed add 0)
    *plan.n_pairs() = bv + v;
    *plan.n_u() = bf + f;
  }
}

// One wave per expert e: its pairs in ascending token order (a ballot over
// the flattened picks), their weights, and each token's pair index at the
// rank of e among the token's picks (plan order = ascending id).
__global__ __launch_bounds__(64) void k_group_fill(const int32_t* __restrict__ header, int m, int topk, int n_routed,
                                                   PlanView plan, const int32_t* __restrict__ grp) {
  const int e = blockIdx.x, lane = threadIdx.x;
  const int32_t* tok_ok = grp;
  const int32_t* e_first = grp + m;
  const int32_t* e_count = e_first + n_routed;
  if (e_count[e] == 0) return;
  int pos = e_first[e];
  const int hw = 1 + 3 * topk;
  const int64_t P = (int64_t)m * topk;
  for (int64_t q0 = 0; q0 < P; q0 += 64) {
    const int64_t q = q0 + lane;
    int t = 0, r = 0;
    bool hit = false;
    if (q < P) {
      t = (int)(q / topk);
      r = (int)(q - (int64_t)t * topk);
      hit = header[(int64_t)t * hw + 1 + r] == e && tok_ok[t] != 0;
    }
    const unsigned long long mask = __ballot(hit);
    if (hit) {
      const int p = pos + __popcll(mask & ((1ull << lane) - 1ull));
      const int32_t* h = header + (int64_t)t * hw;
      plan.pair_tok()[p] = t;
      plan.pair_expert()[p] = e;
      plan.pair_w()[p] = __builtin_bit_cast(float, h[1 + topk + r]);
      int slot = 0;
      for (int r2 = 0; r2 < topk; ++r2) slot += h[1 + r2] < e ? 1 : 0;
      plan.tok_pairs()[(int64_t)t * topk + slot] = p;
    }
    pos += __popcll(mask);
  }
}

// ---------------------------------------------------------------------------
// Gate/up on Q2_K with int8 MFMA + clamped SwiGLU + q8_1 of h.
// Workgroup = (distinct expert u, 32 hidden units). Waves: (gate | up) x
// (first | second half of the q8_1 blocks of k); each wave computes its 32
// rows for up to 16 of the expert's tokens at a time, the halves are added
// in float64 through LDS, then the SwiGLU and the q8_1 of h (32 units = one
// q8_1 block) are written per pair.
// ---------------------------------------------------------------------------
struct GateUpPfArgs {
  moe_experts ex;
  PlanView plan;
  const int8_t* xq;
  const uint16_t* xd;
  int inter;
  float L;
  float* g;
  float* u;
  float* h;
  int8_t* hq;
  uint16_t* hd;
  int32_t* hs;
};

// LDS table indexed by a Q2_K scales byte (low nibble sc, high nibble m):
// word 0 = bytes {0, sc, 2sc, 3sc} (code -> sc * code by v_perm), word 1 = m
// in every byte.
__device__ __forceinline__ void q2k_lut_fill(uint32_t (*lut)[2]) {
  const uint32_t v = threadIdx.x;
  if (v < 256) {
    const uint32_t sc = v & 15u, mn = v >> 4;
    lut[v][0] = (sc * 0x030201u) << 8;
    lut[v][1] = mn * 0x01010101u;
  }
}

template <int NSB, int G>
__device__ __forceinline__ void gateup_pf_tile(const uint8_t* __restrict__ wrow, const int8_t* __restrict__ arow,
                                               const double (*d8)[kChunk], const uint32_t (*lut)[2], int kh,
                                               double (&y)[4 * G]) {
  const int lane = threadIdx.x & 63, hl = lane >> 5;
  constexpr int kSbPer = NSB >= 2 ? NSB / 2 : 1;
  const int sb0 = NSB >= 2 ? kh * kSbPer : 0;
#pragma unroll
  for (int r = 0; r < 4 * G; ++r) y[r] = 0.0;
#pragma unroll 1
  for (int sb = sb0; sb < sb0 + kSbPer; ++sb) {
    const uint8_t* blk = wrow + sb * kQ2KBytes;
    const u32x4a4 scv = *reinterpret_cast<const u32x4a4*>(blk);
    const u32x4a4 qv0 = *reinterpret_cast<const u32x4a4*>(blk + 16 + 16 * hl);
    const u32x4a4 qv1 = *reinterpret_cast<const u32x4a4*>(blk + 48 + 16 * hl);
    const uint32_t ddw = *reinterpret_cast<const uint32_t*>(blk + 80);
    double accS[4 * G], accM[4 * G];
#pragma unroll
    for (int r = 0; r < 4 * G; ++r) accS[r] = accM[r] = 0.0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (NSB == 1 && (t >> 2) != kh) continue;   // one super-block: the halves split its q8_1 blocks
      const int b = 8 * sb + t, j = t & 3;
      const i32x4 A = *reinterpret_cast<const i32x4*>(arow + 32 * b);
      const u32x4a4 qw = t < 4 ? qv0 : qv1;
      const uint32_t sbyte = (scv[t >> 1] >> (8 * (2 * (t & 1) + hl))) & 0xFFu;
      const uint32_t lut_s = lut[sbyte][0], mrep = lut[sbyte][1];
      i32x4 Bs;
#pragma unroll
      for (int i = 0; i < 4; ++i) Bs[i] = (int)__builtin_amdgcn_perm(lut_s, lut_s, (qw[i] >> (2 * j)) & 0x03030303u);
      const i32x4 Bm = {(int)mrep, (int)mrep, (int)mrep, (int)mrep};
      const i32x16 S = mfma_i8(A, Bs);
      const i32x16 M = mfma_i8(A, Bm);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const double* dp = &d8[b][8 * g + 4 * hl];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          accS[4 * g + i] = __builtin_fma(dp[i], (double)S[4 * g + i], accS[4 * g + i]);
          accM[4 * g + i] = __builtin_fma(dp[i], (double)M[4 * g + i], accM[4 * g + i]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // one block's MFMA results live at a time
    }
    const double d = fp16_f64(ddw & 0xFFFFu), dmin = fp16_f64(ddw >> 16);
#pragma unroll
    for (int r = 0; r < 4 * G; ++r) y[r] = __builtin_fma(-dmin, accM[r], __builtin_fma(d, accS[r], y[r]));
  }
}

template <int NSB>
__global__ __launch_bounds__(256) void k_gateup_pf(GateUpPfArgs a) {
  constexpr int dim = 256 * NSB, NB = 8 * NSB;
  __shared__ double d8[NB][kChunk];
  __shared__ double xch[2][kChunk][32];   // the second half's partial sums
  __shared__ float gu[2][kChunk][32];
  __shared__ uint32_t lut[256][2];
  const int ngr = a.inter / 32;
  const int u = blockIdx.x / ngr, grp = blockIdx.x % ngr;
  if (u >= *a.plan.n_u()) return;
  const int e = a.plan.u_expert()[u], first = a.plan.u_first()[u], np = a.plan.u_npairs()[u];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hl = lane >> 5;
  const int mat = wave & 1, kh = wave >> 1;
  q2k_lut_fill(lut);
  const uint8_t* wrow = (const uint8_t*)a.ex.base + (uint64_t)e * a.ex.stride + (mat ? a.ex.up_off : a.ex.gate_off) +
                        (uint64_t)(32 * grp + (lane & 31)) * (NSB * kQ2KBytes);
  for (int c0 = 0; c0 < np; c0 += kChunk) {
    const int nt = min(kChunk, np - c0);
    const int* ptok = a.plan.pair_tok() + first + c0;
    __syncthreads();   // the previous chunk is done with d8 / gu
    for (int i = tid; i < NB * kChunk; i += 256) {
      const int jt = i / NB, b = i % NB;
      d8[b][jt] = jt < nt ? fp16_f64(a.xd[(int64_t)ptok[jt] * NB + b]) : 0.0;
    }
    // token rows past the chunk repeat its last token: their results are never stored
    const int ja = min(lane & 31, nt - 1);
    const int8_t* arow = a.xq + (int64_t)ptok[ja] * dim + 16 * hl;
    __syncthreads();
    double y[4 * kGroups];
    if (nt > 8) {
      gateup_pf_tile<NSB, 2>(wrow, arow, d8, lut, kh, y);
    } else {
      double y1[4];
      gateup_pf_tile<NSB, 1>(wrow, arow, d8, lut, kh, y1);
#pragma unroll
      for (int r = 0; r < 4; ++r) y[r] = y1[r];
#pragma unroll
      for (int r = 4; r < 4 * kGroups; ++r) y[r] = 0.0;
    }
    if (kh == 1) {
#pragma unroll
      for (int r = 0; r < 4 * kGroups; ++r) xch[mat][tile_tok(r, lane)][lane & 31] = y[r];
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
      for (int r = 0; r < 4 * kGroups; ++r) {
        const int tt = tile_tok(r, lane);
        gu[mat][tt][lane & 31] = (float)(y[r] + xch[mat][tt][lane & 31]);
      }
    }
    __syncthreads();
    // SwiGLU + q8_1 of h: a half-wave per token, a lane per hidden unit
    const int unit = lane & 31;
#pragma unroll 1
    for (int tt = 2 * wave + hl; tt < kChunk; tt += 8) {
      const bool live = tt < nt;
      const float gv = gu[0][tt][unit], uv = gu[1][tt][unit];
      const float hv = live ? swiglu(gv, uv, a.L) : 0.0f;
      float am = fabsf(hv);
      for (int s = 16; s >= 1; s >>= 1) am = fmaxf(am, __shfl_xor(am, s));
      const float d = (float)((double)am / 127.0);
      const int q = am == 0.0f ? 0 : q8_code(hv, d);
      int sum = q;
      for (int s = 8; s >= 1; s >>= 1) sum += __shfl_xor(sum, s);
      if (live) {
        const int64_t pair = first + c0 + tt;
        const int64_t o = pair * a.inter + 32 * grp + unit;
        a.g[o] = gv;
        a.u[o] = uv;
        a.h[o] = hv;
        a.hq[o] = (int8_t)q;
        if (unit == 0) a.hd[pair * (a.inter / 32) + grp] = f32_to_fp16_bits(d);
        if ((unit & 15) == 0) a.hs[pair * (a.inter / 16) + 2 * grp + (unit >> 4)] = sum;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Down on Q3_K with int8 MFMA. Workgroup = (distinct expert u, 128 output
// rows), a wave per 32 rows over the whole k, up to 16 pairs at a time.
// A weight is v = q2 + 4*hb - 4 in [-4, 3] with the 6-bit sub-block scale
// s = u6 - 32 in [-32, 31]; the int8 operand is -(v * s) = (4 - idx) * s for
// idx = q2 + 4*hb, which always fits an int8 ([-128, 124]), looked up with
// v_perm from an 8-byte table per scale value. The MFMA sum is -S_b.
// ---------------------------------------------------------------------------
struct DownPfArgs {
  moe_experts ex;
  PlanView plan;
  const int8_t* hq;
  const uint16_t* hd;
  int dim;
  float* y;
};

__device__ __forceinline__ void q3k_lut_fill(uint32_t (*lut)[2]) {
  const int v = threadIdx.x;
  if (v < 64) {
    const int s = v - 32;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= (uint32_t)(((4 - i) * s) & 0xFF) << (8 * i);
      hi |= (uint32_t)(((4 - (i + 4)) * s) & 0xFF) << (8 * i);
    }
    lut[v][0] = lo;
    lut[v][1] = hi;
  }
}

template <int NSB, int G>
__device__ __forceinline__ void down_pf_tile(const uint8_t* __restrict__ wrow, const int8_t* __restrict__ arow,
                                             const double (*d8)[kChunk], const uint32_t (*lut)[2],
                                             double (&y)[4 * G]) {
  const int lane = threadIdx.x & 63, hl = lane >> 5;
#pragma unroll
  for (int r = 0; r < 4 * G; ++r) y[r] = 0.0;
#pragma unroll 1
  for (int sb = 0; sb < NSB; ++sb) {
    const uint8_t* blk = wrow + sb * kQ3KBytes;
    const u32x4a2 hmv = *reinterpret_cast<const u32x4a2*>(blk + 16 * hl);
    const u32x4a2 qv0 = *reinterpret_cast<const u32x4a2*>(blk + 32 + 16 * hl);
    const u32x4a2 qv1 = *reinterpret_cast<const u32x4a2*>(blk + 64 + 16 * hl);
    const u32x2a2 sc01 = *reinterpret_cast<const u32x2a2*>(blk + 96);
    const uint32_t sc2 = (uint32_t)reinterpret_cast<const uint16_t*>(blk + 104)[0] |
                         ((uint32_t)reinterpret_cast<const uint16_t*>(blk + 104)[1] << 16);
    const uint32_t dbits = reinterpret_cast<const uint16_t*>(blk + 108)[0];
    double acc[4 * G];
#pragma unroll
    for (int r = 0; r < 4 * G; ++r) acc[r] = 0.0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int b = 8 * sb + t, h = t >> 2, j = t & 3;
      // sub-block s = 2t + hl: low 4 bits from byte (s % 8) (low nibble for s < 8, else high), high 2 bits
      // from byte 8 + s % 4 at bit 2 * (s / 4)
      const int sl = 2 * (t & 3) + hl;   // s % 8
      const uint32_t lob = ((sl < 4 ? sc01[0] : sc01[1]) >> (8 * (sl & 3))) & 0xFFu;
      const uint32_t lo = t < 4 ? (lob & 15u) : (lob >> 4);
      const uint32_t hib = (sc2 >> (8 * (2 * (t & 1) + hl))) & 0xFFu;
      const uint32_t hi = (hib >> (2 * (t >> 1))) & 3u;
      const uint32_t u6 = lo | (hi << 4);
      const uint32_t lut_lo = lut[u6][0], lut_hi = lut[u6][1];
      const u32x4a2 qw = t < 4 ? qv0 : qv1;
      const int hbit = 4 * h + j;   // the hmask bit of this q8_1 block
      i32x4 B;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t q2 = (qw[i] >> (2 * j)) & 0x03030303u;
        const uint32_t hb = hbit >= 2 ? (hmv[i] >> (hbit - 2)) : (hmv[i] << (2 - hbit));
        B[i] = (int)__builtin_amdgcn_perm(lut_hi, lut_lo, (hb & 0x04040404u) | q2);
      }
      const i32x4 A = *reinterpret_cast<const i32x4*>(arow + 32 * b);
      const i32x16 S = mfma_i8(A, B);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const double* dp = &d8[b][8 * g + 4 * hl];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[4 * g + i] = __builtin_fma(dp[i], (double)S[4 * g + i], acc[4 * g + i]);
      }
      __builtin_amdgcn_sched_barrier(0);   // one block's MFMA result live at a time
    }
    const double nd = -fp16_f64(dbits);   // the MFMA sums are -S_b
#pragma unroll
    for (int r = 0; r < 4 * G; ++r) y[r] = __builtin_fma(nd, acc[r], y[r]);
  }
}

template <int NSB>
__global__ __launch_bounds__(256) void k_down_pf(DownPfArgs a) {
  constexpr int inter = 256 * NSB, NB = 8 * NSB;
  __shared__ double d8[NB][kChunk];
  __shared__ uint32_t lut[64][2];
  const int nrt = a.dim / 128;
  const int u = blockIdx.x / nrt, rt = blockIdx.x % nrt;
  if (u >= *a.plan.n_u()) return;
  const int e = a.plan.u_expert()[u], first = a.plan.u_first()[u], np = a.plan.u_npairs()[u];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hl = lane >> 5;
  q3k_lut_fill(lut);
  const int row = 128 * rt + 32 * wave + (lane & 31);
  const uint8_t* wrow =
      (const uint8_t*)a.ex.base + (uint64_t)e * a.ex.stride + a.ex.down_off + (uint64_t)row * (NSB * kQ3KBytes);
  for (int c0 = 0; c0 < np; c0 += kChunk) {
    const int nt = min(kChunk, np - c0);
    const int64_t p0 = first + c0;
    __syncthreads();
    for (int i = tid; i < NB * kChunk; i += 256) {
      const int jt = i / NB, b = i % NB;
      d8[b][jt] = jt < nt ? fp16_f64(a.hd[(p0 + jt) * NB + b]) : 0.0;
    }
    const int ja = min(lane & 31, nt - 1);   // rows past the chunk repeat its last pair (results not stored)
    const int8_t* arow = a.hq + (p0 + ja) * inter + 16 * hl;
    __syncthreads();
    if (nt > 8) {
      double y[8];
      down_pf_tile<NSB, 2>(wrow, arow, d8, lut, y);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int tt = tile_tok(r, lane);
        if (tt < nt) a.y[(p0 + tt) * a.dim + row] = (float)y[r];
      }
    } else {
      double y[4];
      down_pf_tile<NSB, 1>(wrow, arow, d8, lut, y);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tt = tile_tok(r, lane);
        if (tt < nt) a.y[(p0 + tt) * a.dim + row] = (float)y[r];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Shared expert, bf16 MFMA (v_mfma_f32_32x32x16_bf16: lane l holds 8
// consecutive k of operand row l%32 at k offset 8*(l/32)); f32 accumulation
// in the MFMA's order [moe_v41.rs, module doc: the shared expert runs on the
// dense bf16 GEMM].
// gate/up: a wave = 32 tokens x 32 hidden units, gate and up; a workgroup =
// 4 waves over 128 units sharing the token rows; then sh = bf16(SwiGLU).
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 ld_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(p));
}

__global__ __launch_bounds__(256) void k_shared_gu_pf(const uint16_t* __restrict__ x, int m, int dim, int inter,
                                                      const uint16_t* __restrict__ w1, const uint16_t* __restrict__ w3,
                                                      float* __restrict__ sg, float* __restrict__ su,
                                                      uint16_t* __restrict__ sh, float L) {
  __shared__ float tile[2][32][128 + 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hl = lane >> 5;
  const int tok0 = 32 * blockIdx.y, unit0 = 128 * blockIdx.x;
  const int ta = tok0 + (lane & 31);
  const int un = unit0 + 32 * wave + (lane & 31);
  const uint16_t* xa = x + (int64_t)min(ta, m - 1) * dim + 8 * hl;
  const uint16_t* ga = w1 + (int64_t)un * dim + 8 * hl;
  const uint16_t* ua = w3 + (int64_t)un * dim + 8 * hl;
  f32x16 cg = {}, cu = {};
  const bool arow_ok = ta < m;
#pragma unroll 4
  for (int k = 0; k < dim; k += 16) {
    bf16x8 av = ld_bf16x8(xa + k);
    if (!arow_ok) av = bf16x8{};
    cg = mfma_bf16(av, ld_bf16x8(ga + k), cg);
    cu = mfma_bf16(av, ld_bf16x8(ua + k), cu);
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
  const int tok0 = 32 * blockIdx.y;
  const int ta = tok0 + (lane & 31);
  const int row = 128 * blockIdx.x + 32 * wave + (lane & 31);
  const uint16_t* ha = sh + (int64_t)min(ta, m - 1) * inter + 8 * hl;
  const uint16_t* wa = w2 + (int64_t)row * inter + 8 * hl;
  const bool arow_ok = ta < m;
  f32x16 c = {};
#pragma unroll 4
  for (int k = 0; k < inter; k += 16) {
    bf16x8 av = ld_bf16x8(ha + k);
    if (!arow_ok) av = bf16x8{};
    c = mfma_bf16(av, ld_bf16x8(wa + k), c);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int t = tok0 + tile_tok(r, lane);
    if (t < m) sd[(int64_t)t * dim + row] = c[r];
  }
}

template <int NSB>
hipError_t launch_gateup_pf_t(const GateUpPfArgs& a, int max_u, hipStream_t s) {
  MOE_LAUNCH(MOE_K_GATEUP, k_gateup_pf<NSB>, dim3(max_u * (a.inter / 32)), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int NSB>
hipError_t launch_down_pf_t(const DownPfArgs& a, int max_u, hipStream_t s) {
  MOE_LAUNCH(MOE_K_DOWN, k_down_pf<NSB>, dim3(max_u * (a.dim / 128)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router_pf(const uint16_t* x, int m, const uint16_t* gate_w, const moe_cfg& c, const Ws& w,
                            float* logits_out, hipStream_t s) {
  const int router_blocks = (c.n_routed + 3) / 4;
  const int tgroups = (m + 7) / 8;
  const int64_t quant = (int64_t)m * c.dim / 256;
  const int quant_cols = (int)((quant + tgroups - 1) / tgroups);
  MOE_LAUNCH(MOE_K_ROUTER, k_router_pf, dim3(router_blocks + quant_cols, tgroups), dim3(256), 0, s, x, m, c.dim,
             gate_w, c.n_routed, c.gate_temp, router_blocks, w, logits_out);
  return hipGetLastError();
}

hipError_t launch_group(const int32_t* header, int m, const moe_cfg& c, const Ws& w, int32_t* grp, hipStream_t s) {
  hipLaunchKernelGGL(k_group_count, dim3(1), dim3(1024), 0, s, header, m, c.topk, c.n_routed, w.plan, grp, w.status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_group_fill, dim3(c.n_routed), dim3(64), 0, s, header, m, c.topk, c.n_routed, w.plan, grp);
  return hipGetLastError();
}

hipError_t launch_gateup_pf(const moe_experts& ex, int m, const moe_cfg& c, const Ws& w, hipStream_t s) {
  const int max_u = min(c.n_routed, m * c.topk);
  GateUpPfArgs a{ex, w.plan, w.xq, w.xd, c.inter, c.swiglu_limit, w.g, w.u, w.h, w.hq, w.hd, w.hs};
  switch (c.dim / 256) {
    case 1: return launch_gateup_pf_t<1>(a, max_u, s);
    case 2: return launch_gateup_pf_t<2>(a, max_u, s);
    case 4: return launch_gateup_pf_t<4>(a, max_u, s);
    case 8: return launch_gateup_pf_t<8>(a, max_u, s);
    case 16: return launch_gateup_pf_t<16>(a, max_u, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_down_pf(const moe_experts& ex, int m, const moe_cfg& c, const Ws& w, hipStream_t s) {
  const int max_u = min(c.n_routed, m * c.topk);
  DownPfArgs a{ex, w.plan, w.hq, w.hd, c.dim, w.y};
  switch (c.inter / 256) {
    case 1: return launch_down_pf_t<1>(a, max_u, s);
    case 2: return launch_down_pf_t<2>(a, max_u, s);
    case 4: return launch_down_pf_t<4>(a, max_u, s);
    case 8: return launch_down_pf_t<8>(a, max_u, s);
    case 16: return launch_down_pf_t<16>(a, max_u, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_shared_pf(const uint16_t* x, int m, const moe_layer& layer, const moe_cfg& c, const Ws& w,
                            hipStream_t s) {
  const int tt = (m + 31) / 32;
  MOE_LAUNCH(MOE_K_SHARED_GU, k_shared_gu_pf, dim3(c.inter / 128, tt), dim3(256), 0, s, x, m, c.dim, c.inter,
             layer.sh_w1, layer.sh_w3, w.sg, w.su, w.sh, c.swiglu_limit);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  MOE_LAUNCH(MOE_K_SHARED_DOWN, k_shared_down_pf, dim3(c.dim / 128, tt), dim3(256), 0, s, w.sh, m, c.dim, c.inter,
             layer.sh_w2, w.sd);
  return hipGetLastError();
}

}  // namespace moe
