// Prefill: the layer for many tokens at once (A9) [moe_v41.rs, module doc;
// struct Kernels: gather, scatter_add and the mmq_q2k_* / mmq_q3k_* handles;
// struct MoeV41: the gathered rows and q8_1 activations of one expert group,
// the group-major token rows and weights]. The int8 MFMA tiles below are this
// library's own design for CDNA4.
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
//  (the bf16 shared expert's two GEMMs are in moe_shared_pf.hip).
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
#include "moe_wave.h"
#include "moe_prefill.h"

namespace moe {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));   // 16 bytes, 4-byte aligned
typedef uint32_t u32x4a2 __attribute__((ext_vector_type(4), aligned(2)));   // 16 bytes, 2-byte aligned
typedef uint32_t u32x2a2 __attribute__((ext_vector_type(2), aligned(2)));

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
// Router + q8_1 of x for m tokens. A wave computes 4 expert rows for 8
// tokens (each converted bf16 chunk of x serves 4 rows, each of w 8 tokens);
// every (row, token) is summed in the decode router's order: lane l adds
// fmul(x, w) for positions 512*i + 8*l + j, i ascending, j = 0..7, in f32
// without contraction, then the 64 partials combine by p += shfl_xor(p, s)
// for s = 32 .. 1, so a token's logits are the same bits at any m. Grid
// (router groups of 16 rows, ceil(m / 8)) plus the quantisation workgroups.
// ---------------------------------------------------------------------------
constexpr int kRpRows = 4;
constexpr int kRpTok = 8;

__device__ inline void bf16x8_f32(uint4 v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = bf16_f32((uint16_t)(w[j >> 1] >> (16 * (j & 1))));
}

__device__ void router_rows4(int e0, int t0, const uint16_t* __restrict__ x, int m, int dim,
                             const uint16_t* __restrict__ gate_w, int n_routed, float temp,
                             float* __restrict__ logits, float* __restrict__ scores,
                             float* __restrict__ logits_out, const ScoreTable& st) {
  const int lane = threadIdx.x & 63;
  const int nt = min(kRpTok, m - t0);
  float p[kRpRows][kRpTok];
#pragma unroll
  for (int r = 0; r < kRpRows; ++r)
#pragma unroll
    for (int t = 0; t < kRpTok; ++t) p[r][t] = 0.0f;
  const int nch = dim / 512;   // dim is a multiple of 256; a half chunk is handled below
#pragma unroll 1
  for (int c = 0; c * 512 < dim; ++c) {
    const int k = 512 * c + 8 * lane;
    const bool in = k < dim;
    float wf[kRpRows][8];
#pragma unroll
    for (int r = 0; r < kRpRows; ++r) {
      const int e = min(e0 + r, n_routed - 1);
      const uint4 v = in ? *reinterpret_cast<const uint4*>(gate_w + (int64_t)e * dim + k) : make_uint4(0, 0, 0, 0);
      bf16x8_f32(v, wf[r]);
    }
#pragma unroll
    for (int t = 0; t < kRpTok; ++t) {
      const int tt = min(t0 + t, m - 1);
      const uint4 v = in ? *reinterpret_cast<const uint4*>(x + (int64_t)tt * dim + k) : make_uint4(0, 0, 0, 0);
      float xf[8];
      bf16x8_f32(v, xf);
#pragma unroll
      for (int r = 0; r < kRpRows; ++r) {
        float acc = p[r][t];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc = fadd(acc, fmul(xf[j], wf[r][j]));   // zero padding adds +0: exact
        p[r][t] = acc;
      }
    }
  }
  (void)nch;
#pragma unroll
  for (int r = 0; r < kRpRows; ++r)
#pragma unroll
    for (int t = 0; t < kRpTok; ++t) p[r][t] = wave_sum_xor(p[r][t]);
  // lane 8r + t writes (row e0 + r, token t0 + t)
  if (lane < kRpRows * kRpTok) {
    const int r = lane >> 3, t = lane & 7;
    float lg = 0.0f;
#pragma unroll
    for (int rr = 0; rr < kRpRows; ++rr)
#pragma unroll
      for (int q = 0; q < kRpTok; ++q)
        if (rr == r && q == t) lg = p[rr][q];
    const int e = e0 + r;
    if (t < nt && e < n_routed) {
      const int64_t o = (int64_t)(t0 + t) * n_routed + e;
      logits[o] = lg;
      if (logits_out) logits_out[o] = lg;
      scores[o] = score_mode_of(lg, temp, st);
    }
  }
}

__global__ __launch_bounds__(256) void k_router_pf(const uint16_t* __restrict__ x, int m, int dim,
                                                   const uint16_t* __restrict__ gate_w, int n_routed, float temp,
                                                   int router_blocks, Ws w, float* __restrict__ logits_out,
                                                   ScoreTable st) {
  const int bx = blockIdx.x;
  if (bx == 0 && blockIdx.y == 0 && threadIdx.x < 4) w.status[threadIdx.x] = 0;   // every entry point starts here
  if (bx < router_blocks) {
    const int e0 = (4 * bx + (threadIdx.x >> 6)) * kRpRows;
    if (e0 < n_routed)
      router_rows4(e0, kRpTok * blockIdx.y, x, m, dim, gate_w, n_routed, temp, w.logits, w.scores, logits_out, st);
    return;
  }
  const int qb = (bx - router_blocks) * gridDim.y + blockIdx.y;
  if (qb < (int)((int64_t)m * dim / 256)) front::quant_x_block(qb, x, w.xq, w.xd, w.xs, w.xd64);
}

// ---------------------------------------------------------------------------
// Grouping by expert. Scratch `grp` (int32): tok_ok [m], e_first [n_routed],
// e_count [n_routed].
// ---------------------------------------------------------------------------
// shq = 1: every token that keeps its picks also gets the layer's quantised
// shared expert (id n_routed, weight 1): one more group after all routed
// ones, holding those tokens in ascending order.
__global__ __launch_bounds__(1024) void k_group_count(const int32_t* __restrict__ header, int m, int topk, int n_routed,
                                                     PlanView plan, int32_t* __restrict__ grp,
                                                     int32_t* __restrict__ status, int shq) {
  __shared__ int cnt[kMaxRouted];
  __shared__ int wtot[2][16];
  __shared__ int n_ok;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hw = 1 + 3 * topk;
  const int slots = plan.slots();
  int32_t* tok_ok = grp;
  int32_t* e_first = grp + m;
  int32_t* e_count = e_first + n_routed + 1;
  for (int e = tid; e < n_routed; e += 1024) cnt[e] = 0;
  if (tid == 0) n_ok = 0;
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
        else plan.tok_pairs()[(int64_t)t * slots + r] = -1;
      }
    }
    if (ok && shq) atomicAdd(&n_ok, 1);
    else plan.tok_pairs()[(int64_t)t * slots + topk] = -1;   // no shared entry (k_group_fill writes the others)
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
  if (tid == 1023) {   // totals over all 16 waves (threads past n_routed add 0), then the shared group
    const int np = bv + v, nu = bf + f;
    e_first[n_routed] = np;
    e_count[n_routed] = n_ok;
    // the shared group holds every kept token: its plan entries take kChunk tokens each, one MFMA pass,
    // so that its workgroups spread over the device instead of looping over all the tokens
    const int nsh = (n_ok + kChunk - 1) / kChunk;
    for (int j = 0; j < nsh; ++j) {
      plan.u_expert()[nu + j] = n_routed;
      plan.u_first()[nu + j] = np + kChunk * j;
      plan.u_npairs()[nu + j] = min(kChunk, n_ok - kChunk * j);
    }
    *plan.n_pairs() = np + n_ok;
    *plan.n_u() = nu + nsh;
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
  const int32_t* e_count = e_first + n_routed + 1;
  if (e_count[e] == 0) return;
  int pos = e_first[e];
  const int hw = 1 + 3 * topk;
  const int slots = plan.slots();
  if (e == n_routed) {   // the quantised shared expert: every token that keeps its picks, ascending, weight 1
    for (int t0 = 0; t0 < m; t0 += 64) {
      const int t = t0 + lane;
      const bool hit = t < m && tok_ok[t] != 0;
      const unsigned long long mask = __ballot(hit);
      if (hit) {
        const int p = pos + __popcll(mask & ((1ull << lane) - 1ull));
        plan.pair_tok()[p] = t;
        plan.pair_expert()[p] = e;
        plan.pair_w()[p] = 1.0f;
        plan.tok_pairs()[(int64_t)t * slots + topk] = p;
      }
      pos += __popcll(mask);
    }
    return;
  }
  const int64_t P = (int64_t)m * topk;
  // kB rows of 64 picks at a time: their loads are all issued before any
  // ballot (the plan stores in between would otherwise keep each row's loads
  // waiting behind the previous row's)
  // (token, slot) of pick q advances by (64 / topk, 64 % topk) per row of 64: one division per batch
  constexpr int kB = 16;
  const int dt = 64 / topk, dr = 64 - dt * topk;
  for (int64_t q0 = 0; q0 < P; q0 += 64 * kB) {
    int pk[kB], ok[kB], wbits[kB], tb[kB], rb[kB];
    const int qb = (int)q0 + lane;   // P = m * topk < 2^31
    int t = qb / topk, r = qb - t * topk;
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const int tc = min(t, m - 1);   // rows past the end read the last token (no hit there)
      const int32_t* h = header + (int64_t)tc * hw;
      pk[b] = h[1 + r];
      wbits[b] = h[1 + topk + r];
      ok[b] = tok_ok[tc];
      tb[b] = t;
      rb[b] = r;
      t += dt;
      r += dr;
      if (r >= topk) {
        r -= topk;
        ++t;
      }
    }
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const int64_t q = q0 + 64 * b + lane;
      const bool hit = q < P && pk[b] == e && ok[b] != 0;
      const unsigned long long mask = __ballot(hit);
      if (mask == 0ull) continue;   // (wave-uniform) no pair of e in this row
      const int t = tb[b], r = rb[b];
      // the token's picks sit in lanes lane - r .. lane - r + topk - 1 of this row unless the token
      // straddles two rows: its slot (rank of e among its picks) from the neighbours' registers
      const bool in_row = lane - r >= 0 && lane - r + topk <= 64;
      int slot = 0;
#pragma unroll
      for (int r2 = 0; r2 < kMaxTopk; ++r2) {
        const int v = __shfl(pk[b], min(max(lane - r + r2, 0), 63));
        if (r2 < topk) slot += v < e ? 1 : 0;
      }
      if (hit) {
        const int p = pos + __popcll(mask & ((1ull << lane) - 1ull));
        const int32_t* h = header + (int64_t)t * hw;
        plan.pair_tok()[p] = t;
        plan.pair_expert()[p] = e;
        plan.pair_w()[p] = __builtin_bit_cast(float, wbits[b]);
        if (!in_row) {
          slot = 0;
          for (int r2 = 0; r2 < topk; ++r2) slot += h[1 + r2] < e ? 1 : 0;
        }
        plan.tok_pairs()[(int64_t)t * slots + slot] = p;
      }
      pos += __popcll(mask);
    }
  }
}

// ---------------------------------------------------------------------------
// Gate/up on Q2_K with int8 MFMA + clamped SwiGLU + q8_1 of h.
// Workgroup = (distinct expert u, 64 hidden units): 128 weight rows (the 64
// gate rows, then the 64 up rows), a wave per 32 rows over the whole k, up
// to 16 of the expert's tokens per pass (8 in the kernel of the experts with
// at most 8 pairs). Every operand streams through an LDS ring (3 slots, or 2
// in the small-group kernel), one 256-weight super-block of k per slot,
// filled by buffer-to-LDS dword DMA with the step's offset in a scalar
// register (no VGPRs, no per-step address arithmetic). A slot holds the 128
// rows' super-blocks (84 bytes padded to 96 so that every field is 16-byte
// aligned), the tokens' 256 q8_1 codes (chunk-major, below) and their 8
// block scales as float64 ([block][token]).
// ---------------------------------------------------------------------------
struct GateUpPfArgs {
  XArena ex;
  PlanView plan;
  const int8_t* xq;
  const double* xd64;
  int m;
  int inter;
  float L;
  float* g;
  float* u;
  float* h;
  int8_t* hq;
  uint16_t* hd;
  double* hd64;
  int32_t* hs;
};

constexpr int kGuRows = 128;
constexpr int kGuRowBytes = 96;
constexpr int kGuW = kGuRows * kGuRowBytes;    // 12,288 B: 3072 dwords, 12 per thread
// The codes of a pass's T tokens, chunk-major: 16-byte chunk c (codes
// 16c..16c+15 of the step's super-block) of token i at 16 * (T * c + i), so
// that the lanes reading chunk c of T tokens read consecutive 16-byte pieces
// (no bank conflicts, no padding).
constexpr int kGuA = 16 * 256;                 // 16 tokens: 1024 dwords, 4 per thread
constexpr int kGuD = 8 * kChunk * 8;           // 1,024 B: 256 dwords, 1 per thread
constexpr int kGuSlot = kGuW + kGuA + kGuD;    // 17,408 B
constexpr int kGuSlots = 3;
constexpr int kGuLds = kGuSlots * kGuSlot + 64;   // + the 16-entry code table: 52,288 B, three workgroups per CU
// Experts with at most 8 pairs run in a kernel of their own (one pass of 8
// token rows, no 16-token result registers to carry).
constexpr int kGuASmall = 8 * 256;
constexpr int kGuSlotSmall = kGuW + kGuASmall + kGuD;   // 15,360 B
constexpr int kGuSlotsSmall = 2;
constexpr int kGuLdsSmall = kGuSlotsSmall * kGuSlotSmall + 64;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// One dword per lane from `rsrc` at voff + soff into LDS at `wave_base` + 4 * lane.
__device__ __forceinline__ void dma_dword(__amdgpu_buffer_rsrc_t rsrc, uint8_t* wave_base, uint32_t voff,
                                          uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)wave_base, 4, voff, soff, 0, 0);
}

// The ring: SLOTS slots of one super-block step each (the 128 rows, the
// codes of the pass's tokens in NA dwords per thread, the block scales),
// SLOTS - 1 steps in flight ahead of the one being computed.
template <int NSB, int G, int SLOTS, int NA>
__device__ __forceinline__ void gateup_pf_ring(const GateUpPfArgs& a, uint8_t* lds, const uint32_t* lut,
                                               __amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t ra,
                                               __amdgpu_buffer_rsrc_t rd, const uint32_t (&woff)[12],
                                               const uint32_t (&aoff)[NA], uint32_t doff, double (&y)[4 * G]) {
  constexpr int kA = NA * 1024, kSlot = kGuW + kA + kGuD, kDma = 12 + NA + 1;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hl = lane >> 5;
  auto issue = [&](int s) {
    uint8_t* base = lds + (s % SLOTS) * kSlot + 256 * wave;
#pragma unroll
    for (int k = 0; k < 12; ++k) dma_dword(rw, base + 1024 * k, woff[k], (uint32_t)s * kQ2KBytes);
#pragma unroll
    for (int k = 0; k < NA; ++k) dma_dword(ra, base + kGuW + 1024 * k, aoff[k], (uint32_t)s * 256);
    dma_dword(rd, base + kGuW + kA, doff, (uint32_t)s * 64);
  };
#pragma unroll
  for (int r = 0; r < 4 * G; ++r) y[r] = 0.0;
#pragma unroll
  for (int s = 0; s < SLOTS - 1; ++s)
    if (s < NSB) issue(s);
#pragma unroll 1
  for (int s = 0; s < NSB; ++s) {
    const int after = min(NSB - 1 - s, SLOTS - 2);   // steps issued after s
    static_assert(SLOTS - 2 <= 3 && 3 * kDma < 64, "vmcnt range");
    if (after >= 3) wait_vmcnt<3 * kDma>();
    else if (after == 2) wait_vmcnt<2 * kDma>();
    else if (after == 1) wait_vmcnt<kDma>();
    else wait_vmcnt<0>();
    block_sync_lds();   // every wave's share of step s has landed; every wave is done with step s - 1
    if (s + SLOTS - 1 < NSB) issue(s + SLOTS - 1);   // into the slot step s - 1 used
    const uint8_t* sl = lds + (s % SLOTS) * kSlot;
    const uint8_t* wr = sl + (32 * wave + (lane & 31)) * kGuRowBytes;
    const u32x4a4 scv = *reinterpret_cast<const u32x4a4*>(wr);
    const u32x4a4 qv0 = *reinterpret_cast<const u32x4a4*>(wr + 16 + 16 * hl);
    const u32x4a4 qv1 = *reinterpret_cast<const u32x4a4*>(wr + 48 + 16 * hl);
    const uint32_t ddw = *reinterpret_cast<const uint32_t*>(wr + 80);
    // token rows of the MFMA operand: 8G tokens, repeated (results of the repeats are not used)
    constexpr int T = 4 * NA;   // tokens the slot holds
    const int8_t* ar = reinterpret_cast<const int8_t*>(sl + kGuW) + 16 * (lane & (8 * G - 1)) + 16 * T * hl;
    const double* dr = reinterpret_cast<const double*>(sl + kGuW + kA);
    double accS[4 * G], accM[4 * G];
#pragma unroll
    for (int r = 0; r < 4 * G; ++r) accS[r] = accM[r] = 0.0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int j = t & 3;
      const i32x4 A = *reinterpret_cast<const i32x4*>(ar + 32 * T * t);
      const u32x4a4 qw = t < 4 ? qv0 : qv1;
      const uint32_t sbyte = (scv[t >> 1] >> (8 * (2 * (t & 1) + hl))) & 0xFFu;
      const uint32_t lut_s = lut[sbyte & 15u];
      const uint32_t mrep = __builtin_amdgcn_perm(0u, sbyte >> 4, 0u);   // the min nibble in every byte
      i32x4 Bs;
#pragma unroll
      for (int i = 0; i < 4; ++i) Bs[i] = (int)__builtin_amdgcn_perm(lut_s, lut_s, (qw[i] >> (2 * j)) & 0x03030303u);
      const i32x4 Bm = {(int)mrep, (int)mrep, (int)mrep, (int)mrep};
      const i32x16 S = mfma_i8(A, Bs);
      const i32x16 M = mfma_i8(A, Bm);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const double* dp = dr + t * kChunk + 8 * g + 4 * hl;
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

// SMALL: the experts with at most 8 pairs (one pass, the small ring);
// otherwise the others (passes of 16 pairs, the 4-slot ring).
template <int NSB, bool SMALL>
__device__ __forceinline__ void gateup_pf_body(const GateUpPfArgs& a, uint8_t* lds) {
  constexpr int dim = 256 * NSB, NB = 8 * NSB;
  constexpr int NA = SMALL ? 2 : 4;
  uint32_t* lut = reinterpret_cast<uint32_t*>(lds + (SMALL ? kGuSlotsSmall * kGuSlotSmall : kGuSlots * kGuSlot));
  float (*gu)[kChunk][64] = reinterpret_cast<float (*)[kChunk][64]>(lds);   // after the k loop: [gate|up][tok][unit]
  const int ngr = a.inter / 64;
  const int u = blockIdx.x / ngr, grp = blockIdx.x % ngr;
  if (u >= *a.plan.n_u()) return;
  const int e = a.plan.u_expert()[u], first = a.plan.u_first()[u], np = a.plan.u_npairs()[u];
  if (SMALL ? np > 8 : np <= 8) return;   // the other kernel's expert
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hl = lane >> 5;
  if (tid < 16) lut[tid] = ((uint32_t)tid * 0x030201u) << 8;   // bytes {0, sc, 2sc, 3sc}
  const uint8_t* ebase = a.ex.blocks(e);
  const uint64_t goff = a.ex.goff(e), uoff = a.ex.uoff(e);
  const uint32_t ebytes = (uint32_t)((goff > uoff ? goff : uoff) + (uint64_t)a.inter * NSB * kQ2KBytes);
  const __amdgpu_buffer_rsrc_t rw = buf_rsrc(ebase, ebytes);
  const __amdgpu_buffer_rsrc_t ra = buf_rsrc(a.xq, (uint32_t)((uint64_t)a.m * dim));
  const __amdgpu_buffer_rsrc_t rd = buf_rsrc(a.xd64, (uint32_t)((uint64_t)a.m * NB * 8));
  // the weight dwords this thread moves every step: slot dword i = row * 24 + k (k < 21 real, else padding)
  uint32_t woff[12];
#pragma unroll
  for (int k = 0; k < 12; ++k) {
    const int i = tid + 256 * k, r = i / 24, dw = i % 24;
    const int wr = r >> 5, row = 64 * grp + 32 * (wr & 1) + (r & 31);
    woff[k] = (uint32_t)(((wr >> 1) ? uoff : goff) + (uint64_t)row * (NSB * kQ2KBytes)) +
              4u * (uint32_t)(dw < 21 ? dw : 0);
  }
  for (int c0 = 0; c0 < np; c0 += kChunk) {
    const int nt = min(kChunk, np - c0);
    const int* ptok = a.plan.pair_tok() + first + c0;
    uint32_t aoff[NA];
#pragma unroll
    for (int k = 0; k < NA; ++k) {   // slot dword i: chunk i / (4T), token (i / 4) % T, dword i % 4 (T = 4 NA)
      const int i = tid + 256 * k, c = i / (16 * NA), tk = (i >> 2) % (4 * NA);
      const int tok = ptok[min(tk, nt - 1)];
      aoff[k] = (uint32_t)tok * dim + 16u * c + 4u * (i & 3);
    }
    const int dt = tid >> 5, dtok = (tid & 31) >> 1;   // [block][token] float64, two dwords each
    const uint32_t doff = ((uint32_t)ptok[min(dtok, nt - 1)] * NB + dt) * 8u + 4u * (tid & 1);
    __syncthreads();   // the previous pass is done with the LDS (its SwiGLU phase reads gu)
    double y[4 * kGroups];
    if (!SMALL && nt > 8) {
      gateup_pf_ring<NSB, 2, kGuSlots, NA>(a, lds, lut, rw, ra, rd, woff, aoff, doff, y);
    } else {
      double y1[4];
      if (SMALL) gateup_pf_ring<NSB, 1, kGuSlotsSmall, NA>(a, lds, lut, rw, ra, rd, woff, aoff, doff, y1);
      else gateup_pf_ring<NSB, 1, kGuSlots, NA>(a, lds, lut, rw, ra, rd, woff, aoff, doff, y1);
#pragma unroll
      for (int r = 0; r < 4; ++r) y[r] = y1[r];
#pragma unroll
      for (int r = 4; r < 4 * kGroups; ++r) y[r] = 0.0;
    }
    __syncthreads();   // every wave is done reading the ring
    {
      const int mat = wave >> 1, unit = 32 * (wave & 1) + (lane & 31);
#pragma unroll
      for (int r = 0; r < 4 * kGroups; ++r) gu[mat][tile_tok(r, lane)][unit] = (float)y[r];
    }
    __syncthreads();
    // SwiGLU + q8_1 of h: a half-wave per (token, 32 units = one q8_1 block), a lane per unit
#pragma unroll 1
    for (int job = 2 * wave + hl; job < 2 * (SMALL ? 8 : kChunk); job += 8) {
      const int tt = job >> 1, hb = job & 1, unit = 32 * hb + (lane & 31);
      const bool live = tt < nt;
      const float gv = gu[0][tt][unit], uv = gu[1][tt][unit];
      const float hv = live ? swiglu(gv, uv, a.L) : 0.0f;
      const float am = max32(fabsf(hv));
      const float d = (float)((double)am / 127.0);
      const int q = am == 0.0f ? 0 : q8_code(hv, d);
      const int sum = sum16(q);
      if (live) {
        const int64_t pair = first + c0 + tt;
        const int64_t o = pair * a.inter + 64 * grp + unit;
        const int blk = 2 * grp + hb;
        a.g[o] = gv;
        a.u[o] = uv;
        a.h[o] = hv;
        a.hq[o] = (int8_t)q;
        if ((lane & 31) == 0) {
          const uint16_t d16 = f32_to_fp16_bits(d);
          a.hd[pair * (a.inter / 32) + blk] = d16;
          a.hd64[pair * (a.inter / 32) + blk] = fp16_f64(d16);
        }
        if ((lane & 15) == 0) a.hs[pair * (a.inter / 16) + 2 * blk + ((lane & 31) >> 4)] = sum;
      }
    }
  }
}

template <int NSB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_gateup_pf(GateUpPfArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  gateup_pf_body<NSB, false>(a, lds);
}

template <int NSB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_gateup_pf_small(GateUpPfArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  gateup_pf_body<NSB, true>(a, lds);
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
  XArena ex;
  PlanView plan;
  const int8_t* hq;
  const uint16_t* hd;
  const double* hd64;
  int n_pairs_max;
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
__global__ __launch_bounds__(256) void k_down_pf_direct(DownPfArgs a) {
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
  const uint8_t* wrow = a.ex.down(e) + (uint64_t)row * (NSB * kQ3KBytes);
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

// The same down GEMM through a 3-slot LDS ring (inter >= 512): a slot holds,
// for one super-block of k, the 128 rows' 110-byte blocks in 112-byte rows
// (the DMA window starts on the dword at or before the block, so a block of
// odd index sits 2 bytes into its row), the 16 pairs' h codes (rows 272
// bytes apart) and their 8 block scales as float64 ([block][pair]).
constexpr int kDnRows = 128;
constexpr int kDnRowBytes = 112;
constexpr int kDnW = kDnRows * kDnRowBytes;    // 14,336 B: 3584 dwords, 14 per thread
// Both down rings keep one step in flight ahead: the 16-pair kernel (at most
// 168 VGPRs) then runs three workgroups per CU, the 8-pair one four.
constexpr int kDnSlots = 2;        // experts with more than 8 pairs
constexpr int kDnSlotsSmall = 2;   // the others
// The pairs' h codes are chunk-major as in the gate/up ring (T = 16 pairs: 4
// dwords per thread; T = 8 in the kernel of the experts with at most 8
// pairs: 2 dwords per thread).
template <int NA>
constexpr int dn_slot() { return kDnW + NA * 1024 + kGuD; }
template <int NA>
constexpr int dn_lds() { return (NA == 2 ? kDnSlotsSmall : kDnSlots) * dn_slot<NA>() + 512; }   // + the scale table

template <int NSB, int G, int NA, int SLOTS = (NA == 2 ? kDnSlotsSmall : kDnSlots)>
__device__ __forceinline__ void down_pf_ring(uint8_t* lds, const uint32_t (*lut)[2], __amdgpu_buffer_rsrc_t rw,
                                             __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rd,
                                             const uint32_t (&woff)[14], const uint32_t (&aoff)[NA], uint32_t doff,
                                             double (&y)[4 * G]) {
  constexpr int kA = NA * 1024, kSlot = dn_slot<NA>(), kDnDma = 14 + NA + 1, T = 4 * NA;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hl = lane >> 5;
  auto issue = [&](int s) {
    uint8_t* base = lds + (s % SLOTS) * kSlot + 256 * wave;
    const uint32_t wsoff = (uint32_t)(s * kQ3KBytes - 2 * (s & 1));   // dword-aligned window start
#pragma unroll
    for (int k = 0; k < 14; ++k) dma_dword(rw, base + 1024 * k, woff[k], wsoff);
#pragma unroll
    for (int k = 0; k < NA; ++k) dma_dword(ra, base + kDnW + 1024 * k, aoff[k], (uint32_t)s * 256);
    dma_dword(rd, base + kDnW + kA, doff, (uint32_t)s * 64);
  };
#pragma unroll
  for (int r = 0; r < 4 * G; ++r) y[r] = 0.0;
#pragma unroll
  for (int s = 0; s < SLOTS - 1; ++s)
    if (s < NSB) issue(s);
#pragma unroll 1
  for (int s = 0; s < NSB; ++s) {
    const int after = min(NSB - 1 - s, SLOTS - 2);   // steps issued after s
    static_assert(SLOTS - 2 <= 1, "wait cases");
    if (after >= 1) wait_vmcnt<kDnDma>();
    else wait_vmcnt<0>();
    block_sync_lds();   // step s landed everywhere; step s - 1 is done everywhere
    if (s + SLOTS - 1 < NSB) issue(s + SLOTS - 1);   // into the slot step s - 1 used
    const uint8_t* sl = lds + (s % SLOTS) * kSlot;
    const uint8_t* blk = sl + (32 * wave + (lane & 31)) * kDnRowBytes + 2 * (s & 1);
    const u32x4a2 hmv = *reinterpret_cast<const u32x4a2*>(blk + 16 * hl);
    const u32x4a2 qv0 = *reinterpret_cast<const u32x4a2*>(blk + 32 + 16 * hl);
    const u32x4a2 qv1 = *reinterpret_cast<const u32x4a2*>(blk + 64 + 16 * hl);
    const u32x2a2 sc01 = *reinterpret_cast<const u32x2a2*>(blk + 96);
    const uint32_t sc2 = *reinterpret_cast<const uint32_t __attribute__((aligned(2)))*>(blk + 104);
    const uint32_t dbits = *reinterpret_cast<const uint16_t*>(blk + 108);
    const int8_t* ar = reinterpret_cast<const int8_t*>(sl + kDnW) + 16 * (lane & (8 * G - 1)) + 16 * T * hl;
    const double* dr = reinterpret_cast<const double*>(sl + kDnW + kA);
    double acc[4 * G];
#pragma unroll
    for (int r = 0; r < 4 * G; ++r) acc[r] = 0.0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int h = t >> 2, j = t & 3;
      const int sl8 = 2 * (t & 3) + hl;
      const uint32_t lob = ((sl8 < 4 ? sc01[0] : sc01[1]) >> (8 * (sl8 & 3))) & 0xFFu;
      const uint32_t lo = t < 4 ? (lob & 15u) : (lob >> 4);
      const uint32_t hib = (sc2 >> (8 * (2 * (t & 1) + hl))) & 0xFFu;
      const uint32_t hi = (hib >> (2 * (t >> 1))) & 3u;
      const uint32_t u6 = lo | (hi << 4);
      const uint32_t lut_lo = lut[u6][0], lut_hi = lut[u6][1];
      const u32x4a2 qw = t < 4 ? qv0 : qv1;
      const int hbit = 4 * h + j;
      i32x4 B;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t q2 = (qw[i] >> (2 * j)) & 0x03030303u;
        const uint32_t hb = hbit >= 2 ? (hmv[i] >> (hbit - 2)) : (hmv[i] << (2 - hbit));
        B[i] = (int)__builtin_amdgcn_perm(lut_hi, lut_lo, (hb & 0x04040404u) | q2);
      }
      const i32x4 A = *reinterpret_cast<const i32x4*>(ar + 32 * T * t);
      const i32x16 S = mfma_i8(A, B);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const double* dp = dr + t * kChunk + 8 * g + 4 * hl;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[4 * g + i] = __builtin_fma(dp[i], (double)S[4 * g + i], acc[4 * g + i]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    const double nd = -fp16_f64(dbits);   // the MFMA sums are -S_b
#pragma unroll
    for (int r = 0; r < 4 * G; ++r) y[r] = __builtin_fma(nd, acc[r], y[r]);
  }
}

// SMALL: the experts with at most 8 pairs; otherwise the others.
template <int NSB, bool SMALL>
__device__ __forceinline__ void down_pf_body(const DownPfArgs& a, uint8_t* lds) {
  constexpr int inter = 256 * NSB, NB = 8 * NSB;
  constexpr int NA = SMALL ? 2 : 4;
  uint32_t (*lut)[2] = reinterpret_cast<uint32_t (*)[2]>(lds + dn_lds<NA>() - 512);
  const int nrt = a.dim / kDnRows;
  const int u = blockIdx.x / nrt, rt = blockIdx.x % nrt;
  if (u >= *a.plan.n_u()) return;
  const int e = a.plan.u_expert()[u], first = a.plan.u_first()[u], np = a.plan.u_npairs()[u];
  if (SMALL ? np > 8 : np <= 8) return;   // the other kernel's expert
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  q3k_lut_fill(lut);
  const uint8_t* wbase = a.ex.down(e);
  const __amdgpu_buffer_rsrc_t rw = buf_rsrc(wbase, (uint32_t)((uint64_t)a.dim * NSB * kQ3KBytes));
  const __amdgpu_buffer_rsrc_t ra = buf_rsrc(a.hq, (uint32_t)((uint64_t)a.n_pairs_max * inter));
  const __amdgpu_buffer_rsrc_t rd = buf_rsrc(a.hd64, (uint32_t)((uint64_t)a.n_pairs_max * NB * 8));
  uint32_t woff[14];   // slot dword i = row * 28 + k
#pragma unroll
  for (int k = 0; k < 14; ++k) {
    const int i = tid + 256 * k, r = i / 28, dw = i % 28;
    woff[k] = (uint32_t)(kDnRows * rt + r) * (NSB * kQ3KBytes) + 4u * dw;
  }
  const int row = kDnRows * rt + 32 * wave + (lane & 31);
  for (int c0 = 0; c0 < np; c0 += kChunk) {
    const int nt = min(kChunk, np - c0);
    const int p0 = first + c0;
    uint32_t aoff[NA];
#pragma unroll
    for (int k = 0; k < NA; ++k) {   // slot dword i: chunk i / (4T), pair (i / 4) % T, dword i % 4 (T = 4 NA)
      const int i = tid + 256 * k, c = i / (16 * NA), tk = (i >> 2) % (4 * NA);
      aoff[k] = (uint32_t)(p0 + min(tk, nt - 1)) * inter + 16u * c + 4u * (i & 3);
    }
    const int dt = tid >> 5, dtok = (tid & 31) >> 1;
    const uint32_t doff = ((uint32_t)(p0 + min(dtok, nt - 1)) * NB + dt) * 8u + 4u * (tid & 1);
    __syncthreads();
    if (!SMALL && nt > 8) {
      double y[8];
      down_pf_ring<NSB, 2, NA>(lds, lut, rw, ra, rd, woff, aoff, doff, y);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int tt = tile_tok(r, lane);
        if (tt < nt) a.y[(int64_t)(p0 + tt) * a.dim + row] = (float)y[r];
      }
    } else {
      double y[4];
      down_pf_ring<NSB, 1, NA>(lds, lut, rw, ra, rd, woff, aoff, doff, y);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tt = tile_tok(r, lane);
        if (tt < nt) a.y[(int64_t)(p0 + tt) * a.dim + row] = (float)y[r];
      }
    }
  }
}

template <int NSB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_down_pf(DownPfArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  down_pf_body<NSB, false>(a, lds);
}

template <int NSB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_down_pf_small(DownPfArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  down_pf_body<NSB, true>(a, lds);
}

template <int NSB>
hipError_t launch_gateup_pf_t(const GateUpPfArgs& a, int max_u, int part, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)k_gateup_pf<NSB>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       kGuLds);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)k_gateup_pf_small<NSB>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            kGuLdsSmall);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  if (part == 0)
    MOE_LAUNCH(MOE_K_GATEUP, k_gateup_pf_small<NSB>, dim3(max_u * (a.inter / 64)), dim3(256), kGuLdsSmall, s, a);
  else
    MOE_LAUNCH(MOE_K_GATEUP2, k_gateup_pf<NSB>, dim3(max_u * (a.inter / 64)), dim3(256), kGuLds, s, a);
  return hipGetLastError();
}

template <int NSB>
hipError_t launch_down_pf_t(const DownPfArgs& a, int max_u, int part, hipStream_t s) {
  if constexpr (NSB == 1) {   // one super-block of k: one kernel without the ring for every expert
    if (part == 0) MOE_LAUNCH(MOE_K_DOWN, k_down_pf_direct<NSB>, dim3(max_u * (a.dim / 128)), dim3(256), 0, s, a);
    return hipGetLastError();
  } else {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)k_down_pf<NSB>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       dn_lds<4>());
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)k_down_pf_small<NSB>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            dn_lds<2>());
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  if (part == 0)
    MOE_LAUNCH(MOE_K_DOWN, k_down_pf_small<NSB>, dim3(max_u * (a.dim / kDnRows)), dim3(256), dn_lds<2>(), s, a);
  else
    MOE_LAUNCH(MOE_K_DOWN2, k_down_pf<NSB>, dim3(max_u * (a.dim / kDnRows)), dim3(256), dn_lds<4>(), s, a);
  return hipGetLastError();
  }
}

}  // namespace

hipError_t launch_router_pf(const uint16_t* x, int m, const uint16_t* gate_w, const moe_cfg& c, const Ws& w,
                            float* logits_out, hipStream_t s) {
  const int router_blocks = gate_w ? (c.n_routed + 4 * kRpRows - 1) / (4 * kRpRows) : 0;
  const int tgroups = (m + 7) / 8;
  const int64_t quant = (int64_t)m * c.dim / 256;
  const int quant_cols = (int)((quant + tgroups - 1) / tgroups);
  MOE_LAUNCH(MOE_K_ROUTER, k_router_pf, dim3(router_blocks + quant_cols, tgroups), dim3(256), 0, s, x, m, c.dim,
             gate_w, c.n_routed, c.gate_temp, router_blocks, w, logits_out, score_table_for(c));
  return hipGetLastError();
}

hipError_t launch_group(const int32_t* header, int m, const moe_cfg& c, const Ws& w, int32_t* grp, int shq,
                        hipStream_t s) {
  hipLaunchKernelGGL(k_group_count, dim3(1), dim3(1024), 0, s, header, m, c.topk, c.n_routed, w.plan, grp, w.status,
                     shq);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_group_fill, dim3(c.n_routed + shq), dim3(64), 0, s, header, m, c.topk, c.n_routed, w.plan, grp);
  return hipGetLastError();
}

// Plan entries of a prefill plan: the distinct routed experts, then the
// shared group's entries of kChunk tokens.
int max_entries(const XArena& ex, int m, const moe_cfg& c) {
  return min(c.n_routed, m * c.topk) + (ex.has_shared() ? (m + kChunk - 1) / kChunk : 0);
}

hipError_t launch_gateup_pf(const XArena& ex, int m, const moe_cfg& c, const Ws& w, int part, hipStream_t s) {
  const int max_u = max_entries(ex, m, c);
  GateUpPfArgs a{ex, w.plan, w.xq, w.xd64, m, c.inter, c.swiglu_limit, w.g, w.u, w.h, w.hq, w.hd, w.hd64, w.hs};
  switch (c.dim / 256) {
    case 1: return launch_gateup_pf_t<1>(a, max_u, part, s);
    case 2: return launch_gateup_pf_t<2>(a, max_u, part, s);
    case 4: return launch_gateup_pf_t<4>(a, max_u, part, s);
    case 8: return launch_gateup_pf_t<8>(a, max_u, part, s);
    case 16: return launch_gateup_pf_t<16>(a, max_u, part, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_down_pf(const XArena& ex, int m, const moe_cfg& c, const Ws& w, int part, hipStream_t s) {
  const int max_u = max_entries(ex, m, c);
  DownPfArgs a{ex, w.plan, w.hq, w.hd, w.hd64, m * (c.topk + 1), c.dim, w.y};
  switch (c.inter / 256) {
    case 1: return launch_down_pf_t<1>(a, max_u, part, s);
    case 2: return launch_down_pf_t<2>(a, max_u, part, s);
    case 4: return launch_down_pf_t<4>(a, max_u, part, s);
    case 8: return launch_down_pf_t<8>(a, max_u, part, s);
    case 16: return launch_down_pf_t<16>(a, max_u, part, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
