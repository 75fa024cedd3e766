// Routing kernels (A1-A3) and the front of the layer:
//  * k_front: q8_1 of the input, the router GEMV with the scores, and (for
//    the whole layer) the shared expert's gate/up GEMVs with its SwiGLU, in
//    one launch (the workgroup index picks the part). For the layer, the last
//    router workgroup to finish also runs every token's top-k selection,
//    writes the headers and builds the plan, while the shared rows stream;
//  * k_select: the top-k selection and its header alone (routing only);
//  * k_plan_small: the plan tables from caller-given headers.
#include <hip/hip_runtime.h>

#include "moe_internal.h"
#include "moe_math.h"
#include "moe_front.h"
#include "moe_kquant.h"
#include "moe_select.h"

namespace moe {
namespace {

using front::quant_x_block;
using front::router_rows;
using front::shared_gu_rows;

// ---------------------------------------------------------------------------
// Selection, one wave per token (moe_select.h): writes the header
// [device_route.rs, fn parse_header] and, for the plan, the picks/weights.
// ---------------------------------------------------------------------------
// slot_of (optional, an expert cache's slot-table row): the plan words hold
// the picks' slots instead of their ids, -1 for an absent expert, and an
// absent pick sets MOE_STATUS_MISS [device_route.rs, module doc: the header's
// miss flag and plan slots].
template <int KPER>
__device__ void select_token(const float (&sc)[KPER], const float (&bs)[KPER], int n_routed, int topk, int norm,
                             float route_scale, int32_t* __restrict__ hd, int* picks_out, float* w_out,
                             int32_t* __restrict__ status, const int32_t* __restrict__ slot_of = nullptr) {
  const int lane = threadIdx.x & 63;
  int picks[kMaxTopk];
  float wv = 0.0f;
  bool nan_any = false;
  select_topk_from<KPER>(sc, bs, n_routed, topk, norm, route_scale, picks, wv, nan_any);
  int mypick = 0;
#pragma unroll
  for (int r = 0; r < kMaxTopk; ++r)
    if (r == lane) mypick = picks[r];
  int rank = 0;
#pragma unroll
  for (int r = 0; r < kMaxTopk; ++r)
    if (r < topk) rank += picks[r] < mypick ? 1 : 0;
  const int slot = (slot_of && lane < topk) ? slot_of[mypick] : mypick;
  const bool miss = __any(lane < topk && slot < 0);
  if (lane < topk) {
    hd[1 + lane] = mypick;
    hd[1 + topk + lane] = (int32_t)__builtin_bit_cast(uint32_t, wv);
    hd[1 + 2 * topk + rank] = slot;
    if (picks_out) {
      picks_out[lane] = mypick;
      w_out[lane] = wv;
    }
  }
  if (lane == 0) {
    const int st = (nan_any ? MOE_STATUS_NAN_KEY : 0) | (miss ? MOE_STATUS_MISS : 0);
    hd[0] = st;
    if (st) atomicOr(status, st);
  }
}

// Inclusive prefix sum of v over the 64 lanes by DPP: row_shr 1, 2, 4, 8
// within each row of 16 lanes, then row_bcast:15 and row_bcast:31 across rows
// (out-of-row sources and disabled rows add 0).
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);
  return v;
}

// ---------------------------------------------------------------------------
// Plan tables for m <= 8 tokens, one wave, one lane per pick q = t*topk + r
// (q < 64): the valid (expert, token) pairs sorted by expert id then token,
// the distinct experts, and per token its pairs in plan order (ascending id)
// [device_route.rs, fn device_route_check: weights and pointers in plan order].
// An expert map in LDS (one word per expert id, emap >= 64*KPER words) first
// collects each expert's token mask; a wave scan over the ids (lane l owns ids
// KPER*l .. KPER*l + KPER-1) turns it into, per id, the number of pairs and of
// distinct experts with a smaller id. A pair's position is then its expert's
// pair count plus the tokens below it in the mask.
// ---------------------------------------------------------------------------
// With shq = 1 every token that keeps its picks also gets the layer's
// quantised shared expert (id n_routed, weight 1) as its last plan entry: one
// more distinct expert whose pairs follow all routed pairs, tokens ascending.
template <int KPER>
__device__ void build_plan(const int* picks, const float* wts, const int* tok_ok, int m, int topk, PlanView plan,
                           uint32_t* emap, int shq, int n_routed) {
  static_assert(kMaxDecodeTokens <= 8, "token masks are 8 bits");
  const int lane = threadIdx.x & 63;
  const int P = m * topk;
  const bool mine = lane < P;
  const int t = mine ? lane / topk : 0;
  const bool valid = mine && tok_ok[t];
  const int e = valid ? picks[lane] : 0;   // a disabled token's picks may be out of range
#pragma unroll
  for (int c = 0; c < KPER; ++c) emap[KPER * lane + c] = 0u;
  __builtin_amdgcn_wave_barrier();
  if (valid) atomicOr(&emap[e], 1u << t);
  __builtin_amdgcn_wave_barrier();
  // per id: token mask (bits 0-7), pairs below (bits 8-15), distinct experts below (bits 16-23)
  uint32_t mk[KPER];
  uint32_t own = 0;   // this lane's ids: pairs (low half) and distinct experts (high half)
#pragma unroll
  for (int c = 0; c < KPER; ++c) {
    mk[c] = emap[KPER * lane + c];
    own += (uint32_t)__popc(mk[c]) | (mk[c] ? 0x10000u : 0u);
  }
  const uint32_t incl = wave_incl_sum(own);
  uint32_t run = incl - own;
#pragma unroll
  for (int c = 0; c < KPER; ++c) {
    emap[KPER * lane + c] = mk[c] | (run & 0xffu) << 8 | ((run >> 16) & 0xffu) << 16;
    run += (uint32_t)__popc(mk[c]) | (mk[c] ? 0x10000u : 0u);
  }
  __builtin_amdgcn_wave_barrier();
  const uint32_t v = emap[e];
  const uint32_t below = v & ((1u << t) - 1u);   // tokens below t that picked e
  const int pos = (int)((v >> 8) & 0xffu) + __popc(below);
  int rk = 0;   // rank of e among its token's picks
  for (int r2 = 0; r2 < topk; ++r2) rk += __shfl(e, t * topk + r2) < e ? 1 : 0;
  if (valid) {
    plan.pair_tok()[pos] = t;
    plan.pair_expert()[pos] = e;
    plan.pair_w()[pos] = wts[lane];
    if (below == 0) {
      const int uid = (int)((v >> 16) & 0xffu);
      plan.u_expert()[uid] = e;
      plan.u_first()[uid] = pos;
      plan.u_npairs()[uid] = __popc(v & 0xffu);
    }
    plan.tok_pairs()[t * plan.slots() + rk] = pos;
  } else if (mine) {
    plan.tok_pairs()[t * plan.slots() + (lane - t * topk)] = -1;
  }
  const unsigned long long vb = __ballot(valid);
  const int n_pairs = __popcll(vb);
  const int n_u = (int)(__builtin_amdgcn_readlane((int)incl, 63) >> 16);
  const unsigned long long okm = __ballot(lane < m && tok_ok[lane]) & (shq ? ~0ull : 0ull);
  const int n_ok = __popcll(okm);
  if (lane < m) {   // the token's last plan entry: the quantised shared expert, or none
    int q = -1;
    if ((okm >> lane) & 1ull) {
      q = n_pairs + __popcll(okm & ((1ull << lane) - 1ull));
      plan.pair_tok()[q] = lane;
      plan.pair_expert()[q] = n_routed;
      plan.pair_w()[q] = 1.0f;
    }
    plan.tok_pairs()[lane * plan.slots() + topk] = q;
  }
  if (lane == 0) {
    *plan.n_pairs() = n_pairs + n_ok;
    *plan.n_u() = n_u + (n_ok > 0 ? 1 : 0);
    if (n_ok > 0) {
      plan.u_expert()[n_u] = n_routed;
      plan.u_first()[n_u] = n_pairs;
      plan.u_npairs()[n_u] = n_ok;
    }
  }
}

struct FrontArgs {
  const uint16_t* x;
  int m, dim, inter, n_routed, topk, norm;
  float temp, L, route_scale;
  const uint16_t* gate_w;
  const float* bias;   // non-null: select, write the headers and the plan
  int32_t* header;
  const uint16_t* w1;
  const uint16_t* w3;
  float* logits_out;
  int router_blocks, shared_blocks;
  int shq;   // the plan gets the layer's quantised shared expert (id n_routed) for every token
  ScoreTable st;   // the glibc score mode's table (keys nullptr: correctly rounded scores)
};

// Every token's selection and the plan [moe_v41.rs, fn route_from_logits;
// device_route.rs, fn device_route_check]: wave w of the four selects tokens
// w and w + 4, with both rows' loads issued before either selection.
template <int KPER>
__device__ void select_all(const FrontArgs& a, const Ws& w) {
  static_assert(kMaxDecodeTokens <= 8, "two tokens per wave");
  __shared__ int picks[64];
  __shared__ float wts[64];
  __shared__ int tok_ok[kMaxDecodeTokens];
  __shared__ uint32_t emap[64 * KPER];
  const int wave = threadIdx.x >> 6;
  const int hw = 1 + 3 * a.topk;
  const int t0 = wave, t1 = wave + 4;
  float sc0[KPER], bs0[KPER], sc1[KPER], bs1[KPER];
  select_load<KPER>(w.scores + (int64_t)min(t0, a.m - 1) * a.n_routed, a.bias, a.n_routed, sc0, bs0);
  select_load<KPER>(w.scores + (int64_t)min(t1, a.m - 1) * a.n_routed, a.bias, a.n_routed, sc1, bs1);
  if (t0 < a.m)
    select_token<KPER>(sc0, bs0, a.n_routed, a.topk, a.norm, a.route_scale, a.header + (int64_t)t0 * hw,
                       picks + t0 * a.topk, wts + t0 * a.topk, w.status);
  if (t1 < a.m)
    select_token<KPER>(sc1, bs1, a.n_routed, a.topk, a.norm, a.route_scale, a.header + (int64_t)t1 * hw,
                       picks + t1 * a.topk, wts + t1 * a.topk, w.status);
  if (threadIdx.x < a.m) tok_ok[threadIdx.x] = 1;
  __syncthreads();
  if (wave == 0) build_plan<KPER>(picks, wts, tok_ok, a.m, a.topk, w.plan, emap, a.shq, a.n_routed);
}

__global__ __launch_bounds__(256) void k_front(FrontArgs a, Ws w) {
  __shared__ int s_last;
  int blk = blockIdx.x;
  if (blk == 0 && threadIdx.x < 4) w.status[threadIdx.x] = 0;   // every entry point starts here
  if (blk < a.router_blocks) {
    router_rows(blk, a.x, a.m, a.dim, a.gate_w, a.n_routed, a.temp, w.logits, w.scores, a.logits_out, a.st);
    if (!a.bias) return;
    // Count this workgroup's rows as done; the last of the router workgroups
    // selects. Each wave completes its stores, then one release (one L2
    // write-back) covers the workgroup; the selecting workgroup acquires.
    wait_vmcnt<0>();
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t old = __hip_atomic_fetch_add(&w.ctl->router_done, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      s_last = old + 1 == (uint32_t)a.router_blocks;
    }
    __syncthreads();
    if (!s_last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (a.n_routed <= 384) select_all<6>(a, w);
    else select_all<16>(a, w);
    // the counter is back to zero for the next launch (no other workgroup touches it now)
    if (threadIdx.x == 0) __hip_atomic_store(&w.ctl->router_done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  blk -= a.router_blocks;
  if (blk < a.shared_blocks) {
    shared_gu_rows(blk, a.x, a.m, a.dim, a.inter, a.w1, a.w3, w.sg, w.su, w.sh, a.L);
    return;
  }
  blk -= a.shared_blocks;
  quant_x_block(blk, a.x, w.xq, w.xd, w.xs);
}

template <int KPER>
__global__ __launch_bounds__(64) void k_select(const float* __restrict__ scores, const float* __restrict__ bias,
                                               int n_routed, int topk, int norm, float route_scale,
                                               int32_t* __restrict__ header, int32_t* __restrict__ status,
                                               const int32_t* __restrict__ slot_of) {
  const int t = blockIdx.x;
  float sc[KPER], bs[KPER];
  select_load<KPER>(scores + (int64_t)t * n_routed, bias, n_routed, sc, bs);
  select_token<KPER>(sc, bs, n_routed, topk, norm, route_scale, header + (int64_t)t * (1 + 3 * topk), nullptr,
                     nullptr, status, slot_of);
}

// Plan tables from headers given by the caller (m <= 8): picks outside
// [0, n_routed) or repeated within a token disable that token.
template <int KPER>
__global__ __launch_bounds__(64) void k_plan_small(const int32_t* __restrict__ header, int m, int topk, int n_routed,
                                                   PlanView plan, int32_t* __restrict__ status, int shq) {
  __shared__ int picks[64];
  __shared__ float wts[64];
  __shared__ int tok_ok[kMaxDecodeTokens];
  __shared__ uint32_t emap[64 * KPER];
  const int lane = threadIdx.x;
  const int hw = 1 + 3 * topk;
  if (lane < m * topk) {
    const int t = lane / topk, r = lane % topk;
    picks[lane] = header[t * hw + 1 + r];
    wts[lane] = __builtin_bit_cast(float, header[t * hw + 1 + topk + r]);
  }
  __builtin_amdgcn_wave_barrier();
  if (lane < m) {
    bool ok = true;
    for (int r = 0; r < topk; ++r) {
      const int e = picks[lane * topk + r];
      if (e < 0 || e >= n_routed) ok = false;
      for (int r2 = 0; r2 < r; ++r2)
        if (picks[lane * topk + r2] == e) ok = false;
    }
    tok_ok[lane] = ok ? 1 : 0;
    if (!ok) atomicOr(status, MOE_STATUS_BAD_PICK);
  }
  __builtin_amdgcn_wave_barrier();
  build_plan<KPER>(picks, wts, tok_ok, m, topk, plan, emap, shq, n_routed);
}

// flags as moe_scores: bit 0 the extended path, bit 2 the exp step alone
// (st: the glibc table, with bit 1).
__global__ __launch_bounds__(256) void k_scores(const float* __restrict__ lg, int64_t n, float temp,
                                                float* __restrict__ out, int flags, ScoreTable st) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const bool slow = (flags & 1) != 0;
  if (flags & 4) out[i] = exp_cr(temp == 1.0f ? lg[i] : (float)((double)lg[i] / (double)temp), slow);
  else out[i] = st.keys ? score_mode_of(lg[i], temp, st) : score_of(lg[i], temp, slow);
}

}  // namespace

hipError_t launch_front(const uint16_t* x, int m, const uint16_t* gate_w, const FrontSelect* sel, const uint16_t* w1,
                        const uint16_t* w3, const moe_cfg& c, const Ws& w, float* logits_out, hipStream_t s) {
  FrontArgs a;
  a.x = x;
  a.m = m;
  a.dim = c.dim;
  a.inter = c.inter;
  a.n_routed = c.n_routed;
  a.topk = c.topk;
  a.norm = c.norm_topk_prob;
  a.temp = c.gate_temp;
  a.L = c.swiglu_limit;
  a.route_scale = c.route_scale;
  a.gate_w = gate_w;
  a.bias = (gate_w && sel) ? sel->bias : nullptr;
  a.header = sel ? sel->header : nullptr;
  a.w1 = w1;
  a.w3 = w3;
  a.logits_out = logits_out;
  a.router_blocks = gate_w ? (c.n_routed + 2) / 3 : 0;
  a.shared_blocks = w1 ? (c.inter + 3) / 4 : 0;
  a.shq = sel ? sel->shq : 0;
  a.st = score_table_for(c);
  const int quant_blocks = (int)((int64_t)m * c.dim / 256);
  MOE_LAUNCH(MOE_K_ROUTER, k_front, dim3(a.router_blocks + a.shared_blocks + quant_blocks), dim3(256), 0, s, a, w);
  return hipGetLastError();
}

hipError_t launch_select(const float* bias, int m, const moe_cfg& c, const Ws& w, int32_t* header, hipStream_t s,
                         const int32_t* slot_of) {
  const int kper = (c.n_routed + 63) / 64;
  if (kper == 6)
    hipLaunchKernelGGL(k_select<6>, dim3(m), dim3(64), 0, s, w.scores, bias, c.n_routed, c.topk, c.norm_topk_prob,
                       c.route_scale, header, w.status, slot_of);
  else
    hipLaunchKernelGGL(k_select<16>, dim3(m), dim3(64), 0, s, w.scores, bias, c.n_routed, c.topk, c.norm_topk_prob,
                       c.route_scale, header, w.status, slot_of);
  return hipGetLastError();
}

hipError_t launch_plan(const int32_t* header, int m, const moe_cfg& c, const Ws& w, hipStream_t s, int shq) {
  if (c.n_routed <= 384)
    hipLaunchKernelGGL(k_plan_small<6>, dim3(1), dim3(64), 0, s, header, m, c.topk, c.n_routed, w.plan, w.status, shq);
  else
    hipLaunchKernelGGL(k_plan_small<16>, dim3(1), dim3(64), 0, s, header, m, c.topk, c.n_routed, w.plan, w.status,
                       shq);
  return hipGetLastError();
}

hipError_t launch_quant_x(const uint16_t* x, int m, const moe_cfg& c, const Ws& w, hipStream_t s) {
  return launch_front(x, m, nullptr, nullptr, nullptr, nullptr, c, w, nullptr, s);
}

hipError_t launch_scores(const float* logits, int64_t n, float temp, float* out, int flags, hipStream_t s) {
  if (n == 0) return hipSuccess;
  moe_cfg glibc{};
  glibc.score_mode = MOE_SCORE_GLIBC;
  const ScoreTable st = (flags & 2) ? score_table_for(glibc) : ScoreTable{nullptr, nullptr, nullptr};
  hipLaunchKernelGGL(k_scores, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, logits, n, temp, out, flags, st);
  return hipGetLastError();
}

}  // namespace moe
