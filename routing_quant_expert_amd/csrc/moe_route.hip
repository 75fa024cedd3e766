// Routing kernels: q8_1 of the input, the router GEMV with the scores, the
// top-k selection with its header, and the plan tables (A1-A3).
#include <hip/hip_runtime.h>

#include "moe_internal.h"
#include "moe_math.h"

namespace moe {
namespace {

__device__ inline float fp16_bits_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
__device__ inline uint16_t f32_to_fp16_bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// ---------------------------------------------------------------------------
// q8_1 of bf16 rows: one thread per value, a q8_1 block = 32 consecutive
// lanes. d = amax/127, code = roundf(x/d) (half away from zero), stored scale
// fp16(d), plus the sums of 16 consecutive codes (the q8_1 sum field is not
// used; the GEMV epilogues need per-16 sums of the codes).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_quant_x(const uint16_t* __restrict__ x, int64_t n, int8_t* __restrict__ xq,
                                                 uint16_t* __restrict__ xd, int32_t* __restrict__ xs,
                                                 int32_t* __restrict__ status) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // n is a multiple of 256
  if (blockIdx.x == 0 && threadIdx.x < 4) status[threadIdx.x] = 0;   // first kernel of every entry point
  float v = bf16_f32(x[i]);
  float a = fabsf(v);
  for (int s = 16; s >= 1; s >>= 1) a = fmaxf(a, __shfl_xor(a, s));
  float d = (float)((double)a / 127.0);
  int q = a == 0.0f ? 0 : q8_code(v, d);
  xq[i] = (int8_t)q;
  int sum = q;
  for (int s = 8; s >= 1; s >>= 1) sum += __shfl_xor(sum, s);
  int lane32 = threadIdx.x & 31;
  if (lane32 == 0) xd[i >> 5] = f32_to_fp16_bits(d);
  if ((lane32 & 15) == 0) xs[i >> 4] = sum;
}

// ---------------------------------------------------------------------------
// Router GEMV + scores. One wave64 per expert row, all tokens of the call.
// Lane l accumulates positions 512*i + 8*l + j (i ascending, j = 0..7) in
// f32 (product, then add: every bf16 x bf16 product is exact), then the 64
// partials combine as p += shfl_xor(p, s) for s = 32..1 and lane 0 holds the
// logit. This per-row order is the same for every m, so a token's logits
// never depend on the batch it rides in.
// ---------------------------------------------------------------------------
constexpr int kRouterTok = 8;

__global__ __launch_bounds__(256) void k_router(const uint16_t* __restrict__ x, int m, int dim,
                                                const uint16_t* __restrict__ gate_w, int n_routed, float temp,
                                                float* __restrict__ logits, float* __restrict__ scores,
                                                float* __restrict__ logits_out) {
  int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  int lane = threadIdx.x & 63;
  if (e >= n_routed) return;
  const uint16_t* wr = gate_w + (int64_t)e * dim;
  for (int t0 = 0; t0 < m; t0 += kRouterTok) {
    int nt = min(kRouterTok, m - t0);
    float p[kRouterTok];
#pragma unroll
    for (int t = 0; t < kRouterTok; ++t) p[t] = 0.0f;
    for (int base = 0; base < dim; base += 512) {
      int k = base + 8 * lane;
      if (k < dim) {
        uint4 wv = *reinterpret_cast<const uint4*>(wr + k);
        uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int t = 0; t < kRouterTok; ++t) {
          if (t < nt) {
            uint4 xv = *reinterpret_cast<const uint4*>(x + (int64_t)(t0 + t) * dim + k);
            uint32_t xx[4] = {xv.x, xv.y, xv.z, xv.w};
            float acc = p[t];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              uint16_t xb = (uint16_t)(xx[j >> 1] >> (16 * (j & 1)));
              uint16_t wb = (uint16_t)(ww[j >> 1] >> (16 * (j & 1)));
              acc = fadd(acc, fmul(bf16_f32(xb), bf16_f32(wb)));
            }
            p[t] = acc;
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kRouterTok; ++t) {
      float v = p[t];
      for (int s = 32; s >= 1; s >>= 1) v = fadd(v, __shfl_xor(v, s));
      p[t] = v;
    }
    if (lane < nt) {
      // lane t handles token t0 + t (all lanes hold every token's logit)
      float lg = 0.0f;
#pragma unroll
      for (int t = 0; t < kRouterTok; ++t)
        if (t == lane) lg = p[t];
      int64_t o = (int64_t)(t0 + lane) * n_routed + e;
      logits[o] = lg;
      if (logits_out) logits_out[o] = lg;
      scores[o] = score_of(lg, temp);
    }
  }
}

// ---------------------------------------------------------------------------
// Selection: one wave per token. key = score + bias; the top-k by key,
// larger first, equal keys by ascending id (the pages' stable sort), NaN keys
// last; weights from the unbiased scores of the picks [moe_v41.rs,
// fn route_from_logits]; the header [device_route.rs, fn parse_header].
// ---------------------------------------------------------------------------
__device__ inline bool ranks_before(float ka, int a, float kb, int b) {
  bool na = isnan(ka), nb = isnan(kb);
  if (na != nb) return !na;
  if (!na && ka != kb) return ka > kb;
  return a < b;
}

__global__ __launch_bounds__(64) void k_select(const float* __restrict__ scores, const float* __restrict__ bias,
                                               int n_routed, int topk, int norm, float route_scale,
                                               int32_t* __restrict__ header, int32_t* __restrict__ status) {
  int t = blockIdx.x;
  int lane = threadIdx.x;
  const float* sc = scores + (int64_t)t * n_routed;
  constexpr int kPer = kMaxRouted / 64;
  float key[kPer];
  uint32_t taken = 0;
  bool any_nan = false;
#pragma unroll
  for (int c = 0; c < kPer; ++c) {
    int e = lane + 64 * c;
    key[c] = e < n_routed ? fadd(sc[e], bias[e]) : 0.0f;
    if (e < n_routed && isnan(key[c])) any_nan = true;
  }
  int picks[kMaxTopk];
  for (int r = 0; r < topk; ++r) {
    float bk = 0.0f;
    int bid = 0x7fffffff;
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
      int e = lane + 64 * c;
      if (e < n_routed && !((taken >> c) & 1u) && (bid == 0x7fffffff || ranks_before(key[c], e, bk, bid))) {
        bk = key[c];
        bid = e;
      }
    }
    for (int s = 32; s >= 1; s >>= 1) {
      float ok = __shfl_xor(bk, s);
      int oid = __shfl_xor(bid, s);
      if (oid != 0x7fffffff && (bid == 0x7fffffff || ranks_before(ok, oid, bk, bid))) {
        bk = ok;
        bid = oid;
      }
    }
    picks[r] = bid;
    if ((bid & 63) == lane) taken |= 1u << (bid >> 6);
  }
  bool nan_any = __any(any_nan);
  if (lane == 0) {
    float wt[kMaxTopk];
    for (int i = 0; i < topk; ++i) wt[i] = sc[picks[i]];
    if (norm && topk > 1) {
      float sum = 0.0f;
      for (int i = 0; i < topk; ++i) sum = fadd(sum, wt[i]);
      sum = fadd(sum, 1e-20f);
      for (int i = 0; i < topk; ++i) wt[i] = (float)((double)wt[i] / (double)sum);
    }
    for (int i = 0; i < topk; ++i) wt[i] = fmul(wt[i], route_scale);
    int32_t* hd = header + (int64_t)t * (1 + 3 * topk);
    hd[0] = nan_any ? MOE_STATUS_NAN_KEY : 0;
    int plan[kMaxTopk];
    for (int i = 0; i < topk; ++i) {
      hd[1 + i] = picks[i];
      hd[1 + topk + i] = (int32_t)__builtin_bit_cast(uint32_t, wt[i]);
      plan[i] = picks[i];
    }
    for (int a = 1; a < topk; ++a)
      for (int b = a; b > 0 && plan[b] < plan[b - 1]; --b) {
        int tmp = plan[b];
        plan[b] = plan[b - 1];
        plan[b - 1] = tmp;
      }
    for (int i = 0; i < topk; ++i) hd[1 + 2 * topk + i] = plan[i];
    if (nan_any) atomicOr(status, MOE_STATUS_NAN_KEY);
  }
}

// ---------------------------------------------------------------------------
// Plan tables from the headers: the (expert, token) pairs in ascending
// expert id then token, the distinct experts, and per token its pairs in
// plan order [device_route.rs, fn device_route_check: weights and pointers
// in plan order]. One workgroup; invalid picks disable their token.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_plan(const int32_t* __restrict__ header, int m, int topk, int n_routed,
                                              PlanView plan, int32_t* __restrict__ status) {
  __shared__ int cnt[kMaxRouted];
  __shared__ int off[kMaxRouted];
  __shared__ int uid[kMaxRouted];
  __shared__ int n_u_s, bad_s;
  const int hw = 1 + 3 * topk;
  int tid = threadIdx.x;
  for (int e = tid; e < n_routed; e += 256) cnt[e] = 0;
  if (tid == 0) bad_s = 0;
  __syncthreads();
  // token validity: picks in range and distinct
  for (int t = tid; t < m; t += 256) {
    const int32_t* hd = header + (int64_t)t * hw;
    bool ok = true;
    for (int i = 0; i < topk; ++i) {
      int e = hd[1 + i];
      if (e < 0 || e >= n_routed) ok = false;
      for (int j = 0; j < i; ++j)
        if (hd[1 + j] == e) ok = false;
    }
    if (!ok) {
      atomicOr(&bad_s, 1);
      for (int i = 0; i < topk; ++i) plan.tok_pairs()[t * topk + i] = -1;
    } else {
      for (int i = 0; i < topk; ++i) atomicAdd(&cnt[hd[1 + i]], 1);
    }
  }
  __syncthreads();
  if (tid == 0) {
    int o = 0, nu = 0;
    for (int e = 0; e < n_routed; ++e) {
      off[e] = o;
      uid[e] = cnt[e] ? nu : -1;
      if (cnt[e]) {
        plan.u_expert()[nu] = e;
        plan.u_first()[nu] = o;
        plan.u_npairs()[nu] = cnt[e];
        ++nu;
      }
      o += cnt[e];
    }
    n_u_s = nu;
    *plan.n_u() = nu;
    *plan.n_pairs() = o;
    if (bad_s) atomicOr(status, MOE_STATUS_BAD_PICK);
  }
  __syncthreads();
  int P = m * topk;
  for (int q = tid; q < P; q += 256) {
    int t = q / topk, i = q % topk;
    const int32_t* hd = header + (int64_t)t * hw;
    int e = hd[1 + i];
    bool ok = true;
    for (int a = 0; a < topk; ++a) {
      int ea = hd[1 + a];
      if (ea < 0 || ea >= n_routed) ok = false;
      for (int b = 0; b < a; ++b)
        if (hd[1 + b] == ea) ok = false;
    }
    if (!ok) continue;
    // rank among the valid tokens before t that picked e
    int before = 0;
    for (int t2 = 0; t2 < t; ++t2) {
      const int32_t* h2 = header + (int64_t)t2 * hw;
      bool ok2 = true, has = false;
      for (int a = 0; a < topk; ++a) {
        int ea = h2[1 + a];
        if (ea < 0 || ea >= n_routed) ok2 = false;
        for (int b = 0; b < a; ++b)
          if (h2[1 + b] == ea) ok2 = false;
        if (ea == e) has = true;
      }
      if (ok2 && has) ++before;
    }
    int pos = off[e] + before;
    plan.pair_tok()[pos] = t;
    plan.pair_expert()[pos] = e;
    plan.pair_w()[pos] = __builtin_bit_cast(float, hd[1 + topk + i]);
    // this pick's place in the token's plan order (ascending id)
    int rank = 0;
    for (int a = 0; a < topk; ++a)
      if (hd[1 + a] < e) ++rank;
    plan.tok_pairs()[t * topk + rank] = pos;
  }
}

__global__ __launch_bounds__(256) void k_scores(const float* __restrict__ lg, int64_t n, float temp,
                                                float* __restrict__ out, int force_slow) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = score_of(lg[i], temp, force_slow != 0);
}

}  // namespace

hipError_t launch_quant_x(const uint16_t* x, int m, int dim, const Ws& w, hipStream_t s) {
  int64_t n = (int64_t)m * dim;
  hipLaunchKernelGGL(k_quant_x, dim3((unsigned)(n / 256)), dim3(256), 0, s, x, n, w.xq, w.xd, w.xs, w.status);
  return hipGetLastError();
}

hipError_t launch_router(const uint16_t* x, int m, const uint16_t* gate_w, const moe_cfg& c, const Ws& w,
                         float* logits_out, hipStream_t s) {
  timed_begin(MOE_K_ROUTER, s);
  hipLaunchKernelGGL(k_router, dim3((c.n_routed + 3) / 4), dim3(256), 0, s, x, m, c.dim, gate_w, c.n_routed,
                     c.gate_temp, w.logits, w.scores, logits_out);
  hipError_t err = hipGetLastError();
  timed_end(MOE_K_ROUTER, s);
  return err;
}

hipError_t launch_select(const float* bias, int m, const moe_cfg& c, const Ws& w, int32_t* header, hipStream_t s) {
  hipLaunchKernelGGL(k_select, dim3(m), dim3(64), 0, s, w.scores, bias, c.n_routed, c.topk, c.norm_topk_prob,
                     c.route_scale, header, w.status);
  return hipGetLastError();
}

hipError_t launch_plan(const int32_t* header, int m, const moe_cfg& c, const Ws& w, hipStream_t s) {
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(256), 0, s, header, m, c.topk, c.n_routed, w.plan, w.status);
  return hipGetLastError();
}

hipError_t launch_scores(const float* logits, int64_t n, float temp, float* out, int flags, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_scores, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, logits, n, temp, out, flags & 1);
  return hipGetLastError();
}

}  // namespace moe
