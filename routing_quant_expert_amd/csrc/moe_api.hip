// The C ABI (include/moe.h): argument checks, the workspace layout and the
// launch sequences of the entry points.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <mutex>
#include <string>

#include "moe_host.h"
#include "moe_internal.h"
#include "moe_math.h"
#include "moe_prefill.h"

namespace moe {
namespace {

thread_local std::string g_err;
constexpr int kTimedKernels = 9;   // MOE_K_* ids 1..8
thread_local hipEvent_t g_ev_begin[kTimedKernels] = {};
thread_local hipEvent_t g_ev_end[kTimedKernels] = {};

__global__ void k_zero16(uint4* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = make_uint4(0, 0, 0, 0);
}

// Read-only stream over n16 16-byte words: workgroup b reads its own
// contiguous share (the last one also the remainder), 256 threads with four
// 16-byte loads each in flight per round (of the loop shapes measured, this
// one read fastest). The XOR of everything read decides a store that never
// happens for real data, so no load can be dropped.
__global__ __launch_bounds__(256) void k_read_probe(const uint4* __restrict__ p, uint64_t n16, uint32_t* sink) {
  const uint64_t per = n16 / gridDim.x;
  const uint64_t lo = (uint64_t)blockIdx.x * per;
  const uint64_t hi = blockIdx.x + 1 == gridDim.x ? n16 : lo + per;
  uint32_t acc = 0;
  for (uint64_t i = lo + threadIdx.x; i < hi; i += 4 * 256) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint64_t j = i + u * 256;
      v[u] = j < hi ? p[j] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

int fail(int code, const char* fmt, const char* a, long long b) {
  char buf[512];
  snprintf(buf, sizeof buf, fmt, a, b);
  g_err = buf;
  return code;
}

namespace {

bool pow2_upto16(int v) { return v >= 1 && v <= 16 && (v & (v - 1)) == 0; }

// A prefill layer with a bf16 shared expert runs that expert's two GEMMs on
// a second stream of the device (created on first use, default priority,
// never destroyed), from the start of the call (they need only x), beside
// the router and the routed experts; the caller's stream waits for them
// before the combine. The fork and join are event record/wait pairs, so a
// graph capture of the caller's stream takes the second stream's work in as
// well. A call holds the device's lock while it enqueues (the launches are
// asynchronous, so only for the enqueue), so that calls from several host
// threads cannot interleave their record/wait pairs on the shared events;
// their side work runs in the order the calls took the lock. Everything else
// runs on the caller's stream alone (moe_experts_prefill and layers with a
// K-quant shared expert use no library stream): putting the routed experts
// with more than 8 pairs on the second stream as well gained nothing
// measurable, while the shared GEMMs' overlap with the router saves 2 to 5%
// of a prefill step.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t start = nullptr, done = nullptr;
};
constexpr int kMaxDevices = 64;
SideStream g_side[kMaxDevices];
std::mutex g_side_mu[kMaxDevices];

// The current device's side stream, created on first use, with its lock
// taken into `hold`; nullptr (lock not taken) on failure.
const SideStream* side_stream(std::unique_lock<std::mutex>& hold) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::unique_lock<std::mutex> lock(g_side_mu[dev]);
  SideStream& ss = g_side[dev];
  if (!ss.s) {
    SideStream n;
    if (hipStreamCreateWithFlags(&n.s, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&n.start, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&n.done, hipEventDisableTiming) != hipSuccess)
      return nullptr;
    ss = n;
  }
  hold = std::move(lock);
  return &ss;
}

// `after` (on stream `from`) happens before what is launched next on `to`.
hipError_t fork_join(hipEvent_t after, hipStream_t from, hipStream_t to) {
  hipError_t e = hipEventRecord(after, from);
  if (e != hipSuccess) return e;
  return hipStreamWaitEvent(to, after, 0);
}

}  // namespace

// The single-token kernels: up to 6 picks (a wave each) and down rows of at
// most 8 Q3_K super-blocks (each pick's 16-row tile is staged whole in LDS);
// other shapes take the union path, which is correct for every m <= 8.
// With a K-quant shared expert (shq = 1) its blocks take one more pick's wave
// in place of the two bf16 shared-expert waves.
bool single_token_fits(const moe_cfg& c, int shq) {
  return (shq ? c.topk + 1 <= kMaxTopk : c.topk <= kMaxTopkM1) && c.inter / 256 <= 8;
}

int check_cfg(const moe_cfg* c) {
  if (!c) return fail(MOE_EINVAL, "cfg is NULL%s%lld");
  if (!(c->gate_temp > 0.0f) || !std::isfinite(c->gate_temp) || !std::isfinite(c->route_scale) ||
      !(c->swiglu_limit > 0.0f) || (c->norm_topk_prob != 0 && c->norm_topk_prob != 1))
    return fail(MOE_EINVAL, "cfg value out of range (gate_temp > 0, finite route_scale, swiglu_limit > 0, norm 0/1)%s%lld");
  if (c->dim % 256 || c->inter % 256 || !pow2_upto16(c->dim / 256) || !pow2_upto16(c->inter / 256))
    return fail(MOE_EUNSUPPORTED, "dim and inter must be 256 * a power of two <= 16 %s(dim %lld)", "", c->dim);
  if (c->topk < 1 || c->topk > kMaxTopk || c->n_routed < c->topk || c->n_routed > kMaxRouted)
    return fail(MOE_EUNSUPPORTED, "need 1 <= topk <= 8 and topk <= n_routed <= 1024%s (n_routed %lld)", "", c->n_routed);
  if (c->score_mode != MOE_SCORE_CR && c->score_mode != MOE_SCORE_GLIBC)
    return fail(MOE_EINVAL, "score_mode must be MOE_SCORE_CR or MOE_SCORE_GLIBC%s (%lld)", "", c->score_mode);
  return MOE_OK;
}

// Token counts the kernels index with 32-bit offsets and grid dimensions: at
// most kMaxTokens tokens (the combine's grid rows), and every per-pair
// activation buffer (m * topk rows of max(dim, inter) bytes) under 2^31 bytes
// (the prefill kernels' buffer descriptors and offsets are 32-bit).
int check_m(const moe_cfg& c, int64_t m) {
  if (m < 1) return fail(MOE_EINVAL, "m must be >= 1%s (m %lld)", "", m);
  const int64_t width = c.dim > c.inter ? c.dim : c.inter;
  if (m > kMaxTokens || m * (c.topk + 1) * width >= ((int64_t)1 << 31))
    return fail(MOE_EUNSUPPORTED,
                "too many tokens for one call%s (m %lld; at most 65535 and m*(topk+1)*max(dim,inter) < 2^31)", "", m);
  return MOE_OK;
}

uint64_t take(uint64_t& total, uint64_t bytes) {
  uint64_t off = total;
  total = (total + bytes + 255) & ~(uint64_t)255;
  return off;
}

int check_ws(const moe_cfg& c, int m, void* ws, size_t ws_bytes, moe_ws_layout* L) {
  if (!ws) return fail(MOE_EINVAL, "workspace is NULL%s%lld");
  if ((uintptr_t)ws & 255) return fail(MOE_EINVAL, "workspace must be 256-byte aligned%s%lld");
  layout_of(c, m, L);
  if (ws_bytes < L->total)
    return fail(MOE_EWORKSPACE, "workspace too small%s: need %lld bytes", "", (long long)L->total);
  return MOE_OK;
}

bool a16(const void* p) { return ((uintptr_t)p & 15) == 0; }

int hip_fail(hipError_t e, const char* where) {
  return fail(MOE_EHIP, "HIP error in %s: code %lld", where, (long long)e);
}

int check_experts(const moe_experts* ex) {
  if (!ex || !ex->base) return fail(MOE_EINVAL, "experts / experts->base is NULL%s%lld");
  if (!a16(ex->base) || (ex->stride & 15) || (ex->gate_off & 15) || (ex->up_off & 15) || (ex->down_off & 15))
    return fail(MOE_EINVAL, "expert arena: base, stride and offsets must be multiples of 16 bytes%s%lld");
  // the prefill kernels address a matrix inside an expert with 32-bit offsets
  const uint64_t lim = (uint64_t)1 << 31;
  if (ex->gate_off >= lim || ex->up_off >= lim || ex->down_off >= lim)
    return fail(MOE_EUNSUPPORTED, "expert arena: matrix offsets must be below 2^31 bytes%s%lld");
  return MOE_OK;
}

XArena arena_of(const moe_experts& ex, int n_routed, const moe_experts* shared_q, const int32_t* slot_of) {
  XArena a;
  a.base = static_cast<const uint8_t*>(ex.base);
  a.stride = ex.stride;
  a.gate_off = ex.gate_off;
  a.up_off = ex.up_off;
  a.down_off = ex.down_off;
  a.sbase = shared_q ? static_cast<const uint8_t*>(shared_q->base) : nullptr;
  a.sgate_off = shared_q ? shared_q->gate_off : 0;
  a.sup_off = shared_q ? shared_q->up_off : 0;
  a.sdown_off = shared_q ? shared_q->down_off : 0;
  a.n_routed = n_routed;
  a.slot_of = slot_of;
  return a;
}

// Every token has at most topk + 1 plan entries (its picks and a K-quant
// shared expert), so the pair tables hold max_m * (topk + 1) pairs.
bool layout_of(const moe_cfg& c, int max_m, moe_ws_layout* L) {
  const uint64_t m = max_m, P = (uint64_t)max_m * (c.topk + 1);
  uint64_t t = 0;
  L->ctl = take(t, 256);   // first, so that its place does not depend on m
  L->xq = take(t, m * c.dim);
  L->xd = take(t, m * (c.dim / 32) * 2);
  L->xs = take(t, m * (c.dim / 16) * 4);
  L->logits = take(t, m * c.n_routed * 4);
  L->scores = take(t, m * c.n_routed * 4);
  L->plan_words = PlanView::words((int)P, max_m, c.topk);
  L->plan = take(t, (uint64_t)L->plan_words * 4);
  L->g = take(t, P * c.inter * 4);
  L->u = take(t, P * c.inter * 4);
  L->h = take(t, P * c.inter * 4);
  L->hq = take(t, P * c.inter);
  L->hd = take(t, P * (c.inter / 32) * 2);
  L->hs = take(t, P * (c.inter / 16) * 4);
  L->y = take(t, P * c.dim * 4);
  L->sg = take(t, m * c.inter * 4);
  L->su = take(t, m * c.inter * 4);
  L->sh = take(t, m * c.inter * 2);
  L->sd = take(t, m * c.dim * 4);
  L->yr = take(t, m * c.dim * 4);
  L->status = take(t, 16 + m * (1 + 3 * c.topk) * 4);   // status words, then a header scratch
  L->grp = take(t, (m + 2 * ((uint64_t)c.n_routed + 1)) * 4);
  L->xd64 = take(t, m * (c.dim / 32) * 8);
  L->hd64 = take(t, P * (c.inter / 32) * 8);
  L->total = t;
  L->max_pairs = (int32_t)P;
  return true;
}

Ws ws_view(void* ws, const moe_ws_layout& L, const moe_cfg& c, int max_m) {
  uint8_t* b = static_cast<uint8_t*>(ws);
  Ws w;
  w.xq = reinterpret_cast<int8_t*>(b + L.xq);
  w.xd = reinterpret_cast<uint16_t*>(b + L.xd);
  w.xs = reinterpret_cast<int32_t*>(b + L.xs);
  w.logits = reinterpret_cast<float*>(b + L.logits);
  w.scores = reinterpret_cast<float*>(b + L.scores);
  w.plan = PlanView{reinterpret_cast<int32_t*>(b + L.plan), L.max_pairs, max_m, c.topk};
  w.g = reinterpret_cast<float*>(b + L.g);
  w.u = reinterpret_cast<float*>(b + L.u);
  w.h = reinterpret_cast<float*>(b + L.h);
  w.hq = reinterpret_cast<int8_t*>(b + L.hq);
  w.hd = reinterpret_cast<uint16_t*>(b + L.hd);
  w.hs = reinterpret_cast<int32_t*>(b + L.hs);
  w.y = reinterpret_cast<float*>(b + L.y);
  w.sg = reinterpret_cast<float*>(b + L.sg);
  w.su = reinterpret_cast<float*>(b + L.su);
  w.sh = reinterpret_cast<uint16_t*>(b + L.sh);
  w.sd = reinterpret_cast<float*>(b + L.sd);
  w.yr = reinterpret_cast<float*>(b + L.yr);
  w.status = reinterpret_cast<int32_t*>(b + L.status);
  w.ctl = reinterpret_cast<Ctl*>(b + L.ctl);
  w.xd64 = reinterpret_cast<double*>(b + L.xd64);
  w.hd64 = reinterpret_cast<double*>(b + L.hd64);
  return w;
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero16, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, static_cast<uint4*>(p), n);
  return hipGetLastError();
}

bool take_timed(int which, hipEvent_t* begin, hipEvent_t* end) {
  if (which < 1 || which >= kTimedKernels || !g_ev_begin[which] || !g_ev_end[which]) return false;
  *begin = g_ev_begin[which];
  *end = g_ev_end[which];
  g_ev_begin[which] = g_ev_end[which] = nullptr;
  return true;
}

int check_layer(const moe_layer* layer, bool need_experts) {
  if (!layer || !layer->gate_w || !layer->bias) return fail(MOE_EINVAL, "layer weights must be non-NULL%s%lld");
  if (layer->shared_kind == MOE_SHARED_BF16) {
    if (!layer->sh_w1 || !layer->sh_w2 || !layer->sh_w3)
      return fail(MOE_EINVAL, "the bf16 shared expert's matrices must be non-NULL%s%lld");
    if (!a16(layer->sh_w1) || !a16(layer->sh_w2) || !a16(layer->sh_w3))
      return fail(MOE_EINVAL, "the bf16 weights must be 16-byte aligned%s%lld");
  } else if (layer->shared_kind == MOE_SHARED_KQUANT) {
    if (int r = check_experts(&layer->shared_q)) return r;
  } else {
    return fail(MOE_EINVAL, "unknown shared_kind%s %lld", "", layer->shared_kind);
  }
  if (!a16(layer->gate_w)) return fail(MOE_EINVAL, "gate_w must be 16-byte aligned%s%lld");
  return need_experts ? check_experts(&layer->experts) : MOE_OK;
}

bool shared_bf16(const moe_layer& layer) { return layer.shared_kind == MOE_SHARED_BF16; }

// The prefill expert stage on `s`: gate/up and down of the experts with more
// than 8 pairs, then of the others.
hipError_t prefill_expert_launches(const XArena& ar, int m, const moe_cfg& c, const Ws& w, hipStream_t s) {
  hipError_t e;
  for (int part = 1; part >= 0; --part) {
    if ((e = launch_gateup_pf(ar, m, c, w, part, s)) != hipSuccess) return e;
    if ((e = launch_down_pf(ar, m, c, w, part, s)) != hipSuccess) return e;
  }
  return hipSuccess;
}

XArena layer_arena(const moe_cfg& c, const moe_layer& layer) {
  return arena_of(layer.experts, c.n_routed, shared_bf16(layer) ? nullptr : &layer.shared_q);
}

// One layer's launches on `s` (A1-A7), the result to `o`.
int layer_launches(const moe_cfg& c, const moe_layer& layer, const uint16_t* x, int m, const LayerOut& o,
                   int32_t* hdr, const Ws& w, int32_t* grp, hipStream_t s) {
  hipError_t e;
  const bool bf16 = shared_bf16(layer);
  const XArena ar = layer_arena(c, layer);
  const int shq = ar.has_shared();
  FrontSelect sel{layer.bias, hdr, shq};
  if (m > kMaxDecodeTokens) {   // prefill
    std::unique_lock<std::mutex> hold;
    const SideStream* ss = nullptr;
    if (bf16) {
      if (!(ss = side_stream(hold))) return fail(MOE_EHIP, "could not create the prefill side stream%s%lld");
      if ((e = fork_join(ss->start, s, ss->s)) != hipSuccess) return hip_fail(e, "fork");
      if ((e = launch_shared_pf(x, m, layer, c, w, ss->s)) != hipSuccess) return hip_fail(e, "shared_pf");
    }
    if ((e = launch_router_pf(x, m, layer.gate_w, c, w, nullptr, s)) != hipSuccess) return hip_fail(e, "router_pf");
    if ((e = launch_select(layer.bias, m, c, w, hdr, s)) != hipSuccess) return hip_fail(e, "select");
    if ((e = launch_group(hdr, m, c, w, grp, shq, s)) != hipSuccess) return hip_fail(e, "group");
    if ((e = prefill_expert_launches(ar, m, c, w, s)) != hipSuccess) return hip_fail(e, "experts_pf");
    if (ss && (e = fork_join(ss->done, ss->s, s)) != hipSuccess) return hip_fail(e, "join");
    if ((e = launch_combine(m, c, w, bf16 ? w.sd : nullptr, o, s)) != hipSuccess) return hip_fail(e, "combine");
    return MOE_OK;
  }
  if (m == 1 && single_token_fits(c, shq)) {   // router + q8_1; selection, routed and shared gate/up; down + combine
    if ((e = launch_front(x, 1, layer.gate_w, nullptr, nullptr, nullptr, c, w, nullptr, s)) != hipSuccess)
      return hip_fail(e, "front");
    if ((e = launch_gateup_m1(ar, &sel, nullptr, x, bf16 ? &layer : nullptr, c, w, s)) != hipSuccess)
      return hip_fail(e, "gateup_m1");
    if ((e = launch_down_m1(ar, c, w, bf16 ? layer.sh_w2 : nullptr, o, s)) != hipSuccess) return hip_fail(e, "down_m1");
    return MOE_OK;
  }
  if ((e = launch_front(x, m, layer.gate_w, &sel, bf16 ? layer.sh_w1 : nullptr, bf16 ? layer.sh_w3 : nullptr, c, w,
                        nullptr, s)) != hipSuccess)
    return hip_fail(e, "front");
  if ((e = launch_gateup(ar, m, c, w, s)) != hipSuccess) return hip_fail(e, "gateup");
  if ((e = launch_down(ar, m, c, w, bf16 ? layer.sh_w2 : nullptr, s)) != hipSuccess) return hip_fail(e, "down");
  if ((e = launch_combine(m, c, w, bf16 ? w.sd : nullptr, o, s)) != hipSuccess) return hip_fail(e, "combine");
  return MOE_OK;
}

// Routing of m tokens on `s`: q8_1 of x, the router and its scores, the top-k
// and the headers (slot_of: an expert cache's slot-table row, see launch_select).
hipError_t route_launches(const moe_cfg& c, const uint16_t* x, int m, const uint16_t* gate_w, const float* bias,
                          int32_t* header, const Ws& w, const int32_t* slot_of, hipStream_t s) {
  hipError_t e = m > kMaxDecodeTokens ? launch_router_pf(x, m, gate_w, c, w, nullptr, s)
                                      : launch_front(x, m, gate_w, nullptr, nullptr, nullptr, c, w, nullptr, s);
  if (e != hipSuccess) return e;
  return launch_select(bias, m, c, w, header, s, slot_of);
}

// The layer after its routing, from the picks in `header` (device): the
// routed experts out of arena `ar`, the shared expert and the combine, each
// token's values exactly as layer_launches computes them (the same kernels,
// fed the header instead of selecting).
int layer_launches_hdr(const moe_cfg& c, const moe_layer& layer, const XArena& ar, const uint16_t* x, int m,
                       const int32_t* header, const LayerOut& o, const Ws& w, int32_t* grp, hipStream_t s) {
  hipError_t e;
  const bool bf16 = shared_bf16(layer);
  const int shq = ar.has_shared();
  if (m > kMaxDecodeTokens) {
    std::unique_lock<std::mutex> hold;
    const SideStream* ss = nullptr;
    if (bf16) {
      if (!(ss = side_stream(hold))) return fail(MOE_EHIP, "could not create the prefill side stream%s%lld");
      if ((e = fork_join(ss->start, s, ss->s)) != hipSuccess) return hip_fail(e, "fork");
      if ((e = launch_shared_pf(x, m, layer, c, w, ss->s)) != hipSuccess) return hip_fail(e, "shared_pf");
    }
    if ((e = launch_router_pf(x, m, nullptr, c, w, nullptr, s)) != hipSuccess) return hip_fail(e, "quant_pf");
    if ((e = launch_group(header, m, c, w, grp, shq, s)) != hipSuccess) return hip_fail(e, "group");
    if ((e = prefill_expert_launches(ar, m, c, w, s)) != hipSuccess) return hip_fail(e, "experts_pf");
    if (ss && (e = fork_join(ss->done, ss->s, s)) != hipSuccess) return hip_fail(e, "join");
    if ((e = launch_combine(m, c, w, bf16 ? w.sd : nullptr, o, s)) != hipSuccess) return hip_fail(e, "combine");
    return MOE_OK;
  }
  if (m == 1 && single_token_fits(c, shq)) {
    if ((e = launch_quant_x(x, 1, c, w, s)) != hipSuccess) return hip_fail(e, "quant_x");
    if ((e = launch_gateup_m1(ar, nullptr, header, x, bf16 ? &layer : nullptr, c, w, s)) != hipSuccess)
      return hip_fail(e, "gateup_m1");
    if ((e = launch_down_m1(ar, c, w, bf16 ? layer.sh_w2 : nullptr, o, s)) != hipSuccess) return hip_fail(e, "down_m1");
    return MOE_OK;
  }
  if ((e = launch_front(x, m, nullptr, nullptr, bf16 ? layer.sh_w1 : nullptr, bf16 ? layer.sh_w3 : nullptr, c, w,
                        nullptr, s)) != hipSuccess)
    return hip_fail(e, "front");
  if ((e = launch_plan(header, m, c, w, s, shq)) != hipSuccess) return hip_fail(e, "plan");
  if ((e = launch_gateup(ar, m, c, w, s)) != hipSuccess) return hip_fail(e, "gateup");
  if ((e = launch_down(ar, m, c, w, bf16 ? layer.sh_w2 : nullptr, s)) != hipSuccess) return hip_fail(e, "down");
  if ((e = launch_combine(m, c, w, bf16 ? w.sd : nullptr, o, s)) != hipSuccess) return hip_fail(e, "combine");
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// The fixed scratch of moe_layer_forward_noalloc: one workspace-sized array
// per GPU, held from the library's load until the process ends, so that the
// entry point needs no allocation. Its name is a host-side stand-in, not a
// device address: the address each device's copy has is looked up once per
// device (with that device current) and kept; only that pointer is passed to
// kernels. Every call on a GPU shares the array, so calls that overlap on one
// GPU race.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)6 << 20;   // every supported shape at m <= 8 needs at most 5.7 MiB
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
void* g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mu[kMaxDevices];
}  // namespace

// This device's copy of `scratch`. On the first use on a device: look its
// address up and zero its control words (offset 0 in every workspace layout)
// with a fill kernel on `s`, ahead of the call's own launches; every call
// leaves them zero again. The rest of a workspace needs no initialisation.
int scratch_of_device(hipStream_t s, uint8_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_EUNSUPPORTED, "device index out of range%s (%lld)", "", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu[dev]);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    if ((e = launch_zero(p, 256, s)) != hipSuccess) return hip_fail(e, "scratch control words");
    g_scratch[dev] = p;
  }
  *out = static_cast<uint8_t*>(g_scratch[dev]);
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

int32_t moe_header_words(const moe_cfg* cfg) { return cfg ? 1 + 3 * cfg->topk : 0; }

size_t moe_workspace_bytes(const moe_cfg* cfg, int32_t max_m) {
  if (check_cfg(cfg) != MOE_OK || check_m(*cfg, max_m) != MOE_OK) return 0;
  moe_ws_layout L;
  layout_of(*cfg, max_m, &L);
  return L.total;
}

int moe_workspace_init(const moe_cfg* cfg, int32_t max_m, void* ws, size_t ws_bytes, void* stream) {
  if (int r = check_cfg(cfg)) return r;
  if (int r = check_m(*cfg, max_m)) return r;
  moe_ws_layout L;
  if (int r = check_ws(*cfg, max_m, ws, ws_bytes, &L)) return r;
  hipError_t e = launch_zero(static_cast<uint8_t*>(ws) + L.ctl, 256, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "workspace_init");
}

int moe_workspace_layout(const moe_cfg* cfg, int32_t max_m, moe_ws_layout* out) {
  if (int r = check_cfg(cfg)) return r;
  if (!out) return fail(MOE_EINVAL, "layout output is NULL%s%lld");
  if (int r = check_m(*cfg, max_m)) return r;
  layout_of(*cfg, max_m, out);
  return MOE_OK;
}

int moe_route_select(const moe_cfg* cfg, const uint16_t* x, int32_t m, const uint16_t* gate_w, const float* bias,
                     float* logits, int32_t* header, void* ws, size_t ws_bytes, void* stream) {
  if (int r = check_cfg(cfg)) return r;
  if (int r = check_score_mode(*cfg)) return r;
  if (!x || !gate_w || !bias || !header) return fail(MOE_EINVAL, "x, gate_w, bias and header must be non-NULL%s%lld");
  if (int r = check_m(*cfg, m)) return r;
  if (!a16(x) || !a16(gate_w)) return fail(MOE_EINVAL, "x and gate_w must be 16-byte aligned%s%lld");
  moe_ws_layout L;
  if (int r = check_ws(*cfg, m, ws, ws_bytes, &L)) return r;
  Ws w = ws_view(ws, L, *cfg, m);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if ((e = launch_front(x, m, gate_w, nullptr, nullptr, nullptr, *cfg, w, logits, s)) != hipSuccess)
    return hip_fail(e, "front");
  if ((e = launch_select(bias, m, *cfg, w, header, s)) != hipSuccess) return hip_fail(e, "select");
  return MOE_OK;
}

int moe_experts_decode(const moe_cfg* cfg, const uint16_t* x, int32_t m, const int32_t* header,
                       const moe_experts* experts, float* y_routed, void* ws, size_t ws_bytes, void* stream) {
  if (int r = check_cfg(cfg)) return r;
  if (!x || !header || !y_routed) return fail(MOE_EINVAL, "x, header and y_routed must be non-NULL%s%lld");
  if (m < 1 || m > kMaxDecodeTokens) return fail(MOE_EINVAL, "decode needs 1 <= m <= 8%s (m %lld)", "", m);
  if (!a16(x)) return fail(MOE_EINVAL, "x must be 16-byte aligned%s%lld");
  if (int r = check_experts(experts)) return r;
  moe_ws_layout L;
  if (int r = check_ws(*cfg, m, ws, ws_bytes, &L)) return r;
  Ws w = ws_view(ws, L, *cfg, m);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if ((e = launch_quant_x(x, m, *cfg, w, s)) != hipSuccess) return hip_fail(e, "quant_x");
  const XArena ar = arena_of(*experts, cfg->n_routed, nullptr);
  if (m == 1 && single_token_fits(*cfg)) {
    if ((e = launch_gateup_m1(ar, nullptr, header, x, nullptr, *cfg, w, s)) != hipSuccess)
      return hip_fail(e, "gateup_m1");
    if ((e = launch_down_m1(ar, *cfg, w, nullptr, LayerOut{y_routed, nullptr, nullptr, nullptr}, s)) !=
        hipSuccess)
      return hip_fail(e, "down_m1");
    return MOE_OK;
  }
  if ((e = launch_plan(header, m, *cfg, w, s)) != hipSuccess) return hip_fail(e, "plan");
  if ((e = launch_gateup(ar, m, *cfg, w, s)) != hipSuccess) return hip_fail(e, "gateup");
  if ((e = launch_down(ar, m, *cfg, w, nullptr, s)) != hipSuccess) return hip_fail(e, "down");
  if ((e = launch_combine(m, *cfg, w, nullptr, LayerOut{y_routed, nullptr, nullptr, nullptr}, s)) != hipSuccess)
    return hip_fail(e, "combine");
  return MOE_OK;
}

int moe_experts_prefill(const moe_cfg* cfg, const uint16_t* x, int32_t m, const int32_t* header,
                        const moe_experts* experts, float* y_routed, void* ws, size_t ws_bytes, void* stream) {
  if (int r = check_cfg(cfg)) return r;
  if (!x || !header || !y_routed) return fail(MOE_EINVAL, "x, header and y_routed must be non-NULL%s%lld");
  if (int r = check_m(*cfg, m)) return r;
  if (!a16(x)) return fail(MOE_EINVAL, "x must be 16-byte aligned%s%lld");
  if (int r = check_experts(experts)) return r;
  moe_ws_layout L;
  if (int r = check_ws(*cfg, m, ws, ws_bytes, &L)) return r;
  Ws w = ws_view(ws, L, *cfg, m);
  int32_t* grp = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + L.grp);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if ((e = launch_router_pf(x, m, nullptr, *cfg, w, nullptr, s)) != hipSuccess) return hip_fail(e, "quant_pf");
  if ((e = launch_group(header, m, *cfg, w, grp, 0, s)) != hipSuccess) return hip_fail(e, "group");
  const XArena ar = arena_of(*experts, cfg->n_routed, nullptr);
  if ((e = prefill_expert_launches(ar, m, *cfg, w, s)) != hipSuccess) return hip_fail(e, "experts_pf");
  if ((e = launch_combine(m, *cfg, w, nullptr, LayerOut{y_routed, nullptr, nullptr, nullptr}, s)) != hipSuccess)
    return hip_fail(e, "combine");
  return MOE_OK;
}

int moe_layer_forward(const moe_cfg* cfg, const moe_layer* layer, const uint16_t* x, int32_t m, uint16_t* out_bf16,
                      float* out_f32, int32_t* header, void* ws, size_t ws_bytes, void* stream) {
  if (int r = check_cfg(cfg)) return r;
  if (int r = check_score_mode(*cfg)) return r;
  if (!x || !out_bf16) return fail(MOE_EINVAL, "x and out_bf16 must be non-NULL%s%lld");
  if (int r = check_layer(layer)) return r;
  if (int r = check_m(*cfg, m)) return r;
  if (!a16(x)) return fail(MOE_EINVAL, "x must be 16-byte aligned%s%lld");
  moe_ws_layout L;
  if (int r = check_ws(*cfg, m, ws, ws_bytes, &L)) return r;
  Ws w = ws_view(ws, L, *cfg, m);
  LayerOut o{out_f32, out_bf16, nullptr, nullptr};
  int32_t* grp = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + L.grp);
  return layer_launches(*cfg, *layer, x, m, o, header ? header : w.status + 4, w, grp, (hipStream_t)stream);
}

int moe_stack_forward(const moe_cfg* cfg, const moe_layer* layers, int32_t n_layers, uint16_t* xs, int32_t m,
                      float* out_f32, int32_t* headers, void* ws, size_t ws_bytes, void* stream) {
  if (int r = check_cfg(cfg)) return r;
  if (int r = check_score_mode(*cfg)) return r;
  if (!layers || !xs) return fail(MOE_EINVAL, "layers and xs must be non-NULL%s%lld");
  if (n_layers < 1) return fail(MOE_EINVAL, "n_layers must be >= 1%s (n_layers %lld)", "", n_layers);
  if (int r = check_m(*cfg, m)) return r;
  if (!a16(xs) || ((int64_t)m * cfg->dim * 2) % 16) return fail(MOE_EINVAL, "xs must be 16-byte aligned%s%lld");
  for (int l = 0; l < n_layers; ++l)
    if (int r = check_layer(&layers[l])) return r;
  moe_ws_layout L;
  if (int r = check_ws(*cfg, m, ws, ws_bytes, &L)) return r;
  Ws w = ws_view(ws, L, *cfg, m);
  const int64_t row = (int64_t)m * cfg->dim;
  const int hw = 1 + 3 * cfg->topk;
  int32_t* grp = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + L.grp);
  for (int l = 0; l < n_layers; ++l) {
    LayerOut o{out_f32 ? out_f32 + l * row : nullptr, nullptr, xs + l * row, xs + (l + 1) * row};
    int32_t* hdr = headers ? headers + (int64_t)l * m * hw : w.status + 4;
    if (int r = layer_launches(*cfg, layers[l], xs + l * row, m, o, hdr, w, grp, (hipStream_t)stream)) return r;
  }
  return MOE_OK;
}

// The flag bits of moe_scores and moe_scores_host: 0 the extended path, 1
// the glibc mode, 2 the exp step alone (not with bit 1).
static int check_score_flags(int32_t flags) {
  if ((flags & ~7) || ((flags & 4) && (flags & 2)))
    return fail(MOE_EINVAL, "score flags: bits 0..2, bit 2 not with bit 1 (got %s%lld)", "", (long long)flags);
  return MOE_OK;
}

int moe_scores(const float* logits, int64_t n, float temp, float* out, int32_t flags, void* stream) {
  if (n < 0 || (n > 0 && (!logits || !out))) return fail(MOE_EINVAL, "bad scores arguments%s%lld");
  if (int r = check_score_flags(flags)) return r;
  if (flags & 2) {
    moe_cfg glibc{};
    glibc.score_mode = MOE_SCORE_GLIBC;
    if (int r = check_score_mode(glibc)) return r;
  }
  hipError_t e = launch_scores(logits, n, temp, out, flags, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "scores");
}

int moe_scores_host(const float* logits, int64_t n, float temp, float* out, int32_t flags) {
  if (n < 0 || (n > 0 && (!logits || !out))) return fail(MOE_EINVAL, "bad scores arguments%s%lld");
  if (int r = check_score_flags(flags)) return r;
  if (flags & 4) {
    for (int64_t i = 0; i < n; ++i)
      out[i] = exp_cr(temp == 1.0f ? logits[i] : (float)((double)logits[i] / (double)temp), (flags & 1) != 0);
    return MOE_OK;
  }
  if (flags & 2) {
    return guarded([&] {
      const ScoreTable t = host_score_table();
      for (int64_t i = 0; i < n; ++i) out[i] = score_mode_of(logits[i], temp, t);
      return MOE_OK;
    });
  }
  for (int64_t i = 0; i < n; ++i) out[i] = score_of(logits[i], temp, (flags & 1) != 0);
  return MOE_OK;
}

int moe_swiglu_host(const float* g, const float* u, int64_t n, float limit, float* out) {
  if (n < 0 || (n > 0 && (!g || !u || !out))) return fail(MOE_EINVAL, "bad swiglu arguments%s%lld");
  for (int64_t i = 0; i < n; ++i) out[i] = swiglu(g[i], u[i], limit);
  return MOE_OK;
}

int moe_time_next_launch(int32_t which, void* ev_begin, void* ev_end) {
  if (which < 1 || which >= kTimedKernels) return fail(MOE_EINVAL, "unknown kernel id%s %lld", "", which);
  g_ev_begin[which] = (hipEvent_t)ev_begin;
  g_ev_end[which] = (hipEvent_t)ev_end;
  return MOE_OK;
}

int moe_read_probe(const void* buf, uint64_t bytes, uint32_t* sink, int32_t blocks, void* stream) {
  if (!buf || !sink || blocks < 1 || !a16(buf) || (bytes & 15))
    return fail(MOE_EINVAL, "read probe: non-NULL 16-byte aligned buffer, bytes a multiple of 16, blocks >= 1%s%lld");
  if (bytes == 0) return MOE_OK;
  MOE_LAUNCH(MOE_K_READ_PROBE, k_read_probe, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
             static_cast<const uint4*>(buf), bytes / 16, sink);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOE_OK : hip_fail(e, "read_probe");
}

int moe_layer_forward_noalloc(const moe_cfg* cfg, const moe_layer* layer, const uint16_t* x, int32_t m,
                              uint16_t* out_bf16, float* out_f32, int32_t* header, void* stream) {
  if (int r = check_cfg(cfg)) return r;
  if (int r = check_score_mode(*cfg)) return r;
  if (!x || !out_bf16) return fail(MOE_EINVAL, "x and out_bf16 must be non-NULL%s%lld");
  if (int r = check_layer(layer)) return r;
  if (m < 1 || m > kMaxDecodeTokens)
    return fail(MOE_EINVAL, "the no-allocation entry point takes 1 <= m <= 8 tokens%s (m %lld)", "", m);
  if (!a16(x)) return fail(MOE_EINVAL, "x must be 16-byte aligned%s%lld");
  moe_ws_layout L;
  layout_of(*cfg, m, &L);
  if (L.total > kScratchBytes)
    return fail(MOE_EWORKSPACE, "this shape needs %s%lld bytes of workspace, more than the library's fixed scratch",
                "", (long long)L.total);
  const hipStream_t s = (hipStream_t)stream;
  uint8_t* ws = nullptr;
  if (int r = scratch_of_device(s, &ws)) return r;
  Ws w = ws_view(ws, L, *cfg, m);
  LayerOut o{out_f32, out_bf16, nullptr, nullptr};
  int32_t* grp = reinterpret_cast<int32_t*>(ws + L.grp);
  return layer_launches(*cfg, *layer, x, m, o, header ? header : w.status + 4, w, grp, s);
}

const char* moe_last_error(void) { return g_err.c_str(); }

}  // extern "C"
