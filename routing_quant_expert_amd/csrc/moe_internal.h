// Internal declarations shared by the library's translation units:
// workspace layout, plan tables and the kernel launchers.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"
#include "moe_math.h"

namespace moe {

constexpr int kMaxDecodeTokens = 8;   // the union-of-experts decode path
constexpr int kMaxTokens = 65535;      // tokens of one call (see check_m)
constexpr int kMaxTopk = 8;
constexpr int kMaxTopkM1 = 6;   // the single-token kernels: one wave per pick + two shared-expert waves in 512 threads
constexpr int kMaxSlots = kMaxTopk + 1;   // a token's plan entries: its picks and the quantised shared expert
constexpr int kMaxRouted = 1024;
constexpr int kQ2KBytes = 84;
constexpr int kQ3KBytes = 110;

// Plan tables inside the workspace (int32 words):
//   [0] n_u (distinct experts), [1] n_pairs,
//   then max_pairs entries each of u_expert, u_first, u_npairs, pair_tok,
//   pair_expert, pair_w (f32 bits), then tok_pairs [max_m][topk + 1] (pair
//   index of each of a token's plan entries in ascending expert id: its
//   picks, then, for a layer whose shared expert is quantised, that expert as
//   id n_routed with weight 1; -1 = none).
struct PlanView {
  int32_t* base;
  int max_pairs, max_m, topk;
  __host__ __device__ int32_t* n_u() const { return base; }
  __host__ __device__ int32_t* n_pairs() const { return base + 1; }
  __host__ __device__ int32_t* u_expert() const { return base + 2; }
  __host__ __device__ int32_t* u_first() const { return base + 2 + max_pairs; }
  __host__ __device__ int32_t* u_npairs() const { return base + 2 + 2 * max_pairs; }
  __host__ __device__ int32_t* pair_tok() const { return base + 2 + 3 * max_pairs; }
  __host__ __device__ int32_t* pair_expert() const { return base + 2 + 4 * max_pairs; }
  __host__ __device__ float* pair_w() const { return reinterpret_cast<float*>(base + 2 + 5 * max_pairs); }
  __host__ __device__ int32_t* tok_pairs() const { return base + 2 + 6 * max_pairs; }
  __host__ __device__ int slots() const { return topk + 1; }   // tok_pairs entries per token
  static int words(int max_pairs, int max_m, int topk) { return 2 + 6 * max_pairs + max_m * (topk + 1); }
};

// The expert blocks as the kernels address them: routed expert e < n_routed
// at base + e * stride, each matrix at its offset inside; id n_routed is the
// layer's shared expert when its matrices are K-quant blocks (Q2_K gate/up,
// Q3_K down at sbase + the s*_off offsets), run on the same kernels as one
// more expert of every token [moe_v41.rs, struct MoeV41LayerWeights: the
// shared matrices as resident bf16 or the GGUF's Q2_K/Q3_K blocks on the
// routed experts' kernels].
struct XArena {
  const uint8_t* base;
  uint64_t stride, gate_off, up_off, down_off;
  const uint8_t* sbase;   // nullptr: the layer has no quantised shared expert
  uint64_t sgate_off, sup_off, sdown_off;
  int n_routed;
  // With an expert cache: the layer's row of the device slot table; routed
  // expert e's blocks then sit in slot slot_of[e] of the cache's pool (base,
  // stride). An absent expert (-1) reads slot 0, as the pages' selection
  // points it [device_route.rs, module doc]; the cache makes every pick
  // resident before the expert kernels run. nullptr: expert e is slot e.
  const int32_t* slot_of;
  __host__ __device__ bool shared(int e) const { return e >= n_routed; }
  __device__ int slot(int e) const { return slot_of ? max(slot_of[e], 0) : e; }
  __device__ const uint8_t* blocks(int e) const { return shared(e) ? sbase : base + (uint64_t)slot(e) * stride; }
  __host__ __device__ uint64_t goff(int e) const { return shared(e) ? sgate_off : gate_off; }
  __host__ __device__ uint64_t uoff(int e) const { return shared(e) ? sup_off : up_off; }
  __host__ __device__ uint64_t doff(int e) const { return shared(e) ? sdown_off : down_off; }
  __device__ const uint8_t* gate(int e) const { return blocks(e) + goff(e); }
  __device__ const uint8_t* up(int e) const { return blocks(e) + uoff(e); }
  __device__ const uint8_t* down(int e) const { return blocks(e) + doff(e); }
  __host__ __device__ int has_shared() const { return sbase ? 1 : 0; }
};
// The routed arena alone (shared_q NULL), or with the layer's quantised shared
// expert; slot_of: a slot-table row (the arena is then a cache's slot pool).
XArena arena_of(const moe_experts& ex, int n_routed, const moe_experts* shared_q, const int32_t* slot_of = nullptr);

// Control words (workspace region `ctl`, 256 bytes, zero between calls).
struct Ctl {
  uint32_t router_done;   // router workgroups of the running front launch that have finished
  uint32_t pad[63];
};
static_assert(sizeof(Ctl) == 256, "control region size");

// Device-side view of the workspace for one call.
struct Ws {
  int8_t* xq;
  uint16_t* xd;
  int32_t* xs;
  float* logits;
  float* scores;
  PlanView plan;
  float* g;
  float* u;
  float* h;
  int8_t* hq;
  uint16_t* hd;
  int32_t* hs;
  float* y;
  float* sg;
  float* su;
  uint16_t* sh;
  float* sd;
  float* yr;
  int32_t* status;
  Ctl* ctl;
  double* xd64;   // prefill: the q8_1 scales of x as float64 [max_m][dim/32]
  double* hd64;   // prefill: the q8_1 scales of h as float64 [pairs][inter/32]
};

bool layout_of(const moe_cfg& c, int max_m, moe_ws_layout* L);
Ws ws_view(void* ws, const moe_ws_layout& L, const moe_cfg& c, int max_m);

// Where a layer's result goes: out = the routed sum plus the shared expert
// (f32 and/or its bf16 rounding), and for a layer stack the residual stream
// next = bf16(f32(resid) + out). Every pointer may be NULL.
struct LayerOut {
  float* f32;
  uint16_t* bf16;
  const uint16_t* resid;
  uint16_t* next;
};

// ---- launchers (each returns hipError_t of the launch) ----
// front: status reset, q8_1 of x (and for m = 1 its LDS image), and when
// gate_w is given the router with its scores; when `sel` is given, the last
// router workgroup also selects every token's top-k, writes the headers and
// builds the plan; when w1/w3 are given, the shared expert's gate/up + SwiGLU.
struct FrontSelect {
  const float* bias;
  int32_t* header;
  int shq;   // 1: the plan also gets the layer's quantised shared expert (id n_routed) for every token
};
hipError_t launch_front(const uint16_t* x, int m, const uint16_t* gate_w, const FrontSelect* sel, const uint16_t* w1,
                        const uint16_t* w3, const moe_cfg& c, const Ws& w, float* logits_out, hipStream_t s);
hipError_t launch_quant_x(const uint16_t* x, int m, const moe_cfg& c, const Ws& w, hipStream_t s);
// slot_of (optional): a slot-table row; the header's plan words then hold the
// picks' slots (-1 = absent) and status bit MOE_STATUS_MISS flags an absent pick.
hipError_t launch_select(const float* bias, int m, const moe_cfg& c, const Ws& w, int32_t* header, hipStream_t s,
                         const int32_t* slot_of = nullptr);
// shq = 1: each token's plan also gets the layer's quantised shared expert.
hipError_t launch_plan(const int32_t* header, int m, const moe_cfg& c, const Ws& w, hipStream_t s, int shq = 0);
hipError_t launch_gateup(const XArena& ex, int m, const moe_cfg& c, const Ws& w, hipStream_t s);
// down: routed Q3_K rows, plus the shared expert's down rows when w2 is given.
hipError_t launch_down(const XArena& ex, int m, const moe_cfg& c, const Ws& w, const uint16_t* w2,
                       hipStream_t s);
hipError_t launch_combine(int m, const moe_cfg& c, const Ws& w, const float* sd, const LayerOut& o, hipStream_t s);
hipError_t launch_scores(const float* logits, int64_t n, float temp, float* out, int flags, hipStream_t s);
// single token: the gate/up rows of every pick + SwiGLU + q8_1 of h, with the
// plan selected here from the front launch's scores (`sel` given; the shared
// expert's gate/up rows run in the same launch when `layer` is given too) or
// from the caller's header (checked here); then the down rows of every pick +
// the shared expert's down rows + the combine.
hipError_t launch_gateup_m1(const XArena& ex, const FrontSelect* sel, const int32_t* hdr_in,
                            const uint16_t* x, const moe_layer* layer, const moe_cfg& c, const Ws& w, hipStream_t s);
hipError_t launch_down_m1(const XArena& ex, const moe_cfg& c, const Ws& w, const uint16_t* w2, const LayerOut& o,
                          hipStream_t s);
// The glibc score table registered for the current device when c.score_mode
// is MOE_SCORE_GLIBC (checked by check_cfg), else the empty table.
ScoreTable score_table_for(const moe_cfg& c);
// MOE_OK, or MOE_EINVAL when c asks for the glibc mode and the current device
// has no table registered (every entry point that computes scores).
int check_score_mode(const moe_cfg& c);
// The host's copy of the glibc table (built on first use).
ScoreTable host_score_table();

// ---- argument checks and the error message (moe_api.hip) ----
int fail(int code, const char* fmt, const char* a = "", long long b = 0);   // fmt takes a %s then a %lld
int hip_fail(hipError_t e, const char* where);
int check_cfg(const moe_cfg* c);
int check_m(const moe_cfg& c, int64_t m);
int check_ws(const moe_cfg& c, int m, void* ws, size_t ws_bytes, moe_ws_layout* L);
int check_experts(const moe_experts* ex);
int check_layer(const moe_layer* layer, bool need_experts = true);
bool a16(const void* p);
bool single_token_fits(const moe_cfg& c, int shq = 0);
bool shared_bf16(const moe_layer& layer);
// Routing of m tokens (q8_1 of x, router, scores, top-k, headers); slot_of as in launch_select.
hipError_t route_launches(const moe_cfg& c, const uint16_t* x, int m, const uint16_t* gate_w, const float* bias,
                          int32_t* header, const Ws& w, const int32_t* slot_of, hipStream_t s);
// The layer after its routing, from the device headers: routed experts out of `ar`, shared expert, combine.
int layer_launches_hdr(const moe_cfg& c, const moe_layer& layer, const XArena& ar, const uint16_t* x, int m,
                       const int32_t* header, const LayerOut& o, const Ws& w, int32_t* grp, hipStream_t s);

// Zero-fill of `bytes` bytes (a multiple of 16) with a kernel (no memset node).
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

// Timing hook (moe_time_next_launch): the event pair set for kernel `which`,
// taken (and cleared) by its next launch, which then goes through
// hipExtLaunchKernelGGL so that the events hold the dispatch's own start and
// end times.
bool take_timed(int which, hipEvent_t* begin, hipEvent_t* end);

#define MOE_LAUNCH(which, kern, grid, block, shm, stream, ...)                                          \
  do {                                                                                                \
    hipEvent_t moe_eb_, moe_ee_;                                                                      \
    if (take_timed(which, &moe_eb_, &moe_ee_))                                                        \
      hipExtLaunchKernelGGL(kern, grid, block, shm, stream, moe_eb_, moe_ee_, 0, __VA_ARGS__);        \
    else                                                                                              \
      hipLaunchKernelGGL(kern, grid, block, shm, stream, __VA_ARGS__);                                \
  } while (0)

}  // namespace moe
