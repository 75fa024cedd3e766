// Single-token layer (m = 1) in ONE launch.
//
// At m = 1 every part of the layer is a GEMV of a few tens of MB, so a launch
// per part pays its ramp-up and drain again and again (about 3 us each on
// MI355X) and the HBM pipe idles in between. Here the layer is one grid of
// work items; a workgroup takes the next ticket when it starts and runs that
// item, so items start in ticket order while the hardware keeps every CU
// busy with the next ones:
//
//   item kind   count (dim 4096, inter 2048)   reads                      waits for
//   Q           1                              x                          -
//   R router    n_routed/4  (4 rows each)      gate_w rows (bf16)         -
//   S shared    inter/4     (4 units each)     shared w1/w3 rows (bf16)   -
//   G gate/up   topk * inter/32                two 32-row Q2_K groups     the plan
//   D down      dim/RD      (RD rows each)     RD Q3_K rows of every      all G items (h),
//                                              pick + RD shared w2 rows   all S items (sh)
//
// The last R item to finish runs the top-k selection and publishes the plan
// [moe_v41.rs, fn route_from_logits; device_route.rs, module doc]. A D item
// issues its weight loads before it waits, so the down weights stream while
// the last gate/up items finish, and ends with the combine of its rows in
// plan order plus the shared expert [moe_v41.rs, fn shared_side].
//
// Deadlock freedom: items only wait for items with smaller tickets, and a
// ticket is taken only by a running workgroup, so the oldest unfinished item
// always runs (the argument of decoupled look-back scans). Every wait is
// bounded: when the bound runs out the workgroup records MOE_STATUS_TIMEOUT
// and carries on, so the grid always drains.
//
// The control words (ticket and done counters) live in the caller's
// workspace: they must be zero before the first call (moe_workspace_init),
// and the last workgroup to leave puts them back to zero.
//
// The arithmetic is that of the multi-token kernels (same dot products,
// epilogues and combine order), so the results are bit-identical to them.
#include <hip/hip_runtime.h>

#include "moe_front.h"
#include "moe_internal.h"
#include "moe_kquant.h"
#include "moe_math.h"
#include "moe_select.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kSlots = 3;   // gate/up tiles in flight per workgroup

struct L1Args {
  int mode;   // 0: route here (router, selection, shared expert); 1: the caller's header
  int dim, inter, n_routed, topk, norm;
  float temp, route_scale, L;
  const uint16_t* x;
  const uint16_t* gate_w;
  const float* bias;
  const uint16_t* w1;
  const uint16_t* w3;
  const uint16_t* w2;
  moe_experts ex;
  const int32_t* hdr_in;
  int32_t* hdr_out;
  float* out_f32;
  uint16_t* out_bf16;
  uint16_t* x_next;   // when set: bf16(x + out), the residual stream of a layer stack
  int i_r, i_s, i_g, i_d, n_items;   // first ticket of each item kind; n_items = end
  uint32_t spin_limit;
  Ctl* ctl;
};

struct M1Plan {
  int e[kMaxTopk];   // plan order (ascending id); -1 = none
  float w[kMaxTopk];
  int n_u;
};

// ---- inter-workgroup signalling (agent scope) -------------------------------
__device__ __forceinline__ void fence_release() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ void fence_acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

__device__ __forceinline__ uint32_t ld_acquire(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0 only: wait until *p >= target, at most `limit` polls.
__device__ bool wait_count(const uint32_t* p, uint32_t target, uint32_t limit, uint32_t* fault) {
  for (uint32_t it = 0; it < limit; ++it) {
    if (ld_acquire(p) >= target) return true;
    __builtin_amdgcn_s_sleep(8);
  }
  __hip_atomic_fetch_or(fault, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return false;
}

// Every thread makes its global writes visible at agent scope, then thread 0
// counts the item as done. Returns the previous count (thread 0 only).
__device__ uint32_t signal_done(uint32_t* counter) {
  fence_release();
  __syncthreads();
  uint32_t old = 0;
  if (threadIdx.x == 0) old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
  return old;
}

// ---- the plan ---------------------------------------------------------------
// Wave 0 of one workgroup: the plan from the top-k selection (mode 0) or
// from the caller's header (mode 1, checked), written to the header (mode
// 0), the plan tables and the status word.
template <int KPER>
__device__ void publish_plan(const L1Args& a, const Ws& w) {
  const int lane = threadIdx.x & 63;
  const int topk = a.topk;
  int pick = 0;
  float wv = 0.0f;
  bool nan_any = false, ok = true;
  if (a.mode == 0) {
    int picks[kMaxTopk];
    float wts[kMaxTopk];
    select_topk<KPER>(w.scores, a.bias, a.n_routed, topk, a.norm, a.route_scale, picks, wts, nan_any);
#pragma unroll
    for (int r = 0; r < kMaxTopk; ++r)
      if (r == lane) {
        pick = picks[r];
        wv = wts[r];
      }
  } else {
    const int li = min(lane, topk - 1);
    pick = a.hdr_in[1 + li];
    wv = __builtin_bit_cast(float, a.hdr_in[1 + topk + li]);
    bool bad = lane < topk && (pick < 0 || pick >= a.n_routed);
#pragma unroll
    for (int i = 0; i < kMaxTopk; ++i) {
      const int o = __builtin_amdgcn_readlane(pick, i);
      if (i < topk && lane < topk && i < lane && o == pick) bad = true;
    }
    ok = !__any(bad);
  }
  int rank = 0;
#pragma unroll
  for (int i = 0; i < kMaxTopk; ++i)
    if (i < topk) rank += (__builtin_amdgcn_readlane(pick, i) < pick) ? 1 : 0;
  PlanView plan = w.plan;
  if (a.mode == 0 && lane < topk) {
    a.hdr_out[1 + lane] = pick;
    a.hdr_out[1 + topk + lane] = (int32_t)__builtin_bit_cast(uint32_t, wv);
    a.hdr_out[1 + 2 * topk + rank] = pick;
  }
  if (lane < topk) {
    if (ok) {
      plan.u_expert()[rank] = pick;
      plan.u_first()[rank] = rank;
      plan.u_npairs()[rank] = 1;
      plan.pair_tok()[rank] = 0;
      plan.pair_expert()[rank] = pick;
      plan.pair_w()[rank] = wv;
      plan.tok_pairs()[rank] = rank;
    } else {
      plan.tok_pairs()[lane] = -1;
    }
  }
  if (lane == 0) {
    *plan.n_u() = ok ? topk : 0;
    *plan.n_pairs() = ok ? topk : 0;
    if (a.mode == 0) a.hdr_out[0] = nan_any ? MOE_STATUS_NAN_KEY : 0;
    w.status[0] = (nan_any ? MOE_STATUS_NAN_KEY : 0) | (ok ? 0 : MOE_STATUS_BAD_PICK);
  }
}

__device__ void publish_plan_any(const L1Args& a, const Ws& w) {
  if (a.n_routed <= 384) publish_plan<6>(a, w);
  else publish_plan<16>(a, w);
}

// The plan into this workgroup's LDS copy (after the plan_ready wait). An
// id outside [0, n_routed) (only after a timed-out wait) becomes "none", so
// no load ever leaves the expert arena.
__device__ void load_plan(const Ws& w, int topk, int n_routed, M1Plan& P) {
  const int t = threadIdx.x;
  const int n_u = min(max(*w.plan.n_u(), 0), topk);
  if (t < kMaxTopk) {
    const int e = t < n_u ? w.plan.u_expert()[t] : -1;
    const bool ok = e >= 0 && e < n_routed;
    P.e[t] = ok ? e : -1;
    P.w[t] = ok ? w.plan.pair_w()[t] : 0.0f;
  }
  if (t == 0) P.n_u = n_u;
}

// ---- q8_1 of x straight into the LDS activation layout -----------------------
// Thread c takes 16 consecutive values (half a q8_1 block; its partner c^1 is
// the neighbouring lane): the same d = amax/127 and code = roundf(x/d) as
// the global quantiser, so the codes are identical.
template <int NSB>
__device__ void build_xact(uint8_t* lds, const uint16_t* __restrict__ x, int dim) {
  using AL = ActLds<NSB>;
  for (int c = threadIdx.x; c < dim / 16; c += kThreads) {
    const uint4 v0 = *reinterpret_cast<const uint4*>(x + 16 * c);
    const uint4 v1 = *reinterpret_cast<const uint4*>(x + 16 * c + 8);
    const uint32_t wd[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    float v[16];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      v[j] = bf16_f32((uint16_t)(wd[j >> 1] >> (16 * (j & 1))));
      amax = fmaxf(amax, fabsf(v[j]));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    const float d = (float)((double)amax / 127.0);
    uint32_t packed[4] = {0, 0, 0, 0};
    int sum = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int q = amax == 0.0f ? 0 : q8_code(v[j], d);
      sum += q;
      packed[j >> 2] |= ((uint32_t)(q & 0xFF)) << (8 * (j & 3));
    }
    const int sb = c >> 4, k = c & 15;
    *reinterpret_cast<uint4*>(lds + sb * AL::kCodeStride + 16 * k) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    *reinterpret_cast<int*>(lds + AL::kQ + sb * AL::kQStride + 4 * k) = sum;
    if ((k & 1) == 0)
      *reinterpret_cast<uint16_t*>(lds + AL::kD + 16 * sb + 2 * (k >> 1)) = __builtin_bit_cast(uint16_t, (_Float16)d);
  }
}

// ---- geometry of the down items ----------------------------------------------
template <int NSBI>
struct DownGeom1 {
  static constexpr int kRows = NSBI >= 16 ? 64 / NSBI : 8;       // output rows per item
  static constexpr int kRowBytes = NSBI * kQ3KBytes;
  static constexpr int kChunks = kRows * kRowBytes / 16;          // per pick
  static constexpr int kKC = (kChunks + kThreads - 1) / kThreads;
  static constexpr int kRegion = kKC * kThreads * 16;             // LDS bytes per pick
  static constexpr int kShCh = kRows * NSBI * 32 / kThreads;      // 16-byte shared-w2 chunks per thread
  static constexpr int kShLanes = kThreads / kRows;               // threads per shared row
};

// ---- the kernel -------------------------------------------------------------
template <int NSBD, int NSBI>
__global__ __launch_bounds__(kThreads) void k_layer1(L1Args a, Ws w) {
  using G = GateUpGeom<NSBD>;
  using DG = DownGeom1<NSBI>;
  using AD = ActLds<NSBD>;
  using AI = ActLds<NSBI>;
  extern __shared__ __align__(16) uint8_t dyn[];
  __shared__ __align__(16) uint8_t xact[AD::kBytes];
  __shared__ M1Plan P;
  __shared__ float gu[2][32];
  __shared__ float ys[kMaxTopk][DG::kRows];
  __shared__ float sds[DG::kRows];
  __shared__ uint32_t s_ticket;
  __shared__ int s_sel;     // this workgroup finished the last router item
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  Ctl* ctl = a.ctl;

  if (tid == 0) s_ticket = __hip_atomic_fetch_add(&ctl->ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int item = (int)s_ticket;
  if (item < a.n_items) {   // (a workspace whose control words were not zeroed hands out tickets past the end)

    if (item < a.i_r) {
      // ---- Q: q8_1 of x into the workspace (and, with a caller's header, the plan)
      for (int blk = 0; blk < a.dim / 256; ++blk) front::quant_x_block(blk, a.x, w.xq, w.xd, w.xs);
      if (a.mode == 1) {
        if (wave == 0) publish_plan_any(a, w);
        fence_release();
        __syncthreads();
        if (tid == 0) __hip_atomic_store(&ctl->plan_ready, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else if (item < a.i_s) {
      // ---- R: four router rows and their scores; the last one selects
      front::router_rows(item - a.i_r, a.x, 1, a.dim, a.gate_w, a.n_routed, a.temp, w.logits, w.scores, nullptr);
      const uint32_t old = signal_done(&ctl->r_done);
      if (tid == 0) s_sel = old + 1 == (uint32_t)(a.i_s - a.i_r) ? 1 : 0;
      __syncthreads();
      if (s_sel) {
        fence_acquire();
        if (wave == 0) publish_plan_any(a, w);
        fence_release();
        __syncthreads();
        if (tid == 0) __hip_atomic_store(&ctl->plan_ready, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else if (item < a.i_g) {
      // ---- S: four shared-expert units (gate/up, SwiGLU, bf16 h)
      front::shared_gu_rows(item - a.i_s, a.x, 1, a.dim, a.inter, a.w1, a.w3, w.sg, w.su, w.sh, a.L);
      signal_done(&ctl->s_done);
    } else {
      // ---- G and D need the plan
      if (tid == 0) wait_count(&ctl->plan_ready, 1u, a.spin_limit, &ctl->fault);
      __syncthreads();
      fence_acquire();
      load_plan(w, a.topk, a.n_routed, P);
      __syncthreads();
      if (item < a.i_d) {
        // ---- G: a 32-row group of one pick's gate and up rows
        const int ngr = a.inter / 32;
        const int gi = item - a.i_g;
        const int slot = gi / ngr, grp = gi % ngr;
        build_xact<NSBD>(xact, a.x, a.dim);
        __syncthreads();   // also completes this wave's loads: from here on vmcnt counts only the tile DMA
        const int e = P.e[slot];
        if (e >= 0) {
          const int sb = tid % NSBD;
          Act A;
          load_act_lds<NSBD>(A, xact, sb);
          const uint8_t* ebase = (const uint8_t*)a.ex.base + (uint64_t)e * a.ex.stride;
          auto tile_src = [&](int c) -> const uint8_t* {
            const uint64_t off = (c & 1) ? a.ex.up_off : a.ex.gate_off;
            return ebase + off + (uint64_t)(32 * grp + 16 * (c >> 1)) * G::kRowBytes;
          };
#pragma unroll
          for (int c = 0; c < kSlots; ++c) dma_tile<G::kKC>(tile_src(c), dyn + c * G::kSlotBytes, G::kTileChunks);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int issued = (c + kSlots < 4 ? c + kSlots : 4);
            const int after = issued - c - 1;
            if (after == 2) wait_vmcnt<2 * G::kKC>();
            else if (after == 1) wait_vmcnt<1 * G::kKC>();
            else wait_vmcnt<0>();
            block_sync_lds();
            const uint8_t* sl = dyn + (c % kSlots) * G::kSlotBytes;
            const int mat = c & 1, r0 = 16 * (c >> 1);
#pragma unroll
            for (int it = 0; it < G::kIters; ++it) {
              const int i = it * kThreads + tid;
              const bool act = i < G::kItems;
              const int row = i / NSBD;
              double part = act ? dot_q2k(sl + row * G::kRowBytes + kQ2KBytes * sb, A) : 0.0;
              part = seg_sum_f64<NSBD>(part);
              if (act && sb == 0) gu[mat][r0 + row] = (float)part;
            }
            if (c + kSlots < 4) {
              wait_lgkm0();
              block_sync_lds();
              dma_tile<G::kKC>(tile_src(c + kSlots), dyn + (c % kSlots) * G::kSlotBytes, G::kTileChunks);
            }
          }
          __syncthreads();
          if (wave == 0) {   // SwiGLU + q8_1 of the 32 h values (one q8_1 block)
            const int r = lane & 31;
            const float gv = gu[0][r], uv = gu[1][r];
            const float hv = swiglu(gv, uv, a.L);
            float am = fabsf(hv);
            for (int s = 16; s >= 1; s >>= 1) am = fmaxf(am, __shfl_xor(am, s));
            const float d = (float)((double)am / 127.0);
            const int q = am == 0.0f ? 0 : q8_code(hv, d);
            int sum = q;
            for (int s = 8; s >= 1; s >>= 1) sum += __shfl_xor(sum, s);
            if (lane < 32) {
              const int64_t row = (int64_t)slot * a.inter + 32 * grp + r;
              w.g[row] = gv;
              w.u[row] = uv;
              w.h[row] = hv;
              w.hq[row] = (int8_t)q;
              if (r == 0) w.hd[(int64_t)slot * (a.inter / 32) + grp] = __builtin_bit_cast(uint16_t, (_Float16)d);
              if ((r & 15) == 0) w.hs[(int64_t)slot * (a.inter / 16) + 2 * grp + (r >> 4)] = sum;
            }
          }
        }
        signal_done(&ctl->g_done);
      } else {
        // ---- D: RD output rows: every pick's Q3_K down rows, the shared
        // expert's down rows, and the combine
        const int row0 = (item - a.i_d) * DG::kRows;
        const int topk = a.topk, n_u = P.n_u;
        // 1. the picks' rows, HBM -> LDS (no dependency on h)
        for (int i = 0; i < topk; ++i) {
          const int e = P.e[i];
          if (e >= 0)
            dma_tile<DG::kKC>((const uint8_t*)a.ex.base + (uint64_t)e * a.ex.stride + a.ex.down_off +
                                  (uint64_t)row0 * DG::kRowBytes,
                              dyn + i * DG::kRegion, DG::kChunks);
        }
        // 2. the shared expert's rows into registers
        const bool shared = a.mode == 0;
        const int srow = tid / DG::kShLanes, slane = tid % DG::kShLanes;
        uint4 wsh[DG::kShCh];
        if (shared) {
#pragma unroll
          for (int c = 0; c < DG::kShCh; ++c)
            wsh[c] = load_nt16(a.w2 + (int64_t)(row0 + srow) * a.inter + 8 * (slane + DG::kShLanes * c));
        }
        // 3. h of every pick (all G items) and sh (all S items)
        if (tid == 0) {
          wait_count(&ctl->g_done, (uint32_t)(a.i_d - a.i_g), a.spin_limit, &ctl->fault);
          if (shared) wait_count(&ctl->s_done, (uint32_t)(a.i_g - a.i_s), a.spin_limit, &ctl->fault);
        }
        __syncthreads();
        fence_acquire();
        uint8_t* hact = dyn + topk * DG::kRegion;
        for (int i = 0; i < topk; ++i)
          if (P.e[i] >= 0)
            for (int p = tid; p < AI::kChunks; p += kThreads)
              act_piece_to_lds<NSBI>(hact + i * AI::kBytes, w.hq + (int64_t)i * a.inter,
                                     w.hs + (int64_t)i * (a.inter / 16), w.hd + (int64_t)i * (a.inter / 32), p);
        float sp = 0.0f;
        if (shared) {
#pragma unroll
          for (int c = 0; c < DG::kShCh; ++c) {
            const uint4 hv4 = *reinterpret_cast<const uint4*>(w.sh + 8 * (slane + DG::kShLanes * c));
            const uint32_t hh[4] = {hv4.x, hv4.y, hv4.z, hv4.w};
            const uint32_t ww[4] = {wsh[c].x, wsh[c].y, wsh[c].z, wsh[c].w};
#pragma unroll
            for (int j = 0; j < 8; ++j)
              sp = __builtin_fmaf(bf16_f32((uint16_t)(ww[j >> 1] >> (16 * (j & 1)))),
                                  bf16_f32((uint16_t)(hh[j >> 1] >> (16 * (j & 1)))), sp);
          }
          for (int s = DG::kShLanes / 2; s >= 1; s >>= 1) sp += __shfl_xor(sp, s);
        }
        __syncthreads();   // the rows and the activations are in LDS
        if (shared && slane == 0) {
          sds[srow] = sp;
          w.sd[row0 + srow] = sp;
        }
        const int units = topk * DG::kRows * NSBI;
        for (int u0 = 0; u0 < units; u0 += kThreads) {
          const int u = u0 + tid;
          const bool act = u < units;
          const int pi = act ? u / (DG::kRows * NSBI) : 0;
          const int row = (u / NSBI) % DG::kRows, sb = u % NSBI;
          const bool live = act && P.e[pi] >= 0;
          double part = 0.0;
          if (live) {
            Act A;
            load_act_lds<NSBI>(A, hact + pi * AI::kBytes, sb);
            part = dot_q3k(dyn + pi * DG::kRegion + row * DG::kRowBytes + kQ3KBytes * sb, A);
          }
          part = seg_sum_f64<NSBI>(part);
          if (act && sb == 0) {
            ys[pi][row] = live ? (float)part : 0.0f;
            if (live) w.y[(int64_t)pi * a.dim + row0 + row] = (float)part;
          }
        }
        __syncthreads();
        if (tid < DG::kRows) {
          const int r = tid;
          float acc = 0.0f;
          for (int i = 0; i < topk; ++i)
            if (i < n_u) acc = fadd(acc, fmul(P.w[i], ys[i][r]));
          if (shared) acc = fadd(acc, sds[r]);
          if (a.out_f32) a.out_f32[row0 + r] = acc;
          if (a.out_bf16) a.out_bf16[row0 + r] = bf16_rne(acc);
          if (a.x_next) a.x_next[row0 + r] = bf16_rne(fadd(bf16_f32(a.x[row0 + r]), acc));
        }
      }
    }
  }

  // The last workgroup to leave reports a timed-out wait and puts the
  // control words back to zero for the next call.
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(&ctl->exited, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1 == gridDim.x) {
      if (__hip_atomic_load(&ctl->fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
        __hip_atomic_fetch_or((uint32_t*)&w.status[0], (uint32_t)MOE_STATUS_TIMEOUT, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
      uint32_t* words = reinterpret_cast<uint32_t*>(ctl);
      for (int i = 0; i < (int)(sizeof(Ctl) / 4); ++i)
        __hip_atomic_store(words + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      fence_release();
    }
  }
}

template <int NSBD, int NSBI>
size_t dyn_lds_bytes(int topk) {
  const size_t g = (size_t)kSlots * GateUpGeom<NSBD>::kSlotBytes;
  const size_t d = (size_t)topk * (DownGeom1<NSBI>::kRegion + ActLds<NSBI>::kBytes);
  return g > d ? g : d;
}

template <int NSBD, int NSBI>
hipError_t launch_t(const L1Args& a, const Ws& w, hipStream_t s) {
  auto kern = k_layer1<NSBD, NSBI>;
  const size_t shm = dyn_lds_bytes<NSBD, NSBI>(a.topk);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static bool attr_of[64] = {false};   // per device: the LDS attribute, set once for the largest topk
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!attr_of[dev]) {
    if ((e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)dyn_lds_bytes<NSBD, NSBI>(kMaxTopk))) != hipSuccess)
      return e;
    attr_of[dev] = true;
  }
  MOE_LAUNCH(MOE_K_LAYER, kern, dim3(a.n_items), dim3(kThreads), shm, s, a, w);
  return hipGetLastError();
}

}  // namespace

bool layer1_supported(const moe_cfg& c) {
  const int nd = c.dim / 256, ni = c.inter / 256;
  return nd >= 1 && nd <= 16 && ni >= 1 && ni <= nd && (nd & (nd - 1)) == 0 && (ni & (ni - 1)) == 0;
}

hipError_t launch_layer1(int mode, const moe_cfg& c, const uint16_t* x, const moe_layer* layer,
                         const moe_experts& ex, const int32_t* hdr_in, int32_t* hdr_out, float* out_f32,
                         uint16_t* out_bf16, uint16_t* x_next, const Ws& w, hipStream_t s) {
  L1Args a;
  a.mode = mode;
  a.dim = c.dim;
  a.inter = c.inter;
  a.n_routed = c.n_routed;
  a.topk = c.topk;
  a.norm = c.norm_topk_prob;
  a.temp = c.gate_temp;
  a.route_scale = c.route_scale;
  a.L = c.swiglu_limit;
  a.x = x;
  a.gate_w = layer ? layer->gate_w : nullptr;
  a.bias = layer ? layer->bias : nullptr;
  a.w1 = layer ? layer->sh_w1 : nullptr;
  a.w3 = layer ? layer->sh_w3 : nullptr;
  a.w2 = layer ? layer->sh_w2 : nullptr;
  a.ex = ex;
  a.hdr_in = hdr_in;
  a.hdr_out = hdr_out;
  a.out_f32 = out_f32;
  a.out_bf16 = out_bf16;
  a.x_next = x_next;
  const int n_r = mode == 0 ? (c.n_routed + 3) / 4 : 0;
  const int n_s = mode == 0 ? c.inter / 4 : 0;
  const int n_g = c.topk * (c.inter / 32);
  a.i_r = 1;
  a.i_s = a.i_r + n_r;
  a.i_g = a.i_s + n_s;
  a.i_d = a.i_g + n_g;
  const int nsbi = c.inter / 256;
  const int rows = nsbi >= 16 ? 64 / nsbi : 8;
  a.n_items = a.i_d + c.dim / rows;
  a.spin_limit = spin_limit();
  a.ctl = w.ctl;
  const int nd = c.dim / 256, ni = c.inter / 256;
#define MOE_L1(D, I) \
  if (nd == D && ni == I) return launch_t<D, I>(a, w, s);
  MOE_L1(1, 1)
  MOE_L1(2, 1)
  MOE_L1(2, 2)
  MOE_L1(4, 1)
  MOE_L1(4, 2)
  MOE_L1(4, 4)
  MOE_L1(8, 1)
  MOE_L1(8, 2)
  MOE_L1(8, 4)
  MOE_L1(8, 8)
  MOE_L1(16, 1)
  MOE_L1(16, 2)
  MOE_L1(16, 4)
  MOE_L1(16, 8)
  MOE_L1(16, 16)
#undef MOE_L1
  return hipErrorInvalidValue;
}

}  // namespace moe
