// Single-token decode (m = 1), after the front launch (router + q8_1 of x):
//  * k_gateup_m1: the first workgroups compute the shared expert's gate/up
//    rows (16 hidden units each, bf16 rows streamed through registers); they
//    need no plan, so the HBM pipe is busy from the start. Every other
//    workgroup first derives the token's plan itself (the top-k selection
//    from the scores, or the caller's header) while its other waves stage the
//    q8_1 activation in LDS, then runs one 32-row group of one picked
//    expert's Q2_K gate/up rows + SwiGLU + q8_1 of h. The first of them also
//    writes the header and the plan tables.
//  * k_down_m1: one workgroup per 16 output rows: each picked expert's rows
//    are split over waves of 64 (row, super-block) items; a wave streams its
//    rows' Q3_K blocks into LDS and dots them with the expert's q8_1(h); four
//    more waves compute the shared expert's down rows; then the combine in
//    plan order adds them up [moe_v41.rs, Kernels: accumulate, finish; fn
//    shared_side].
// The arithmetic is that of the general kernels (same dot-product and
// combine order), so the results are bit-identical to them.
#include <hip/hip_runtime.h>

#include "moe_front.h"
#include "moe_internal.h"
#include "moe_kquant.h"
#include "moe_math.h"
#include "moe_select.h"
#include "moe_wave.h"

namespace moe {
namespace {

struct M1Plan {
  int e[kMaxTopk];     // plan order (ascending id; a quantised shared expert last); -1 = dropped
  float w[kMaxTopk];
  int n_u;
};

// Wave 0 fills the block's plan (LDS) from the scores (mode 0) or from the
// caller's header (mode 1, checked: ids in range, no repeats); the `writer`
// workgroup also writes the header (mode 0), the plan tables and the status.
// shq = 1: the layer's quantised shared expert (id n_routed, weight 1) is the
// plan's last entry.
template <int KPER>
__device__ void plan_m1(int mode, bool writer, const float* __restrict__ scores, const float* __restrict__ bias,
                        const int32_t* __restrict__ header_in, int n_routed, int topk, int norm, float route_scale,
                        int32_t* __restrict__ header_out, PlanView plan, int32_t* __restrict__ status, M1Plan& P,
                        int shq) {
  const int lane = threadIdx.x & 63;
  int pick = 0;
  float wv = 0.0f;
  bool nan_any = false, ok = true;
  if (mode == 0) {
    int picks[kMaxTopk];
    select_topk<KPER>(scores, bias, n_routed, topk, norm, route_scale, picks, wv, nan_any);
#pragma unroll
    for (int r = 0; r < kMaxTopk; ++r)
      if (r == lane) pick = picks[r];
  } else {
    const int li = min(lane, topk - 1);
    pick = header_in[1 + li];
    wv = __builtin_bit_cast(float, header_in[1 + topk + li]);
    bool bad = lane < topk && (pick < 0 || pick >= n_routed);
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
  if (lane < kMaxTopk) P.e[lane] = -1;        // a rejected header leaves every slot empty
  if (lane < topk && ok) {
    P.e[rank] = pick;
    P.w[rank] = wv;
  }
  if (lane == topk && shq && ok) {
    P.e[topk] = n_routed;
    P.w[topk] = 1.0f;
  }
  if (lane == 0) P.n_u = ok ? topk + shq : 0;
  if (writer) {
    if (mode == 0 && lane < topk) {
      header_out[1 + lane] = pick;
      header_out[1 + topk + lane] = (int32_t)__builtin_bit_cast(uint32_t, wv);
      header_out[1 + 2 * topk + rank] = pick;
    }
    if (lane < topk || (lane == topk && shq)) {
      const int slot = lane < topk ? rank : topk;
      const int ex_id = lane < topk ? pick : n_routed;
      if (ok) {
        plan.u_expert()[slot] = ex_id;
        plan.u_first()[slot] = slot;
        plan.u_npairs()[slot] = 1;
        plan.pair_tok()[slot] = 0;
        plan.pair_expert()[slot] = ex_id;
        plan.pair_w()[slot] = lane < topk ? wv : 1.0f;
        plan.tok_pairs()[slot] = slot;
      } else {
        plan.tok_pairs()[lane] = -1;
      }
    } else if (lane == topk) {
      plan.tok_pairs()[topk] = -1;   // no shared entry
    }
    if (lane == 0) {
      *plan.n_u() = ok ? topk + shq : 0;
      *plan.n_pairs() = ok ? topk + shq : 0;
      if (mode == 0) header_out[0] = nan_any ? MOE_STATUS_NAN_KEY : 0;
      const int st = (nan_any ? MOE_STATUS_NAN_KEY : 0) | (ok ? 0 : MOE_STATUS_BAD_PICK);
      if (st) atomicOr(status, st);
    }
  }
}

struct GateUp1Args {
  int mode;                 // 0: select from the scores; 1: the caller's header
  int shared_blocks;        // leading workgroups that only run shared-expert units (mode 0 with the layer)
  int shared_units;         // hidden units of the bf16 shared expert done here (0: none)
  XArena ex;                // the routed experts, and a quantised shared expert as id n_routed
  int slots;                // plan entries with a gate/up row group each: topk, + 1 for a quantised shared expert
  const float* bias;
  const int32_t* hdr_in;
  int32_t* hdr_out;
  int n_routed, topk, norm;
  float route_scale;
  int dim, inter;
  float L;
  const uint16_t* x;
  const uint16_t* w1;
  const uint16_t* w3;
};

// Shared-expert units per workgroup: a routed workgroup's waves 1..3 take one
// each while wave 0 selects (that wait would otherwise leave them idle);
// the leading shared-only workgroups take the rest, seven each (two per wave,
// one after the other). With 384 routed and 128 shared-only workgroups at
// dim 4096 every workgroup reads about the same number of bytes.
constexpr int kUnitsRouted = 3;
constexpr int kUnitsShared = 7;

// ---------------------------------------------------------------------------
template <int NSB, int SLOTS, int KPER>
__global__ __launch_bounds__(256) void k_gateup_m1(GateUp1Args a, Ws w) {
  using G = GateUpGeom<NSB>;
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ float gu[2][32];
  __shared__ float sgu[2][kUnitsShared];
  __shared__ M1Plan P;
  __shared__ __align__(16) uint8_t act_lds[ActLds<NSB>::kBytes];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool shared_only = (int)blockIdx.x < a.shared_blocks;
  const int blk = blockIdx.x - a.shared_blocks;
  const int routed_blocks = gridDim.x - a.shared_blocks;
  // first shared unit of this workgroup and how many
  const int u0 = shared_only ? kUnitsRouted * routed_blocks + kUnitsShared * (int)blockIdx.x : kUnitsRouted * blk;
  const int nu = max(0, min(shared_only ? kUnitsShared : kUnitsRouted, a.shared_units - u0));
  if (shared_only) {
    // wave k takes units k and k + 4, both units' loads in flight together
    static_assert(kUnitsShared <= 8, "two units per wave");
    front::SharedUnitLoads L0, L1;
    const bool has0 = wave < nu, has1 = wave + 4 < nu;
    if (has0) front::shared_gu_issue(u0 + wave, a.x, a.dim, a.w1, a.w3, L0);
    if (has1) front::shared_gu_issue(u0 + wave + 4, a.x, a.dim, a.w1, a.w3, L1);
    if (has0) {
      float g, u;
      front::shared_gu_sum(L0, a.dim, g, u);
      if (lane == 0) {
        sgu[0][wave] = g;
        sgu[1][wave] = u;
      }
    }
    if (has1) {
      float g, u;
      front::shared_gu_sum(L1, a.dim, g, u);
      if (lane == 0) {
        sgu[0][wave + 4] = g;
        sgu[1][wave + 4] = u;
      }
    }
    __syncthreads();
  } else {
    const int ngr = a.inter / 32;
    const int slot = blk / ngr, grp = blk % ngr;
    const int sb = threadIdx.x % NSB;
    if (wave == 0) {
      plan_m1<KPER>(a.mode, blk == 0, w.scores, a.bias, a.hdr_in, a.n_routed, a.topk, a.norm, a.route_scale,
                    a.hdr_out, w.plan, w.status, P, a.slots - a.topk);
    } else {   // meanwhile the other waves stage the token's q8_1 activation and run a shared unit each;
               // the unit's loads and the activation's are in flight together
      const bool unit = wave - 1 < nu;
      front::SharedUnitLoads SL;
      if (unit) front::shared_gu_issue(u0 + wave - 1, a.x, a.dim, a.w1, a.w3, SL);
      constexpr int kAP = (ActLds<NSB>::kChunks + 191) / 192;
      u32x4 piece[kAP];
#pragma unroll
      for (int k = 0; k < kAP; ++k) {
        const int i = min((int)threadIdx.x - 64 + 192 * k, ActLds<NSB>::kChunks - 1);
        piece[k] = *reinterpret_cast<const u32x4*>(act_piece_src<NSB>(w.xq, w.xs, w.xd, i));
      }
#pragma unroll
      for (int k = 0; k < kAP; ++k) {
        const int i = (int)threadIdx.x - 64 + 192 * k;
        if (i < ActLds<NSB>::kChunks) *reinterpret_cast<u32x4*>(act_piece_dst<NSB>(act_lds, i)) = piece[k];
      }
      if (unit) {
        float g, u;
        front::shared_gu_sum(SL, a.dim, g, u);
        if (lane == 0) {
          sgu[0][wave - 1] = g;
          sgu[1][wave - 1] = u;
        }
      }
    }
    __syncthreads();   // also completes every wave's outstanding loads: the tile DMA below is all vmcnt sees
    const int e = P.e[slot];
    if (e >= 0) {
      Act A;
      load_act_lds<NSB>(A, act_lds, sb);
      const uint8_t* gbase = a.ex.gate(e);
      const uint8_t* ubase = a.ex.up(e);
      auto tile_src = [&](int c) -> const uint8_t* {
        return ((c & 1) ? ubase : gbase) + (uint64_t)(32 * grp + 16 * (c >> 1)) * G::kRowBytes;
      };
#pragma unroll
      for (int c = 0; c < SLOTS && c < 4; ++c)
        dma_tile<G::kKC>(tile_src(c), lds + c * G::kSlotBytes, G::kTileChunks);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int issued = (c + SLOTS < 4 ? c + SLOTS : 4);
        const int after = issued - c - 1;
        if (after == 3) wait_vmcnt<3 * G::kKC>();
        else if (after == 2) wait_vmcnt<2 * G::kKC>();
        else if (after == 1) wait_vmcnt<1 * G::kKC>();
        else wait_vmcnt<0>();
        block_sync_lds();
        const uint8_t* sl = lds + (c % SLOTS) * G::kSlotBytes;
        const int mat = c & 1, r0 = 16 * (c >> 1);
#pragma unroll
        for (int it = 0; it < G::kIters; ++it) {
          const int i = it * 256 + threadIdx.x;
          const bool act = i < G::kItems;
          const int row = i / NSB;
          double part = act ? dot_q2k(sl + row * G::kRowBytes + kQ2KBytes * sb, A) : 0.0;
          part = seg_sum_f64<NSB>(part);
          if (act && sb == 0) gu[mat][r0 + row] = (float)part;
        }
        if (c + SLOTS < 4) {
          wait_lgkm0();
          block_sync_lds();
          dma_tile<G::kKC>(tile_src(c + SLOTS), lds + (c % SLOTS) * G::kSlotBytes, G::kTileChunks);
        }
      }
      __syncthreads();
    }
  }
  // One SwiGLU site for every pair the workgroup made (the function is
  // large): lanes 0..31 the routed rows (if any), lanes 32.. (or 0.. in a
  // shared-only workgroup) the shared units.
  if (wave == 0) {
    const int ebl = shared_only ? -1 : P.e[blk / (a.inter / 32)];
    const int k = shared_only ? lane : lane - 32;
    const bool is_shared = k >= 0 && k < nu;
    const bool is_routed = ebl >= 0 && lane < 32;
    const float gv = is_shared ? sgu[0][k] : (is_routed ? gu[0][lane] : 0.0f);
    const float uv = is_shared ? sgu[1][k] : (is_routed ? gu[1][lane] : 0.0f);
    const float hv = swiglu(gv, uv, a.L);
    if (is_shared) {
      w.sg[u0 + k] = gv;
      w.su[u0 + k] = uv;
      w.sh[u0 + k] = bf16_rne(hv);
    }
    if (!shared_only && ebl >= 0) {   // q8_1 of the 32 h values (one block), lanes 0..31
      const int slot = blk / (a.inter / 32), grp = blk % (a.inter / 32);
      const int r = lane & 31;
      const float am = max32(fabsf(hv));
      const float d = (float)((double)am / 127.0);
      const int q = am == 0.0f ? 0 : q8_code(hv, d);
      const int sum = sum16(q);
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
}

// ---------------------------------------------------------------------------
// Per-wave DMA of `nchunks` 16-byte chunks (lanes past the end re-read the
// last chunk into the padding after it).
template <int NCH>
__device__ __forceinline__ void dma_wave(const uint8_t* g, uint8_t* dst) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 0; k < (NCH + 63) / 64; ++k) {
    const int i = 64 * k + lane;
    const int src = i < NCH ? i : NCH - 1;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(g + 16 * src),
                                     (__attribute__((address_space(3))) void*)(dst + 16 * 64 * k), 16, 0,
                                     kWeightStream);
  }
}

// A routed wave takes kRows rows of one pick (64 (row, super-block) items,
// one per lane; all 16 of the block's rows when they make at most 64 items).
template <int NSB>
struct DownM1Geom {
  static constexpr int kRows = 16 * NSB > 64 ? 64 / NSB : 16;   // rows of one pick per routed wave
  static constexpr int kParts = 16 / kRows;                     // routed waves per pick
  static constexpr int kRowBytes = NSB * kQ3KBytes;
  static constexpr int kChunks = kRows * kRowBytes / 16;
  static constexpr int kWaveBytes = ((kChunks + 63) / 64) * 1024;
  static constexpr int kItems = kRows * NSB;                    // per routed wave, <= 64
};

constexpr int kDownRows = 16;
constexpr int kSharedDownWaves = 4;   // bf16 shared expert: kDownRows / 4 rows per wave
constexpr int kMaxDownWaves = 16;

// The leading scalar arguments are what the first loads need (the plan's
// words, and the routed arena's base, stride and down offset; pbase = nullptr
// when the arena is a cache's slot pool): the build has the hardware preload
// them into SGPRs at wave launch (-amdgpu-kernarg-preload-count), so the plan
// and row loads do not wait for a load of the argument block first.
// slots: the plan entries (the picks, and a quantised shared expert as the
// last, weight 1), each taken by kParts routed waves; SHARED: four more waves
// for the bf16 shared expert's rows. Waves w and w + 4 share a SIMD, so with
// six picks at two waves each and the four shared waves every SIMD holds three
// routed waves and one shared wave; a routed wave's latency is one item.
template <int NSB, bool SHARED>
__global__ __launch_bounds__(1024) void k_down_m1(const int32_t* __restrict__ pplan, const uint8_t* __restrict__ pbase,
                                                  uint64_t pstride, uint64_t pdoff, int pnr, XArena ex, Ws w, int dim,
                                                  int inter, int slots, const uint16_t* __restrict__ w2, LayerOut o) {
  using G = DownM1Geom<NSB>;
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ __align__(16) uint8_t act_lds[kMaxDownWaves][ActLds<NSB>::kBytes];
  __shared__ float ys[kMaxTopk][kDownRows];
  __shared__ float sds[kDownRows];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row0 = blockIdx.x * kDownRows;
  const int n_u = pplan[0];
  const int nrw = slots * G::kParts;
  // The combine's other inputs (the plan's weights, the residual rows) are
  // loaded first: they arrive with the weight streams instead of costing a
  // round trip after the last dot product.
  float pw[kMaxTopk];
  uint16_t res = 0;
  if (threadIdx.x < kDownRows) {
#pragma unroll
    for (int i = 0; i < kMaxTopk; ++i) pw[i] = i < slots ? w.plan.pair_w()[i] : 0.0f;
    if (o.next) res = o.resid[row0 + threadIdx.x];
  }
  if (wave < nrw) {
    const int pk = wave % slots, r0 = G::kRows * (wave / slots);
    const int e_slot = pplan[2 + pk];   // (loaded together with n_u: no dependent round trip)
    const int e = pk < n_u ? e_slot : -1;
    if (e >= 0) {
      const int sb = lane % NSB;
      uint8_t* mine = lds + wave * G::kWaveBytes;
      // the rows, then this expert's q8_1(h) into registers: every load is in
      // flight at once, and one wait covers them all
      const uint8_t* dsrc = (pbase && e < pnr) ? pbase + (uint64_t)e * pstride + pdoff : ex.down(e);
      dma_wave<G::kChunks>(dsrc + (uint64_t)(row0 + r0) * G::kRowBytes, mine);
      constexpr int kAP = (ActLds<NSB>::kChunks + 63) / 64;
      u32x4 piece[kAP];
#pragma unroll
      for (int k = 0; k < kAP; ++k) {
        const int i = min(lane + 64 * k, ActLds<NSB>::kChunks - 1);
        piece[k] = *reinterpret_cast<const u32x4*>(act_piece_src<NSB>(
            w.hq + (int64_t)pk * inter, w.hs + (int64_t)pk * (inter / 16), w.hd + (int64_t)pk * (inter / 32), i));
      }
      uint8_t* al = act_lds[wave];
      wait_vmcnt<0>();
      asm volatile("" ::: "memory");
#pragma unroll
      for (int k = 0; k < kAP; ++k)
        if (lane + 64 * k < ActLds<NSB>::kChunks)
          *reinterpret_cast<u32x4*>(act_piece_dst<NSB>(al, lane + 64 * k)) = piece[k];
      Act A;
      load_act_lds<NSB>(A, al, sb);
      const bool act = lane < G::kItems;
      const int row = lane / NSB;
      double part = act ? dot_q3k(mine + row * G::kRowBytes + kQ3KBytes * sb, A) : 0.0;
      part = seg_sum_f64<NSB>(part);
      if (act && sb == 0) {
        ys[pk][r0 + row] = (float)part;
        w.y[(int64_t)pk * dim + row0 + r0 + row] = (float)part;
      }
    } else if (lane < G::kRows) {
      ys[pk][r0 + lane] = 0.0f;
    }
  } else if (SHARED && wave < nrw + kSharedDownWaves) {
    // shared expert down rows: a quarter of the block's rows per wave, f32
    constexpr int kR = kDownRows / kSharedDownWaves;
    constexpr int kCh = NSB >= 2 ? NSB / 2 : 1;   // 16-byte chunks of a row per lane (inter = 256*NSB)
    const int rbase = row0 + kR * (wave - nrw);
    float p[kR];
#pragma unroll
    for (int r = 0; r < kR; ++r) p[r] = 0.0f;
    uint4 wv[kR][kCh];
    uint4 hvv[kCh];
#pragma unroll
    for (int c = 0; c < kCh; ++c) {        // every load issued before any is used
      const int k = 8 * lane + 512 * c;
      const bool in = k < inter;
      hvv[c] = in ? *reinterpret_cast<const uint4*>(w.sh + k) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < kR; ++r) wv[r][c] = in ? load_nt16(w2 + (int64_t)(rbase + r) * inter + k) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < kCh; ++c)
#pragma unroll
      for (int r = 0; r < kR; ++r) p[r] = dot8_bf16(wv[r][c], hvv[c], p[r]);
#pragma unroll
    for (int r = 0; r < kR; ++r) p[r] = wave_sum_xor(p[r]);
    if (lane < kR) {
      float v = 0.0f;
#pragma unroll
      for (int r = 0; r < kR; ++r)
        if (r == lane) v = p[r];
      sds[kR * (wave - nrw) + lane] = v;
      w.sd[rbase + lane] = v;
    }
  }
  __syncthreads();
  if (threadIdx.x < kDownRows) {
    const int r = threadIdx.x;
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxTopk; ++i)
      if (i < slots && i < n_u) acc = fadd(acc, fmul(pw[i], ys[i][r]));   // a quantised shared expert last, weight 1
    if (SHARED) acc = fadd(acc, sds[r]);
    if (o.f32) o.f32[row0 + r] = acc;
    if (o.bf16) o.bf16[row0 + r] = bf16_rne(acc);
    if (o.next) o.next[row0 + r] = bf16_rne(fadd(bf16_f32(res), acc));
  }
}

template <int NSB>
hipError_t launch_gateup_m1_t(const GateUp1Args& a, const moe_cfg& c, const Ws& w, hipStream_t s) {
  using G = GateUpGeom<NSB>;
  constexpr int kSlots = 3;
  const size_t shm = (size_t)kSlots * G::kSlotBytes;
  auto kern6 = k_gateup_m1<NSB, kSlots, 6>;
  auto kern16 = k_gateup_m1<NSB, kSlots, 16>;
  const bool small = c.n_routed <= 384;
  auto kern = small ? kern6 : kern16;
  static bool attr_set[2] = {false, false};
  const int ai = small ? 0 : 1;
  if (!attr_set[ai]) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
    attr_set[ai] = true;
  }
  MOE_LAUNCH(MOE_K_GATEUP, kern, dim3(a.shared_blocks + a.slots * (c.inter / 32)), dim3(256), shm, s, a, w);
  return hipGetLastError();
}

template <int NSB>
hipError_t launch_down_m1_t(const XArena& ex, const moe_cfg& c, const Ws& w, const uint16_t* w2, const LayerOut& o,
                            hipStream_t s) {
  using G = DownM1Geom<NSB>;
  const int slots = c.topk + ex.has_shared();
  const size_t shm = (size_t)slots * G::kParts * G::kWaveBytes;
  const int waves = slots * G::kParts + (w2 ? kSharedDownWaves : 0);
  if (waves > kMaxDownWaves) return hipErrorInvalidValue;   // (shapes the single-token path does not take)
  const int threads = 64 * waves;
  auto kern = w2 ? k_down_m1<NSB, true> : k_down_m1<NSB, false>;
  static bool attr_set[2] = {false, false};
  const int ai = w2 ? 1 : 0;
  if (!attr_set[ai]) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)(kMaxDownWaves * G::kWaveBytes));
    if (e != hipSuccess) return e;
    attr_set[ai] = true;
  }
  MOE_LAUNCH(MOE_K_DOWN, kern, dim3(c.dim / kDownRows), dim3(threads), shm, s, w.plan.base,
             ex.slot_of ? nullptr : ex.base, ex.stride, ex.down_off, ex.n_routed, ex, w, c.dim, c.inter, slots, w2, o);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gateup_m1(const XArena& ex, const FrontSelect* sel, const int32_t* hdr_in,
                            const uint16_t* x, const moe_layer* layer, const moe_cfg& c, const Ws& w, hipStream_t s) {
  GateUp1Args a;
  a.mode = sel ? 0 : 1;
  a.slots = c.topk + ex.has_shared();
  const int routed_blocks = a.slots * (c.inter / 32);
  a.shared_units = layer ? c.inter : 0;   // (with either plan source)
  const int rest = a.shared_units - kUnitsRouted * routed_blocks;
  a.shared_blocks = rest > 0 ? (rest + kUnitsShared - 1) / kUnitsShared : 0;
  a.ex = ex;
  a.bias = sel ? sel->bias : nullptr;
  a.hdr_in = hdr_in;
  a.hdr_out = sel ? sel->header : nullptr;
  a.n_routed = c.n_routed;
  a.topk = c.topk;
  a.norm = c.norm_topk_prob;
  a.route_scale = c.route_scale;
  a.dim = c.dim;
  a.inter = c.inter;
  a.L = c.swiglu_limit;
  a.x = x;
  a.w1 = layer ? layer->sh_w1 : nullptr;
  a.w3 = layer ? layer->sh_w3 : nullptr;
  switch (c.dim / 256) {
    case 1: return launch_gateup_m1_t<1>(a, c, w, s);
    case 2: return launch_gateup_m1_t<2>(a, c, w, s);
    case 4: return launch_gateup_m1_t<4>(a, c, w, s);
    case 8: return launch_gateup_m1_t<8>(a, c, w, s);
    case 16: return launch_gateup_m1_t<16>(a, c, w, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_down_m1(const XArena& ex, const moe_cfg& c, const Ws& w, const uint16_t* w2, const LayerOut& o,
                          hipStream_t s) {
  hipError_t err;
  switch (c.inter / 256) {
    case 1: err = launch_down_m1_t<1>(ex, c, w, w2, o, s); break;
    case 2: err = launch_down_m1_t<2>(ex, c, w, w2, o, s); break;
    case 4: err = launch_down_m1_t<4>(ex, c, w, w2, o, s); break;
    case 8: err = launch_down_m1_t<8>(ex, c, w, w2, o, s); break;
    case 16: err = launch_down_m1_t<16>(ex, c, w, w2, o, s); break;
    default: err = hipErrorInvalidValue; break;
  }
  return err;
}

}  // namespace moe
