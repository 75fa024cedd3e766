// Launchers of the prefill kernels (moe_prefill.hip): the layer for m tokens
// with the pairs grouped by expert and the expert GEMMs on int8 MFMA.
#pragma once

#include "moe_internal.h"

namespace moe {

// Router + scores for m tokens, a wave per (expert row, 8 tokens), plus the
// q8_1 of x; zeroes the workspace status words first.
hipError_t launch_router_pf(const uint16_t* x, int m, const uint16_t* gate_w, const moe_cfg& c, const Ws& w,
                            float* logits_out, hipStream_t s);
// The plan tables from m headers (picks validated: a token with a pick
// outside [0, n_routed) or repeated is left out and flagged MOE_STATUS_BAD_PICK);
// shq = 1 adds the layer's quantised shared expert (id n_routed) to every kept token.
// grp: int32 scratch of m + 2 * (n_routed + 1) words.
hipError_t launch_group(const int32_t* header, int m, const moe_cfg& c, const Ws& w, int32_t* grp, int shq,
                        hipStream_t s);
// Gate/up (Q2_K) + SwiGLU + q8_1 of h for every pair of the plan.
// part 0: the experts with at most 8 pairs (inter = 256: every expert's down), part 1: the others
hipError_t launch_gateup_pf(const XArena& ex, int m, const moe_cfg& c, const Ws& w, int part, hipStream_t s);
// Down (Q3_K) for every pair of the plan: y [pairs][dim].
hipError_t launch_down_pf(const XArena& ex, int m, const moe_cfg& c, const Ws& w, int part, hipStream_t s);
// The shared expert for m tokens: sg, su, sh = bf16(SwiGLU), sd.
hipError_t launch_shared_pf(const uint16_t* x, int m, const moe_layer& layer, const moe_cfg& c, const Ws& w,
                            hipStream_t s);

}  // namespace moe
