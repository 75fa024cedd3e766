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
#include "moe_math.h"

namespace moe {
namespace {

__device__ inline double fp16_f64(uint32_t bits16) {
  return (double)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
__device__ inline uint16_t f32_to_fp16_bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// Copies the byte range [g, g+nbytes) into LDS with 16-byte loads of the
// aligned chunks that cover it (never touching a page the range does not
// touch). Returns the offset in LDS of byte g.
__device__ inline int stage_rows(uint8_t* lds, const uint8_t* g, int nbytes) {
  uintptr_t a = (uintptr_t)g;
  uintptr_t a0 = a & ~(uintptr_t)15;
  int pad = (int)(a - a0);
  int nchunks = (int)(((a + nbytes + 15) & ~(uintptr_t)15) - a0) >> 4;
  const uint4* src = reinterpret_cast<const uint4*>(a0);
  uint4* dst = reinterpret_cast<uint4*>(lds);
  for (int i = threadIdx.x; i < nchunks; i += blockDim.x) dst[i] = load_nt16(src + i);
  return pad;
}

// The activation of one token for the super-block `sb`: 64 words of int8
// codes, the 16 per-16 code sums, the 8 q8_1 scales as float64.
struct Act {
  uint32_t a[64];
  int Q[16];
  double D8[8];
};

__device__ inline void load_act(Act& A, const int8_t* q, const uint16_t* d, const int32_t* s, int sb) {
  const uint4* q4 = reinterpret_cast<const uint4*>(q + 256 * sb);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint4 v = q4[i];
    A.a[4 * i] = v.x;
    A.a[4 * i + 1] = v.y;
    A.a[4 * i + 2] = v.z;
    A.a[4 * i + 3] = v.w;
  }
  const int4* s4 = reinterpret_cast<const int4*>(s + 16 * sb);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int4 v = s4[i];
    A.Q[4 * i] = v.x;
    A.Q[4 * i + 1] = v.y;
    A.Q[4 * i + 2] = v.z;
    A.Q[4 * i + 3] = v.w;
  }
  uint4 dv = *reinterpret_cast<const uint4*>(d + 8 * sb);
  uint32_t dw[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
  for (int t = 0; t < 8; ++t) A.D8[t] = fp16_f64((dw[t >> 1] >> (16 * (t & 1))) & 0xFFFFu);
}

// Weight w of a super-block: h = w/128, j = (w%128)/32, l = w%32, s = w/16.
// Code word wi (bytes 4wi..4wi+3 of the 64 code bytes) holds, at bit pair j,
// the codes of weights 128*(wi/8) + 32*j + 4*(wi%8) + 0..3, i.e. sub-block
// s = 8*(wi/8) + 2*j + (wi%8)/4, activation word 32*(wi/8) + 8*j + wi%8.

// Q2_K (84 B: scales[16], qs[64], d, dmin) at a 4-byte aligned LDS address.
__device__ inline double dot_q2k(const uint8_t* p, const Act& A) {
  const uint32_t* p32 = reinterpret_cast<const uint32_t*>(p);
  uint32_t sc[4], qs[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) sc[i] = p32[i];
#pragma unroll
  for (int i = 0; i < 16; ++i) qs[i] = p32[4 + i];
  uint32_t dd = p32[20];
  int I[16];
#pragma unroll
  for (int s = 0; s < 16; ++s) I[s] = 0;
#pragma unroll
  for (int wi = 0; wi < 16; ++wi) {
    const int h = wi >> 3, t4 = wi & 7, half = t4 >> 2;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t v = (qs[wi] >> (2 * j)) & 0x03030303u;
      I[8 * h + 2 * j + half] = __builtin_amdgcn_sdot4((int)v, (int)A.a[32 * h + 8 * j + t4], I[8 * h + 2 * j + half], false);
    }
  }
  double accS = 0.0, accM = 0.0;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    uint32_t b0 = (sc[t >> 1] >> (16 * (t & 1))) & 0xFFu;
    uint32_t b1 = (sc[t >> 1] >> (16 * (t & 1) + 8)) & 0xFFu;
    int S = (int)(b0 & 15u) * I[2 * t] + (int)(b1 & 15u) * I[2 * t + 1];
    int M = (int)(b0 >> 4) * A.Q[2 * t] + (int)(b1 >> 4) * A.Q[2 * t + 1];
    accS = __builtin_fma(A.D8[t], (double)S, accS);
    accM = __builtin_fma(A.D8[t], (double)M, accM);
  }
  double d = fp16_f64(dd & 0xFFFFu), dmin = fp16_f64(dd >> 16);
  return d * accS - dmin * accM;
}

__device__ inline uint32_t ld32_a2(const uint8_t* p) {   // 2-byte aligned LDS dword
  const uint16_t* p16 = reinterpret_cast<const uint16_t*>(p);
  return (uint32_t)p16[0] | ((uint32_t)p16[1] << 16);
}

// Q3_K (110 B: hmask[32], qs[64], scales[12], d) at a 2-byte aligned LDS address.
__device__ inline double dot_q3k(const uint8_t* p, const Act& A) {
  uint32_t hm[8], qs[16], sc[3];
#pragma unroll
  for (int i = 0; i < 8; ++i) hm[i] = ld32_a2(p + 4 * i);
#pragma unroll
  for (int i = 0; i < 16; ++i) qs[i] = ld32_a2(p + 32 + 4 * i);
#pragma unroll
  for (int i = 0; i < 3; ++i) sc[i] = ld32_a2(p + 96 + 4 * i);
  uint32_t dbits = reinterpret_cast<const uint16_t*>(p)[54];
  int I[16];
#pragma unroll
  for (int s = 0; s < 16; ++s) I[s] = 0;
#pragma unroll
  for (int wi = 0; wi < 16; ++wi) {
    const int h = wi >> 3, t4 = wi & 7, half = t4 >> 2;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t q2 = (qs[wi] >> (2 * j)) & 0x03030303u;
      uint32_t hb = (hm[t4] >> (4 * h + j)) & 0x01010101u;
      uint32_t v = q2 | (hb << 2);   // value + 4, in 0..7
      I[8 * h + 2 * j + half] = __builtin_amdgcn_sdot4((int)v, (int)A.a[32 * h + 8 * j + t4], I[8 * h + 2 * j + half], false);
    }
  }
  double acc = 0.0;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    int S = 0;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int s = 2 * t + k;
      uint32_t lo_b = (sc[(s & 7) >> 2] >> (8 * (s & 3))) & 0xFFu;   // byte s (s<8) or s-8
      uint32_t lo = s < 8 ? (lo_b & 15u) : (lo_b >> 4);
      uint32_t hi_b = (sc[2] >> (8 * (s & 3))) & 0xFFu;               // byte 8 + s%4
      uint32_t hi = (hi_b >> (2 * (s >> 2))) & 3u;
      int us = (int)(lo | (hi << 4)) - 32;
      S += us * (I[s] - 4 * A.Q[s]);
    }
    acc = __builtin_fma(A.D8[t], (double)S, acc);
  }
  return fp16_f64(dbits) * acc;
}

// ---------------------------------------------------------------------------
// Gate/up on Q2_K + clamped SwiGLU + q8_1 of h. Workgroup = (distinct expert
// u, 32-row group): its 32 gate rows and 32 up rows for every token that
// picked u. Rows are staged in LDS `rc` at a time; a row's super-blocks go to
// `nsb` consecutive lanes and are summed by a float64 butterfly.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gateup(moe_experts ex, PlanView plan, const int8_t* __restrict__ xq,
                                                const uint16_t* __restrict__ xd, const int32_t* __restrict__ xs,
                                                int dim, int inter, int nsb, int rc, float* __restrict__ g_out,
                                                float* __restrict__ u_out, float* __restrict__ h_out,
                                                int8_t* __restrict__ hq, uint16_t* __restrict__ hd,
                                                int32_t* __restrict__ hs, float L) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ float gu[2][kMaxDecodeTokens][32];
  const int ngr = inter / 32;
  const int u = blockIdx.x / ngr, grp = blockIdx.x % ngr;
  if (u >= *plan.n_u()) return;
  const int e = plan.u_expert()[u], first = plan.u_first()[u], np = plan.u_npairs()[u];
  const int RB = nsb * kQ2KBytes;
  const int sb = threadIdx.x % nsb;
  Act A;
  for (int mat = 0; mat < 2; ++mat) {
    const uint8_t* mbase = (const uint8_t*)ex.base + (uint64_t)e * ex.stride + (mat ? ex.up_off : ex.gate_off);
    for (int r0 = 0; r0 < 32; r0 += rc) {
      __syncthreads();
      int pad = stage_rows(lds, mbase + (uint64_t)(32 * grp + r0) * RB, rc * RB);
      __syncthreads();
      const int items = rc * nsb;
      for (int j = 0; j < np; ++j) {
        const int tok = plan.pair_tok()[first + j];
        load_act(A, xq + (int64_t)tok * dim, xd + (int64_t)tok * (dim / 32), xs + (int64_t)tok * (dim / 16), sb);
        for (int base = 0; base < items; base += 256) {
          const int i = base + threadIdx.x;
          const bool act = i < items;
          const int row = i / nsb;
          double part = act ? dot_q2k(lds + pad + row * RB + kQ2KBytes * sb, A) : 0.0;
          for (int s = 1; s < nsb; s <<= 1) part += __shfl_xor(part, s);
          if (act && sb == 0) gu[mat][j][r0 + row] = (float)part;
        }
      }
    }
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 31;
  for (int j = wave; j < np; j += 4) {
    const int pair = first + j;
    float gv = gu[0][j][r], uv = gu[1][j][r];
    float hv = swiglu(gv, uv, L);
    float a = fabsf(hv);
    for (int s = 16; s >= 1; s >>= 1) a = fmaxf(a, __shfl_xor(a, s));
    float d = (float)((double)a / 127.0);
    int q = a == 0.0f ? 0 : q8_code(hv, d);
    int sum = q;
    for (int s = 8; s >= 1; s >>= 1) sum += __shfl_xor(sum, s);
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
// Down on Q3_K: workgroup = (distinct expert u, 32 output rows), every token
// that picked u. y[pair][row] = RN32(the row's float64 sum).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_down(moe_experts ex, PlanView plan, const int8_t* __restrict__ hq,
                                              const uint16_t* __restrict__ hd, const int32_t* __restrict__ hs,
                                              int dim, int inter, int nsb, int rc, float* __restrict__ y) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int ngr = dim / 32;
  const int u = blockIdx.x / ngr, grp = blockIdx.x % ngr;
  if (u >= *plan.n_u()) return;
  const int e = plan.u_expert()[u], first = plan.u_first()[u], np = plan.u_npairs()[u];
  const int RB = nsb * kQ3KBytes;
  const int sb = threadIdx.x % nsb;
  const uint8_t* mbase = (const uint8_t*)ex.base + (uint64_t)e * ex.stride + ex.down_off;
  Act A;
  for (int r0 = 0; r0 < 32; r0 += rc) {
    __syncthreads();
    int pad = stage_rows(lds, mbase + (uint64_t)(32 * grp + r0) * RB, rc * RB);
    __syncthreads();
    const int items = rc * nsb;
    for (int j = 0; j < np; ++j) {
      const int pair = first + j;
      load_act(A, hq + (int64_t)pair * inter, hd + (int64_t)pair * (inter / 32), hs + (int64_t)pair * (inter / 16), sb);
      for (int base = 0; base < items; base += 256) {
        const int i = base + threadIdx.x;
        const bool act = i < items;
        const int row = i / nsb;
        double part = act ? dot_q3k(lds + pad + row * RB + kQ3KBytes * sb, A) : 0.0;
        for (int s = 1; s < nsb; s <<= 1) part += __shfl_xor(part, s);
        if (act && sb == 0) y[(int64_t)pair * dim + 32 * grp + r0 + row] = (float)part;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Combine: acc = +0; over the token's picks in plan order (ascending id)
// acc = acc + w*y; then acc = acc + sd when the shared expert is present
// [moe_v41.rs, fn shared_side: added after the routed experts].
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_combine(PlanView plan, const float* __restrict__ y, int dim, int topk,
                                                 const float* __restrict__ sd, float* __restrict__ out_f32,
                                                 uint16_t* __restrict__ out_bf16) {
  const int t = blockIdx.y;
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= dim) return;
  float acc = 0.0f;
  for (int i = 0; i < topk; ++i) {
    int p = plan.tok_pairs()[t * topk + i];
    if (p >= 0) acc = fadd(acc, fmul(plan.pair_w()[p], y[(int64_t)p * dim + r]));
  }
  if (sd) acc = fadd(acc, sd[(int64_t)t * dim + r]);
  if (out_f32) out_f32[(int64_t)t * dim + r] = acc;
  if (out_bf16) out_bf16[(int64_t)t * dim + r] = bf16_rne(acc);
}

int rows_per_stage(int row_bytes) {
  int rc = 32;
  while (rc > 1 && rc * row_bytes + 16 > 48 * 1024) rc >>= 1;
  return rc;
}

}  // namespace

hipError_t launch_gateup(const moe_experts& ex, int m, const moe_cfg& c, const Ws& w, hipStream_t s) {
  int max_u = min(c.n_routed, m * c.topk);
  int nsb = c.dim / 256;
  int rc = rows_per_stage(nsb * kQ2KBytes);
  size_t shm = (size_t)rc * nsb * kQ2KBytes + 32;
  timed_begin(MOE_K_GATEUP, s);
  hipLaunchKernelGGL(k_gateup, dim3(max_u * (c.inter / 32)), dim3(256), shm, s, ex, w.plan, w.xq, w.xd, w.xs, c.dim,
                     c.inter, nsb, rc, w.g, w.u, w.h, w.hq, w.hd, w.hs, c.swiglu_limit);
  hipError_t err = hipGetLastError();
  timed_end(MOE_K_GATEUP, s);
  return err;
}

hipError_t launch_down(const moe_experts& ex, int m, const moe_cfg& c, const Ws& w, hipStream_t s) {
  int max_u = min(c.n_routed, m * c.topk);
  int nsb = c.inter / 256;
  int rc = rows_per_stage(nsb * kQ3KBytes);
  size_t shm = (size_t)rc * nsb * kQ3KBytes + 32;
  timed_begin(MOE_K_DOWN, s);
  hipLaunchKernelGGL(k_down, dim3(max_u * (c.dim / 32)), dim3(256), shm, s, ex, w.plan, w.hq, w.hd, w.hs, c.dim,
                     c.inter, nsb, rc, w.y);
  hipError_t err = hipGetLastError();
  timed_end(MOE_K_DOWN, s);
  return err;
}

hipError_t launch_combine(int m, const moe_cfg& c, const Ws& w, const float* sd, float* out_f32, uint16_t* out_bf16,
                          hipStream_t s) {
  hipLaunchKernelGGL(k_combine, dim3((c.dim + 255) / 256, m), dim3(256), 0, s, w.plan, w.y, c.dim, c.topk, sd,
                     out_f32, out_bf16);
  return hipGetLastError();
}

}  // namespace moe
