// Device building blocks of the K-quant GEMVs shared by the general and
// the single-token kernels: direct-to-LDS tile staging, the per-lane
// activation of one super-block, and the Q2_K / Q3_K super-block dot
// products (exact integer sums, float64 epilogue).
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "moe_internal.h"
#include "moe_math.h"
#include "moe_wave.h"

namespace moe {

__device__ inline double fp16_f64(uint32_t bits16) {
  return (double)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
__device__ inline uint16_t f32_to_fp16_bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// ---- direct-to-LDS staging --------------------------------------------------
// Cache policy of the weight streams: the nt (non-temporal) bit. Each weight
// byte is read once per launch; without the bit those lines push the code,
// the router rows and the activations out of the L2 between launches (a
// decode step was 2 us slower).
constexpr int kWeightStream = 2;

// A tile of rows is copied HBM -> LDS with global_load_lds_dwordx4 (no VGPRs,
// no wait at issue). Workgroups are 256 threads; wave w copies 16-byte chunks
// w*64 + 256*k + lane (k < KC), so every wave issues exactly KC instructions
// per tile (lanes past the tile's end re-read its last chunk into the slot's
// padding) and a tile's arrival is a compile-time vmcnt.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }
__device__ __forceinline__ void block_sync_lds() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int KC>
__device__ __forceinline__ void dma_tile(const uint8_t* g, uint8_t* slot, int nchunks) {
  // the source chunk per lane, the LDS destination per wave (uniform: m0 from scalar arithmetic)
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    const int i = (int)threadIdx.x + 256 * k;
    const int src = i < nchunks ? i : nchunks - 1;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(g + 16 * src),
                                     (__attribute__((address_space(3))) void*)(slot + 16 * (w * 64 + 256 * k)), 16,
                                     0, kWeightStream);
  }
}

// As dma_tile, but the tile occupies exactly nchunks*16 bytes (nchunks >= 64,
// no padding): an instruction that would run past the end copies the tile's
// last 64 chunks instead (the same bytes again to the same place).
template <int KC>
__device__ __forceinline__ void dma_tile_exact(const uint8_t* g, uint8_t* slot, int nchunks) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    const int base = min(w * 64 + 256 * k, nchunks - 64);
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(g + 16 * (base + lane)),
                                     (__attribute__((address_space(3))) void*)(slot + 16 * base), 16, 0,
                                     kWeightStream);
  }
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

// The same activation staged once per workgroup in LDS (instead of every
// lane fetching its own copy from L2): per super-block sb the 256 codes,
// then the 16 code sums, then the 8 scales. The codes and sums of
// consecutive sb are padded by 16 bytes so that the 16 lanes of a quarter
// wave (16 different sb) read different LDS banks.
template <int NSB>
struct ActLds {
  static constexpr int kCodeStride = 256 + 16;
  static constexpr int kQStride = 64 + 16;
  static constexpr int kQ = NSB * kCodeStride;
  static constexpr int kD = kQ + NSB * kQStride;
  static constexpr int kBytes = kD + NSB * 16;
  static constexpr int kChunks = NSB * 21;   // 16-byte pieces: 16 code, 4 sum, 1 scale per sb
};

// Piece i (< ActLds<NSB>::kChunks) of one token's q8_1 activation: where it
// is in global memory (codes q, per-16 sums s, scales d) and in the LDS image.
template <int NSB>
__device__ __forceinline__ const uint4* act_piece_src(const int8_t* q, const int32_t* s, const uint16_t* d, int i) {
  if (i < NSB * 16) return reinterpret_cast<const uint4*>(q + 16 * i);
  if (i < NSB * 20) return reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(s) + 16 * (i - NSB * 16));
  return reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(d) + 16 * (i - NSB * 20));
}
template <int NSB>
__device__ __forceinline__ uint4* act_piece_dst(uint8_t* lds, int i) {
  using AL = ActLds<NSB>;
  if (i < NSB * 16) return reinterpret_cast<uint4*>(lds + (i >> 4) * AL::kCodeStride + 16 * (i & 15));
  if (i < NSB * 20) {
    const int j = i - NSB * 16;
    return reinterpret_cast<uint4*>(lds + AL::kQ + (j >> 2) * AL::kQStride + 16 * (j & 3));
  }
  return reinterpret_cast<uint4*>(lds + AL::kD + 16 * (i - NSB * 20));
}
// Copies piece i of one token's q8_1 activation into the LDS image.
template <int NSB>
__device__ __forceinline__ void act_piece_to_lds(uint8_t* lds, const int8_t* q, const int32_t* s, const uint16_t* d,
                                                 int i) {
  *act_piece_dst<NSB>(lds, i) = *act_piece_src<NSB>(q, s, d, i);
}

template <int NSB>
__device__ __forceinline__ void load_act_lds(Act& A, const uint8_t* lds, int sb) {
  using AL = ActLds<NSB>;
  const uint4* q4 = reinterpret_cast<const uint4*>(lds + sb * AL::kCodeStride);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint4 v = q4[i];
    A.a[4 * i] = v.x;
    A.a[4 * i + 1] = v.y;
    A.a[4 * i + 2] = v.z;
    A.a[4 * i + 3] = v.w;
  }
  const int4* s4 = reinterpret_cast<const int4*>(lds + AL::kQ + sb * AL::kQStride);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int4 v = s4[i];
    A.Q[4 * i] = v.x;
    A.Q[4 * i + 1] = v.y;
    A.Q[4 * i + 2] = v.z;
    A.Q[4 * i + 3] = v.w;
  }
  const uint4 dv = *reinterpret_cast<const uint4*>(lds + AL::kD + 16 * sb);
  const uint32_t dw[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
  for (int t = 0; t < 8; ++t) A.D8[t] = fp16_f64((dw[t >> 1] >> (16 * (t & 1))) & 0xFFFFu);
}

// Weight w of a super-block: h = w/128, j = (w%128)/32, l = w%32, s = w/16.
// Code word wi (bytes 4wi..4wi+3 of the 64 code bytes) holds, at bit pair j,
// the codes of weights 128*(wi/8) + 32*j + 4*(wi%8) + 0..3, i.e. sub-block
// s = 8*(wi/8) + 2*j + (wi%8)/4, activation word 32*(wi/8) + 8*j + wi%8.
//
// To save the shifts, bit pairs j = 1 and 2 are masked in place: their bytes
// hold 4*code and 16*code (still < 128, so the signed dot4 is exact), and the
// sub-block sums carry that factor 4^j until the float64 step, where the
// q8_1 block scale is divided by it (an exact power of two). The 24-bit
// multiplies (full rate) are exact: every operand is below 2^23.

__device__ __forceinline__ int mad24(int a, int b, int c) { return __mul24(a, b) + c; }

// sdot4(a, b, 0) in the VOP3 form with an inline zero: the compiler otherwise
// picks the VOP2 form and zeroes a register first (one instruction more per
// accumulator; the routed gate/up tiles are issue-bound where two routed
// workgroups share a CU).
__device__ __forceinline__ int dot4_zero(int a, int b) {
  int r;
  asm("v_dot4_i32_i8 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// The two signed 16-bit halves of a and b multiplied pairwise and summed
// (v_dot2_i32_i16, VOP3 form with an inline zero addend).
__device__ __forceinline__ int dot2_zero(uint32_t a, uint32_t b) {
  int r;
  asm("v_dot2_i32_i16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Sum of v over aligned groups of NSB lanes (every lane of a group gets the
// group's sum; the same fixed order on every run).
template <int NSB>
__device__ __forceinline__ double seg_sum_f64(double v) {
  auto step = [](double x, auto ctrl_tag) -> double {
    constexpr int CTRL = decltype(ctrl_tag)::value;
    const uint64_t b = __builtin_bit_cast(uint64_t, x);
    // every lane has a source under these controls, so the old value is never read: no zeroed register
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)b, CTRL, 0xf, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), CTRL, 0xf, 0xf, false);
    return x + __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
  };
  if constexpr (NSB >= 2) v = step(v, std::integral_constant<int, 0xb1>{});    // lane ^ 1
  if constexpr (NSB >= 4) v = step(v, std::integral_constant<int, 0x4e>{});    // lane ^ 2
  if constexpr (NSB >= 8) v = step(v, std::integral_constant<int, 0x141>{});   // other quad of the half row
  if constexpr (NSB >= 16) v = step(v, std::integral_constant<int, 0x140>{});  // other half of the row
  if constexpr (NSB >= 32) v = sum_xor16_f64(v);
  if constexpr (NSB >= 64) v = sum_xor32_f64(v);
  return v;
}

// Q2_K (84 B: scales[16], qs[64], d, dmin) at a 4-byte aligned LDS address.
__device__ inline double dot_q2k(const uint8_t* p, const Act& A) {
  const uint32_t* p32 = reinterpret_cast<const uint32_t*>(p);
  uint32_t sc[4], qs[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) sc[i] = p32[i];
#pragma unroll
  for (int i = 0; i < 16; ++i) qs[i] = p32[4 + i];
  const uint32_t dd = p32[20];
  int I[16];
#pragma unroll
  for (int s = 0; s < 16; ++s) I[s] = 0;
#pragma unroll
  for (int wi = 0; wi < 16; ++wi) {
    const int h = wi >> 3, t4 = wi & 7, half = t4 >> 2;
    const uint32_t w = qs[wi];
    const uint32_t v0 = w & 0x03030303u;           // 1 * code
    const uint32_t v1 = w & 0x0C0C0C0Cu;           // 4 * code
    const uint32_t v2 = w & 0x30303030u;           // 16 * code
    const uint32_t v3 = (w >> 6) & 0x03030303u;    // 1 * code
    int* Ih = I + 8 * h + half;
    const bool first = (t4 & 3) == 0;   // each accumulator's first product: the VOP3 form with a zero addend
    Ih[0] = first ? dot4_zero((int)v0, (int)A.a[32 * h + t4]) : __builtin_amdgcn_sdot4((int)v0, (int)A.a[32 * h + t4], Ih[0], false);
    Ih[2] = first ? dot4_zero((int)v1, (int)A.a[32 * h + 8 + t4]) : __builtin_amdgcn_sdot4((int)v1, (int)A.a[32 * h + 8 + t4], Ih[2], false);
    Ih[4] = first ? dot4_zero((int)v2, (int)A.a[32 * h + 16 + t4]) : __builtin_amdgcn_sdot4((int)v2, (int)A.a[32 * h + 16 + t4], Ih[4], false);
    Ih[6] = first ? dot4_zero((int)v3, (int)A.a[32 * h + 24 + t4]) : __builtin_amdgcn_sdot4((int)v3, (int)A.a[32 * h + 24 + t4], Ih[6], false);
  }
  double accS = 0.0, accM = 0.0;
  uint32_t mins[4];   // the 4-bit mins of sub-blocks 4i..4i+3 as bytes
#pragma unroll
  for (int i = 0; i < 4; ++i) mins[i] = (sc[i] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t word = sc[t >> 1] >> (16 * (t & 1));
    const int sa = (int)(word & 15u), sb_ = (int)((word >> 8) & 15u);
    const int S = mad24(sa, I[2 * t], __mul24(sb_, I[2 * t + 1]));
    // ma*Q[2t] + mb*Q[2t+1] in one signed 16-bit pair product (|Q| <= 16*127)
    const uint32_t mp = __builtin_amdgcn_perm(0u, mins[t >> 1], (t & 1) ? 0x0C030C02u : 0x0C010C00u);
    const uint32_t qp = __builtin_amdgcn_perm((uint32_t)A.Q[2 * t + 1], (uint32_t)A.Q[2 * t], 0x05040100u);
    const int M = dot2_zero(mp, qp);
    const int j = t & 3;
    const double fj = j == 1 ? 0.25 : (j == 2 ? 0.0625 : 1.0);   // undo the in-place 4^j
    accS = __builtin_fma(A.D8[t] * fj, (double)S, accS);
    accM = __builtin_fma(A.D8[t], (double)M, accM);
  }
  const double d = fp16_f64(dd & 0xFFFFu), dmin = fp16_f64(dd >> 16);
  return d * accS - dmin * accM;
}

__device__ inline uint32_t ld32_a2(const uint8_t* p) {   // 2-byte aligned LDS dword
  const uint16_t* p16 = reinterpret_cast<const uint16_t*>(p);
  return (uint32_t)p16[0] | ((uint32_t)p16[1] << 16);
}

// Q3_K (110 B: hmask[32], qs[64], scales[12], d) at a 2-byte aligned LDS
// address. A weight is q2 + 4*hb - 4 (q2 the 2-bit code, hb its hmask bit);
// the dot4 runs on q2 + 4*hb (0..7, scaled by 4^j in place for j = 1, 2) and
// the -4 comes back through the per-16 activation sums.
__device__ inline double dot_q3k(const uint8_t* p, const Act& A) {
  uint32_t hm[8], qs[16], sc[3];
#pragma unroll
  for (int i = 0; i < 8; ++i) hm[i] = ld32_a2(p + 4 * i);
#pragma unroll
  for (int i = 0; i < 16; ++i) qs[i] = ld32_a2(p + 32 + 4 * i);
#pragma unroll
  for (int i = 0; i < 3; ++i) sc[i] = ld32_a2(p + 96 + 4 * i);
  const uint32_t dbits = reinterpret_cast<const uint16_t*>(p)[54];
  int I[16];
#pragma unroll
  for (int s = 0; s < 16; ++s) I[s] = 0;
#pragma unroll
  for (int wi = 0; wi < 16; ++wi) {
    const int h = wi >> 3, t4 = wi & 7, half = t4 >> 2;
    const uint32_t w = qs[wi], m = hm[t4];
    // bytes of (q2 + 4*hb) * f_j: hb is bit 4h+j of each hmask byte, moved to bit 2+2j (j<3) or 2 (j=3)
    const uint32_t v0 = (w & 0x03030303u) | (((m >> (4 * h)) << 2) & 0x04040404u);
    const uint32_t v1 = (w & 0x0C0C0C0Cu) | ((4 * h + 1 >= 4 ? (m >> (4 * h + 1 - 4)) : (m << (4 - 4 * h - 1))) & 0x10101010u);
    const uint32_t v2 = (w & 0x30303030u) | ((4 * h + 2 >= 6 ? (m >> (4 * h + 2 - 6)) : (m << (6 - 4 * h - 2))) & 0x40404040u);
    const uint32_t v3 = ((w >> 6) & 0x03030303u) | ((4 * h + 3 >= 2 ? (m >> (4 * h + 3 - 2)) : (m << (2 - 4 * h - 3))) & 0x04040404u);
    int* Ih = I + 8 * h + half;
    const bool first = (t4 & 3) == 0;   // each accumulator's first product: the VOP3 form with a zero addend
    Ih[0] = first ? dot4_zero((int)v0, (int)A.a[32 * h + t4]) : __builtin_amdgcn_sdot4((int)v0, (int)A.a[32 * h + t4], Ih[0], false);
    Ih[2] = first ? dot4_zero((int)v1, (int)A.a[32 * h + 8 + t4]) : __builtin_amdgcn_sdot4((int)v1, (int)A.a[32 * h + 8 + t4], Ih[2], false);
    Ih[4] = first ? dot4_zero((int)v2, (int)A.a[32 * h + 16 + t4]) : __builtin_amdgcn_sdot4((int)v2, (int)A.a[32 * h + 16 + t4], Ih[4], false);
    Ih[6] = first ? dot4_zero((int)v3, (int)A.a[32 * h + 24 + t4]) : __builtin_amdgcn_sdot4((int)v3, (int)A.a[32 * h + 24 + t4], Ih[6], false);
  }
  // The 6-bit scales u of sub-blocks 4k..4k+3 as the signed bytes 4*(u - 32) of
  // one word: the low nibble (bytes 0-3 of scales[], low nibbles for k < 2,
  // high for k >= 2) to bits 2-5, its two high bits (bits 2k, 2k+1 of bytes
  // 8-11) to bits 6-7, then bit 7 flipped (4u - 128 in two's complement).
  uint32_t P[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t lo = (k < 2 ? (sc[k & 1] << 2) : (sc[k & 1] >> 2)) & 0x3C3C3C3Cu;
    const uint32_t hi = sc[2] << (6 - 2 * k);
    P[k] = ((hi & 0xC0C0C0C0u) | lo) ^ 0x80808080u;
  }
  double acc = 0.0;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int j = t & 3;
    const int fj = j == 1 ? 4 : (j == 2 ? 16 : 1);
    int S4 = 0;   // 4 * the sub-block pair's integer sum
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int s = 2 * t + k;
      const int sc4 = (int)(int8_t)(P[s >> 2] >> (8 * (s & 3)));
      S4 = mad24(sc4, I[s] - 4 * fj * A.Q[s], S4);
    }
    const double fjd = j == 1 ? 0.25 : (j == 2 ? 0.0625 : 1.0);
    acc = __builtin_fma(A.D8[t] * (0.25 * fjd), (double)S4, acc);   // the power of two exactly undone
  }
  return fp16_f64(dbits) * acc;
}

template <int NSB>
struct GateUpGeom {
  static constexpr int kRowBytes = NSB * kQ2KBytes;
  static constexpr int kTileChunks = 16 * kRowBytes / 16;        // 16 rows per tile
  static constexpr int kKC = (kTileChunks + 255) / 256;
  static constexpr int kSlotBytes = kKC * 4096;
  static constexpr int kTileBytes = 16 * kRowBytes;               // an exact (unpadded) slot
  static constexpr int kItems = 16 * NSB;                         // (row, super-block) per tile
  static constexpr int kIters = (kItems + 255) / 256;
};

}  // namespace moe
