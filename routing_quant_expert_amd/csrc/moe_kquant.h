// Device building blocks of the K-quant GEMVs shared by the general and
// the single-token kernels: direct-to-LDS tile staging, the per-lane
// activation of one super-block, and the Q2_K / Q3_K super-block dot
// products (exact integer sums, float64 epilogue).
#pragma once

#include <hip/hip_runtime.h>

#include "moe_internal.h"
#include "moe_math.h"

namespace moe {

__device__ inline double fp16_f64(uint32_t bits16) {
  return (double)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
__device__ inline uint16_t f32_to_fp16_bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// ---- direct-to-LDS staging --------------------------------------------------
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
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    const int i = w * 64 + 256 * k + lane;
    const int src = i < nchunks ? i : nchunks - 1;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(g + 16 * src),
                                     (__attribute__((address_space(3))) void*)(slot + 16 * (w * 64 + 256 * k)), 16,
                                     0, 0);
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

template <int NSB>
struct GateUpGeom {
  static constexpr int kRowBytes = NSB * kQ2KBytes;
  static constexpr int kTileChunks = 16 * kRowBytes / 16;        // 16 rows per tile
  static constexpr int kKC = (kTileChunks + 255) / 256;
  static constexpr int kSlotBytes = kKC * 4096;
  static constexpr int kItems = 16 * NSB;                         // (row, super-block) per tile
  static constexpr int kIters = (kItems + 255) / 256;
};

}  // namespace moe
