// Device-side twin of the numpy input generator in synth/__init__.py.
//
// Holds only the seeded draws and the per-field value recipes (integer ops and
// single IEEE-754 roundings, no FMA contraction: built with -ffp-contract=off),
// so its bytes equal the host's. Used to fill multi-GB expert arenas in place.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kMix1 = 0xBF58476D1CE4E5B9ull;
constexpr uint64_t kMix2 = 0x94D049BB133111EBull;

__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * kMix1;
  z = (z ^ (z >> 27)) * kMix2;
  return z ^ (z >> 31);
}

__host__ __device__ inline uint64_t stream_start(uint64_t seed, uint64_t tag) {
  return mix64((seed ^ tag) + kGolden);
}

__device__ inline uint64_t draw(uint64_t s0, uint64_t i) { return mix64(s0 + (i + 1) * kGolden); }

__device__ inline uint16_t scale_f16(uint32_t u32) {
  double u = (double)u32 * 0x1p-32;
  double v = 1e-3 + 9e-3 * u;
  float f = (float)v;
  _Float16 h = (_Float16)f;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ inline uint16_t f32_to_bf16_bits(float v) {
  uint32_t b = __builtin_bit_cast(uint32_t, v);
  uint32_t lsb = (b >> 16) & 1u;
  return (uint16_t)((b + 0x7FFFu + lsb) >> 16);
}

__global__ void k_q2k(uint8_t* __restrict__ dst, uint64_t s0, uint64_t b0, uint64_t nb) {
  uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= nb) return;
  uint64_t base = (b0 + j) * 11ull;
  uint32_t* o = reinterpret_cast<uint32_t*>(dst + j * 84ull);  // 84 = 4*21: dword aligned
  for (int w = 0; w < 10; ++w) {
    uint64_t r = draw(s0, base + w);
    o[2 * w] = (uint32_t)r;
    o[2 * w + 1] = (uint32_t)(r >> 32);
  }
  uint64_t r = draw(s0, base + 10);
  uint32_t d = scale_f16((uint32_t)r);
  uint32_t dmin = scale_f16((uint32_t)(r >> 32));
  o[20] = d | (dmin << 16);
}

__global__ void k_q3k(uint8_t* __restrict__ dst, uint64_t s0, uint64_t b0, uint64_t nb) {
  uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= nb) return;
  uint64_t base = (b0 + j) * 15ull;
  uint16_t* o = reinterpret_cast<uint16_t*>(dst + j * 110ull);  // 110 = 2*55: half-word aligned
  for (int w = 0; w < 14; ++w) {
    uint64_t r = draw(s0, base + w);
    for (int h = 0; h < 4; ++h) {
      int idx = 4 * w + h;        // half-word index within the block
      if (idx < 54) o[idx] = (uint16_t)(r >> (16 * h));
    }
  }
  uint64_t r = draw(s0, base + 14);
  o[54] = scale_f16((uint32_t)r);
}

__global__ void k_normal_bf16(uint16_t* __restrict__ dst, uint64_t s0, uint64_t i0, uint64_t n, double sigma) {
  uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  uint64_t base = 6ull * (i0 + j);
  int64_t s = 0;
  for (int w = 0; w < 6; ++w) {
    uint64_t r = draw(s0, base + w);
    s += (int64_t)(r & 0xFFFFFFFFull) + (int64_t)(r >> 32);
  }
  s -= (int64_t)6 << 32;
  double z = (double)s * 0x1p-32;
  float v = (float)(z * sigma);
  dst[j] = f32_to_bf16_bits(v);
}

__global__ void k_uniform_f32(float* __restrict__ dst, uint64_t s0, uint64_t i0, uint64_t n, double lo, double span) {
  uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  uint64_t r = draw(s0, i0 + j);
  double u = (double)(r >> 11) * 0x1p-53;
  dst[j] = (float)(lo + span * u);
}

inline unsigned grid_of(uint64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

extern "C" {

// Q2_K super-blocks b0..b0+nb-1 of stream (seed, tag) into dst (nb*84 bytes, 4-byte aligned).
int synth_q2k_blocks(void* dst, uint64_t seed, uint64_t tag, uint64_t b0, uint64_t nb, void* stream) {
  if (nb == 0) return 0;
  if (!dst || ((uintptr_t)dst & 3u)) return -1;
  hipLaunchKernelGGL(k_q2k, dim3(grid_of(nb)), dim3(256), 0, (hipStream_t)stream, (uint8_t*)dst,
                     stream_start(seed, tag), b0, nb);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Q3_K super-blocks b0..b0+nb-1 of stream (seed, tag) into dst (nb*110 bytes, 2-byte aligned).
int synth_q3k_blocks(void* dst, uint64_t seed, uint64_t tag, uint64_t b0, uint64_t nb, void* stream) {
  if (nb == 0) return 0;
  if (!dst || ((uintptr_t)dst & 1u)) return -1;
  hipLaunchKernelGGL(k_q3k, dim3(grid_of(nb)), dim3(256), 0, (hipStream_t)stream, (uint8_t*)dst,
                     stream_start(seed, tag), b0, nb);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int synth_normal_bf16(uint16_t* dst, uint64_t seed, uint64_t tag, uint64_t i0, uint64_t n, double sigma,
                      void* stream) {
  if (n == 0) return 0;
  if (!dst) return -1;
  hipLaunchKernelGGL(k_normal_bf16, dim3(grid_of(n)), dim3(256), 0, (hipStream_t)stream, dst,
                     stream_start(seed, tag), i0, n, sigma);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int synth_uniform_f32(float* dst, uint64_t seed, uint64_t tag, uint64_t i0, uint64_t n, double lo, double span,
                      void* stream) {
  if (n == 0) return 0;
  if (!dst) return -1;
  hipLaunchKernelGGL(k_uniform_f32, dim3(grid_of(n)), dim3(256), 0, (hipStream_t)stream, dst,
                     stream_start(seed, tag), i0, n, lo, span);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
