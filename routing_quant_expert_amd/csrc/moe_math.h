// Correctly rounded f32 exp and log1p, and the f32 helpers of the score and
// SwiGLU chains. Every function is __host__ __device__: the device build is
// the product; the host build lets the CPU tests check the same code.
//
// Method (own design; the pages only ask that the device selection equal the
// host reference bit for bit [device_route.rs, module doc]; read here as
// "every elementary step correctly rounded to f32"):
//  * fast path: evaluate in float64 with the straight-line estimates exp_est
//    and log1p_est below (relative error under 2^-50), round to f32, and
//    accept unless the float64 value may lie within 2^-47 (relative) of the
//    midpoint between two f32 neighbours (Ziv's rounding test: A. Ziv, "Fast
//    evaluation of elementary mathematical functions with correctly rounded
//    last bit", ACM TOMS 1991), read off the estimate's bits (ziv_reject);
//    the fast paths are straight-line code (selects, no branches) and only
//    the rare rejected inputs branch to the slow path;
//  * slow path: double-double arithmetic (Dekker 1971 products and Knuth's
//    two-sum): exp by Cody-Waite reduction x = k ln2 + r with ln2 in three
//    parts, exp(r/256) by its Taylor series to degree 9, then eight
//    squarings (relative error below 2^-95); log1p by one Newton step on
//    y - log1p(x) from the float64 estimate, which doubles its precision.
//    The double-double value is then rounded to f32 exactly.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace moe {

struct dd {
  double hi, lo;
};

__host__ __device__ inline dd two_sum(double a, double b) {
  double s = a + b;
  double bb = s - a;
  double e = (a - (s - bb)) + (b - bb);
  return {s, e};
}

__host__ __device__ inline dd quick_two_sum(double a, double b) {  // |a| >= |b|
  double s = a + b;
  return {s, b - (s - a)};
}

__host__ __device__ inline dd two_prod(double a, double b) {
  double p = a * b;
  return {p, __builtin_fma(a, b, -p)};
}

__host__ __device__ inline dd dd_add(dd a, dd b) {
  dd s = two_sum(a.hi, b.hi);
  dd t = two_sum(a.lo, b.lo);
  s.lo += t.hi;
  s = quick_two_sum(s.hi, s.lo);
  s.lo += t.lo;
  return quick_two_sum(s.hi, s.lo);
}

__host__ __device__ inline dd dd_mul(dd a, dd b) {
  dd p = two_prod(a.hi, b.hi);
  p.lo += a.hi * b.lo + a.lo * b.hi;
  return quick_two_sum(p.hi, p.lo);
}

// 1/n! as a double-double, from exact integers: hi = RN(1/f), lo = RN(residual/f).
__host__ __device__ inline dd inv_factorial(int n) {
  double f = 1.0;
  for (int i = 2; i <= n; ++i) f *= (double)i;  // exact for n <= 18
  double hi = 1.0 / f;
  double lo = __builtin_fma(-hi, f, 1.0) / f;
  return {hi, lo};
}

constexpr double kInvLn2 = 0x1.71547652b82fep+0;
constexpr double kLn2Hi = 0x1.62e42fefa3800p-1;   // ln2 to 42 bits: k*kLn2Hi exact for |k| < 2^11
constexpr double kLn2Lo = 0x1.ef35793c76730p-45;  // the next 53 bits

// exp(x) for a double x in [-746, 710] as a double-double (relative error < 2^-95).
__host__ __device__ inline dd exp_dd(double x) {
  const double kL1 = kLn2Hi;
  const double kL2 = kLn2Lo;
  const double kL3 = 0x1.f97b57a079a19p-103;
  double k = rint(x * kInvLn2);
  double r1 = x - k * kL1;                    // exact (Sterbenz)
  dd t = two_prod(k, kL2);
  dd r = two_sum(r1, -t.hi);
  r.lo += -t.lo - k * kL3;
  r = quick_two_sum(r.hi, r.lo);
  dd rs = {r.hi * 0x1p-8, r.lo * 0x1p-8};     // |rs| < 0.00136
  dd p = inv_factorial(9);
  for (int n = 8; n >= 0; --n) p = dd_add(dd_mul(p, rs), inv_factorial(n));
  for (int i = 0; i < 8; ++i) p = dd_mul(p, p);
  int ki = (int)k;
  return {ldexp(p.hi, ki), ldexp(p.lo, ki)};
}

// The fast paths' float64 estimates: straight-line code (the callers handle
// the ends of the ranges), relative error below 2^-50, a factor 8 inside
// Ziv's 2^-47 margin. FMA rounding u = 2^-53 throughout.
//
// exp_est(x), |x| <= 745: x = k ln2 + r by Cody-Waite (kLn2Hi*k exact, so
// r = x - k ln2 up to one rounding of the kLn2Lo term), |r| <= ln2/2; e^r
// by its Taylor polynomial of degree 13 in Horner form (the omitted terms
// are below r^14/14! < 2^-57 e^r); then times 2^k. The Horner steps add
// under 2u relative (each step's rounding is damped by |r|^i), the rounded
// coefficients under 1.5u and the reduction under u: about 2^-51 in all.
__host__ __device__ inline double exp_est(double x) {
  const double k = rint(x * kInvLn2);
  const double r = __builtin_fma(-k, kLn2Lo, __builtin_fma(-k, kLn2Hi, x));
  double p = 1.0 / 6227020800.0;   // 1/13!
  p = __builtin_fma(p, r, 1.0 / 479001600.0);
  p = __builtin_fma(p, r, 1.0 / 39916800.0);
  p = __builtin_fma(p, r, 1.0 / 3628800.0);
  p = __builtin_fma(p, r, 1.0 / 362880.0);
  p = __builtin_fma(p, r, 1.0 / 40320.0);
  p = __builtin_fma(p, r, 1.0 / 5040.0);
  p = __builtin_fma(p, r, 1.0 / 720.0);
  p = __builtin_fma(p, r, 1.0 / 120.0);
  p = __builtin_fma(p, r, 1.0 / 24.0);
  p = __builtin_fma(p, r, 1.0 / 6.0);
  p = __builtin_fma(p, r, 0.5);
  p = __builtin_fma(p, r, 1.0);
  p = __builtin_fma(p, r, 1.0);
  return ldexp(p, (int)k);
}

// log1p_est(x) for an f32 value x > -1: u = 1 + x is exact (x's last bit
// is at or above 2^-47 when |x| >= 2^-24, and for x >= 2^53 the rounding of
// u changes the logarithm by under 2^-58). u = m 2^k with m in
// [sqrt(1/2), sqrt(2)), f = m - 1 exact (Sterbenz); log(1 + f) = 2 atanh(s)
// with s = f / (2 + f), |s| <= 0.1716, by its series to s^19 (the omitted
// terms are below 2^-55 relative); then + k ln2. s carries about 3u
// (the rounded 2 + f and the division), the series u, the sum with k ln2
// under u: about 2^-51 in all.
__host__ __device__ inline double log1p_est(double x) {
  const double u = 1.0 + x;
  int k;
  double m = frexp(u, &k);
  const bool below = m < 0x1.6a09e667f3bcdp-1;   // sqrt(1/2)
  m = below ? m + m : m;
  k = below ? k - 1 : k;
  const double f = m - 1.0;
  const double s = f / (2.0 + f);
  const double s2 = s * s;
  double q = 2.0 / 19.0;
  q = __builtin_fma(q, s2, 2.0 / 17.0);
  q = __builtin_fma(q, s2, 2.0 / 15.0);
  q = __builtin_fma(q, s2, 2.0 / 13.0);
  q = __builtin_fma(q, s2, 2.0 / 11.0);
  q = __builtin_fma(q, s2, 2.0 / 9.0);
  q = __builtin_fma(q, s2, 2.0 / 7.0);
  q = __builtin_fma(q, s2, 2.0 / 5.0);
  q = __builtin_fma(q, s2, 2.0 / 3.0);
  const double l = __builtin_fma(s * s2, q, 2.0 * s);   // 2s + 2s^3/3 + ... + 2s^19/19
  const double kd = (double)k;
  return __builtin_fma(kd, kLn2Hi, __builtin_fma(kd, kLn2Lo, l));
}

// An f32 value as a double, with the infinity that rounding overflows to
// standing for 2^128 (so that the midpoint above FLT_MAX is finite).
__host__ __device__ inline double f32_as_double(float f) {
  return isinf(f) ? copysign(0x1p128, (double)f) : (double)f;
}

__host__ __device__ inline float next_toward(float f, double y) {
  uint32_t b = __builtin_bit_cast(uint32_t, f);
  double fd = f32_as_double(f);
  if (y > fd) return (f >= 0.0f) ? __builtin_bit_cast(float, b + 1u) : (b == 0x80000000u ? __builtin_bit_cast(float, 1u) : __builtin_bit_cast(float, b - 1u));
  return (f > 0.0f) ? __builtin_bit_cast(float, b - 1u) : (b == 0u ? __builtin_bit_cast(float, 0x80000001u) : __builtin_bit_cast(float, b + 1u));
}

// Midpoint between f and its neighbour toward y (exact in double).
__host__ __device__ inline double midpoint_toward(float f, double y) {
  float nb = next_toward(f, y);
  return 0.5 * (f32_as_double(f) + f32_as_double(nb));
}

// Ziv's test on the bits of a float64 estimate y (relative error < 2^-50)
// whose f32 rounding is wanted: true when y may round differently from the
// exact value. For y in the normal f32 range the rounding discards the low 29
// bits D of y's significand, and the midpoint between the two f32 neighbours
// has D = 2^28; |y - mid| = |D - 2^28| ulp64(y) while 2^-47 |y| < 64 ulp64(y),
// so testing |D - 2^28| <= 64 catches every y within 2^-47 |y| of a midpoint
// (and a few more, which the slow path rounds just as well). Below 2^-126 the
// f32 rounding point lies further up the significand: always rejected.
// NaN and infinite y are the callers' to exclude.
__host__ __device__ inline bool ziv_reject(double y) {
  const uint32_t d = (uint32_t)__builtin_bit_cast(uint64_t, y) & 0x1FFFFFFFu;
  return d - 0x0FFFFFC0u <= 128u || fabs(y) < 0x1p-126;
}

// Correct f32 rounding of a normalised double-double.
__host__ __device__ inline float round_dd_to_f32(dd v) {
  float f = (float)v.hi;
  double fd = f32_as_double(f);
  if (fd == v.hi) {
    // hi is an f32; the tail is far below half an f32 ulp
    return f;
  }
  double mid = midpoint_toward(f, v.hi);
  if (v.hi != mid) return f;   // |hi - mid| >= one double ulp > |lo|
  // hi sits exactly on the midpoint: the tail decides
  float nb = next_toward(f, v.hi);
  bool toward_nb_side = (v.lo > 0.0) == (f32_as_double(nb) > fd);
  if (v.lo == 0.0) return (__builtin_bit_cast(uint32_t, f) & 1u) ? nb : f;
  return toward_nb_side ? nb : f;
}

// The fast path of exp_cr for any f32 x: the estimate rounded to f32 (or the
// exact value of a special input) and whether Ziv's test rejects it.
__host__ __device__ inline float exp_fast(float x, bool& reject) {
  const bool in = x >= -104.0f && x <= 89.0f;   // false for NaN
  const double y = exp_est((double)(in ? x : 0.0f));
  reject = in && ziv_reject(y);
  // exp(x) < 2^-150 below -104 (rounds to +0); above 89 it overflows; NaN stays
  const float sp = x > 89.0f ? __builtin_inff() : (x < -104.0f ? 0.0f : x);
  return in ? (float)y : sp;
}

// RN32(exp(x)) for any f32 x.
__host__ __device__ inline float exp_cr(float x, bool force_slow = false) {
  bool reject;
  const float f = exp_fast(x, reject);
  if (!(reject || force_slow) || !(x >= -104.0f && x <= 89.0f)) return f;
  return round_dd_to_f32(exp_dd((double)x));
}

// The fast path of log1p_cr for any f32 x, as exp_fast.
__host__ __device__ inline float log1p_fast(float x, bool& reject) {
  const bool in = fabsf(x) >= 0x1p-24f && x > -1.0f && x < __builtin_inff();   // false for NaN
  const double y = log1p_est((double)(in ? x : 1.0f));
  reject = in && ziv_reject(y);
  // |x| < 2^-24: |log1p(x) - x| < x^2/2, x is the nearest f32; +inf and NaN
  // stay; -1 gives -inf, below -1 NaN
  const float sp = x == -1.0f ? -__builtin_inff() : (x < -1.0f ? __builtin_nanf("") : x);
  return in ? (float)y : sp;
}

// RN32(log1p(x)) for f32 x >= -1 (NaN for x < -1).
__host__ __device__ inline float log1p_cr(float x, bool force_slow = false) {
  bool reject;
  const float f = log1p_fast(x, reject);
  if (!(reject || force_slow) || !(fabsf(x) >= 0x1p-24f && x > -1.0f && x < __builtin_inff())) return f;
  // Newton on f(y) = (1+x) e^-y - 1: y1 = y0 + (1+x) e^-y0 - 1
  const double y0 = log1p_est((double)x);
  dd u = two_sum(1.0, (double)x);
  dd e = exp_dd(-y0);
  dd p = dd_mul(u, e);
  dd r = dd_add(p, dd{-1.0, 0.0});
  dd y = dd_add(dd{y0, 0.0}, r);
  return round_dd_to_f32(y);
}

// 16-byte streaming load (non-temporal: read once, do not keep in the caches).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ inline uint4 load_nt16(const void* p) {
  u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// f32 operations that must not be contracted into FMAs.
__host__ __device__ inline float fmul(float a, float b) { return a * b; }
__host__ __device__ inline float fadd(float a, float b) { return a + b; }

// score = sqrt(softplus(logit / temp)), softplus(z) = z > 20 ? z : log1p(exp(z))
// [moe_v41.rs, fn softplus, fn route_from_logits]. sqrt and the division are
// correctly rounded in f32: through float64 (53 >= 2*24+2, so the double
// rounding is harmless); temp = 1 divides exactly, so the division is skipped.
// Both fast paths run straight through; if either rejects (or force_slow),
// the chain is redone on the slow paths.
__host__ __device__ inline float score_of(float logit, float temp, bool force_slow = false) {
  const float z = temp == 1.0f ? logit : (float)((double)logit / (double)temp);
  bool r1, r2;
  const float e = exp_fast(z, r1);
  float sp = log1p_fast(e, r2);
  if (!(z > 20.0f) && (r1 || r2 || force_slow)) sp = log1p_cr(exp_cr(z, true), true);
  sp = z > 20.0f ? z : sp;
  return (float)sqrt((double)sp);
}

// The glibc score mode's exceptions (moe_glibc_score_table): keys = the f32
// bits of the inputs z <= 20 whose glibc chain differs from the correctly
// rounded one, ascending; vals = glibc's scores; index[p] = the first key with
// prefix (bits >> kScorePrefixShift) >= p. keys == nullptr: the correctly
// rounded mode.
constexpr int kScorePrefixShift = 8;   // 2^24 buckets of 256 inputs
struct ScoreTable {
  const uint32_t* keys;
  const uint32_t* vals;
  const uint32_t* index;
};

// score_of, or in the glibc mode glibc's value where it differs: the input's
// prefix bucket, then a binary search of its keys (about one per bucket).
__host__ __device__ inline float score_mode_of(float logit, float temp, const ScoreTable& t) {
  const float s = score_of(logit, temp);
  if (!t.keys) return s;
  const float z = (float)((double)logit / (double)temp);
  if (!(z <= 20.0f)) return s;
  const uint32_t b = __builtin_bit_cast(uint32_t, z);
  const uint32_t p = b >> kScorePrefixShift;
  uint32_t lo = t.index[p], hi = t.index[p + 1];
  const uint32_t end = hi;
  while (lo < hi) {
    const uint32_t mid = (lo + hi) >> 1;
    if (t.keys[mid] < b) lo = mid + 1;
    else hi = mid;
  }
  return (lo < end && t.keys[lo] == b) ? __builtin_bit_cast(float, t.vals[lo]) : s;
}

// Clamped SwiGLU: silu(min(g, L)) * clamp(u, -L, L), silu(z) = z / (1 + exp(-z)).
__host__ __device__ inline float swiglu(float g, float u, float L) {
  float zg = g > L ? L : g;
  float e = exp_cr(-zg);
  float den = fadd(1.0f, e);
  float silu = (float)((double)zg / (double)den);
  float uc = u > L ? L : (u < -L ? -L : u);
  return fmul(silu, uc);
}

// f32 -> bf16 round to nearest even on the bits [moe_v41.rs, fn bf16_bytes].
__host__ __device__ inline uint16_t bf16_rne(float f) {
  uint32_t b = __builtin_bit_cast(uint32_t, f);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

__host__ __device__ inline float bf16_f32(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }

// q8_1 of one value given the block's f32 scale d (amax/127): roundf(x/d),
// half away from zero; 0 when amax == 0.
__host__ __device__ inline int q8_code(float x, float d) {
  if (d == 0.0f) return 0;
  float v = (float)((double)x / (double)d);
  float t = truncf(v);
  if (fabsf(v - t) >= 0.5f) t += copysignf(1.0f, v);
  return (int)t;
}

}  // namespace moe
