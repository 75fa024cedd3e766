/*
 * Oracle: a plain, slow, CPU reference of the MoE decode layer.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU
 * baseline of the benchmark may load this library. It shares no code with the
 * HIP path (no headers, tables or helpers) and never calls it.
 *
 * Built with gcc -O2 -ffp-contract=off (no fast-math) on x86-64, so every
 * float/double operation below is one IEEE-754 rounding (SSE2); the order of
 * operations is the order written. Correctly rounded exp / log1p come from
 * libquadmath (a quad-precision result rounded once to float).
 *
 * Sources (the pages of the spark_model documentation):
 *   [moe_v41.rs]       module doc; fn softplus; fn route_from_logits;
 *                      fn bf16_bytes; struct MoeV41Cfg; the Kernels list.
 *   [device_route.rs]  module doc (header contents); fn header_words;
 *                      fn parse_header; fn device_route_check (plan order).
 * Where the pages are silent (the Q2_K/Q3_K/q8_1 layouts, the router's
 * accumulation order, the SwiGLU clamp, the exact value of a K-quant dot
 * product) each function states the reading it implements.
 *
 * Parity pins: every exported function is pinned by the CPU tests
 * (tests/test_oracle_*.py) against closed forms, brute force, mpmath or
 * numpy library routines. None is "parity unpinned".
 */
#include <math.h>
#include <quadmath.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define EXPORT __attribute__((visibility("default")))

typedef struct {
  int32_t dim, inter, n_routed, topk, norm_topk_prob;
  float gate_temp, route_scale, swiglu_limit;
  int32_t score_mode; /* 0: correctly rounded chain, 1: the host's glibc chain */
} ocfg;

static void die(const char* msg) {
  fprintf(stderr, "oracle: %s\n", msg);
  abort();
}

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* bf16 -> f32: the bf16 bits are the top half of the f32 bits (exact). */
EXPORT float oracle_bf16_to_f32(uint16_t b) { return u2f((uint32_t)b << 16); }

/* f32 -> bf16, round to nearest even by adding 0x7FFF plus the kept LSB
 * [moe_v41.rs, fn bf16_bytes]. Inputs are finite. */
EXPORT uint16_t oracle_f32_to_bf16(float f) {
  uint32_t b = f2u(f);
  uint32_t lsb = (b >> 16) & 1u;
  return (uint16_t)((b + 0x7FFFu + lsb) >> 16);
}

/* IEEE binary16 value as an exact double. */
EXPORT double oracle_fp16_to_f64(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 31) v = m ? NAN : INFINITY;
  else if (e == 0) v = ldexp((double)m, -24);
  else v = ldexp((double)(1024 + m), e - 25);
  return s ? -v : v;
}

/* f32 -> IEEE binary16, round to nearest even, subnormals kept, overflow to
 * infinity (written from the IEEE-754 definition of the format). */
EXPORT uint16_t oracle_f32_to_fp16(float f) {
  uint32_t b = f2u(f);
  uint16_t sign = (uint16_t)((b >> 16) & 0x8000u);
  int exp = (int)((b >> 23) & 255);
  uint32_t man = b & 0x7FFFFFu;
  if (exp == 255) return sign | 0x7C00u | (man ? 0x200u : 0u);
  if (exp == 0 && man == 0) return sign;
  /* value = sig * 2^(e2) with sig a 24-bit integer (or smaller for subnormal f32) */
  uint32_t sig = exp ? (man | 0x800000u) : man;
  int e2 = (exp ? exp : 1) - 150;          /* value = sig * 2^e2 */
  /* binary16: value = M * 2^(E-25) for E in 1..30 (M in [1024,2048)), or M * 2^-24 subnormal */
  /* pick the target quantum q = 2^qe: normal quantum 2^(E-25) with E from the leading bit */
  int lead = 31 - __builtin_clz(sig);      /* position of the leading 1 */
  int vexp = e2 + lead;                    /* value in [2^vexp, 2^(vexp+1)) */
  int qe = vexp - 10;                      /* quantum for a normal binary16 */
  if (qe < -24) qe = -24;                  /* subnormal range */
  int shift = qe - e2;                     /* bits to drop from sig */
  uint32_t q;                              /* the rounded count of quanta */
  if (shift <= 0) {
    q = sig << (-shift);
  } else if (shift > 25) {
    q = 0;
  } else {
    uint32_t kept = sig >> shift;
    uint32_t rem = sig & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (kept & 1u))) kept += 1;
    q = kept;
  }
  /* q quanta of 2^qe; renormalise */
  if (q == 0) return sign;
  int E;
  uint32_t M;
  if (qe == -24 && q < 1024) { E = 0; M = q; }
  else {
    if (q >= 2048) { q >>= 1; qe += 1; }   /* rounding carried into a new binade (q was 2048) */
    E = qe + 25;
    M = q - 1024;
  }
  if (E >= 31) return sign | 0x7C00u;
  return sign | (uint16_t)(E << 10) | (uint16_t)M;
}

/* fp16 value as a signed integer count of 2^-24 (exact); aborts on inf/nan. */
static int64_t fp16_units(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  if (e == 31) die("non-finite fp16 scale");
  int64_t n = e == 0 ? (int64_t)m : ((int64_t)(1024 + m) << (e - 1));
  return s ? -n : n;
}

/* ------------------------------------------------------------------------ */
/* Correctly rounded elementary functions (one rounding from quad).          */
/* The pages ask for the host reference's softplus bit for bit              */
/* [device_route.rs, module doc]; the host reference calls the platform     */
/* libm. Reading: every elementary step is correctly rounded to f32.         */
/* ------------------------------------------------------------------------ */

EXPORT float oracle_exp_cr(float x) { return (float)expq((__float128)x); }
EXPORT float oracle_log1p_cr(float x) { return (float)log1pq((__float128)x); }

/* softplus with the pages' cut at 20 [moe_v41.rs, fn softplus]. */
static float softplus(float x) {
  if (x > 20.0f) return x;
  return oracle_log1p_cr(oracle_exp_cr(x));
}

/* score = sqrt(softplus(logit / temp)) [moe_v41.rs, fn route_from_logits]. */
EXPORT float oracle_score(float logit, float temp) {
  float z = logit / temp;
  return sqrtf(softplus(z));
}

EXPORT void oracle_scores(const float* logits, int64_t n, float temp, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_score(logits[i], temp);
}

/* The glibc mode: the same chain with the host C library's f32 expf, log1pf  */
/* and sqrtf, as the pages' host reference evaluates it (f32 exp, ln_1p and   */
/* sqrt) [moe_v41.rs, fn softplus, fn route_from_logits; device_route.rs,     */
/* module doc: glibc-exact softplus].                                         */
EXPORT float oracle_score_glibc(float logit, float temp) {
  float z = logit / temp;
  float sp = z > 20.0f ? z : log1pf(expf(z));
  return sqrtf(sp);
}

EXPORT void oracle_scores_glibc(const float* logits, int64_t n, float temp, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_score_glibc(logits[i], temp);
}

/* ------------------------------------------------------------------------ */
/* K-quant super-blocks (256 weights). Reading: the public GGUF layouts.     */
/*   Q2_K (84 B): scales[16] (low nibble scale, high nibble min), qs[64],    */
/*                fp16 d, fp16 dmin.                                          */
/*   Q3_K (110 B): hmask[32], qs[64], scales[12] (16 x 6 bit), fp16 d.       */
/* For weight i: h = i/128, j = (i%128)/32, l = i%32, s = i/16.              */
/* ------------------------------------------------------------------------ */

static uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* integer parts of weight i of a Q2_K block: w = d*sc*q - dmin*mn */
static void q2k_parts(const uint8_t* blk, int i, int* q, int* sc, int* mn) {
  int h = i / 128, j = (i % 128) / 32, l = i % 32, s = i / 16;
  const uint8_t* scales = blk;
  const uint8_t* qs = blk + 16;
  *q = (qs[32 * h + l] >> (2 * j)) & 3;
  *sc = scales[s] & 15;
  *mn = scales[s] >> 4;
}

/* integer parts of weight i of a Q3_K block: w = d*(u-32)*v */
static void q3k_parts(const uint8_t* blk, int i, int* v, int* u) {
  int h = i / 128, j = (i % 128) / 32, l = i % 32, s = i / 16;
  const uint8_t* hmask = blk;
  const uint8_t* qs = blk + 32;
  const uint8_t* sc = blk + 96;
  int q2 = (qs[32 * h + l] >> (2 * j)) & 3;
  int hb = (hmask[l] >> (4 * h + j)) & 1;
  *v = q2 - (hb ? 0 : 4);
  int lo = s < 8 ? (sc[s] & 15) : (sc[s - 8] >> 4);
  int hi = (sc[8 + s % 4] >> (2 * (s / 4))) & 3;
  *u = lo | (hi << 4);
}

/* Exact dequantisation (f64 holds each weight exactly for finite scales). */
EXPORT void oracle_q2k_dequant(const uint8_t* blocks, int64_t nblk, double* w) {
  for (int64_t b = 0; b < nblk; ++b) {
    const uint8_t* blk = blocks + 84 * b;
    double d = oracle_fp16_to_f64(rd16(blk + 80)), dmin = oracle_fp16_to_f64(rd16(blk + 82));
    for (int i = 0; i < 256; ++i) {
      int q, sc, mn;
      q2k_parts(blk, i, &q, &sc, &mn);
      w[256 * b + i] = d * sc * q - dmin * mn;
    }
  }
}

EXPORT void oracle_q3k_dequant(const uint8_t* blocks, int64_t nblk, double* w) {
  for (int64_t b = 0; b < nblk; ++b) {
    const uint8_t* blk = blocks + 110 * b;
    double d = oracle_fp16_to_f64(rd16(blk + 108));
    for (int i = 0; i < 256; ++i) {
      int v, u;
      q3k_parts(blk, i, &v, &u);
      w[256 * b + i] = d * (u - 32) * v;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* q8_1 over 32 consecutive values [moe_v41.rs, module doc: the activation   */
/* is quantised to q8_1 before gate/up and again before down]. Reading (the  */
/* GGUF convention): d = amax/127, q = roundf(x/d) (division, half away from */
/* zero), stored scale d16 = fp16(d). The q8_1 sum field is not used here.   */
/* ------------------------------------------------------------------------ */

EXPORT void oracle_q8_1(const float* x, int64_t n, int8_t* q, uint16_t* d16) {
  if (n % 32) die("q8_1 length not a multiple of 32");
  for (int64_t t = 0; t < n / 32; ++t) {
    const float* xb = x + 32 * t;
    float amax = 0.0f;
    for (int k = 0; k < 32; ++k) {
      float a = fabsf(xb[k]);
      if (a > amax) amax = a;
    }
    float d = amax / 127.0f;
    for (int k = 0; k < 32; ++k) q[32 * t + k] = amax == 0.0f ? 0 : (int8_t)roundf(xb[k] / d);
    d16[t] = oracle_f32_to_fp16(d);
  }
}

/* ------------------------------------------------------------------------ */
/* Router logits: bf16 x . bf16 gate row, f32 accumulation                    */
/* [moe_v41.rs, module doc; Kernels: router_gemv is a strict-order GEMV].    */
/* Reading of the unstated order: 64 partial sums; partial l accumulates the */
/* products of positions 512*i + 8*l + j (i ascending, then j = 0..7), then  */
/* partials combine pairwise as p[l] += p[l ^ s] for s = 32,16,8,4,2,1 and   */
/* the logit is p[0]. Every bf16 x bf16 product is exact in f32.             */
/* ------------------------------------------------------------------------ */

EXPORT void oracle_router_logits(const uint16_t* x, int64_t m, const uint16_t* gate_w, int64_t n_routed,
                                 int64_t dim, float* logits) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t t = 0; t < m; ++t) {
    for (int64_t e = 0; e < n_routed; ++e) {
      const uint16_t* xr = x + t * dim;
      const uint16_t* wr = gate_w + e * dim;
      float p[64], nx[64];
      for (int l = 0; l < 64; ++l) {
        float acc = 0.0f;
        for (int64_t i = 0; 512 * i < dim; ++i)
          for (int j = 0; j < 8; ++j) {
            int64_t k = 512 * i + 8 * l + j;
            if (k < dim) acc = acc + oracle_bf16_to_f32(xr[k]) * oracle_bf16_to_f32(wr[k]);
          }
        p[l] = acc;
      }
      for (int s = 32; s >= 1; s >>= 1) {
        for (int l = 0; l < 64; ++l) nx[l] = p[l] + p[l ^ s];
        memcpy(p, nx, sizeof p);
      }
      logits[t * n_routed + e] = p[0];
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Selection [moe_v41.rs, fn route_from_logits; device_route.rs, module doc, */
/* fn header_words, fn parse_header, fn device_route_check].                 */
/* Header per token, 1 + 3*topk i32 words:                                   */
/*   [0] status: bit 0 miss (never set: all experts resident),               */
/*       bit 1 a NaN ranking key (the pages' "finite scores" failure)        */
/*   [1 .. topk]          picks in pick order                                */
/*   [1+topk .. 2*topk]   f32 bits of the pick-order weights                 */
/*   [1+2*topk .. 3*topk] the plan: the picks in ascending expert id         */
/* ------------------------------------------------------------------------ */

/* "a ranks before b": larger key first; equal keys keep ascending id (the    */
/* pages' sort is stable over ids 0..n-1); NaN keys sink below all others.    */
static int ranks_before(float ka, int a, float kb, int b) {
  int na = isnan(ka), nb = isnan(kb);
  if (na != nb) return !na;
  if (!na && ka != kb) return ka > kb;
  return a < b;
}

EXPORT void oracle_select(const ocfg* c, const float* logits, int64_t m, const float* bias, int32_t* header,
                          float* scores_out) {
  int n = c->n_routed, k = c->topk;
  if (k < 1 || k > n || k > 64) die("bad topk");
  float* scores = (float*)malloc(sizeof(float) * n);
  float* key = (float*)malloc(sizeof(float) * n);
  int* order = (int*)malloc(sizeof(int) * n);
  for (int64_t t = 0; t < m; ++t) {
    int nan_key = 0;
    for (int e = 0; e < n; ++e) {
      scores[e] = c->score_mode == 1 ? oracle_score_glibc(logits[t * n + e], c->gate_temp)
                                     : oracle_score(logits[t * n + e], c->gate_temp);
      key[e] = scores[e] + bias[e];
      if (isnan(key[e])) nan_key = 1;
      if (scores_out) scores_out[t * n + e] = scores[e];
    }
    /* stable insertion sort of the ids by key, descending */
    for (int e = 0; e < n; ++e) order[e] = e;
    for (int a = 1; a < n; ++a) {
      int id = order[a], b = a;
      while (b > 0 && ranks_before(key[id], id, key[order[b - 1]], order[b - 1])) {
        order[b] = order[b - 1];
        --b;
      }
      order[b] = id;
    }
    float wt[64];
    for (int i = 0; i < k; ++i) wt[i] = scores[order[i]];
    if (c->norm_topk_prob && k > 1) {
      float sum = 0.0f;
      for (int i = 0; i < k; ++i) sum = sum + wt[i];
      sum = sum + 1e-20f;
      for (int i = 0; i < k; ++i) wt[i] = wt[i] / sum;
    }
    for (int i = 0; i < k; ++i) wt[i] = wt[i] * c->route_scale;
    int32_t* hd = header + t * (1 + 3 * k);
    hd[0] = nan_key ? 2 : 0;
    for (int i = 0; i < k; ++i) {
      hd[1 + i] = order[i];
      hd[1 + k + i] = (int32_t)f2u(wt[i]);
    }
    /* the plan: picks in ascending id */
    int plan[64];
    for (int i = 0; i < k; ++i) plan[i] = order[i];
    for (int a = 1; a < k; ++a)
      for (int b = a; b > 0 && plan[b] < plan[b - 1]; --b) {
        int tmp = plan[b];
        plan[b] = plan[b - 1];
        plan[b - 1] = tmp;
      }
    for (int i = 0; i < k; ++i) hd[1 + 2 * k + i] = plan[i];
  }
  free(scores);
  free(key);
  free(order);
}

/* ------------------------------------------------------------------------ */
/* K-quant GEMV [moe_v41.rs, module doc: each expert runs as three K-quant   */
/* GEMVs on the raw blocks against q8_1 activations]. Reading of the unstated */
/* accumulation: y = RN32 of the exact sum of (weight * activation) over the  */
/* row, where weight and activation are the exact dequantised values. With   */
/* every fp16 scale an integer count of 2^-24, each product is an integer     */
/* count of 2^-48 and the row sum is held exactly in __int128.                */
/* near[r] = 1 when the exact sum lies within 2^-44 * A of the midpoint       */
/* between two floats, A = the sum of the magnitudes of every product's parts */
/* (scale part and min part separately for Q2_K). Any float64 accumulation    */
/* of those parts with fewer than ~500 roundings in a chain errs by less than */
/* that, so there either neighbour is an accepted rounding.                   */
/* ------------------------------------------------------------------------ */

static float exact_to_f32(__int128 s, unsigned __int128 sabs, uint8_t* near) {
  __float128 y = ldexpq((__float128)s, -48);
  float f = (float)y;
  if (near) {
    *near = 0;
    if ((__float128)f != y) {
      float nb = nextafterf(f, y > (__float128)f ? INFINITY : -INFINITY);
      __float128 mid = ((__float128)f + (__float128)nb) / 2;
      __float128 dist = fabsq(y - mid);
      __float128 tol = ldexpq((__float128)sabs, -48 - 44);
      if (dist <= tol) *near = 1;
    }
  }
  return f;
}

/* act: int8 codes [cols]; d16: fp16 scale per 32 codes [cols/32]. */
EXPORT void oracle_q2k_gemv(const uint8_t* w, int64_t rows, int64_t cols, const int8_t* act, const uint16_t* d16,
                            float* y, uint8_t* near) {
  int64_t nsb = cols / 256;
  if (cols % 256) die("Q2_K row length not a multiple of 256");
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    __int128 s = 0;
    unsigned __int128 sabs = 0;
    for (int64_t b = 0; b < nsb; ++b) {
      const uint8_t* blk = w + (r * nsb + b) * 84;
      int64_t nd = fp16_units(rd16(blk + 80)), nm = fp16_units(rd16(blk + 82));
      for (int i = 0; i < 256; ++i) {
        int q, sc, mn;
        q2k_parts(blk, i, &q, &sc, &mn);
        int64_t k = 256 * b + i;
        int64_t ai = fp16_units(d16[k / 32]) * act[k];
        __int128 ps = (__int128)(nd * sc * q) * ai, pm = (__int128)(nm * mn) * ai;
        s += ps - pm;
        sabs += (unsigned __int128)(ps < 0 ? -ps : ps) + (unsigned __int128)(pm < 0 ? -pm : pm);
      }
    }
    y[r] = exact_to_f32(s, sabs, near ? near + r : NULL);
  }
}

EXPORT void oracle_q3k_gemv(const uint8_t* w, int64_t rows, int64_t cols, const int8_t* act, const uint16_t* d16,
                            float* y, uint8_t* near) {
  int64_t nsb = cols / 256;
  if (cols % 256) die("Q3_K row length not a multiple of 256");
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    __int128 s = 0;
    unsigned __int128 sabs = 0;
    for (int64_t b = 0; b < nsb; ++b) {
      const uint8_t* blk = w + (r * nsb + b) * 110;
      int64_t nd = fp16_units(rd16(blk + 108));
      for (int i = 0; i < 256; ++i) {
        int v, u;
        q3k_parts(blk, i, &v, &u);
        int64_t k = 256 * b + i;
        int64_t wi = nd * (u - 32) * v;
        int64_t ai = fp16_units(d16[k / 32]) * act[k];
        __int128 p = (__int128)wi * ai;
        s += p;
        sabs += (unsigned __int128)(p < 0 ? -p : p);
      }
    }
    y[r] = exact_to_f32(s, sabs, near ? near + r : NULL);
  }
}

/* ------------------------------------------------------------------------ */
/* Clamped SwiGLU [moe_v41.rs, struct MoeV41Cfg: swiglu_limit; Kernels:      */
/* swiglu, swiglu_q8]. Reading of the unstated clamp: the gate is capped     */
/* above at L, the up value clamped to [-L, L]:                              */
/*   h = silu(min(g, L)) * clamp(u, -L, L),  silu(z) = z / (1 + exp(-z)),    */
/* each step one f32 rounding, exp correctly rounded.                        */
/* ------------------------------------------------------------------------ */

EXPORT float oracle_swiglu(float g, float u, float limit) {
  float zg = g > limit ? limit : g;
  float e = oracle_exp_cr(-zg);
  float den = 1.0f + e;
  float silu = zg / den;
  float uc = u > limit ? limit : (u < -limit ? -limit : u);
  return silu * uc;
}

/* ------------------------------------------------------------------------ */
/* One routed expert for one token: gate/up on Q2_K, SwiGLU, q8_1 of h, down */
/* on Q3_K [moe_v41.rs, module doc].                                          */
/*   gate_w, up_w: Q2_K [inter][dim/256] blocks; down_w: Q3_K [dim][inter/256] */
/* ------------------------------------------------------------------------ */

EXPORT void oracle_expert(const ocfg* c, const int8_t* xq, const uint16_t* xd16, const uint8_t* gate_w,
                          const uint8_t* up_w, const uint8_t* down_w, float* g, float* u, float* h, int8_t* hq,
                          uint16_t* hd16, float* y, uint8_t* near_g, uint8_t* near_u, uint8_t* near_y) {
  oracle_q2k_gemv(gate_w, c->inter, c->dim, xq, xd16, g, near_g);
  oracle_q2k_gemv(up_w, c->inter, c->dim, xq, xd16, u, near_u);
  for (int r = 0; r < c->inter; ++r) h[r] = oracle_swiglu(g[r], u[r], c->swiglu_limit);
  oracle_q8_1(h, c->inter, hq, hd16);
  oracle_q3k_gemv(down_w, c->dim, c->inter, hq, hd16, y, near_y);
}

/* ------------------------------------------------------------------------ */
/* Shared expert: resident bf16, dense [moe_v41.rs, module doc; struct        */
/* MoeV41LayerWeights: shared_w1 [inter,dim], shared_w2 [dim,inter],          */
/* shared_w3 [inter,dim]]. Dot products are float64 sums of exact products    */
/* rounded once to f32 (the device sums in f32 in its own order; compared     */
/* with a tolerance). The SwiGLU output is stored as bf16 for the down GEMV.  */
/* ------------------------------------------------------------------------ */

EXPORT void oracle_shared(const ocfg* c, const uint16_t* x, const uint16_t* w1, const uint16_t* w3,
                          const uint16_t* w2, float* sg, float* su, uint16_t* sh, float* sd) {
  int64_t dim = c->dim, inter = c->inter;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < inter; ++i) {
    double a = 0.0, b = 0.0;
    for (int64_t k = 0; k < dim; ++k) {
      double xv = oracle_bf16_to_f32(x[k]);
      a += (double)oracle_bf16_to_f32(w1[i * dim + k]) * xv;
      b += (double)oracle_bf16_to_f32(w3[i * dim + k]) * xv;
    }
    sg[i] = (float)a;
    su[i] = (float)b;
    sh[i] = oracle_f32_to_bf16(oracle_swiglu(sg[i], su[i], c->swiglu_limit));
  }
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < dim; ++r) {
    double a = 0.0;
    for (int64_t i = 0; i < inter; ++i)
      a += (double)oracle_bf16_to_f32(w2[r * inter + i]) * (double)oracle_bf16_to_f32(sh[i]);
    sd[r] = (float)a;
  }
}

/* ------------------------------------------------------------------------ */
/* Combine [moe_v41.rs, Kernels: accumulate, finish; fn shared_side: the      */
/* shared output is added after the routed experts]. acc = +0; over the plan  */
/* (ascending expert id) acc = acc + w_e * y_e; then acc = acc + sd (when sd  */
/* is given); out_f32 = acc, out_bf16 = bf16(acc).                            */
/*   ys: [k][dim] routed outputs in plan order, w: plan-order weights.        */
/* ------------------------------------------------------------------------ */

EXPORT void oracle_combine(int64_t dim, int64_t k, const float* ys, const float* w, const float* sd,
                           float* out_f32, uint16_t* out_bf16) {
  for (int64_t r = 0; r < dim; ++r) {
    float acc = 0.0f;
    for (int64_t e = 0; e < k; ++e) acc = acc + w[e] * ys[e * dim + r];
    if (sd) acc = acc + sd[r];
    out_f32[r] = acc;
    if (out_bf16) out_bf16[r] = oracle_f32_to_bf16(acc);
  }
}

EXPORT int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads the OpenMP loops above use from now on (n >= 1); the CPU baseline
 * times the oracle at one thread and at all host threads. */
EXPORT void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ------------------------------------------------------------------------ */
/* Array forms of the scalar functions above (for the Python tests).         */
/* ------------------------------------------------------------------------ */

EXPORT void oracle_bf16_to_f32_n(const uint16_t* a, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_to_f32(a[i]);
}
EXPORT void oracle_f32_to_bf16_n(const float* a, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_bf16(a[i]);
}
EXPORT void oracle_f32_to_fp16_n(const float* a, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_fp16(a[i]);
}
EXPORT void oracle_fp16_to_f64_n(const uint16_t* a, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_fp16_to_f64(a[i]);
}
EXPORT void oracle_exp_cr_n(const float* a, int64_t n, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_exp_cr(a[i]);
}
EXPORT void oracle_log1p_cr_n(const float* a, int64_t n, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_log1p_cr(a[i]);
}
EXPORT void oracle_swiglu_n(const float* g, const float* u, int64_t n, float limit, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_swiglu(g[i], u[i], limit);
}
EXPORT void oracle_scores_par(const float* logits, int64_t n, float temp, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_score(logits[i], temp);
}

/* ------------------------------------------------------------------------ */
/* The four entry points of the layer library, mirrored on host memory so    */
/* that one suite can drive both implementations through one interface: the */
/* same argument order and struct layouts as the library's C ABI (declared   */
/* here independently), each composed from the functions above with no      */
/* arithmetic of its own. Return 0, or -1 for a NULL argument or m < 1. A    */
/* token whose header has a pick outside [0, n_routed) or a repeated pick    */
/* gets a zero routed output [device_route.rs, fn parse_header: picks in     */
/* range].                                                                   */
/* ------------------------------------------------------------------------ */

typedef struct {
  const void* base;
  uint64_t stride, gate_off, up_off, down_off;
} oexperts;

typedef struct {
  const uint16_t* gate_w;
  const float* bias;
  oexperts experts;
  const uint16_t *sh_w1, *sh_w3, *sh_w2;
  int32_t shared_kind; /* 0: bf16 sh_w*, 1: K-quant blocks in shared_q */
  oexperts shared_q;
} olayer;

EXPORT int moe_ref_route_select(const ocfg* c, const uint16_t* x, int32_t m, const uint16_t* gate_w,
                                const float* bias, float* logits, int32_t* header) {
  if (!c || !x || !gate_w || !bias || !header || m < 1) return -1;
  float* lg = logits ? logits : (float*)malloc(sizeof(float) * (size_t)m * c->n_routed);
  oracle_router_logits(x, m, gate_w, c->n_routed, c->dim, lg);
  oracle_select(c, lg, m, bias, header, NULL);
  if (!logits) free(lg);
  return 0;
}

/* One token's routed experts: their outputs ys [k][dim] and weights w in plan
 * order (ascending expert id), and the token's q8_1(x); 0 when the header's
 * picks are out of range or repeated. */
static int ref_token_experts(const ocfg* c, const uint16_t* xrow, const int32_t* hd, const oexperts* ex,
                             int8_t* xq, uint16_t* xd16, float* ys, float* w) {
  int k = c->topk, dim = c->dim, inter = c->inter;
  float* xf = (float*)malloc(sizeof(float) * dim);
  for (int i = 0; i < dim; ++i) xf[i] = oracle_bf16_to_f32(xrow[i]);
  oracle_q8_1(xf, dim, xq, xd16);
  free(xf);
  for (int r = 0; r < k; ++r) {
    if (hd[1 + r] < 0 || hd[1 + r] >= c->n_routed) return 0;
    for (int r2 = 0; r2 < r; ++r2)
      if (hd[1 + r2] == hd[1 + r]) return 0;
  }
  int ids[64];
  for (int r = 0; r < k; ++r) {
    ids[r] = hd[1 + r];
    uint32_t b = (uint32_t)hd[1 + k + r];
    memcpy(&w[r], &b, 4);
  }
  for (int a = 1; a < k; ++a) /* plan order: ascending expert id, weights with their picks */
    for (int b = a; b > 0 && ids[b] < ids[b - 1]; --b) {
      int ti = ids[b]; ids[b] = ids[b - 1]; ids[b - 1] = ti;
      float tw = w[b]; w[b] = w[b - 1]; w[b - 1] = tw;
    }
  float *g = (float*)malloc(sizeof(float) * inter), *u = (float*)malloc(sizeof(float) * inter);
  float* h = (float*)malloc(sizeof(float) * inter);
  int8_t* hq = (int8_t*)malloc(inter);
  uint16_t* hd16 = (uint16_t*)malloc(2 * (inter / 32));
  for (int r = 0; r < k; ++r) {
    const uint8_t* e = (const uint8_t*)ex->base + (uint64_t)ids[r] * ex->stride;
    oracle_expert(c, xq, xd16, e + ex->gate_off, e + ex->up_off, e + ex->down_off, g, u, h, hq, hd16,
                  ys + (size_t)r * dim, NULL, NULL, NULL);
  }
  free(g); free(u); free(h); free(hq); free(hd16);
  return 1;
}

EXPORT int moe_ref_experts_decode(const ocfg* c, const uint16_t* x, int32_t m, const int32_t* header,
                                  const oexperts* experts, float* y_routed) {
  if (!c || !x || !header || !experts || !experts->base || !y_routed || m < 1) return -1;
  int k = c->topk, dim = c->dim, hw = 1 + 3 * k;
  int8_t* xq = (int8_t*)malloc(dim);
  uint16_t* xd16 = (uint16_t*)malloc(2 * (dim / 32));
  float* ys = (float*)malloc(sizeof(float) * (size_t)k * dim);
  float w[64];
  for (int32_t t = 0; t < m; ++t) {
    float* yt = y_routed + (int64_t)t * dim;
    if (ref_token_experts(c, x + (int64_t)t * dim, header + (int64_t)t * hw, experts, xq, xd16, ys, w))
      oracle_combine(dim, k, ys, w, NULL, yt, NULL);
    else
      for (int i = 0; i < dim; ++i) yt[i] = 0.0f;
  }
  free(xq); free(xd16); free(ys);
  return 0;
}

/* Each token of a prefill batch is defined exactly as at m = 1. */
EXPORT int moe_ref_experts_prefill(const ocfg* c, const uint16_t* x, int32_t m, const int32_t* header,
                                   const oexperts* experts, float* y_routed) {
  return moe_ref_experts_decode(c, x, m, header, experts, y_routed);
}

EXPORT int moe_ref_layer_forward(const ocfg* c, const olayer* layer, const uint16_t* x, int32_t m,
                                 uint16_t* out_bf16, float* out_f32, int32_t* header) {
  if (!c || !layer || !x || !out_bf16 || m < 1) return -1;
  if (layer->shared_kind == 0 ? (!layer->sh_w1 || !layer->sh_w3 || !layer->sh_w2) : !layer->shared_q.base) return -1;
  int k = c->topk, dim = c->dim, inter = c->inter, hw = 1 + 3 * k;
  int32_t* hdr = header ? header : (int32_t*)malloc(sizeof(int32_t) * (size_t)m * hw);
  moe_ref_route_select(c, x, m, layer->gate_w, layer->bias, NULL, hdr);
  int8_t* xq = (int8_t*)malloc(dim);
  uint16_t* xd16 = (uint16_t*)malloc(2 * (dim / 32));
  float* ys = (float*)malloc(sizeof(float) * (size_t)k * dim);
  float* sd = (float*)malloc(sizeof(float) * dim);
  float* o32 = (float*)malloc(sizeof(float) * dim);
  float *sg = (float*)malloc(sizeof(float) * inter), *su = (float*)malloc(sizeof(float) * inter);
  float* sh32 = (float*)malloc(sizeof(float) * inter);
  uint16_t* sh = (uint16_t*)malloc(2 * inter);
  int8_t* hq = (int8_t*)malloc(inter);
  uint16_t* hd16 = (uint16_t*)malloc(2 * (inter / 32));
  float w[64];
  for (int32_t t = 0; t < m; ++t) {
    const uint16_t* xrow = x + (int64_t)t * dim;
    ref_token_experts(c, xrow, hdr + (int64_t)t * hw, &layer->experts, xq, xd16, ys, w);
    if (layer->shared_kind == 0) {
      oracle_shared(c, xrow, layer->sh_w1, layer->sh_w3, layer->sh_w2, sg, su, sh, sd);
    } else {   /* the K-quant shared expert: one more expert on the same q8_1(x) */
      const uint8_t* b = (const uint8_t*)layer->shared_q.base;
      oracle_expert(c, xq, xd16, b + layer->shared_q.gate_off, b + layer->shared_q.up_off,
                    b + layer->shared_q.down_off, sg, su, sh32, hq, hd16, sd, NULL, NULL, NULL);
    }
    /* the routed sum in plan order, then the shared output added after it */
    oracle_combine(dim, k, ys, w, sd, o32, out_bf16 + (int64_t)t * dim);
    if (out_f32) memcpy(out_f32 + (int64_t)t * dim, o32, sizeof(float) * dim);
  }
  free(xq); free(xd16); free(ys); free(sd); free(o32); free(sg); free(su); free(sh32); free(sh); free(hq); free(hd16);
  if (!header) free(hdr);
  return 0;
}
