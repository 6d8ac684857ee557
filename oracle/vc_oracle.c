/*
 * vc_oracle.c -- plain, slow CPU oracle for the VC-Attention hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header, table or constant generator
 * with the HIP library.
 *
 * Sources (web pages, cited by title and place):
 *   [VC]   "VC-Attention: Value Smoothing and Softmax Casting for Low-bit
 *          Attention" (arXiv 2609.15810).
 *   [OVC]  "Open-VC Attention: an open-source, error-tunable variant of
 *          VC-Attention" (machgen.ai blog).
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (no -ffast-math:
 * every fp32 operation here is an IEEE-754 operation in round-to-nearest-
 * even, denormals kept).  Floating point steps the GPU performs in fp32 are
 * written out one by one in fp32 (fmaf where the method folds a multiply-add,
 * plain * and / otherwise); sums the matrix cores accumulate are done here
 * in fp64.
 *
 * Readings where the pages leave a step open are stated at each function.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define EXPORT __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ */
/* bf16 <-> fp32                                                            */
/* ------------------------------------------------------------------------ */

static float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Round-to-nearest-even of an fp32 value to bf16 (finite inputs). */
static uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffff) ? 0x40 : 0));
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

EXPORT uint16_t vco_f32_to_bf16(float f) { return f32_to_bf16_rne(f); }

/* ------------------------------------------------------------------------ */
/* E4M3 (OCP E4M3FN: bias 7, no infinities, 0x7F/0xFF are NaN, max 448).    */
/* [VC] §3.3: a byte with exponent field e and mantissa field m encodes      */
/* 2^(e-7)(1+m/8); e = 0 holds the subnormals m * 2^-9.                     */
/* ------------------------------------------------------------------------ */

EXPORT double vco_e4m3_decode(uint8_t c) {
  int e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return (c & 0x80) ? -v : v;
}

static double g_e4m3_pos[127]; /* decoded values of codes 0..126 */
static double g_e4m3_all[256]; /* decoded values of all 256 bytes */
static int g_e4m3_init = 0;

static void e4m3_table_init(void) {
  if (g_e4m3_init) return;
  for (int c = 0; c < 256; ++c) g_e4m3_all[c] = vco_e4m3_decode((uint8_t)c);
  for (int c = 0; c < 127; ++c) g_e4m3_pos[c] = g_e4m3_all[c];
  g_e4m3_init = 1;
}

#define DEC(c) (g_e4m3_all[(uint8_t)(c)])

/*
 * Encode: the finite E4M3 code nearest to x, ties to the code with an even
 * mantissa (= even code), magnitudes beyond 448 saturating to 448 (the
 * nearest finite code).  The sign bit is x's sign bit.  Written as a search
 * over all 127 non-negative codes so that it is correct by inspection.
 * Reading: the pages fix the format and round-to-nearest-even but not the
 * handling of overflow; saturation is used (inputs here never exceed 448 by
 * more than an fp32 rounding).
 */
EXPORT uint8_t vco_e4m3_encode(float x) {
  e4m3_table_init();
  double a = fabs((double)x);
  int best = 0;
  double bd = fabs(a - g_e4m3_pos[0]);
  for (int c = 1; c < 127; ++c) {
    double d = fabs(a - g_e4m3_pos[c]);
    if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) {
      bd = d;
      best = c;
    }
  }
  return (uint8_t)(best | (signbit(x) ? 0x80 : 0));
}

EXPORT void vco_e4m3_encode_array(const float* x, int64_t n, uint8_t* codes) {
  for (int64_t i = 0; i < n; ++i) codes[i] = vco_e4m3_encode(x[i]);
}

/* ------------------------------------------------------------------------ */
/* ExpCast-FP8 code, [VC] §3.3 Eq. 7 and Fig. 2:                            */
/*   c = clip_[0,120]( Round( a*x + b ) ),  Round = round-half-even,         */
/* with a*x+b formed by one fp32 fused multiply-add.                         */
/* ------------------------------------------------------------------------ */

static int expcast_code_f32(float a, float x, float b) {
  float y = fmaf(a, x, b);
  float r = nearbyintf(y); /* default rounding mode: nearest-even */
  if (!(r > 0.0f)) return 0; /* also maps -inf to code 0 */
  if (r > 120.0f) return 120;
  return (int)r;
}

EXPORT void vco_expcast_codes(const float* x, const float* a, const float* b, int64_t n,
                              int32_t row_len, uint8_t* codes) {
  for (int64_t i = 0; i < n; ++i) {
    int64_t row = i / row_len;
    codes[i] = (uint8_t)expcast_code_f32(a[row], x[i], b[row]);
  }
}

/* Real-number closed form of Eq. 7 evaluated in fp64 for a log2-domain u. */
EXPORT int vco_expcast_code_u(double u, double beta) {
  double y = 8.0 * (u + 8.0) + 56.0 + beta;
  double r = nearbyint(y);
  if (!(r > 0.0)) return 0;
  if (r > 120.0) return 120;
  return (int)r;
}

/* ------------------------------------------------------------------------ */
/* Quantizers, [OVC] "Scheduling around ExpCast": Q and K take one scale per */
/* 128-token block, V one scale per head; X_q = s_X * Xhat ([VC] §3.1).      */
/* The pages leave the value of a scale open.  Readings:                     */
/*  - V (per head) and the V-Smooth residual (per channel): s = amax/448,    */
/*    codes E4M3(x * (448/amax)), both quotients rounded to fp32;            */
/*  - Q and K blocks: s = 2^e, the smallest power of two (e >= -127) with    */
/*    amax <= 448 * 2^e, codes E4M3(x * 2^-e) -- a scale a block-scaled      */
/*    matrix product applies exactly.  Q is first multiplied (fp32) by       */
/*    G = 8 fl(sm_scale * log2 e), the factor [OVC] folds into the code's     */
/*    multiply-add, so 8 * (log2-domain score) = s_Q s_K (Qhat . Khat).      */
/* A block of zeros takes s = 1.                                             */
/* ------------------------------------------------------------------------ */

static void scale_pair(float amax, float* s, float* inv) {
  if (amax > 0.0f) {
    *s = amax / 448.0f;
    *inv = 448.0f / amax;
  } else {
    *s = 1.0f;
    *inv = 1.0f;
  }
}

/* The power-of-two block exponent: smallest e >= -127 with amax <= 448*2^e. */
static int pow2_block_exp(float amax) {
  if (!(amax > 0.0f)) return 0;
  int e = ilogbf(amax) - 9; /* 448 * 2^(E-9) < 2^E <= amax: one step too low */
  if (e < -127) e = -127;
  while (amax > ldexpf(448.0f, e)) ++e;
  return e;
}

/*
 * One head, Q or K.  x: bf16 rows, row r at x + r*ld (D contiguous); pre is
 * the fp32 factor applied first (G for Q, 1 for K).
 * Out: codes [nblk*128][D] (rows >= S are zero), scale [nblk] = 2^e.
 */
EXPORT void vco_quantize_blocks_pow2(const uint16_t* x, int64_t ld, int32_t S, int32_t D, float pre,
                                     uint8_t* codes, float* scale) {
  int32_t nblk = (S + 127) / 128;
  for (int32_t j = 0; j < nblk; ++j) {
    int32_t r0 = j * 128, r1 = r0 + 128 < S ? r0 + 128 : S;
    float amax = 0.0f;
    for (int32_t r = r0; r < r1; ++r)
      for (int32_t d = 0; d < D; ++d) amax = fmaxf(amax, fabsf(bf16_to_f32(x[r * ld + d]) * pre));
    int e = pow2_block_exp(amax);
    scale[j] = ldexpf(1.0f, e);
    for (int32_t r = r0; r < j * 128 + 128; ++r)
      for (int32_t d = 0; d < D; ++d)
        codes[(int64_t)r * D + d] =
            (r < S) ? vco_e4m3_encode(ldexpf(bf16_to_f32(x[r * ld + d]) * pre, -e)) : 0;
  }
}

/* ------------------------------------------------------------------------ */
/* Preprocessing of Q and K ahead of the quantiser, [VC] §3.4 and App. B:   */
/* rotary embedding, the key channel mean (centring) and the QK Hadamard    */
/* rotation.  The pages leave their exact forms open.  Readings:            */
/*  - RoPE rotates the pairs (2i, 2i+1) of a row by the caller's angle for   */
/*    the token's position p: (a, b) -> (a c - b s, a s + b c), c, s =       */
/*    cos/sin[p][i], each product and difference rounded to fp32;            */
/*  - centring subtracts from every key the channel mean over the head's S   */
/*    keys (after RoPE): sums in 64-bit fixed point with 24 fraction bits    */
/*    (order independent), mean = fl32(sum / (S 2^24)) in fp64.  Any vector  */
/*    subtracted from all keys leaves each softmax row unchanged;            */
/*  - the rotation is the unnormalised Walsh-Hadamard transform over D       */
/*    (H H^T = D I, so scores grow by exactly D, which Q's pre-factor takes  */
/*    back), computed as radix-2 butterflies (a, b) -> (a + b, a - b) over    */
/*    strides 1, 2, ..., D/2 in that order, in fp32.                         */
/* ------------------------------------------------------------------------ */

static int64_t fx24(float v);  /* 64-bit fixed point, 24 fraction bits (k-means section) */

#define VCO_PREP_ROPE 1
#define VCO_PREP_HADAMARD 2
#define VCO_PREP_CENTER 4

static void rope_row(float* v, int32_t D, const float* c, const float* s) {
  for (int32_t i = 0; i < D / 2; ++i) {
    float a = v[2 * i], b = v[2 * i + 1];
    float ac = a * c[i], bs = b * s[i], as = a * s[i], bc = b * c[i];
    v[2 * i] = ac - bs;
    v[2 * i + 1] = as + bc;
  }
}

static void fwht_row(float* v, int32_t D) {
  for (int32_t h = 1; h < D; h <<= 1)
    for (int32_t i = 0; i < D; ++i)
      if (!(i & h)) {
        float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
}

/*
 * One head: x bf16 rows (row r at x + r*ld, token position r), flags as
 * above, cos/sin fp32 [S][D/2] (used with VCO_PREP_ROPE).  Out y fp32 [S][D]
 * in the order RoPE, centring, rotation; mean (if not NULL) gets the channel
 * mean used for centring.
 */
EXPORT void vco_prep_rows(const uint16_t* x, int64_t ld, int32_t S, int32_t D, int32_t flags, const float* cosb,
                          const float* sinb, float* y, float* mean) {
  for (int32_t r = 0; r < S; ++r) {
    float* v = y + (int64_t)r * D;
    for (int32_t d = 0; d < D; ++d) v[d] = bf16_to_f32(x[r * ld + d]);
    if (flags & VCO_PREP_ROPE) rope_row(v, D, cosb + (int64_t)r * (D / 2), sinb + (int64_t)r * (D / 2));
  }
  if (flags & VCO_PREP_CENTER) {
    for (int32_t d = 0; d < D; ++d) {
      int64_t sum = 0;
      for (int32_t r = 0; r < S; ++r) sum += fx24(y[(int64_t)r * D + d]);
      float c = (float)((double)sum / ((double)S * 16777216.0));
      if (mean) mean[d] = c;
      for (int32_t r = 0; r < S; ++r) y[(int64_t)r * D + d] -= c;
    }
  }
  if (flags & VCO_PREP_HADAMARD)
    for (int32_t r = 0; r < S; ++r) fwht_row(y + (int64_t)r * D, D);
}

/* Power-of-two block quantiser of fp32 rows y [S][D] (as vco_quantize_blocks_pow2, after pre). */
EXPORT void vco_quantize_f32_blocks_pow2(const float* y, int32_t S, int32_t D, float pre, uint8_t* codes,
                                         float* scale) {
  int32_t nblk = (S + 127) / 128;
  for (int32_t j = 0; j < nblk; ++j) {
    int32_t r0 = j * 128, r1 = r0 + 128 < S ? r0 + 128 : S;
    float amax = 0.0f;
    for (int32_t r = r0; r < r1; ++r)
      for (int32_t d = 0; d < D; ++d) amax = fmaxf(amax, fabsf(y[(int64_t)r * D + d] * pre));
    int e = pow2_block_exp(amax);
    scale[j] = ldexpf(1.0f, e);
    for (int32_t r = r0; r < j * 128 + 128; ++r)
      for (int32_t d = 0; d < D; ++d)
        codes[(int64_t)r * D + d] = (r < S) ? vco_e4m3_encode(ldexpf(y[(int64_t)r * D + d] * pre, -e)) : 0;
  }
}

/*
 * Per-head V (plain path).  Out: codes in key-contiguous order
 * codes_t[d][S_pad] (pad keys zero), one scale.
 */
EXPORT float vco_quantize_v_head(const uint16_t* x, int64_t ld, int32_t S, int32_t D,
                                 uint8_t* codes_t) {
  int32_t S_pad = (S + 127) / 128 * 128;
  float amax = 0.0f;
  for (int32_t r = 0; r < S; ++r)
    for (int32_t d = 0; d < D; ++d) amax = fmaxf(amax, fabsf(bf16_to_f32(x[r * ld + d])));
  float s, inv;
  scale_pair(amax, &s, &inv);
  for (int32_t d = 0; d < D; ++d)
    for (int32_t r = 0; r < S_pad; ++r)
      codes_t[(int64_t)d * S_pad + r] = (r < S) ? vco_e4m3_encode(bf16_to_f32(x[r * ld + d]) * inv) : 0;
  return s;
}

/* ------------------------------------------------------------------------ */
/* V residual repair, [OVC] "Why V residual repair": with one V scale per    */
/* head, token j leaves the residual r_j = V_j - s_V Vhat_j; the top rho*S  */
/* tokens by energy sum_c r_jc^2 become extra value rows (their residuals)  */
/* paired with copies of their keys, visited last, numerator only.          */
/* Readings: r = fl32(v - fl32(s_V dec(code))); the energy is summed in fp64 */
/* over c = 0 .. D-1 in order; ties in energy go to the lower index; the    */
/* selected indices are returned in ascending order; a residual row is      */
/* quantised in the head's own V scale, code = E4M3(fl32(r * 448/amax)), so */
/* the kernel's single epilogue multiply covers it too.                     */
/* ------------------------------------------------------------------------ */

typedef struct {
  double e;
  int32_t j;
} vco_energy_t;
static int cmp_energy_desc(const void* a, const void* b) {
  const vco_energy_t* x = (const vco_energy_t*)a;
  const vco_energy_t* y = (const vco_energy_t*)b;
  if (x->e > y->e) return -1;
  if (x->e < y->e) return 1;
  return (x->j > y->j) - (x->j < y->j);
}
static int cmp_i32(const void* a, const void* b) {
  int32_t i = *(const int32_t*)a, j = *(const int32_t*)b;
  return (i > j) - (i < j);
}

/* One head's residual energies (energy [S]) and the R selected indices (idx [R], ascending). */
EXPORT void vco_repair_select(const uint16_t* x, int64_t ld, int32_t S, int32_t D, int32_t R, int32_t* idx,
                              double* energy) {
  float amax = 0.0f;
  for (int32_t r = 0; r < S; ++r)
    for (int32_t d = 0; d < D; ++d) amax = fmaxf(amax, fabsf(bf16_to_f32(x[r * ld + d])));
  float s, inv;
  scale_pair(amax, &s, &inv);
  vco_energy_t* order = (vco_energy_t*)malloc(sizeof(vco_energy_t) * (size_t)S);
  for (int32_t j = 0; j < S; ++j) {
    double e = 0.0;
    for (int32_t d = 0; d < D; ++d) {
      float v = bf16_to_f32(x[j * ld + d]);
      float deq = s * (float)DEC(vco_e4m3_encode(v * inv));
      float r = v - deq;
      e += (double)r * (double)r;
    }
    energy[j] = e;
    order[j].e = e;
    order[j].j = j;
  }
  qsort(order, (size_t)S, sizeof(vco_energy_t), cmp_energy_desc);
  for (int32_t i = 0; i < R; ++i) idx[i] = order[i].j;
  qsort(idx, (size_t)R, sizeof(int32_t), cmp_i32);
  free(order);
}

/* Residual codes of the selected tokens, key-contiguous: r_codes_t [D][Rpad]
 * (Rpad = R rounded up to 128; pad keys zero). */
EXPORT void vco_repair_rows(const uint16_t* x, int64_t ld, int32_t S, int32_t D, const int32_t* idx, int32_t R,
                            uint8_t* r_codes_t) {
  float amax = 0.0f;
  for (int32_t r = 0; r < S; ++r)
    for (int32_t d = 0; d < D; ++d) amax = fmaxf(amax, fabsf(bf16_to_f32(x[r * ld + d])));
  float s, inv;
  scale_pair(amax, &s, &inv);
  int32_t Rpad = (R + 127) / 128 * 128;
  for (int32_t d = 0; d < D; ++d)
    for (int32_t i = 0; i < Rpad; ++i) {
      uint8_t c = 0;
      if (i < R) {
        float v = bf16_to_f32(x[(int64_t)idx[i] * ld + d]);
        float r = v - s * (float)DEC(vco_e4m3_encode(v * inv));
        c = vco_e4m3_encode(r * inv);
      }
      r_codes_t[(int64_t)d * Rpad + i] = c;
    }
}

/* ------------------------------------------------------------------------ */
/* V-Smooth grouping, [VC] §3.2 "Value-guided permutation" and "Unbalanced   */
/* clusters cost little": per (b,h) an online k-means over the value tokens  */
/* gives labels z; pi = argsort(z); K' = K[pi], V' = V[pi].                  */
/* Readings (the pages give no initialisation, precision or tie rule):       */
/*  - Lloyd iterations, Forgy initialisation: k distinct token indices from  */
/*    a partial Fisher-Yates shuffle driven by SplitMix64;                   */
/*  - squared distance up to the token's own norm, |c|^2 - 2 v.c, each dot    */
/*    product one fp32 fused-multiply-add chain over channels 0..D-1, ties   */
/*    to the lowest cluster index;                                           */
/*  - cluster sums in 64-bit fixed point with 24 fraction bits, so the sum   */
/*    does not depend on the order tokens are added; an empty cluster keeps  */
/*    its centroid;                                                          */
/*  - labels are those of the last assignment, centroids those after the    */
/*    last update;                                                           */
/*  - argsort is stable (ties keep token order).                             */
/* ------------------------------------------------------------------------ */

/* SplitMix64 (Steele, Lea and Flood, 2014), from its published definition. */
static uint64_t splitmix64_next(uint64_t* st) {
  uint64_t z = (*st += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* The first n outputs of a SplitMix64 stream started at state `seed`. */
EXPORT void vco_splitmix64_stream(uint64_t seed, int32_t n, uint64_t* out) {
  uint64_t st = seed;
  for (int32_t i = 0; i < n; ++i) out[i] = splitmix64_next(&st);
}

/* The k initial token indices for head (b, h) of a batch with H heads. */
EXPORT void vco_forgy_indices(uint64_t seed, int32_t b, int32_t h, int32_t H, int32_t S, int32_t k,
                              int32_t* idx) {
  int32_t* a = (int32_t*)malloc(sizeof(int32_t) * (size_t)S);
  for (int32_t i = 0; i < S; ++i) a[i] = i;
  uint64_t st = seed + 0x9E3779B97F4A7C15ull * (uint64_t)(1 + (int64_t)b * H + h);
  for (int32_t i = 0; i < k; ++i) {
    uint64_t r = splitmix64_next(&st);
    uint32_t j = (uint32_t)i + (uint32_t)(((r >> 32) * (uint64_t)(uint32_t)(S - i)) >> 32);
    int32_t t = a[i];
    a[i] = a[j];
    a[j] = t;
  }
  for (int32_t i = 0; i < k; ++i) idx[i] = a[i];
  free(a);
}

static int64_t fx24(float v) { return llrint((double)v * 16777216.0); }

static float fx24_mean(int64_t sum, int64_t n) {
  return (float)(((double)sum * (1.0 / 16777216.0)) / (double)n);
}

/* Squared-norm chain of one centroid. */
static float cnorm(const float* c, int32_t D) {
  float n = 0.0f;
  for (int32_t d = 0; d < D; ++d) n = fmaf(c[d], c[d], n);
  return n;
}

/*
 * One head.  v: bf16 rows at v + r*ld.  cent [k][D] fp32: initial centroids
 * on entry when warm != 0, else overwritten from the Forgy indices; final
 * centroids on exit.  labels [S].
 */
EXPORT void vco_kmeans(const uint16_t* v, int64_t ld, int32_t S, int32_t D, int32_t k, int32_t iters,
                       uint64_t seed, int32_t b, int32_t h, int32_t H, int32_t warm, float* cent,
                       int32_t* labels) {
  if (!warm) {
    int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    vco_forgy_indices(seed, b, h, H, S, k, idx);
    for (int32_t c = 0; c < k; ++c)
      for (int32_t d = 0; d < D; ++d) cent[c * D + d] = bf16_to_f32(v[(int64_t)idx[c] * ld + d]);
    free(idx);
  }
  float* nrm = (float*)malloc(sizeof(float) * (size_t)k);
  int64_t* sum = (int64_t*)malloc(sizeof(int64_t) * (size_t)k * D);
  int64_t* cnt = (int64_t*)malloc(sizeof(int64_t) * (size_t)k);
  for (int32_t it = 0; it < iters; ++it) {
    for (int32_t c = 0; c < k; ++c) nrm[c] = cnorm(cent + (int64_t)c * D, D);
    /* assignment: tokens are independent */
#pragma omp parallel for schedule(static)
    for (int32_t t = 0; t < S; ++t) {
      float vt[256];
      for (int32_t d = 0; d < D; ++d) vt[d] = bf16_to_f32(v[(int64_t)t * ld + d]);
      int32_t best = 0;
      float bd = 0.0f;
      for (int32_t c = 0; c < k; ++c) {
        const float* cc = cent + (int64_t)c * D;
        float dot = 0.0f;
        for (int32_t d = 0; d < D; ++d) dot = fmaf(vt[d], cc[d], dot);
        float dist = fmaf(-2.0f, dot, nrm[c]);
        if (c == 0 || dist < bd) {
          bd = dist;
          best = c;
        }
      }
      labels[t] = best;
    }
    /* update: member means */
    memset(sum, 0, sizeof(int64_t) * (size_t)k * D);
    memset(cnt, 0, sizeof(int64_t) * (size_t)k);
    for (int32_t t = 0; t < S; ++t) {
      int32_t c = labels[t];
      cnt[c] += 1;
      for (int32_t d = 0; d < D; ++d) sum[(int64_t)c * D + d] += fx24(bf16_to_f32(v[(int64_t)t * ld + d]));
    }
    for (int32_t c = 0; c < k; ++c)
      if (cnt[c] > 0)
        for (int32_t d = 0; d < D; ++d) cent[(int64_t)c * D + d] = fx24_mean(sum[(int64_t)c * D + d], cnt[c]);
  }
  free(nrm);
  free(sum);
  free(cnt);
}

/* pi = stable argsort of the labels (counting sort). */
EXPORT void vco_argsort_labels(const int32_t* labels, int32_t S, int32_t k, int32_t* perm) {
  int64_t* off = (int64_t*)calloc((size_t)k + 1, sizeof(int64_t));
  for (int32_t t = 0; t < S; ++t) off[labels[t] + 1] += 1;
  for (int32_t c = 0; c < k; ++c) off[c + 1] += off[c];
  for (int32_t t = 0; t < S; ++t) perm[off[labels[t]]++] = t;
  free(off);
}

/*
 * Block demeaning and residual quantisation, [VC] §3.2 Eq. 4 and Appendix B:
 * mu_j is the mean of block j of V' (B_v = 128 rows), stored as a 16-bit
 * vector; R_j = V'_j - 1 mu_j^T goes through the per-channel E4M3 value
 * quantiser; the means are stored divided by the per-channel value scale.
 * Readings: mu is bf16 (round-to-nearest-even of the fp32 mean); the tail
 * block averages over its valid rows; the scaled mean is kept in fp32;
 * K' is quantised per 128-row block in permuted order like K.
 *
 * Out (one head): mu_bf16 [nblk][D], mu_scaled [nblk][D], r_codes_t [D][S_pad]
 * (key-contiguous, pad zero), r_scale [D], k_codes [S_pad][D], k_scale [nblk].
 */
EXPORT void vco_smooth_apply(const uint16_t* k, int64_t ldk, const uint16_t* v, int64_t ldv, int32_t S,
                             int32_t D, const int32_t* perm, uint16_t* mu_bf16, float* mu_scaled,
                             uint8_t* r_codes_t, float* r_scale, uint8_t* k_codes, float* k_scale) {
  int32_t nblk = (S + 127) / 128, S_pad = nblk * 128;
  float* R = (float*)malloc(sizeof(float) * (size_t)S * D);
  float* amax = (float*)calloc((size_t)D, sizeof(float));
  for (int32_t j = 0; j < nblk; ++j) {
    int32_t r0 = j * 128, r1 = r0 + 128 < S ? r0 + 128 : S;
    for (int32_t d = 0; d < D; ++d) {
      int64_t s = 0;
      for (int32_t r = r0; r < r1; ++r) s += fx24(bf16_to_f32(v[(int64_t)perm[r] * ldv + d]));
      uint16_t mu = f32_to_bf16_rne(fx24_mean(s, r1 - r0));
      mu_bf16[(int64_t)j * D + d] = mu;
      float muf = bf16_to_f32(mu);
      for (int32_t r = r0; r < r1; ++r) {
        float x = bf16_to_f32(v[(int64_t)perm[r] * ldv + d]) - muf;
        R[(int64_t)r * D + d] = x;
        amax[d] = fmaxf(amax[d], fabsf(x));
      }
    }
  }
  for (int32_t d = 0; d < D; ++d) {
    float s, inv;
    scale_pair(amax[d], &s, &inv);
    r_scale[d] = s;
    for (int32_t r = 0; r < S_pad; ++r)
      r_codes_t[(int64_t)d * S_pad + r] = (r < S) ? vco_e4m3_encode(R[(int64_t)r * D + d] * inv) : 0;
    for (int32_t j = 0; j < nblk; ++j)
      mu_scaled[(int64_t)j * D + d] = bf16_to_f32(mu_bf16[(int64_t)j * D + d]) * inv;
  }
  /* K' = K[pi], quantised per block */
  uint16_t* kp = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)S * D);
  for (int32_t r = 0; r < S; ++r)
    for (int32_t d = 0; d < D; ++d) kp[(int64_t)r * D + d] = k[(int64_t)perm[r] * ldk + d];
  vco_quantize_blocks_pow2(kp, D, S, D, 1.0f, k_codes, k_scale);
  free(kp);
  free(R);
  free(amax);
}

/* ------------------------------------------------------------------------ */
/* Attention emulation, one query row at a time.                            */
/*  - online softmax recurrence: [VC] §3.1 Eq. 1;                            */
/*  - running maximum on the true score, every increase applied, and the    */
/*    scale folding into one fused multiply-add per score: [OVC]            */
/*    "Scheduling around ExpCast";                                          */
/*  - ExpCast code: [VC] §3.3 Eq. 7 (beta = -0.35, so the additive constant  */
/*    is 120 + beta = 119.65);                                              */
/*  - row sum over the same decoded codes: [OVC] "A consistent denominator"; */
/*  - mean restoration A <- aA + P R_q + r mu^T: [VC] §3.2 Eq. 6;           */
/*  - mid-window key order: [OVC] "Mid-window key traversal".               */
/* ------------------------------------------------------------------------ */

/* Visit order of the key blocks for query tile qt.  The kernel holds two    */
/* 128-row query tiles, 2p and 2p + 1, that share one pass over K/V ([OVC] */
/* "A warp-specialized pipeline"), so the mid-window start is taken past   */
/* the pair's diagonal: start = min((qt | 1) + window, nblk - 1), then     */
/* down to block 0, then the blocks after start ([OVC] "Mid-window key     */
/* traversal").                                                            */
EXPORT void vco_tile_order(int32_t qt, int32_t nblk, int32_t window, int32_t sequential, int32_t* order) {
  if (sequential) {
    for (int32_t i = 0; i < nblk; ++i) order[i] = i;
    return;
  }
  int32_t last = qt | 1; /* diagonal block of the pair's second tile */
  int32_t start = last + window < nblk - 1 ? last + window : nblk - 1;
  int32_t n = 0;
  for (int32_t t = start; t >= 0; --t) order[n++] = t;
  for (int32_t t = start + 1; t < nblk; ++t) order[n++] = t;
}

#define VCO_SEQUENTIAL 1
#define VCO_EXACT_EXP 2
/* 4-bit path: a tile whose maximum exceeds the running max M by at most
 * VCO_HEADROOM4 leaves M as it is (the headroom a path without ExpCast has,
 * [OVC] "Mid-window key traversal"); with an integer M this changes no
 * output (vco_attn4_emulate_rows) */
#define VCO_DEFER4 4
#define VCO_HEADROOM4 8.0f

/*
 * q_codes [S_pad][D] with q_scale [nblk] (query rows in token order),
 * k_codes [S_pad][D] with k_scale [nblk], v_codes_t [D][S_pad] with
 * v_scale [D], mu_scaled [nblk][D] or NULL for the plain path.
 * c1: the log2-domain score per unit of q_scale * k_scale * (Qhat.Khat):
 * fl(sm_scale * log2 e) for codes of the raw Q, 1/8 for Q carrying G.
 * rows: n query indices.  Out: out_f32 [n][D] (pre-rounding output, fp32)
 * and out_bf16 [n][D]; stats (may be NULL) [n][2] = {rescales, final max M}.
 */
EXPORT void vco_attn_emulate_rows(const uint8_t* q_codes, const float* q_scale, const uint8_t* k_codes,
                                  const float* k_scale, const uint8_t* v_codes_t, const float* v_scale,
                                  const float* mu_scaled, int32_t S, int32_t D, float c1,
                                  int32_t window, int32_t flags, const int32_t* rows, int32_t n,
                                  const uint8_t* rk_codes, const float* rk_scale, const uint8_t* rv_codes_t,
                                  int32_t R, float* out_f32, uint16_t* out_bf16, double* stats) {
  int32_t nblk = (S + 127) / 128, S_pad = nblk * 128;
  int32_t nrb = R > 0 ? (R + 127) / 128 : 0, R_pad = nrb * 128; /* repair tiles, visited last */
  double dq[256];
  e4m3_table_init();
#pragma omp parallel for schedule(dynamic, 1) private(dq)
  for (int32_t ri = 0; ri < n; ++ri) {
    int32_t i = rows[ri];
    int32_t qt = i / 128;
    int32_t* order = (int32_t*)malloc(sizeof(int32_t) * (size_t)nblk);
    vco_tile_order(qt, nblk, window, flags & VCO_SEQUENTIAL, order);
    double* A = (double*)calloc((size_t)D, sizeof(double));
    float acc[128];
    double l = 0.0;
    float M = -INFINITY;
    int32_t rescales = 0;
    float c2 = c1 * q_scale[qt];
    for (int32_t d = 0; d < D; ++d) dq[d] = DEC(q_codes[(int64_t)i * D + d]);
    for (int32_t oi = 0; oi < nblk + nrb; ++oi) {
      /* repair tiles ([OVC] "Why V residual repair"): their keys, residual
       * rows, scales and row count; numerator only */
      const int repair = oi >= nblk;
      int32_t t = repair ? oi - nblk : order[oi];
      int32_t lim = repair ? R : S;
      const uint8_t* kc = repair ? rk_codes : k_codes;
      const uint8_t* vct = repair ? rv_codes_t : v_codes_t;
      int32_t vld = repair ? R_pad : S_pad;
      int32_t k0 = t * 128, k1 = k0 + 128 < lim ? k0 + 128 : lim;
      float mxacc = -INFINITY;
      for (int32_t kk = k0; kk < k1; ++kk) {
        double s = 0.0; /* exact: FP8 x FP8 products summed over D <= 256 fit in fp64 */
        for (int32_t d = 0; d < D; ++d) s += dq[d] * DEC(kc[(int64_t)kk * D + d]);
        acc[kk - k0] = (float)s;
        mxacc = fmaxf(mxacc, acc[kk - k0]);
      }
      float g = c2 * (repair ? rk_scale[t] : k_scale[t]);
      float mx = g * mxacc;
      float Mn = fmaxf(M, mx);
      if (Mn > M) {
        double alpha = (M == -INFINITY) ? 0.0 : exp2((double)M - (double)Mn);
        for (int32_t d = 0; d < D; ++d) A[d] *= alpha;
        l *= alpha;
        if (M != -INFINITY) rescales += 1;
        M = Mn;
      }
      float a = 8.0f * g;
      float b = 119.65f - 8.0f * M;
      double r = 0.0;
      for (int32_t kk = k0; kk < k1; ++kk) {
        double w;
        if (flags & VCO_EXACT_EXP) {
          /* diagnostic: fp32 exponential then an E4M3 cast ([VC] Prop. 3.1 text) */
          float u = g * acc[kk - k0] - M;
          w = DEC(vco_e4m3_encode(exp2f(u + 8.0f)));
        } else {
          w = DEC(expcast_code_f32(a, acc[kk - k0], b));
        }
        if (w == 0.0) continue;
        r += w;
        for (int32_t d = 0; d < D; ++d) A[d] += w * DEC(vct[(int64_t)d * vld + kk]);
      }
      if (repair) continue; /* the denominator already counts these keys */
      if (mu_scaled)
        for (int32_t d = 0; d < D; ++d) A[d] += r * (double)mu_scaled[(int64_t)t * D + d];
      l += r;
    }
    for (int32_t d = 0; d < D; ++d) {
      float o = (float)((A[d] / l) * (double)v_scale[d]);
      out_f32[(int64_t)ri * D + d] = o;
      out_bf16[(int64_t)ri * D + d] = f32_to_bf16_rne(o);
    }
    if (stats) {
      stats[2 * ri] = rescales;
      stats[2 * ri + 1] = M;
    }
    free(A);
    free(order);
  }
}

/* ------------------------------------------------------------------------ */
/* 4-bit path: V-Smooth at 4 bits, no ExpCast ([VC] §4.1 "Implementation":  */
/* 4 bits with V-Smooth alone; [VC] §4.1 "Scope of ExpCast-FP8": P is kept  */
/* as a microscaled 4-bit format, no affine log-to-code map exists for it). */
/* The pages' format is NVFP4 (per-16 E4M3 scales); the format here is     */
/* OCP MXFP4, the one gfx950's matrix cores take: E2M1 elements, one E8M0    */
/* (power-of-two) scale per 32 elements.                                    */
/* Readings: the block scale is the smallest 2^e (e >= -127) with           */
/* amax <= 6 * 2^e (2^0 for a block of zeros), as for the FP8 Q/K blocks;   */
/* elements are E2M1 round-half-even of x * 2^-e (saturating at 6, never    */
/* reached with that scale); Q/K blocks are 32 channels of a row (Q first   */
/* multiplied by fl(sm_scale * log2 e), so scores come out in log2 units);  */
/* V (or V-Smooth's residual) and P blocks are 32 consecutive keys of a     */
/* 128-key tile, per channel and per query row; p = fl32(2^(s - M)) with    */
/* M the running max rounded up to an integer (log2 units; s - M is then   */
/* exact), every increase of that integer applied;                          */
/* the row sum adds the dequantised P; the block mean is restored per tile  */
/* as A += r mu ([VC] §3.2 Eq. 6).                                           */
/* ------------------------------------------------------------------------ */

/* E2M1 (OCP MX): sign, 2 exponent bits (bias 1), 1 mantissa bit. */
EXPORT double vco_e2m1_decode(uint8_t c) {
  const int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
  const double mag = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -mag : mag;
}

/* Nearest E2M1 value, ties to the even code (mantissa bit 0), magnitudes
 * above 6 saturating to 6; -0 for negative inputs that round to zero. */
EXPORT uint8_t vco_e2m1_encode(float y) {
  const double a = fabs((double)y);
  int best = 0;
  double bd = a; /* distance to code 0 */
  for (int c = 1; c < 8; ++c) {
    const double d = fabs(a - vco_e2m1_decode((uint8_t)c));
    if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) {
      bd = d;
      best = c;
    }
  }
  if (a > 6.0) best = 7;
  return (uint8_t)(best | (signbit(y) ? 8 : 0));
}

/* Smallest e >= -127 with amax <= 6 * 2^e; 0 for amax == 0. */
EXPORT int vco_mx_block_exp(float amax) {
  if (!(amax > 0.0f)) return 0;
  int e = -127;
  while ((double)amax > ldexp(6.0, e)) ++e;
  return e;
}

/* Rows of y (fp32 [S][D]) times pre, in blocks of 32 channels: codes [S][D]
 * (one E2M1 code per byte) and exponents [S][D/32]. */
EXPORT void vco_mxfp4_rows(const float* y, int32_t S, int32_t D, float pre, uint8_t* codes, int32_t* exps) {
  for (int32_t r = 0; r < S; ++r)
    for (int32_t b = 0; b < D / 32; ++b) {
      float amax = 0.0f;
      for (int32_t c = 32 * b; c < 32 * b + 32; ++c) amax = fmaxf(amax, fabsf(y[(int64_t)r * D + c] * pre));
      const int e = vco_mx_block_exp(amax);
      exps[(int64_t)r * (D / 32) + b] = e;
      for (int32_t c = 32 * b; c < 32 * b + 32; ++c)
        codes[(int64_t)r * D + c] = vco_e2m1_encode(ldexpf(y[(int64_t)r * D + c] * pre, -e));
    }
}

/* Columns of x (fp32 [S][D], rows = keys) in blocks of 32 keys per channel:
 * codes_t [D][S_pad], exps [D][S_pad/32]; keys >= S are code 0 and do not
 * enter the block maximum. */
EXPORT void vco_mxfp4_cols(const float* x, int32_t S, int32_t D, uint8_t* codes_t, int32_t* exps) {
  const int32_t S_pad = (S + 127) / 128 * 128, nb = S_pad / 32;
  for (int32_t d = 0; d < D; ++d)
    for (int32_t b = 0; b < nb; ++b) {
      float amax = 0.0f;
      for (int32_t k = 32 * b; k < 32 * b + 32 && k < S; ++k) amax = fmaxf(amax, fabsf(x[(int64_t)k * D + d]));
      const int e = vco_mx_block_exp(amax);
      exps[(int64_t)d * nb + b] = e;
      for (int32_t k = 32 * b; k < 32 * b + 32; ++k)
        codes_t[(int64_t)d * S_pad + k] = k < S ? vco_e2m1_encode(ldexpf(x[(int64_t)k * D + d], -e)) : 0;
    }
}

/*
 * 4-bit attention, one query row at a time (rows in token order).
 * The running max is kept as an integer M (log2 units): a rescale is then an
 * exact power of two, and moving M by an integer n moves each P block's
 * exponent by n and leaves its codes as they are.  So whether a rise is
 * applied at once or later (VCO_DEFER4) does not change the output, which is
 * what lets the kernel skip the rescale of most rises.
 * q_codes [S_pad][D] / q_exps [S_pad][D/32] (Q carrying fl(sm log2 e)),
 * k_codes, k_exps likewise, v_codes_t [D][S_pad] / v_exps [D][S_pad/32],
 * mu [nblk][D] fp32 block means or NULL (plain).  Key blocks in the order
 * of vco_tile_order.  Out: out_f32 [n][D], out_bf16 [n][D], stats [n][2] =
 * {rescales, final max} (may be NULL).
 */
EXPORT void vco_attn4_emulate_rows(const uint8_t* q_codes, const int32_t* q_exps, const uint8_t* k_codes,
                                   const int32_t* k_exps, const uint8_t* v_codes_t, const int32_t* v_exps,
                                   const float* mu, int32_t S, int32_t D, int32_t window, int32_t flags,
                                   const int32_t* rows, int32_t n, float* out_f32, uint16_t* out_bf16,
                                   double* stats) {
  const int32_t nblk = (S + 127) / 128, S_pad = nblk * 128, nb32 = S_pad / 32;
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t ri = 0; ri < n; ++ri) {
    const int32_t i = rows[ri];
    int32_t* order = (int32_t*)malloc(sizeof(int32_t) * (size_t)nblk);
    vco_tile_order(i / 128, nblk, window, flags & VCO_SEQUENTIAL, order);
    double* qd = (double*)malloc(sizeof(double) * (size_t)D);
    double* A = (double*)calloc((size_t)D, sizeof(double));
    for (int32_t d = 0; d < D; ++d)
      qd[d] = ldexp(vco_e2m1_decode(q_codes[(int64_t)i * D + d]), q_exps[(int64_t)i * (D / 32) + d / 32]);
    float acc[128], p[128];
    double l = 0.0;
    float M = -INFINITY;
    int32_t rescales = 0;
    for (int32_t oi = 0; oi < nblk; ++oi) {
      const int32_t t = order[oi], k0 = t * 128, k1 = k0 + 128 < S ? k0 + 128 : S;
      float mx = -INFINITY;
      for (int32_t kk = k0; kk < k1; ++kk) {
        double s = 0.0; /* exact for the operands' few significant bits */
        for (int32_t d = 0; d < D; ++d)
          s += qd[d] * ldexp(vco_e2m1_decode(k_codes[(int64_t)kk * D + d]), k_exps[(int64_t)kk * (D / 32) + d / 32]);
        acc[kk - k0] = (float)s;
        mx = fmaxf(mx, acc[kk - k0]);
      }
      const float Mn = fmaxf(M, ceilf(mx));
      const int defer = (flags & VCO_DEFER4) && M != -INFINITY && mx - M <= VCO_HEADROOM4;
      if (Mn > M && !defer) {
        if (M != -INFINITY) {
          const double alpha = exp2((double)M - (double)Mn);
          for (int32_t d = 0; d < D; ++d) A[d] *= alpha;
          l *= alpha;
          rescales += 1;
        }
        M = Mn;
      }
      for (int32_t kk = k0; kk < k1; ++kk) p[kk - k0] = (float)exp2((double)acc[kk - k0] - (double)M);
      double r = 0.0;
      for (int32_t b0 = k0; b0 < k1; b0 += 32) { /* P's blocks of 32 keys */
        const int32_t b1 = b0 + 32 < k1 ? b0 + 32 : k1;
        float amax = 0.0f;
        for (int32_t kk = b0; kk < b1; ++kk) amax = fmaxf(amax, p[kk - k0]);
        const int e = vco_mx_block_exp(amax);
        for (int32_t kk = b0; kk < b1; ++kk) {
          const double w = ldexp(vco_e2m1_decode(vco_e2m1_encode(ldexpf(p[kk - k0], -e))), e);
          if (w == 0.0) continue;
          r += w;
          for (int32_t d = 0; d < D; ++d)
            A[d] += w * ldexp(vco_e2m1_decode(v_codes_t[(int64_t)d * S_pad + kk]), v_exps[(int64_t)d * nb32 + kk / 32]);
        }
      }
      if (mu)
        for (int32_t d = 0; d < D; ++d) A[d] += r * (double)mu[(int64_t)t * D + d];
      l += r;
    }
    for (int32_t d = 0; d < D; ++d) {
      const float o = (float)(A[d] / l);
      out_f32[(int64_t)ri * D + d] = o;
      out_bf16[(int64_t)ri * D + d] = f32_to_bf16_rne(o);
    }
    if (stats) {
      stats[2 * ri] = rescales;
      stats[2 * ri + 1] = M;
    }
    free(A);
    free(qd);
    free(order);
  }
}
