/*
 * qemb_oracle.c -- plain, slow CPU oracle for row-wise quantized embeddings.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The product path
 * (the HIP library under int4_row_wise_amd/) never calls, links or includes
 * anything here, and this file includes nothing from it.
 *
 * What it computes, and where each step comes from:
 *
 *  - Row-wise uniform quantization with a per-row scale and bias, clipped
 *    either to the row's range or to thresholds found by a greedy search over
 *    the row's squared error ("Post-Training 4-bit Quantization on Embedding
 *    Tables", review page, sections "Proposed method" and "Main findings").
 *  - Scale and bias stored as binary16 (same page, "Proposed method": fp16
 *    storage of scale and bias; "Main findings": 13.28% of fp32 size at d=128).
 *  - Two 4-bit codes packed per byte (DQRM repository page, paragraph on the
 *    Android demo: INT4 vectors must be bit-packed into INT8 storage); 2-bit
 *    codes (one of the baselines' widths) four per byte, element i at bits
 *    2 (i mod 4) of byte i / 4.
 *  - Pooled embedding-bag lookup of sparse categorical ids ("Deep Learning
 *    Recommendation Model for Personalization and Recommendation Systems",
 *    review page, "Proposed method": embedding tables map sparse inputs to
 *    dense vectors), with sum or weighted-sum pooling over CSR bags.
 *  - Normalized l2 error of the quantized rows (Post-Training 4-bit page,
 *    "Proposed method": quantization error measured by a normalized l2 loss).
 *  - Codebook quantization: each row's values are mapped to 16 non-uniformly
 *    placed levels found by k-means clustering (same page, "Proposed method"
 *    and "Main findings": a k-means codebook gives the lowest l2 loss at
 *    18.8%-37.5% of the fp32 size, i.e. 4-bit codes plus 16 fp32 levels per
 *    row at d = 256 and d = 64).  The clustering is 1-D Lloyd iteration from
 *    the row's uniform grid, a fixed number of times (rules below).
 *  - Quantizer baselines the same page compares against ("Proposed method":
 *    ACIQ, histogram-based clipping, symmetric quantization; "Main
 *    findings": the greedy search beats them): symmetric uniform rows
 *    (y = s q, q in [-(2^(b-1) - 1), 2^(b-1) - 1]), percentile clipping of the
 *    row's values, and ACIQ's clipping for a Laplace prior, all stored in
 *    the same packed row format.
 *  - Dot interaction of the pooled embeddings ("Deep Learning Recommendation
 *    Model ..." review page, "Proposed method": explicit second-order
 *    interactions are dot products between the embedding vectors and the
 *    processed dense features, concatenated with those dense features).
 *    Per sample the dense vector and the T pooled vectors are the rows of a
 *    (T+1) x d matrix Z; the output is the dense vector followed by
 *    <z_i, z_j> for every pair 0 <= j < i <= T, row by row.
 *
 *  - Error-bounded lossy compression of the pooled embeddings that devices
 *    exchange ("Avancées dans les recommandations en Deep Learning",
 *    scisimple page, "Méthodes de Compression des Données" and "Stratégies
 *    de Compression Adaptative": a user-set maximum error, one per table):
 *    a uniform quantizer of bin width twice the bound, zigzag codes packed
 *    at each vector's bit width, vectors that cannot meet the bound stored
 *    verbatim.
 *
 * The pages give no formulas.  The numeric rules used here (binary32 RNE with
 * one rounding per written operation, no contraction, IEEE division, fp16
 * round-to-nearest-even, ties-to-even code rounding, the contiguous-halves
 * pairwise sum for the row error, the shrink-from-either-end greedy walk) are
 * readings of those passages; the project's design notes list each one.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp -shared
 *        -fPIC.  x86-64 SSE arithmetic has no excess precision.
 * OpenMP is used only across independent rows and bags with a static
 * schedule, so results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_OK 0
#define OR_INVALID -1
#define OR_PRECONDITION -5

#define OR_MAX_DIM 4096

/* ------------------------------------------------------------------ */
/* binary16 <-> binary32, written out from the IEEE-754 encodings.      */
/* ------------------------------------------------------------------ */

static uint32_t bits_of(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

static float float_of(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Round a binary32 value to the nearest binary16 value, ties to even. */
static uint16_t to_half(float f) {
  uint32_t u = bits_of(f);
  uint32_t sign = (u >> 16) & 0x8000u;
  uint32_t a = u & 0x7fffffffu;
  if (a >= 0x7f800000u) {              /* inf or nan */
    return (uint16_t)(sign | 0x7c00u | (a > 0x7f800000u ? 0x0200u : 0u));
  }
  int e = (int)(a >> 23);              /* biased binary32 exponent */
  uint32_t mant = a & 0x7fffffu;
  if (e >= 113) {                      /* |f| >= 2^-14: binary16 normal range */
    if (e > 142) return (uint16_t)(sign | 0x7c00u);  /* >= 2^16: overflow */
    uint32_t base = ((uint32_t)(e - 112) << 10) | (mant >> 13);
    uint32_t rem = mant & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (base & 1u))) base += 1u;
    if (base >= 0x7c00u) base = 0x7c00u;  /* rounded past the largest finite */
    return (uint16_t)(sign | base);
  }
  /* Below 2^-14: result is a binary16 subnormal (units of 2^-24) or zero.
     value = mant24 * 2^(e-150) = mant24 * 2^(e-126) units of 2^-24. */
  if (e == 0) return (uint16_t)sign;   /* binary32 subnormal: far below 2^-25 */
  int shift = 126 - e;                 /* >= 14 */
  if (shift > 24) return (uint16_t)sign;
  uint32_t mant24 = mant | 0x800000u;
  uint32_t q = mant24 >> shift;
  uint32_t rem = mant24 & ((1u << shift) - 1u);
  uint32_t half = 1u << (shift - 1);
  if (rem > half || (rem == half && (q & 1u))) q += 1u;
  return (uint16_t)(sign | q);
}

/* Exact binary16 -> binary32. */
static float from_half(uint16_t h) {
  uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
  uint32_t E = ((uint32_t)h >> 10) & 0x1fu;
  uint32_t m = (uint32_t)h & 0x3ffu;
  if (E == 0) {
    float v = ldexpf((float)m, -24);   /* exact: m < 2^10 */
    return sign ? -v : v;
  }
  if (E == 31) return float_of(sign | 0x7f800000u | (m << 13));
  return float_of(sign | ((E + 112u) << 23) | (m << 13));
}

/* ------------------------------------------------------------------ */
/* Row layout                                                          */
/* ------------------------------------------------------------------ */

/* Code bytes of one row: two 4-bit codes per byte, or one 8-bit code. */
static int64_t code_bytes(int dim, int bits) {
  return ((int64_t)dim * bits + 7) / 8;
}

/* Row stride: codes, fp16 scale, fp16 bias, zero padding to 16 bytes. */
int64_t oracle_row_stride(int dim, int bits) {
  if (dim < 1 || (bits != 2 && bits != 4 && bits != 8)) return -1;
  int64_t raw = code_bytes(dim, bits) + 4;
  return (raw + 15) / 16 * 16;
}

/* ------------------------------------------------------------------ */
/* One row: range, parameters, codes, dequantized values, error.       */
/* ------------------------------------------------------------------ */

/* Row range (min and max), with -0 folded to +0 by adding +0. */
static void row_range(const float* x, int d, float* lo, float* hi) {
  float mn = x[0], mx = x[0];
  for (int i = 1; i < d; ++i) {
    if (x[i] < mn) mn = x[i];
    if (x[i] > mx) mx = x[i];
  }
  *lo = mn + 0.0f;
  *hi = mx + 0.0f;
}

/* Parameters for the clipping window [lo, hi]: the scale is the window over
   Q = 2^bits - 1 steps and the bias is the window's low end, both rounded to
   binary16; the codes are computed against the stored (rounded) values. */
typedef struct {
  uint16_t s16, b16;
  float sf, bf;
} params_t;

static params_t make_params(float lo, float hi, int Q) {
  params_t p;
  float s = (hi - lo) / (float)Q;
  if (!(s > 0.0f)) s = 0.0f;
  p.s16 = to_half(s);
  p.b16 = to_half(lo);
  p.sf = from_half(p.s16);
  p.bf = from_half(p.b16);
  return p;
}

/* Integer code of one element: round-half-even of (x - bias) * (1/scale),
   clamped to [0, Q]; every code is 0 when the stored scale is 0. */
static int code_of(float x, params_t p, float r, int Q) {
  if (p.sf == 0.0f) return 0;
  float t = (x - p.bf) * r;
  float q = rintf(t);
  if (q < 0.0f) q = 0.0f;
  if (q > (float)Q) q = (float)Q;
  return (int)q;
}

/* Dequantized value of code q: scale * q + bias with a single rounding. */
static float dequant_value(float sf, float bf, int q) {
  return fmaf(sf, (float)q, bf);
}

/* Pairwise sum over contiguous halves of a power-of-two length n. */
static float pairwise_sum(const float* u, int n) {
  if (n == 1) return u[0];
  int h = n / 2;
  return pairwise_sum(u, h) + pairwise_sum(u + h, h);
}

static int next_pow2(int d) {
  int n = 1;
  while (n < d) n <<= 1;
  return n;
}

/* Sum of squared errors of the row encoded with window [lo, hi]. */
static float window_sse(const float* x, int d, float lo, float hi, int Q) {
  float u[OR_MAX_DIM];
  int n = next_pow2(d);
  params_t p = make_params(lo, hi, Q);
  float r = (p.sf == 0.0f) ? 0.0f : 1.0f / p.sf;
  for (int i = 0; i < d; ++i) {
    int q = code_of(x[i], p, r, Q);
    float e = x[i] - dequant_value(p.sf, p.bf, q);
    u[i] = e * e;
  }
  for (int i = d; i < n; ++i) u[i] = 0.0f;
  return pairwise_sum(u, n);
}

/* Greedy clip search.  The window starts at the row's range and moves one
   step of width (max - min) / n_bins at a time, from whichever end gives the
   lower squared error (ties move the high end); after n_steps moves, the
   window with the lowest error seen (strictly lower replaces) is kept. */
static void greedy_window(const float* x, int d, int Q, int n_bins, int n_steps,
                          float* lo_out, float* hi_out, int* bi, int* bj) {
  float xmin, xmax;
  row_range(x, d, &xmin, &xmax);
  *lo_out = xmin;
  *hi_out = xmax;
  *bi = 0;
  *bj = 0;
  if (xmax == xmin) return;
  float delta = (xmax - xmin) / (float)n_bins;
  int i = 0, j = 0;
  float best = window_sse(x, d, xmin, xmax, Q);
  int best_i = 0, best_j = 0;
  for (int step = 0; step < n_steps; ++step) {
    float lo_next = fmaf((float)(i + 1), delta, xmin) + 0.0f;
    float lo_cur = fmaf((float)i, delta, xmin) + 0.0f;
    float hi_cur = fmaf(-(float)j, delta, xmax) + 0.0f;
    float hi_next = fmaf(-(float)(j + 1), delta, xmax) + 0.0f;
    float la = window_sse(x, d, lo_next, hi_cur, Q);  /* raise the low end */
    float lb = window_sse(x, d, lo_cur, hi_next, Q);  /* lower the high end */
    float l;
    if (la < lb) {
      i += 1;
      l = la;
    } else {
      j += 1;
      l = lb;
    }
    if (l < best) {
      best = l;
      best_i = i;
      best_j = j;
    }
  }
  *lo_out = fmaf((float)best_i, delta, xmin) + 0.0f;
  *hi_out = fmaf(-(float)best_j, delta, xmax) + 0.0f;
  *bi = best_i;
  *bj = best_j;
}

/* Code i of a row: 8 / bits codes per byte, element i in bits
   [bits * (i mod (8 / bits)), ...) of byte i / (8 / bits) -- for 4-bit codes
   the even element in the low nibble. */
static void put_code(uint8_t* row, int i, int bits, int q) {
  int per = 8 / bits;
  row[i / per] = (uint8_t)(row[i / per] | (q << (bits * (i % per))));
}

/* Encode one row into its packed form at window [lo, hi]. */
static void encode_row(const float* x, int d, int bits, float lo, float hi,
                       uint8_t* row, int64_t stride) {
  int Q = (1 << bits) - 1;
  params_t p = make_params(lo, hi, Q);
  float r = (p.sf == 0.0f) ? 0.0f : 1.0f / p.sf;
  int64_t C = code_bytes(d, bits);
  memset(row, 0, (size_t)stride);
  for (int i = 0; i < d; ++i) put_code(row, i, bits, code_of(x[i], p, r, Q));
  row[C + 0] = (uint8_t)(p.s16 & 0xff);
  row[C + 1] = (uint8_t)(p.s16 >> 8);
  row[C + 2] = (uint8_t)(p.b16 & 0xff);
  row[C + 3] = (uint8_t)(p.b16 >> 8);
}

/* Read back code i and the parameters of a packed row. */
static int row_code(const uint8_t* row, int i, int bits) {
  int per = 8 / bits;
  return (row[i / per] >> (bits * (i % per))) & ((1 << bits) - 1);
}

static void row_params(const uint8_t* row, int d, int bits, float* sf, float* bf) {
  int64_t C = code_bytes(d, bits);
  uint16_t s16 = (uint16_t)(row[C] | (row[C + 1] << 8));
  uint16_t b16 = (uint16_t)(row[C + 2] | (row[C + 3] << 8));
  *sf = from_half(s16);
  *bf = from_half(b16);
}

static int row_precondition_ok(const float* x, int d) {
  for (int i = 0; i < d; ++i) {
    if (!isfinite(x[i]) || fabsf(x[i]) > 65504.0f) return 0;
  }
  return 1;
}

/* ------------------------------------------------------------------ */
/* Exported entry points (host pointers)                               */
/* ------------------------------------------------------------------ */

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* Element-wise binary32 -> binary16 bits, for the conversion check. */
void oracle_f32_to_f16(const float* in, uint16_t* out, int64_t n) {
  for (int64_t k = 0; k < n; ++k) out[k] = to_half(in[k]);
}

void oracle_f16_to_f32(const uint16_t* in, float* out, int64_t n) {
  for (int64_t k = 0; k < n; ++k) out[k] = from_half(in[k]);
}

/* clip_mode 0 = row range, 1 = greedy search.  best_ij (nullable) receives
   the greedy window indices (i, j) per row.  Returns OR_PRECONDITION if any
   value is non-finite or beyond the binary16 range. */
int oracle_quantize_rowwise(const float* x, int64_t rows, int dim, int bits,
                            int clip_mode, int n_bins, int n_steps,
                            uint8_t* packed, int32_t* best_ij) {
  if (rows < 0 || dim < 1 || dim > OR_MAX_DIM || (bits != 2 && bits != 4 && bits != 8)) return OR_INVALID;
  if (clip_mode != 0 && clip_mode != 1) return OR_INVALID;
  if (clip_mode == 1 && (n_bins < 1 || n_steps < 0 || n_steps >= n_bins)) return OR_INVALID;
  int64_t stride = oracle_row_stride(dim, bits);
  int Q = (1 << bits) - 1;
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t r = 0; r < rows; ++r) {
    const float* xr = x + r * (int64_t)dim;
    if (!row_precondition_ok(xr, dim)) {
      bad = 1;
      continue;
    }
    float lo, hi;
    int bi = 0, bj = 0;
    if (clip_mode == 0) {
      row_range(xr, dim, &lo, &hi);
    } else {
      greedy_window(xr, dim, Q, n_bins, n_steps, &lo, &hi, &bi, &bj);
    }
    if (best_ij) {
      best_ij[2 * r] = bi;
      best_ij[2 * r + 1] = bj;
    }
    encode_row(xr, dim, bits, lo, hi, packed + r * stride, stride);
  }
  return bad ? OR_PRECONDITION : OR_OK;
}

/* ------------------------------------------------------------------ */
/* Quantizer baselines (same packed rows).                              */
/* ------------------------------------------------------------------ */

#define OR_BASE_SYMMETRIC 0
#define OR_BASE_PERCENTILE 1
#define OR_BASE_ACIQ 2

/* ACIQ's clip ratio for M-bit codes and a Laplace(b) prior: the expected
   squared error 2 b^2 exp(-a/b) (clipped tails) + a^2 / (3 4^M) (rounding in
   2^M bins over [-a, a]) is smallest where (a/b) exp(a/b) = 3 4^M, i.e.
   a/b = W(3 4^M) (Lambert W), solved here by Newton's method in binary64. */
double oracle_aciq_ratio(int bits) {
  double c = 3.0 * ldexp(1.0, 2 * bits);
  double t = log(c) - log(log(c));
  for (int it = 0; it < 100; ++it) {
    double e = exp(t);
    double step = (t * e - c) / (e * (t + 1.0));
    t -= step;
    if (fabs(step) <= 1e-16 * t) break;
  }
  return t;
}

/* q-quantile of ascending values v[0..d-1], linear between order statistics:
   h = (d - 1) q, i = floor(h), v[i] + (h - i)(v[i+1] - v[i]) in binary32 with
   one rounding for the last multiply-add. */
static float quantile_sorted(const float* v, int d, float q) {
  float h = (float)(d - 1) * q;
  int i = (int)floorf(h);
  if (i >= d - 1) return v[d - 1];
  float f = h - (float)i;
  return fmaf(f, v[i + 1] - v[i], v[i]);
}

/* Percentile clipping: the window is the row's (1 - p) and p quantiles. */
static void percentile_window(const float* x, int d, float p, float* lo, float* hi) {
  float v[OR_MAX_DIM];
  for (int i = 0; i < d; ++i) {
    float t = x[i];
    int j = i;
    while (j > 0 && v[j - 1] > t) {
      v[j] = v[j - 1];
      --j;
    }
    v[j] = t;
  }
  *lo = quantile_sorted(v, d, 1.0f - p) + 0.0f;
  *hi = quantile_sorted(v, d, p) + 0.0f;
}

/* ACIQ clipping: mean mu and mean absolute deviation b of the row (each a
   pairwise sum of the row padded with +0 to a power of two, divided by d),
   window [mu - a, mu + a] with a = W(3 4^M) b, kept inside the row range. */
static void aciq_window(const float* x, int d, int bits, float* lo, float* hi) {
  float u[OR_MAX_DIM];
  float mn, mx;
  row_range(x, d, &mn, &mx);
  int n = next_pow2(d);
  for (int i = 0; i < n; ++i) u[i] = i < d ? x[i] : 0.0f;
  float mu = pairwise_sum(u, n) / (float)d;
  for (int i = 0; i < n; ++i) u[i] = i < d ? fabsf(x[i] - mu) : 0.0f;
  float b = pairwise_sum(u, n) / (float)d;
  float a = (float)oracle_aciq_ratio(bits) * b;
  float l = mu - a, h = mu + a;
  *lo = (l > mn ? l : mn) + 0.0f;
  *hi = (h < mx ? h : mx) + 0.0f;
}

/* Symmetric uniform row: s = max|x| / (2^(b-1) - 1) stored in binary16 (at
   most 65504 / 2^(b-1), so that the bias stays finite), q = rint(x / s)
   (times the reciprocal of the stored scale) clamped to [-(2^(b-1) - 1),
   2^(b-1) - 1]; stored as code q + 2^(b-1) with bias -2^(b-1) s (exact), so
   the unchanged decode fmaf(s, code, bias) gives s q exactly. */
static void encode_symmetric(const float* x, int d, int bits, uint8_t* row, int64_t stride) {
  int H = 1 << (bits - 1), Qs = H - 1;
  float m = 0.0f;
  for (int i = 0; i < d; ++i) {
    float a = fabsf(x[i]);
    if (a > m) m = a;
  }
  float s = m / (float)Qs;
  uint16_t s16 = to_half(s);
  float sf = from_half(s16);
  float smax = 65504.0f / (float)H;
  if (sf > smax) {
    s16 = to_half(smax);
    sf = smax;
  }
  uint16_t b16 = to_half(-(float)H * sf);
  float r = sf == 0.0f ? 0.0f : 1.0f / sf;
  int64_t C = code_bytes(d, bits);
  memset(row, 0, (size_t)stride);
  for (int i = 0; i < d; ++i) {
    float q = sf == 0.0f ? 0.0f : rintf(x[i] * r);
    if (q < -(float)Qs) q = -(float)Qs;
    if (q > (float)Qs) q = (float)Qs;
    put_code(row, i, bits, (int)q + H);
  }
  row[C + 0] = (uint8_t)(s16 & 0xff);
  row[C + 1] = (uint8_t)(s16 >> 8);
  row[C + 2] = (uint8_t)(b16 & 0xff);
  row[C + 3] = (uint8_t)(b16 >> 8);
}

/* The window a baseline picks for one row (symmetric: [-max|x|, max|x|]). */
int oracle_baseline_window(const float* x, int dim, int bits, int method, float param,
                           float* lo_hi) {
  if (dim < 1 || dim > OR_MAX_DIM || (bits != 2 && bits != 4 && bits != 8)) return OR_INVALID;
  float lo, hi;
  if (method == OR_BASE_SYMMETRIC) {
    float m = 0.0f;
    for (int i = 0; i < dim; ++i) m = fabsf(x[i]) > m ? fabsf(x[i]) : m;
    lo = -m;
    hi = m;
  } else if (method == OR_BASE_PERCENTILE) {
    if (!(param >= 0.5f && param <= 1.0f)) return OR_INVALID;
    percentile_window(x, dim, param, &lo, &hi);
  } else if (method == OR_BASE_ACIQ) {
    aciq_window(x, dim, bits, &lo, &hi);
  } else {
    return OR_INVALID;
  }
  lo_hi[0] = lo;
  lo_hi[1] = hi;
  return OR_OK;
}

/* method: OR_BASE_SYMMETRIC, OR_BASE_PERCENTILE (param = p in [0.5, 1]) or
   OR_BASE_ACIQ; rows in the packed format of oracle_quantize_rowwise. */
int oracle_quantize_baseline(const float* x, int64_t rows, int dim, int bits, int method,
                             float param, uint8_t* packed) {
  if (rows < 0 || dim < 1 || dim > OR_MAX_DIM || (bits != 2 && bits != 4 && bits != 8)) return OR_INVALID;
  if (method < OR_BASE_SYMMETRIC || method > OR_BASE_ACIQ) return OR_INVALID;
  if (method == OR_BASE_PERCENTILE && !(param >= 0.5f && param <= 1.0f)) return OR_INVALID;
  int64_t stride = oracle_row_stride(dim, bits);
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t r = 0; r < rows; ++r) {
    const float* xr = x + r * (int64_t)dim;
    if (!row_precondition_ok(xr, dim)) {
      bad = 1;
      continue;
    }
    uint8_t* row = packed + r * stride;
    if (method == OR_BASE_SYMMETRIC) {
      encode_symmetric(xr, dim, bits, row, stride);
    } else {
      float lo, hi;
      if (method == OR_BASE_PERCENTILE) {
        percentile_window(xr, dim, param, &lo, &hi);
      } else {
        aciq_window(xr, dim, bits, &lo, &hi);
      }
      encode_row(xr, dim, bits, lo, hi, row, stride);
    }
  }
  return bad ? OR_PRECONDITION : OR_OK;
}

/* Squared error of one row at greedy window (i, j), for lattice checks. */
float oracle_window_sse(const float* x, int dim, int bits, int n_bins, int i, int j) {
  float xmin, xmax;
  row_range(x, dim, &xmin, &xmax);
  float delta = (xmax - xmin) / (float)n_bins;
  float lo = fmaf((float)i, delta, xmin) + 0.0f;
  float hi = fmaf(-(float)j, delta, xmax) + 0.0f;
  return window_sse(x, dim, lo, hi, (1 << bits) - 1);
}

/* Squared error of a packed row against its source row, in the same order. */
float oracle_row_sse(const float* x, const uint8_t* row, int dim, int bits) {
  float u[OR_MAX_DIM];
  int n = next_pow2(dim);
  float sf, bf;
  row_params(row, dim, bits, &sf, &bf);
  for (int i = 0; i < dim; ++i) {
    float e = x[i] - dequant_value(sf, bf, row_code(row, i, bits));
    u[i] = e * e;
  }
  for (int i = dim; i < n; ++i) u[i] = 0.0f;
  return pairwise_sum(u, n);
}

int oracle_dequantize(const uint8_t* packed, int64_t rows, int dim, int bits, float* y) {
  if (rows < 0 || dim < 1 || dim > OR_MAX_DIM || (bits != 2 && bits != 4 && bits != 8)) return OR_INVALID;
  int64_t stride = oracle_row_stride(dim, bits);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const uint8_t* row = packed + r * stride;
    float sf, bf;
    row_params(row, dim, bits, &sf, &bf);
    for (int i = 0; i < dim; ++i) y[r * dim + i] = dequant_value(sf, bf, row_code(row, i, bits));
  }
  return OR_OK;
}

/* ------------------------------------------------------------------ */
/* Codebook rows: 16 fp32 levels per row (k-means), 4-bit codes.        */
/* ------------------------------------------------------------------ */

#define OR_CB_K 16
#define OR_FMT_CB 16 /* row format tag of codebook rows (4 and 8: uniform rows) */

/* Row layout: levels c_0..c_15 (fp32, little-endian, 64 bytes) | codes
   (ceil(d/2) bytes, element 2k in the low nibble of byte k) | zero padding
   to a multiple of 16 bytes. */
int64_t oracle_codebook_row_stride(int dim) {
  if (dim < 1) return 0;
  int64_t c = ((int64_t)dim + 1) / 2;
  return 16 * ((64 + c + 15) / 16);
}

/* Index of the level nearest to x: the smallest k minimizing |x - c_k|
   (each distance one fp32 subtraction, exact absolute value). */
static int nearest_level(float x, const float* c) {
  int best = 0;
  float bd = fabsf(x - c[0]);
  for (int k = 1; k < OR_CB_K; ++k) {
    float dk = fabsf(x - c[k]);
    if (dk < bd) {
      bd = dk;
      best = k;
    }
  }
  return best;
}

/* k-means codebook of one row.
   1. lo, hi: the row range (as for range quantization, -0 canonicalized).
   2. Start from the uniform grid c_k = fmaf(k, (hi - lo)/15, lo) + 0.
   3. n_iter times: assign every element to its nearest level (with the
      levels at the start of the iteration); then every level with at least
      one member becomes the mean of its members -- their sum taken as the
      contiguous-halves pairwise sum of the row-length vector holding the
      members' values and +0 elsewhere (padded with +0 to a power of two),
      divided by the member count (IEEE division), + 0; a level without
      members keeps its value.
   4. Codes: the nearest level to each element with the final levels. */
static void codebook_row(const float* x, int d, int n_iter, float* c, int* code) {
  float lo, hi;
  row_range(x, d, &lo, &hi);
  float delta = (hi - lo) / (float)(OR_CB_K - 1);
  for (int k = 0; k < OR_CB_K; ++k) c[k] = fmaf((float)k, delta, lo) + 0.0f;
  int n = next_pow2(d);
  float v[OR_MAX_DIM];
  for (int it = 0; it < n_iter; ++it) {
    for (int i = 0; i < d; ++i) code[i] = nearest_level(x[i], c);
    float next[OR_CB_K];
    for (int k = 0; k < OR_CB_K; ++k) {
      int count = 0;
      for (int i = 0; i < d; ++i) {
        v[i] = code[i] == k ? x[i] : 0.0f;
        count += code[i] == k;
      }
      for (int i = d; i < n; ++i) v[i] = 0.0f;
      next[k] = count > 0 ? pairwise_sum(v, n) / (float)count + 0.0f : c[k];
    }
    for (int k = 0; k < OR_CB_K; ++k) c[k] = next[k];
  }
  for (int i = 0; i < d; ++i) code[i] = nearest_level(x[i], c);
}

static void put_f32(uint8_t* p, float f) {
  uint32_t u = bits_of(f);
  for (int b = 0; b < 4; ++b) p[b] = (uint8_t)(u >> (8 * b));
}

static float get_f32(const uint8_t* p) {
  uint32_t u = (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
  return float_of(u);
}

int oracle_quantize_codebook(const float* x, int64_t rows, int dim, int n_iter, uint8_t* packed) {
  if (rows < 0 || dim < 1 || dim > OR_MAX_DIM || n_iter < 0) return OR_INVALID;
  int64_t stride = oracle_codebook_row_stride(dim);
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t r = 0; r < rows; ++r) {
    const float* xr = x + r * (int64_t)dim;
    if (!row_precondition_ok(xr, dim)) {
      bad |= 1;
      continue;
    }
    float c[OR_CB_K];
    int code[OR_MAX_DIM];
    codebook_row(xr, dim, n_iter, c, code);
    uint8_t* row = packed + r * stride;
    memset(row, 0, (size_t)stride);
    for (int k = 0; k < OR_CB_K; ++k) put_f32(row + 4 * k, c[k]);
    for (int i = 0; i < dim; ++i) row[64 + i / 2] |= (uint8_t)(code[i] << (4 * (i & 1)));
  }
  return bad ? OR_PRECONDITION : OR_OK;
}

/* Decoded fp32 values of a packed row of format fmt (4, 8: uniform rows;
   OR_FMT_CB: codebook rows). */
static void decode_row(const uint8_t* row, int d, int fmt, float* y) {
  if (fmt == OR_FMT_CB) {
    for (int i = 0; i < d; ++i) y[i] = get_f32(row + 4 * ((row[64 + i / 2] >> (4 * (i & 1))) & 15));
  } else {
    float sf, bf;
    row_params(row, d, fmt, &sf, &bf);
    for (int i = 0; i < d; ++i) y[i] = dequant_value(sf, bf, row_code(row, i, fmt));
  }
}

static int64_t fmt_stride(int dim, int fmt) {
  return fmt == OR_FMT_CB ? oracle_codebook_row_stride(dim) : oracle_row_stride(dim, fmt);
}

int oracle_dequantize_codebook(const uint8_t* packed, int64_t rows, int dim, float* y) {
  if (rows < 0 || dim < 1 || dim > OR_MAX_DIM) return OR_INVALID;
  int64_t stride = oracle_codebook_row_stride(dim);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) decode_row(packed + r * stride, dim, OR_FMT_CB, y + r * (int64_t)dim);
  return OR_OK;
}

static int64_t load_index(const void* p, int64_t k, int index_type) {
  return index_type == 0 ? (int64_t)((const int32_t*)p)[k] : ((const int64_t*)p)[k];
}

/* Pooled lookup over CSR bags.  Bag g = t * B + b covers positions
   [offsets[g], offsets[g+1]) of indices/weights; its terms are
   w_p * dequant(row table_offsets[t] + indices[p]), summed in binary64 in
   position order (w_p = 1 for plain sum).  out is [B][T][dim] (binary64);
   abs_terms (nullable) gets the sum of |w_p * y| per output element.
   Invalid data never faults: an index outside the table, or a table whose
   row range lies outside [0, total_rows), skips that term; a bag whose
   offsets decrease or leave [0, nnz] is empty.  Each such event adds one to
   *err_count (nullable). */
static int bag_forward_fmt(const uint8_t* packed, int64_t total_rows,
                           const int64_t* table_offsets, int T, int64_t B, int dim,
                           int fmt, const void* indices, const void* offsets,
                           int64_t nnz, int index_type, int pool_mode,
                           const float* weights, double* out, double* abs_terms,
                           int64_t* err_count) {
  if (T < 0 || B < 0 || dim < 1 || dim > OR_MAX_DIM) return OR_INVALID;
  if (index_type != 0 && index_type != 1) return OR_INVALID;
  if (pool_mode != 0 && pool_mode != 1) return OR_INVALID;
  if (pool_mode == 1 && weights == NULL) return OR_INVALID;
  int64_t stride = fmt_stride(dim, fmt);
  int64_t errors = 0;
  int64_t G = (int64_t)T * B;
#pragma omp parallel for schedule(static) reduction(+ : errors)
  for (int64_t g = 0; g < G; ++g) {
    int64_t t = g / B, b = g % B;
    double* o = out + (b * T + t) * (int64_t)dim;
    double* a = abs_terms ? abs_terms + (b * T + t) * (int64_t)dim : NULL;
    for (int j = 0; j < dim; ++j) {
      o[j] = 0.0;
      if (a) a[j] = 0.0;
    }
    int64_t p0 = load_index(offsets, g, index_type);
    int64_t p1 = load_index(offsets, g + 1, index_type);
    if (p0 < 0 || p1 < p0 || p1 > nnz) {
      errors += 1;
      continue;
    }
    int64_t t0 = table_offsets[t], t1 = table_offsets[t + 1];
    int table_ok = (t0 >= 0 && t1 >= t0 && t1 <= total_rows);
    for (int64_t p = p0; p < p1; ++p) {
      int64_t idx = load_index(indices, p, index_type);
      if (!table_ok || idx < 0 || idx >= t1 - t0) {
        errors += 1;
        continue;
      }
      float y[OR_MAX_DIM];
      decode_row(packed + (t0 + idx) * stride, dim, fmt, y);
      double w = pool_mode == 1 ? (double)weights[p] : 1.0;
      for (int j = 0; j < dim; ++j) {
        double term = w * (double)y[j];
        o[j] += term;
        if (a) a[j] += fabs(term);
      }
    }
  }
  if (err_count) *err_count = errors;
  return OR_OK;
}

int oracle_bag_forward(const uint8_t* packed, int64_t total_rows,
                       const int64_t* table_offsets, int T, int64_t B, int dim,
                       int bits, const void* indices, const void* offsets,
                       int64_t nnz, int index_type, int pool_mode,
                       const float* weights, double* out, double* abs_terms,
                       int64_t* err_count) {
  if (bits != 2 && bits != 4 && bits != 8) return OR_INVALID;
  return bag_forward_fmt(packed, total_rows, table_offsets, T, B, dim, bits, indices, offsets,
                         nnz, index_type, pool_mode, weights, out, abs_terms, err_count);
}

/* The same lookup over codebook rows. */
int oracle_bag_forward_codebook(const uint8_t* packed, int64_t total_rows,
                                const int64_t* table_offsets, int T, int64_t B, int dim,
                                const void* indices, const void* offsets, int64_t nnz,
                                int index_type, int pool_mode, const float* weights,
                                double* out, double* abs_terms, int64_t* err_count) {
  return bag_forward_fmt(packed, total_rows, table_offsets, T, B, dim, OR_FMT_CB, indices, offsets,
                         nnz, index_type, pool_mode, weights, out, abs_terms, err_count);
}

/* Normalized l2 error of a quantized table against its source:
   out4[0] = mean over rows with ||x|| > 0 of ||x - y|| / ||x||,
   out4[1] = number of such rows,
   out4[2] = sum over all rows of ||x - y||^2,
   out4[3] = sum over all rows of ||x||^2  (binary64 throughout).
   Rows are summed in fixed blocks of 4096 rows and the blocks in order, so
   the result does not depend on the thread count. */
#define OR_L2_BLOCK 4096
static int l2_error_fmt(const float* x, const uint8_t* packed, int64_t rows, int dim,
                        int fmt, double* out4) {
  if (rows < 0 || dim < 1 || dim > OR_MAX_DIM) return OR_INVALID;
  int64_t stride = fmt_stride(dim, fmt);
  int64_t nblk = (rows + OR_L2_BLOCK - 1) / OR_L2_BLOCK;
  double* part = (double*)calloc((size_t)(nblk > 0 ? nblk : 1) * 4, sizeof(double));
  if (!part) return OR_INVALID;
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < nblk; ++k) {
    double sum_ratio = 0.0, n_rows = 0.0, sum_err = 0.0, sum_x = 0.0;
    int64_t r_end = (k + 1) * OR_L2_BLOCK < rows ? (k + 1) * OR_L2_BLOCK : rows;
    for (int64_t r = k * OR_L2_BLOCK; r < r_end; ++r) {
      const float* xr = x + r * (int64_t)dim;
      float yr[OR_MAX_DIM];
      decode_row(packed + r * stride, dim, fmt, yr);
      double e2 = 0.0, x2 = 0.0;
      for (int i = 0; i < dim; ++i) {
        double y = (double)yr[i];
        double e = (double)xr[i] - y;
        e2 += e * e;
        x2 += (double)xr[i] * (double)xr[i];
      }
      sum_err += e2;
      sum_x += x2;
      if (x2 > 0.0) {
        sum_ratio += sqrt(e2) / sqrt(x2);
        n_rows += 1.0;
      }
    }
    part[4 * k + 0] = sum_ratio;
    part[4 * k + 1] = n_rows;
    part[4 * k + 2] = sum_err;
    part[4 * k + 3] = sum_x;
  }
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  for (int64_t k = 0; k < nblk; ++k)
    for (int c = 0; c < 4; ++c) acc[c] += part[4 * k + c];
  free(part);
  out4[0] = acc[1] > 0.0 ? acc[0] / acc[1] : 0.0;
  out4[1] = acc[1];
  out4[2] = acc[2];
  out4[3] = acc[3];
  return OR_OK;
}

int oracle_l2_error(const float* x, const uint8_t* packed, int64_t rows, int dim,
                    int bits, double* out4) {
  if (bits != 2 && bits != 4 && bits != 8) return OR_INVALID;
  return l2_error_fmt(x, packed, rows, dim, bits, out4);
}

int oracle_l2_error_codebook(const float* x, const uint8_t* packed, int64_t rows, int dim,
                             double* out4) {
  return l2_error_fmt(x, packed, rows, dim, OR_FMT_CB, out4);
}

/* ------------------------------------------------------------------ */
/* Dot interaction of pooled embeddings.                                */
/* ------------------------------------------------------------------ */

/* Output width of one sample: d dense values + T(T+1)/2 dots. */
int64_t oracle_interaction_width(int T, int dim) {
  if (T < 0 || dim < 1) return -1;
  return (int64_t)dim + (int64_t)T * (T + 1) / 2;
}

/* Per sample b: Z row 0 = dense[b], Z row 1 + t = pooled[b][t] (the lookup's
   [B][T][d] output).  out[b] = dense[b] (copied) followed by, for i = 1..T
   and j = 0..i-1 in that order, sum_k Z[i][k] * Z[j][k] in binary64 (each
   product of two fp32 values is exact in binary64; the sum runs over k in
   order).  abs_terms[b] (nullable) holds sum_k |Z[i][k] * Z[j][k]| at the
   same positions and 0 at the dense positions. */
int oracle_dot_interaction(const float* dense, const float* pooled, int64_t B, int T, int dim,
                           double* out, double* abs_terms) {
  if (B < 0 || T < 0 || dim < 1) return OR_INVALID;
  const int64_t W = oracle_interaction_width(T, dim);
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < B; ++b) {
    double* o = out + b * W;
    double* a = abs_terms ? abs_terms + b * W : NULL;
    const float* x = dense + b * (int64_t)dim;
    const float* e = pooled + b * (int64_t)T * dim;
    for (int k = 0; k < dim; ++k) {
      o[k] = (double)x[k];
      if (a) a[k] = 0.0;
    }
    int64_t pos = dim;
    for (int i = 1; i <= T; ++i) {
      const float* zi = e + (int64_t)(i - 1) * dim;
      for (int j = 0; j < i; ++j) {
        const float* zj = j == 0 ? x : e + (int64_t)(j - 1) * dim;
        double s = 0.0, sa = 0.0;
        for (int k = 0; k < dim; ++k) {
          double p = (double)zi[k] * (double)zj[k];
          s += p;
          sa += fabs(p);
        }
        o[pos] = s;
        if (a) a[pos] = sa;
        ++pos;
      }
    }
  }
  return OR_OK;
}

/* ------------------------------------------------------------------ */
/* Error-bounded compression of pooled embeddings.                      */
/* ------------------------------------------------------------------ */

/* "Avancées dans les recommandations en Deep Learning" (scisimple page,
   sections "Défis de Communication", "Méthodes de Compression des Données"
   and "Stratégies de Compression Adaptative"): the embeddings that devices
   exchange in the all-to-all are compressed by a lossy method whose
   reconstruction error stays within a bound the user sets, and each table
   may have a bound of its own.  The page names no scheme; the reading here
   is the plainest error-bounded one, a uniform quantizer of bin width twice
   the bound followed by a fixed-width bit packing of each vector's codes:

     step = 2 eb, inv = 1 / step (IEEE division, once per table),
     q = rint(x * inv) (ties to even), x' = step * (float)q, all binary32,
     kept only if |x - x'| <= eb;
     u = 2q for q >= 0, -2q - 1 for q < 0 (zigzag), w = bit length of the
     vector's largest u (0 .. 31), element i's u at bits [i w, i w + w) of a
     little-endian bit stream of dwords.

   The code is taken against the reciprocal of the bin width, as the
   row-wise quantizer takes its codes against the reciprocal of the stored
   scale; the check that follows catches the rare element that this
   rounding (or any other) puts past the bound.  A vector with a non-finite
   element, a |q| >= 2^30 or an element that misses the bound, or whose
   table's eb is not a positive finite number (or makes step infinite), is
   stored verbatim (header 32).  The bound then holds for every element of
   every vector.

   Record of a vector: a uint32 header (w, or 32 for a verbatim vector), then
   ceil(d w / 32) payload dwords (d fp32 values when verbatim).  Vector v of
   n = B T (the [B][T][d] order of the lookup's output) uses the bound of
   table v mod T.  Records follow each other in vector order; offs[v] is the
   byte offset of record v, offs[0] = 0 and offs[n] the total size. */
#define OR_RAW_W 32

int64_t oracle_record_bytes(int dim, int w) {
  if (dim < 1 || w < 0 || w > OR_RAW_W) return -1;
  if (w == OR_RAW_W) return 4 + 4 * (int64_t)dim;
  return 4 + 4 * (((int64_t)dim * w + 31) / 32);
}

int64_t oracle_compress_bound(int64_t n, int dim) {
  if (n < 0 || dim < 1) return -1;
  return n * oracle_record_bytes(dim, OR_RAW_W);
}

static uint32_t zigzag(int32_t q) {
  return q >= 0 ? 2u * (uint32_t)q : 2u * (uint32_t)(-(int64_t)q) - 1u;
}

static int32_t unzigzag(uint32_t u) {
  return (u & 1u) ? -(int32_t)((u - 1u) / 2u) - 1 : (int32_t)(u / 2u);
}

static int bit_length(uint32_t v) {
  int w = 0;
  while (v) {
    ++w;
    v >>= 1;
  }
  return w;
}

/* The width of a vector (0 .. 31), or OR_RAW_W if it is stored verbatim;
   u[i] receives the zigzag codes when it is not. */
static int vector_width(const float* x, int d, float eb, uint32_t* u) {
  if (!(eb > 0.0f) || !isfinite(eb)) return OR_RAW_W;
  const float step = 2.0f * eb;
  if (!isfinite(step)) return OR_RAW_W;
  const float inv = 1.0f / step;
  uint32_t umax = 0;
  for (int i = 0; i < d; ++i) {
    if (!isfinite(x[i])) return OR_RAW_W;
    const float r = rintf(x[i] * inv);
    if (!(fabsf(r) < 1073741824.0f)) return OR_RAW_W; /* |q| < 2^30 */
    const int32_t q = (int32_t)r;
    const float xr = step * (float)q;
    if (!(fabsf(x[i] - xr) <= eb)) return OR_RAW_W;
    u[i] = zigzag(q);
    if (u[i] > umax) umax = u[i];
  }
  return bit_length(umax);
}

static void put_u32(uint8_t* p, uint32_t v) {
  for (int k = 0; k < 4; ++k) p[k] = (uint8_t)(v >> (8 * k));
}

static uint32_t get_u32(const uint8_t* p) {
  return (uint32_t)p[0] | (uint32_t)p[1] << 8 | (uint32_t)p[2] << 16 | (uint32_t)p[3] << 24;
}

/* x: [n][dim] fp32 (vector v of table v mod T); eb: [T]; out: at least
   oracle_compress_bound(n, dim) bytes, of which offs[n] are written;
   offs: [n + 1].  widths (nullable): [n], each vector's header. */
int oracle_compress_pooled(const float* x, int64_t n, int dim, int T, const float* eb,
                           uint8_t* out, int64_t* offs, int32_t* widths) {
  if (n < 0 || dim < 1 || dim > OR_MAX_DIM || T < 1 || (n > 0 && (!x || !eb || !out)) || !offs)
    return OR_INVALID;
  int32_t* w = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  if (!w) return OR_INVALID;
#pragma omp parallel
  {
    uint32_t* u = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)dim);
#pragma omp for schedule(static)
    for (int64_t v = 0; v < n; ++v) w[v] = vector_width(x + v * dim, dim, eb[v % T], u);
    free(u);
  }
  offs[0] = 0;
  for (int64_t v = 0; v < n; ++v) offs[v + 1] = offs[v] + oracle_record_bytes(dim, w[v]);
#pragma omp parallel
  {
    uint32_t* u = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)dim);
#pragma omp for schedule(static)
    for (int64_t v = 0; v < n; ++v) {
      const float* xv = x + v * dim;
      uint8_t* rec = out + offs[v];
      put_u32(rec, (uint32_t)w[v]);
      if (w[v] == OR_RAW_W) {
        memcpy(rec + 4, xv, 4 * (size_t)dim);
        continue;
      }
      vector_width(xv, dim, eb[v % T], u);
      const int64_t nbytes = oracle_record_bytes(dim, w[v]) - 4;
      memset(rec + 4, 0, (size_t)nbytes);
      for (int i = 0; i < dim; ++i)
        for (int k = 0; k < w[v]; ++k)
          if ((u[i] >> k) & 1u) {
            const int64_t bit = (int64_t)i * w[v] + k;
            rec[4 + bit / 8] |= (uint8_t)(1u << (bit % 8));
          }
    }
    free(u);
  }
  if (widths)
    for (int64_t v = 0; v < n; ++v) widths[v] = w[v];
  free(w);
  return OR_OK;
}

/* Inverse of oracle_compress_pooled.  in: in_bytes bytes; offs: [n + 1];
   y: [n][dim].  A record whose offsets are out of order or outside
   [0, in_bytes], whose header exceeds 32, or whose size differs from what
   its header implies, is decoded as zeros and counted in *n_bad. */
int oracle_decompress_pooled(const uint8_t* in, int64_t in_bytes, const int64_t* offs, int64_t n,
                             int dim, int T, const float* eb, float* y, int64_t* n_bad) {
  if (n < 0 || dim < 1 || dim > OR_MAX_DIM || T < 1 || in_bytes < 0 || !offs ||
      (n > 0 && (!eb || !y)) || (in_bytes > 0 && !in))
    return OR_INVALID;
  int64_t bad = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
  for (int64_t v = 0; v < n; ++v) {
    float* yv = y + v * dim;
    const int64_t a = offs[v], b = offs[v + 1];
    int ok = a >= 0 && a <= b && b <= in_bytes && b - a >= 4;
    uint32_t hdr = ok ? get_u32(in + a) : 0;
    ok = ok && hdr <= OR_RAW_W && b - a == oracle_record_bytes(dim, (int)hdr);
    if (!ok) {
      for (int i = 0; i < dim; ++i) yv[i] = 0.0f;
      ++bad;
      continue;
    }
    const uint8_t* p = in + a + 4;
    if (hdr == OR_RAW_W) {
      memcpy(yv, p, 4 * (size_t)dim);
      continue;
    }
    const float step = 2.0f * eb[v % T];
    for (int i = 0; i < dim; ++i) {
      uint32_t uu = 0;
      for (int k = 0; k < (int)hdr; ++k) {
        const int64_t bit = (int64_t)i * hdr + k;
        uu |= (uint32_t)((p[bit / 8] >> (bit % 8)) & 1u) << k;
      }
      yv[i] = step * (float)unzigzag(uu);
    }
  }
  if (n_bad) *n_bad = bad;
  return OR_OK;
}
