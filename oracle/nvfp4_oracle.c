/*
 * nvfp4_oracle.c -- plain, slow, scalar CPU oracle for the NVFP4 block-scaled
 * quantize / dequantize / qmv / qqmm / gather_qmm path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file: only the tests, the package smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant
 * generator with the HIP kernels.
 *
 * Pages cited (titles as published):
 *   [DIFF-8]  "mlx 0.30.7.2 -> 0.30.7.6" source diff, page 8 (my.diffend.io):
 *             ops.cpp hunks fp_quantize / fp_dequantize / validate_global_scale
 *             / qqmm, primitives.cpp hunk QQMatmul::vjp.
 *   [DIFF-7]  same diff, page 7: fp_quantize.cu hunks (fp_quantize_dequantize,
 *             fp_quantize_rowwise, fp_dequantize), qqmm.cpp (QQMatmul::eval_gpu).
 *   [PR4458]  "[Metal] global scale for qmm" (ml-explore/mlx pull request 4458):
 *             statement and "Example" section.
 *   [PR31]    osaurus-ai/mlx pull request 31 (CPU qqmm ignores nvfp4 global
 *             scales): sections "What fails", "The test", "The fix",
 *             "Verification".
 *   [PR1772]  the pull request referenced from [PR4458]'s page, "fix(mlx):
 *             bump MLX pin to 81ba1c6a so mxfp8 block scales round up"
 *             (lablup/mlxcel 1772): sections "Why" and "Validation".
 *
 * Arithmetic rules (each restated where it is used):
 *   - every step the pages perform in float32 is done here in float32 with
 *     IEEE round-to-nearest-even; the build uses -ffp-contract=off and no
 *     fast-math, and x86-64 SSE evaluates float expressions in float;
 *   - the e2m1 and e4m3 encoders are written as "nearest representable value,
 *     ties to the even code, saturating", by exhaustive search over the code
 *     set (no bit tricks), which is the format definition itself;
 *   - rounding to bfloat16 / float16 is IEEE round-to-nearest-even with
 *     overflow to infinity, written from the definition in double arithmetic;
 *   - the matrix products accumulate in double, which is exact enough that
 *     the only rounding that matters is the final one to the output type.
 *
 * Readings where the pages leave a step open (also listed in the design notes):
 *   R1  nibble order: element 2j is the low nibble of byte j.
 *   R2  a value that rounds to zero keeps its sign: -0 encodes to code 0x8.
 *   R3  a block whose e4m3 scale is 0 gets encode factor 0, so its codes are
 *       +-0 and it decodes to +-0 ([PR31] "The fix": "0 when s is 0").
 *   R4  encode order of the CUDA rowwise kernel ([DIFF-7] fp_quantize_rowwise):
 *       sd = (amax/6)*enc, enc_b = enc/sf, q = e2m1(x*enc_b), all in float32.
 *   R5  e2m1 and e4m3 conversions round to nearest even and saturate.
 *   R6  decode factor is g/2688 everywhere ([DIFF-8] fp_dequantize fallback).
 *   R7  the global decode factor multiplies the block scale, not the sum
 *       ([PR4458] statement; [PR31] "The fix").
 *   R19 mx modes ([DIFF-8] fp_quantize / fp_dequantize: group size 32 outside
 *       nvfp4, 8 bits for mxfp8, 4 otherwise, scales converted to e8m0 and
 *       decoded as 2^(s - 127); validate_global_scale: no global scale
 *       outside nvfp4): mxfp4 = e2m1 codes packed as R1, mxfp8 = one e4m3
 *       byte per element, one E8M0 byte per 32 consecutive elements.
 *   R20 the E8M0 block scale is the smallest power of two >= amax / maxval
 *       (maxval 6 or 448, the division in float32), clamped to the E8M0
 *       range [2^-127, 2^127] ([PR1772] "Why": rounding log2 to nearest
 *       saturated block maxima, the CUDA conversion rounds up).
 *   R21 the element encode of R4 with enc = 1: enc_b = 1 / float(s), then
 *       e2m1 / e4m3 of x * enc_b (R2, R5).
 *   R22 decode T(value(q) * 2^(s - 127)); the product is exact in float32.
 *   R23 mx qqmm: both operands go through their mx encode and the products
 *       of the decoded values are summed without rounding either operand to
 *       T first (the pages hand both operands' codes and scales to a
 *       block-scaled product); only the sum is rounded to T.
 *   R27 gather_qmm in an mx mode: the routed product of R10 with the
 *       expert's weight decoded as R22 (float32, exact), x used as given and
 *       no global scale (validate_global_scale admits none outside nvfp4);
 *       the pages' gather_qmm takes the same mode argument as the other
 *       quantized products.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_F16 1
#define ORC_BF16 2

/* Test-only switches that plant a known mistake (see orc_set_mutant). */
#define MUT_NONE 0
#define MUT_DROP_GW 1        /* (i)   decode of w ignores g_w                    */
#define MUT_DROP_GX 2        /* (ii)  round trip of x ignores g_x                */
#define MUT_GW_ON_SUM 3      /* (iii) g_w/2688 applied to a T-precision sum      */
#define MUT_AMAX6_BF16 4     /* (iv)  amax/6 rounded to bfloat16 before * enc    */
#define MUT_ENC_ORDER 5      /* (v)   q = e2m1((x*enc)/sf) instead of x*(enc/sf) */
#define MUT_E8M0_NEAREST 6   /* (vi)  mx block scale rounded to nearest, not up  */

static int g_mutant = MUT_NONE;

void orc_set_mutant(int m) { g_mutant = m; }
int orc_get_mutant(void) { return g_mutant; }

/* ------------------------------------------------------------------------ */
/* Formats                                                                  */
/* ------------------------------------------------------------------------ */

/* e2m1 (OCP Microscaling v1.0 FP4): bit 3 sign, bits 2..1 exponent (bias 1),
 * bit 0 mantissa; exponent 0 is subnormal with step 0.5.  No inf, no NaN. */
double orc_e2m1_value(unsigned code) {
  unsigned e = (code >> 1) & 3u, m = code & 1u;
  double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
  return (code & 8u) ? -mag : mag;
}

/* Nearest e2m1 value to v, ties to the even code (mantissa bit 0), magnitudes
 * above the largest finite value 6 saturate to 6.  The sign bit of v is kept,
 * including for results of magnitude 0 (reading R2). */
unsigned orc_e2m1_encode(float v) {
  double a = fabs((double)v);
  unsigned best = 7;
  if (!(a > 6.0)) {
    double bestd = INFINITY;
    for (unsigned c = 0; c < 8; ++c) {
      double d = fabs(a - orc_e2m1_value(c));
      if (d < bestd || (d == bestd && (c & 1u) == 0)) {
        best = c;
        bestd = d;
      }
    }
  }
  return best | (signbit(v) ? 8u : 0u);
}

/* e4m3 (OCP 8-bit floating point, "E4M3FN"): bit 7 sign, bits 6..3 exponent
 * (bias 7), bits 2..0 mantissa; exponent 0 is subnormal (m/8 * 2^-6);
 * S.1111.111 is NaN; the largest finite value is 448 = 0x7E. */
double orc_e4m3_value(unsigned b) {
  unsigned e = (b >> 3) & 15u, m = b & 7u;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
  return (b & 0x80u) ? -mag : mag;
}

/* Nearest finite e4m3 value to v, ties to the even byte, saturating at 448
 * ([DIFF-7] F8E4M3_MAX = 448; reading R5).  Exhaustive over the 127 finite
 * non-negative bytes. */
unsigned orc_e4m3_encode(float v) {
  double a = fabs((double)v);
  unsigned sign = signbit(v) ? 0x80u : 0u;
  unsigned best = 0x7E;
  if (!(a >= 448.0)) {
    double bestd = INFINITY;
    for (unsigned b = 0; b <= 0x7E; ++b) {
      double d = fabs(a - orc_e4m3_value(b));
      if (d < bestd || (d == bestd && (b & 1u) == 0)) {
        best = b;
        bestd = d;
      }
    }
  }
  return best | sign;
}

/* Round a double to an IEEE binary format with p fraction bits, minimum normal
 * exponent emin and maximum exponent emax: round to nearest, ties to even,
 * gradual underflow, overflow to infinity. */
double orc_round_ieee(double v, int p, int emin, int emax) {
  if (v == 0.0 || isnan(v) || isinf(v)) return v;
  double a = fabs(v);
  int e;
  (void)frexp(a, &e); /* a = f * 2^e with f in [0.5, 1) */
  e -= 1;             /* a = f' * 2^e with f' in [1, 2) */
  if (e < emin) e = emin;
  double ulp = ldexp(1.0, e - p);
  double r = nearbyint(a / ulp) * ulp; /* a/ulp is exact; nearbyint is RNE */
  double maxv = ldexp(2.0 - ldexp(1.0, -p), emax);
  if (r > maxv) r = INFINITY;
  return copysign(r, v);
}

/* Value of v after storing it in the element type T (float32, float16 or
 * bfloat16); the result is exactly representable in float. */
float orc_round_to(float v, int dtype) {
  switch (dtype) {
    case ORC_F16: return (float)orc_round_ieee((double)v, 10, -14, 15);
    case ORC_BF16: return (float)orc_round_ieee((double)v, 7, -126, 127);
    default: return v;
  }
}

/* ------------------------------------------------------------------------ */
/* Scalars                                                                  */
/* ------------------------------------------------------------------------ */

/* Tensor amax as float32: max |x| over all elements ([DIFF-8] QQMatmul::vjp
 * takes the cotangent's max(abs(.)) as float32).  Exact. */
float orc_tensor_amax(const float* x, int64_t n) {
  float m = 0.0f;
  for (int64_t i = 0; i < n; ++i) {
    float a = fabsf(x[i]);
    if (a > m) m = a;
  }
  return m;
}

/* Global encode factor 2688/g and decode factor g/2688, each one float32
 * division; both 1 without a global scale ([DIFF-7] fp_quantize_rowwise,
 * fp_dequantize; [DIFF-8] fp_dequantize fallback; reading R6). */
static float global_enc(int has_g, float g) {
  volatile float c = 448.0f * 6.0f;
  return has_g ? c / g : 1.0f;
}
static float global_dec(int has_g, float g) {
  volatile float c = 448.0f * 6.0f;
  return has_g ? g / c : 1.0f;
}

/* ------------------------------------------------------------------------ */
/* Block encode / decode                                                    */
/* ------------------------------------------------------------------------ */

/* Encode one group of 16 contiguous values ([DIFF-7] fp_quantize_rowwise:
 * block amax, decode scale (amax/6)*enc stored as e4m3, encode factor
 * enc/float(s), each element converted to e2m1 after multiplying by it;
 * readings R2-R5).  Writes 16 codes and returns the scale byte. */
static unsigned encode_group(const float* xb, float enc, unsigned char* q) {
  float amax = 0.0f;
  for (int i = 0; i < 16; ++i) {
    float a = fabsf(xb[i]);
    if (a > amax) amax = a;
  }
  float sd;
  if (g_mutant == MUT_AMAX6_BF16) {
    /* the op-level fallback divides in the input dtype (bfloat16 here) */
    float t = orc_round_to(amax / 6.0f, ORC_BF16);
    sd = t * enc;
  } else {
    volatile float t = amax / 6.0f;
    sd = t * enc;
  }
  unsigned s = orc_e4m3_encode(sd);
  float sf = (float)orc_e4m3_value(s);
  float enc_b = (sf == 0.0f) ? 0.0f : enc / sf; /* reading R3 */
  for (int i = 0; i < 16; ++i) {
    float y;
    if (g_mutant == MUT_ENC_ORDER) {
      volatile float t = xb[i] * enc;
      y = (sf == 0.0f) ? t * 0.0f : t / sf;
    } else {
      y = xb[i] * enc_b;
    }
    q[i] = (unsigned char)orc_e2m1_encode(y);
  }
  return s;
}

/* quantize: x [rows, k] (k % 16 == 0) -> codes [rows, k/2] (element 2j in the
 * low nibble of byte j, reading R1) and e4m3 scales [rows, k/16]
 * ([DIFF-8] fp_quantize; [DIFF-7] fp_quantize_rowwise). */
void orc_quantize(const float* x, int64_t rows, int64_t k, int has_g, float g,
                  uint8_t* codes, uint8_t* scales) {
  float enc = global_enc(has_g, g);
  unsigned char q[16];
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < k / 16; ++b) {
      unsigned s = encode_group(x + r * k + b * 16, enc, q);
      scales[r * (k / 16) + b] = (uint8_t)s;
      for (int j = 0; j < 8; ++j)
        codes[r * (k / 2) + b * 8 + j] = (uint8_t)(q[2 * j] | (q[2 * j + 1] << 4));
    }
  }
}

static unsigned code_at(const uint8_t* codes_row, int64_t i) {
  uint8_t byte = codes_row[i >> 1];
  return (i & 1) ? (unsigned)(byte >> 4) : (unsigned)(byte & 15u);
}

/* Effective decode scale of one block: float(e4m3(s)) * (g/2688) in float32,
 * the global factor on the block scale ([DIFF-7] fp_dequantize; [DIFF-8]
 * fp_dequantize fallback; [PR31] "The fix"; reading R7). */
static float block_scale(unsigned s, float dec) {
  float sf = (float)orc_e4m3_value(s);
  return sf * dec;
}

/* dequantize: codes/scales [rows, k] -> T values, x_hat = T(e2m1(q) * scale),
 * where scale = float(e4m3(s)) * g/2688 ([DIFF-7] fp_dequantize). */
void orc_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k,
                    int has_g, float g, int out_dtype, float* out) {
  float dec = global_dec(has_g, g);
  for (int64_t r = 0; r < rows; ++r) {
    const uint8_t* cr = codes + r * (k / 2);
    for (int64_t i = 0; i < k; ++i) {
      float sc = block_scale(scales[r * (k / 16) + i / 16], dec);
      float v = (float)orc_e2m1_value(code_at(cr, i)) * sc;
      out[r * k + i] = orc_round_to(v, out_dtype);
    }
  }
}

/* quant_dequant: quantize then dequantize with the same g, result in x's type
 * ([DIFF-7] fp_quantize_dequantize; [PR31] "The fix": x_hat = s*q/scale_enc,
 * 0 when s is 0). */
void orc_quant_dequant(const float* x, int64_t rows, int64_t k, int has_g, float g,
                       int dtype, float* xhat) {
  float dec = global_dec(has_g, g);
  float enc = global_enc(has_g, g);
  unsigned char q[16];
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < k / 16; ++b) {
      unsigned s = encode_group(x + r * k + b * 16, enc, q);
      float sc = block_scale(s, dec);
      for (int i = 0; i < 16; ++i)
        xhat[r * k + b * 16 + i] = orc_round_to((float)orc_e2m1_value(q[i]) * sc, dtype);
    }
  }
}

/* Dequantized weight row in float32, not rounded to any narrower type: the
 * float32 contraction operand w = e2m1(q) * (float(e4m3(s)) * g/2688). */
static void weight_row_f32(const uint8_t* codes_row, const uint8_t* scales_row, int64_t k,
                           float dec, float* wrow) {
  for (int64_t i = 0; i < k; ++i) {
    float sc = block_scale(scales_row[i / 16], dec);
    wrow[i] = (float)orc_e2m1_value(code_at(codes_row, i)) * sc;
  }
}

/* Mutant (iii): block scale without g_w, product and running sum kept in T,
 * g_w/2688 applied to the final sum ([PR31] "Verification", first mutation). */
static float sum_in_t_then_scale(const float* xh, const uint8_t* codes_row,
                                 const uint8_t* scales_row, int64_t k, float dec, int dtype) {
  float acc = 0.0f;
  for (int64_t i = 0; i < k; ++i) {
    float sf = orc_round_to((float)orc_e4m3_value(scales_row[i / 16]), dtype);
    float w = orc_round_to((float)orc_e2m1_value(code_at(codes_row, i)) * sf, dtype);
    acc = orc_round_to(acc + orc_round_to(xh[i] * w, dtype), dtype);
  }
  return orc_round_to(acc * dec, dtype);
}

/* qqmm / qmv on a subset of the output: rows mi[0..nm) of x and columns
 * ni[0..nn) of w.  x [m, k] holds values of type dtype; it goes through the
 * nvfp4 round trip with g_x (reading: as [DIFF-7] QQMatmul::eval_gpu does for
 * the activations), w is given quantized (codes [n, k/2], scales [n, k/16])
 * and decoded with g_w on the block scale; the contraction sums
 * x_hat * w in double; the result is rounded to dtype
 * ([DIFF-8] qqmm; [PR31] "The fix"; [PR4458] statement).
 * has_g: both global scales present (1) or neither (0) ([DIFF-8]
 * validate_qqmm_inputs).  out is [nm, nn]. */
void orc_qqmm_subset(const float* x, int dtype, int64_t m, int64_t k, int has_g, float gx,
                     float gw, const uint8_t* wcodes, const uint8_t* wscales, int64_t n,
                     const int64_t* mi, int64_t nm, const int64_t* ni, int64_t nn, float* out,
                     int nthreads) {
  (void)m;
  (void)n;
  int gx_on = has_g && g_mutant != MUT_DROP_GX;
  float dec_w = (has_g && g_mutant != MUT_DROP_GW) ? global_dec(1, gw) : 1.0f;
  float* xh = (float*)malloc(sizeof(float) * (size_t)(nm * k));
  float* wr = (float*)malloc(sizeof(float) * (size_t)(nn * k));
  for (int64_t a = 0; a < nm; ++a)
    orc_quant_dequant(x + mi[a] * k, 1, k, gx_on, gx, dtype, xh + a * k);
  for (int64_t b = 0; b < nn; ++b)
    weight_row_f32(wcodes + ni[b] * (k / 2), wscales + ni[b] * (k / 16), k, dec_w,
                   wr + b * k);
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
  for (int64_t a = 0; a < nm; ++a) {
    for (int64_t b = 0; b < nn; ++b) {
      float r;
      if (g_mutant == MUT_GW_ON_SUM) {
        r = sum_in_t_then_scale(xh + a * k, wcodes + ni[b] * (k / 2),
                                wscales + ni[b] * (k / 16), k, global_dec(has_g, gw), dtype);
      } else {
        double acc = 0.0;
        for (int64_t i = 0; i < k; ++i) acc += (double)xh[a * k + i] * (double)wr[b * k + i];
        r = orc_round_to((float)acc, dtype);
      }
      out[a * nn + b] = r;
    }
  }
  free(xh);
  free(wr);
}

/* gather_qmm on a subset of (token, slot) pairs and output columns:
 * out[t, j, n] = T( sum_k x[t, k] * w_e[n, k] ), e = idx[t, j], with
 * w_e decoded with that expert's global scale g[e]/2688 on the block scale
 * ([PR4458] statement: x @ dequant(W) with the global scale inside the
 * dequantization; per-expert scales of shape [E, 1, 1] in the test loops).
 * x is used as given (reading: the pages quantize no activations here).
 * g may be NULL (no global scale).  pairs holds np (t, j) pairs; out is
 * [np, nn]. */
void orc_gather_qmm_subset(const float* x, int dtype, int64_t t_count, int64_t k,
                           const uint8_t* wcodes, const uint8_t* wscales, const float* g,
                           int64_t e_count, int64_t n, const int32_t* idx, int64_t top_k,
                           const int64_t* pairs_t, const int64_t* pairs_j, int64_t np,
                           const int64_t* ni, int64_t nn, float* out, int nthreads) {
  (void)t_count;
  (void)e_count;
#pragma omp parallel num_threads(nthreads)
  {
    float* wr = (float*)malloc(sizeof(float) * (size_t)k);
#pragma omp for schedule(dynamic, 1)
    for (int64_t a = 0; a < np; ++a) {
      int64_t t = pairs_t[a], j = pairs_j[a];
      int64_t e = idx[t * top_k + j];
      float dec = (g && g_mutant != MUT_DROP_GW) ? global_dec(1, g[e]) : 1.0f;
      for (int64_t b = 0; b < nn; ++b) {
        const uint8_t* cr = wcodes + (e * n + ni[b]) * (k / 2);
        const uint8_t* sr = wscales + (e * n + ni[b]) * (k / 16);
        weight_row_f32(cr, sr, k, dec, wr);
        double acc = 0.0;
        for (int64_t i = 0; i < k; ++i) acc += (double)x[t * k + i] * (double)wr[i];
        out[a * nn + b] = orc_round_to((float)acc, dtype);
      }
    }
    free(wr);
  }
}

/* gather_qmm in its general indexed form, on a subset of output rows and
 * columns ([PR4458] statement and test loops: every dtype, transpose True and
 * False, per-expert global scales; the op's lhs_indices / rhs_indices):
 *   x is [b, mr, k]: b batch entries of mr rows; pair p (0 <= p < L) takes x
 *   entry lhs[p] (p when lhs is NULL) and expert rhs[p]; output row
 *   q = p * mr + r is T( sum_k x[lhs[p], r, k] * w_e[n, k] ), e = rhs[p].
 *   transpose = 1: expert e's weight is [n, k] quantized along k (codes
 *   [e, n, k/2], scales [e, n, k/16]), the product x @ w_e^T;
 *   transpose = 0: it is [k, n] quantized along n (codes [e, k, n/2], scales
 *   [e, k, n/16]), the product x @ w_e, whose element (n, k) is the decoded
 *   [k, n] weight at row k, column n.
 * x is used as given (reading R10); the global scale g[e] / 2688 multiplies
 * the block scale (R7); products summed in double, one rounding to T. */
void orc_gather_qmm_indexed_subset(const float* x, int dtype, int64_t b, int64_t mr, int64_t k,
                                   const uint8_t* wcodes, const uint8_t* wscales, const float* g,
                                   int64_t e_count, int64_t n, int transpose, const int32_t* lhs,
                                   const int32_t* rhs, int64_t L, const int64_t* qi, int64_t nq,
                                   const int64_t* ni, int64_t nn, float* out, int nthreads) {
  (void)b;
  (void)L;
  (void)e_count;
#pragma omp parallel num_threads(nthreads)
  {
    float* wr = (float*)malloc(sizeof(float) * (size_t)k);
#pragma omp for schedule(dynamic, 1)
    for (int64_t a = 0; a < nq; ++a) {
      const int64_t q = qi[a], p = q / mr, r = q % mr;
      const int64_t ent = lhs ? (int64_t)lhs[p] : p;
      const int64_t e = rhs[p];
      const float* xr = x + (ent * mr + r) * k;
      float dec = (g && g_mutant != MUT_DROP_GW) ? global_dec(1, g[e]) : 1.0f;
      for (int64_t c = 0; c < nn; ++c) {
        const int64_t col = ni[c];
        if (transpose) {
          weight_row_f32(wcodes + (e * n + col) * (k / 2), wscales + (e * n + col) * (k / 16), k, dec,
                         wr);
        } else {
          for (int64_t i = 0; i < k; ++i) {
            const uint8_t* crow = wcodes + (e * k + i) * (n / 2);
            const uint8_t* srow = wscales + (e * k + i) * (n / 16);
            wr[i] = (float)orc_e2m1_value(code_at(crow, col)) * block_scale(srow[col / 16], dec);
          }
        }
        double acc = 0.0;
        for (int64_t i = 0; i < k; ++i) acc += (double)xr[i] * (double)wr[i];
        out[a * nn + c] = orc_round_to((float)acc, dtype);
      }
    }
    free(wr);
  }
}

/* Routing reference: tokens grouped by expert, stable (ascending t, then j).
 * offsets [e_count + 1] is the exclusive prefix sum of the per-expert counts;
 * perm [t_count * top_k] lists flat pair ids t*top_k + j in that order.
 * Returns 0, or -1 if an index is out of range. */
int orc_moe_route(const int32_t* idx, int64_t t_count, int64_t top_k, int64_t e_count,
                  int32_t* offsets, int32_t* perm) {
  int64_t total = t_count * top_k;
  for (int64_t e = 0; e <= e_count; ++e) offsets[e] = 0;
  for (int64_t p = 0; p < total; ++p) {
    if (idx[p] < 0 || idx[p] >= e_count) return -1;
    offsets[idx[p] + 1] += 1;
  }
  for (int64_t e = 0; e < e_count; ++e) offsets[e + 1] += offsets[e];
  int64_t pos = 0;
  for (int64_t e = 0; e < e_count; ++e)
    for (int64_t p = 0; p < total; ++p)
      if (idx[p] == e) perm[pos++] = (int32_t)p;
  return 0;
}

/* ------------------------------------------------------------------------ */
/* MX modes: mxfp4 / mxfp8 (readings R19-R23)                               */
/* ------------------------------------------------------------------------ */

/* E8M0 (OCP Microscaling v1.0 scale type): byte b is 2^(b - 127); 0xFF is
 * NaN.  No sign, no mantissa, no zero. */
double orc_e8m0_value(unsigned b) {
  if ((b & 0xFFu) == 0xFFu) return NAN;
  return ldexp(1.0, (int)(b & 0xFFu) - 127);
}

/* Round-up conversion of v >= 0 to E8M0 (reading R20): the smallest byte b
 * in 0..254 with 2^(b - 127) >= v, found by search over the bytes; values
 * above 2^127 clamp to 254. */
unsigned orc_e8m0_encode_up(float v) {
  for (unsigned b = 0; b <= 254; ++b)
    if (orc_e8m0_value(b) >= (double)v) return b;
  return 254;
}

/* Value of a code of the mx element type: e2m1 (bits 4) or e4m3 (bits 8). */
static double mx_code_value(unsigned q, int bits) {
  return bits == 8 ? orc_e4m3_value(q) : orc_e2m1_value(q);
}

/* Encode one group of 32 contiguous values (readings R20, R21): the block
 * amax, its float32 quotient by maxval rounded up to an E8M0 scale s, the
 * encode factor 1/float(s), and each element's code of x * enc_b.  Writes 32
 * codes and returns the scale byte. */
static unsigned mx_encode_group(const float* xb, int bits, unsigned* q) {
  float amax = 0.0f;
  for (int i = 0; i < 32; ++i) {
    float a = fabsf(xb[i]);
    if (a > amax) amax = a;
  }
  volatile float maxval = bits == 8 ? 448.0f : 6.0f;
  volatile float sd = amax / maxval;
  unsigned s = orc_e8m0_encode_up(sd);
  if (g_mutant == MUT_E8M0_NEAREST) {
    /* the rejected encode: 2^round(log2(amax / maxval)), ties away */
    s = sd > 0.0f ? (unsigned)lround(log2((double)sd) + 127.0) : 0u;
  }
  volatile float sf = (float)orc_e8m0_value(s);
  float enc_b = 1.0f / sf;
  for (int i = 0; i < 32; ++i) {
    float y = xb[i] * enc_b;
    q[i] = bits == 8 ? orc_e4m3_encode(y) : orc_e2m1_encode(y);
  }
  return s;
}

static int64_t mx_row_bytes(int64_t k, int bits) { return bits == 8 ? k : k / 2; }

static unsigned mx_code_at(const uint8_t* codes_row, int64_t i, int bits) {
  return bits == 8 ? (unsigned)codes_row[i] : code_at(codes_row, i);
}

/* mx quantize: x [rows, k] (k % 32 == 0) -> codes [rows, k/2] (mxfp4, R1
 * nibble order) or [rows, k] (mxfp8), E8M0 scales [rows, k/32]
 * ([DIFF-8] fp_quantize; [DIFF-7] fp_quantize_rowwise with use_mx_scale). */
void orc_mx_quantize(const float* x, int64_t rows, int64_t k, int bits, uint8_t* codes,
                     uint8_t* scales) {
  int64_t rb = mx_row_bytes(k, bits);
  /* rows are independent: one thread per row at a time */
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    unsigned q[32];
    for (int64_t b = 0; b < k / 32; ++b) {
      scales[r * (k / 32) + b] = (uint8_t)mx_encode_group(x + r * k + b * 32, bits, q);
      uint8_t* out = codes + r * rb + (bits == 8 ? b * 32 : b * 16);
      if (bits == 8)
        for (int j = 0; j < 32; ++j) out[j] = (uint8_t)q[j];
      else
        for (int j = 0; j < 16; ++j) out[j] = (uint8_t)(q[2 * j] | (q[2 * j + 1] << 4));
    }
  }
}

/* Decoded value of element i of a quantized mx row in float32 (exact,
 * reading R22). */
static float mx_value(const uint8_t* codes_row, const uint8_t* scales_row, int64_t i, int bits) {
  return (float)(mx_code_value(mx_code_at(codes_row, i, bits), bits) *
                 orc_e8m0_value(scales_row[i / 32]));
}

/* mx dequantize: T(value(q) * 2^(s - 127)) ([DIFF-8] fp_dequantize: e8m0
 * scales decoded as a power of two; reading R22). */
void orc_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k,
                       int bits, int out_dtype, float* out) {
  int64_t rb = mx_row_bytes(k, bits);
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t i = 0; i < k; ++i)
      out[r * k + i] = orc_round_to(mx_value(codes + r * rb, scales + r * (k / 32), i, bits),
                                    out_dtype);
}

/* mx quant_dequant: the encode then the decode, result in type T
 * ([DIFF-7] fp_quantize_dequantize with use_mx_scale). */
void orc_mx_quant_dequant(const float* x, int64_t rows, int64_t k, int bits, int dtype,
                          float* xhat) {
  unsigned q[32];
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < k / 32; ++b) {
      unsigned s = mx_encode_group(x + r * k + b * 32, bits, q);
      double sc = orc_e8m0_value(s);
      for (int i = 0; i < 32; ++i)
        xhat[r * k + b * 32 + i] = orc_round_to((float)(mx_code_value(q[i], bits) * sc), dtype);
    }
  }
}

/* mx qqmm / qmv on a subset of the output (rows mi of x, columns ni of w):
 * out = T( sum_k x_hat[m, k] * w_hat[n, k] ), with x_hat the float32 decode
 * of x's own mx encode and w_hat that of the given codes and scales, summed
 * in double (reading R23; [DIFF-8] qqmm, where the mode selects the group
 * size and scale type for both operands). */
void orc_mx_qqmm_subset(const float* x, int dtype, int64_t m, int64_t k, int bits,
                        const uint8_t* wcodes, const uint8_t* wscales, int64_t n,
                        const int64_t* mi, int64_t nm, const int64_t* ni, int64_t nn, float* out,
                        int nthreads) {
  (void)m;
  (void)n;
  int64_t rb = mx_row_bytes(k, bits);
  float* xh = (float*)malloc(sizeof(float) * (size_t)(nm * k));
  float* wr = (float*)malloc(sizeof(float) * (size_t)(nn * k));
  uint8_t* xc = (uint8_t*)malloc((size_t)rb);
  uint8_t* xs = (uint8_t*)malloc((size_t)(k / 32));
  for (int64_t a = 0; a < nm; ++a) {
    orc_mx_quantize(x + mi[a] * k, 1, k, bits, xc, xs);
    for (int64_t i = 0; i < k; ++i) xh[a * k + i] = mx_value(xc, xs, i, bits);
  }
  for (int64_t b = 0; b < nn; ++b)
    for (int64_t i = 0; i < k; ++i)
      wr[b * k + i] = mx_value(wcodes + ni[b] * rb, wscales + ni[b] * (k / 32), i, bits);
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
  for (int64_t a = 0; a < nm; ++a) {
    for (int64_t b = 0; b < nn; ++b) {
      double acc = 0.0;
      for (int64_t i = 0; i < k; ++i) acc += (double)xh[a * k + i] * (double)wr[b * k + i];
      out[a * nn + b] = orc_round_to((float)acc, dtype);
    }
  }
  free(xh);
  free(wr);
  free(xc);
  free(xs);
}

/* gather_qmm in an mx mode on a subset of (token, slot) pairs and output
 * columns (reading R27): out[t, j, n] = T( sum_k x[t, k] * w_e[n, k] ),
 * e = idx[t, j], w_e the float32 decode of expert e's mx codes [e, n, row
 * bytes] and E8M0 scales [e, n, k/32] (R22); products summed in double, one
 * rounding to T.  A pair whose expert lies outside [0, e_count) multiplies
 * nothing: its row is zero (the library's documented contract for such
 * pairs; the pages define no product for them).  out is [np, nn]. */
void orc_mx_gather_qmm_subset(const float* x, int dtype, int64_t k, int bits,
                              const uint8_t* wcodes, const uint8_t* wscales, int64_t e_count,
                              int64_t n, const int32_t* idx, int64_t top_k,
                              const int64_t* pairs_t, const int64_t* pairs_j, int64_t np,
                              const int64_t* ni, int64_t nn, float* out, int nthreads) {
  const int64_t rb = mx_row_bytes(k, bits);
#pragma omp parallel num_threads(nthreads)
  {
    float* wr = (float*)malloc(sizeof(float) * (size_t)k);
#pragma omp for schedule(dynamic, 1)
    for (int64_t a = 0; a < np; ++a) {
      const int64_t t = pairs_t[a], j = pairs_j[a];
      const int64_t e = idx[t * top_k + j];
      for (int64_t b = 0; b < nn; ++b) {
        if (e < 0 || e >= e_count) {
          out[a * nn + b] = 0.0f;
          continue;
        }
        const int64_t row = e * n + ni[b];
        for (int64_t i = 0; i < k; ++i)
          wr[i] = mx_value(wcodes + row * rb, wscales + row * (k / 32), i, bits);
        double acc = 0.0;
        for (int64_t i = 0; i < k; ++i) acc += (double)x[t * k + i] * (double)wr[i];
        out[a * nn + b] = orc_round_to((float)acc, dtype);
      }
    }
    free(wr);
  }
}
