/*
 * CPU oracle for the fused gated-linear-unit activation with block-scaled
 * ("microscaling") output.
 *
 * TEST INFRASTRUCTURE ONLY.  The only callers are the tests, the smoke check and
 * the benchmark's CPU-baseline leg.  The GPU library never links, loads or calls
 * this file, and the two share no code, header, table or constant generator.
 *
 * Everything is evaluated in binary64 from the textbook definitions, then encoded
 * by a nearest-value search over each number format's own value table (ties to
 * the even code).  Nothing here is blocked, fused or reordered for speed beyond
 * an OpenMP split over independent rows and blocks.
 *
 * Sources, cited by page title and section:
 *   [MX] "Add swiglu + MXFP8 fused CuTe DSL kernel"
 *        - Summary: SwiGLU fused with the RCEIL MXFP8 cast; rowwise (1x32),
 *          colwise (32x1) or both scalings from one pass.
 *        - API: gated_input packs [gate | up]; backward returns [dGate | dUp].
 *        - Numerics and tests: the fused result equals the activation followed by
 *          the standalone quantizers (so the quantizer sees the BF16 activation).
 *   [NV] "feat(phyai-kernel): add Thor NVFP4 GeGLU kernel for pi0.5"
 *        - Summary: GeGLU fold followed by a compact NVFP4 store.
 *        - Supported contract: packed E2M1 values, FP8 E4M3 block scales in the
 *          CUTLASS/FlashInfer 128x4 layout, global scale 1, pairwise-interleaved
 *          gate/up columns (gate0, up0, gate1, up1, ...).
 *   [GE] "perf: tile wide GeGLU rows on SM103"
 *        - Summary and Testing Done: GeGLU forward and its two gradients da, db.
 *   [H]  "[WS1] Add batch-invariant h_aggregate kernel"
 *        - Fixed numerical paths: FP32 (here FP64) math with exactly one
 *          conversion to BF16 at the final store.
 *
 * Readings where the pages leave the arithmetic open (each is repeated at the
 * function that uses it):
 *   - the quantizer consumes the BF16-rounded activation, rounded once;
 *   - GELU is the tanh approximation with sqrt(2/pi) and 0.044715;
 *   - two further activations through the same path (the [MX] page's Follow-ups
 *     plan more than SiLU; none is named): GeGLU with the exact,
 *     erf-based GELU x * Phi(x), and ReLU^2 GLU, max(x, 0)^2 * up;
 *   - RCEIL: the scale is the smallest power of two 2^e, e in [-127, 127], with
 *     448 * 2^e >= amax (an all-zero block takes e = -127);
 *   - E4M3 saturates to +-448; E2M1 saturates to +-6;
 *   - NVFP4 scale = E4M3(amax / 6) rounded to nearest; codes = E2M1(x / S);
 *     S == 0 gives signed-zero codes; even element in the low nibble;
 *   - a block holding NaN or Inf gets a NaN scale (MX 0xFF, NV 0x7F) and NaN
 *     codes (MX 0x7F) or zero codes (NV);
 *   - MXFP8 scales may also be asked for in the same zero-padded 128x4 layout
 *     (the GEMM-ready block-scale layout; no page fixes one for MXFP8);
 *   - an NVFP4 backward quantizes [da | db] as one [M, 2N] matrix in 16-element
 *     row blocks, the MXFP8 backward's placement (no page defines one);
 *   - the GEMM epilogue form takes block-scaled operands with E8M0 scales per 32
 *     along K (the block scaling gfx950's matrix cores take): E4M3 codes (MXFP8), or
 *     E2M1 codes packed two per byte, even element in the low nibble (MXFP4, the
 *     closest form of [NV]'s packed E2M1 operands); W = [W_gate | W_up] or, as [NV]
 *     Supported contract's weight layout row fixes, pairwise-interleaved gate/up
 *     rows (gate0, up0, gate1, up1, ...);
 *   - two-level NVFP4 (a global scale from the tensor's amax, relaxing [NV]'s global
 *     scale 1) is defined by IEEE FP32 operations: s = 2688 / amax (capped at
 *     2^100), block scale E4M3(bamax * fl(s / 6)), codes E2M1(x * fl(s / S)).
 * Parity unpinned: the NaN/Inf block rule, the nibble order, and the 128x4
 * scale layout beyond its being a zero-padded permutation.  No page prints a
 * value for any of them.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#if defined(__FAST_MATH__)
#error "the oracle must be built without fast-math"
#endif

enum { ORC_SWIGLU = 0, ORC_GEGLU_TANH = 1, ORC_GEGLU_ERF = 2, ORC_RELU2 = 3 };
enum { ORC_SPLIT = 0, ORC_PAIRED = 1 };
enum { ORC_ROWWISE = 1, ORC_COLWISE = 2, ORC_SF_SWIZZLED = 4 };
enum { ORC_SF_ROWMAJOR = 0, ORC_SF_128x4 = 1 };

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------- */
/* Number formats: value tables and nearest-value encoders                    */
/* ------------------------------------------------------------------------- */

/* BF16: 1 sign, 8 exponent (bias 127), 7 mantissa bits.  Magnitude code c
 * (0 .. 0x7F7F finite) has value m * 2^-133 when the exponent field is zero and
 * (1 + m/128) * 2^(E-127) otherwise.  Code 0x7F80 is +Inf; for rounding it is
 * treated as the next step, 2^128, so that overflow follows round-to-nearest-even. */
static double bf16_mag_def(uint32_t c) {
  uint32_t E = c >> 7, m = c & 0x7F;
  if (c == 0x7F80) return ldexp(1.0, 128);
  if (E == 0) return ldexp((double)m, -133);
  return ldexp(1.0 + m / 128.0, (int)E - 127);
}
/* The definition above, tabulated once when the library loads. */
static double bf16_table[0x7F81];
__attribute__((constructor)) static void fill_bf16_table(void) {
  for (uint32_t c = 0; c <= 0x7F80; c++) bf16_table[c] = bf16_mag_def(c);
}
static double bf16_mag(uint32_t c) { return bf16_table[c]; }

double orc_bf16_to_f64(uint16_t b) {
  uint32_t c = b & 0x7FFF;
  double s = (b & 0x8000) ? -1.0 : 1.0;
  if (c > 0x7F80) return NAN;
  if (c == 0x7F80) return s * INFINITY;
  return s * bf16_mag(c);
}

/* Nearest code in [0, top] of a monotone magnitude table, ties to the even code.
 * mag(top) is the largest value the search may return. */
static uint32_t nearest_code(double a, double (*mag)(uint32_t), uint32_t top) {
  if (a >= mag(top)) return top;
  uint32_t lo = 0, hi = top; /* invariant: mag(lo) <= a < mag(hi) */
  while (hi - lo > 1) {
    uint32_t mid = lo + (hi - lo) / 2;
    if (mag(mid) <= a) lo = mid; else hi = mid;
  }
  double midpoint = 0.5 * (mag(lo) + mag(hi)); /* exact: both have few bits */
  if (a < midpoint) return lo;
  if (a > midpoint) return hi;
  return (lo % 2 == 0) ? lo : hi;
}

/* Round a binary64 value to BF16, nearest, ties to even; overflow to Inf. */
uint16_t orc_bf16_from_f64(double v) {
  if (isnan(v)) return 0x7FC0;
  uint16_t s = signbit(v) ? 0x8000 : 0;
  return (uint16_t)(s | nearest_code(fabs(v), bf16_mag, 0x7F80));
}

/* OCP FP8 E4M3 ("FN" flavour): 1 sign, 4 exponent (bias 7), 3 mantissa bits, no
 * infinities, S.1111.111 is NaN, largest finite 448 (0x7E), subnormals k * 2^-9. */
static double e4m3_mag(uint32_t c) {
  uint32_t E = c >> 3, m = c & 7;
  if (E == 0) return ldexp((double)m, -9);
  return ldexp(1.0 + m / 8.0, (int)E - 7);
}

double orc_e4m3_to_f64(uint8_t c) {
  double s = (c & 0x80) ? -1.0 : 1.0;
  if ((c & 0x7F) == 0x7F) return NAN;
  return s * e4m3_mag(c & 0x7F);
}

/* Nearest E4M3, ties to even, saturating at +-448 (reading: the pages never let a
 * scaled value exceed 448, and saturation keeps anything larger finite). */
uint8_t orc_e4m3_from_f64(double y) {
  if (isnan(y)) return 0x7F;
  uint8_t s = signbit(y) ? 0x80 : 0;
  return (uint8_t)(s | nearest_code(fabs(y), e4m3_mag, 0x7E));
}

/* FP4 E2M1: magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}, sign bit 0x8. */
static double e2m1_mag(uint32_t c) {
  if (c < 2) return 0.5 * c;
  return ldexp(1.0 + (c & 1) / 2.0, (int)(c >> 1) - 1);
}

double orc_e2m1_to_f64(uint8_t c) {
  double s = (c & 0x8) ? -1.0 : 1.0;
  return s * e2m1_mag(c & 7);
}

/* Nearest E2M1, ties to even, saturating at +-6. */
uint8_t orc_e2m1_from_f64(double y) {
  if (isnan(y)) return 0x7; /* never reached: NaN blocks are handled first */
  uint8_t s = signbit(y) ? 0x8 : 0;
  return (uint8_t)(s | nearest_code(fabs(y), e2m1_mag, 7));
}

/* RCEIL E8M0 scale exponent for MXFP8 E4M3 ([MX] Summary names RCEIL; reading):
 * the smallest e in [-127, 127] with 448 * 2^e >= amax.  The scale byte is e + 127. */
int orc_mx_scale_exponent(double amax) {
  int e = -127;
  if (amax > 0) {
    e = ilogb(amax) - 9; /* 448 * 2^(k-9) < 2^k <= amax, so this guess is low */
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    while (e > -127 && ldexp(448.0, e - 1) >= amax) e--;
    while (e < 127 && ldexp(448.0, e) < amax) e++;
  }
  return e;
}

/* ------------------------------------------------------------------------- */
/* Activations ([MX] Summary: swiglu = silu(gate) * up; [NV] Summary and [GE]     */
/* Summary: GeGLU = gelu(gate) * up, tanh approximation by reading; [MX]         */
/* Follow-ups: more activations planned, here erf-GELU and ReLU^2 by reading)    */
/* ------------------------------------------------------------------------- */

static const double GELU_K0 = 0.79788456080286535588; /* sqrt(2/pi) */
static const double GELU_K1 = 0.044715;

/* logistic function; 1/(1+exp(-z)) is accurate in both tails in binary64 */
static double logistic(double z) { return 1.0 / (1.0 + exp(-z)); }

/* Standard normal CDF and density: Phi(x) = erfc(-x / sqrt 2) / 2 (erfc keeps its
 * relative accuracy for x << 0, where 1 + erf(x / sqrt 2) cancels), phi(x) =
 * exp(-x^2 / 2) / sqrt(2 pi). */
static const double SQRT1_2 = 0.70710678118654752440;    /* 1/sqrt(2) */
static const double INV_SQRT_2PI = 0.39894228040143267794; /* 1/sqrt(2 pi) */
static double normal_cdf(double x) { return 0.5 * erfc(-x * SQRT1_2); }
static double normal_pdf(double x) { return INV_SQRT_2PI * exp(-0.5 * x * x); }

/* ReLU^2: max(x, 0)^2, with NaN kept NaN (a plain max would drop it). */
static double relu(double x) { return x > 0.0 ? x : (x <= 0.0 ? 0.0 : x); }

/* act(x):  silu(x) = x * sigma(x);
 *          gelu_tanh(x) = x/2 * (1 + tanh(k0 (x + k1 x^3)));
 *          gelu_erf(x) = x * Phi(x);
 *          relu2(x) = max(x, 0)^2.
 * 1 + tanh(u) is evaluated as 2 * sigma(2u), the same quantity written without
 * the cancellation that 1 + tanh(u) suffers for u << 0. */
double orc_act(int act, double x) {
  if (act == ORC_SWIGLU) return x * logistic(x);
  if (act == ORC_GEGLU_ERF) return x * normal_cdf(x);
  if (act == ORC_RELU2) return relu(x) * relu(x);
  double u = GELU_K0 * (x + GELU_K1 * x * x * x);
  double one_plus_t = 2.0 * logistic(2.0 * u);
  return 0.5 * x * one_plus_t;
}

/* act'(x):  silu'(x) = sigma(x) (1 + x (1 - sigma(x)));
 *           gelu_tanh'(x) = (1 + t)/2 + x/2 (1 - t^2) k0 (1 + 3 k1 x^2);
 *           gelu_erf'(x) = Phi(x) + x phi(x);
 *           relu2'(x) = 2 max(x, 0)  (0 at the kink x = 0, where both sides agree).
 * 1 - sigma(x) is sigma(-x); 1 - t^2 = (1 + t)(1 - t) with 1 -+ t = 2 sigma(-+2u)
 * for the same reason as above.  gelu_tanh' is taken in the factored form
 * (1 + t)/2 * (1 + x (1 - t) k0 (1 + 3 k1 x^2)), the same value, so that where it
 * underflows (x << 0) the zero keeps the sign of the exact, negative, derivative
 * instead of the +0 that a sum of two underflowed terms gives; gelu_erf' returns -0
 * there for the same reason. */
double orc_act_grad(int act, double x) {
  if (act == ORC_SWIGLU) return logistic(x) * (1.0 + x * logistic(-x));
  if (act == ORC_GEGLU_ERF) {
    double d = normal_cdf(x) + x * normal_pdf(x);
    /* both terms underflow for x << 0, where the exact derivative is negative */
    return (d == 0.0 && x < 0.0 && isfinite(x)) ? -0.0 : d;
  }
  if (act == ORC_RELU2) return 2.0 * relu(x);
  double u = GELU_K0 * (x + GELU_K1 * x * x * x);
  double one_plus_t = 2.0 * logistic(2.0 * u);
  double one_minus_t = 2.0 * logistic(-2.0 * u);
  return 0.5 * one_plus_t *
         (1.0 + x * one_minus_t * GELU_K0 * (1.0 + 3.0 * GELU_K1 * x * x));
}

/* ------------------------------------------------------------------------- */
/* GLU forward / backward on BF16 operands, one rounding at the store          */
/* ------------------------------------------------------------------------- */

/* Operand addressing.  SPLIT: gate and up are two [M, N] matrices with row
 * stride ld (the concatenated [gate | up] of [MX] API is SPLIT with up = gate + N
 * and ld = 2N).  PAIRED: one [M, 2N] matrix whose column 2j is gate_j and column
 * 2j+1 is up_j ([NV] Supported contract, weight layout row). */
static void load_pair(int layout, const uint16_t* gate, const uint16_t* up, int64_t ld,
                      int64_t m, int64_t j, double* g, double* u) {
  if (layout == ORC_PAIRED) {
    *g = orc_bf16_to_f64(gate[m * ld + 2 * j]);
    *u = orc_bf16_to_f64(gate[m * ld + 2 * j + 1]);
  } else {
    *g = orc_bf16_to_f64(gate[m * ld + j]);
    *u = orc_bf16_to_f64(up[m * ld + j]);
  }
}

/* h[m, j] = BF16(act(g) * u)  ([H] Fixed numerical paths: a single final rounding) */
void orc_glu_fwd(int act, int layout, int64_t M, int64_t N, const uint16_t* gate,
                 const uint16_t* up, int64_t ld, uint16_t* h, int64_t ldh) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; m++)
    for (int64_t j = 0; j < N; j++) {
      double g, u;
      load_pair(layout, gate, up, ld, m, j, &g, &u);
      h[m * ldh + j] = orc_bf16_from_f64(orc_act(act, g) * u);
    }
}

/* da = BF16(dh * u * act'(g)),  db = BF16(dh * act(g))  ([GE] Testing Done names
 * forward, da and db; [MX] API returns [dGate | dUp]).  SPLIT writes da and db as
 * two [M, N] matrices with row stride ldo; PAIRED writes one [M, 2N] matrix in the
 * input's interleaved order (da to column 2j, db to column 2j+1), db unused. */
void orc_glu_bwd(int act, int layout, int64_t M, int64_t N, const uint16_t* gate,
                 const uint16_t* up, int64_t ld, const uint16_t* dh, int64_t lddh,
                 uint16_t* da, uint16_t* db, int64_t ldo) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; m++)
    for (int64_t j = 0; j < N; j++) {
      double g, u;
      load_pair(layout, gate, up, ld, m, j, &g, &u);
      double d = orc_bf16_to_f64(dh[m * lddh + j]);
      uint16_t ra = orc_bf16_from_f64(d * u * orc_act_grad(act, g));
      uint16_t rb = orc_bf16_from_f64(d * orc_act(act, g));
      if (layout == ORC_PAIRED) {
        da[m * ldo + 2 * j] = ra;
        da[m * ldo + 2 * j + 1] = rb;
      } else {
        da[m * ldo + j] = ra;
        db[m * ldo + j] = rb;
      }
    }
}

/* ------------------------------------------------------------------------- */
/* MXFP8 quantizer ([MX] Summary: RCEIL E8M0 scale per 32 elements, E4M3 data)  */
/* ------------------------------------------------------------------------- */

/* One block of 32 values: scale byte and 32 codes. */
static void mx_block(const double* v, uint8_t* codes, uint8_t* scale) {
  int finite = 1;
  double amax = 0.0;
  for (int i = 0; i < 32; i++) {
    if (!isfinite(v[i])) finite = 0;
    else if (fabs(v[i]) > amax) amax = fabs(v[i]);
  }
  if (!finite) { /* reading: NaN scale and NaN codes */
    *scale = 0xFF;
    for (int i = 0; i < 32; i++) codes[i] = 0x7F;
    return;
  }
  int e = orc_mx_scale_exponent(amax);
  *scale = (uint8_t)(e + 127);
  for (int i = 0; i < 32; i++) codes[i] = orc_e4m3_from_f64(ldexp(v[i], -e)); /* exact */
}

/* Bytes of a [rows, nb] scale matrix: row-major, or the zero-padded 128x4 layout
 * (reading: the GEMM-ready layout the pages name for block scales, also used for the
 * MXFP8 scales when asked for; rows padded to a multiple of 128, columns to 4). */
int64_t orc_mx_sf_bytes(int64_t rows, int64_t nb, int swizzled) {
  if (!swizzled) return rows * nb;
  return (rows + 127) / 128 * 128 * ((nb + 3) / 4 * 4);
}

int64_t orc_sf128x4_offset(int64_t r, int64_t c, int64_t scale_cols_padded);

/* Position of scale (r, c) of a [rows, nb] scale matrix. */
static int64_t sf_pos(int64_t r, int64_t c, int64_t nb, int swizzled) {
  return swizzled ? orc_sf128x4_offset(r, c, (nb + 3) / 4 * 4) : r * nb + c;
}

/* X is a row-major [M, N] matrix of FP32 values (BF16 values widened exactly are
 * FP32 values).  Rowwise: blocks X[m, 32b .. 32b+31], codes [M, N], scales
 * [M, N/32].  Colwise: blocks X[32b .. 32b+31, j], codes stored transposed as
 * [N, M] (row j holds column j of X), scales [N, M/32].  With ORC_SF_SWIZZLED in
 * flags both scale matrices use the zero-padded 128x4 layout instead. */
void orc_quant_mxfp8(int64_t M, int64_t N, const float* X, int flags, uint8_t* q_row,
                     uint8_t* s_row, uint8_t* q_col, uint8_t* s_col) {
  const int swz = (flags & ORC_SF_SWIZZLED) != 0;
  if (flags & ORC_ROWWISE) {
    if (swz) memset(s_row, 0, (size_t)orc_mx_sf_bytes(M, N / 32, 1));
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++)
      for (int64_t b = 0; b < N / 32; b++) {
        double v[32];
        uint8_t c[32];
        for (int i = 0; i < 32; i++) v[i] = X[m * N + 32 * b + i];
        mx_block(v, c, &s_row[sf_pos(m, b, N / 32, swz)]);
        memcpy(&q_row[m * N + 32 * b], c, 32);
      }
  }
  if (flags & ORC_COLWISE) {
    if (swz) memset(s_col, 0, (size_t)orc_mx_sf_bytes(N, M / 32, 1));
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < N; j++)
      for (int64_t b = 0; b < M / 32; b++) {
        double v[32];
        uint8_t c[32];
        for (int i = 0; i < 32; i++) v[i] = X[(32 * b + i) * N + j];
        mx_block(v, c, &s_col[sf_pos(j, b, M / 32, swz)]);
        memcpy(&q_col[j * M + 32 * b], c, 32);
      }
  }
}

/* ------------------------------------------------------------------------- */
/* NVFP4 quantizer, global scale 1 ([NV] Supported contract)                   */
/* ------------------------------------------------------------------------- */

/* Byte offset of scale (r, c) in the 128x4 layout (reading: the public
 * cuBLAS/CUTLASS block-scale layout that the page names; rows padded to a
 * multiple of 128, scale columns to a multiple of 4). */
int64_t orc_sf128x4_offset(int64_t r, int64_t c, int64_t scale_cols_padded) {
  return ((r / 128) * (scale_cols_padded / 4) + c / 4) * 512 + (r % 32) * 16 +
         ((r % 128) / 32) * 4 + (c % 4);
}

/* One block of 16 values: E4M3 scale byte and 16 E2M1 codes (one per byte). */
static void nv_block(const double* v, uint8_t* codes, uint8_t* scale) {
  int finite = 1;
  double amax = 0.0;
  for (int i = 0; i < 16; i++) {
    if (!isfinite(v[i])) finite = 0;
    else if (fabs(v[i]) > amax) amax = fabs(v[i]);
  }
  if (!finite) { /* reading: NaN scale, zero codes */
    *scale = 0x7F;
    memset(codes, 0, 16);
    return;
  }
  /* Reading: S = E4M3(amax / 6), nearest; then codes = E2M1(x / S).  The binary64
   * quotients take the same rounding decision as the exact ones for FP32 inputs. */
  uint8_t sc = orc_e4m3_from_f64(amax / 6.0);
  double S = orc_e4m3_to_f64(sc);
  *scale = sc;
  for (int i = 0; i < 16; i++) {
    if (S == 0.0) codes[i] = signbit(v[i]) ? 0x8 : 0x0;
    else codes[i] = orc_e2m1_from_f64(v[i] / S);
  }
}

/* X is row-major [M, H] FP32.  q is [M, H/2] bytes, element 2k in the low nibble
 * of byte k and element 2k+1 in the high nibble.  sf is [M, H/16] row-major, or
 * the zero-padded 128x4 layout of ceil(M/128)*128 rows x ceil(H/64)*4 columns. */
void orc_quant_nvfp4(int64_t M, int64_t H, const float* X, uint8_t* q, uint8_t* sf,
                     int sf_layout) {
  int64_t nb = H / 16;
  int64_t cols_padded = (nb + 3) / 4 * 4;
  int64_t rows_padded = (M + 127) / 128 * 128;
  if (sf_layout == ORC_SF_128x4) memset(sf, 0, (size_t)(rows_padded * cols_padded));
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; m++)
    for (int64_t b = 0; b < nb; b++) {
      double v[16];
      uint8_t c[16], s;
      for (int i = 0; i < 16; i++) v[i] = X[m * H + 16 * b + i];
      nv_block(v, c, &s);
      for (int k = 0; k < 8; k++)
        q[m * (H / 2) + 8 * b + k] = (uint8_t)(c[2 * k] | (c[2 * k + 1] << 4));
      if (sf_layout == ORC_SF_128x4) sf[orc_sf128x4_offset(m, b, cols_padded)] = s;
      else sf[m * nb + b] = s;
    }
}

/* ------------------------------------------------------------------------- */
/* NVFP4 with a global scale (two-level scaling).  [NV] Supported contract fixes */
/* global scale 1; this is the relaxation real recipes use, by reading: every   */
/* step below is one IEEE FP32 operation, as the kernels take it.               */
/* ------------------------------------------------------------------------- */

/* Global encode scale: 448 * 6 / amax in FP32, so that the block holding the tensor's
 * amax gets (about) the largest E4M3 scale; 1 when amax is zero, negative or not finite.
 * Capped at 2^100 (amax below about 2^-89): then s / S and x * s / S stay finite for
 * every E4M3 scale S >= 2^-9 and every x up to amax. */
float orc_nvfp4_global_scale(float amax) {
  if (!(amax > 0.0f) || !isfinite(amax)) return 1.0f;
  const float s = 2688.0f / amax;
  return s < 0x1p100f ? s : 0x1p100f;
}

/* One block of 16 FP32 values at global encode scale s (k = fl(s / 6)):
 *   scale code = E4M3(fl(bamax * k)), nearest even, saturating at 448;
 *   codes      = E2M1(fl(x * r)), r = fl(s / S) with S the scale code's value (r = 0
 *                when S = 0, giving signed zeros), nearest even, saturating at 6;
 * a block holding NaN or Inf gets scale 0x7F and zero codes, as with global scale 1. */
static void nv_block_gs(const float* v, float s, float k, uint8_t* codes, uint8_t* scale) {
  float amax = 0.0f;
  for (int i = 0; i < 16; i++) {
    if (!isfinite(v[i])) {
      *scale = 0x7F;
      memset(codes, 0, 16);
      return;
    }
    if (fabsf(v[i]) > amax) amax = fabsf(v[i]);
  }
  const float d = amax * k;
  const uint8_t sc = orc_e4m3_from_f64((double)d);
  const float S = (float)orc_e4m3_to_f64(sc);
  const float r = S == 0.0f ? 0.0f : s / S;
  *scale = sc;
  for (int i = 0; i < 16; i++) {
    const float y = v[i] * r;
    codes[i] = orc_e2m1_from_f64((double)y);
  }
}

/* As orc_quant_nvfp4, with the global encode scale of `amax`. */
void orc_quant_nvfp4_gs(int64_t M, int64_t H, const float* X, float amax, uint8_t* q,
                        uint8_t* sf, int sf_layout) {
  const float s = orc_nvfp4_global_scale(amax);
  const float k = s / 6.0f;
  int64_t nb = H / 16;
  int64_t cols_padded = (nb + 3) / 4 * 4;
  int64_t rows_padded = (M + 127) / 128 * 128;
  if (sf_layout == ORC_SF_128x4) memset(sf, 0, (size_t)(rows_padded * cols_padded));
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; m++)
    for (int64_t b = 0; b < nb; b++) {
      uint8_t c[16], sc;
      nv_block_gs(&X[m * H + 16 * b], s, k, c, &sc);
      for (int j = 0; j < 8; j++)
        q[m * (H / 2) + 8 * b + j] = (uint8_t)(c[2 * j] | (c[2 * j + 1] << 4));
      if (sf_layout == ORC_SF_128x4) sf[orc_sf128x4_offset(m, b, cols_padded)] = sc;
      else sf[m * nb + b] = sc;
    }
}

/* ------------------------------------------------------------------------- */
/* Fused paths = GLU (one BF16 rounding) followed by the quantizer             */
/* ([MX] Numerics and tests: equal to the activation then the quantizers)      */
/* ------------------------------------------------------------------------- */

static float* widen_bf16(const uint16_t* b, int64_t n) {
  float* f = (float*)malloc((size_t)n * sizeof(float));
  if (!f) return NULL;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) f[i] = (float)orc_bf16_to_f64(b[i]);
  return f;
}

/* Returns 0 on success, -1 if host memory ran out. */
int orc_glu_fwd_mxfp8(int act, int layout, int64_t M, int64_t N, const uint16_t* gate,
                      const uint16_t* up, int64_t ld, int flags, uint8_t* q_row,
                      uint8_t* s_row, uint8_t* q_col, uint8_t* s_col) {
  uint16_t* h = (uint16_t*)malloc((size_t)(M * N) * sizeof(uint16_t));
  if (!h) return -1;
  orc_glu_fwd(act, layout, M, N, gate, up, ld, h, N);
  float* x = widen_bf16(h, M * N);
  free(h);
  if (!x) return -1;
  orc_quant_mxfp8(M, N, x, flags, q_row, s_row, q_col, s_col);
  free(x);
  return 0;
}

/* Backward: the quantized matrix is [da | db], [M, 2N] ([MX] API). */
int orc_glu_bwd_mxfp8(int act, int64_t M, int64_t N, const uint16_t* gate,
                      const uint16_t* up, int64_t ld, const uint16_t* dh, int64_t lddh,
                      int flags, uint8_t* q_row, uint8_t* s_row, uint8_t* q_col,
                      uint8_t* s_col) {
  uint16_t* d = (uint16_t*)malloc((size_t)(M * 2 * N) * sizeof(uint16_t));
  if (!d) return -1;
  orc_glu_bwd(act, ORC_SPLIT, M, N, gate, up, ld, dh, lddh, d, d + N, 2 * N);
  float* x = widen_bf16(d, M * 2 * N);
  free(d);
  if (!x) return -1;
  orc_quant_mxfp8(M, 2 * N, x, flags, q_row, s_row, q_col, s_col);
  free(x);
  return 0;
}

int orc_glu_fwd_nvfp4(int act, int layout, int64_t M, int64_t H, const uint16_t* gate,
                      const uint16_t* up, int64_t ld, uint8_t* q, uint8_t* sf,
                      int sf_layout) {
  uint16_t* h = (uint16_t*)malloc((size_t)(M * H) * sizeof(uint16_t));
  if (!h) return -1;
  orc_glu_fwd(act, layout, M, H, gate, up, ld, h, H);
  float* x = widen_bf16(h, M * H);
  free(h);
  if (!x) return -1;
  orc_quant_nvfp4(M, H, x, q, sf, sf_layout);
  free(x);
  return 0;
}

/* Backward with NVFP4 output: [da | db], [M, 2N], quantized in 16-element row blocks as
 * the forward's h is (the MXFP8 backward's placement, [MX] API, carried over to NVFP4;
 * no page defines an NVFP4 backward). */
int orc_glu_bwd_nvfp4(int act, int64_t M, int64_t N, const uint16_t* gate,
                      const uint16_t* up, int64_t ld, const uint16_t* dh, int64_t lddh,
                      uint8_t* q, uint8_t* sf, int sf_layout) {
  uint16_t* d = (uint16_t*)malloc((size_t)(M * 2 * N) * sizeof(uint16_t));
  if (!d) return -1;
  orc_glu_bwd(act, ORC_SPLIT, M, N, gate, up, ld, dh, lddh, d, d + N, 2 * N);
  float* x = widen_bf16(d, M * 2 * N);
  free(d);
  if (!x) return -1;
  orc_quant_nvfp4(M, 2 * N, x, q, sf, sf_layout);
  free(x);
  return 0;
}

/* Largest |h| of h = bf16(act(gate) * up) over [M, N]: NaN if some h is NaN.  The amax
 * pass of two-level NVFP4 scaling.  Returns -1 in *ok if host memory ran out. */
float orc_glu_amax(int act, int layout, int64_t M, int64_t N, const uint16_t* gate,
                   const uint16_t* up, int64_t ld, int* ok) {
  uint16_t* h = (uint16_t*)malloc((size_t)(M * N) * sizeof(uint16_t));
  *ok = h ? 0 : -1;
  if (!h) return 0.0f;
  orc_glu_fwd(act, layout, M, N, gate, up, ld, h, N);
  float amax = 0.0f;
  int nan = 0;
  for (int64_t i = 0; i < M * N; i++) {
    const float a = fabsf((float)orc_bf16_to_f64(h[i]));
    if (isnan(a)) nan = 1;
    else if (a > amax) amax = a;
  }
  free(h);
  return nan ? NAN : amax;
}

/* Fused forward with two-level NVFP4 scaling: h as orc_glu_fwd, quantized with the global
 * encode scale of the given amax (normally orc_glu_amax of the same operands). */
int orc_glu_fwd_nvfp4_gs(int act, int layout, int64_t M, int64_t H, const uint16_t* gate,
                         const uint16_t* up, int64_t ld, float amax, uint8_t* q, uint8_t* sf,
                         int sf_layout) {
  uint16_t* h = (uint16_t*)malloc((size_t)(M * H) * sizeof(uint16_t));
  if (!h) return -1;
  orc_glu_fwd(act, layout, M, H, gate, up, ld, h, H);
  float* x = widen_bf16(h, M * H);
  free(h);
  if (!x) return -1;
  orc_quant_nvfp4_gs(M, H, x, amax, q, sf, sf_layout);
  free(x);
  return 0;
}

/* ------------------------------------------------------------------------- */
/* Merged gate/up MXFP8 GEMM with the GLU (and its quantizer) as the epilogue:  */
/* the placement of [NV] Summary (the fold follows the merged GEMM), in the     */
/* MXFP8 form of [MX] Performance's fused-w13 MoE composite; [MX] API fixes the */
/* [gate | up] packing of what a fused w13 projection produces.                */
/* ------------------------------------------------------------------------- */

/* E8M0 scale byte -> 2^(b - 127); 0xFF is NaN. */
static double e8m0(uint8_t b) { return b == 0xFF ? NAN : ldexp(1.0, (int)b - 127); }

enum { ORC_FMT_E4M3 = 0, ORC_FMT_E2M1 = 1 };

/* Decoded code of element k of a GEMM operand row: E4M3 one per byte, or E2M1 two per byte
 * with element 2j in the low nibble of byte j. */
static double operand_code(int fmt, const uint8_t* row, int64_t k) {
  if (fmt == ORC_FMT_E2M1) {
    const uint8_t b = row[k / 2];
    return orc_e2m1_to_f64((uint8_t)((k & 1) ? b >> 4 : b & 15));
  }
  return orc_e4m3_to_f64(row[k]);
}

/* Y = X W^T in binary64: X is [M, K] codes with E8M0 scales [M, K/32] (32-element blocks
 * along K), W is [N2, K] codes with scales [N2, K/32]; codes in format fmt (a row of K
 * elements takes K bytes for E4M3, K/2 for E2M1).  Every product of two decoded values is
 * exact in binary64; the sum runs over k in order.  Y keeps W's row order. */
void orc_mx_gemm_nt(int fmt, int64_t M, int64_t N2, int64_t K, const uint8_t* Xq,
                    const uint8_t* Xs, const uint8_t* Wq, const uint8_t* Ws, double* Y) {
  const int64_t kb = K / 32, rb = fmt == ORC_FMT_E2M1 ? K / 2 : K;
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; m++)
    for (int64_t n = 0; n < N2; n++) {
      double acc = 0.0;
      for (int64_t b = 0; b < kb; b++) {
        const double sx = e8m0(Xs[m * kb + b]), sw = e8m0(Ws[n * kb + b]);
        double blk = 0.0;
        for (int64_t k = 32 * b; k < 32 * b + 32; k++)
          blk += operand_code(fmt, Xq + m * rb, k) * operand_code(fmt, Wq + n * rb, k);
        acc += blk * sx * sw;
      }
      Y[m * N2 + n] = acc;
    }
}

/* Columns of Y = X W^T holding gate and up output j: W = [W_gate | W_up] puts them at j and
 * N + j; pairwise-interleaved W rows at 2j and 2j + 1. */
static int64_t gate_col(int w_layout, int64_t j) { return w_layout == ORC_PAIRED ? 2 * j : j; }
static int64_t up_col(int w_layout, int64_t N, int64_t j) { return w_layout == ORC_PAIRED ? 2 * j + 1 : N + j; }

/* h = bf16(act(Y_gate) * Y_up) with Y = X W^T, W [2N, K] in w_layout.  One rounding, from
 * binary64. */
int orc_glu_gemm(int act, int fmt, int w_layout, int64_t M, int64_t N, int64_t K,
                 const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq, const uint8_t* Ws,
                 uint16_t* h) {
  double* Y = (double*)malloc((size_t)(M * 2 * N) * sizeof(double));
  if (!Y) return -1;
  orc_mx_gemm_nt(fmt, M, 2 * N, K, Xq, Xs, Wq, Ws, Y);
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; m++)
    for (int64_t j = 0; j < N; j++)
      h[m * N + j] = orc_bf16_from_f64(orc_act(act, Y[m * 2 * N + gate_col(w_layout, j)]) *
                                       Y[m * 2 * N + up_col(w_layout, N, j)]);
  free(Y);
  return 0;
}

/* The same with h quantized to MXFP8 rowwise (1x32 blocks along N). */
int orc_glu_gemm_mxfp8(int act, int fmt, int w_layout, int64_t M, int64_t N, int64_t K,
                       const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq, const uint8_t* Ws,
                       uint8_t* q_row, uint8_t* s_row) {
  uint16_t* h = (uint16_t*)malloc((size_t)(M * N) * sizeof(uint16_t));
  if (!h) return -1;
  if (orc_glu_gemm(act, fmt, w_layout, M, N, K, Xq, Xs, Wq, Ws, h) != 0) {
    free(h);
    return -1;
  }
  float* x = widen_bf16(h, M * N);
  free(h);
  if (!x) return -1;
  orc_quant_mxfp8(M, N, x, ORC_ROWWISE, q_row, s_row, NULL, NULL);
  free(x);
  return 0;
}

/* Element-wise encoders over arrays, for the format pins. */
void orc_bf16_from_f64_array(const double* v, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) out[i] = orc_bf16_from_f64(v[i]);
}
void orc_e4m3_from_f64_array(const double* v, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) out[i] = orc_e4m3_from_f64(v[i]);
}
void orc_e2m1_from_f64_array(const double* v, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) out[i] = orc_e2m1_from_f64(v[i]);
}
void orc_act_array(int act, const double* x, int64_t n, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) out[i] = orc_act(act, x[i]);
}
void orc_act_grad_array(int act, const double* x, int64_t n, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) out[i] = orc_act_grad(act, x[i]);
}
