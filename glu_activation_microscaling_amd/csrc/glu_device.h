// Device helpers for the fused GLU + microscaling kernels (gfx950, wave64).
//
// Numerics, following "Add swiglu + MXFP8 fused CuTe DSL kernel" (Summary; Numerics and
// tests) and "[WS1] Add batch-invariant h_aggregate kernel" (Fixed numerical paths):
// the activation is evaluated in FP32 and rounded once to BF16 (nearest even); the
// quantizers then see exactly that BF16 value.  All quantizer decisions below are exact
// for every finite FP32 input: the MX scale is a power of two (the scaled value is
// exact), and the NVFP4 decisions compare against exactly representable thresholds.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "glu_common.h"

#if defined(__FAST_MATH__)
#error "build without fast-math: the quantizer decisions rely on IEEE FP32 arithmetic"
#endif

namespace glu {

// ---------------------------------------------------------------------------------
// BF16 <-> FP32
// ---------------------------------------------------------------------------------

// The two BF16 halves of a 32-bit word, widened exactly.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// FP32 -> BF16 bits, round to nearest even; FP32 subnormals round like any other value;
// NaN becomes a quiet NaN with its sign.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  return ((u & 0x7fffffffu) > 0x7f800000u) ? (((u >> 16) & 0x8000u) | 0x7fc0u) : r;
}

// Rounds to BF16 and returns the rounded value as FP32 (what the quantizer consumes).
__device__ __forceinline__ float round_bf16(float f) { return __uint_as_float(bf16_rne(f) << 16); }

// ---------------------------------------------------------------------------------
// Activations, act(g) applied to the gate and multiplied by up:
//   SWIGLU       silu(x) = x sigma(x);
//   GEGLU_TANH   x/2 (1 + tanh(u)), u = k0 (x + k1 x^3), written as x sigma(2u);
//   GEGLU_ERF    x Phi(x), Phi the standard normal CDF (the exact GELU);
//   RELU2        max(x, 0)^2.
// For the first two act(x) = x sigma(z(x)) and act'(x) = sigma(z) (1 + x sigma(-z) z'(x)).
// Each activation has a fast FP32 path and a rare FP64 tail path for the elements where the
// fast path could lose accuracy; fwd_tail_needed / bwd_tail_needed say which, and the kernels
// recompute those elements (wave-divergent, rare for real data):
//   sigmoid forms: z log2(e) < -125, where e^z leaves the FP32 normal range;
//   erf-GELU:      x < -12.5, where Phi(x) nears the bottom of the FP32 normal range;
//   ReLU^2:        an intermediate product that is not an FP32 normal number (see relu).
// ---------------------------------------------------------------------------------

constexpr float LOG2E = 1.44269504088896340736f;
constexpr double GELU_K0 = 0.79788456080286535588;  // sqrt(2/pi)
constexpr double GELU_K1 = 0.044715;
constexpr float GEGLU_C0 = (float)(2.0 * GELU_K0 * 1.44269504088896340736);            // 2 k0 log2 e
constexpr float GEGLU_C1 = (float)(2.0 * GELU_K0 * GELU_K1 * 1.44269504088896340736);  // 2 k0 k1 log2 e
constexpr float GEGLU_D0 = (float)(2.0 * GELU_K0);                                     // z'(x) = D0 + D1 x^2
constexpr float GEGLU_D1 = (float)(6.0 * GELU_K0 * GELU_K1);
constexpr float TAIL_ZL2 = -125.0f;
constexpr double SQRT1_2 = 0.70710678118654752440;       // 1/sqrt(2)
constexpr double INV_SQRT_2PI = 0.39894228040143267794;  // 1/sqrt(2 pi)
constexpr float ERF_TAIL_X = -12.5f;

// z(x) * log2(e) of the sigmoid forms
template <int ACT>
__device__ __forceinline__ float zl2(float x) {
  if constexpr (ACT == SWIGLU) {
    return x * LOG2E;
  } else {
    return x * __builtin_fmaf(x * x, GEGLU_C1, GEGLU_C0);
  }
}

// Wave-level trigger of the tail path from raw BF16 gate bit patterns: m16 is their maximum
// as unsigned 16-bit numbers, under which negative values order by magnitude above 0x8000
// and non-negative ones stay below.  True when some gate value is below G, where every
// g >= G takes the fast path: SwiGLU G = -80 (zl2 >= -115.5), tanh-GeGLU G = -9.5
// (zl2 >= -110.2), erf-GeGLU G = -12.5 (the bound itself).  Negative NaNs trigger it too
// (harmless: both paths return NaN).
// ReLU^2's tail depends on all operands, so it has no trigger of this kind.
template <int ACT>
constexpr bool tail_from_gate_bits() { return ACT != RELU2; }
template <int ACT>
__device__ __forceinline__ bool tail_possible(uint32_t m16) {
  static_assert(tail_from_gate_bits<ACT>());
  return m16 > (ACT == SWIGLU ? 0xC2A0u : ACT == GEGLU_TANH ? 0xC118u : 0xC148u);  // -80, -9.5, -12.5
}

// e^-z = 2^-zl and sigma(z) = 1 / (1 + e^-z) from zl = z log2(e); accurate for
// zl >= TAIL_ZL2 (for zl << 0 the exp overflows towards +Inf and sigma goes to 0, which the
// FP64 tail path replaces).  sigma(-z) = e^-z sigma(z) is accurate in the same range.
__device__ __forceinline__ float exp_neg(float zl) { return __builtin_amdgcn_exp2f(-zl); }
__device__ __forceinline__ float sigmoid_from(float e) { return __builtin_amdgcn_rcpf(1.0f + e); }

// z'(x); x is clamped so that z' stays finite (where it would not, sigma(-z) is 0).
template <int ACT>
__device__ __forceinline__ float dz(float x) {
  if constexpr (ACT == SWIGLU) {
    return 1.0f;
  } else {
    float xc = __builtin_amdgcn_fmed3f(x, -1.0e15f, 1.0e15f);
    return __builtin_fmaf(xc * xc, GEGLU_D1, GEGLU_D0);
  }
}

// Tail path of the sigmoid forms, z log2(e) = zl < TAIL_ZL2: e^z = 2^zl is below the FP32
// normal range, so it is formed in FP64 as exp2(f) * 2^n with n = floor(zl), f = zl - n
// (exact), and the products are taken in FP64 (no intermediate overflow or underflow).
// There 1 + e^z == 1, so sigma(z) = e^z and sigma(-z) = 1.  zl is clamped where e^z is 0
// in FP64 anyway.
__device__ __forceinline__ double exp2_tail(float zl) {
  const float zc = __builtin_fmaxf(zl, -1100.0f);
  const float n = __builtin_floorf(zc);
  return __builtin_ldexp((double)__builtin_amdgcn_exp2f(zc - n), (int)n);
}

// erf-GELU.  Phi(x) = erfc(-x / sqrt 2) / 2 and phi(x) = exp(-x^2 / 2) / sqrt(2 pi);
// act'(x) = Phi(x) + x phi(x).
//
// FP32 fast path (x >= -12.5; below that the FP64 tail): with z = |x| / sqrt 2,
//   erfc(z) = t e^(-z^2 + Q(t)),  t = 1 / (1 + z/2),
// Q a degree-7 polynomial fitted to ln(erfc(z)/t) + z^2 for |x| <= 12.75 (max error
// 7.0e-7; gen_erfc_poly.py prints the coefficients), and Phi = erfc(z)/2 for x < 0,
// 1 - erfc(z)/2 otherwise.  x is clamped to +-12.75: beyond it Phi is 1 in FP32 (x > 0) or
// the tail path applies (x < 0).  z^2 = x^2 / 2 is exact for a BF16 x, and e^(-z^2 + q) is
// one exp2 of the FP32 exponent (q - z^2) log2(e): its two roundings cost at most 7e-6
// (relative) at |x| = 12.75 and under 2e-7 for |x| < 2, against 7e-7 for Q.  (Carrying the
// exponent to 40 bits as 2^n 2^f, with log2 e split so that its 8-bit head times z^2 is
// exact, took five more instructions per exponential and changed no BF16 result of a CPU
// model on random data.)
constexpr float ERFC_Q[8] = {-1.265515924e+00f, 9.991499186e-01f,  3.906860054e-01f,
                             -2.971511893e-02f, 3.325169683e-01f,  -9.836239219e-01f,
                             7.421878576e-01f,  -1.856864840e-01f};
constexpr float ERF_X_CLAMP = 12.75f;

// e^(-w + q) for 0 <= w <= 82, |q| <= 2 (the result stays a normal FP32 number).
__device__ __forceinline__ float exp_neg_w_plus(float w, float q) {
  return __builtin_amdgcn_exp2f((q - w) * LOG2E);
}

struct ErfParts {
  float xc, w, t, q;  // clamped x, z^2 = xc^2 / 2, t, Q(t)
};
__device__ __forceinline__ ErfParts erf_parts(float x) {
  ErfParts p;
  p.xc = __builtin_amdgcn_fmed3f(x, -ERF_X_CLAMP, ERF_X_CLAMP);
  p.w = (0.5f * p.xc) * p.xc;
  p.t = __builtin_amdgcn_rcpf(__builtin_fmaf(__builtin_fabsf(p.xc), (float)(0.5 * SQRT1_2), 1.0f));
  float q = ERFC_Q[7];
#pragma unroll
  for (int i = 6; i >= 0; i--) q = __builtin_fmaf(q, p.t, ERFC_Q[i]);
  p.q = q;
  return p;
}
// Phi from erfc(|x| / sqrt 2)
__device__ __forceinline__ float phi_from_erfc(float xc, float e) {
  return xc < 0.0f ? 0.5f * e : __builtin_fmaf(-0.5f, e, 1.0f);
}
__device__ __forceinline__ float phi_cdf(float x) {
  const ErfParts p = erf_parts(x);
  return phi_from_erfc(p.xc, p.t * exp_neg_w_plus(p.w, p.q));
}
// Phi(x) and phi(x) together, sharing e^(-z^2); phi is 0 beyond the clamp (so that x phi(x)
// is 0 for large finite x and NaN for infinite x, as in x e^(-x^2/2)).
__device__ __forceinline__ void phi_cdf_pdf(float x, float& cdf, float& pdf) {
  const ErfParts p = erf_parts(x);
  const float ew = exp_neg_w_plus(p.w, 0.0f);
  cdf = phi_from_erfc(p.xc, (p.t * __builtin_amdgcn_exp2f(p.q * LOG2E)) * ew);
  pdf = __builtin_fabsf(x) <= ERF_X_CLAMP ? (float)INV_SQRT_2PI * ew : 0.0f;
}

// FP64 tail, x < -12.5 (z = |x|/sqrt 2 > 8.8): Phi(x) = phi(x) S(v) / |x| with the asymptotic
// series of the Mills ratio, S = 1 - v + 3v^2 - 15v^3 + 105v^4 - 945v^5 + 10395v^6,
// v = 1/x^2 (truncation error below 1e-10 relative at x = -12.5, smaller beyond).  FP64 is
// there for the range (phi(x) leaves FP32 near x = -13.5); e^(-x^2/2) = 2^y is formed as
// exp2(f) 2^n with n = floor(y), f = y - n, and is 0 where it is below the FP64 range.
__device__ __forceinline__ void phi_tail64(float x, double& cdf, double& grad) {
  const double xd = (double)x;
  const double r = 1.0 / __builtin_fabs(xd), v = r * r;
  double pdf, sv = 10395.0;
  sv = __builtin_fma(sv, v, -945.0);
  sv = __builtin_fma(sv, v, 105.0);
  sv = __builtin_fma(sv, v, -15.0);
  sv = __builtin_fma(sv, v, 3.0);
  sv = __builtin_fma(sv, v, -1.0);
  sv = __builtin_fma(sv, v, 1.0);
  const double y = __builtin_fmax(-0.5 * xd * xd * 1.44269504088896340736, -1100.0);
  const double n = __builtin_floor(y);
  pdf = INV_SQRT_2PI * __builtin_ldexp((double)__builtin_amdgcn_exp2f((float)(y - n)), (int)n);
  cdf = (pdf * sv) * r;
  grad = pdf * (sv * r + xd);  // Phi + x phi, negative (or -0 where phi underflows)
}

// ReLU^2.  r = max(x, 0) with NaN kept NaN.  A product of two BF16 values has at most 16
// significant bits and one of three at most 24, so in FP32 each is exact while it is a
// normal number, and the last product is the correctly rounded exact value whatever its
// range.  The fast path forms h = (r r) u, db = (dh r) r, da = ((dh + dh) u) r; an element
// whose first product (r r, dh r or (dh + dh) u) is not a normal FP32 number (over- or
// underflow, a zero that is not exact, or NaN) goes to the FP64 tail, where every product is
// exact.
__device__ __forceinline__ float relu(float x) { return x <= 0.0f ? 0.0f : x; }
__device__ __forceinline__ bool fp32_normal(float x) {
  return __builtin_amdgcn_classf(x, 0x108);  // -normal | +normal
}

template <int ACT>
__device__ __forceinline__ bool fwd_tail_needed(float g, float u) {
  if constexpr (ACT == RELU2) {
    const float r = relu(g);
    return r != 0.0f && !fp32_normal(r * r);
  } else if constexpr (ACT == GEGLU_ERF) {
    return g < ERF_TAIL_X;
  } else {
    return zl2<ACT>(g) < TAIL_ZL2;
  }
}
template <int ACT>
__device__ __forceinline__ bool bwd_tail_needed(float g, float u, float d) {
  if constexpr (ACT == RELU2) {
    const float r = relu(g);
    return !fp32_normal((d + d) * u) || (r != 0.0f && !fp32_normal(d * r));
  } else {
    return fwd_tail_needed<ACT>(g, u);
  }
}

// Forward: act(g) * u in FP32 (the caller rounds it to BF16); the tail elements are
// recomputed by glu_fwd_tail.
template <int ACT>
__device__ __forceinline__ float glu_fwd_fast(float g, float u) {
  if constexpr (ACT == GEGLU_ERF) {
    return (g * phi_cdf(g)) * u;
  } else if constexpr (ACT == RELU2) {
    const float r = relu(g);
    return (r * r) * u;
  } else {
    return (g * sigmoid_from(exp_neg(zl2<ACT>(g)))) * u;
  }
}
template <int ACT>
__device__ __forceinline__ float glu_fwd_elem(float g, float u, bool& tail) {
  tail |= fwd_tail_needed<ACT>(g, u);
  return glu_fwd_fast<ACT>(g, u);
}

template <int ACT>
__device__ __forceinline__ float glu_fwd_tail(float g, float u) {
  if constexpr (ACT == GEGLU_ERF) {
    double cdf, grad;
    phi_tail64(g, cdf, grad);
    return (float)((double)g * cdf * (double)u);
  } else if constexpr (ACT == RELU2) {
    const double r = (double)relu(g);
    return (float)((r * r) * (double)u);
  } else {
    return (float)((double)g * exp2_tail(zl2<ACT>(g)) * (double)u);
  }
}

// Backward: da = dh u act'(g), db = dh act(g), FP32 before rounding.  Sigmoid forms:
// q = dh sigma(z), db = q g, da = (q u)(1 + (g sigma(-z)) z'(g)); g sigma(-z) is taken
// before z'(g): for large g, z'(g) g overflows while sigma(-z) is 0.
template <int ACT>
__device__ __forceinline__ void glu_bwd_fast(float g, float u, float d, float& da, float& db) {
  if constexpr (ACT == GEGLU_ERF) {
    float p, pd;
    phi_cdf_pdf(g, p, pd);
    db = d * (g * p);
    da = (d * u) * __builtin_fmaf(g, pd, p);
  } else if constexpr (ACT == RELU2) {
    const float r = relu(g);
    db = (d * r) * r;
    da = ((d + d) * u) * r;
  } else {
    const float e = exp_neg(zl2<ACT>(g));
    const float sp = sigmoid_from(e);  // sigma(z)
    const float q = d * sp;
    db = q * g;
    const float sn = e * sp;           // sigma(-z)
    const float s = ACT == SWIGLU ? __builtin_fmaf(g, sn, 1.0f) : __builtin_fmaf(g * sn, dz<ACT>(g), 1.0f);
    da = (q * u) * s;
  }
}
template <int ACT>
__device__ __forceinline__ void glu_bwd_elem(float g, float u, float d, float& da, float& db,
                                             bool& tail) {
  tail |= bwd_tail_needed<ACT>(g, u, d);
  glu_bwd_fast<ACT>(g, u, d, da, db);
}

template <int ACT>
__device__ __forceinline__ void glu_bwd_tail(float g, float u, float d, float& da, float& db) {
  const double gd = (double)g;
  if constexpr (ACT == GEGLU_ERF) {
    double cdf, grad;
    phi_tail64(g, cdf, grad);
    db = (float)((double)d * (gd * cdf));
    da = (float)((double)d * (double)u * grad);
  } else if constexpr (ACT == RELU2) {
    const double r = (double)relu(g), dd = (double)d;
    db = (float)(dd * (r * r));
    da = (float)((dd * (double)u) * (2.0 * r));
  } else {
    const double t = exp2_tail(zl2<ACT>(g));
    da = (float)((double)d * (double)u * t * (1.0 + gd * (double)dz<ACT>(g)));
    db = (float)((double)d * gd * t);
  }
}

// ---------------------------------------------------------------------------------
// gfx950 conversion instructions.  Each is used only where it was shown, on the device, to
// equal the software encoder in this file bit for bit over its whole input domain:
//   v_cvt_pk_bf16_f32            == bf16_rne on every non-NaN FP32 (NaN stays NaN);
//   v_cvt_pk_fp8_f32             == e4m3_sw on every FP32 with |y| <= 448;
//   v_cvt_scalef32_pk_fp8_bf16   == e4m3_sw(x * 2^-e) for every BF16 x and scale 2^e,
//                                   e in [-127, 120], with |x * 2^-e| <= 448 (the scale
//                                   operand's exponent alone is used; 2^-127 is passed as
//                                   the FP32 subnormal 0x00400000);
//   v_cvt_scalef32_pk_fp4_f32    == nearest-even E2M1 with saturation at scale 1.
// ---------------------------------------------------------------------------------

typedef short v2i16 __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));
typedef float v2f32 __attribute__((ext_vector_type(2)));

// Two FP32 values -> packed BF16 pair (lo in bits 0..15), nearest even.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  v2f32 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, v2bf16));
}

// E4M3 codes of a packed BF16 pair scaled by 2^-e (scale = 2^e as FP32), written into the
// low (hi_word = false) or high 16 bits of `old`: low byte = lo element, high byte = hi.
template <bool HI_WORD>
__device__ __forceinline__ uint32_t fp8x2_scaled(uint32_t old, uint32_t bf16_pair, float scale) {
  v2i16 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(__builtin_bit_cast(v2i16, old),
                                                      __builtin_bit_cast(v2bf16, bf16_pair), scale,
                                                      HI_WORD);
  return __builtin_bit_cast(uint32_t, r);
}

// E4M3 codes of two FP32 values (|y| <= 448), into the low or high 16 bits of `old`.
template <bool HI_WORD>
__device__ __forceinline__ uint32_t fp8x2(uint32_t old, float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI_WORD);
}

// E2M1 codes (nearest even, saturating at 6) of two FP32 values into nibbles 2*SEL and
// 2*SEL + 1 of `old` (SEL in 0..3).
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// FP32 value of an E8M0 scale byte b (2^(b-127)); byte 0 is the subnormal 2^-127.
__device__ __forceinline__ float e8m0_value(uint32_t b) {
  const uint32_t f = b << 23;
  return __uint_as_float(f > 0x00400000u ? f : 0x00400000u);
}

// ---------------------------------------------------------------------------------
// MXFP8: E8M0 RCEIL scale and E4M3 codes
// ---------------------------------------------------------------------------------

// Scale byte for a finite block whose largest magnitude has FP32 bit pattern amax_bits:
// e + 127 for the smallest e >= -127 with 448 * 2^e >= amax.  With amax = 1.f * 2^E,
// 448 = 1.75 * 2^8, so e = E - 135 + (f > 1.75); finite FP32 never reaches e = 127.
__device__ __forceinline__ uint32_t mx_scale_byte(uint32_t amax_bits) {
  int code = (int)(amax_bits >> 23) - 8 + ((amax_bits & 0x7fffffu) > 0x600000u ? 1 : 0);
  return code < 0 ? 0u : (uint32_t)code;
}

// 2^-e as FP32 for scale byte b = e + 127 (b <= 247).
__device__ __forceinline__ float mx_inv_scale(uint32_t b) {
  return __uint_as_float((254u - b) << 23);
}

// E4M3 code of y, nearest even, for |y| <= 448 (larger magnitudes saturate to 0x7E).
// Normal range: round the FP32 mantissa to 3 bits and rebias (the carry propagates into
// the exponent).  Below 2^-6 the E4M3 grid is k * 2^-9: y * 512 is exact and rint rounds
// it to nearest even.
__device__ __forceinline__ uint32_t e4m3_sw(float y) {
  uint32_t u = __float_as_uint(y);
  uint32_t s = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7fffffffu;
  uint32_t n = ((a + 0x7ffffu + ((a >> 20) & 1u)) >> 20) - 0x3c0u;  // (127 - 7) << 3
  n = n > 0x7eu ? 0x7eu : n;
  uint32_t d = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  return s | (a >= 0x3c800000u ? n : d);
}

__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  return e4m3_sw(a) | (e4m3_sw(b) << 8) | (e4m3_sw(c) << 16) | (e4m3_sw(d) << 24);
}

// ---------------------------------------------------------------------------------
// NVFP4: E4M3 scale of amax / 6 and E2M1 codes
// ---------------------------------------------------------------------------------

// Value of a non-negative finite E4M3 code (0 .. 0x7E): 2^(E - 7) (1 + m/8), or m 2^-9 for
// E = 0.  gfx950's v_cvt_f32_fp8 decodes the OCP E4M3 format exactly (every code 0 .. 0xFF
// from every byte position matched this definition on the device), in one instruction where
// the field arithmetic took a branch between the two forms.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  return __builtin_amdgcn_cvt_f32_fp8((int)c, 0);
}

// Nearest E4M3 code to amax / 6 (ties to even, saturating at 448), decided exactly: the
// candidate from amax * (1/6) is within one code of the answer, and 6 * midpoint is
// exact in FP32, so comparing amax with it settles the rounding without a division.
__device__ __forceinline__ uint32_t nv_scale_code(float amax) {
  uint32_t c = e4m3_sw(amax * (1.0f / 6.0f));
  if (c < 0x7eu) {
    float up = 6.0f * (0.5f * (e4m3_value(c) + e4m3_value(c + 1)));
    if (amax > up || (amax == up && ((c + 1) & 1u) == 0)) return c + 1;
  }
  if (c > 0u) {
    float dn = 6.0f * (0.5f * (e4m3_value(c - 1) + e4m3_value(c)));
    if (amax < dn || (amax == dn && ((c - 1) & 1u) == 0)) return c - 1;
  }
  return c;
}

// The same decision for a BF16-valued amax (every block maximum of the fused paths): the
// FP32 product amax * fl(1/6), clamped to 448, rounds to the same E4M3 code as amax / 6
// does, for every finite BF16 amax (an exhaustive check over all of them), so the hardware
// convert decides it directly.
__device__ __forceinline__ uint32_t nv_scale_code_bf16(float amax) {
  const float y = __builtin_fminf(amax * (1.0f / 6.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.0f, 0, false) & 0xffu;
}

// Two-level NVFP4 (global scale from the tensor amax): s = fl(2688 / amax), capped at 2^100,
// 1 for an amax that is zero, negative or not finite; k = fl(s / 6).  Every step is one
// IEEE FP32 operation (the divisions are correctly rounded).
struct GlobalScale {
  float s = 1.0f, k = 1.0f / 6.0f;
};
__device__ __forceinline__ GlobalScale global_scale(float amax) {
  GlobalScale g;
  if (amax > 0.0f && __builtin_isfinite(amax)) {
    const float s = 2688.0f / amax;
    g.s = s < 0x1p100f ? s : 0x1p100f;
  }
  g.k = g.s / 6.0f;
  return g;
}

// E2M1 decision thresholds at scale S: S * {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5}, each exact
// in FP32.  S == 0 maps every magnitude to code 0 (thresholds at +Inf).
struct E2m1Thresholds {
  float t[7];
};

__device__ __forceinline__ E2m1Thresholds e2m1_thresholds(float S) {
  const float k[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
  E2m1Thresholds r;
#pragma unroll
  for (int i = 0; i < 7; i++) r.t[i] = S > 0.0f ? S * k[i] : __builtin_inff();
  return r;
}

// E2M1 code nibble of x / S: three exact comparisons pick the code bit by bit.  Ties go
// to the even code: 0.75, 1.75 and 3.5 round up (>=), 0.25, 1.25, 2.5 and 5 round down (>).
__device__ __forceinline__ uint32_t e2m1_code(float x, const E2m1Thresholds& T) {
  float a = __builtin_fabsf(x);
  bool b2 = a >= T.t[3];
  bool b1 = a >= (b2 ? T.t[5] : T.t[1]);
  float t0 = b2 ? (b1 ? T.t[6] : T.t[4]) : (b1 ? T.t[2] : T.t[0]);
  bool b0 = a > t0;
  uint32_t s = (__float_as_uint(x) >> 28) & 8u;
  return s | (b2 ? 4u : 0u) | (b1 ? 2u : 0u) | (b0 ? 1u : 0u);
}

// E2M1 codes of x / S for BF16-valued x and an E4M3 scale S, two at a time: y = x * R with R
// within one FP32 ulp of 1 / S (the hardware reciprocal) is within 2^-22 of x / S, which for
// such x either is an E2M1 tie exactly or lies at least 2^-8 (relative) away from every tie.
// Rounding y to BF16 (8 significant bits, error at most 2^-9 relative) therefore restores the
// ties without moving any other value onto or across one, and the hardware E2M1 convert of
// the BF16 pair (nearest even, saturating at 6) decides exactly.  The whole domain (every
// BF16 x, every finite E4M3 S, R = fl(1/S) and its two FP32 neighbours) is checked against
// the exact quotient on the host.  R = 0 for S = 0 gives signed zeros.  The result goes into
// nibbles 2 SEL and 2 SEL + 1 of `old`.
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_of_quotients(uint32_t old, float x0, float x1, float R) {
  const uint32_t y = pack_bf16(x0 * R, x1 * R);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(old, __builtin_bit_cast(v2bf16, y), 1.0f, SEL);
}

// Byte offset of NVFP4 scale (r, c) in the 128x4 layout; cp = padded scale columns.
__device__ __forceinline__ int64_t sf128x4_offset(int64_t r, int64_t c, int64_t cp) {
  return ((r >> 7) * (cp >> 2) + (c >> 2)) * 512 + (r & 31) * 16 + ((r & 127) >> 5) * 4 +
         (c & 3);
}

// ---------------------------------------------------------------------------------
// Wave-level exchanges (wave64).  DPP permutes stay inside a 16-lane row; the xor-16
// step uses ds_swizzle (within 32 lanes).
// ---------------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  // every pattern below has a source lane for every lane, so no lane keeps an old value
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, false);
}
constexpr int DPP_XOR1 = 0xb1;         // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4e;         // quad_perm [2,3,0,1]
constexpr int DPP_ROW_ROR8 = 0x128;    // rotate by 8 inside a row of 16: lane ^ 8
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <-> 7 - i inside each group of 8

__device__ __forceinline__ uint32_t swz_xor16(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401f);  // and 0x1f, xor 0x10
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// ---------------------------------------------------------------------------------
// Packed 16-bit helpers (two BF16 bit patterns per 32-bit word).
// ---------------------------------------------------------------------------------

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u16x2 as_u16x2(uint32_t w) { return __builtin_bit_cast(u16x2, w); }
__device__ __forceinline__ uint32_t as_u32(u16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ uint32_t pkmax(uint32_t a, uint32_t b) {
  return as_u32(__builtin_elementwise_max(as_u16x2(a), as_u16x2(b)));
}
__device__ __forceinline__ uint32_t lo16(uint32_t w) { return w & 0xffffu; }
__device__ __forceinline__ uint32_t hi16(uint32_t w) { return w >> 16; }
// (a.lo, b.lo) and (a.hi, b.hi) as packed pairs
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// ---------------------------------------------------------------------------------
// Raw buffer access.  A descriptor's base is a wave-uniform address (computed on the scalar
// unit); lanes pass 32-bit byte offsets.  An offset of kOob or more is outside the
// descriptor's range: the hardware returns zeros for such a load and drops such a store.
// ---------------------------------------------------------------------------------

constexpr uint32_t kOob = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base) {
  // gfx9 descriptor word 3: 32-bit data format, raw (stride 0) addressing
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(kOob - 1),
                                           0x00020000);
}

}  // namespace glu
