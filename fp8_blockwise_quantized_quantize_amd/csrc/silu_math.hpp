// SiLU(gate) * up of one element, rounded to BF16 exactly as the exact real
// value would be (the gated MLP of the MoE expert layers: FP8-RL summary
// page, §3.4.1 "Quantization Scope"; the nonlinearity stays in higher
// precision, §3.4.1 "Static vs. Dynamic Quantization").  Shared by the
// SiLU*up quantizer and the fc1 GEMM whose epilogue applies it, so both give
// the same bits.
#pragma once

#include <math.h>

#include "device_common.hpp"

namespace fp8bq {

namespace {

// h = SiLU(g) * u rounded to BF16, correctly rounded from the exact value.
// Fast path in float32 for |g| <= 80:
//   e^-g = 2^x, x = -g log2(e), split exactly as x = xh + xl (xh = fl(-g L)
//   with L = fl32(log2 e), xl = the product's rounding error by fma plus
//   -g (log2 e - L)); t = v_exp_f32(xh) * (1 + xl ln 2) (|xl| < 2^-17, the
//   dropped terms are below 2^-33); h32 = fl(fl(g * rcp(fl(1 + t))) * u).
// With v_exp_f32 and v_rcp_f32 within 2 ulp each, h32 is within 3 * 2^-22
// (relative) of the exact value, i.e. within 12 float32 ulps, so its BF16
// rounding is the exact value's whenever h32 is more than 48 float32 ulps
// away from a BF16 midpoint (low 16 bits 0x8000), and |h32| is in the
// normal range.  Otherwise (about one value in 700, and every value outside
// the fast range) the product is formed in float64 and rounded straight to
// BF16.
//
// Two regimes put the exact value structurally close to a midpoint, closer
// than float64 resolves: for |g| < 2^-20, SiLU(g) u = a (1 + g/2 + O(g^2))
// with a = g u / 2, and for g > 20, SiLU(g) u = a (1 - e^-g + ...) with
// a = g u; a is a product of two BF16 values (16 significant bits, exact in
// float64) and can be exactly a midpoint.  There the correction decides:
// beyond the midpoint in magnitude for a tiny positive g, short of it
// otherwise.  When a is not a midpoint it is at least 2^-16 (relative) away
// from every midpoint and the correction (below 2^-21) cannot cross one.
// Elsewhere SiLU(g) u is transcendental and has no such structure.
__device__ __noinline__ uint32_t silu_mul_bf16_f64(float g, float u) {
  const double gd = g, ud = u;
  double h;
  int tie = 0;  // for an exact midpoint: +1 rounds up in magnitude, -1 down
  if (fabs(gd) < 0x1p-20) {
    h = gd * ud * 0.5;
    tie = gd > 0.0 ? 1 : -1;
  } else if (gd > 20.0) {
    h = gd * ud;
    tie = -1;
  } else {
    h = gd / (1.0 + exp(-gd)) * ud;
  }
  if (h == 0.0 || !isfinite(h)) return __float_as_uint(static_cast<float>(h)) >> 16;
  int ex;
  (void)frexp(h, &ex);                                 // |h| in [2^(ex-1), 2^ex)
  const int q = (ex - 1 > -126 ? ex - 1 : -126) - 7;  // BF16 spacing 2^q
  const double m = ldexp(h, -q);                       // exact; |m| < 2^9
  const double fl = floor(m);
  double r;
  if (tie != 0 && m - fl == 0.5)
    r = ((tie > 0) == (m > 0.0)) ? fl + 1.0 : fl;      // away from / toward zero
  else
    r = rint(m);                                       // nearest even
  const double v = ldexp(r, q);
  if (fabs(v) > 3.3895313892515355e38) return (h < 0 ? 0xff80u : 0x7f80u);  // beyond BF16 max
  if (v == 0.0) return h < 0.0 ? 0x8000u : 0u;
  return __float_as_uint(static_cast<float>(v)) >> 16;  // exact conversion
}

// silu_mul_bf16's float32 path without a branch, for a caller that takes
// the float64 decisions of many values together (the fused fc1 epilogue):
// the path's result, and in *ok whether it is final (false:
// silu_mul_bf16_f64(g, u) is the result).  The exponential is taken of g
// clamped to [-80, 80]; outside that range, and for a NaN g, *ok is false.
// The same arithmetic as silu_mul_bf16 below, written out twice on
// purpose: the compiler schedules each caller's kernel best from its own
// form (one shared helper measured 4% slower on the SiLU*up quantizer and
// 5% slower on the fused fc1).
__device__ __forceinline__ uint32_t silu_mul_bf16_fast(float g, float u, bool* ok) {
  constexpr float kLog2e = 1.44269502162933349609375f;      // fl32(log2 e)
  constexpr float kLog2eLo = 1.925963033500011079e-8f;      // log2 e - kLog2e
  constexpr float kLn2 = 0.693147180559945309f;
  const float gc = fminf(fmaxf(g, -80.0f), 80.0f);
  const float xh = -gc * kLog2e;
  const float xl = fmaf(-gc, kLog2e, -xh) + (-gc) * kLog2eLo;
  const float p = __builtin_amdgcn_exp2f(xh);
  const float t = fmaf(p, xl * kLn2, p);
  const float h = (g * __builtin_amdgcn_rcpf(1.0f + t)) * u;
  const uint32_t b = __float_as_uint(h);
  const float ah = fabsf(h);
  const uint32_t low = b & 0xffffu;
  const uint32_t dist = low > 0x8000u ? low - 0x8000u : 0x8000u - low;
  const bool zero = h == 0.0f;
  *ok = fabsf(g) <= 80.0f && (zero || (ah >= 0x1p-100f && ah <= 0x1p120f && dist > 48u));
  return zero ? b >> 16 : (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t silu_mul_bf16(float g, float u) {
  if (fabsf(g) <= 80.0f) {
    constexpr float kLog2e = 1.44269502162933349609375f;      // fl32(log2 e)
    constexpr float kLog2eLo = 1.925963033500011079e-8f;      // log2 e - kLog2e
    constexpr float kLn2 = 0.693147180559945309f;
    const float xh = -g * kLog2e;
    const float xl = fmaf(-g, kLog2e, -xh) + (-g) * kLog2eLo;
    const float p = __builtin_amdgcn_exp2f(xh);
    const float t = fmaf(p, xl * kLn2, p);
    const float h = (g * __builtin_amdgcn_rcpf(1.0f + t)) * u;
    const uint32_t b = __float_as_uint(h);
    const float ah = fabsf(h);
    const uint32_t low = b & 0xffffu;
    const uint32_t dist = low > 0x8000u ? low - 0x8000u : 0x8000u - low;
    if (h == 0.0f) return b >> 16;
    if (ah >= 0x1p-100f && ah <= 0x1p120f && dist > 48u) return (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
  }
  return silu_mul_bf16_f64(g, u);
}

}  // namespace

}  // namespace fp8bq
