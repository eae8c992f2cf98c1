// Device helpers shared by the quantizer and GEMM kernels (gfx950 only).
//
// E4M3 codes follow the OCP "e4m3fn" layout used by gfx950's FP8 matrix
// cores and by the FP8-RL pages (summary page, §3.4.1 "Quantization Format
// and Granularity": 4 exponent bits, 3 mantissa bits, max 448).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bq {

constexpr int kBlock = 128;          // weight block edge and activation group width
constexpr float kE4M3Max = 448.0f;   // largest finite E4M3 magnitude

typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16-byte load/store unit
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));  // 8-byte load/store unit

// BF16 pair packed in one 32-bit word -> the two float32 values (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Running max of |bf16| over a packed pair, on the bit patterns: clearing the
// sign bit leaves an unsigned integer that orders like the magnitude (inputs
// are finite), so the max is exact and independent of the FP32 denorm mode.
__device__ __forceinline__ uint32_t amax_pair(uint32_t acc, uint32_t w) {
  ushort2_t a = __builtin_bit_cast(ushort2_t, acc);
  ushort2_t b = __builtin_bit_cast(ushort2_t, w & 0x7fff7fffu);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
}

__device__ __forceinline__ uint32_t amax_fold(uint32_t pair) {
  uint32_t lo = pair & 0xffffu, hi = pair >> 16;
  return lo > hi ? lo : hi;
}

// Block/group scale: s = fl32(amax / 448) with IEEE division (the compiler
// emits the correctly rounded sequence; denormals are kept).
__device__ __forceinline__ float scale_from_amax_bits(uint32_t amax_bf16) {
  return __uint_as_float(amax_bf16 << 16) / kE4M3Max;
}

// Per-tile divisor context.  The quantized value is E4M3(fl32(x / s)).
// For 2^-64 <= s the float32 quotient is formed without a per-element
// divide: q0 = x * r with r = fl32(1 / s), then one Markstein correction
//   e = fma(q0, s, -x)  (exact: q0 is within an ulp of x / s)
//   q = fma(-e, r, q0)
// which returns the correctly rounded quotient when r is the correctly
// rounded reciprocal and q0 is within one ulp (P. Markstein, "IA-64 and
// Elementary Functions", 2000; the division theorem also in Muller et al.,
// "Handbook of Floating-Point Arithmetic", ch. 4).  Quotients below 2^-11
// encode to a signed zero whatever their last bits, so underflow of those
// quotients does not matter.  The residual e is exact only while the product
// q0 * s keeps its low bits above the float32 denormal grid, which holds for
// s >= 2^-92 when |x / s| >= 2^-11; tiles with s < 2^-64 (amax < 448 * 2^-64)
// therefore use the IEEE division directly.  The sign of a zero x is preserved by the
// order of the operands (-0 * r = -0; fma(-0, s, +0) = +0; fma(-(+0), r, -0)
// = -0).
struct Divisor {
  float s, r;
  bool fast;
  __device__ __forceinline__ explicit Divisor(float scale) : s(scale) {
    r = 1.0f / scale;
    fast = scale >= 0x1p-64f;
  }
  __device__ __forceinline__ float quotient_fast(float x) const {
    float q0 = x * r;
    float e = __builtin_fmaf(q0, s, -x);
    return __builtin_fmaf(-e, r, q0);
  }
  __device__ __forceinline__ float quotient_ieee(float x) const { return x / s; }
};

// Integer-bit E4M3 encoder (round to nearest even, saturate at 448).  The
// standalone encoder entry point offers it beside the hardware conversion
// below, so that both can be checked against the oracle over every float32.
__device__ __forceinline__ uint32_t encode_e4m3_soft(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7fffffffu;
  // subnormal range |v| < 2^-6: m = RNE(|v| * 2^9) via one FMA onto 2^23,
  // whose float32 ulp is 1 (the FMA rounds once, to nearest even).
  float t = __builtin_fmaf(__uint_as_float(a), 512.0f, 8388608.0f);
  uint32_t sub = __float_as_uint(t) - 0x4b000000u;
  // normal range: keep 3 mantissa bits with round-to-nearest-even on the
  // 20 dropped bits, then rebias the exponent from 127 to 7 (120 << 3).
  uint32_t rnd = a + 0x7ffffu + ((a >> 20) & 1u);
  uint32_t nrm = (rnd >> 20) - (120u << 3);
  uint32_t code = a < 0x3c800000u ? sub : nrm;   // 2^-6
  code = a >= 0x43e00000u ? 0x7eu : code;        // >= 448 saturates
  return code | sign;
}

// Hardware conversion of two float32 values to E4M3 (v_cvt_pk_fp8_f32,
// round to nearest even in the OCP e4m3fn format on gfx950), written into
// byte lanes 0/1 (hi = false) or 2/3 (hi = true) of `old`.  Used without a
// clamp only where |v| < 464 is guaranteed: every quantizer quotient has
// |x / s| <= amax / s <= 448 * (1 + 2^-8) (s may lose bits as a denormal),
// and values in [448, 464) round to 448.  The saturating encoder clamps to
// +-448 first.  Both uses are checked over every float32 in that range.
template <bool kHi>
__device__ __forceinline__ uint32_t cvt_pk_e4m3(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, kHi);
}

// Four quotients -> one little-endian word of four E4M3 codes.
__device__ __forceinline__ uint32_t pack4_e4m3(float q0, float q1, float q2, float q3) {
  uint32_t w = cvt_pk_e4m3<false>(q0, q1, 0u);
  return cvt_pk_e4m3<true>(q2, q3, w);
}

// Wave-wide (64 lanes) max of a uint32.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t o = __shfl_xor(v, off, 64);
    v = v > o ? v : o;
  }
  return v;
}

}  // namespace fp8bq
