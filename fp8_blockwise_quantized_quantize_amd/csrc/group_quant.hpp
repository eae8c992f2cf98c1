// Encoding of BF16 values into E4M3 codes for one tile whose scale is known,
// in 8-element (16-byte) units.  Shared by the weight and activation
// quantizers and by the fused producers that quantize activation groups
// (FP8-RL summary page, §3.4.1: q = E4M3_RNE(fl32(x / s))).
#pragma once

#include "device_common.hpp"

namespace fp8bq {

// 8 BF16 values (one 16-byte load) -> 8 E4M3 codes (one 8-byte store).
template <bool kFast>
__device__ __forceinline__ u32x2 quant8(u32x4 v, const Divisor& d) {
  float x[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
  float q[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) q[j] = kFast ? d.quotient_fast(x[j]) : d.quotient_ieee(x[j]);
  return u32x2{pack4_e4m3(q[0], q[1], q[2], q[3]), pack4_e4m3(q[4], q[5], q[6], q[7])};
}

// Codes of an all-zero tile: the sign of each input zero (0x00 / 0x80).
__device__ __forceinline__ u32x2 zero8(u32x4 v) {
  uint32_t lo = ((v.x >> 8) & 0x80u) | ((v.x >> 16) & 0x8000u) | ((v.y << 8) & 0x800000u) | (v.y & 0x80000000u);
  uint32_t hi = ((v.z >> 8) & 0x80u) | ((v.z >> 16) & 0x8000u) | ((v.w << 8) & 0x800000u) | (v.w & 0x80000000u);
  return u32x2{lo, hi};
}

__device__ __forceinline__ u32x2 encode8(u32x4 v, float s) {
  if (s == 0.0f) return zero8(v);
  Divisor d(s);
  return d.fast ? quant8<true>(v, d) : quant8<false>(v, d);
}

// One element, any tile: used on ragged edges only.
__device__ __forceinline__ uint8_t encode1(uint16_t bits, float s) {
  if (s == 0.0f) return (uint8_t)((bits >> 8) & 0x80u);
  float x = __uint_as_float((uint32_t)bits << 16);
  Divisor d(s);
  float q = d.fast ? d.quotient_fast(x) : d.quotient_ieee(x);
  return (uint8_t)(cvt_pk_e4m3<false>(q, 0.0f, 0u) & 0xffu);
}

__device__ __forceinline__ uint32_t amax8(uint32_t m, u32x4 v) {
  m = amax_pair(m, v.x);
  m = amax_pair(m, v.y);
  m = amax_pair(m, v.z);
  return amax_pair(m, v.w);
}

}  // namespace fp8bq
