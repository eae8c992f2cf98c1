// Token-level importance weights of the FP8 rollout correction.
//
// "FP8-RL: A Practical and Stable Low-Precision Stack for LLM Reinforcement
// Learning" (paper-graph-ui summary), §3.4.3: each sampled token gets the
// ratio of the training policy's probability to the FP8 rollout policy's,
// w = exp(logp_train - logp_rollout); TIS limits w to [1/C, C]; the weight
// multiplies the token's advantage.  MIS (named there as the stronger
// alternative) is read as: tokens whose weight falls outside [1/C, C] get 0.
//
// One streaming pass, HBM-bound: each lane handles four consecutive tokens
// with 16-byte loads and stores.  The response mask is read first; a lane
// whose four tokens are all padding loads nothing else and writes zeros, so
// the padded tail of a [responses][max_len] batch costs its mask byte and
// its output only.
//
// Precision: the float32 difference s = fl32(lt - lr) and its rounding error
// e (TwoSum, exact) give w = exp(s) * (1 + e), so the weight carries only the
// error of expf (not the rounding of the difference, which for |d| >> 1
// would be many ulps).  The MIS band test uses s itself against fl32(ln C).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "launch.hpp"

namespace fp8bq {
namespace {

constexpr int kThreads = 256;
constexpr int kVec = 4;

struct Args {
  const float* lt;
  const float* lr;
  const uint8_t* mask;
  const float* adv;
  float* w;
  float* wa;
  int64_t n;
  float lo;     // fl32(1 / C)
  float hi;     // C
  float log_c;  // fl32(ln C), the MIS band edge
};

template <bool kMis>
__device__ __forceinline__ float weight_of(float lt, float lr, const Args& p) {
  const float s = lt - lr;
  // TwoSum of lt + (-lr): s + err == lt - lr exactly when s is finite.
  const float bb = s - lt;
  const float err = isfinite(s) ? ((lt - (s - bb)) + (-lr - bb)) : 0.0f;
  const float e = expf(s);
  float w = (e < INFINITY) ? fmaf(e, err, e) : e;  // e * (1 + err); inf / NaN pass through
  w = (w < p.lo) ? p.lo : ((w > p.hi) ? p.hi : w);  // a NaN stays NaN
  if (kMis) w = (fabsf(s) <= p.log_c) ? w : 0.0f;   // NaN fails the test
  return w;
}

template <bool kMis, bool kMask, bool kAdv>
__device__ __forceinline__ void one_token(const Args& p, int64_t i) {
  float w = 0.0f;
  if (!kMask || p.mask[i] != 0) w = weight_of<kMis>(p.lt[i], p.lr[i], p);
  p.w[i] = w;
  if (kAdv) p.wa[i] = (w == 0.0f) ? 0.0f : w * p.adv[i];
}

template <bool kMis, bool kMask, bool kAdv>
__global__ void __launch_bounds__(kThreads) importance_weight_kernel(Args p) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) * kVec;
  if (i >= p.n) return;
  if (i + kVec > p.n) {  // ragged tail: fewer than four tokens left
    for (int64_t j = i; j < p.n; ++j) one_token<kMis, kMask, kAdv>(p, j);
    return;
  }
  const uint32_t m4 = kMask ? *reinterpret_cast<const uint32_t*>(p.mask + i) : 0x01010101u;
  float4 w4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  float4 wa4 = w4;
  if (m4 != 0) {
    const float4 a = *reinterpret_cast<const float4*>(p.lt + i);
    const float4 b = *reinterpret_cast<const float4*>(p.lr + i);
    float4 adv = w4;
    if (kAdv) adv = *reinterpret_cast<const float4*>(p.adv + i);
    const float av[kVec] = {a.x, a.y, a.z, a.w};
    const float bv[kVec] = {b.x, b.y, b.z, b.w};
    const float cv[kVec] = {adv.x, adv.y, adv.z, adv.w};
    float wv[kVec], wav[kVec];
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      const bool valid = ((m4 >> (8 * j)) & 0xffu) != 0;
      wv[j] = valid ? weight_of<kMis>(av[j], bv[j], p) : 0.0f;
      wav[j] = (wv[j] == 0.0f) ? 0.0f : wv[j] * cv[j];
    }
    w4 = make_float4(wv[0], wv[1], wv[2], wv[3]);
    wa4 = make_float4(wav[0], wav[1], wav[2], wav[3]);
  }
  *reinterpret_cast<float4*>(p.w + i) = w4;
  if (kAdv) *reinterpret_cast<float4*>(p.wa + i) = wa4;
}

template <bool kMis, bool kMask, bool kAdv>
hipError_t launch_cfg(const Args& p, hipStream_t stream) {
  const int64_t lanes = (p.n + kVec - 1) / kVec;
  const int64_t blocks = (lanes + kThreads - 1) / kThreads;
  hipLaunchKernelGGL((importance_weight_kernel<kMis, kMask, kAdv>), dim3(static_cast<uint32_t>(blocks)),
                     dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <bool kMis>
hipError_t launch_mode(const Args& p, hipStream_t stream) {
  if (p.mask) return p.adv ? launch_cfg<kMis, true, true>(p, stream) : launch_cfg<kMis, true, false>(p, stream);
  return p.adv ? launch_cfg<kMis, false, true>(p, stream) : launch_cfg<kMis, false, false>(p, stream);
}

}  // namespace

hipError_t launch_importance_weights(const float* logp_train, const float* logp_rollout, const uint8_t* mask,
                                     const float* advantages, float* weights, float* weighted_adv, int64_t n,
                                     float lo, float hi, float log_c, bool mis, hipStream_t stream) {
  const Args p{logp_train, logp_rollout, mask, advantages, weights, weighted_adv, n, lo, hi, log_c};
  return mis ? launch_mode<true>(p, stream) : launch_mode<false>(p, stream);
}

}  // namespace fp8bq
