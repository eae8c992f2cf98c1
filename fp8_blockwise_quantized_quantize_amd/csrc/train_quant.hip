// Quantization of FP8 training operands in both layouts from one read.
//
// "FP8-RL: A Practical and Stable Low-Precision Stack for LLM Reinforcement
// Learning" (paper-graph-ui summary), §3.4.5: end-to-end FP8 runs the
// trainer's forward and backward GEMMs in FP8 too.  With the §3.4.1 rule
// applied in the layout each GEMM reduces over, the forward pass needs x in
// 1x128 groups along K and W in 128x128 blocks, dgrad needs W^T ([K][N]) in
// 128x128 blocks, and wgrad needs x^T (and dy^T) in 1x128 groups along the
// token axis.  Each kernel here reads a BF16 tile once and writes both
// layouts: the forward codes directly, the transposed ones through an LDS
// byte tile.
//
// One 256-thread workgroup per 128 x 128 tile (rows r0.., columns c0..).
// Thread t owns the 16-byte column chunk c = t & 15 (columns 8c..8c+7) of
// tile rows 64 h + 4 j + i (h = 0, 1; i = 0..3; j = t >> 4), so the four
// consecutive rows of a (h, j) pair give one 4-byte word of a transposed
// row.
//   activations: scale of tile row r = max |x[r, c0..c0+127]| / 448 (a
//     per-token group); scale of tile column k = max |x[r0..r0+127, k]| / 448
//     (a group of 128 tokens of channel k);
//   weights: one scale per 128 x 128 block, shared by W and W^T.
#include "device_common.hpp"
#include "group_quant.hpp"
#include "launch.hpp"

namespace fp8bq {

namespace {

constexpr int kDualThreads = 256;
constexpr int kTStride = 132;  // LDS bytes per transposed tile row (128 + 4 spreads the banks)

// Per-16-bit-half max of two packed BF16 magnitude pairs.
__device__ __forceinline__ uint32_t max_halves(uint32_t a, uint32_t b) {
  const uint32_t lo = (a & 0xffffu) > (b & 0xffffu) ? (a & 0xffffu) : (b & 0xffffu);
  const uint32_t hi = (a >> 16) > (b >> 16) ? (a >> 16) : (b >> 16);
  return lo | (hi << 16);
}

// Max over the 16 lanes of a quarter wave.
__device__ __forceinline__ uint32_t quarter_max(uint32_t a) {
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) {
    const uint32_t o = __shfl_xor(a, off, 16);
    a = a > o ? a : o;
  }
  return a;
}

__device__ __forceinline__ float bf16_at(const u32x4& v, int e) {
  const uint32_t w = e < 2 ? v.x : (e < 4 ? v.y : (e < 6 ? v.z : v.w));
  return (e & 1) ? bf16_hi(w) : bf16_lo(w);
}

__device__ __forceinline__ float quotient(const Divisor& d, float s, float x) {
  if (s == 0.0f) return x;  // an all-zero group: the code is the zero's sign
  return d.fast ? d.quotient_fast(x) : d.quotient_ieee(x);
}

// x [R][C] BF16 (per batch entry blockIdx.y) -> q [R][C] + s, qt [C][R] + st.
// kWeight: s [nbr][nbc] and st [nbc][nbr] per 128 x 128 block.
// activations: s [R][nbc] (groups along C), st [C][nbr] (groups along R).
// kFwd false: q and s are not written.
template <bool kWeight, bool kFwd>
__global__ __launch_bounds__(kDualThreads) void dual_quant_kernel(const uint16_t* __restrict__ x,
                                                                  uint8_t* __restrict__ q, float* __restrict__ s,
                                                                  uint8_t* __restrict__ qt, float* __restrict__ st,
                                                                  int64_t R, int64_t C, int nbr, int nbc) {
  __shared__ uint8_t tt[128 * kTStride];
  __shared__ uint32_t red[kDualThreads / 64][16][4];
  __shared__ uint32_t blk[kDualThreads / 64];
  const int64_t b = blockIdx.y;
  x += b * R * C;
  qt += b * R * C;
  if (kFwd) q += b * R * C;
  const int64_t nblk = static_cast<int64_t>(nbr) * nbc;
  const int br = static_cast<int>(blockIdx.x / nbc), bc = static_cast<int>(blockIdx.x % nbc);
  const int64_t r0 = static_cast<int64_t>(br) * kBlock, c0 = static_cast<int64_t>(bc) * kBlock;
  const int tid = threadIdx.x, c = tid & 15, j = tid >> 4, lane = tid & 63, wave = tid >> 6;
  const int64_t col = c0 + 8 * c;
  const bool colok = col < C;  // C % 8 == 0: a chunk is wholly in or out

  u32x4 v[8];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = r0 + 64 * h + 4 * j + i;
      v[4 * h + i] = (row < R && colok) ? *reinterpret_cast<const u32x4*>(x + row * C + col) : u32x4{0u, 0u, 0u, 0u};
    }

  float sblk = 0.0f;
  if constexpr (kWeight) {
    uint32_t m = 0u;
#pragma unroll
    for (int k = 0; k < 8; ++k) m = amax8(m, v[k]);
    m = wave_max_u32(amax_fold(m));
    if (lane == 0) blk[wave] = m;
    __syncthreads();
    m = blk[0];
#pragma unroll
    for (int w = 1; w < kDualThreads / 64; ++w) m = m > blk[w] ? m : blk[w];
    sblk = scale_from_amax_bits(m);
    if (tid == 0) {
      st[b * nblk + static_cast<int64_t>(bc) * nbr + br] = sblk;
      if (kFwd) s[b * nblk + static_cast<int64_t>(br) * nbc + bc] = sblk;
    }
  }

  // forward layout
  if constexpr (kFwd) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t row = r0 + 64 * (k >> 2) + 4 * j + (k & 3);
      float sr = sblk;
      if constexpr (!kWeight) {
        sr = scale_from_amax_bits(quarter_max(amax_fold(amax8(0u, v[k]))));
        if (c == 0 && row < R) s[row * nbc + bc] = sr;
      }
      if (row < R && colok) *reinterpret_cast<u32x2*>(q + row * C + col) = encode8(v[k], sr);
    }
  }

  // transposed layout: per-column scales, codes into the LDS tile
  float sc[8];
  if constexpr (kWeight) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sc[e] = sblk;
  } else {
    uint32_t cm[4] = {0u, 0u, 0u, 0u};  // column maxima, two channels per word
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      cm[0] = max_halves(cm[0], v[k].x & 0x7fff7fffu);
      cm[1] = max_halves(cm[1], v[k].y & 0x7fff7fffu);
      cm[2] = max_halves(cm[2], v[k].z & 0x7fff7fffu);
      cm[3] = max_halves(cm[3], v[k].w & 0x7fff7fffu);
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      cm[w] = max_halves(cm[w], __shfl_xor(cm[w], 16));
      cm[w] = max_halves(cm[w], __shfl_xor(cm[w], 32));
      if (lane < 16) red[wave][c][w] = cm[w];
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t m = red[0][c][w];
#pragma unroll
      for (int ww = 1; ww < kDualThreads / 64; ++ww) m = max_halves(m, red[ww][c][w]);
      sc[2 * w] = scale_from_amax_bits(m & 0xffffu);
      sc[2 * w + 1] = scale_from_amax_bits(m >> 16);
    }
    if (j == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (col + e < C) st[(col + e) * nbr + br] = sc[e];
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const Divisor d(sc[e] != 0.0f ? sc[e] : 1.0f);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float q0 = quotient(d, sc[e], bf16_at(v[4 * h + 0], e));
      const float q1 = quotient(d, sc[e], bf16_at(v[4 * h + 1], e));
      const float q2 = quotient(d, sc[e], bf16_at(v[4 * h + 2], e));
      const float q3 = quotient(d, sc[e], bf16_at(v[4 * h + 3], e));
      *reinterpret_cast<uint32_t*>(&tt[(8 * c + e) * kTStride + 64 * h + 4 * j]) = pack4_e4m3(q0, q1, q2, q3);
    }
  }
  __syncthreads();

  // transposed rows k = c0 + kl, tokens r0 + 16 part .. + 15
  const bool vec = (R % 16) == 0;
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int qi = tid + kDualThreads * n;
    const int kl = qi >> 3, part = qi & 7;
    const int64_t k = c0 + kl, m = r0 + 16 * part;
    if (k >= C || m >= R) continue;
    const uint8_t* src = &tt[kl * kTStride + 16 * part];
    uint8_t* dst = qt + k * R + m;
    if (vec) {
      const u32x4 w = u32x4{*reinterpret_cast<const uint32_t*>(src), *reinterpret_cast<const uint32_t*>(src + 4),
                            *reinterpret_cast<const uint32_t*>(src + 8), *reinterpret_cast<const uint32_t*>(src + 12)};
      *reinterpret_cast<u32x4*>(dst) = w;
    } else {
      for (int bb = 0; bb < 16 && m + bb < R; ++bb) dst[bb] = src[bb];
    }
  }
}

template <bool kWeight>
hipError_t launch_dual(const uint16_t* x, uint8_t* q, float* s, uint8_t* qt, float* st, int64_t batch, int64_t R,
                       int64_t C, hipStream_t stream) {
  const int64_t nbr = (R + kBlock - 1) / kBlock, nbc = (C + kBlock - 1) / kBlock;
  const int64_t tiles = nbr * nbc;
  if (tiles == 0 || batch == 0) return hipSuccess;
  if (tiles > 0x7fffffffLL || batch > 65535) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>(batch));
  if (q)
    hipLaunchKernelGGL((dual_quant_kernel<kWeight, true>), grid, dim3(kDualThreads), 0, stream, x, q, s, qt, st, R, C,
                       static_cast<int>(nbr), static_cast<int>(nbc));
  else
    hipLaunchKernelGGL((dual_quant_kernel<kWeight, false>), grid, dim3(kDualThreads), 0, stream, x, q, s, qt, st, R,
                       C, static_cast<int>(nbr), static_cast<int>(nbc));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_weight_dual(const uint16_t* w, uint8_t* q, float* s, uint8_t* qt, float* st, int64_t batch,
                                    int64_t N, int64_t K, hipStream_t stream) {
  return launch_dual<true>(w, q, s, qt, st, batch, N, K, stream);
}

hipError_t launch_quant_act_dual(const uint16_t* x, uint8_t* q, float* s, uint8_t* qt, float* st, int64_t M,
                                 int64_t K, hipStream_t stream) {
  return launch_dual<false>(x, q, s, qt, st, 1, M, K, stream);
}

}  // namespace fp8bq
