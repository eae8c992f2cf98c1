// MoE expert-FFN glue around the grouped block-scaled GEMMs (gfx950).
//
// "FP8-RL: A Practical and Stable Low-Precision Stack for LLM Reinforcement
// Learning" (paper-graph-ui summary), §3.4.1 "Quantization Scope": the
// expert layers fc1 / fc2 are FP8 W8A8 linears; the gated MLP multiplies
// the gate and up activations element-wise before the down projection;
// §3.4.1 "Static vs. Dynamic Quantization": activations are quantized on
// the fly in 1x128 tiles while the nonlinearity stays in higher precision.
//
//   moe_sort_kernel          routing pairs -> rows grouped by expert
//   gather_quant_act_kernel  FP8 rows of the sorted pairs (1x128 groups)
//   silu_mul_quant_kernel    h = SiLU(gate) * up -> BF16 -> 1x128 groups
//   combine_kernel           routing-weighted sum of each token's k rows
#include <math.h>

#include "device_common.hpp"
#include "group_quant.hpp"
#include "launch.hpp"
#include "silu_math.hpp"

namespace fp8bq {

namespace {

// ---------------------------------------------------------------------------
// Sort by expert.  One workgroup per expert e, no atomics, deterministic:
//   first row of e = number of pairs routed to experts below e;
//   row of pair p   = first row + number of pairs q < p routed to e.
// The pairs are taken in rounds of kSortWaves * kSortRun * 64; in a round
// wave w owns the contiguous segment of kSortRun * 64 pairs starting at
// w * kSortRun * 64 and reads it with coalesced loads (load i, lane l: pair
// i * 64 + l of the segment).  Pass 1 counts the pairs below e; pass 2
// ranks e's pairs inside the segment from one ballot per load (pair order
// is (i, l) order) and across segments from the waves' totals, so rows keep
// pair order.  Every workgroup reads the whole id list, which stays in L2;
// when the pairs fit one round (up to kSortRound, e.g. 4096 tokens x top-8)
// both passes come from one read of it.
// ---------------------------------------------------------------------------
constexpr int kSortThreads = 1024;
constexpr int kSortWaves = kSortThreads / 64;
constexpr int kSortRun = 32;
constexpr int32_t kSortSegment = kSortRun * 64;
constexpr int32_t kSortRound = kSortWaves * kSortSegment;

__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

// The kSortRun ids of this lane in the segment at `seg` (-1 past P).
__device__ __forceinline__ void load_segment(const int32_t* __restrict__ ids, int32_t seg, int lane, int32_t P,
                                             int32_t (&id)[kSortRun]) {
#pragma unroll
  for (int i = 0; i < kSortRun; ++i) {
    const int32_t p = seg + i * 64 + lane;
    id[i] = p < P ? ids[p] : -1;
  }
}

__global__ __launch_bounds__(kSortThreads) void moe_sort_kernel(const int32_t* __restrict__ ids, int32_t P, int32_t E,
                                                                int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ sorted_pair,
                                                                int32_t* __restrict__ pair_row) {
  __shared__ int32_t part[kSortWaves];
  __shared__ int32_t part2[kSortWaves];
  const int32_t e = static_cast<int32_t>(blockIdx.x);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  if (P <= kSortRound) {  // one round: both counts and the ranks from one read of the ids
    const int32_t seg = wave * kSortSegment;
    int32_t id[kSortRun];
    load_segment(ids, seg, lane, P, id);
    uint64_t mask[kSortRun];
    int below = 0;
    int32_t count = 0;  // e's pairs in this wave's segment (wave-uniform)
#pragma unroll
    for (int i = 0; i < kSortRun; ++i) {
      below += (id[i] >= 0 && id[i] < e) ? 1 : 0;
      mask[i] = __ballot(id[i] == e);
      count += __popcll(mask[i]);
    }
    below = wave_sum_i32(below);
    if (lane == 0) {
      part[wave] = below;
      part2[wave] = count;
    }
    __syncthreads();
    int32_t first = 0, before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kSortWaves; ++w) {
      first += part[w];
      before += (w < wave) ? part2[w] : 0;
      total += part2[w];
    }
    int32_t r = first + before;
#pragma unroll
    for (int i = 0; i < kSortRun; ++i) {
      const int32_t p = seg + i * 64 + lane;
      if (id[i] == e) {
        const int32_t row = r + static_cast<int32_t>(lanes_below(mask[i]));
        sorted_pair[row] = p;
        pair_row[p] = row;
      }
      if (e == 0 && p < P && (id[i] < 0 || id[i] >= E)) pair_row[p] = -1;  // no expert, no row
      r += __popcll(mask[i]);
    }
    if (tid == 0) {
      offsets[e] = first;
      if (e == E - 1) offsets[E] = first + total;
    }
    return;
  }

  int below = 0;
  for (int32_t base = 0; base < P; base += kSortRound) {
    int32_t id[kSortRun];
    load_segment(ids, base + wave * kSortSegment, lane, P, id);
#pragma unroll
    for (int i = 0; i < kSortRun; ++i) below += (id[i] >= 0 && id[i] < e) ? 1 : 0;
  }
  below = wave_sum_i32(below);
  if (lane == 0) part[wave] = below;
  __syncthreads();
  int32_t first = 0;
#pragma unroll
  for (int w = 0; w < kSortWaves; ++w) first += part[w];
  __syncthreads();

  int32_t running = first;
  for (int32_t base = 0; base < P; base += kSortRound) {
    const int32_t seg = base + wave * kSortSegment;
    int32_t id[kSortRun];
    load_segment(ids, seg, lane, P, id);
    uint64_t mask[kSortRun];
    int32_t count = 0;  // e's pairs in this wave's segment (wave-uniform)
#pragma unroll
    for (int i = 0; i < kSortRun; ++i) {
      mask[i] = __ballot(id[i] == e);
      count += __popcll(mask[i]);
    }
    if (lane == 0) part[wave] = count;
    __syncthreads();
    int32_t before = 0, round_total = 0;
#pragma unroll
    for (int w = 0; w < kSortWaves; ++w) {
      before += (w < wave) ? part[w] : 0;
      round_total += part[w];
    }
    int32_t r = running + before;
#pragma unroll
    for (int i = 0; i < kSortRun; ++i) {
      const int32_t p = seg + i * 64 + lane;
      if (id[i] == e) {
        const int32_t row = r + static_cast<int32_t>(lanes_below(mask[i]));
        sorted_pair[row] = p;
        pair_row[p] = row;
      }
      if (e == 0 && p < P && (id[i] < 0 || id[i] >= E)) pair_row[p] = -1;  // no expert, no row
      r += __popcll(mask[i]);
    }
    running += round_total;
    __syncthreads();
  }
  if (tid == 0) {
    offsets[e] = first;
    if (e == E - 1) offsets[E] = running;
  }
}

// ---------------------------------------------------------------------------
// 1x128 groups, one 16-lane quarter wave per (row, group), each lane owning
// 8 consecutive values, as in the activation quantizer: the group amax is a
// 4-step xor shuffle inside the quarter wave.
// ---------------------------------------------------------------------------
constexpr int kGroupThreads = 256;
constexpr int kGroupsPerBlock = kGroupThreads / 16;

__device__ __forceinline__ float quarter_wave_scale(u32x4 v) {
  uint32_t a = amax_fold(amax8(0u, v));
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) {
    const uint32_t o = __shfl_xor(a, off, 16);
    a = a > o ? a : o;
  }
  return scale_from_amax_bits(a);
}

// Gathered activation rows: row r of the output is token sorted_pair[r] / k
// of x, quantized in 1x128 groups (the same codes as quantizing x and then
// copying rows).  Rows whose pair names no token are written as zeros.
// One wave per row: the row's token is a scalar load, and each lane issues
// its 16-byte loads for all groups of the row before any of them is used;
// in pass i the quarter wave q handles group 4 i + q.
constexpr int kGatherRowsPerBlock = kGroupThreads / 64;

__global__ __launch_bounds__(kGroupThreads) void gather_quant_act_kernel(const uint16_t* __restrict__ x,
                                                                         const int32_t* __restrict__ sorted_pair,
                                                                         uint8_t* __restrict__ q,
                                                                         float* __restrict__ scale, int64_t R,
                                                                         int64_t T, int32_t k, int64_t K, int G) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * kGatherRowsPerBlock +
                    __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (r >= R) return;  // whole waves leave
  const int lane = threadIdx.x & 63, li = lane & 15, quarter = lane >> 4;
  const int32_t pair = sorted_pair[r];
  const int64_t t = pair >= 0 ? pair / k : -1;
  const bool ok = t >= 0 && t < T;
  const uint16_t* src = x + (ok ? t : 0) * K;
  uint8_t* dst = q + r * K;
  constexpr int kPassesMax = 8;  // rows of up to 32 groups (K <= 4096) in registers
  for (int g0 = 0; g0 < G; g0 += 4 * kPassesMax) {
    u32x4 v[kPassesMax];
#pragma unroll
    for (int i = 0; i < kPassesMax; ++i) {
      const int g = g0 + 4 * i + quarter;
      v[i] = u32x4{0u, 0u, 0u, 0u};
      if (ok && g < G) v[i] = *reinterpret_cast<const u32x4*>(src + static_cast<int64_t>(g) * kBlock + li * 8);
    }
#pragma unroll
    for (int i = 0; i < kPassesMax; ++i) {
      const int g = g0 + 4 * i + quarter;
      if (g0 + 4 * i >= G) break;  // uniform: no group of this pass exists
      const float s = quarter_wave_scale(v[i]);
      if (g < G) {
        if (li == 0) scale[r * G + g] = s;
        *reinterpret_cast<u32x2*>(dst + static_cast<int64_t>(g) * kBlock + li * 8) = encode8(v[i], s);
      }
    }
  }
}

// fc1 output rows [M][2F] = [gate | up] -> h codes [M][F] and scales
// [M][ceil(F/128)] (and, if asked, the BF16 h itself).  F % 8 == 0; a
// partial last group has idle lanes.
template <bool kStoreH>
__global__ __launch_bounds__(kGroupThreads) void silu_mul_quant_kernel(const uint16_t* __restrict__ y,
                                                                       uint8_t* __restrict__ q,
                                                                       float* __restrict__ scale,
                                                                       uint16_t* __restrict__ hb, int64_t M,
                                                                       int64_t F, int G) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kGroupsPerBlock + (threadIdx.x >> 4);
  if (gid >= M * G) return;
  const int li = threadIdx.x & 15;
  const int64_t m = gid / G;
  const int g = static_cast<int>(gid % G);
  const int64_t col = static_cast<int64_t>(g) * kBlock + li * 8;
  const bool in = col < F;  // F % 8 == 0: a lane is wholly in or out
  u32x4 h = u32x4{0u, 0u, 0u, 0u};
  if (in) {
    const u32x4 gv = *reinterpret_cast<const u32x4*>(y + m * 2 * F + col);
    const u32x4 uv = *reinterpret_cast<const u32x4*>(y + m * 2 * F + F + col);
    const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
    const uint32_t uw[4] = {uv.x, uv.y, uv.z, uv.w};
    uint32_t hw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      hw[j] = silu_mul_bf16(bf16_lo(gw[j]), bf16_lo(uw[j])) | (silu_mul_bf16(bf16_hi(gw[j]), bf16_hi(uw[j])) << 16);
    h = u32x4{hw[0], hw[1], hw[2], hw[3]};
    if (kStoreH) *reinterpret_cast<u32x4*>(hb + m * F + col) = h;
  }
  const float s = quarter_wave_scale(h);
  if (li == 0) scale[m * G + g] = s;
  if (in) *reinterpret_cast<u32x2*>(q + m * F + col) = encode8(h, s);
}

// ---------------------------------------------------------------------------
// Combine: out[t] = sum_j w[t][j] * y[pair_row[t k + j]], float32 fma chain in
// slot order, rounded once to BF16.  One workgroup per token, each lane owns
// 8 columns (16-byte loads of each routed row).  Rows outside [0, M) are
// skipped.
// ---------------------------------------------------------------------------
constexpr int kCombineThreads = 256;

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // NaN stays NaN
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Up to kCombineAhead routed rows are loaded before the first of them is
// summed, so a lane keeps that many 16-byte loads in flight.
constexpr int kCombineAhead = 8;

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const uint16_t* __restrict__ y,
                                                                  const int32_t* __restrict__ pair_row,
                                                                  const float* __restrict__ w,
                                                                  uint16_t* __restrict__ out, int32_t k, int64_t H,
                                                                  int64_t M) {
  const int64_t t = blockIdx.x;
  for (int64_t c = static_cast<int64_t>(threadIdx.x) * 8; c < H; c += kCombineThreads * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int32_t j0 = 0; j0 < k; j0 += kCombineAhead) {
      u32x4 v[kCombineAhead];
      float wj[kCombineAhead];
#pragma unroll
      for (int jj = 0; jj < kCombineAhead; ++jj) {
        const int32_t j = j0 + jj;
        const int32_t r = j < k ? pair_row[t * k + j] : -1;
        const bool ok = r >= 0 && r < M;
        wj[jj] = ok ? w[t * k + j] : 0.0f;
        v[jj] = ok ? *reinterpret_cast<const u32x4*>(y + static_cast<int64_t>(r) * H + c) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int jj = 0; jj < kCombineAhead; ++jj) {
        if (j0 + jj >= k) break;
        const int32_t r = pair_row[t * k + j0 + jj];
        if (r < 0 || r >= M) continue;  // rows outside [0, M) contribute nothing
        const uint32_t vw[4] = {v[jj].x, v[jj].y, v[jj].z, v[jj].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = fmaf(wj[jj], bf16_lo(vw[i]), acc[2 * i]);
          acc[2 * i + 1] = fmaf(wj[jj], bf16_hi(vw[i]), acc[2 * i + 1]);
        }
      }
    }
    u32x4 o;
    o.x = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
    o.y = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
    o.z = f32_to_bf16_rne(acc[4]) | (f32_to_bf16_rne(acc[5]) << 16);
    o.w = f32_to_bf16_rne(acc[6]) | (f32_to_bf16_rne(acc[7]) << 16);
    *reinterpret_cast<u32x4*>(out + t * H + c) = o;
  }
}

int64_t group_blocks(int64_t groups) { return (groups + kGroupsPerBlock - 1) / kGroupsPerBlock; }

}  // namespace

hipError_t launch_moe_sort(const int32_t* ids, int64_t P, int64_t E, int32_t* offsets, int32_t* sorted_pair,
                           int32_t* pair_row, hipStream_t stream) {
  hipLaunchKernelGGL(moe_sort_kernel, dim3(static_cast<uint32_t>(E)), dim3(kSortThreads), 0, stream, ids,
                     static_cast<int32_t>(P), static_cast<int32_t>(E), offsets, sorted_pair, pair_row);
  return hipGetLastError();
}

hipError_t launch_gather_quant_act(const uint16_t* x, const int32_t* sorted_pair, int64_t R, int64_t T, int64_t k,
                                   int64_t K, uint8_t* q, float* scale, hipStream_t stream) {
  const int64_t G = K / kBlock;
  if (R == 0 || G == 0) return hipSuccess;
  const int64_t blocks = (R + kGatherRowsPerBlock - 1) / kGatherRowsPerBlock;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gather_quant_act_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kGroupThreads), 0, stream, x,
                     sorted_pair, q, scale, R, T, static_cast<int32_t>(k), K, static_cast<int>(G));
  return hipGetLastError();
}

hipError_t launch_silu_mul_quant(const uint16_t* y, int64_t M, int64_t F, uint8_t* q, float* scale, uint16_t* h,
                                 hipStream_t stream) {
  const int64_t G = (F + kBlock - 1) / kBlock;
  const int64_t blocks = group_blocks(M * G);
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (h)
    hipLaunchKernelGGL(silu_mul_quant_kernel<true>, dim3(static_cast<uint32_t>(blocks)), dim3(kGroupThreads), 0,
                       stream, y, q, scale, h, M, F, static_cast<int>(G));
  else
    hipLaunchKernelGGL(silu_mul_quant_kernel<false>, dim3(static_cast<uint32_t>(blocks)), dim3(kGroupThreads), 0,
                       stream, y, q, scale, h, M, F, static_cast<int>(G));
  return hipGetLastError();
}

hipError_t launch_moe_combine(const uint16_t* y, const int32_t* pair_row, const float* w, int64_t T, int64_t k,
                              int64_t H, int64_t M, uint16_t* out, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (T > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(combine_kernel, dim3(static_cast<uint32_t>(T)), dim3(kCombineThreads), 0, stream, y, pair_row, w,
                     out, static_cast<int32_t>(k), H, M);
  return hipGetLastError();
}

}  // namespace fp8bq
