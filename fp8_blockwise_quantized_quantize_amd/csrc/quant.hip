// Blockwise (128x128) weight quantizer, per-token 1x128 activation quantizer
// and the standalone E4M3 encoder, for gfx950.
//
// Both quantizers compute, per tile: amax -> s = fl32(amax / 448) ->
// q = E4M3_RNE(fl32(x / s)) (FP8-RL summary page, §3.4.1 formula for W^ and
// §3.4.2 Phase 2 step 2; 1x128 activation tiles per §3.4.1 "Static vs.
// Dynamic Quantization").  They are HBM-bound: each BF16 element is read
// once (2 B) and its code written once (1 B), the tile stays in registers
// between the amax pass and the encode pass.
#include "device_common.hpp"
#include "group_quant.hpp"
#include "launch.hpp"

namespace fp8bq {

namespace {

// ---------------------------------------------------------------------------
// Weight blocks: one 256-thread workgroup per 128x128 block.  Thread t owns
// the 16-byte column chunk (t % 16) of rows (t / 16) + 16 i, i = 0..7, so a
// wave reads 4 full 256-byte block rows per load instruction and the whole
// block (64 BF16 per thread) is held in 32 VGPRs.
// ---------------------------------------------------------------------------
constexpr int kQwThreads = 256;

// Byte offset of code (n, k) of an [N][K] matrix in MFMA fragment order
// (N % 16 == 0, K % 128 == 0): per 16-row group and K-block one 2 KB unit,
// in it half (k % 128) / 64, piece ((k % 64) / 16) 16 + n % 16, byte k % 16.
__device__ __forceinline__ int64_t frag_offset(int64_t n, int64_t k, int64_t KB) {
  return ((((n >> 4) * KB + (k >> 7)) * 2 + ((k >> 6) & 1)) << 10) + ((((k >> 4) & 3) << 4) + (n & 15)) * 16 +
         (k & 15);
}

// Block (bn, bk) of one [N][K] matrix; its scale goes to *sslot.  `red`:
// qw_lds_words<kFrag>() words of LDS.  kFrag: codes in MFMA fragment order
// (N % 16 == 0, K % 128 == 0, checked by the host).
template <bool kFrag>
__device__ __forceinline__ void quant_weight_block(const uint16_t* __restrict__ wm, uint8_t* __restrict__ qm,
                                                   float* __restrict__ sslot, int64_t N, int64_t K, int bn, int bk,
                                                   uint32_t* red) {
  const int64_t row0 = (int64_t)bn * kBlock, col0 = (int64_t)bk * kBlock;
  const int tid = threadIdx.x;
  const bool full = (row0 + kBlock <= N) && (col0 + kBlock <= K) && ((K & 7) == 0);

  if (full) {
    const int cc = tid & 15, rr = tid >> 4;
    const uint16_t* src = wm + (row0 + rr) * K + col0 + cc * 8;
    u32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (int64_t)16 * i * K));
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = amax8(m, v[i]);
    m = wave_max_u32(amax_fold(m));
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    m = red[0];
#pragma unroll
    for (int i = 1; i < kQwThreads / 64; ++i) m = m > red[i] ? m : red[i];
    const float s = scale_from_amax_bits(m);
    if (tid == 0) *sslot = s;
    uint8_t* dst = qm + (row0 + rr) * K + col0 + cc * 8;
    // One store loop for the three cases (the choice is uniform per block):
    // 2% faster on the 36-layer sweep than a store loop per case.
    const Divisor d(s != 0.0f ? s : 1.0f);
    if constexpr (kFrag) {
      // The block's 8 fragment units (2 KB each: rows 16 i .., 16 K bytes
      // apart in memory) go through LDS, so that each wave then stores 1 KB
      // contiguous pieces: code row rr + 16 i, bytes cc 8 .. sit in unit i,
      // half cc / 8, piece ((cc % 8) / 2) 16 + rr, bytes (cc % 2) 8 ..
      uint8_t* stage = reinterpret_cast<uint8_t*>(red + kQwThreads / 64);
      const int loff = (cc >> 3) * 1024 + (((cc & 7) >> 1) * 16 + rr) * 16 + (cc & 1) * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const u32x2 o = s == 0.0f ? zero8(v[i]) : (d.fast ? quant8<true>(v[i], d) : quant8<false>(v[i], d));
        *reinterpret_cast<u32x2*>(stage + i * 2048 + loff) = o;
      }
      __syncthreads();
      uint8_t* unit0 = qm + frag_offset(row0, col0, K / kBlock);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int b = j * 4096 + tid * 16;  // unit b / 2048, byte b % 2048 of it
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(stage + b),
                                    reinterpret_cast<u32x4*>(unit0 + (int64_t)(b >> 11) * 16 * K + (b & 2047)));
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x2 o = s == 0.0f ? zero8(v[i]) : (d.fast ? quant8<true>(v[i], d) : quant8<false>(v[i], d));
      __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(dst + (int64_t)16 * i * K));
    }
    return;
  }

  // Partial block (ragged N or K) or rows not 16-byte aligned: element-wise.
  const int rows = (int)((N - row0) < kBlock ? (N - row0) : kBlock);
  const int cols = (int)((K - col0) < kBlock ? (K - col0) : kBlock);
  uint32_t m = 0;
  for (int e = tid; e < kBlock * kBlock; e += kQwThreads) {
    const int r = e >> 7, c = e & 127;
    if (r < rows && c < cols) {
      uint32_t bits = wm[(row0 + r) * K + col0 + c] & 0x7fffu;
      m = m > bits ? m : bits;
    }
  }
  m = wave_max_u32(m);
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = red[0];
  for (int i = 1; i < kQwThreads / 64; ++i) m = m > red[i] ? m : red[i];
  const float s = scale_from_amax_bits(m);
  if (tid == 0) *sslot = s;
  for (int e = tid; e < kBlock * kBlock; e += kQwThreads) {
    const int r = e >> 7, c = e & 127;
    if (r < rows && c < cols) {
      const int64_t off = (row0 + r) * K + col0 + c;
      qm[kFrag ? frag_offset(row0 + r, col0 + c, K / kBlock) : off] = encode1(wm[off], s);
    }
  }
}


// LDS words of a weight workgroup: the amax reduction, then (fragment
// order) the 16 KB block of codes
template <bool kFrag>
constexpr int qw_lds_words() {
  return kQwThreads / 64 + (kFrag ? kBlock * kBlock / 4 : 0);
}

template <bool kFrag>
__global__ __launch_bounds__(kQwThreads) void quant_weight_kernel(const uint16_t* __restrict__ w,
                                                                  uint8_t* __restrict__ q,
                                                                  float* __restrict__ scale, int64_t N,
                                                                  int64_t K, int nb, int kb) {
  __shared__ __align__(16) uint32_t red[qw_lds_words<kFrag>()];
  const int64_t blk = blockIdx.x;  // == index into scale[batch][nb][kb]
  const int bk = (int)(blk % kb);
  const int64_t rest = blk / kb;
  const int bn = (int)(rest % nb);
  const int64_t b = rest / nb;
  quant_weight_block<kFrag>(w + b * N * K, q + b * N * K, scale + blk, N, K, bn, bk, red);
}

// Several matrices in one launch: workgroup g takes block g - first[t] of
// the matrix t with first[t] <= g < first[t + 1] (descriptors in the kernel
// arguments, largest matrices first).
template <bool kFrag>
__global__ __launch_bounds__(kQwThreads) void quant_weight_multi_kernel(const WeightBatch batch) {
  __shared__ __align__(16) uint32_t red[qw_lds_words<kFrag>()];
  const int64_t g = blockIdx.x;
  int t = 0;
  while (t + 1 < batch.count && g >= batch.first[t + 1]) ++t;  // uniform scan over <= 64 entries
  const WeightDesc& d = batch.desc[t];
  const int kb = (int)((d.K + kBlock - 1) / kBlock);
  const int64_t local = g - batch.first[t];
  const int bk = (int)(local % kb), bn = (int)(local / kb);
  quant_weight_block<kFrag>(d.w, d.q, d.s + local, d.N, d.K, bn, bk, red);
}

// ---------------------------------------------------------------------------
// Activation groups: a 16-lane quarter wave per (token, group); each lane
// owns 8 consecutive BF16 (16 bytes).  The group amax is a 4-step xor
// shuffle inside the quarter wave, so a wave quantizes 4 groups at once and
// no LDS or barrier is needed.
// ---------------------------------------------------------------------------
constexpr int kQaThreads = 256;
// Groups per quarter wave, loaded before any is reduced: 4 for large
// problems (more bytes in flight per lane), 1 when that would leave too few
// workgroups to fill the 256 CUs (decode-sized activations).
constexpr int kQaPassesLarge = 4;
constexpr int64_t kQaLargeGroups = 65536;

struct ActGroup {
  int64_t m, col;
  int g;
  bool valid, vec;
  u32x4 v;
};

__device__ __forceinline__ ActGroup act_group_load(const uint16_t* __restrict__ x, int64_t M, int64_t K, int G,
                                                   int64_t gid, int li) {
  ActGroup a;
  a.valid = gid < M * G;
  a.m = a.valid ? gid / G : 0;
  a.g = a.valid ? (int)(gid % G) : 0;
  a.col = (int64_t)a.g * kBlock + li * 8;
  a.vec = a.valid && ((K & 7) == 0) && (a.col + 8 <= K);
  const uint16_t* src = x + a.m * K + a.col;
  a.v = u32x4{0u, 0u, 0u, 0u};
  if (a.vec) {
    a.v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
  } else if (a.valid) {
    uint16_t e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = (a.col + j < K) ? src[j] : (uint16_t)0;
    a.v = u32x4{e[0] | ((uint32_t)e[1] << 16), e[2] | ((uint32_t)e[3] << 16), e[4] | ((uint32_t)e[5] << 16),
                e[6] | ((uint32_t)e[7] << 16)};
  }
  return a;
}

// Group amax over the quarter wave (every lane of the wave takes part), then
// the scale and the codes.
__device__ __forceinline__ void act_group_store(const ActGroup& a, uint8_t* __restrict__ q,
                                                float* __restrict__ scale, int64_t K, int G, int li) {
  uint32_t am = amax_fold(amax8(0u, a.v));
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) {
    uint32_t o = __shfl_xor(am, off, 16);
    am = am > o ? am : o;
  }
  const float s = scale_from_amax_bits(am);
  if (a.valid && li == 0) scale[a.m * G + a.g] = s;
  uint8_t* dst = q + a.m * K + a.col;
  if (a.vec) {
    __builtin_nontemporal_store(encode8(a.v, s), reinterpret_cast<u32x2*>(dst));
  } else if (a.valid) {
    const uint32_t e[8] = {a.v.x & 0xffffu, a.v.x >> 16, a.v.y & 0xffffu, a.v.y >> 16,
                           a.v.z & 0xffffu, a.v.z >> 16, a.v.w & 0xffffu, a.v.w >> 16};
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (a.col + j < K) dst[j] = encode1((uint16_t)e[j], s);
  }
}

// Pass p of quarter wave w (w = threadIdx / 16) takes group
// blockIdx * 16 * kPasses + 16 p + w, so each pass is one coalesced sweep
// over 16 consecutive groups.
template <int kPasses>
__global__ __launch_bounds__(kQaThreads) void quant_act_kernel(const uint16_t* __restrict__ x,
                                                               uint8_t* __restrict__ q,
                                                               float* __restrict__ scale, int64_t M, int64_t K,
                                                               int G) {
  const int li = threadIdx.x & 15;
  const int64_t g0 = (int64_t)blockIdx.x * (kQaThreads / 16) * kPasses + (threadIdx.x >> 4);
  ActGroup grp[kPasses];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) grp[p] = act_group_load(x, M, K, G, g0 + 16 * p, li);
#pragma unroll
  for (int p = 0; p < kPasses; ++p) act_group_store(grp[p], q, scale, K, G, li);
}

// Several activations in one launch (the four of a decode layer step take
// one launch instead of four latency-bound ones): workgroup b takes groups
// 32 (b - first[t]) .. + 31 of the activation t with first[t] <= b <
// first[t + 1], two per quarter wave (both loaded before either is
// reduced; 6.4 vs 6.6 us for one per quarter wave on the four Qwen3-8B
// decode activations, 6.9 us with four).
constexpr int kQaMultiPasses = 2;
__global__ __launch_bounds__(kQaThreads) void quant_act_multi_kernel(const ActBatch batch) {
  static_assert(kQaThreads / 16 * kQaMultiPasses == kActGroupsPerWg, "groups per workgroup");
  const int64_t b = blockIdx.x;
  int t = 0;
  while (t + 1 < batch.count && b >= batch.first[t + 1]) ++t;  // uniform scan over <= 16 entries
  const ActDesc& d = batch.desc[t];
  const int G = (int)((d.K + kBlock - 1) / kBlock);
  const int li = threadIdx.x & 15;
  const int64_t g0 = (b - batch.first[t]) * kActGroupsPerWg + (threadIdx.x >> 4);
  ActGroup grp[kQaMultiPasses];
#pragma unroll
  for (int p = 0; p < kQaMultiPasses; ++p) grp[p] = act_group_load(d.x, d.M, d.K, G, g0 + 16 * p, li);
#pragma unroll
  for (int p = 0; p < kQaMultiPasses; ++p) act_group_store(grp[p], d.q, d.s, d.K, G, li);
}

// ---------------------------------------------------------------------------
// Standalone encoder: method 0 = the hardware conversion exactly as the
// quantizers apply it (valid for |v| < 464), 1 = saturating encoder (clamp
// to +-448, then the hardware conversion), 2 = integer-bit encoder.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void encode_kernel(const float* __restrict__ in, uint8_t* __restrict__ out,
                                                     int64_t n, int method) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float v = in[i];
  uint32_t c;
  if (method == 0) {
    c = cvt_pk_e4m3<false>(v, 0.0f, 0u) & 0xffu;
  } else if (method == 1) {
    c = cvt_pk_e4m3<false>(__builtin_fminf(__builtin_fmaxf(v, -kE4M3Max), kE4M3Max), 0.0f, 0u) & 0xffu;
  } else {
    c = encode_e4m3_soft(v);
  }
  out[i] = (uint8_t)c;
}

// ---------------------------------------------------------------------------
// Activation codes in the MFMA fragment order of the GEMM's activation
// operand: per 16-row group R and K-block g a 2 KB block in which lane
// l = 16 c + r (r = row within the group) holds bytes 16 c .. 16 c + 15 of
// row 16 R + r's K-block at l * 16 and bytes 64 + 16 c .. 79 + 16 c at
// 1024 + l * 16.  One wave per (R, g).  Load i (0..3) of lane l reads the
// 16-byte chunk l % 16 of row 4 i + l / 16, so each load instruction reads
// four whole 256-byte rows (coalesced); a row's amax is a 4-step xor
// shuffle over its 16 lanes.  The codes go through a 2 KB LDS tile into
// fragment order and leave as two contiguous 1 KB stores.  Same scales and
// codes as quant_act_kernel (M % 16 == 0, K % 128 == 0).  (A first form
// loaded each lane's own fragment bytes straight from the rows, 16-byte
// pieces 32 bytes apart: 62 vs 49 us for the row-major quantizer at 8192 x
// 12288.)
// ---------------------------------------------------------------------------
// One unit (16 rows R x K-block g, unit = R G + g) of one activation, by
// one wave; `t` is the wave's 2 KB of LDS.
__device__ __forceinline__ void frag_unit(const uint16_t* __restrict__ x, uint8_t* __restrict__ q,
                                          float* __restrict__ scale, int64_t K, int G, int64_t unit, uint8_t* t) {
  const int lane = threadIdx.x & 63, cc = lane & 15, rq = lane >> 4;
  const int64_t R = unit / G;
  const int g = (int)(unit % G);
  const uint16_t* src = x + (R * 16 + rq) * K + (int64_t)g * kBlock + 8 * cc;
  u32x4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (int64_t)4 * i * K));
  // fragment position of this lane's 8 codes of row r = 4 i + rq, columns
  // 8 cc .. 8 cc + 7: half cc / 8, 16-byte chunk (cc % 8) / 2, byte 8 (cc % 2)
  const int pos = (cc >> 3) * 1024 + ((cc & 7) >> 1) * 256 + (cc & 1) * 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t am = amax_fold(amax8(0u, v[i]));
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) {
      const uint32_t o = __shfl_xor(am, off, 16);
      am = am > o ? am : o;
    }
    const float s = scale_from_amax_bits(am);
    const int r = 4 * i + rq;
    if (cc == 0) scale[(R * 16 + r) * G + g] = s;
    *reinterpret_cast<u32x2*>(t + pos + r * 16) = encode8(v[i], s);
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // the wave's LDS writes before its reads
  const u32x4 lo = *reinterpret_cast<const u32x4*>(t + lane * 16);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(t + 1024 + lane * 16);
  uint8_t* dst = q + (R * G + g) * 2048 + lane * 16;
  __builtin_nontemporal_store(lo, reinterpret_cast<u32x4*>(dst));
  __builtin_nontemporal_store(hi, reinterpret_cast<u32x4*>(dst + 1024));
}

__global__ __launch_bounds__(kQaThreads) void quant_act_frag_kernel(const uint16_t* __restrict__ x,
                                                                    uint8_t* __restrict__ q,
                                                                    float* __restrict__ scale, int64_t M,
                                                                    int64_t K, int G) {
  __shared__ __align__(16) uint8_t tile[kQaThreads / 64][2048];
  const int wave = threadIdx.x >> 6;
  const int64_t unit = (int64_t)blockIdx.x * (kQaThreads / 64) + wave;
  if (unit >= (M / 16) * G) return;  // whole waves
  frag_unit(x, q, scale, K, G, unit, tile[wave]);
}

// Several activations in fragment order in one launch: workgroup b takes
// units 4 (b - first[t]) .. + 3 (16 rows x one K-block each) of activation
// t, one per wave, as quant_act_frag_kernel does for one activation.
__global__ __launch_bounds__(kQaThreads) void quant_act_frag_multi_kernel(const ActBatch batch) {
  __shared__ __align__(16) uint8_t tile[kQaThreads / 64][2048];
  const int64_t b = blockIdx.x;
  int t = 0;
  while (t + 1 < batch.count && b >= batch.first[t + 1]) ++t;  // uniform scan over <= 16 entries
  const ActDesc& d = batch.desc[t];
  const int G = (int)(d.K / kBlock);
  const int wave = threadIdx.x >> 6;
  const int64_t unit = (b - batch.first[t]) * (kQaThreads / 64) + wave;
  if (unit >= (d.M / 16) * G) return;  // whole waves
  frag_unit(d.x, d.q, d.s, d.K, G, unit, tile[wave]);
}

}  // namespace

hipError_t launch_quant_weight(const uint16_t* w, uint8_t* q, float* scale, int64_t batch, int64_t N, int64_t K,
                               bool frag, hipStream_t stream) {
  const int64_t nb = (N + kBlock - 1) / kBlock, kb = (K + kBlock - 1) / kBlock;
  const int64_t blocks = batch * nb * kb;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (frag && ((N % 16) != 0 || (K % kBlock) != 0)) return hipErrorInvalidValue;
  if (frag)
    hipLaunchKernelGGL(quant_weight_kernel<true>, dim3((unsigned)blocks), dim3(kQwThreads), 0, stream, w, q, scale, N,
                       K, (int)nb, (int)kb);
  else
    hipLaunchKernelGGL(quant_weight_kernel<false>, dim3((unsigned)blocks), dim3(kQwThreads), 0, stream, w, q, scale,
                       N, K, (int)nb, (int)kb);
  return hipGetLastError();
}

hipError_t launch_quant_weight_multi(const WeightBatch& batch, int64_t blocks, bool frag, hipStream_t stream) {
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (frag)
    hipLaunchKernelGGL(quant_weight_multi_kernel<true>, dim3((unsigned)blocks), dim3(kQwThreads), 0, stream, batch);
  else
    hipLaunchKernelGGL(quant_weight_multi_kernel<false>, dim3((unsigned)blocks), dim3(kQwThreads), 0, stream, batch);
  return hipGetLastError();
}

hipError_t launch_quant_act_frag(const uint16_t* x, uint8_t* q, float* scale, int64_t M, int64_t K,
                                 hipStream_t stream) {
  const int64_t G = K / kBlock;
  const int64_t units = (M / 16) * G;
  if (units == 0) return hipSuccess;
  if (M % 16 != 0 || K % kBlock != 0) return hipErrorInvalidValue;
  const int64_t blocks = (units + kQaThreads / 64 - 1) / (kQaThreads / 64);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quant_act_frag_kernel, dim3((unsigned)blocks), dim3(kQaThreads), 0, stream, x, q, scale, M, K,
                     (int)G);
  return hipGetLastError();
}

hipError_t launch_quant_act(const uint16_t* x, uint8_t* q, float* scale, int64_t M, int64_t K, hipStream_t stream) {
  const int64_t G = (K + kBlock - 1) / kBlock;
  const int64_t groups = M * G;
  if (groups == 0) return hipSuccess;
  const bool large = groups >= kQaLargeGroups;
  const int64_t per_block = (kQaThreads / 16) * (large ? kQaPassesLarge : 1);
  const int64_t blocks = (groups + per_block - 1) / per_block;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (large)
    hipLaunchKernelGGL(quant_act_kernel<kQaPassesLarge>, dim3((unsigned)blocks), dim3(kQaThreads), 0, stream, x, q,
                       scale, M, K, (int)G);
  else
    hipLaunchKernelGGL(quant_act_kernel<1>, dim3((unsigned)blocks), dim3(kQaThreads), 0, stream, x, q, scale, M, K,
                       (int)G);
  return hipGetLastError();
}

hipError_t launch_quant_act_multi(const ActBatch& batch, int64_t blocks, hipStream_t stream) {
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quant_act_multi_kernel, dim3((unsigned)blocks), dim3(kQaThreads), 0, stream, batch);
  return hipGetLastError();
}

hipError_t launch_quant_act_frag_multi(const ActBatch& batch, int64_t blocks, hipStream_t stream) {
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quant_act_frag_multi_kernel, dim3((unsigned)blocks), dim3(kQaThreads), 0, stream, batch);
  return hipGetLastError();
}

hipError_t launch_encode(const float* in, uint8_t* out, int64_t n, int method, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(encode_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, in, out, n, method);
  return hipGetLastError();
}

}  // namespace fp8bq
