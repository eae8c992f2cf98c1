// FP8 KV cache for gfx950: per-step K/V scale calibration and the
// quantizing cache write.
//
// "FP8-RL: A Practical and Stable Low-Precision Stack for LLM Reinforcement
// Learning" (paper-graph-ui summary), §3.4.4 "KV-Cache Quantization": the
// cache holds K and V as 1-byte E4M3 values; because the weights change
// every RL step, the per-layer or per-head scales are recomputed from the K
// and V of the first forward pass of each rollout and then kept for the
// rest of it.  The scale is the tile rule of the linear layers (§3.4.1):
// s = fl32(amax / 448).  Later tokens quantize with the fixed scales,
// q = E4M3_RNE(fl32(x / s)), and saturate to +-448 beyond the calibrated
// range.
//
//   kv_amax_kernel      per-head (or per-layer) max |x| over all tokens:
//                       registers -> LDS max per head -> one global atomic
//                       max per head per workgroup (on the BF16 magnitude
//                       bits, an order-independent exact max)
//   kv_scale_kernel     amax bits -> s in place
//   kv_write_kernel     quantize each token's K / V and store it in its slot
//                       (up to four 16-byte chunks per lane, loads issued first)
#include "device_common.hpp"
#include "group_quant.hpp"
#include "launch.hpp"

namespace fp8bq {

namespace {

constexpr int kKvThreads = 256;
constexpr int kKvMaxChunks = 4 * kKvThreads;  // H * D / 8 <= 1024 (H * D <= 8192)
// Calibration workgroups per tensor: about one per CU, so that few global
// atomics (one per head per workgroup) meet on the same scale words.
constexpr int kKvMaxBlocks = 256;

// K's entries (and V's, when present) of the amax / scale arrays.
__device__ __forceinline__ uint32_t* kv_entry(uint32_t* kb, uint32_t* vb, int n, int i) {
  return i < n ? kb + i : vb + (i - n);
}

__global__ __launch_bounds__(64) void kv_amax_init_kernel(uint32_t* __restrict__ kb, uint32_t* __restrict__ vb,
                                                          int n, int total) {
  for (int i = threadIdx.x; i < total; i += 64) *kv_entry(kb, vb, n, i) = 0u;
}

// grid (blocks, 1 or 2): y = 0 reduces K, y = 1 reduces V.  Block b covers
// tokens [b * per, min(T, (b + 1) * per)).  A thread owns 16-byte chunk
// columns of the [T][H * D] rows, so its head never changes.
__global__ __launch_bounds__(kKvThreads) void kv_amax_kernel(const uint16_t* __restrict__ k,
                                                             const uint16_t* __restrict__ v,
                                                             uint32_t* __restrict__ kbits,
                                                             uint32_t* __restrict__ vbits, int64_t T, int H, int D,
                                                             int per_head, int64_t per) {
  __shared__ uint32_t lmax[kKvMaxChunks];  // one per head (H <= H * D / 8)
  const uint16_t* x = blockIdx.y == 0 ? k : v;
  uint32_t* bits = blockIdx.y == 0 ? kbits : vbits;
  const int tid = threadIdx.x;
  const int C = H * D / 8;  // chunks per token
  const int heads = per_head ? H : 1;
  for (int h = tid; h < heads; h += kKvThreads) lmax[h] = 0u;
  __syncthreads();
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * per;
  const int64_t t1 = (t0 + per < T) ? t0 + per : T;
  const int64_t HD = static_cast<int64_t>(H) * D;
  auto flush = [&](int col, uint32_t m) {
    m = amax_fold(m);
    if (m != 0u) atomicMax(&lmax[per_head ? (col * 8) / D : 0], m);
  };
  if (C <= kKvThreads) {
    const int rows = kKvThreads / C;  // tokens per pass
    const int col = tid % C, r0 = tid / C;
    if (r0 < rows) {
      uint32_t m = 0u;
#pragma unroll 8
      for (int64_t t = t0 + r0; t < t1; t += rows)
        m = amax8(m, *reinterpret_cast<const u32x4*>(x + t * HD + col * 8));
      flush(col, m);
    }
  } else {
    for (int col = tid; col < C; col += kKvThreads) {
      uint32_t m = 0u;
      for (int64_t t = t0; t < t1; ++t) m = amax8(m, *reinterpret_cast<const u32x4*>(x + t * HD + col * 8));
      flush(col, m);
    }
  }
  __syncthreads();
  for (int h = tid; h < heads; h += kKvThreads)
    if (lmax[h] != 0u) atomicMax(&bits[h], lmax[h]);
}

// The BF16 magnitude bits of each amax -> s = fl32(amax / 448), in place.
__global__ __launch_bounds__(64) void kv_scale_kernel(uint32_t* __restrict__ kb, uint32_t* __restrict__ vb, int n,
                                                     int total) {
  for (int i = threadIdx.x; i < total; i += 64) {
    uint32_t* e = kv_entry(kb, vb, n, i);
    *e = __float_as_uint(scale_from_amax_bits(*e));
  }
}

// 8 BF16 values -> 8 E4M3 codes with a fixed scale s > 0: the quotient is
// clamped to +-512 s first (an exact power-of-two multiple; any quotient
// beyond it saturates anyway), formed as fl32(x / s), limited to +-448 and
// converted.
__device__ __forceinline__ u32x2 encode8_sat(u32x4 v, float s) {
  const float x[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                      bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
  float q[8];
  if (s == 0.0f) {  // x / 0 = +-inf saturates; 0 / 0 keeps the zero's sign
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = x[j] == 0.0f ? x[j] : (x[j] > 0.0f ? kE4M3Max : -kE4M3Max);
  } else {
    const float c = 512.0f * s;
    const Divisor d(s);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float xc = __builtin_fminf(__builtin_fmaxf(x[j], -c), c);
      const float qq = d.fast ? d.quotient_fast(xc) : d.quotient_ieee(xc);
      q[j] = __builtin_fminf(__builtin_fmaxf(qq, -kE4M3Max), kE4M3Max);
    }
  }
  return u32x2{pack4_e4m3(q[0], q[1], q[2], q[3]), pack4_e4m3(q[4], q[5], q[6], q[7])};
}

// grid (ceil(T * C / (256 kPer)), 1 or 2): lane l of workgroup b handles
// the 16-byte chunks 256 (b kPer + u) + l, u = 0..kPer-1 (consecutive lanes,
// consecutive chunks).  All the chunks' loads (value, slot, scale) are
// issued before any of them is used, and before the slot decides whether
// anything is stored: with one chunk per lane the value load waited for the
// slot, and too few bytes were in flight to keep HBM busy.  Lanes past the
// last chunk re-load the last one and store nothing.  kPer = 4 for large
// writes (a prefill chunk); 1 for small ones (decode steps), which need the
// workgroups more than the bytes in flight per lane.
template <int kKvWritePer>
__global__ __launch_bounds__(kKvThreads) void kv_write_kernel(const uint16_t* __restrict__ k,
                                                              const uint16_t* __restrict__ v,
                                                              const int32_t* __restrict__ slots,
                                                              const float* __restrict__ ks,
                                                              const float* __restrict__ vs,
                                                              uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
                                                              int64_t T, int H, int D, int per_head, int64_t S) {
  const int C = H * D / 8;
  const int64_t n = T * C;
  const bool is_v = blockIdx.y == 1;
  const uint16_t* x = is_v ? v : k;
  const float* sc = is_v ? vs : ks;
  uint8_t* cache = is_v ? vc : kc;
  const int64_t HD = static_cast<int64_t>(H) * D;
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * (kKvThreads * kKvWritePer) + threadIdx.x;
  int64_t t[kKvWritePer];
  int col[kKvWritePer];
#pragma unroll
  for (int u = 0; u < kKvWritePer; ++u) {
    int64_t i = i0 + u * kKvThreads;
    i = i < n ? i : n - 1;
    if (n <= 0x7fffffffLL) {  // uniform: 32-bit division
      const uint32_t tt = static_cast<uint32_t>(i) / static_cast<uint32_t>(C);
      t[u] = tt;
      col[u] = static_cast<int>(static_cast<uint32_t>(i) - tt * static_cast<uint32_t>(C));
    } else {
      t[u] = i / C;
      col[u] = static_cast<int>(i - t[u] * C);
    }
  }
  int32_t slot[kKvWritePer];
  float s[kKvWritePer];
  u32x4 val[kKvWritePer];
#pragma unroll
  for (int u = 0; u < kKvWritePer; ++u) {
    slot[u] = slots[t[u]];
    s[u] = sc[per_head ? (col[u] * 8) / D : 0];
    val[u] = *reinterpret_cast<const u32x4*>(x + t[u] * HD + col[u] * 8);
  }
#pragma unroll
  for (int u = 0; u < kKvWritePer; ++u) {
    const bool mine = i0 + u * kKvThreads < n;
    if (!mine || slot[u] < 0 || slot[u] >= S) continue;  // past the end, or padding: nothing stored
    *reinterpret_cast<u32x2*>(cache + static_cast<int64_t>(slot[u]) * HD + col[u] * 8) = encode8_sat(val[u], s[u]);
  }
}

}  // namespace

hipError_t launch_kv_calibrate(const uint16_t* k, const uint16_t* v, int64_t T, int64_t H, int64_t D, bool per_head,
                               float* ks, float* vs, hipStream_t stream) {
  const int heads = per_head ? static_cast<int>(H) : 1;
  uint32_t* kb = reinterpret_cast<uint32_t*>(ks);
  uint32_t* vb = reinterpret_cast<uint32_t*>(vs);
  const unsigned ny = vs ? 2u : 1u;
  const int total = heads * static_cast<int>(ny);
  hipLaunchKernelGGL(kv_amax_init_kernel, dim3(1), dim3(64), 0, stream, kb, vb, heads, total);
  if (T > 0) {
    const int64_t blocks = T < kKvMaxBlocks ? T : kKvMaxBlocks;
    const int64_t per = (T + blocks - 1) / blocks;
    const int64_t used = (T + per - 1) / per;
    hipLaunchKernelGGL(kv_amax_kernel, dim3(static_cast<unsigned>(used), ny), dim3(kKvThreads), 0, stream, k, v, kb,
                       vb, T, static_cast<int>(H), static_cast<int>(D), per_head ? 1 : 0, per);
  }
  hipLaunchKernelGGL(kv_scale_kernel, dim3(1), dim3(64), 0, stream, kb, vb, heads, total);
  return hipGetLastError();
}

hipError_t launch_kv_write(const uint16_t* k, const uint16_t* v, const int32_t* slots, const float* ks,
                           const float* vs, bool per_head, uint8_t* kc, uint8_t* vc, int64_t T, int64_t H, int64_t D,
                           int64_t S, hipStream_t stream) {
  const int64_t chunks = T * (H * D / 8);
  if (chunks == 0) return hipSuccess;
  // four chunks per lane while that still leaves >= 512 workgroups per tensor
  const bool wide = chunks >= 512LL * kKvThreads * 4;
  const int per = wide ? 4 : 1;
  const int64_t blocks = (chunks + kKvThreads * per - 1) / (kKvThreads * per);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks), vs ? 2u : 1u);
  if (wide)
    hipLaunchKernelGGL(kv_write_kernel<4>, grid, dim3(kKvThreads), 0, stream, k, v, slots, ks, vs, kc, vc, T,
                       static_cast<int>(H), static_cast<int>(D), per_head ? 1 : 0, S);
  else
    hipLaunchKernelGGL(kv_write_kernel<1>, grid, dim3(kKvThreads), 0, stream, k, v, slots, ks, vs, kc, vc, T,
                       static_cast<int>(H), static_cast<int>(D), per_head ? 1 : 0, S);
  return hipGetLastError();
}

}  // namespace fp8bq
