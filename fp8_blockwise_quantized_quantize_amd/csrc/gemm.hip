// Block-scaled W8A8 FP8 GEMM and its ragged grouped (MoE) form, gfx950.
//
//   y[m][n] = sum_kb a_scale[m][kb] * w_scale[n/128][kb] * P[m][n][kb]
//   P[m][n][kb] = sum_{k in K-block kb} dec(a[m][k]) * dec(w[n][k])
//
// (FP8-RL summary page, §3.4.2 Phase 3: FP8 x FP8 matrix multiplication
// with FP32 accumulation, converted back to BF16; §3.4.1 "Quantization
// Scope" for the MoE expert layers.)
//
// One K-block of 128 is exactly one v_mfma_f32_16x16x128_f8f6f4: each MFMA
// produces a fresh FP32 partial P for a 16x16 tile, which is folded into the
// FP32 accumulator with one FMA per element using the combined scale
// a_scale[m][kb] * w_scale[nb][kb].  Weights are the MFMA's A operand (rows
// n) and activations its B operand (columns m), so each lane's four
// accumulator values are four consecutive n of one output row m.
//
// Workgroup tile: 128 (n) x 128 (m), BK = 128, 256 threads = 4 waves in a
// 2 x 2 arrangement, each wave 64 x 64 = 4 x 4 MFMA tiles.  A and W tiles
// are staged through LDS (double-buffered, 2 x 32 KB) with a 16-byte-chunk
// XOR swizzle (chunk ^ (row & 7)) so that the 16 lanes reading 16 rows at
// the same K offset hit distinct banks.  The 128-wide n tile coincides with
// one weight scale block, so w_scale is uniform across the workgroup.
#include "device_common.hpp"
#include "launch.hpp"

namespace fp8bq {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kTile = 128;           // n and m extent of a workgroup tile
constexpr int kThreads = 256;
constexpr int kTileBytes = kTile * kBlock;  // 16 KB of FP8 per operand tile

// D(16x16, FP32) = A(16x128, E4M3) x B(128x16, E4M3); format selectors 0 = E4M3.
__device__ __forceinline__ v4f mfma_16x16x128_e4m3(v8i a, v8i b) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// float32 -> BF16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * kBlock + ((chunk ^ (row & 7)) << 4); }

// Rows [row_lo, row_hi) of an operand, K-block kb: each thread loads four
// 16-byte chunks (rows tid/8 + 32 i, chunk tid % 8); rows outside the range
// read as zero.
struct TileLoader {
  u32x4 v[4];
  __device__ __forceinline__ void load(const uint8_t* base, int64_t ld, int64_t row_lo, int64_t row_hi, int kb,
                                       int tid) {
    const int chunk = tid & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = row_lo + (tid >> 3) + 32 * i;
      if (row < row_hi)
        v[i] = *reinterpret_cast<const u32x4*>(base + row * ld + (int64_t)kb * kBlock + chunk * 16);
      else
        v[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(uint8_t* lds, int tid) const {
    const int chunk = tid & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (tid >> 3) + 32 * i;
      *reinterpret_cast<u32x4*>(lds + swz(row, chunk)) = v[i];
    }
  }
};

// Operand fragment of one 16x128 MFMA tile from LDS: lane l takes row
// (l % 16) and the 32 bytes at K offset 32 * (l / 16).  Weights and
// activations use the same K assignment, so every product pairs equal k.
__device__ __forceinline__ v8i load_frag(const uint8_t* lds, int row0, int lane) {
  const int row = row0 + (lane & 15);
  const int c = (lane >> 4) * 2;
  u32x4 lo = *reinterpret_cast<const u32x4*>(lds + swz(row, c));
  u32x4 hi = *reinterpret_cast<const u32x4*>(lds + swz(row, c + 1));
  v8i f;
  f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
  f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
  return f;
}

struct Smem {
  uint8_t w[2][kTileBytes];
  uint8_t a[2][kTileBytes];
  float sa[2][kTile];
};

// One output tile: activation rows [m_lo, m_hi), weight rows [n0, n0 + 128)
// clipped to N.  `w`/`sw` point at this matrix (expert) and its scale grid.
__device__ __forceinline__ void gemm_tile(Smem& sm, const uint8_t* __restrict__ a, const float* __restrict__ sa,
                                          const uint8_t* __restrict__ w, const float* __restrict__ sw,
                                          uint16_t* __restrict__ y, int64_t m_lo, int64_t m_hi, int64_t n0,
                                          int64_t N, int64_t K) {
  const int KB = (int)(K / kBlock);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int64_t nb = n0 / kTile;  // weight scale block row

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  TileLoader lw, la;
  float sa_reg = 0.f;
  const int64_t n_hi = (n0 + kTile < N) ? n0 + kTile : N;
  if (KB > 0) {
    lw.load(w, K, n0, n_hi, 0, tid);
    la.load(a, K, m_lo, m_hi, 0, tid);
    if (tid < kTile && m_lo + tid < m_hi) sa_reg = sa[(m_lo + tid) * KB];
    lw.store(sm.w[0], tid);
    la.store(sm.a[0], tid);
    if (tid < kTile) sm.sa[0][tid] = sa_reg;
  }

  for (int kb = 0; kb < KB; ++kb) {
    const int cur = kb & 1;
    __syncthreads();
    const bool more = kb + 1 < KB;
    if (more) {
      lw.load(w, K, n0, n_hi, kb + 1, tid);
      la.load(a, K, m_lo, m_hi, kb + 1, tid);
      sa_reg = (tid < kTile && m_lo + tid < m_hi) ? sa[(m_lo + tid) * KB + kb + 1] : 0.f;
    }
    const float swv = sw[nb * KB + kb];
    float cs[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) cs[j] = sm.sa[cur][wm * 64 + j * 16 + (lane & 15)] * swv;
    v8i fw[4], fa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) fw[i] = load_frag(sm.w[cur], wn * 64 + i * 16, lane);
#pragma unroll
    for (int j = 0; j < 4; ++j) fa[j] = load_frag(sm.a[cur], wm * 64 + j * 16, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v4f p = mfma_16x16x128_e4m3(fw[i], fa[j]);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(p[r], cs[j], acc[i][j][r]);
      }
    if (more) {
      lw.store(sm.w[cur ^ 1], tid);
      la.store(sm.a[cur ^ 1], tid);
      if (tid < kTile) sm.sa[cur ^ 1][tid] = sa_reg;
    }
  }

  // Epilogue: lane holds n = n0 + wn*64 + i*16 + (lane/16)*4 + r, m = m_lo + wm*64 + j*16 + lane%16.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t m = m_lo + wm * 64 + j * 16 + (lane & 15);
    if (m >= m_hi) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t n = n0 + wn * 64 + i * 16 + (lane >> 4) * 4;
      uint16_t* dst = y + m * N + n;
      if (n + 4 <= N && (N & 3) == 0) {
        u32x2 pk;
        pk.x = bf16_rne(acc[i][j][0]) | (bf16_rne(acc[i][j][1]) << 16);
        pk.y = bf16_rne(acc[i][j][2]) | (bf16_rne(acc[i][j][3]) << 16);
        *reinterpret_cast<u32x2*>(dst) = pk;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < N) dst[r] = (uint16_t)bf16_rne(acc[i][j][r]);
      }
    }
  }
}

__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(const uint8_t* __restrict__ a,
                                                           const float* __restrict__ sa,
                                                           const uint8_t* __restrict__ w,
                                                           const float* __restrict__ sw, uint16_t* __restrict__ y,
                                                           int64_t M, int64_t N, int64_t K, int tiles_n) {
  __shared__ Smem sm;
  const int tn = blockIdx.x % tiles_n;
  const int64_t tm = blockIdx.x / tiles_n;
  const int64_t m_lo = tm * kTile;
  const int64_t m_hi = (m_lo + kTile < M) ? m_lo + kTile : M;
  gemm_tile(sm, a, sa, w, sw, y, m_lo, m_hi, (int64_t)tn * kTile, N, K);
}

// Grouped form: workgroup slot t (blockIdx.x / tiles_n) is mapped to (expert,
// m-tile) by a prefix sum over ceil(rows_e / 128) computed from the device
// offsets inside the workgroup; slots past the last tile exit.  Offsets are
// clamped so that every row index stays in [0, M).
__global__ __launch_bounds__(kThreads, 2) void grouped_gemm_kernel(
    const uint8_t* __restrict__ a, const float* __restrict__ sa, const uint8_t* __restrict__ w,
    const float* __restrict__ sw, const int32_t* __restrict__ offsets, uint16_t* __restrict__ y, int64_t M,
    int64_t N, int64_t K, int G, int tiles_n) {
  __shared__ Smem sm;
  __shared__ int found_e, found_t;
  __shared__ int wave_sum[kThreads / 64];
  const int tn = blockIdx.x % tiles_n;
  const int slot = blockIdx.x / tiles_n;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) found_e = -1;
  int base = 0;  // tiles of experts before this chunk
  for (int c0 = 0; c0 < G; c0 += kThreads) {
    const int e = c0 + tid;
    int tiles = 0;
    if (e < G) {
      int lo = offsets[e], hi = offsets[e + 1];
      lo = lo < 0 ? 0 : (lo > M ? (int)M : lo);
      hi = hi < lo ? lo : (hi > M ? (int)M : hi);
      tiles = (hi - lo + kTile - 1) / kTile;
    }
    // inclusive scan over the workgroup
    int incl = tiles;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    __syncthreads();
    if (lane == 63) wave_sum[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int i = 0; i < wave; ++i) before += wave_sum[i];
    incl += before;
    const int excl = incl - tiles;
    if (e < G && slot >= base + excl && slot < base + incl) {
      found_e = e;
      found_t = slot - base - excl;
    }
    int total = 0;
    for (int i = 0; i < kThreads / 64; ++i) total += wave_sum[i];
    base += total;
  }
  __syncthreads();
  const int e = found_e;
  if (e < 0) return;  // uniform: beyond the last tile
  int lo = offsets[e], hi = offsets[e + 1];
  lo = lo < 0 ? 0 : (lo > M ? (int)M : lo);
  hi = hi < lo ? lo : (hi > M ? (int)M : hi);
  const int64_t m_lo = (int64_t)lo + (int64_t)found_t * kTile;
  const int64_t m_hi = (m_lo + kTile < hi) ? m_lo + kTile : hi;
  const int64_t KB = K / kBlock;
  const int64_t NB = (N + kTile - 1) / kTile;
  gemm_tile(sm, a, sa, w + (int64_t)e * N * K, sw + (int64_t)e * NB * KB, y, m_lo, m_hi, (int64_t)tn * kTile, N, K);
}

}  // namespace

hipError_t launch_gemm(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw, uint16_t* y, int64_t M,
                       int64_t N, int64_t K, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int64_t tiles_n = (N + kTile - 1) / kTile, tiles_m = (M + kTile - 1) / kTile;
  const int64_t blocks = tiles_n * tiles_m;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemm_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a, sa, w, sw, y, M, N, K,
                     (int)tiles_n);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw,
                               const int32_t* offsets, uint16_t* y, int64_t M, int64_t N, int64_t K, int64_t G,
                               hipStream_t stream) {
  if (M == 0 || N == 0 || G == 0) return hipSuccess;
  const int64_t tiles_n = (N + kTile - 1) / kTile;
  const int64_t slots = (M + kTile - 1) / kTile + G;  // >= sum_e ceil(rows_e / 128)
  const int64_t blocks = tiles_n * slots;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(grouped_gemm_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a, sa, w, sw, offsets,
                     y, M, N, K, (int)G, (int)tiles_n);
  return hipGetLastError();
}

}  // namespace fp8bq
