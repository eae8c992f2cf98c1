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
// produces a fresh FP32 partial P for a 16x16 tile, folded into the FP32
// accumulator with one FMA per element using a_scale[m][kb] * w_scale[nb][kb].
// Weights are the MFMA's A operand (rows n), activations its B operand
// (columns m), so each lane's four results are four consecutive n of one
// output row m (8-byte BF16 stores).
//
// Two tile kernels share that inner step:
//
//  * skinny<BN, BM> (few activation rows, e.g. decode with M = 256): a
//    BN x BM output tile per 4-wave workgroup; the four waves split the
//    K-blocks (wave w takes kb = w, w+4, ...), each loading its own
//    operands straight from global memory into MFMA fragment registers
//    (nothing is loaded twice within the workgroup), two K-blocks ahead;
//    the four partial tiles are summed through LDS at the end.  Per-CU
//    operand traffic is (BN + BM) * K, which is what bounds these shapes
//    (the activation panel is re-read from L2 by every workgroup).
//
//  * wide (many rows: prefill, MoE experts): a 128 (n) x 256 (m) tile per
//    4-wave workgroup, waves split along m (64 rows each).  The 128 x 128
//    weight K-block is shared by all four waves, so it is staged through
//    LDS (register-staged, double-buffered, 16-byte XOR swizzle); each
//    wave's activation rows are private and go straight from global memory
//    into fragment registers.  Loads run two K-blocks ahead.
//
// Tiles are ordered so that the workgroups resident on one XCD at a time
// (consecutive workgroup ids of the same id % 8) share weight and
// activation panels in that XCD's L2.
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace fp8bq {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kXcds = 8;

// D(16x16, FP32) = A(16x128, E4M3) x B(128x16, E4M3); format selectors 0 = E4M3.
__device__ __forceinline__ v4f mfma_e4m3(v8i a, v8i b) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// float32 -> BF16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ v8i to_v8i(u32x4 lo, u32x4 hi) {
  v8i f;
  f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
  f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
  return f;
}

// Raw buffer resource over [base, base + bytes): loads past the end return
// zero instead of faulting, and the K offset of a K-block goes in an SGPR.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

__device__ __forceinline__ float bload_f32(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

// Operand fragment of a 16-row x 128-K tile: lane l holds row (l & 15) and
// the 16-byte K chunks g = l >> 4 and g + 4 of the K-block.  Every operand
// uses this same assignment, so the MFMA pairs equal k in A and B.  `voff`
// is row * K + 16 g within the panel, `koff` = 128 kb.
__device__ __forceinline__ v8i frag_buf(__amdgpu_buffer_rsrc_t r, int voff, int koff) {
  return to_v8i(bload16(r, voff, koff), bload16(r, voff + 64, koff));
}

// LDS tile of 128 rows x 128 bytes, 16-byte chunk c of row r stored at
// chunk position c ^ (r & 7): the 8 lanes of one LDS cycle read 8 rows at
// the same logical chunk and hit 8 distinct bank groups.
__device__ __forceinline__ int swz(int row, int chunk) { return row * kBlock + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ v8i frag_lds(const uint8_t* lds, int row, int g) {
  const u32x4 lo = *reinterpret_cast<const u32x4*>(lds + swz(row, g));
  const u32x4 hi = *reinterpret_cast<const u32x4*>(lds + swz(row, g + 4));
  return to_v8i(lo, hi);
}

// Fence for both the IR optimizer and the machine scheduler: loads and MFMAs
// stay on their side, so prefetches are issued before the compute that
// overlaps them (otherwise the compiler sinks them and then waits on them).
__device__ __forceinline__ void order_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Rows of one output tile: activation rows [m_lo, m_hi), weight rows
// [n0, min(n0 + BN, N)); `w`/`sw` point at this matrix (expert).
struct Tile {
  const uint8_t* a;
  const float* sa;
  const uint8_t* w;
  const float* sw;
  uint16_t* y;
  int64_t m_lo, m_hi, n0, N, K;
  // K-block rotation: the tile visits K-blocks starting at `rot` (mod KB).
  // Rows of one K-block column are K bytes apart and land on few L2
  // channels; spreading the workgroups' K positions spreads the channels.
  int rot;
};

// Store four consecutive n of output row m (BF16, RNE).
__device__ __forceinline__ void store4(uint16_t* __restrict__ y, int64_t N, int64_t m, int64_t n, v4f v) {
  uint16_t* dst = y + m * N + n;
  if (n + 4 <= N && (N & 3) == 0) {
    u32x2 pk;
    pk.x = bf16_rne(v[0]) | (bf16_rne(v[1]) << 16);
    pk.y = bf16_rne(v[2]) | (bf16_rne(v[3]) << 16);
    *reinterpret_cast<u32x2*>(dst) = pk;
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (n + r < N) dst[r] = (uint16_t)bf16_rne(v[r]);
  }
}

// ---------------------------------------------------------------------------
// skinny<BN, BM>: K split across the 4 waves.  Each wave stages its own
// K-block (BN weight rows + BM activation rows, 128 bytes each) through its
// own LDS slice: coalesced 16-byte global loads (8 lanes per 128-byte row)
// into registers one K-block ahead, ds_write into the swizzled slice, and
// MFMA fragments read back with ds_read_b128.  Waves never share LDS data,
// so the K loop has no workgroup barrier.
// ---------------------------------------------------------------------------
template <int BN, int BM>
struct Skinny {
  static constexpr int TN = BN / 16, TM = BM / 16;
  static constexpr int kRows = BN + BM;                 // rows staged per K-block
  static constexpr int kLoads = kRows / 8;              // 16-byte loads per lane per K-block
  static constexpr int kSlice = kRows * kBlock;         // LDS bytes per wave
  static constexpr int kRed = 4 * BN * BM * 4;          // four partial tiles, FP32
  static constexpr int kLdsBytes = (4 * kSlice > kRed) ? 4 * kSlice : kRed;
  static constexpr int kWavesPerSimd = 1;               // one workgroup per CU; registers to 512

  struct Stage {
    u32x4 v[kLoads];
    float sav[TM], swv[TN];
  };

  __device__ static __forceinline__ void run(const Tile& t, float* red) {
    const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int64_t K = t.K;
    const int KB = (int)(K / kBlock);
    const int64_t n_hi = (t.n0 + BN < t.N) ? t.n0 + BN : t.N;
    const auto wr = make_rsrc(t.w + t.n0 * K, (n_hi - t.n0) * K);
    const auto ar = make_rsrc(t.a + t.m_lo * K, (t.m_hi - t.m_lo) * K);
    const auto sr = make_rsrc(t.sa + t.m_lo * KB, (t.m_hi - t.m_lo) * KB * 4);
    const float* swrow[TN];  // a 16-row n-tile lies in one 128-row scale block
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      int64_t nt = t.n0 + i * 16;
      nt = nt < t.N ? nt : t.N - 1;
      swrow[i] = t.sw + (nt / kBlock) * KB;
    }
    // staging: lane owns chunk (lane & 7) of rows (lane >> 3) + 8 q; slice
    // rows 0..BN-1 are weight rows, BN..BN+BM-1 activation rows
    const int lrow = lane >> 3, lchunk = lane & 7;
    const int gvoff = lrow * (int)K + lchunk * 16;
    const int svoff = r16 * KB * 4;  // + 16 j KB 4
    uint8_t* slice = reinterpret_cast<uint8_t*>(red) + wave * kSlice;

    v4f acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    auto load_stage = [&](Stage& s, int step) {
      int kb = step + t.rot;  // rotated K-block id, step < KB
      kb = kb < KB ? kb : kb - KB;
      const int koff = kb * kBlock;
#pragma unroll
      for (int q = 0; q < BN / 8; ++q) s.v[q] = bload16(wr, gvoff + 8 * q * (int)K, koff);
#pragma unroll
      for (int q = 0; q < BM / 8; ++q) s.v[BN / 8 + q] = bload16(ar, gvoff + 8 * q * (int)K, koff);
#pragma unroll
      for (int j = 0; j < TM; ++j) s.sav[j] = bload_f32(sr, svoff + j * 16 * KB * 4, kb * 4);
#pragma unroll
      for (int i = 0; i < TN; ++i) s.swv[i] = swrow[i][kb];
    };
    auto store_stage = [&](const Stage& s) {
#pragma unroll
      for (int q = 0; q < kLoads; ++q) *reinterpret_cast<u32x4*>(slice + swz(lrow + 8 * q, lchunk)) = s.v[q];
    };
    auto compute = [&](const Stage& s) {
      v8i fa[TM];
#pragma unroll
      for (int j = 0; j < TM; ++j) fa[j] = frag_lds(slice, BN + j * 16 + r16, g);
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        const v8i fw = frag_lds(slice, i * 16 + r16, g);
#pragma unroll
        for (int j = 0; j < TM; ++j) {
          const v4f p = mfma_e4m3(fw, fa[j]);
          const float c = s.sav[j] * s.swv[i];
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(p[r], c, acc[i][j][r]);
        }
      }
    };

    // this wave's K-blocks: wave, wave + 4, ...  Stage sX holds the
    // registers of the next K-block while the LDS slice holds the current.
    // Prefetches past the last K-block re-read the last one (clamped).
    const int kb_last = KB - 1;
    auto nxt = [&](int kb) { return kb < KB ? kb : kb_last; };
    Stage s0, s1;
    int kb = wave;
    if (kb < KB) {
      order_fence();
      load_stage(s0, kb);
      order_fence();
      store_stage(s0);
      load_stage(s1, nxt(kb + 4));
      order_fence();
    }
    for (; kb + 4 < KB; kb += 8) {
      compute(s0);                      // K-block kb from the slice, scales from s0
      order_fence();
      load_stage(s0, nxt(kb + 8));
      order_fence();
      store_stage(s1);                  // K-block kb + 4 into the slice
      order_fence();
      compute(s1);
      order_fence();
      load_stage(s1, nxt(kb + 12));
      order_fence();
      store_stage(s0);                  // K-block kb + 8
      order_fence();
    }
    if (kb < KB) compute(s0);

    // Sum the four waves' partial tiles through LDS; thread t then owns 16
    // consecutive floats of the tile in fragment order.
    __syncthreads();  // every wave is done with its staging slice
    float* mine = red + wave * (BN * BM);
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) *reinterpret_cast<v4f*>(mine + ((i * TM + j) * 64 + lane) * 4) = acc[i][j];
    __syncthreads();
    constexpr int kGroups = BN * BM / 16;  // groups of 16 floats: 4 lanes x 4 values of one (i, j)
#pragma unroll
    for (int q = 0; q < (kGroups + kThreads - 1) / kThreads; ++q) {
      const int gi = q * kThreads + threadIdx.x;
      if (gi >= kGroups) break;
      const int base = gi * 16;
      v4f sum[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        sum[u] = *reinterpret_cast<const v4f*>(red + base + 4 * u);
#pragma unroll
        for (int w2 = 1; w2 < 4; ++w2) sum[u] += *reinterpret_cast<const v4f*>(red + w2 * (BN * BM) + base + 4 * u);
      }
      const int ij = base / 256, l0 = (base / 4) % 64;
      const int i = ij / TM, j = ij % TM;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int l = l0 + u;
        const int64_t m = t.m_lo + j * 16 + (l & 15);
        const int64_t n = t.n0 + i * 16 + (l >> 4) * 4;
        if (m < t.m_hi) store4(t.y, t.N, m, n, sum[u]);
      }
    }
  }
};

// ---------------------------------------------------------------------------
// wide: 128 (n) x 256 (m) tile, W K-blocks through LDS, activations direct.
// ---------------------------------------------------------------------------
struct Wide {
  static constexpr int BN = 128, BM = 256, TN = 8, TM = 4;
  static constexpr int kLdsBytes = 2 * BN * kBlock;  // double-buffered W K-block
  static constexpr int kWavesPerSimd = 2;             // two workgroups per CU hide MFMA latency

  struct AStage {
    v8i fa[TM];
    float sav[TM];
    float swv;
  };

  __device__ static __forceinline__ void run(const Tile& t, uint8_t* lds) {
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int64_t K = t.K;
    const int KB = (int)(K / kBlock);
    const int64_t n_hi = (t.n0 + BN < t.N) ? t.n0 + BN : t.N;
    const float* swrow = t.sw + (t.n0 / kBlock) * KB;  // n0 is a multiple of 128: one scale block
    const auto wr = make_rsrc(t.w + t.n0 * K, (n_hi - t.n0) * K);
    const int64_t am_lo = t.m_lo + wave * 64;  // this wave's activation rows
    const int64_t am_hi = (am_lo + 64 < t.m_hi) ? am_lo + 64 : t.m_hi;
    const int64_t arows = am_hi > am_lo ? am_hi - am_lo : 0;
    const auto ar = make_rsrc(t.a + am_lo * K, arows * K);
    const auto sr = make_rsrc(t.sa + am_lo * KB, arows * KB * 4);

    // W staging: thread owns chunk (tid & 7) of rows (tid >> 3) + 32 q, q = 0..3
    const int wchunk = tid & 7;
    const int wvoff = (tid >> 3) * (int)K + wchunk * 16;  // + 32 q K
    const int avoff = r16 * (int)K + 16 * g;              // + 16 j K
    const int svoff = r16 * KB * 4;                       // + 16 j KB 4

    v4f acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    u32x4 wreg[4];
    auto rotk = [&](int step) {  // rotated K-block id, step < KB
      const int kb = step + t.rot;
      return kb < KB ? kb : kb - KB;
    };
    auto load_w = [&](int step) {
      const int kb = rotk(step);
#pragma unroll
      for (int q = 0; q < 4; ++q) wreg[q] = bload16(wr, wvoff + 32 * q * (int)K, kb * kBlock);
    };
    auto store_w = [&](uint8_t* buf) {
#pragma unroll
      for (int q = 0; q < 4; ++q) *reinterpret_cast<u32x4*>(buf + swz((tid >> 3) + 32 * q, wchunk)) = wreg[q];
    };
    auto load_a = [&](AStage& s, int step) {
      const int kb = rotk(step);
#pragma unroll
      for (int j = 0; j < TM; ++j) s.fa[j] = frag_buf(ar, avoff + j * 16 * (int)K, kb * kBlock);
#pragma unroll
      for (int j = 0; j < TM; ++j) s.sav[j] = bload_f32(sr, svoff + j * 16 * KB * 4, kb * 4);
      s.swv = swrow[kb];
    };
    auto compute = [&](const AStage& s, const uint8_t* buf) {
      float c[TM];
#pragma unroll
      for (int j = 0; j < TM; ++j) c[j] = s.sav[j] * s.swv;
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        const v8i fw = frag_lds(buf, i * 16 + r16, g);
#pragma unroll
        for (int j = 0; j < TM; ++j) {
          const v4f p = mfma_e4m3(fw, s.fa[j]);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(p[r], c[j], acc[i][j][r]);
        }
      }
    };

    uint8_t* buf0 = lds;
    uint8_t* buf1 = lds + BN * kBlock;
    AStage s0, s1;
    const int kb_last = KB - 1;
    auto nxt = [&](int kb) { return kb < KB ? kb : kb_last; };  // clamped prefetch index
    if (KB > 0) {
      order_fence();
      load_w(0);
      load_a(s0, 0);
      order_fence();
      store_w(buf0);
      load_w(nxt(1));
      order_fence();
      load_a(s1, nxt(1));
      order_fence();
    }
    // iteration kb: W(kb) in LDS, W(kb+1) in wreg, activations of kb in stage kb&1
    int kb = 0;
    for (; kb + 1 < KB; kb += 2) {
      __syncthreads();  // buf0 holds W(kb); buf1 is free
      store_w(buf1);
      load_w(nxt(kb + 2));
      order_fence();
      compute(s0, buf0);
      order_fence();
      load_a(s0, nxt(kb + 2));
      order_fence();
      __syncthreads();  // buf1 holds W(kb+1); buf0 is free
      store_w(buf0);
      load_w(nxt(kb + 3));
      order_fence();
      compute(s1, buf1);
      order_fence();
      load_a(s1, nxt(kb + 3));
      order_fence();
    }
    if (kb < KB) {
      __syncthreads();
      compute(s0, buf0);
    }

#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int64_t m = t.m_lo + wave * 64 + j * 16 + r16;
      if (m >= t.m_hi) continue;
#pragma unroll
      for (int i = 0; i < TN; ++i) store4(t.y, t.N, m, t.n0 + i * 16 + g * 4, acc[i][j]);
    }
  }
};

// ---------------------------------------------------------------------------
// Tile order: XCD-aware remap of the workgroup id, then groups of kGroupM
// m-tiles swept along n (m fastest inside a group).
// ---------------------------------------------------------------------------
constexpr int kGroupM = 8;

__device__ __forceinline__ int64_t xcd_linear(int64_t bid, int64_t total) {
  const int64_t x = bid % kXcds, local = bid / kXcds;
  const int64_t per = total / kXcds, extra = total % kXcds;
  return x * per + (x < extra ? x : extra) + local;
}

__device__ __forceinline__ void tile_of(int64_t L, int64_t tiles_m, int64_t tiles_n, int64_t* tm, int64_t* tn) {
  const int64_t group = L / (kGroupM * tiles_n);
  const int64_t first_m = group * kGroupM;
  const int64_t rem = tiles_m - first_m;
  const int64_t gsize = rem < kGroupM ? rem : kGroupM;
  const int64_t idx = L % (kGroupM * tiles_n);
  *tm = first_m + idx % gsize;
  *tn = idx / gsize;
}

template <class Kern, int BN, int BM>
__global__ __launch_bounds__(kThreads, Kern::kWavesPerSimd) void gemm_dense_kernel(const uint8_t* __restrict__ a,
                                                                 const float* __restrict__ sa,
                                                                 const uint8_t* __restrict__ w,
                                                                 const float* __restrict__ sw,
                                                                 uint16_t* __restrict__ y, int64_t M, int64_t N,
                                                                 int64_t K, int64_t tiles_m, int64_t tiles_n) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int64_t L = xcd_linear(blockIdx.x, tiles_m * tiles_n);
  int64_t tm, tn;
  tile_of(L, tiles_m, tiles_n, &tm, &tn);
  Tile t;
  t.a = a; t.sa = sa; t.w = w; t.sw = sw; t.y = y;
  t.m_lo = tm * BM;
  t.m_hi = (t.m_lo + BM < M) ? t.m_lo + BM : M;
  t.n0 = tn * BN;
  t.N = N; t.K = K;
  t.rot = (int)((L * 4) % (K / kBlock > 0 ? K / kBlock : 1));
  if constexpr (std::is_same<Kern, Wide>::value)
    Wide::run(t, smem);
  else
    Kern::run(t, reinterpret_cast<float*>(smem));
}

// Grouped form: workgroup slot s is mapped to (expert, m-tile) by a prefix
// sum over ceil(rows_e / BM) computed in the workgroup from the device
// offsets; slots past the last tile exit.  Offsets are clamped to [0, M].
template <class Kern, int BN, int BM>
__global__ __launch_bounds__(kThreads, Kern::kWavesPerSimd) void gemm_grouped_kernel(
    const uint8_t* __restrict__ a, const float* __restrict__ sa, const uint8_t* __restrict__ w,
    const float* __restrict__ sw, const int32_t* __restrict__ offsets, uint16_t* __restrict__ y, int64_t M,
    int64_t N, int64_t K, int G, int64_t slots, int64_t tiles_n) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int found_e, found_t;
  __shared__ int wave_sum[kThreads / 64];
  const int64_t L = xcd_linear(blockIdx.x, slots * tiles_n);
  // n fastest: the workgroups of one (expert, m-tile) share its activation rows
  const int64_t tn = L % tiles_n;
  const int slot = (int)(L / tiles_n);
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
      tiles = (hi - lo + BM - 1) / BM;
    }
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
  const int64_t KB = K / kBlock;
  const int64_t NB = (N + kBlock - 1) / kBlock;
  Tile t;
  t.a = a; t.sa = sa;
  t.w = w + (int64_t)e * N * K;
  t.sw = sw + (int64_t)e * NB * KB;
  t.y = y;
  t.m_lo = (int64_t)lo + (int64_t)found_t * BM;
  t.m_hi = (t.m_lo + BM < hi) ? t.m_lo + BM : hi;
  t.n0 = tn * BN;
  t.N = N; t.K = K;
  t.rot = (int)((L * 4) % (KB > 0 ? KB : 1));
  if constexpr (std::is_same<Kern, Wide>::value)
    Wide::run(t, smem);
  else
    Kern::run(t, reinterpret_cast<float*>(smem));
}

enum class Cfg { kSkinny64x64, kSkinny96x64, kWide };

// Per-workgroup cycle estimate: operand bytes through L1 (64 B/clk/CU) vs
// FP8 MFMA (8192 FLOP/clk/CU), times the rounds of workgroups over 256 CUs.
double est_cycles(int64_t M, int64_t N, int64_t K, int bn, int bm, double cus) {
  const double tiles = (double)((N + bn - 1) / bn) * (double)((M + bm - 1) / bm);
  const double rounds = tiles / cus < 1.0 ? 1.0 : (tiles + cus - 1) / cus;
  const double l1 = (double)(bn + bm) * (double)K / 64.0;
  const double mfma = 2.0 * bn * bm * (double)K / 8192.0;
  return rounds * (l1 > mfma ? l1 : mfma);
}

Cfg choose(int64_t M, int64_t N, int64_t K) {
  const double cus = 256.0;
  double best = est_cycles(M, N, K, Wide::BN, Wide::BM, cus);
  Cfg c = Cfg::kWide;
  const double s64 = est_cycles(M, N, K, 64, 64, cus) * 1.05;  // partial-tile reduction overhead
  if (s64 < best) { best = s64; c = Cfg::kSkinny64x64; }
  const double s96 = est_cycles(M, N, K, 96, 64, cus) * 1.05;
  if (s96 < best) { best = s96; c = Cfg::kSkinny96x64; }
  return c;
}

template <class Kern, int BN, int BM>
hipError_t launch_dense_cfg(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw, uint16_t* y,
                            int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int64_t blocks = tiles_m * tiles_n;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_dense_kernel<Kern, BN, BM>), dim3((unsigned)blocks), dim3(kThreads),
                     (size_t)Kern::kLdsBytes, stream, a, sa, w, sw, y, M, N, K, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw, uint16_t* y, int64_t M,
                       int64_t N, int64_t K, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  switch (choose(M, N, K)) {
    case Cfg::kSkinny64x64:
      return launch_dense_cfg<Skinny<64, 64>, 64, 64>(a, sa, w, sw, y, M, N, K, stream);
    case Cfg::kSkinny96x64:
      return launch_dense_cfg<Skinny<96, 64>, 96, 64>(a, sa, w, sw, y, M, N, K, stream);
    default:
      return launch_dense_cfg<Wide, Wide::BN, Wide::BM>(a, sa, w, sw, y, M, N, K, stream);
  }
}

hipError_t launch_grouped_gemm(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw,
                               const int32_t* offsets, uint16_t* y, int64_t M, int64_t N, int64_t K, int64_t G,
                               hipStream_t stream) {
  if (M == 0 || N == 0 || G == 0) return hipSuccess;
  const int64_t tiles_n = (N + Wide::BN - 1) / Wide::BN;
  const int64_t slots = (M + Wide::BM - 1) / Wide::BM + G;  // >= sum_e ceil(rows_e / BM)
  const int64_t blocks = tiles_n * slots;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_grouped_kernel<Wide, Wide::BN, Wide::BM>), dim3((unsigned)blocks), dim3(kThreads),
                     (size_t)Wide::kLdsBytes, stream, a, sa, w, sw, offsets, y, M, N, K, (int)G, slots, tiles_n);
  return hipGetLastError();
}

}  // namespace fp8bq
