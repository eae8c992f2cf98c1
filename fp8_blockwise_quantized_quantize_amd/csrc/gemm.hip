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
//  * skinny<64, 48 or 96, 64> (few activation rows, e.g. decode with
//    M = 256): a 64 (48, 96) x 64 output tile per 4-wave workgroup; the four
//    waves split the K-blocks (wave w takes kb = w, w+4, ...).  Row-major
//    operands are staged through each wave's private LDS slice (coalesced
//    16-byte loads into registers one K-block ahead, ds_write, fragment
//    reads); fragment-order operands are loaded straight into the MFMA's
//    registers.  The four partial tiles are summed through LDS at the end.
//
//  * panel<BN, BM, ..., S> (many rows: prefill with a 256 x 256 tile, two
//    stages; MoE experts with a 256 x 128 tile, three stages; decode with
//    many weight rows with a 128 x 256 or 192 x 128 tile, three stages):
//    eight waves (two per SIMD).  Both operands of a K-block and its scales
//    go global -> LDS directly (buffer_load ... lds) into a ring of S
//    stages, one barrier per K-block; the loads of K-block k + S - 1 are
//    spread over the MFMAs of K-block k.
//
// The grouped GEMM runs the panel persistently: one workgroup per CU takes
// expert tiles in turn, and the ring runs on from one tile's K-blocks into
// the next tile's, so no tile waits for its pipeline to fill.
//
// Tiles are ordered so that the workgroups resident on one XCD at a time
// (consecutive workgroup ids of the same id % 8) share weight and
// activation panels in that XCD's L2.
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"
#include "silu_math.hpp"

namespace fp8bq {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

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

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// bf16_rne(a) | bf16_rne(b) << 16 in one v_cvt_pk_bf16_f32 (gfx950).  The
// same bits as bf16_rne for every non-NaN float32, denormals and
// infinities included (all 2^32 inputs compared on an MI355X); a NaN stays
// a NaN.
__device__ __forceinline__ uint32_t bf16_pack2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
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

// LDS tile of 128 rows x 128 bytes, 16-byte chunk c of row r stored at
// chunk position c ^ (r & 7): the 8 lanes of one LDS cycle read 8 rows at
// the same logical chunk and hit 8 distinct bank groups.
__device__ __forceinline__ int swz(int row, int chunk) { return row * kBlock + ((chunk ^ (row & 7)) << 4); }


// Per-lane byte offsets of the two fragment chunks inside a 16-row group of
// a swizzled LDS tile ((row0 + r16) & 7 == r16 & 7 for row0 % 16 == 0), so
// a fragment read is one base register plus an immediate row offset.
struct FragLds {
  int lo, hi;
  __device__ __forceinline__ FragLds(int lane) {
    const int g = lane >> 4, r16 = lane & 15;
    lo = r16 * kBlock + ((g ^ (r16 & 7)) << 4);
    hi = r16 * kBlock + (((g + 4) ^ (r16 & 7)) << 4);
  }
  // fragment of stage rows row0 .. row0 + 15 (row0 a multiple of 16)
  __device__ __forceinline__ v8i operator()(const uint8_t* buf, int row0) const {
    const uint8_t* p = buf + row0 * kBlock;
    return to_v8i(*reinterpret_cast<const u32x4*>(p + lo), *reinterpret_cast<const u32x4*>(p + hi));
  }
};

// Fence for both the IR optimizer and the machine scheduler: loads and MFMAs
// stay on their side, so prefetches are issued before the compute that
// overlaps them (otherwise the compiler sinks them and then waits on them).
__device__ __forceinline__ void order_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// acc[i][j] += (P(i, j) = MFMA(fw_i, fa_j)) * c(i, j) over a TN x TM grid of
// 16x16 tiles, software-pipelined: the FMAs of MFMA t are issued after MFMA
// t + kDelay, with the partials in a ring of kDelay + 1 registers, so the
// MFMA pipe need not wait for its own result (with two waves per SIMD a
// short delay suffices: the other wave fills the gap).  sched_group_barrier pins the
// interleave (one MFMA, then the four FMAs of an older one).
// fw[0 .. kAhead-1] hold the first weight fragments on entry; the rest are
// loaded kAhead row groups ahead of their use (pinned there for kAhead >= 2:
// prefill 2.4-3.6% faster, MoE fc2 2% faster).
struct NoExtra {
  __device__ __forceinline__ bool operator()(int) const { return false; }
};

// `extra(t)` may issue one more instruction after MFMA t (returns whether
// it did, so the scheduler keeps it at that point).
template <int TN, int TM, int kDelay, int kAhead, class LoadW, class Scale, class Extra = NoExtra>
__device__ __forceinline__ void tile_product(v4f (&acc)[TN][TM], const v8i (&fa)[TM], v8i (&fw)[kAhead + 1],
                                             LoadW load_w, Scale scale, Extra extra = Extra()) {
  constexpr int T = TN * TM;
  v4f ring[kDelay + 1];
#pragma unroll
  for (int t = 0; t < T + kDelay; ++t) {
    if (t < T) {
      const int i = t / TM, j = t % TM;
      if (j == 0 && i + kAhead < TN) {
        fw[(i + kAhead) % (kAhead + 1)] = load_w(i + kAhead);
        // Keep the read here, kAhead row groups ahead of its MFMAs: left free,
        // the scheduler sinks it to just before its first use and waits on it
        // there (one fragment register set instead of kAhead + 1).
        if constexpr (kAhead >= 2) __builtin_amdgcn_sched_barrier(0);
      }
      ring[t % (kDelay + 1)] = mfma_e4m3(fw[i % (kAhead + 1)], fa[j]);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      if (extra(t)) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // a VMEM read
    }
    if (t >= kDelay) {
      const int u = t - kDelay, i = u / TM, j = u % TM;
      const float c = scale(i, j);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(ring[u % (kDelay + 1)][r], c, acc[i][j][r]);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // its four FMAs
    }
  }
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
  // K-blocks [kb0, kb1) of the product (the panel tile only; a K-split
  // piece), and where that piece goes: FP32 partial rows of stride N at
  // `part` (nullptr: the BF16 output y).
  int kb0, kb1;
  float* part;
  // Gathered activations (grouped GEMM only): output row m reads row
  // a_rows[m] / a_div of a (of a_nrows rows); others read zeros.
  const int32_t* a_rows;
  int a_div;
  int64_t a_nrows;
  // SiLU(gate) * up tiles (grouped fc1 only): h codes [M][N/2] and their
  // 1x128 scales [M][N/256]
  uint8_t* hq;
  float* hs;
};

// A buffer offset past every record: the load returns zeros.  Buffers that
// use it hold fewer than 2^31 bytes.
constexpr int kOob = (int)0x80000000u;

// Store four consecutive n of output row m (BF16, RNE).  kHwCvt: pack with
// the conversion instruction (the dense tiles: prefill 2-2.5% faster); the
// persistent grouped tiles keep the integer form, which the compiler
// schedules there in fewer registers (175 vs 209 VGPRs; fc1 1.5-3% faster).
// Both give the same bits.
template <bool kHwCvt = true>
__device__ __forceinline__ void store4(uint16_t* __restrict__ y, int64_t N, int64_t m, int64_t n, v4f v) {
  uint16_t* dst = y + m * N + n;
  if (n + 4 <= N && (N & 3) == 0) {
    u32x2 pk;
    pk.x = kHwCvt ? bf16_pack2(v[0], v[1]) : (bf16_rne(v[0]) | (bf16_rne(v[1]) << 16));
    pk.y = kHwCvt ? bf16_pack2(v[2], v[3]) : (bf16_rne(v[2]) | (bf16_rne(v[3]) << 16));
    *reinterpret_cast<u32x2*>(dst) = pk;
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (n + r < N) dst[r] = (uint16_t)bf16_rne(v[r]);
  }
}

// Store four consecutive n of FP32 partial row m (a K-split piece).
__device__ __forceinline__ void store4_f32(float* __restrict__ p, int64_t N, int64_t m, int64_t n, v4f v) {
  float* dst = p + m * N + n;
  if (n + 4 <= N && (N & 3) == 0) {
    *reinterpret_cast<v4f*>(dst) = v;
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (n + r < N) dst[r] = v[r];
  }
}

// ---------------------------------------------------------------------------
// skinny<BN, BM>: K split across the 4 waves.  Each wave stages its own
// K-block (BN weight rows + BM activation rows, 128 bytes each) through its
// own LDS slice: coalesced 16-byte global loads (8 lanes per 128-byte row)
// into registers one K-block ahead, ds_write into the swizzled slice, and
// MFMA fragments read back with ds_read_b128.  Waves never share LDS data,
// so the K loop has no workgroup barrier.  The activation scales of four
// steps arrive in one load per 16-row group (one K-block per lane group):
// per-lane scale loads touch a cache line per row, and one per step made
// the scale loads a fifth of the kernel's vector-memory work.
//
// kAfrag: the activations are in MFMA fragment order (launch_quant_act_frag)
// and each wave loads its activation fragments straight into registers
// with the K-block's weight rows; only the weight rows go through the
// slice.  kWfrag (with kAfrag): the weights are in fragment order too and
// their fragments are loaded straight into registers as well, so the K
// loop uses no LDS at all.
// ---------------------------------------------------------------------------
template <int BN, int BM, int NW, bool kAfrag = false, bool kWfrag = false>
struct Skinny {
  static_assert(kAfrag || !kWfrag, "fragment-order weights come with fragment-order activations");
  static constexpr int TN = BN / 16, TM = BM / 16;
  static constexpr int kRows = kAfrag ? (kWfrag ? 0 : BN) : BN + BM;  // rows staged per K-block
  static constexpr int kWL = kWfrag ? 2 * TN : BN / 8;  // 16-byte weight loads per lane per K-block
  static constexpr int kLoads = kWL + (kAfrag ? 2 * TM : BM / 8);  // 16-byte loads per lane per K-block
  static constexpr int kStaged = kRows / 8;             // of which staged through the slice
  static constexpr int kSlice = kRows * kBlock;         // LDS bytes per wave
  static constexpr int kRed = NW * BN * BM * 4;         // the waves' partial tiles, FP32
  static constexpr int kLdsBytes = (NW * kSlice > kRed) ? NW * kSlice : kRed;
  static constexpr int kThreadsPerWg = 64 * NW;
  // register budget: the waves of every workgroup that fits a CU's LDS
  static constexpr int kWavesPerSimd = (NW / 4) * (2 * kLdsBytes <= 160 * 1024 ? 2 : 1);
  static_assert(NW == 4 || NW == 8, "one or two waves per SIMD");

  // swa / swb: the K-block's scales of the tile's first and (if its rows
  // straddle two) second weight scale block (wave-uniform: scalar loads)
  struct Stage {
    u32x4 v[kLoads];
    float swa, swb;
  };
  // The activation scales of four consecutive steps of a wave, rows
  // 16 j + r16: lane group g (lanes 16 g .. 16 g + 15) holds those of step
  // 4 q + g; a step takes its values from its lane group with ds_bpermute.
  struct Group {
    float sa[TM];
  };

  __device__ static __forceinline__ void run(const Tile& t, uint8_t* smem) {
    float* red = reinterpret_cast<float*>(smem);
    const int lane = threadIdx.x & 63, r16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int64_t K = t.K;
    const int KB = (int)(K / kBlock);
    const int64_t n_hi = (t.n0 + BN < t.N) ? t.n0 + BN : t.N;
    const auto wr = make_rsrc(t.w + t.n0 * K, (n_hi - t.n0) * K);
    const auto ar = make_rsrc(t.a + t.m_lo * K, (t.m_hi - t.m_lo) * K);
    const auto sr = make_rsrc(t.sa + t.m_lo * KB, (t.m_hi - t.m_lo) * KB * 4);
    // BN <= 128: the tile's rows lie in weight scale blocks nba and nbb =
    // nba or nba + 1; a 16-row n-tile lies in one of them (b_mask: in nbb)
    static_assert(BN <= kBlock, "two weight scale blocks at most");
    const int64_t nba = t.n0 / kBlock, nbb = (n_hi - 1) / kBlock;
    const float* swa_row = t.sw + nba * KB;
    const float* swb_row = t.sw + nbb * KB;
    uint32_t b_mask = 0;
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      int64_t nt = t.n0 + i * 16;
      nt = nt < t.N ? nt : t.N - 1;
      if (nt / kBlock > nba) b_mask |= 1u << i;
    }
    // staging: lane owns chunk (lane & 7) of rows (lane >> 3) + 8 q; slice
    // rows 0..BN-1 are weight rows, BN..BN+BM-1 activation rows.  The row
    // offset is part of the per-lane offset, which the buffer range check
    // covers: rows past the tile's last row read zeros, never memory.
    const int lrow = lane >> 3, lchunk = lane & 7;
    const int gvoff = lrow * (int)K + lchunk * 16;
    const int svoff = r16 * KB * 4;  // + 16 j KB 4
    const int grp = lane >> 4;
    uint8_t* slice = reinterpret_cast<uint8_t*>(red) + wave * kSlice;
    const FragLds fl(lane);

    v4f acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    auto load_stage = [&](Stage& s, int kb) {
      const int koff = kb * kBlock;
      if constexpr (kWfrag) {
        // weight fragment i, half h: 1 KB at (16 i) K + 2048 kb + 1024 h
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
          for (int h = 0; h < 2; ++h) s.v[2 * i + h] = bload16(wr, 16 * i * (int)K + h * 1024 + lane * 16, kb * 2048);
      } else {
#pragma unroll
        for (int q = 0; q < BN / 8; ++q) s.v[q] = bload16(wr, gvoff + 8 * q * (int)K, koff);
      }
      if constexpr (kAfrag) {
        // fragment j, half h of K-block kb: 1 KB at (16 j) K + 2048 kb + 1024 h
#pragma unroll
        for (int j = 0; j < TM; ++j)
#pragma unroll
          for (int h = 0; h < 2; ++h) s.v[kWL + 2 * j + h] = bload16(ar, 16 * j * (int)K + h * 1024 + lane * 16, kb * 2048);
      } else {
#pragma unroll
        for (int q = 0; q < BM / 8; ++q) s.v[BN / 8 + q] = bload16(ar, gvoff + 8 * q * (int)K, koff);
      }
      s.swa = swa_row[kb];
      s.swb = swb_row[kb];
    };
    const int kb_last = KB - 1;
    auto nxt = [&](int kb) { return kb < KB ? kb : kb_last; };
    // scales of steps 4 q .. 4 q + 3 (steps past the last re-read the last K-block)
    auto load_group = [&](Group& G, int q) {
      const int kb = nxt(wave + NW * (4 * q + grp));
#pragma unroll
      for (int j = 0; j < TM; ++j) G.sa[j] = bload_f32(sr, svoff + j * 16 * KB * 4 + kb * 4, 0);
    };
    auto store_stage = [&](const Stage& s) {
#pragma unroll
      for (int q = 0; q < kStaged; ++q) *reinterpret_cast<u32x4*>(slice + swz(lrow + 8 * q, lchunk)) = s.v[q];
    };
    auto bperm = [](float v, int addr) {
      return __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(v)));
    };
    auto compute = [&](const Stage& s, const Group& G, int step) {
      const int addr = ((((step & 3) << 4) | r16) << 2);
      float sa[TM];
#pragma unroll
      for (int j = 0; j < TM; ++j) sa[j] = bperm(G.sa[j], addr);
      v8i fa[TM];
#pragma unroll
      for (int j = 0; j < TM; ++j)
        fa[j] = kAfrag ? to_v8i(s.v[kWL + 2 * j], s.v[kWL + 2 * j + 1]) : fl(slice, BN + j * 16);
      auto wfrag = [&](int i) { return kWfrag ? to_v8i(s.v[2 * i], s.v[2 * i + 1]) : fl(slice, i * 16); };
      v8i fw[2];
      fw[0] = wfrag(0);
      tile_product<TN, TM, 4, 1>(
          acc, fa, fw, wfrag,
          [&](int i, int j) { return sa[j] * (((b_mask >> i) & 1u) ? s.swb : s.swa); });
    };

    // this wave's K-blocks: wave, wave + NW, ... (step 0, 1, ...).  Stage sX
    // holds the registers of the next K-block while the LDS slice holds the
    // current.  Prefetches past the last K-block re-read the last one
    // (clamped).
    Stage s0, s1;
    Group ga;
    int kb = wave, step = 0;
    if (kb < KB) {
      order_fence();
      load_group(ga, 0);
      load_stage(s0, kb);
      order_fence();
      store_stage(s0);
      load_stage(s1, nxt(kb + NW));
      order_fence();
    }
    // Steps step2 and step2 + 1 (K-blocks kb2 and kb2 + NW), each followed
    // by the prefetch of the K-block two steps on and the move of the next
    // one into the slice.
    auto two_steps = [&](int kb2, int step2, bool next_group) {
      compute(s0, ga, step2);           // K-block kb2 from the slice
      order_fence();
      load_stage(s0, nxt(kb2 + 2 * NW));
      order_fence();
      store_stage(s1);                  // K-block kb2 + NW into the slice
      order_fence();
      compute(s1, ga, step2 + 1);
      order_fence();
      // after the last step of a group has read its scales, the next group
      // is fetched into the same registers (a step ahead of its first use)
      if (next_group) load_group(ga, (step2 >> 2) + 1);
      load_stage(s1, nxt(kb2 + 3 * NW));
      order_fence();
      store_stage(s0);                  // K-block kb2 + 2 NW
      order_fence();
    };
    // whole groups of four steps (no branch inside: the group load has a
    // fixed place), then at most three steps of the last group
    for (; kb + 3 * NW < KB; kb += 4 * NW, step += 4) {
      two_steps(kb, step, false);
      two_steps(kb + 2 * NW, step + 2, true);
    }
    if (kb + NW < KB) {
      two_steps(kb, step, false);
      kb += 2 * NW;
      step += 2;
    }
    if (kb < KB) compute(s0, ga, step);

    // Sum the waves' partial tiles through LDS.  Each wave stores its tile
    // in fragment order (unit (i TM + j) 64 + lane = that lane's four
    // values of MFMA tile (i, j)); thread t then sums units q 256 + t over
    // the waves, so a wave's reads are 1 KB contiguous (no bank conflicts).
    __syncthreads();  // every wave is done with its staging slice
    float* mine = red + wave * (BN * BM);
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) *reinterpret_cast<v4f*>(mine + ((i * TM + j) * 64 + lane) * 4) = acc[i][j];
    __syncthreads();
    constexpr int kUnits = BN * BM / 4;
    static_assert(kUnits % kThreadsPerWg == 0, "whole rounds of units");
#pragma unroll
    for (int q = 0; q < kUnits / kThreadsPerWg; ++q) {
      const int unit = q * kThreadsPerWg + threadIdx.x;
      v4f sum = *reinterpret_cast<const v4f*>(red + 4 * unit);
#pragma unroll
      for (int w2 = 1; w2 < NW; ++w2) sum += *reinterpret_cast<const v4f*>(red + w2 * (BN * BM) + 4 * unit);
      const int ij = unit / 64, l = unit % 64;
      const int i = ij / TM, j = ij % TM;
      const int64_t m = t.m_lo + j * 16 + (l & 15);
      const int64_t n = t.n0 + i * 16 + (l >> 4) * 4;
      if (m < t.m_hi) store4(t.y, t.N, m, n, sum);
    }
  }
};

// ---------------------------------------------------------------------------
// panel<BN, BM, WGN, WGM, S>: a BN (n) x BM (m) tile per 8-wave workgroup
// (two waves per SIMD, so one wave's MFMAs fill the other's stalls), waves
// in a WGN (n) x WGM (m) grid.  Both operands of a K-block (BN weight rows
// + BM activation rows, 128 bytes each) go global -> LDS directly
// (buffer_load ... lds, 16 bytes per lane, 8 lanes per 128-byte row) into
// a ring of S stages, and so do the K-block's scales (one dword per lane),
// so no load in the K loop writes a VGPR; fragments are read with
// ds_read_b128 and scales with ds_read.
// Phase k: wait for this wave's loads of K-block k; barrier (everyone's
// data has landed, and everyone is done with the stage read in phase k-1);
// compute k while issuing the loads of K-block k + S - 1 into that stage
// between the MFMAs.  Two-stage panels instead have waves 0-3 issue all
// of those loads as one burst right after the barrier, and waves 4-7 only
// compute (split loading, in run_impl).
// ---------------------------------------------------------------------------
// kWfrag: the weight codes are in MFMA fragment order.
// kSilu (persistent grouped tiles only): the fc1 form.  The weights are
// [gate; up] of N = 2F rows and a tile computes 128 columns c0.. of
// h = SiLU(gate) * up: its weight rows are gate c0..c0+63, up c0..c0+63,
// gate c0+64..c0+127, up c0+64..c0+127, so each wave holds the gate and up
// values of the same 64 columns in the same lanes (fragments i and i + 4),
// and the epilogue stores h as E4M3 codes in 1x128 groups (the group amax
// crosses the two waves of a row through LDS).
// kSplit3: split loading (below, in run_impl) for a three-stage tile too.
template <int BN_, int BM_, int WGN, int WGM, int S, bool kWfrag = false, bool kSilu = false, bool kSplit3 = false>
struct Panel {
  static constexpr int BN = BN_, BM = BM_;
  static constexpr bool kSiluForm = kSilu;
  static_assert(WGN * WGM == 8, "eight waves");
  static constexpr int WNR = BN / WGN, WMR = BM / WGM;  // rows of a wave's tile
  static constexpr int TN = WNR / 16, TM = WMR / 16;
  static_assert(WNR % 16 == 0 && WMR % 16 == 0 && WNR <= 128, "wave tile");
  static_assert(BN % 64 == 0 && BM % 64 == 0, "each load instruction covers 8 rows of one operand, 8 waves");
  static constexpr int kRows = BN + BM;                 // rows staged per K-block
  static constexpr int kLoads = kRows / 64;             // load instructions per wave per K-block
  static constexpr int kStage = kRows * kBlock;
  // Each stage also holds that K-block's scales, staged like the operands:
  // 64 dwords per wave (activation scales of the tile's rows 0..BM-1, then
  // the tile's weight scale blocks), after the S operand stages.
  static constexpr int kScaleBytes = 8 * 64 * 4;
  static_assert(BM / 64 < 8, "a wave left over for the weight scales");
  static constexpr int kAmaxOff = S * (kStage + kScaleBytes);  // kSilu: 2 x BM row maxima
  static constexpr int kLdsBytes = kAmaxOff + (kSilu ? 2 * BM * 4 : 0);
  static_assert(S == 2 || S == 3, "stages");
  static_assert(kLdsBytes <= 160 * 1024, "LDS");
  static constexpr int kThreadsPerWg = 512;
  static constexpr int kWavesPerSimd = 2;
  // a wave's weight rows lie in one 128-row scale block when tiles start at
  // multiples of 128 and the wave's share divides 128
  static constexpr bool kOneScaleBlock = (BN % kBlock == 0) && (kBlock % WNR == 0) && !kSilu;
  static_assert(!kSilu || (BN == 256 && WGN == 2 && TN == 8 && !kWfrag), "the fc1 form's row interleave");

  __device__ static __forceinline__ void run(const Tile& t, uint8_t* lds) { run_impl<false>(t, lds); }
  // activation rows gathered through t.a_rows (grouped GEMM)
  __device__ static __forceinline__ void run_gather(const Tile& t, uint8_t* lds) { run_impl<true>(t, lds); }

  // kAfrag: the activations are in MFMA fragment order (2 KB per 16 rows x
  // K-block, launch_quant_act_frag) and stay in that order in LDS: each
  // DMA load copies one contiguous 1 KB half-unit, and a fragment is two
  // contiguous 1 KB reads (no swizzle needed, no bank conflicts).  Same
  // values in the MFMAs, same results.
  template <bool kGather, bool kAfrag = false>
  __device__ static __forceinline__ void run_impl(const Tile& t, uint8_t* lds) {
    static_assert(!(kGather && kAfrag), "gathered rows are row-major");
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int wn = wave % WGN, wm = wave / WGN;
    const int64_t K = t.K;
    const int KB = (int)(K / kBlock);  // K-blocks of a row (strides)
    // this tile's K-blocks: kb0 + 0 .. kb0 + NKB - 1
    const int kb0 = t.kb0, NKB = t.kb1 - t.kb0;
    const int64_t n_hi = (t.n0 + BN < t.N) ? t.n0 + BN : t.N;
    // weight scale blocks of this wave's rows: nb0, and nb0 + 1 for the
    // fragments in hi_mask (only when a wave's rows can straddle a block);
    // wsl0 / wsl1 are their positions among the tile's blocks nbt, nbt + 1, ..
    const int64_t NBm1 = (t.N - 1) / kBlock;
    const int64_t nbt = t.n0 / kBlock;
    const int64_t wrow0 = t.n0 + wn * WNR;
    const int64_t nb0 = ((wrow0 < t.N) ? wrow0 : t.N - 1) / kBlock;
    const int64_t nb1 = nb0 + 1 < NBm1 ? nb0 + 1 : NBm1;
    const int wsl0 = (int)(nb0 - nbt), wsl1 = (int)(nb1 - nbt);
    uint32_t hi_mask = 0;
#pragma unroll
    for (int i = 0; i < TN; ++i)
      if ((wrow0 + i * 16) / kBlock > nb0) hi_mask |= 1u << i;
    const auto wr = make_rsrc(t.w + t.n0 * K, (n_hi - t.n0) * K);
    const auto ar = kGather ? make_rsrc(t.a, t.a_nrows * K) : make_rsrc(t.a + t.m_lo * K, (t.m_hi - t.m_lo) * K);
    const int64_t am_lo = t.m_lo + wm * WMR;  // this wave's first activation row
    // Source row of output row m: itself, or the gathered row (-1: none).
    auto src_row = [&](int64_t m) -> int64_t {
      if (m >= t.m_hi) return -1;
      if (!kGather) return m - t.m_lo;  // relative to the tile's buffer
      const int32_t p = t.a_rows[m];
      const int64_t r = p >= 0 ? p / t.a_div : -1;
      return r < t.a_nrows ? r : -1;
    };
    // a ragged last tile (e.g. an expert's rows past a multiple of BM) can
    // leave whole waves without a valid activation row: they skip the MFMAs
    const bool idle = am_lo >= t.m_hi;
    // Scale staging, one buffer_load_dword ... lds per wave and K-block into
    // the wave's 64 dwords of the stage's scale area: waves w < BM/64 load
    // the activation scales of tile rows 64 w + lane, the others the
    // weight scale blocks nbt + lane.  As for the operands, rows and blocks
    // past the end sit outside the buffer range and read zeros.
    constexpr int kLoaders = 4;
    constexpr bool kSplit = !kGather && (S == 2 || kSplit3) && kRows % (8 * kLoaders) == 0 &&
                            BN % (8 * kLoaders) == 0 && BM / 64 <= kLoaders;
    // Split loading: waves 0-3 issue the loads, or waves 4-7 in a tile whose
    // last row of waves has no valid activation row (a ragged last tile),
    // so that the waves that skip the MFMAs are the ones that load.
    const bool swap = kSplit && t.m_lo + (WGM - 1) * WMR >= t.m_hi;
    const bool loader = swap ? wave >= kLoaders : wave < kLoaders;
    const int slot = kSplit ? (wave & (kLoaders - 1)) : wave;  // a loading wave's rows and scale slot
    const bool act_scales = slot < BM / 64;
    const auto scr = act_scales ? (kGather ? make_rsrc(t.sa, t.a_nrows * KB * 4)
                                           : make_rsrc(t.sa + t.m_lo * KB, (t.m_hi - t.m_lo) * KB * 4))
                                : make_rsrc(t.sw + nbt * KB, (NBm1 - nbt + 1) * KB * 4);
    int scvoff = lane * KB * 4;
    if (act_scales) {
      const int64_t r = src_row(t.m_lo + 64 * slot + lane);
      scvoff = kGather ? (r >= 0 ? (int)(r * KB * 4) : kOob) : (64 * slot + lane) * KB * 4;
    }

    // DMA staging: load q of wave w fills stage rows R0..R0+7 with
    // R0 = 8 (8 q + w); lane l writes LDS row R0 + l/8 at physical chunk
    // l%8, so it fetches logical chunk (l%8) ^ (l/8) (the XOR swizzle).
    // The row offset is part of the per-lane offset, which the buffer range
    // check covers: rows past the tile's last row read zeros, never memory.
    const int chunk_off = ((lane & 7) ^ (lane >> 3)) << 4;
    const int dvoff = (lane >> 3) * (int)K + chunk_off;
    // gathered activations: the offset of this lane's row in each A load
    int aoff[kGather ? BM / 64 : 1];
    if constexpr (kGather) {
#pragma unroll
      for (int qa = 0; qa < BM / 64; ++qa) {
        const int64_t r = src_row(t.m_lo + 8 * (8 * (BN / 64 + qa) + wave) - BN + (lane >> 3));
        aoff[qa] = r >= 0 ? (int)(r * K) + chunk_off : kOob;
      }
    }
    const FragLds fl(lane);

    v4f acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    auto dma_scales = [&](int kb, int stage) {
      auto* dst = (__attribute__((address_space(3))) void*)(lds + S * kStage + stage * kScaleBytes + wave * 256);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(scr, dst, 4, scvoff, (kb0 + kb) * 4, 0, 0);
    };
    auto dma_q = [&](int q, int kb, uint8_t* buf) {
      const int koff = (kb0 + kb) * kBlock;
      const int r0 = 8 * (8 * q + wave);  // stage row of this wave's load q
      auto* dst = (__attribute__((address_space(3))) void*)(buf + r0 * kBlock);
      if (q < BN / 64 && kWfrag)  // stage rows 0..BN-1: half r0 / 8 % 2 of the weight unit of rows n0 + r0 / 16 16
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, dst, 16, (r0 >> 4) * 16 * (int)K + (r0 & 8) * 128 + lane * 16,
                                                 (kb0 + kb) * 16 * kBlock, 0, 0);
      else if (q < BN / 64)  // stage rows 0..BN-1: weight rows n0 + r0 ..
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, dst, 16, dvoff + r0 * (int)K, koff, 0, 0);
      else if (kGather)  // stage rows BN..: the gathered activation rows
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, dst, 16, aoff[kGather ? q - BN / 64 : 0], koff, 0, 0);
      else if (kAfrag)  // stage rows BN..: half (r0 - BN) / 8 % 2 of the unit of rows m_lo + (r0 - BN) / 16 16
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, dst, 16,
                                                 ((r0 - BN) >> 4) * 16 * (int)K + ((r0 - BN) & 8) * 128 + lane * 16,
                                                 (kb0 + kb) * 16 * kBlock, 0, 0);
      else              // stage rows BN..: activation rows m_lo + r0 - BN ..
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, dst, 16, dvoff + (r0 - BN) * (int)K, koff, 0, 0);
    };
    // all loads of one K-block: the operand rows, then the scales
    auto dma_kblock = [&](int kb, int stage) {
#pragma unroll
      for (int q = 0; q < kLoads; ++q) dma_q(q, kb, lds + stage * kStage);
      dma_scales(kb, stage);
    };
    // Split loading (the two-stage panels, and kSplit3 tiles): the waves of
    // a SIMD do not progress together.  The first-dispatched wave of each
    // SIMD (waves 0-3) takes the MFMA pipe first and finishes its phase ~30%
    // sooner, then waits at the barrier while the second one (waves 4-7)
    // finishes alone.  So waves 0-3 issue all of a K-block's loads, as one
    // burst right after the barrier (operand rows 8 (kLoaders q + w) .., the
    // activation scales of their 64-row slots, and one of them the weight
    // scales), and waves 4-7 only compute: prefill 4.6-5.3% faster, the same
    // bits.  With three stages the 192 x 128 decode panel gains 4-8%
    // (M = 192, 256); the 128 x 256 one gains only where waves 4-7 have no
    // rows (M <= 128: they load, waves 0-3 compute) and loses 5-9% at
    // M = 176-208, K = 2048, so it runs split only there.
    constexpr int kLoadsL = kRows / (8 * kLoaders);  // operand loads per loading wave and K-block
    constexpr int kWScaleWave = BM / 64 < kLoaders ? BM / 64 : 0;  // the loader that fetches the weight scales
    const auto scr_w = make_rsrc(t.sw + nbt * KB, (NBm1 - nbt + 1) * KB * 4);
    auto dma_q_split = [&](int q, int kb, uint8_t* buf) {
      const int koff = (kb0 + kb) * kBlock;
      const int r0 = 8 * (kLoaders * q + slot);
      auto* dst = (__attribute__((address_space(3))) void*)(buf + r0 * kBlock);
      if (q < BN / (8 * kLoaders) && kWfrag)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, dst, 16, (r0 >> 4) * 16 * (int)K + (r0 & 8) * 128 + lane * 16,
                                                 (kb0 + kb) * 16 * kBlock, 0, 0);
      else if (q < BN / (8 * kLoaders))
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, dst, 16, dvoff + r0 * (int)K, koff, 0, 0);
      else if (kAfrag)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, dst, 16,
                                                 ((r0 - BN) >> 4) * 16 * (int)K + ((r0 - BN) & 8) * 128 + lane * 16,
                                                 (kb0 + kb) * 16 * kBlock, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, dst, 16, dvoff + (r0 - BN) * (int)K, koff, 0, 0);
    };
    auto dma_scales_split = [&](int kb, int stage) {
      uint8_t* area = lds + S * kStage + stage * kScaleBytes;
      if (slot < BM / 64)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(scr, (__attribute__((address_space(3))) void*)(area + slot * 256), 4,
                                                 scvoff, (kb0 + kb) * 4, 0, 0);
      if (slot == kWScaleWave)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(scr_w, (__attribute__((address_space(3))) void*)(area + (BM / 64) * 256),
                                                 4, lane * KB * 4, (kb0 + kb) * 4, 0, 0);
    };
    // three stages: every loading wave issues two scale loads (its own slot:
    // activation scales below BM / 64, weight scales above; and a copy of
    // the weight scales into slot 4 + w), so all have kLoadsL + 2 loads per
    // K-block and one vmcnt immediate fits them
    auto dma_scales_split3 = [&](int kb, int stage) {
      uint8_t* area = lds + S * kStage + stage * kScaleBytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(scr, (__attribute__((address_space(3))) void*)(area + slot * 256), 4,
                                               scvoff, (kb0 + kb) * 4, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(scr_w, (__attribute__((address_space(3))) void*)(area + (kLoaders + slot) * 256),
                                               4, lane * KB * 4, (kb0 + kb) * 4, 0, 0);
    };
    auto dma_kblock_split = [&](int kb, int stage) {
      if (loader) {
#pragma unroll
        for (int q = 0; q < kLoadsL; ++q) dma_q_split(q, kb, lds + stage * kStage);
        if constexpr (S == 2)
          dma_scales_split(kb, stage);
        else
          dma_scales_split3(kb, stage);
      }
    };
    constexpr int kAhead = 2;  // weight fragments are read two row groups ahead
    auto load_w = [&](const uint8_t* buf, int i) -> v8i {
      if constexpr (kWfrag) {  // the 2 KB unit of weight rows wn WNR + 16 i
        const uint8_t* p = buf + (wn * WNR + i * 16) * kBlock + lane * 16;
        return to_v8i(*reinterpret_cast<const u32x4*>(p), *reinterpret_cast<const u32x4*>(p + 1024));
      } else {
        return fl(buf, wn * WNR + i * 16);
      }
    };
    auto load_a = [&](const uint8_t* buf, int j) -> v8i {
      if constexpr (kAfrag) {  // the 2 KB unit of rows wm WMR + 16 j
        const uint8_t* p = buf + (BN + wm * WMR + j * 16) * kBlock + lane * 16;
        return to_v8i(*reinterpret_cast<const u32x4*>(p), *reinterpret_cast<const u32x4*>(p + 1024));
      } else {
        return fl(buf, BN + wm * WMR + j * 16);
      }
    };
    // The first fragments of a phase, read right after its barrier; the
    // first MFMA's two operands go first so that it waits for them only.
    auto first_frags = [&](v8i (&fa)[TM], v8i (&fw)[kAhead + 1], const uint8_t* buf) {
      fw[0] = load_w(buf, 0);
      fa[0] = load_a(buf, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 1; j < TM; ++j) fa[j] = load_a(buf, j);
#pragma unroll
      for (int p = 1; p < kAhead && p < TN; ++p) fw[p] = load_w(buf, p);
    };
    // One phase: the product of the K-block in stage `cur`, with the loads
    // of K-block `kb` into stage `fill` issued after every second MFMA
    // (after every MFMA when there are few), so that the L2 and LDS-write
    // traffic does not arrive as one burst right after the barrier.  The
    // scales come from the stage's scale area; their products are formed
    // while the first MFMAs run.
    constexpr int kT = TN * TM;
    constexpr int kPhaseLoads = kLoads + 1;
    constexpr int kEvery = (kT >= 2 * kPhaseLoads) ? 2 : 1;
    static_assert(kT >= kPhaseLoads, "enough MFMAs to carry the loads");
    auto phase = [&](int cur, int kb, int fill) {
      const uint8_t* buf = lds + cur * kStage;
      v8i fa[TM], fw[kAhead + 1];
      first_frags(fa, fw, buf);
      const float* scl = reinterpret_cast<const float*>(lds + S * kStage + cur * kScaleBytes);
      const float sw0 = scl[BM + wsl0];
      const float sw1 = kOneScaleBlock ? sw0 : scl[BM + wsl1];
      float c0[TM], c1[TM];
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const float sa = scl[wm * WMR + j * 16 + r16];
        c0[j] = sa * sw0;
        c1[j] = kOneScaleBlock ? c0[j] : sa * sw1;
      }
      tile_product<TN, TM, 2, kAhead>(
          acc, fa, fw, [&](int i) { return load_w(buf, i); },
          [&](int i, int j) { return (kOneScaleBlock || !((hi_mask >> i) & 1u)) ? c0[j] : c1[j]; },
          [&](int tt) {
            if constexpr (kSplit) {
              return false;
            } else {
              if (tt % kEvery != 0 || tt / kEvery >= kPhaseLoads) return false;
              const int q = tt / kEvery;
              if (q < kLoads)
                dma_q(q, kb, lds + fill * kStage);
              else
                dma_scales(kb, fill);
              return true;
            }
          });
    };
    // The compiler does not track LDS writes by buffer_load ... lds: wait
    // for them explicitly before the barrier that publishes the stage.  With
    // three stages the loads of the next K-block may stay in flight.
    auto wait_stage = [&]() {
      // the loads of K-block k + 1 have (S - 2) * kPhaseLoads loads issued after them
      if constexpr (S == 2) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      } else if constexpr (kSplit) {
        if (loader)
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"((S - 2) * (kLoadsL + 2)) : "memory");
        else
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((S - 2) * kPhaseLoads) : "memory");
      }
    };
    // The workgroup barrier of a phase.  Not __syncthreads(): its fence
    // would wait for every load in flight (vmcnt(0)), including the later
    // K-blocks' prefetches that the ring keeps in flight on purpose.  The
    // LDS writes this barrier publishes were waited for by wait_stage();
    // the LDS reads of the previous phase are waited for here, so no wave
    // refills a stage that another is still reading.
    auto barrier = [&]() {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      order_fence();
    };
    auto wait_all = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

    const int kb_last = NKB - 1;
    auto nxt = [&](int kb) { return kb < NKB ? kb : kb_last; };  // clamped prefetch
    if (NKB > 0) {
#pragma unroll
      for (int st = 0; st < S - 1; ++st) {
        if constexpr (kSplit)
          dma_kblock_split(nxt(st), st);
        else
          dma_kblock(nxt(st), st);
      }
    }
    // Loads past the last K-block re-load it into a stage nobody reads
    // again, keeping the loop body free of branches.
    int cur = 0;  // stage of K-block k
    for (int k = 0; k < NKB; ++k) {
      wait_stage();
      barrier();  // stage cur holds K-block k; stage cur - 1 is free
      const int fill = (cur == 0) ? S - 1 : cur - 1;
      if constexpr (kSplit) {
        dma_kblock_split(nxt(k + S - 1), fill);  // waves 0..kLoaders-1 only
        order_fence();
        if (!idle) phase(cur, nxt(k + S - 1), fill);
      } else {
        if (idle) {  // no valid activation row: only this wave's share of the loads
          dma_kblock(nxt(k + S - 1), fill);
        } else {
          phase(cur, nxt(k + S - 1), fill);
        }
      }
      order_fence();
      cur = (cur + 1 == S) ? 0 : cur + 1;
    }
    wait_all();  // no LDS write may be in flight when the workgroup ends

#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int64_t m = t.m_lo + wm * WMR + j * 16 + r16;
      if (m >= t.m_hi) continue;
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        const int64_t n = t.n0 + wn * WNR + i * 16 + g * 4;
        if (t.part != nullptr)
          store4_f32(t.part, t.N, m, n, acc[i][j]);
        else
          store4(t.y, t.N, m, n, acc[i][j]);
      }
    }
  }

  // Several tiles per workgroup: tile r = 0 .. ntiles-1 comes from
  // tile_at(r), and the K-blocks of consecutive tiles stream through the
  // one ring of S stages, so the first loads of tile r + 1 are in flight
  // while tile r finishes and stores its outputs (no per-tile pipeline
  // fill).  The loads follow the tile of the step being prefetched ("load
  // side"), the MFMAs, scales and stores the tile being computed ("compute
  // side").  Prefetches past the last step re-load the last K-block into a
  // stage nobody reads again.  run_impl stays a loop of its own: routing
  // the one-tile case through this one (4-8 more VGPRs, stores before the
  // final wait) made the prefill tiles 3-7% slower.
  template <bool kGather, class TileAt>
  __device__ static __forceinline__ void run_persistent(int ntiles, TileAt tile_at, uint8_t* lds) {
    static_assert(!kWfrag, "the grouped tiles read row-major weights");
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int wn = wave % WGN, wm = wave / WGN;
    const bool act_scales = wave < BM / 64;
    const int chunk_off = ((lane & 7) ^ (lane >> 3)) << 4;
    const FragLds fl(lane);

    // ---- load side: operand and scale buffers of the tile being prefetched
    Tile lt = tile_at(0);
    const int64_t K = lt.K;
    const int KB = (int)(K / kBlock);
    const int dvoff = (lane >> 3) * (int)K + chunk_off;
    __amdgpu_buffer_rsrc_t wr, ar, scr;
    int scvoff = 0;
    int aoff[kGather ? BM / 64 : 1];
    // Split loading (as in run_impl): waves 0..3 issue every load of a
    // K-block, as one burst after the barrier, in rounds of 32 rows (wave
    // w: rows 32 q + 8 w ..); the other waves only compute.  Expert fc1
    // 7.6% and fc2 3.6% faster, the same bits; not the SiLU*up form, whose
    // epilogue work on the loading waves made it 1.5% slower.
    constexpr int kLoaders = 4;
    constexpr bool kPSplit =
        S == 3 && !kSilu && (BN + BM) % (8 * kLoaders) == 0 && BN % 64 == 0 && BM / 64 < kLoaders;
    constexpr int kLoadsL = (BN + BM) / (8 * kLoaders);
    const bool loader = wave < kLoaders;
    int aoff_s[kGather ? BM / (8 * kLoaders) : 1];
    auto src_row = [&](const Tile& t, int64_t m) -> int64_t {
      if (m >= t.m_hi) return -1;
      if (!kGather) return m - t.m_lo;
      const int32_t pr = t.a_rows[m];
      const int64_t r = pr >= 0 ? pr / t.a_div : -1;
      return r < t.a_nrows ? r : -1;
    };
    auto setup_load = [&](const Tile& t) {
      const int64_t n_hi = (t.n0 + BN < t.N) ? t.n0 + BN : t.N;
      const int64_t NBm1 = (t.N - 1) / kBlock, nbt = t.n0 / kBlock;
      if constexpr (kSilu) {
        // gate rows n0 .. n0 + 127 and up rows F + n0 .. F + n0 + 127 (F = N / 2,
        // n0 a multiple of 128); weight scale blocks n0 / 128 (slot 0) and
        // (F + n0) / 128 (slot 1)
        const int64_t F = t.N / 2;
        wr = make_rsrc(t.w + t.n0 * K, (F + kBlock) * K);
        scr = act_scales ? make_rsrc(t.sa, t.a_nrows * KB * 4)
                         : make_rsrc(t.sw + nbt * KB, (F / kBlock + 1) * KB * 4);
        scvoff = lane == 0 ? 0 : (lane == 1 ? (int)(F / kBlock) * KB * 4 : kOob);
      } else {
        wr = make_rsrc(t.w + t.n0 * K, (n_hi - t.n0) * K);
        scr = act_scales ? (kGather ? make_rsrc(t.sa, t.a_nrows * KB * 4)
                                    : make_rsrc(t.sa + t.m_lo * KB, (t.m_hi - t.m_lo) * KB * 4))
                         : make_rsrc(t.sw + nbt * KB, (NBm1 - nbt + 1) * KB * 4);
        scvoff = lane * KB * 4;
      }
      ar = kGather ? make_rsrc(t.a, t.a_nrows * K) : make_rsrc(t.a + t.m_lo * K, (t.m_hi - t.m_lo) * K);
      if (act_scales) {
        const int64_t r = src_row(t, t.m_lo + 64 * wave + lane);
        scvoff = kGather ? (r >= 0 ? (int)(r * KB * 4) : kOob) : (64 * wave + lane) * KB * 4;
      }
      if constexpr (kGather) {
#pragma unroll
        for (int qa = 0; qa < BM / 64; ++qa) {
          const int64_t r = src_row(t, t.m_lo + 8 * (8 * (BN / 64 + qa) + wave) - BN + (lane >> 3));
          aoff[qa] = r >= 0 ? (int)(r * K) + chunk_off : kOob;
        }
        if constexpr (kPSplit) {
#pragma unroll
          for (int qa = 0; qa < BM / (8 * kLoaders); ++qa) {
            const int64_t r = src_row(t, t.m_lo + 32 * qa + 8 * (wave & (kLoaders - 1)) + (lane >> 3));
            aoff_s[qa] = r >= 0 ? (int)(r * K) + chunk_off : kOob;
          }
        }
      }
    };
    setup_load(lt);
    int lt_r = 0, lt_kb = 0;
    // the next step to prefetch (clamped to the last K-block of the last tile)
    auto advance_load = [&]() {
      if (lt_kb + 1 < KB) {
        ++lt_kb;
      } else if (lt_r + 1 < ntiles) {
        ++lt_r;
        lt_kb = 0;
        lt = tile_at(lt_r);
        setup_load(lt);
      }
    };

    // ---- compute side: scales, MFMAs and stores of the tile being computed
    Tile ct = lt;
    int wsl0 = 0, wsl1 = 0;
    uint32_t hi_mask = 0;
    bool idle = false;
    auto setup_compute = [&](const Tile& t) {
      if constexpr (kSilu) {  // fragments 0..3 gate (scale slot 0), 4..7 up (slot 1)
        wsl0 = 0;
        wsl1 = 1;
        hi_mask = 0xF0u;
      } else {
        const int64_t NBm1 = (t.N - 1) / kBlock, nbt = t.n0 / kBlock;
        const int64_t wrow0 = t.n0 + wn * WNR;
        const int64_t nb0 = ((wrow0 < t.N) ? wrow0 : t.N - 1) / kBlock;
        const int64_t nb1 = nb0 + 1 < NBm1 ? nb0 + 1 : NBm1;
        wsl0 = (int)(nb0 - nbt);
        wsl1 = (int)(nb1 - nbt);
        hi_mask = 0;
#pragma unroll
        for (int i = 0; i < TN; ++i)
          if ((wrow0 + i * 16) / kBlock > nb0) hi_mask |= 1u << i;
      }
      idle = t.m_lo + wm * WMR >= t.m_hi;
    };
    setup_compute(ct);
    int ct_r = 0, ct_kb = 0;

    v4f acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    auto dma_scales = [&](int kb, int stage) {
      auto* dst = (__attribute__((address_space(3))) void*)(lds + S * kStage + stage * kScaleBytes + wave * 256);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(scr, dst, 4, scvoff, kb * 4, 0, 0);
    };
    // kSilu: load q < 4 fills tile rows 64 q .. 64 q + 63 with gate (q even)
    // or up (q odd) rows 64 (q / 2) .. of the tile's 128 columns
    const int fup = kSilu ? (int)(lt.N / 2) * (int)K : 0;
    auto dma_q = [&](int q, int kb, uint8_t* buf) {
      const int koff = kb * kBlock;
      const int r0 = 8 * (8 * q + wave);
      auto* dst = (__attribute__((address_space(3))) void*)(buf + r0 * kBlock);
      if (q < BN / 64 && kSilu)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, dst, 16,
                                                 dvoff + ((q & 1) ? fup : 0) + ((q >> 1) * 64 + 8 * wave) * (int)K,
                                                 koff, 0, 0);
      else if (q < BN / 64)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, dst, 16, dvoff + r0 * (int)K, koff, 0, 0);
      else if (kGather)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, dst, 16, aoff[kGather ? q - BN / 64 : 0], koff, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, dst, 16, dvoff + (r0 - BN) * (int)K, koff, 0, 0);
    };
    auto dma_kblock = [&](int kb, int stage) {
#pragma unroll
      for (int q = 0; q < kLoads; ++q) dma_q(q, kb, lds + stage * kStage);
      dma_scales(kb, stage);
    };
    // round q of loading wave w: tile rows r0 = 32 q + 8 w ..; for kSilu the
    // 64-row piece r0 / 64 is gate (even) or up (odd) rows 64 (piece / 2) ..
    auto dma_q_split = [&](int q, int kb, uint8_t* buf) {
      const int koff = kb * kBlock;
      const int w4 = wave & (kLoaders - 1);
      const int r0 = 8 * (kLoaders * q + w4);
      auto* dst = (__attribute__((address_space(3))) void*)(buf + r0 * kBlock);
      constexpr int kWR = BN / (8 * kLoaders);  // weight rounds
      if (q < kWR && kSilu) {
        const int piece = q >> 1;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            wr, dst, 16, dvoff + ((piece & 1) ? fup : 0) + ((piece >> 1) * 64 + 32 * (q & 1) + 8 * w4) * (int)K, koff,
            0, 0);
      } else if (q < kWR) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, dst, 16, dvoff + r0 * (int)K, koff, 0, 0);
      } else if (kGather) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, dst, 16, aoff_s[kGather ? q - kWR : 0], koff, 0, 0);
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, dst, 16, dvoff + (r0 - BN) * (int)K, koff, 0, 0);
      }
    };
    // loading waves: their rounds, then one scale load each (activation
    // scales for waves below BM / 64, weight scales for the others: the
    // same count on every loading wave, so one vmcnt immediate fits all)
    auto dma_kblock_split = [&](int kb, int stage) {
      if (loader) {
#pragma unroll
        for (int q = 0; q < kLoadsL; ++q) dma_q_split(q, kb, lds + stage * kStage);
        dma_scales(kb, stage);
      }
    };
    constexpr int kAhead = 2;
    auto load_w = [&](const uint8_t* buf, int i) { return fl(buf, wn * WNR + i * 16); };
    auto first_frags = [&](v8i (&fa)[TM], v8i (&fw)[kAhead + 1], const uint8_t* buf) {
      fw[0] = load_w(buf, 0);
      fa[0] = fl(buf, BN + wm * WMR);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 1; j < TM; ++j) fa[j] = fl(buf, BN + wm * WMR + j * 16);
#pragma unroll
      for (int pp = 1; pp < kAhead && pp < TN; ++pp) fw[pp] = load_w(buf, pp);
    };
    constexpr int kT = TN * TM;
    constexpr int kPhaseLoads = kLoads + 1;
    constexpr int kEvery = (kT >= 2 * kPhaseLoads) ? 2 : 1;
    static_assert(kT >= kPhaseLoads, "enough MFMAs to carry the loads");
    auto phase = [&](int cur, int kb, int fill) {
      const uint8_t* buf = lds + cur * kStage;
      v8i fa[TM], fw[kAhead + 1];
      first_frags(fa, fw, buf);
      const float* scl = reinterpret_cast<const float*>(lds + S * kStage + cur * kScaleBytes);
      const float sw0 = scl[BM + wsl0];
      const float sw1 = kOneScaleBlock ? sw0 : scl[BM + wsl1];
      float c0[TM], c1[TM];
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const float sa = scl[wm * WMR + j * 16 + r16];
        c0[j] = sa * sw0;
        c1[j] = kOneScaleBlock ? c0[j] : sa * sw1;
      }
      tile_product<TN, TM, 2, kAhead>(
          acc, fa, fw, [&](int i) { return load_w(buf, i); },
          [&](int i, int j) { return (kOneScaleBlock || !((hi_mask >> i) & 1u)) ? c0[j] : c1[j]; },
          [&](int tt) {
            if constexpr (kPSplit) {
              return false;
            } else {
              if (tt % kEvery != 0 || tt / kEvery >= kPhaseLoads) return false;
              const int q = tt / kEvery;
              if (q < kLoads)
                dma_q(q, kb, lds + fill * kStage);
              else
                dma_scales(kb, fill);
              return true;
            }
          });
    };
    // The same waits and barrier as run_impl.  After a tile's stores the
    // vmcnt wait also covers them (stores count in vmcnt): it waits longer
    // then, never too little.
    auto wait_stage = [&]() {
      if constexpr (S == 2) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      } else if constexpr (kPSplit) {
        if (loader)
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"((S - 2) * (kLoadsL + 1)) : "memory");
        else
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((S - 2) * kPhaseLoads) : "memory");
      }
    };
    auto barrier = [&]() {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      order_fence();
    };

#pragma unroll
    for (int st = 0; st < S - 1; ++st) {
      if constexpr (kPSplit)
        dma_kblock_split(lt_kb, st);
      else
        dma_kblock(lt_kb, st);
      advance_load();
    }
    // kSilu: lane (r16, g) holds, for rows wm WMR + 16 j + r16, the gate and
    // up accumulators of columns 64 wn + 16 i + 4 g + r (fragments i and
    // i + 4, i, r < 4).  Each is rounded to BF16 (the fc1 output the
    // unfused chain would store), h = SiLU(gate) * up is rounded to BF16
    // exactly (silu_mul_bf16's result: its float32 path for all 32 values,
    // then its float64 decision for the values that path leaves open), and
    // the row's 1x128 group (the columns of both waves wn = 0, 1) is
    // quantized: amax over the wave's lanes by shuffles, across the two
    // waves through LDS, s = fl32(amax / 448), codes E4M3(fl32(h / s)).
    auto silu_epilogue = [&](const Tile& t) {
      const int64_t F = t.N / 2;
      static_assert(4 * TM * 4 <= 32, "one deferral bit per value");
      uint32_t hb[4][TM][4];
      uint32_t mx[TM];
      // The float32 path for every value first, with no branch; values it
      // cannot settle are marked in `defer` (bit (i TM + j) 4 + r).
      uint32_t defer = 0;
#pragma unroll
      for (int j = 0; j < TM; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float gv = __uint_as_float(bf16_rne(acc[i][j][r]) << 16);
            const float uv = __uint_as_float(bf16_rne(acc[i + 4][j][r]) << 16);
            bool ok;
            hb[i][j][r] = silu_mul_bf16_fast(gv, uv, &ok);
            defer |= ok ? 0u : 1u << ((i * TM + j) * 4 + r);
          }
      // Then the float64 decisions: each lane hands its lowest deferred
      // value to one call per round (values picked and written back by
      // compile-time index), so a wave makes as many calls as its lane with
      // the most deferred values has (usually one), not one per position.
      while (__ballot(defer != 0u) != 0ull) {
        const int sel = defer != 0u ? __builtin_ctz(defer) : -1;
        float ga = 0.0f, ua = 0.0f;
#pragma unroll
        for (int j = 0; j < TM; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (sel == (i * TM + j) * 4 + r) {
                ga = acc[i][j][r];
                ua = acc[i + 4][j][r];
              }
        uint32_t hr = 0;
        if (defer != 0u)
          hr = silu_mul_bf16_f64(__uint_as_float(bf16_rne(ga) << 16), __uint_as_float(bf16_rne(ua) << 16));
#pragma unroll
        for (int j = 0; j < TM; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (sel == (i * TM + j) * 4 + r) hb[i][j][r] = hr;
        defer &= defer - 1u;
      }
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        mx[j] = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t ah = hb[i][j][r] & 0x7fffu;
            mx[j] = mx[j] > ah ? mx[j] : ah;
          }
        mx[j] = max(mx[j], (uint32_t)__shfl_xor((int)mx[j], 16));
        mx[j] = max(mx[j], (uint32_t)__shfl_xor((int)mx[j], 32));
      }
      uint32_t* am = reinterpret_cast<uint32_t*>(lds + kAmaxOff);
      if (g == 0) {
#pragma unroll
        for (int j = 0; j < TM; ++j) am[wn * BM + wm * WMR + j * 16 + r16] = mx[j];
      }
      barrier();
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const uint32_t other = am[(1 - wn) * BM + wm * WMR + j * 16 + r16];
        const float sc = scale_from_amax_bits(mx[j] > other ? mx[j] : other);
        const int64_t m = t.m_lo + wm * WMR + j * 16 + r16;
        if (m >= t.m_hi) continue;
        const Divisor d(sc != 0.0f ? sc : 1.0f);
        uint8_t* dst = t.hq + m * F + t.n0 + 64 * wn + 4 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t code;
          if (sc == 0.0f) {  // the sign of each input zero
            code = ((hb[i][j][0] >> 8) & 0x80u) | (hb[i][j][1] & 0x8000u) | ((hb[i][j][2] << 8) & 0x800000u) |
                   ((hb[i][j][3] << 16) & 0x80000000u);
          } else {
            float q[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float x = __uint_as_float(hb[i][j][r] << 16);
              q[r] = d.fast ? d.quotient_fast(x) : d.quotient_ieee(x);
            }
            code = pack4_e4m3(q[0], q[1], q[2], q[3]);
          }
          *reinterpret_cast<uint32_t*>(dst + 16 * i) = code;
        }
        if (wn == 0 && g == 0) t.hs[m * (F / kBlock) + t.n0 / kBlock] = sc;
      }
    };
    const int64_t steps = (int64_t)ntiles * KB;
    int cur = 0;
    for (int64_t step = 0; step < steps; ++step) {
      wait_stage();
      barrier();
      const int fill = (cur == 0) ? S - 1 : cur - 1;
      if constexpr (kPSplit) {
        dma_kblock_split(lt_kb, fill);
        order_fence();
        if (!idle) phase(cur, lt_kb, fill);
      } else {
        if (idle) {
          dma_kblock(lt_kb, fill);
        } else {
          phase(cur, lt_kb, fill);
        }
      }
      order_fence();
      advance_load();
      cur = (cur + 1 == S) ? 0 : cur + 1;
      if (++ct_kb == KB) {  // the compute tile's last K-block: store it, start the next
        if constexpr (kSilu) {
          silu_epilogue(ct);
        } else {
#pragma unroll
          for (int j = 0; j < TM; ++j) {
            const int64_t m = ct.m_lo + wm * WMR + j * 16 + r16;
            if (m >= ct.m_hi) continue;
#pragma unroll
            for (int i = 0; i < TN; ++i) store4<false>(ct.y, ct.N, m, ct.n0 + wn * WNR + i * 16 + g * 4, acc[i][j]);
          }
        }
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
          for (int j = 0; j < TM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
        ct_kb = 0;
        if (++ct_r < ntiles) {
          ct = tile_at(ct_r);
          setup_compute(ct);
        }
        order_fence();
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no LDS write may be in flight when the workgroup ends
  }
};

// A panel tile reading fragment-order activations through its LDS ring.
template <class P>
struct PanelFragA {
  static constexpr int BN = P::BN, BM = P::BM;
  static constexpr int kLdsBytes = P::kLdsBytes;
  static constexpr int kThreadsPerWg = P::kThreadsPerWg;
  static constexpr int kWavesPerSimd = P::kWavesPerSimd;
  __device__ static __forceinline__ void run(const Tile& t, uint8_t* lds) {
    P::template run_impl<false, true>(t, lds);
  }
};


using Wide = Panel<256, 256, 2, 4, 2>;
using DecodePanel = Panel<128, 256, 2, 4, 3>;
// The decode panel at M <= 128 (one tile of rows, waves 4-7 without rows):
// split loading, waves 4-7 load and waves 0-3 compute (Qwen3-8B gate_up
// shape N = 24576, K = 4096 at M = 128: 36.8 -> 35.7 us).
template <bool kW = false>
using DecodePanelSplit = Panel<128, 256, 2, 4, 3, kW, false, true>;
// Three stages of 256 weight rows: two K-blocks of weights (64 KB) in flight
// per workgroup instead of the wide tile's one, for weights streamed from
// HBM once (MoE experts, whose weights no other tile reads).
using Deep = Panel<256, 128, 2, 4, 3>;
// Decode with exactly one round of tiles: at M = 256 and N = 24576 the
// 192 x 128 panel gives 256 tiles (one per CU), where the 128 x 256 panel
// leaves 64 CUs idle (48.4 vs 52.6 us on the Qwen3-8B gate_up at M = 256).
using Panel192 = Panel<192, 128, 2, 4, 3, false, false, true>;

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

template <class Kern>
constexpr int threads_of() {
  return Kern::kThreadsPerWg;
}

template <class Kern, int BN, int BM>
__global__ __launch_bounds__(threads_of<Kern>(), Kern::kWavesPerSimd) void gemm_dense_kernel(const uint8_t* __restrict__ a,
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
  t.a_rows = nullptr; t.a_div = 1; t.a_nrows = 0;
  t.kb0 = 0; t.kb1 = (int)(K / kBlock); t.part = nullptr;
  Kern::run(t, smem);
}

// K split: workgroup L takes piece s = L' % S of tile L' / S (L' the
// XCD-aware rank), the K-blocks [s KB / S, (s + 1) KB / S), and stores its
// FP32 partial tile to part + s * M * N; splitk_reduce_kernel sums them.
template <class Kern, int BN, int BM>
__global__ __launch_bounds__(threads_of<Kern>(), Kern::kWavesPerSimd) void gemm_splitk_kernel(
    const uint8_t* __restrict__ a, const float* __restrict__ sa, const uint8_t* __restrict__ w,
    const float* __restrict__ sw, float* __restrict__ part, int64_t M, int64_t N, int64_t K, int64_t tiles_m,
    int64_t tiles_n, int S) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int64_t L = xcd_linear(blockIdx.x, tiles_m * tiles_n * S);
  const int piece = (int)(L % S);
  int64_t tm, tn;
  tile_of(L / S, tiles_m, tiles_n, &tm, &tn);
  const int KB = (int)(K / kBlock);
  Tile t;
  t.a = a; t.sa = sa; t.w = w; t.sw = sw; t.y = nullptr;
  t.m_lo = tm * BM;
  t.m_hi = (t.m_lo + BM < M) ? t.m_lo + BM : M;
  t.n0 = tn * BN;
  t.N = N; t.K = K;
  t.a_rows = nullptr; t.a_div = 1; t.a_nrows = 0;
  t.kb0 = (int)((int64_t)piece * KB / S);
  t.kb1 = (int)((int64_t)(piece + 1) * KB / S);
  t.part = part + (int64_t)piece * M * N;
  Kern::run(t, smem);
}

// y = BF16_RNE(p_0 + p_1 + ... + p_{S-1}), summed in that order in FP32
// (deterministic: the pieces and the order do not depend on timing).  One
// thread per four consecutive outputs.
constexpr int kReduceThreads = 256;
__global__ __launch_bounds__(kReduceThreads) void splitk_reduce_kernel(const float* __restrict__ part,
                                                                       uint16_t* __restrict__ y, int64_t M,
                                                                       int64_t N, int S) {
  const int64_t MN = M * N;
  const int64_t i = ((int64_t)blockIdx.x * kReduceThreads + threadIdx.x) * 4;
  if (i >= MN) return;
  if ((N & 3) == 0) {
    v4f acc = *reinterpret_cast<const v4f*>(part + i);
    for (int s = 1; s < S; ++s) acc += *reinterpret_cast<const v4f*>(part + (int64_t)s * MN + i);
    u32x2 pk;
    pk.x = bf16_rne(acc[0]) | (bf16_rne(acc[1]) << 16);
    pk.y = bf16_rne(acc[2]) | (bf16_rne(acc[3]) << 16);
    *reinterpret_cast<u32x2*>(y + i) = pk;
  } else {
    for (int64_t e = i; e < i + 4 && e < MN; ++e) {
      float acc = part[e];
      for (int s = 1; s < S; ++s) acc += part[(int64_t)s * MN + e];
      y[e] = (uint16_t)bf16_rne(acc);
    }
  }
}

// Grouped form: workgroup slot s is mapped to (expert, m-tile) by a prefix
// sum over ceil(rows_e / BM) computed in the workgroup from the device
// offsets; slots past the last tile exit.  Offsets are clamped to [0, M].
// kGather: activation row m is row a_rows[m] / a_div of a (the MoE token
// of a routed pair), read straight from the token-major buffer.
template <class Kern, int BN, int BM, bool kGather>
__global__ __launch_bounds__(threads_of<Kern>(), Kern::kWavesPerSimd) void gemm_grouped_kernel(
    const uint8_t* __restrict__ a, const float* __restrict__ sa, const uint8_t* __restrict__ w,
    const float* __restrict__ sw, const int32_t* __restrict__ offsets, uint16_t* __restrict__ y, int64_t M,
    int64_t N, int64_t K, int G, int64_t slots, int64_t tiles_n, const int32_t* __restrict__ a_rows, int a_div,
    int64_t a_nrows) {
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr int NT = threads_of<Kern>();
  __shared__ int found_e, found_t;
  __shared__ int wave_sum[NT / 64];
  const int64_t L = xcd_linear(blockIdx.x, slots * tiles_n);
  // n fastest: the workgroups of one (expert, m-tile) share its activation rows
  const int64_t tn = L % tiles_n;
  const int slot = (int)(L / tiles_n);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) found_e = -1;
  int base = 0;  // tiles of experts before this chunk
  for (int c0 = 0; c0 < G; c0 += NT) {
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
    for (int i = 0; i < NT / 64; ++i) total += wave_sum[i];
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
  t.a_rows = a_rows; t.a_div = a_div; t.a_nrows = a_nrows;
  t.kb0 = 0; t.kb1 = (int)KB; t.part = nullptr;
  if constexpr (kGather)
    Kern::run_gather(t, smem);
  else
    Kern::run(t, smem);
}

// Persistent grouped form: `gridDim.x` workgroups (at most one per CU)
// each take tiles pos, pos + P, pos + 2P, .. of the (expert, m-tile, n-tile)
// list, where P = gridDim.x and pos is the XCD-aware rank of the workgroup,
// so that the workgroups of one XCD run consecutive tiles (the n-tiles of
// one expert's rows) at the same time.  The workgroup first builds the
// prefix of ceil(rows_e / BM) over the experts in LDS; a tile's expert is
// then a binary search in it.  Offsets are clamped to [0, M] as in the
// per-tile kernel.
constexpr int kMaxPersistentExperts = 1024;

template <class Kern, bool kGather>
__global__ __launch_bounds__(threads_of<Kern>(), Kern::kWavesPerSimd) void gemm_grouped_persistent_kernel(
    const uint8_t* __restrict__ a, const float* __restrict__ sa, const uint8_t* __restrict__ w,
    const float* __restrict__ sw, const int32_t* __restrict__ offsets, uint16_t* __restrict__ y, int64_t M,
    int64_t N, int64_t K, int G, int64_t tiles_n, const int32_t* __restrict__ a_rows, int a_div, int64_t a_nrows,
    uint8_t* __restrict__ hq, float* __restrict__ hs) {
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr int NT = threads_of<Kern>();
  constexpr int BM = Kern::BM, BN = Kern::BN;
  __shared__ int pre[kMaxPersistentExperts + 1];
  __shared__ int wave_sum[NT / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  auto clamped = [&](int e, int* lo, int* hi) {
    int l = offsets[e], h = offsets[e + 1];
    l = l < 0 ? 0 : (l > M ? (int)M : l);
    h = h < l ? l : (h > M ? (int)M : h);
    *lo = l;
    *hi = h;
  };
  if (tid == 0) pre[0] = 0;
  int base = 0;
  for (int c0 = 0; c0 < G; c0 += NT) {
    const int e = c0 + tid;
    int tiles = 0;
    if (e < G) {
      int lo, hi;
      clamped(e, &lo, &hi);
      tiles = (hi - lo + BM - 1) / BM;
    }
    int incl = tiles;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    __syncthreads();
    if (lane == 63) wave_sum[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int i = 0; i < wave; ++i) before += wave_sum[i];
    if (e < G) pre[e + 1] = base + before + incl;
    int total = 0;
    for (int i = 0; i < NT / 64; ++i) total += wave_sum[i];
    base += total;
  }
  __syncthreads();
  const int64_t tiles = (int64_t)pre[G] * tiles_n;
  const int64_t P = gridDim.x;
  const int64_t pos = xcd_linear(blockIdx.x, P);
  if (pos >= tiles) return;  // uniform
  const int ntiles = (int)((tiles - pos + P - 1) / P);
  const int64_t KB = K / kBlock;
  const int64_t NB = (N + kBlock - 1) / kBlock;
  auto tile_at = [&](int r) {
    const int64_t L = pos + (int64_t)r * P;
    const int64_t tn = L % tiles_n;
    const int slot = (int)(L / tiles_n);
    int lo_e = 0, hi_e = G - 1;  // the largest e with pre[e] <= slot
    while (lo_e < hi_e) {
      const int mid = (lo_e + hi_e + 1) >> 1;
      if (pre[mid] <= slot) lo_e = mid; else hi_e = mid - 1;
    }
    const int e = lo_e;
    int lo, hi;
    clamped(e, &lo, &hi);
    Tile t;
    t.a = a; t.sa = sa;
    t.w = w + (int64_t)e * N * K;
    t.sw = sw + (int64_t)e * NB * KB;
    t.y = y;
    t.m_lo = (int64_t)lo + (int64_t)(slot - pre[e]) * BM;
    t.m_hi = (t.m_lo + BM < hi) ? t.m_lo + BM : hi;
    t.n0 = tn * (Kern::kSiluForm ? kBlock : BN);  // the fc1 form's tiles are 128 columns of h
    t.N = N; t.K = K;
    t.a_rows = a_rows; t.a_div = a_div; t.a_nrows = a_nrows;
    t.kb0 = 0; t.kb1 = (int)KB; t.part = nullptr;
    t.hq = hq; t.hs = hs;
    return t;
  };
  Kern::template run_persistent<kGather>(ntiles, tile_at, smem);
}

enum class Cfg { kSkinny64x64, kSkinny48x64, kWide, kDecodePanel, kDeep, kPanel192, kSkinny96x64 };

// Per-workgroup cycle estimate: operand bytes through L1 (64 B/clk/CU) vs
// FP8 MFMA (8192 FLOP/clk/CU), times the rounds of workgroups over the CUs.
double est_cycles(int64_t M, int64_t N, int64_t K, int bn, int bm, double cus) {
  const double tiles = (double)((N + bn - 1) / bn) * (double)((M + bm - 1) / bm);
  const double rounds = std::ceil(tiles / cus);  // waves of workgroups over the CUs
  const double l1 = (double)(bn + bm) * (double)K / 64.0;
  const double mfma = 2.0 * bn * bm * (double)K / 8192.0;
  return rounds * (l1 > mfma ? l1 : mfma);
}

// The CU count of the device (256 on MI355X; 256 if it cannot be read).
double cu_count() {
  const int n = device_cus();
  return n > 0 ? (double)n : 256.0;
}

// Skinny tiles 64 or 48 weight rows wide: whichever fills its rounds of one
// workgroup per CU more evenly (tiles / (rounds * CUs)); ties keep 64.  At
// M = 256 the 48-row tile gives qkv (N = 6144) 512 tiles, two per CU, where
// the 64-row one gives 384 (19.7 vs 21.7 us); o and down (N = 4096) stay at
// 256 tiles of 64 rows.
Cfg skinny_narrow(int64_t M, int64_t N) {
  const double cus = cu_count();
  auto fill = [&](int bn) {
    const double t = (double)((N + bn - 1) / bn) * (double)((M + 63) / 64);
    return t / (std::ceil(t / cus) * cus);
  };
  return fill(48) > fill(64) ? Cfg::kSkinny48x64 : Cfg::kSkinny64x64;
}

Cfg choose(int64_t M, int64_t N, int64_t K) {
  const double cus = cu_count();
  // Few activation rows (65 .. 256) but many weight rows: one 128 x 256
  // panel covers every row of the activation panel, so each weight row is
  // read once.  At M <= 64 the K-split skinny tiles are faster (Qwen3-8B
  // gate_up, M = 64: 24.2 us on the 96-row tile, 27.7 on the 48-row one,
  // 33.9 on the panel).
  if (M > 64 && M <= DecodePanel::BM && (N + DecodePanel::BN - 1) / DecodePanel::BN >= (int64_t)(0.625 * cus)) {
    // the 192 x 128 panel when its tiles fill 7/8 or more of the CUs in one round
    const int64_t t192 = ((N + Panel192::BN - 1) / Panel192::BN) * ((M + Panel192::BM - 1) / Panel192::BM);
    if (t192 >= (int64_t)(0.875 * cus) && t192 <= (int64_t)cus) return Cfg::kPanel192;
    return Cfg::kDecodePanel;
  }
  double best = est_cycles(M, N, K, Wide::BN, Wide::BM, cus);
  Cfg c = Cfg::kWide;
  const double s64 = est_cycles(M, N, K, 64, 64, cus) * 1.05;  // partial-tile reduction overhead
  if (s64 < best) {
    auto tiles = [&](int bn) { return (double)((N + bn - 1) / bn) * (double)((M + 63) / 64); };
    c = skinny_narrow(M, N);
    // The 96-row tile moves (96 + 64) K bytes per tile against (48 + 64) K
    // or (64 + 64) K, but runs one wave per SIMD: it pays when its tiles
    // fill the CUs and its rounds x bytes per tile come out smaller.  At
    // M = 256 qkv (N = 6144) takes 256 tiles of 96 rows (one round) instead
    // of 512 of 48 (15.4 vs 19.1 us); at M = 64 gate_up (N = 24576) 256
    // instead of 512 (24.2 vs 28.3 us).  Fewer tiles than CUs lose (M = 128,
    // N = 6144: 14.8 vs 11.8 us).
    const int bn = c == Cfg::kSkinny48x64 ? 48 : 64;
    const double r96 = std::ceil(tiles(96) / cus) * (96 + 64);
    const double rc = std::ceil(tiles(bn) / cus) * (bn + 64);
    if (tiles(96) >= 0.875 * cus && r96 < rc) c = Cfg::kSkinny96x64;
  }
  return c;
}

template <class Kern, int BN, int BM>
hipError_t launch_dense_cfg(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw, uint16_t* y,
                            int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int64_t blocks = tiles_m * tiles_n;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_dense_kernel<Kern, BN, BM>), dim3((unsigned)blocks), dim3(threads_of<Kern>()),
                     (size_t)Kern::kLdsBytes, stream, a, sa, w, sw, y, M, N, K, tiles_m, tiles_n);
  return hipGetLastError();
}

// A named tile kernel (FP8BQ_TILE_* of the C ABI; 0 = the cost model).
bool tile_cfg(int tile, int64_t M, int64_t N, int64_t K, Cfg* c) {
  switch (tile) {
    case 0: *c = choose(M, N, K); return true;
    case 1: *c = Cfg::kSkinny64x64; return true;
    case 2: *c = Cfg::kSkinny48x64; return true;
    case 3: *c = Cfg::kWide; return true;
    case 4: *c = Cfg::kDecodePanel; return true;
    case 5: *c = Cfg::kDeep; return true;
    case 6: *c = Cfg::kPanel192; return true;
    case 8: *c = Cfg::kSkinny96x64; return true;
    default: return false;
  }
}

template <class Kern, bool kGather>
hipError_t launch_grouped_cfg(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw,
                              const int32_t* offsets, uint16_t* y, int64_t M, int64_t N, int64_t K, int64_t G,
                              const int32_t* a_rows, int a_div, int64_t a_nrows, hipStream_t stream) {
  const int64_t tiles_n = (N + Kern::BN - 1) / Kern::BN;
  const int64_t slots = (M + Kern::BM - 1) / Kern::BM + G;  // >= sum_e ceil(rows_e / BM)
  const int64_t blocks = tiles_n * slots;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_grouped_kernel<Kern, Kern::BN, Kern::BM, kGather>), dim3((unsigned)blocks),
                     dim3(Kern::kThreadsPerWg), (size_t)Kern::kLdsBytes, stream, a, sa, w, sw, offsets, y, M, N, K,
                     (int)G, slots, tiles_n, a_rows, a_div, a_nrows);
  return hipGetLastError();
}

template <class Kern, bool kGather>
hipError_t launch_grouped_persistent(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw,
                                     const int32_t* offsets, uint16_t* y, int64_t M, int64_t N, int64_t K, int64_t G,
                                     const int32_t* a_rows, int a_div, int64_t a_nrows, hipStream_t stream,
                                     uint8_t* hq = nullptr, float* hs = nullptr) {
  // the fc1 form: N = 2F weight rows, one tile per 128 columns of h
  const int64_t tiles_n = Kern::kSiluForm ? N / 2 / kBlock : (N + Kern::BN - 1) / Kern::BN;
  const int64_t bound = tiles_n * ((M + Kern::BM - 1) / Kern::BM + G);  // >= the tiles there are
  const int64_t cus = (int64_t)cu_count();
  const int64_t P = bound < cus ? bound : cus;  // one workgroup per CU (the tile's LDS allows one)
  hipLaunchKernelGGL((gemm_grouped_persistent_kernel<Kern, kGather>), dim3((unsigned)P), dim3(Kern::kThreadsPerWg),
                     (size_t)Kern::kLdsBytes, stream, a, sa, w, sw, offsets, y, M, N, K, (int)G, tiles_n, a_rows,
                     a_div, a_nrows, hq, hs);
  return hipGetLastError();
}

template <bool kGather>
hipError_t launch_grouped_any(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw,
                              const int32_t* offsets, uint16_t* y, int64_t M, int64_t N, int64_t K, int64_t G,
                              const int32_t* a_rows, int a_div, int64_t a_nrows, int tile, hipStream_t stream) {
  if (M == 0 || N == 0 || G == 0) return hipSuccess;
  // The expert tiles: each expert's weights are read by its own few tiles
  // only, so they stream from HBM, and the deep (three-stage) panel keeps
  // more of them in flight.  Measured on the Qwen3-30B-A3B expert layer
  // (128 experts, ~256 rows each): fc1 234 vs 263 us, fc2 168 vs 178 us
  // for the 256 x 256 two-stage tile.  Run persistent (one workgroup per
  // CU, the ring carried across tiles) while the expert table fits in LDS:
  // fc1 224-228 vs 240 us, fc2 131 vs 167 us (its tiles have 6 K-blocks,
  // so the per-tile pipeline fill weighed most).  The others when named.
  if (tile == 4)
    return launch_grouped_cfg<DecodePanel, kGather>(a, sa, w, sw, offsets, y, M, N, K, G, a_rows, a_div, a_nrows,
                                                    stream);
  if (tile == 3)
    return launch_grouped_cfg<Wide, kGather>(a, sa, w, sw, offsets, y, M, N, K, G, a_rows, a_div, a_nrows, stream);
  if (tile != 0 && tile != 5 && tile != 7) return hipErrorInvalidValue;
  // K = 0: the per-tile kernel stores the zero products (the persistent one
  // has no K-block step to end a tile on)
  const bool per_tile = tile == 5 || K == 0;
  if (per_tile || G > kMaxPersistentExperts)
    return launch_grouped_cfg<Deep, kGather>(a, sa, w, sw, offsets, y, M, N, K, G, a_rows, a_div, a_nrows, stream);
  return launch_grouped_persistent<Deep, kGather>(a, sa, w, sw, offsets, y, M, N, K, G, a_rows, a_div, a_nrows,
                                                  stream);
}

}  // namespace

hipError_t launch_gemm(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw, uint16_t* y, int64_t M,
                       int64_t N, int64_t K, int tile, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  Cfg cfg;
  if (!tile_cfg(tile, M, N, K, &cfg)) return hipErrorInvalidValue;
  // Row-major operands stage both tiles through LDS; at 96 weight rows that
  // form holds more than its registers (qkv at M = 256: 21.5 vs 20.0 us on
  // the 48-row tile), so the cost model's 96-row choice runs as 48 / 64
  // here.  Every skinny width sums in the same order: the same bits.
  if (tile == 0 && cfg == Cfg::kSkinny96x64) cfg = skinny_narrow(M, N);
  switch (cfg) {
    case Cfg::kSkinny64x64:
      return launch_dense_cfg<Skinny<64, 64, 4>, 64, 64>(a, sa, w, sw, y, M, N, K, stream);
    case Cfg::kSkinny48x64:
      return launch_dense_cfg<Skinny<48, 64, 4>, 48, 64>(a, sa, w, sw, y, M, N, K, stream);
    case Cfg::kSkinny96x64:
      return launch_dense_cfg<Skinny<96, 64, 4>, 96, 64>(a, sa, w, sw, y, M, N, K, stream);
    case Cfg::kDecodePanel:
      if (2 * M <= DecodePanel::BM)
        return launch_dense_cfg<DecodePanelSplit<>, DecodePanel::BN, DecodePanel::BM>(a, sa, w, sw, y, M, N, K, stream);
      return launch_dense_cfg<DecodePanel, DecodePanel::BN, DecodePanel::BM>(a, sa, w, sw, y, M, N, K, stream);
    case Cfg::kPanel192:
      return launch_dense_cfg<Panel192, Panel192::BN, Panel192::BM>(a, sa, w, sw, y, M, N, K, stream);
    case Cfg::kDeep:
      return launch_dense_cfg<Deep, Deep::BN, Deep::BM>(a, sa, w, sw, y, M, N, K, stream);
    default:
      return launch_dense_cfg<Wide, Wide::BN, Wide::BM>(a, sa, w, sw, y, M, N, K, stream);
  }
}

namespace {

// Pieces of K for the split form.  The FP32 partials cost 2 S M N 4 bytes
// of traffic next to the N K weight bytes, so the split pays only where K
// is long against M and each piece keeps enough K-blocks; measured on
// MI355X (graph replays, weights rotated past the Infinity Cache; us,
// unsplit -> 8 pieces): M = 16, N = 4096, K = 12288: 21.6 -> 15.9; M = 128
// same N, K: 23.4 -> 21.6; M = 16, N = 1024, K = 16384: 26.8 -> 16.2; but
// M = 256, K = 12288: 29.2 -> 30.6 and every K = 4096 shape slower (M = 16,
// N = 4096: 10.6 -> 11.3; M = 256: 13.5 -> 22.4), with 2 or 4 pieces slower
// still.  Rule: 8 pieces (fewer when the 128-row weight tiles times 8 do
// not fit one round of the CUs, at least 4) when M <= 256, 96 M <= K and
// every piece has at least 8 K-blocks.  1 = no split.
int splitk_pieces(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || M > DecodePanel::BM || N <= 0 || 96 * M > K) return 1;
  const int64_t tiles = (N + DecodePanel::BN - 1) / DecodePanel::BN;
  const int64_t cus = (int64_t)cu_count();
  int64_t S = cus / tiles;
  if (S > 8) S = 8;
  if (S < 4 || K / kBlock < 8 * S) return 1;
  return (int)S;
}

}  // namespace

int64_t gemm_splitk_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const int S = splitk_pieces(M, N, K);
  return S > 1 ? (int64_t)S * M * N * 4 : 0;
}

hipError_t launch_gemm_splitk(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw, uint16_t* y,
                              int64_t M, int64_t N, int64_t K, void* workspace, int64_t workspace_bytes,
                              hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int S = splitk_pieces(M, N, K);
  if (S == 1) return launch_gemm(a, sa, w, sw, y, M, N, K, 0, stream);
  if (workspace == nullptr || workspace_bytes < (int64_t)S * M * N * 4) return hipErrorInvalidValue;
  using Kern = DecodePanel;
  const int64_t tiles_m = (M + Kern::BM - 1) / Kern::BM, tiles_n = (N + Kern::BN - 1) / Kern::BN;
  float* part = static_cast<float*>(workspace);
  hipLaunchKernelGGL((gemm_splitk_kernel<Kern, Kern::BN, Kern::BM>), dim3((unsigned)(tiles_m * tiles_n * S)),
                     dim3(threads_of<Kern>()), (size_t)Kern::kLdsBytes, stream, a, sa, w, sw, part, M, N, K, tiles_m,
                     tiles_n, S);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t units = (M * N + 3) / 4;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((units + kReduceThreads - 1) / kReduceThreads)),
                     dim3(kReduceThreads), 0, stream, part, y, M, N, S);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The K split without a caller workspace, for callers that cannot allocate
// (code under graph capture, serving loops that forbid it): the partials go
// to `scratch`, a file-scope device array of kScratchBytes that each GPU the
// library runs on holds until the process ends.  Its device address is
// looked up once per device (hipGetSymbolAddress, with that device
// current) and passed to the kernels like a workspace; host code never
// uses the array's name for its memory.  Every call on a GPU shares the
// array: calls that overlap on one GPU race.  The partials are written in
// full before they are read, so nothing needs clearing between calls.
// ---------------------------------------------------------------------------
constexpr int64_t kScratchBytes = int64_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch[kMaxScratchDevices];

// The device address of `scratch` on the current device.
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

int64_t gemm_splitk_scratch_bytes() { return kScratchBytes; }

hipError_t launch_gemm_splitk_noalloc(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw,
                                      uint16_t* y, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  if (gemm_splitk_workspace_bytes(M, N, K) > kScratchBytes) return hipErrorInvalidValue;
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return e;
  return launch_gemm_splitk(a, sa, w, sw, y, M, N, K, ws, kScratchBytes, stream);
}

// Fragment-order activations: the tile the cost model picks for row-major
// ones, in its fragment-order form (the skinny tiles load the activation
// fragments straight into registers; the panels keep them in fragment
// order in their LDS ring).  Qwen3-8B decode shapes at M = 256 (us,
// row-major -> fragment order, bit-identical): qkv 19.3 -> 18.0, o 14.1 ->
// 12.5, gate_up 45.9 -> 43.5, down 28.8 -> 24.8; the four prefill shapes at
// M = 8192 on quantized normal data: 1.77 -> 1.95 PF (the four-wave
// 128 x 256 panel that loads activation fragments into registers, two per
// CU: 1.90 PF).
//
// Weights in fragment order as well (wfrag): the same tiles with the weight
// fragments loaded straight into registers (K-split tiles) or copied 1 KB at
// a time into the LDS ring (panels); bit-identical again.  Prefill shapes on
// quantized normal data: 1.95 -> 2.01 PF.
template <bool kW>
hipError_t launch_gemm_frag_cfg(Cfg cfg, const uint8_t* a, const float* sa, const uint8_t* w, const float* sw,
                                uint16_t* y, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  switch (cfg) {
    case Cfg::kSkinny64x64:
      return launch_dense_cfg<Skinny<64, 64, 4, true, kW>, 64, 64>(a, sa, w, sw, y, M, N, K, stream);
    case Cfg::kSkinny48x64:
      return launch_dense_cfg<Skinny<48, 64, 4, true, kW>, 48, 64>(a, sa, w, sw, y, M, N, K, stream);
    case Cfg::kSkinny96x64:
      return launch_dense_cfg<Skinny<96, 64, 4, true, kW>, 96, 64>(a, sa, w, sw, y, M, N, K, stream);
    case Cfg::kPanel192:
      return launch_dense_cfg<PanelFragA<Panel<192, 128, 2, 4, 3, kW, false, true>>, 192, 128>(a, sa, w, sw, y, M, N,
                                                                                               K, stream);
    case Cfg::kDecodePanel:
      if (2 * M <= DecodePanel::BM)
        return launch_dense_cfg<PanelFragA<DecodePanelSplit<kW>>, 128, 256>(a, sa, w, sw, y, M, N, K, stream);
      return launch_dense_cfg<PanelFragA<Panel<128, 256, 2, 4, 3, kW>>, 128, 256>(a, sa, w, sw, y, M, N, K, stream);
    default:
      return launch_dense_cfg<PanelFragA<Panel<256, 256, 2, 4, 2, kW>>, 256, 256>(a, sa, w, sw, y, M, N, K, stream);
  }
}

hipError_t launch_gemm_afrag(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw, uint16_t* y,
                             int64_t M, int64_t N, int64_t K, bool wfrag, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (M % 16 != 0 || K % kBlock != 0 || (wfrag && N % 16 != 0)) return hipErrorInvalidValue;
  const Cfg cfg = choose(M, N, K);
  return wfrag ? launch_gemm_frag_cfg<true>(cfg, a, sa, w, sw, y, M, N, K, stream)
               : launch_gemm_frag_cfg<false>(cfg, a, sa, w, sw, y, M, N, K, stream);
}

hipError_t launch_grouped_gemm(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw,
                               const int32_t* offsets, uint16_t* y, int64_t M, int64_t N, int64_t K, int64_t G,
                               int tile, hipStream_t stream) {
  return launch_grouped_any<false>(a, sa, w, sw, offsets, y, M, N, K, G, nullptr, 1, 0, tile, stream);
}

// The MoE fc1 GEMM with the SiLU(gate) * up quantization in its epilogue:
// the persistent deep tile in its fc1 form (weights [G][2F][K], F % 128 ==
// 0, G <= kMaxPersistentExperts), rows gathered through a_rows.
hipError_t launch_grouped_gemm_gather_silu(const uint8_t* a, const float* sa, const int32_t* a_rows, int64_t a_div,
                                           int64_t a_nrows, const uint8_t* w, const float* sw, const int32_t* offsets,
                                           uint8_t* hq, float* hs, int64_t M, int64_t F, int64_t K, int64_t G,
                                           hipStream_t stream) {
  if (M == 0 || F == 0 || G == 0) return hipSuccess;
  if (F % kBlock != 0 || G > kMaxPersistentExperts) return hipErrorInvalidValue;
  using Kern = Panel<256, 128, 2, 4, 3, false, true>;
  return launch_grouped_persistent<Kern, true>(a, sa, w, sw, offsets, nullptr, M, 2 * F, K, G, a_rows, (int)a_div,
                                               a_nrows, stream, hq, hs);
}

hipError_t launch_grouped_gemm_gather(const uint8_t* a, const float* sa, const int32_t* a_rows, int64_t a_div,
                                      int64_t a_nrows, const uint8_t* w, const float* sw, const int32_t* offsets,
                                      uint16_t* y, int64_t M, int64_t N, int64_t K, int64_t G, int tile,
                                      hipStream_t stream) {
  return launch_grouped_any<true>(a, sa, w, sw, offsets, y, M, N, K, G, a_rows, (int)a_div, a_nrows, tile, stream);
}

}  // namespace fp8bq
