// C-ABI layer of libfp8bq.so: argument checks, device check, launches.
// The contract of every entry point is documented in include/fp8bq.h.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/fp8bq.h"
#include "launch.hpp"

static_assert(FP8BQ_MAX_WEIGHT_DESCS == fp8bq::kMaxWeightDescs, "descriptor limits of the header and the launcher");
static_assert(FP8BQ_MAX_ACT_DESCS == fp8bq::kMaxActDescs, "descriptor limits of the header and the launcher");
static_assert(FP8BQ_SCRATCH_BYTES == 32 * 1024 * 1024, "static scratch size of the header and the GEMM source");

namespace {

constexpr int kMaxDevices = 64;
// per-device cache of the architecture check: 0 = unknown, 1 = gfx950, 2 = other
std::atomic<int> g_arch_ok[kMaxDevices];

fp8bq_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FP8BQ_ERR_DEVICE;
  if (dev >= kMaxDevices) return FP8BQ_ERR_DEVICE;
  int state = g_arch_ok[dev].load(std::memory_order_acquire);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FP8BQ_ERR_DEVICE;
    state = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch_ok[dev].store(state, std::memory_order_release);
  }
  return state == 1 ? FP8BQ_OK : FP8BQ_ERR_DEVICE;
}

}  // namespace

namespace fp8bq {

int device_cus() {
  static std::atomic<int> cached[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int n = cached[dev].load(std::memory_order_acquire);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
    cached[dev].store(n, std::memory_order_release);
  }
  return n;
}

}  // namespace fp8bq

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Largest GEMM K: the GEMM kernels address an operand panel of at most 256
// rows x K bytes with 32-bit buffer offsets.
constexpr int64_t kMaxGemmK = int64_t(1) << 22;

// Largest elementwise problem: its one-dimensional grid of 256-lane
// workgroups, four elements per lane, must stay below 2^31 workgroups.
constexpr int64_t kMaxElementwise = int64_t(1) << 40;

// a * b without int64 overflow (both >= 0)
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a == 0 || b == 0) {
    *out = 0;
    return true;
  }
  if (a > INT64_MAX / b) return false;
  *out = a * b;
  return true;
}

fp8bq_status launched(hipError_t e) { return e == hipSuccess ? FP8BQ_OK : FP8BQ_ERR_LAUNCH; }

// The grouped GEMMs' offsets contract, checked on the host: [0] = 0,
// non-decreasing, [G] = M_total (the offsets are copied on `stream`, which
// the call waits for).
fp8bq_status check_offsets(const int32_t* offsets, int64_t G, int64_t M_total, hipStream_t stream) {
  std::vector<int32_t> h(static_cast<size_t>(G + 1));
  if (hipMemcpyAsync(h.data(), offsets, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return FP8BQ_ERR_LAUNCH;
  if (h[0] != 0 || h[static_cast<size_t>(G)] != M_total) return FP8BQ_ERR_BAD_SHAPE;
  for (int64_t g = 0; g < G; ++g)
    if (h[static_cast<size_t>(g + 1)] < h[static_cast<size_t>(g)]) return FP8BQ_ERR_BAD_SHAPE;
  return FP8BQ_OK;
}

// Debug mode for the grouped GEMMs' device-side precondition: with
// FP8BQ_CHECK_OFFSETS=1 in the environment (read once, at the first grouped
// GEMM call of the process) every grouped call checks its offsets first.
fp8bq_status check_offsets_if_asked(const int32_t* offsets, int64_t G, int64_t M_total, hipStream_t stream) {
  static const bool enabled = [] {
    const char* e = std::getenv("FP8BQ_CHECK_OFFSETS");
    return e != nullptr && std::strcmp(e, "1") == 0;
  }();
  return enabled ? check_offsets(offsets, G, M_total, stream) : FP8BQ_OK;
}

// Clears a stale runtime error so that the post-launch check reports ours.
void clear_last_error() { (void)hipGetLastError(); }

}  // namespace

extern "C" {

const char* fp8bq_status_string(fp8bq_status s) {
  switch (s) {
    case FP8BQ_OK: return "ok";
    case FP8BQ_ERR_NULL_PTR: return "null pointer for a non-empty tensor";
    case FP8BQ_ERR_BAD_SHAPE: return "invalid shape (negative size, GEMM K not a multiple of 128 or above 2^22, or size overflow)";
    case FP8BQ_ERR_MISALIGNED: return "tensor pointer not 16-byte aligned";
    case FP8BQ_ERR_LAUNCH: return "kernel launch failed";
    case FP8BQ_ERR_DEVICE: return "current device is not an AMD gfx950 GPU";
    case FP8BQ_ERR_BAD_ARG: return "invalid scalar argument or option combination";
    case FP8BQ_ERR_WORKSPACE: return "workspace missing, misaligned or too small for this call";
    case FP8BQ_ERR_SCRATCH: return "the call needs more than the library's static scratch (FP8BQ_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

}  // extern "C"

namespace {

// The weight quantizers: row-major codes, or (frag) MFMA fragment order,
// which needs N % 16 == 0 and K % 128 == 0.
fp8bq_status quantize_weight(const uint16_t* w_bf16, uint8_t* w_fp8, float* w_scale, int64_t batch, int64_t N,
                             int64_t K, bool frag, void* stream) {
  try {
    if (batch < 0 || N < 0 || K < 0) return FP8BQ_ERR_BAD_SHAPE;
    if (frag && ((N % 16) != 0 || (K % 128) != 0)) return FP8BQ_ERR_BAD_SHAPE;
    int64_t nk, total, bytes;
    if (!mul_ok(N, K, &nk) || !mul_ok(nk, batch, &total) || !mul_ok(total, 2, &bytes)) return FP8BQ_ERR_BAD_SHAPE;
    if (total == 0) return FP8BQ_OK;
    if (!w_bf16 || !w_fp8 || !w_scale) return FP8BQ_ERR_NULL_PTR;
    if (!aligned16(w_bf16) || !aligned16(w_fp8) || !aligned16(w_scale)) return FP8BQ_ERR_MISALIGNED;
    fp8bq_status st = check_device();
    if (st != FP8BQ_OK) return st;
    clear_last_error();
    return launched(fp8bq::launch_quant_weight(w_bf16, w_fp8, w_scale, batch, N, K, frag,
                                               static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FP8BQ_ERR_LAUNCH;
  }
}

fp8bq_status quantize_weights_multi(const fp8bq_weight_desc* descs, int64_t count, bool frag, void* stream) {
  try {
    if (count < 0 || count > FP8BQ_MAX_WEIGHT_DESCS) return FP8BQ_ERR_BAD_SHAPE;
    if (count == 0) return FP8BQ_OK;
    if (!descs) return FP8BQ_ERR_NULL_PTR;
    // validate each matrix as quantize_weight_blockwise would, keep the non-empty ones
    std::vector<int> idx;
    std::vector<int64_t> nblk(static_cast<size_t>(count), 0);
    for (int64_t i = 0; i < count; ++i) {
      const fp8bq_weight_desc& d = descs[i];
      if (d.N < 0 || d.K < 0) return FP8BQ_ERR_BAD_SHAPE;
      if (frag && ((d.N % 16) != 0 || (d.K % 128) != 0)) return FP8BQ_ERR_BAD_SHAPE;
      int64_t nk, bytes;
      if (!mul_ok(d.N, d.K, &nk) || !mul_ok(nk, 2, &bytes)) return FP8BQ_ERR_BAD_SHAPE;
      if (nk == 0) continue;
      if (!d.w_bf16 || !d.w_fp8 || !d.w_scale) return FP8BQ_ERR_NULL_PTR;
      if (!aligned16(d.w_bf16) || !aligned16(d.w_fp8) || !aligned16(d.w_scale)) return FP8BQ_ERR_MISALIGNED;
      nblk[static_cast<size_t>(i)] = ((d.N + 127) / 128) * ((d.K + 127) / 128);
      idx.push_back(static_cast<int>(i));
    }
    if (idx.empty()) return FP8BQ_OK;
    // largest matrices first: the small ones fill in at the end of the launch
    std::stable_sort(idx.begin(), idx.end(), [&](int a, int b) { return nblk[a] > nblk[b]; });
    fp8bq::WeightBatch batch{};
    batch.count = static_cast<int>(idx.size());
    int64_t blocks = 0;
    for (int t = 0; t < batch.count; ++t) {
      const fp8bq_weight_desc& d = descs[idx[static_cast<size_t>(t)]];
      batch.desc[t] = fp8bq::WeightDesc{d.w_bf16, d.w_fp8, d.w_scale, d.N, d.K};
      batch.first[t] = blocks;
      blocks += nblk[static_cast<size_t>(idx[static_cast<size_t>(t)])];
    }
    batch.first[batch.count] = blocks;
    if (blocks > 0x7fffffffLL) return FP8BQ_ERR_BAD_SHAPE;
    fp8bq_status st = check_device();
    if (st != FP8BQ_OK) return st;
    clear_last_error();
    return launched(fp8bq::launch_quant_weight_multi(batch, blocks, frag, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FP8BQ_ERR_LAUNCH;
  }
}

}  // namespace

extern "C" {

fp8bq_status quantize_weight_blockwise(const uint16_t* w_bf16, uint8_t* w_fp8, float* w_scale, int64_t batch,
                                       int64_t N, int64_t K, void* stream) {
  return quantize_weight(w_bf16, w_fp8, w_scale, batch, N, K, false, stream);
}

fp8bq_status quantize_weight_blockwise_frag(const uint16_t* w_bf16, uint8_t* w_fp8_frag, float* w_scale,
                                            int64_t batch, int64_t N, int64_t K, void* stream) {
  return quantize_weight(w_bf16, w_fp8_frag, w_scale, batch, N, K, true, stream);
}

fp8bq_status quantize_weights_blockwise_multi(const fp8bq_weight_desc* descs, int64_t count, void* stream) {
  return quantize_weights_multi(descs, count, false, stream);
}

fp8bq_status quantize_weights_blockwise_frag_multi(const fp8bq_weight_desc* descs, int64_t count, void* stream) {
  return quantize_weights_multi(descs, count, true, stream);
}

fp8bq_status quantize_act_per_token_group(const uint16_t* x_bf16, uint8_t* x_fp8, float* x_scale, int64_t M,
                                          int64_t K, void* stream) {
  try {
    if (M < 0 || K < 0) return FP8BQ_ERR_BAD_SHAPE;
    int64_t total, bytes;
    if (!mul_ok(M, K, &total) || !mul_ok(total, 2, &bytes)) return FP8BQ_ERR_BAD_SHAPE;
    if (total == 0) return FP8BQ_OK;
    if (!x_bf16 || !x_fp8 || !x_scale) return FP8BQ_ERR_NULL_PTR;
    if (!aligned16(x_bf16) || !aligned16(x_fp8) || !aligned16(x_scale)) return FP8BQ_ERR_MISALIGNED;
    fp8bq_status st = check_device();
    if (st != FP8BQ_OK) return st;
    clear_last_error();
    return launched(fp8bq::launch_quant_act(x_bf16, x_fp8, x_scale, M, K, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FP8BQ_ERR_LAUNCH;
  }
}

}  // extern "C"

namespace {

// The two multi-activation quantizers: row-major (32 groups per workgroup)
// or fragment order (4 units of 16 rows x one K-block per workgroup, M % 16
// == 0 and K % 128 == 0 for each activation).
fp8bq_status quantize_acts_multi(const fp8bq_act_desc* descs, int64_t count, bool frag, void* stream) {
  try {
    if (count < 0 || count > FP8BQ_MAX_ACT_DESCS) return FP8BQ_ERR_BAD_SHAPE;
    if (count == 0) return FP8BQ_OK;
    if (!descs) return FP8BQ_ERR_NULL_PTR;
    fp8bq::ActBatch batch{};
    int64_t blocks = 0;
    for (int64_t i = 0; i < count; ++i) {
      const fp8bq_act_desc& d = descs[i];
      if (d.M < 0 || d.K < 0) return FP8BQ_ERR_BAD_SHAPE;
      if (frag && ((d.M % 16) != 0 || (d.K % 128) != 0)) return FP8BQ_ERR_BAD_SHAPE;
      int64_t mk, bytes;
      if (!mul_ok(d.M, d.K, &mk) || !mul_ok(mk, 2, &bytes)) return FP8BQ_ERR_BAD_SHAPE;
      if (mk == 0) continue;
      if (!d.x_bf16 || !d.x_fp8 || !d.x_scale) return FP8BQ_ERR_NULL_PTR;
      if (!aligned16(d.x_bf16) || !aligned16(d.x_fp8) || !aligned16(d.x_scale)) return FP8BQ_ERR_MISALIGNED;
      batch.desc[batch.count] = fp8bq::ActDesc{d.x_bf16, d.x_fp8, d.x_scale, d.M, d.K};
      batch.first[batch.count] = blocks;
      if (frag) {
        const int64_t units = (d.M / 16) * (d.K / 128);
        blocks += (units + fp8bq::kActFragUnitsPerWg - 1) / fp8bq::kActFragUnitsPerWg;
      } else {
        const int64_t groups = d.M * ((d.K + 127) / 128);
        blocks += (groups + fp8bq::kActGroupsPerWg - 1) / fp8bq::kActGroupsPerWg;
      }
      if (blocks > 0x7fffffffLL) return FP8BQ_ERR_BAD_SHAPE;
      ++batch.count;
    }
    batch.first[batch.count] = blocks;
    if (batch.count == 0) return FP8BQ_OK;
    fp8bq_status st = check_device();
    if (st != FP8BQ_OK) return st;
    clear_last_error();
    const hipStream_t s = static_cast<hipStream_t>(stream);
    return launched(frag ? fp8bq::launch_quant_act_frag_multi(batch, blocks, s)
                         : fp8bq::launch_quant_act_multi(batch, blocks, s));
  } catch (...) {
    return FP8BQ_ERR_LAUNCH;
  }
}

}  // namespace

extern "C" {

fp8bq_status quantize_acts_per_token_group_multi(const fp8bq_act_desc* descs, int64_t count, void* stream) {
  return quantize_acts_multi(descs, count, false, stream);
}

fp8bq_status quantize_acts_per_token_group_frag_multi(const fp8bq_act_desc* descs, int64_t count, void* stream) {
  return quantize_acts_multi(descs, count, true, stream);
}

fp8bq_status gemm_w8a8_blockscaled_tile(const uint8_t* a_fp8, const float* a_scale, const uint8_t* w_fp8,
                                        const float* w_scale, uint16_t* y_bf16, int64_t M, int64_t N, int64_t K,
                                        int tile, void* stream) {
  try {
    if (tile < FP8BQ_TILE_AUTO || (tile > FP8BQ_TILE_PANEL192 && tile != FP8BQ_TILE_SKINNY96))
      return FP8BQ_ERR_BAD_ARG;
    if (M < 0 || N < 0 || K < 0 || (K % 128) != 0 || K > kMaxGemmK) return FP8BQ_ERR_BAD_SHAPE;
    int64_t mk, nk, mn, bytes;
    if (!mul_ok(M, K, &mk) || !mul_ok(N, K, &nk) || !mul_ok(M, N, &mn) || !mul_ok(mn, 2, &bytes))
      return FP8BQ_ERR_BAD_SHAPE;
    if (mn == 0) return FP8BQ_OK;
    if (!y_bf16) return FP8BQ_ERR_NULL_PTR;
    if (K > 0 && (!a_fp8 || !a_scale || !w_fp8 || !w_scale)) return FP8BQ_ERR_NULL_PTR;
    if (!aligned16(y_bf16) || (K > 0 && (!aligned16(a_fp8) || !aligned16(a_scale) || !aligned16(w_fp8) ||
                                         !aligned16(w_scale))))
      return FP8BQ_ERR_MISALIGNED;
    fp8bq_status st = check_device();
    if (st != FP8BQ_OK) return st;
    clear_last_error();
    return launched(fp8bq::launch_gemm(a_fp8, a_scale, w_fp8, w_scale, y_bf16, M, N, K, tile,
                                       static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FP8BQ_ERR_LAUNCH;
  }
}

fp8bq_status gemm_w8a8_blockscaled(const uint8_t* a_fp8, const float* a_scale, const uint8_t* w_fp8,
                                   const float* w_scale, uint16_t* y_bf16, int64_t M, int64_t N, int64_t K,
                                   void* stream) {
  return gemm_w8a8_blockscaled_tile(a_fp8, a_scale, w_fp8, w_scale, y_bf16, M, N, K, FP8BQ_TILE_AUTO, stream);
}

// The GEMM shape checks shared by the dense entry points.
fp8bq_status check_gemm_shape(int64_t M, int64_t N, int64_t K, int64_t* mn) {
  if (M < 0 || N < 0 || K < 0 || (K % 128) != 0 || K > kMaxGemmK) return FP8BQ_ERR_BAD_SHAPE;
  int64_t mk, nk, bytes;
  if (!mul_ok(M, K, &mk) || !mul_ok(N, K, &nk) || !mul_ok(M, N, mn) || !mul_ok(*mn, 4, &bytes))
    return FP8BQ_ERR_BAD_SHAPE;
  return FP8BQ_OK;
}

fp8bq_status gemm_w8a8_blockscaled_splitk_workspace(int64_t M, int64_t N, int64_t K, int64_t* bytes) {
  try {
    if (!bytes) return FP8BQ_ERR_NULL_PTR;
    int64_t mn;
    fp8bq_status st = check_gemm_shape(M, N, K, &mn);
    if (st != FP8BQ_OK) return st;
    st = check_device();
    if (st != FP8BQ_OK) return st;
    *bytes = mn == 0 ? 0 : fp8bq::gemm_splitk_workspace_bytes(M, N, K);
    return FP8BQ_OK;
  } catch (...) {
    return FP8BQ_ERR_LAUNCH;
  }
}

fp8bq_status gemm_w8a8_blockscaled_splitk(const uint8_t* a_fp8, const float* a_scale, const uint8_t* w_fp8,
                                          const float* w_scale, uint16_t* y_bf16, int64_t M, int64_t N, int64_t K,
                                          void* workspace, int64_t workspace_bytes, void* stream) {
  try {
    int64_t mn;
    fp8bq_status st = check_gemm_shape(M, N, K, &mn);
    if (st != FP8BQ_OK) return st;
    if (mn == 0) return FP8BQ_OK;
    if (!y_bf16) return FP8BQ_ERR_NULL_PTR;
    if (K > 0 && (!a_fp8 || !a_scale || !w_fp8 || !w_scale)) return FP8BQ_ERR_NULL_PTR;
    if (!aligned16(y_bf16) || (K > 0 && (!aligned16(a_fp8) || !aligned16(a_scale) || !aligned16(w_fp8) ||
                                         !aligned16(w_scale))))
      return FP8BQ_ERR_MISALIGNED;
    st = check_device();
    if (st != FP8BQ_OK) return st;
    const int64_t need = fp8bq::gemm_splitk_workspace_bytes(M, N, K);
    if (need > 0 && (!workspace || !aligned16(workspace) || workspace_bytes < need)) return FP8BQ_ERR_WORKSPACE;
    clear_last_error();
    return launched(fp8bq::launch_gemm_splitk(a_fp8, a_scale, w_fp8, w_scale, y_bf16, M, N, K, workspace,
                                              workspace_bytes, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FP8BQ_ERR_LAUNCH;
  }
}

fp8bq_status gemm_w8a8_blockscaled_splitk_noalloc(const uint8_t* a_fp8, const float* a_scale, const uint8_t* w_fp8,
                                                  const float* w_scale, uint16_t* y_bf16, int64_t M, int64_t N,
                                                  int64_t K, void* stream) {
  try {
    int64_t mn;
    fp8bq_status st = check_gemm_shape(M, N, K, &mn);
    if (st != FP8BQ_OK) return st;
    if (mn == 0) return FP8BQ_OK;
    if (!y_bf16) return FP8BQ_ERR_NULL_PTR;
    if (K > 0 && (!a_fp8 || !a_scale || !w_fp8 || !w_scale)) return FP8BQ_ERR_NULL_PTR;
    if (!aligned16(y_bf16) || (K > 0 && (!aligned16(a_fp8) || !aligned16(a_scale) || !aligned16(w_fp8) ||
                                         !aligned16(w_scale))))
      return FP8BQ_ERR_MISALIGNED;
    st = check_device();
    if (st != FP8BQ_OK) return st;
    if (fp8bq::gemm_splitk_workspace_bytes(M, N, K) > fp8bq::gemm_splitk_scratch_bytes()) return FP8BQ_ERR_SCRATCH;
    clear_last_error();
    return launched(fp8bq::launch_gemm_splitk_noalloc(a_fp8, a_scale, w_fp8, w_scale, y_bf16, M, N, K,
                                                      static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FP8BQ_ERR_LAUNCH;
  }
}

fp8bq_status quantize_act_per_token_group_frag(const uint16_t* x_bf16, uint8_t* x_fp8_frag, float* x_scale,
                                               int64_t M, int64_t K, void* stream) {
  try {
    if (M < 0 || K < 0 || (M % 16) != 0 || (K % 128) != 0) return FP8BQ_ERR_BAD_SHAPE;
    int64_t total, bytes;
    if (!mul_ok(M, K, &total) || !mul_ok(total, 2, &bytes)) return FP8BQ_ERR_BAD_SHAPE;
    if (total == 0) return FP8BQ_OK;
    if (!x_bf16 || !x_fp8_frag || !x_scale) return FP8BQ_ERR_NULL_PTR;
    if (!aligned16(x_bf16) || !aligned16(x_fp8_frag) || !aligned16(x_scale)) return FP8BQ_ERR_MISALIGNED;
    fp8bq_status st = check_device();
    if (st != FP8BQ_OK) return st;
    clear_last_error();
    return launched(
        fp8bq::launch_quant_act_frag(x_bf16, x_fp8_frag, x_scale, M, K, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FP8BQ_ERR_LAUNCH;
  }
}

}  // extern "C"

namespace {

// The GEMMs on fragment-order activations: weights row-major, or (wfrag)
// in fragment order too (N % 16 == 0).
fp8bq_status gemm_frag(const uint8_t* a_fp8_frag, const float* a_scale, const uint8_t* w_fp8, const float* w_scale,
                       uint16_t* y_bf16, int64_t M, int64_t N, int64_t K, bool wfrag, void* stream) {
  try {
    if (M < 0 || N < 0 || K < 0 || (M % 16) != 0 || (K % 128) != 0 || K > kMaxGemmK) return FP8BQ_ERR_BAD_SHAPE;
    if (wfrag && (N % 16) != 0) return FP8BQ_ERR_BAD_SHAPE;
    int64_t mk, nk, mn, bytes;
    if (!mul_ok(M, K, &mk) || !mul_ok(N, K, &nk) || !mul_ok(M, N, &mn) || !mul_ok(mn, 2, &bytes))
      return FP8BQ_ERR_BAD_SHAPE;
    if (mn == 0) return FP8BQ_OK;
    if (!y_bf16) return FP8BQ_ERR_NULL_PTR;
    if (K > 0 && (!a_fp8_frag || !a_scale || !w_fp8 || !w_scale)) return FP8BQ_ERR_NULL_PTR;
    if (!aligned16(y_bf16) || (K > 0 && (!aligned16(a_fp8_frag) || !aligned16(a_scale) || !aligned16(w_fp8) ||
                                         !aligned16(w_scale))))
      return FP8BQ_ERR_MISALIGNED;
    fp8bq_status st = check_device();
    if (st != FP8BQ_OK) return st;
    clear_last_error();
    return launched(fp8bq::launch_gemm_afrag(a_fp8_frag, a_scale, w_fp8, w_scale, y_bf16, M, N, K, wfrag,
                                             static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FP8BQ_ERR_LAUNCH;
  }
}

}  // namespace

extern "C" {

fp8bq_status gemm_w8a8_blockscaled_afrag(const uint8_t* a_fp8_frag, const float* a_scale, const uint8_t* w_fp8,
                                         const float* w_scale, uint16_t* y_bf16, int64_t M, int64_t N, int64_t K,
                                         void* stream) {
  return gemm_frag(a_fp8_frag, a_scale, w_fp8, w_scale, y_bf16, M, N, K, false, stream);
}

fp8bq_status gemm_w8a8_blockscaled_frag(const uint8_t* a_fp8_frag, const float* a_scale, const uint8_t* w_fp8_frag,
                                        const float* w_scale, uint16_t* y_bf16, int64_t M, int64_t N, int64_t K,
                                        void* stream) {
  return gemm_frag(a_fp8_frag, a_scale, w_fp8_frag, w_scale, y_bf16, M, N, K, true, stream);
}

}  // extern "C"

namespace {

// The grouped GEMMs: plain (a_fp8 has M_total rows) or gathered (output row
// m reads row a_rows[m] / a_row_div of the M_a rows of a_fp8).
fp8bq_status grouped_gemm(bool gather, const uint8_t* a_fp8, const float* a_scale, int64_t M_a,
                          const int32_t* a_rows, int64_t a_row_div, const uint8_t* w_fp8, const float* w_scale,
                          const int32_t* group_offsets, uint16_t* y_bf16, int64_t M_total, int64_t N, int64_t K,
                          int64_t G, int tile, void* stream) {
  try {
    if (tile != FP8BQ_TILE_AUTO && tile != FP8BQ_TILE_WIDE && tile != FP8BQ_TILE_DECODE_PANEL &&
        tile != FP8BQ_TILE_DEEP && tile != FP8BQ_TILE_DEEP_PERSISTENT)
      return FP8BQ_ERR_BAD_ARG;
    if (!gather) {
      M_a = M_total;
      a_row_div = 1;
    }
    if (M_a < 0 || M_total < 0 || N < 0 || K < 0 || G < 0 || (K % 128) != 0 || K > kMaxGemmK)
      return FP8BQ_ERR_BAD_SHAPE;
    if (a_row_div < 1 || a_row_div > 0x7fffffffLL) return FP8BQ_ERR_BAD_SHAPE;
    int64_t ak, nk, gnk, mn, bytes;
    if (!mul_ok(M_a, K, &ak) || !mul_ok(N, K, &nk) || !mul_ok(nk, G, &gnk) || !mul_ok(M_total, N, &mn) ||
        !mul_ok(mn, 2, &bytes))
      return FP8BQ_ERR_BAD_SHAPE;
    if (gather && ak >= (int64_t(1) << 31)) return FP8BQ_ERR_BAD_SHAPE;
    if (G > 0 && M_total + 128 * G > 0x7fffffffLL) return FP8BQ_ERR_BAD_SHAPE;
    if (mn == 0) return FP8BQ_OK;
    if (G == 0) return FP8BQ_ERR_BAD_SHAPE;  // rows to produce but no expert to own them
    if (!y_bf16 || !group_offsets || (gather && !a_rows)) return FP8BQ_ERR_NULL_PTR;
    if (K > 0 && (!w_fp8 || !w_scale || (M_a > 0 && (!a_fp8 || !a_scale)))) return FP8BQ_ERR_NULL_PTR;
    if (!aligned16(y_bf16) || (gather && !aligned16(a_rows)) ||
        (K > 0 && (!aligned16(w_fp8) || !aligned16(w_scale) || (M_a > 0 && (!aligned16(a_fp8) || !aligned16(a_scale))))))
      return FP8BQ_ERR_MISALIGNED;
    if ((reinterpret_cast<uintptr_t>(group_offsets) & (gather ? 15u : 3u)) != 0) return FP8BQ_ERR_MISALIGNED;
    fp8bq_status st = check_device();
    if (st != FP8BQ_OK) return st;
    st = check_offsets_if_asked(group_offsets, G, M_total, static_cast<hipStream_t>(stream));
    if (st != FP8BQ_OK) return st;
    clear_last_error();
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (gather)
      return launched(fp8bq::launch_grouped_gemm_gather(a_fp8, a_scale, a_rows, a_row_div, M_a, w_fp8, w_scale,
                                                        group_offsets, y_bf16, M_total, N, K, G, tile, s));
    return launched(fp8bq::launch_grouped_gemm(a_fp8, a_scale, w_fp8, w_scale, group_offsets, y_bf16, M_total, N, K,
                                               G, tile, s));
  } catch (...) {
    return FP8BQ_ERR_LAUNCH;
  }
}

}  // namespace

extern "C" {

fp8bq_status grouped_gemm_w8a8_blockscaled_gather_silu(const uint8_t* a_fp8, const float* a_scale, int64_t M_a,
                                                       const int32_t* a_rows, int64_t a_row_div, const uint8_t* w_fp8,
                                                       const float* w_scale, const int32_t* group_offsets,
                                                       uint8_t* h_fp8, float* h_scale, int64_t M_total, int64_t F,
                                                       int64_t K, int64_t G, void* stream) {
  try {
    if (M_a < 0 || M_total < 0 || F < 0 || K <= 0 || G < 0 || (F % 128) != 0 || (K % 128) != 0 || K > kMaxGemmK)
      return FP8BQ_ERR_BAD_SHAPE;
    if (a_row_div < 1 || a_row_div > 0x7fffffffLL || G > 1024) return FP8BQ_ERR_BAD_SHAPE;
    int64_t ak, fk, gfk, mf;
    if (!mul_ok(M_a, K, &ak) || !mul_ok(F + 128, K, &fk) || !mul_ok(M_total, F, &mf)) return FP8BQ_ERR_BAD_SHAPE;
    if (ak >= (int64_t(1) << 31) || fk >= (int64_t(1) << 31)) return FP8BQ_ERR_BAD_SHAPE;
    if (!mul_ok(2 * fk, G, &gfk)) return FP8BQ_ERR_BAD_SHAPE;  // 2 fk < 2^32: no overflow
    if (G > 0 && M_total + 128 * G > 0x7fffffffLL) return FP8BQ_ERR_BAD_SHAPE;
    if (mf == 0) return FP8BQ_OK;
    if (G == 0) return FP8BQ_ERR_BAD_SHAPE;  // rows to produce but no expert to own them
    if (!h_fp8 || !h_scale || !group_offsets || !a_rows || !w_fp8 || !w_scale) return FP8BQ_ERR_NULL_PTR;
    if (M_a > 0 && (!a_fp8 || !a_scale)) return FP8BQ_ERR_NULL_PTR;
    if (!aligned16(h_fp8) || !aligned16(h_scale) || !aligned16(a_rows) || !aligned16(w_fp8) || !aligned16(w_scale) ||
        !aligned16(group_offsets) || (M_a > 0 && (!aligned16(a_fp8) || !aligned16(a_scale))))
      return FP8BQ_ERR_MISALIGNED;
    fp8bq_status st = check_device();
    if (st != FP8BQ_OK) return st;
    st = check_offsets_if_asked(group_offsets, G, M_total, static_cast<hipStream_t>(stream));
    if (st != FP8BQ_OK) return st;
    clear_last_error();
    return launched(fp8bq::launch_grouped_gemm_gather_silu(a_fp8, a_scale, a_rows, a_row_div, M_a, w_fp8, w_scale,
                                                           group_offsets, h_fp8, h_scale, M_total, F, K, G,
                                                           static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FP8BQ_ERR_LAUNCH;
  }
}

fp8bq_status grouped_gemm_w8a8_blockscaled_tile(const uint8_t* a_fp8, const float* a_scale, int64_t M_a,
                                                const int32_t* a_rows, int64_t a_row_div, const uint8_t* w_fp8,
                                                const float* w_scale, const int32_t* group_offsets,
                                                uint16_t* y_bf16, int64_t M_total, int64_t N, int64_t K, int64_t G,
                                                int tile, void* stream) {
  return grouped_gemm(a_rows != nullptr, a_fp8, a_scale, M_a, a_rows, a_row_div, w_fp8, w_scale, group_offsets,
                      y_bf16, M_total, N, K, G, tile, stream);
}

fp8bq_status grouped_gemm_w8a8_blockscaled(const uint8_t* a_fp8, const float* a_scale, const uint8_t* w_fp8,
                                           const float* w_scale, const int32_t* group_offsets, uint16_t* y_bf16,
                                           int64_t M_total, int64_t N, int64_t K, int64_t G, void* stream) {
  return grouped_gemm(false, a_fp8, a_scale, M_total, nullptr, 1, w_fp8, w_scale, group_offsets, y_bf16, M_total, N,
                      K, G, FP8BQ_TILE_AUTO, stream);
}

fp8bq_status grouped_gemm_w8a8_blockscaled_gather(const uint8_t* a_fp8, const float* a_scale, int64_t M_a,
                                                  const int32_t* a_rows, int64_t a_row_div, const uint8_t* w_fp8,
                                                  const float* w_scale, const int32_t* group_offsets,
                                                  uint16_t* y_bf16, int64_t M_total, int64_t N, int64_t K, int64_t G,
                                                  void* stream) {
  return grouped_gemm(true, a_fp8, a_scale, M_a, a_rows, a_row_div, w_fp8, w_scale, group_offsets, y_bf16, M_total,
                      N, K, G, FP8BQ_TILE_AUTO, stream);
}

fp8bq_status fp8bq_check_group_offsets(const int32_t* group_offsets, int64_t G, int64_t M_total, void* stream) {
  try {
    if (G < 1 || G > 0x7fffffffLL || M_total < 0) return FP8BQ_ERR_BAD_SHAPE;
    if (!group_offsets) return FP8BQ_ERR_NULL_PTR;
    if ((reinterpret_cast<uintptr_t>(group_offsets) & 3u) != 0) return FP8BQ_ERR_MISALIGNED;
    fp8bq_status st = check_device();
    if (st != FP8BQ_OK) return st;
    return check_offsets(group_offsets, G, M_total, static_cast<hipStream_t>(stream));
  } catch (...) {
    return FP8BQ_ERR_LAUNCH;
  }
}

fp8bq_status fp8bq_encode_e4m3(const float* in, uint8_t* out, int64_t n, int method, void* stream) {
  try {
    if (n < 0 || method < 0 || method > 2) return FP8BQ_ERR_BAD_SHAPE;
    if (n == 0) return FP8BQ_OK;
    if (!in || !out) return FP8BQ_ERR_NULL_PTR;
    if (!aligned16(in) || !aligned16(out)) return FP8BQ_ERR_MISALIGNED;
    fp8bq_status st = check_device();
    if (st != FP8BQ_OK) return st;
    clear_last_error();
    return launched(fp8bq::launch_encode(in, out, n, method, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FP8BQ_ERR_LAUNCH;
  }
}

fp8bq_status token_importance_weights(const float* logp_train, const float* logp_rollout, const uint8_t* mask,
                                      const float* advantages, float* weights, float* weighted_adv, int64_t n,
                                      float C, int mode, void* stream) {
  try {
    if (!(C >= 1.0f) || (mode != FP8BQ_IW_TIS && mode != FP8BQ_IW_MIS)) return FP8BQ_ERR_BAD_ARG;
    if ((advantages == nullptr) != (weighted_adv == nullptr)) return FP8BQ_ERR_BAD_ARG;
    if (n < 0 || n > kMaxElementwise) return FP8BQ_ERR_BAD_SHAPE;
    if (n == 0) return FP8BQ_OK;
    if (!logp_train || !logp_rollout || !weights) return FP8BQ_ERR_NULL_PTR;
    if (!aligned16(logp_train) || !aligned16(logp_rollout) || !aligned16(weights) ||
        (mask && !aligned16(mask)) || (advantages && (!aligned16(advantages) || !aligned16(weighted_adv))))
      return FP8BQ_ERR_MISALIGNED;
    fp8bq_status st = check_device();
    if (st != FP8BQ_OK) return st;
    // clip bounds and the MIS band edge, each rounded once to float32
    const float lo = 1.0f / C;
    const float log_c = static_cast<float>(std::log(static_cast<double>(C)));
    clear_last_error();
    return launched(fp8bq::launch_importance_weights(logp_train, logp_rollout, mask, advantages, weights,
                                                     weighted_adv, n, lo, C, log_c, mode == FP8BQ_IW_MIS,
                                                     static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FP8BQ_ERR_LAUNCH;
  }
}

fp8bq_status moe_sort_by_expert(const int32_t* topk_ids, int64_t T, int64_t k, int64_t E, int32_t* group_offsets,
                                int32_t* sorted_pair, int32_t* pair_row, void* stream) {
  try {
    if (T < 0 || k < 0 || E < 1 || E > 0x7fffffffLL) return FP8BQ_ERR_BAD_SHAPE;
    int64_t P;
    if (!mul_ok(T, k, &P) || P > 0x7fffffffLL) return FP8BQ_ERR_BAD_SHAPE;
    if (!group_offsets || (P > 0 && (!topk_ids || !sorted_pair || !pair_row))) return FP8BQ_ERR_NULL_PTR;
    if (!aligned16(group_offsets) || (P > 0 && (!aligned16(topk_ids) || !aligned16(sorted_pair) ||
                                                !aligned16(pair_row))))
      return FP8BQ_ERR_MISALIGNED;
    fp8bq_status st = check_device();
    if (st != FP8BQ_OK) return st;
    clear_last_error();
    return launched(fp8bq::launch_moe_sort(topk_ids, P, E, group_offsets, sorted_pair, pair_row,
                                           static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FP8BQ_ERR_LAUNCH;
  }
}

fp8bq_status moe_gather_quantize_act(const uint16_t* x_bf16, const int32_t* sorted_pair, int64_t rows, int64_t T,
                                     int64_t k, int64_t K, uint8_t* a_fp8, float* a_scale, void* stream) {
  try {
    if (rows < 0 || T < 0 || k < 1 || K < 0 || (K % 128) != 0) return FP8BQ_ERR_BAD_SHAPE;
    int64_t rk, tk, bytes;
    if (!mul_ok(rows, K, &rk) || !mul_ok(T, K, &tk) || !mul_ok(tk, 2, &bytes) || k > 0x7fffffffLL)
      return FP8BQ_ERR_BAD_SHAPE;
    if (rk == 0) return FP8BQ_OK;
    if (!sorted_pair || !a_fp8 || !a_scale || (T > 0 && !x_bf16)) return FP8BQ_ERR_NULL_PTR;
    if (!aligned16(sorted_pair) || !aligned16(a_fp8) || !aligned16(a_scale) || (T > 0 && !aligned16(x_bf16)))
      return FP8BQ_ERR_MISALIGNED;
    fp8bq_status st = check_device();
    if (st != FP8BQ_OK) return st;
    clear_last_error();
    return launched(fp8bq::launch_gather_quant_act(x_bf16, sorted_pair, rows, T, k, K, a_fp8, a_scale,
                                                   static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FP8BQ_ERR_LAUNCH;
  }
}

fp8bq_status silu_mul_quantize_act(const uint16_t* y_bf16, int64_t M, int64_t F, uint8_t* h_fp8, float* h_scale,
                                   uint16_t* h_bf16, void* stream) {
  try {
    if (M < 0 || F < 0 || (F % 8) != 0) return FP8BQ_ERR_BAD_SHAPE;
    int64_t mf, bytes;
    if (!mul_ok(M, F, &mf) || !mul_ok(mf, 4, &bytes)) return FP8BQ_ERR_BAD_SHAPE;
    if (mf == 0) return FP8BQ_OK;
    if (!y_bf16 || !h_fp8 || !h_scale) return FP8BQ_ERR_NULL_PTR;
    if (!aligned16(y_bf16) || !aligned16(h_fp8) || !aligned16(h_scale) || (h_bf16 && !aligned16(h_bf16)))
      return FP8BQ_ERR_MISALIGNED;
    fp8bq_status st = check_device();
    if (st != FP8BQ_OK) return st;
    clear_last_error();
    return launched(
        fp8bq::launch_silu_mul_quant(y_bf16, M, F, h_fp8, h_scale, h_bf16, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FP8BQ_ERR_LAUNCH;
  }
}

fp8bq_status moe_combine(const uint16_t* y_bf16, const int32_t* pair_row, const float* topk_weights, int64_t T,
                         int64_t k, int64_t H, int64_t M_rows, uint16_t* out_bf16, void* stream) {
  try {
    if (T < 0 || k < 0 || H < 0 || M_rows < 0 || (H % 8) != 0 || T > 0x7fffffffLL) return FP8BQ_ERR_BAD_SHAPE;
    int64_t tk, th, mh, bytes;
    if (!mul_ok(T, k, &tk) || tk > 0x7fffffffLL || !mul_ok(T, H, &th) || !mul_ok(M_rows, H, &mh) ||
        !mul_ok(mh > th ? mh : th, 2, &bytes))
      return FP8BQ_ERR_BAD_SHAPE;
    if (th == 0) return FP8BQ_OK;
    if (!out_bf16 || (tk > 0 && (!pair_row || !topk_weights)) || (mh > 0 && !y_bf16)) return FP8BQ_ERR_NULL_PTR;
    if (!aligned16(out_bf16) || (tk > 0 && (!aligned16(pair_row) || !aligned16(topk_weights))) ||
        (mh > 0 && !aligned16(y_bf16)))
      return FP8BQ_ERR_MISALIGNED;
    fp8bq_status st = check_device();
    if (st != FP8BQ_OK) return st;
    clear_last_error();
    return launched(fp8bq::launch_moe_combine(y_bf16, pair_row, topk_weights, T, k, H, M_rows, out_bf16,
                                              static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FP8BQ_ERR_LAUNCH;
  }
}

fp8bq_status quantize_weight_blockwise_dual(const uint16_t* w_bf16, uint8_t* w_fp8, float* w_scale, uint8_t* wt_fp8,
                                            float* wt_scale, int64_t batch, int64_t N, int64_t K, void* stream) {
  try {
    if (batch < 0 || N < 0 || K < 0 || (K % 8) != 0 || batch > 65535) return FP8BQ_ERR_BAD_SHAPE;
    if ((w_fp8 == nullptr) != (w_scale == nullptr)) return FP8BQ_ERR_BAD_ARG;
    int64_t nk, total, bytes;
    if (!mul_ok(N, K, &nk) || !mul_ok(nk, batch, &total) || !mul_ok(total, 2, &bytes)) return FP8BQ_ERR_BAD_SHAPE;
    if (total == 0) return FP8BQ_OK;
    if (!w_bf16 || !wt_fp8 || !wt_scale) return FP8BQ_ERR_NULL_PTR;
    if (!aligned16(w_bf16) || !aligned16(wt_fp8) || !aligned16(wt_scale) ||
        (w_fp8 && (!aligned16(w_fp8) || !aligned16(w_scale))))
      return FP8BQ_ERR_MISALIGNED;
    fp8bq_status st = check_device();
    if (st != FP8BQ_OK) return st;
    clear_last_error();
    return launched(fp8bq::launch_quant_weight_dual(w_bf16, w_fp8, w_scale, wt_fp8, wt_scale, batch, N, K,
                                                    static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FP8BQ_ERR_LAUNCH;
  }
}

fp8bq_status quantize_act_dual(const uint16_t* x_bf16, uint8_t* x_fp8, float* x_scale, uint8_t* xt_fp8,
                               float* xt_scale, int64_t M, int64_t K, void* stream) {
  try {
    if (M < 0 || K < 0 || (K % 8) != 0) return FP8BQ_ERR_BAD_SHAPE;
    if ((x_fp8 == nullptr) != (x_scale == nullptr)) return FP8BQ_ERR_BAD_ARG;
    int64_t mk, bytes;
    if (!mul_ok(M, K, &mk) || !mul_ok(mk, 2, &bytes)) return FP8BQ_ERR_BAD_SHAPE;
    if (mk == 0) return FP8BQ_OK;
    if (!x_bf16 || !xt_fp8 || !xt_scale) return FP8BQ_ERR_NULL_PTR;
    if (!aligned16(x_bf16) || !aligned16(xt_fp8) || !aligned16(xt_scale) ||
        (x_fp8 && (!aligned16(x_fp8) || !aligned16(x_scale))))
      return FP8BQ_ERR_MISALIGNED;
    fp8bq_status st = check_device();
    if (st != FP8BQ_OK) return st;
    clear_last_error();
    return launched(
        fp8bq::launch_quant_act_dual(x_bf16, x_fp8, x_scale, xt_fp8, xt_scale, M, K, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FP8BQ_ERR_LAUNCH;
  }
}

// K / V layout checks shared by the two KV-cache entry points.
fp8bq_status kv_shape(int64_t T, int64_t H, int64_t D) {
  if (T < 0 || H < 1 || D < 8 || (D % 8) != 0 || H * D > 8192) return FP8BQ_ERR_BAD_SHAPE;
  int64_t thd, bytes;
  if (!mul_ok(T, H * D, &thd) || !mul_ok(thd, 2, &bytes) || thd > (int64_t(1) << 40)) return FP8BQ_ERR_BAD_SHAPE;
  return FP8BQ_OK;
}

fp8bq_status kv_scale_calibrate(const uint16_t* k_bf16, const uint16_t* v_bf16, int64_t T, int64_t H, int64_t D,
                                int per_head, float* k_scale, float* v_scale, void* stream) {
  try {
    if (per_head != 0 && per_head != 1) return FP8BQ_ERR_BAD_ARG;
    fp8bq_status st = kv_shape(T, H, D);
    if (st != FP8BQ_OK) return st;
    // V takes part when v_scale is given
    if (!v_scale && v_bf16) return FP8BQ_ERR_BAD_ARG;
    if (!k_scale || (T > 0 && (!k_bf16 || (v_scale && !v_bf16)))) return FP8BQ_ERR_NULL_PTR;
    if (!aligned16(k_scale) || (v_scale && !aligned16(v_scale)) ||
        (T > 0 && (!aligned16(k_bf16) || (v_bf16 && !aligned16(v_bf16)))))
      return FP8BQ_ERR_MISALIGNED;
    st = check_device();
    if (st != FP8BQ_OK) return st;
    clear_last_error();
    return launched(fp8bq::launch_kv_calibrate(k_bf16, v_bf16, T, H, D, per_head == 1, k_scale, v_scale,
                                               static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FP8BQ_ERR_LAUNCH;
  }
}

fp8bq_status kv_cache_write_fp8(const uint16_t* k_bf16, const uint16_t* v_bf16, const int32_t* slot_mapping,
                                const float* k_scale, const float* v_scale, int per_head, uint8_t* k_cache,
                                uint8_t* v_cache, int64_t T, int64_t H, int64_t D, int64_t S, void* stream) {
  try {
    if (per_head != 0 && per_head != 1) return FP8BQ_ERR_BAD_ARG;
    // V takes part when v_scale is given
    if (!v_scale && (v_bf16 || v_cache)) return FP8BQ_ERR_BAD_ARG;
    fp8bq_status st = kv_shape(T, H, D);
    if (st != FP8BQ_OK) return st;
    int64_t shd;
    if (S < 0 || S > 0x7fffffffLL || !mul_ok(S, H * D, &shd)) return FP8BQ_ERR_BAD_SHAPE;
    if (T == 0) return FP8BQ_OK;
    if (!k_bf16 || !slot_mapping || !k_scale || (S > 0 && !k_cache)) return FP8BQ_ERR_NULL_PTR;
    if (v_scale && (!v_bf16 || (S > 0 && !v_cache))) return FP8BQ_ERR_NULL_PTR;
    if (!aligned16(k_bf16) || !aligned16(slot_mapping) || !aligned16(k_scale) || (S > 0 && !aligned16(k_cache)) ||
        (v_bf16 && (!aligned16(v_bf16) || !aligned16(v_scale) || (S > 0 && !aligned16(v_cache)))))
      return FP8BQ_ERR_MISALIGNED;
    st = check_device();
    if (st != FP8BQ_OK) return st;
    clear_last_error();
    return launched(fp8bq::launch_kv_write(k_bf16, v_bf16, slot_mapping, k_scale, v_scale, per_head == 1, k_cache,
                                           v_cache, T, H, D, S, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FP8BQ_ERR_LAUNCH;
  }
}

}  // extern "C"
