// Internal launchers: one per kernel family.  Arguments are already
// validated by the C-ABI layer (api.hip); launchers only size the grid.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bq {

// Compute units of the current device, read from its properties once per
// device (0 when they cannot be read).
int device_cus();

// Matrices re-quantized by one launch (passed by value in the kernel
// arguments): desc[t] is an [N][K] BF16 matrix with its outputs; its blocks
// are workgroups first[t] .. first[t + 1] - 1.
constexpr int kMaxWeightDescs = 48;  // FP8BQ_MAX_WEIGHT_DESCS of the C ABI
struct WeightDesc {
  const uint16_t* w;
  uint8_t* q;
  float* s;
  int64_t N, K;
};
struct WeightBatch {
  WeightDesc desc[kMaxWeightDescs];
  int64_t first[kMaxWeightDescs + 1];
  int count;
};

// frag: codes in MFMA fragment order (N % 16 == 0, K % 128 == 0)
hipError_t launch_quant_weight(const uint16_t* w, uint8_t* q, float* scale, int64_t batch, int64_t N, int64_t K,
                               bool frag, hipStream_t stream);

hipError_t launch_quant_weight_multi(const WeightBatch& batch, int64_t blocks, bool frag, hipStream_t stream);

hipError_t launch_quant_act(const uint16_t* x, uint8_t* q, float* scale, int64_t M, int64_t K, hipStream_t stream);

// Activations quantized by one launch (descriptors by value in the kernel
// arguments): desc[t] is an [M][K] BF16 matrix with its outputs; its groups
// go to workgroups first[t] .. first[t + 1] - 1 (32 groups each).
constexpr int kMaxActDescs = 16;  // FP8BQ_MAX_ACT_DESCS of the C ABI
struct ActDesc {
  const uint16_t* x;
  uint8_t* q;
  float* s;
  int64_t M, K;
};
struct ActBatch {
  ActDesc desc[kMaxActDescs];
  int64_t first[kMaxActDescs + 1];
  int count;
};
constexpr int kActGroupsPerWg = 32;

hipError_t launch_quant_act_multi(const ActBatch& batch, int64_t blocks, hipStream_t stream);
// the same in fragment order: first[] counts workgroups of 4 units (16 rows x one K-block)
constexpr int kActFragUnitsPerWg = 4;
hipError_t launch_quant_act_frag_multi(const ActBatch& batch, int64_t blocks, hipStream_t stream);
// the same codes in the MFMA fragment order of the activation operand (M % 16 == 0, K % 128 == 0)
hipError_t launch_quant_act_frag(const uint16_t* x, uint8_t* q, float* scale, int64_t M, int64_t K,
                                 hipStream_t stream);
// the GEMM on fragment-order activations (M % 16 == 0, K % 128 == 0); wfrag:
// fragment-order weights too (N % 16 == 0)
hipError_t launch_gemm_afrag(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw, uint16_t* y,
                             int64_t M, int64_t N, int64_t K, bool wfrag, hipStream_t stream);

// `tile`: FP8BQ_TILE_* of the C ABI (0 = the cost model's choice); an
// unknown value returns hipErrorInvalidValue.
hipError_t launch_gemm(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw, uint16_t* y, int64_t M,
                       int64_t N, int64_t K, int tile, hipStream_t stream);

// The K-split form for few activation rows: workspace bytes it needs for
// this shape on the current device (0: it runs the unsplit GEMM), and the
// launch (hipErrorInvalidValue when the workspace is smaller).
int64_t gemm_splitk_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_splitk(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw, uint16_t* y,
                              int64_t M, int64_t N, int64_t K, void* workspace, int64_t workspace_bytes,
                              hipStream_t stream);

// The K split with the library's static scratch instead of a workspace:
// its size, and the launch (hipErrorInvalidValue when the shape needs more).
int64_t gemm_splitk_scratch_bytes();
hipError_t launch_gemm_splitk_noalloc(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw,
                                      uint16_t* y, int64_t M, int64_t N, int64_t K, hipStream_t stream);

hipError_t launch_grouped_gemm(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw,
                               const int32_t* offsets, uint16_t* y, int64_t M, int64_t N, int64_t K, int64_t G,
                               int tile, hipStream_t stream);

// The MoE fc1 GEMM (weights [G][2F][K] = [gate; up] per expert, rows
// gathered as in launch_grouped_gemm_gather) with h = SiLU(gate) * up
// quantized in 1x128 groups in its epilogue: codes hq [M][F], scales
// hs [M][F/128] (F % 128 == 0, K > 0, G <= 1024).
hipError_t launch_grouped_gemm_gather_silu(const uint8_t* a, const float* sa, const int32_t* a_rows, int64_t a_div,
                                           int64_t a_nrows, const uint8_t* w, const float* sw, const int32_t* offsets,
                                           uint8_t* hq, float* hs, int64_t M, int64_t F, int64_t K, int64_t G,
                                           hipStream_t stream);
hipError_t launch_grouped_gemm_gather(const uint8_t* a, const float* sa, const int32_t* a_rows, int64_t a_div,
                                      int64_t a_nrows, const uint8_t* w, const float* sw, const int32_t* offsets,
                                      uint16_t* y, int64_t M, int64_t N, int64_t K, int64_t G, int tile,
                                      hipStream_t stream);

hipError_t launch_encode(const float* in, uint8_t* out, int64_t n, int method, hipStream_t stream);

hipError_t launch_importance_weights(const float* logp_train, const float* logp_rollout, const uint8_t* mask,
                                     const float* advantages, float* weights, float* weighted_adv, int64_t n,
                                     float lo, float hi, float log_c, bool mis, hipStream_t stream);

hipError_t launch_moe_sort(const int32_t* ids, int64_t P, int64_t E, int32_t* offsets, int32_t* sorted_pair,
                           int32_t* pair_row, hipStream_t stream);

hipError_t launch_gather_quant_act(const uint16_t* x, const int32_t* sorted_pair, int64_t R, int64_t T, int64_t k,
                                   int64_t K, uint8_t* q, float* scale, hipStream_t stream);

hipError_t launch_silu_mul_quant(const uint16_t* y, int64_t M, int64_t F, uint8_t* q, float* scale, uint16_t* h,
                                 hipStream_t stream);

hipError_t launch_moe_combine(const uint16_t* y, const int32_t* pair_row, const float* w, int64_t T, int64_t k,
                              int64_t H, int64_t M, uint16_t* out, hipStream_t stream);

hipError_t launch_kv_calibrate(const uint16_t* k, const uint16_t* v, int64_t T, int64_t H, int64_t D, bool per_head,
                               float* ks, float* vs, hipStream_t stream);

hipError_t launch_kv_write(const uint16_t* k, const uint16_t* v, const int32_t* slots, const float* ks,
                           const float* vs, bool per_head, uint8_t* kc, uint8_t* vc, int64_t T, int64_t H, int64_t D,
                           int64_t S, hipStream_t stream);

hipError_t launch_quant_weight_dual(const uint16_t* w, uint8_t* q, float* s, uint8_t* qt, float* st, int64_t batch,
                                    int64_t N, int64_t K, hipStream_t stream);

hipError_t launch_quant_act_dual(const uint16_t* x, uint8_t* q, float* s, uint8_t* qt, float* st, int64_t M,
                                 int64_t K, hipStream_t stream);

}  // namespace fp8bq
