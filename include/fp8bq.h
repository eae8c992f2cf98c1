/*
 * fp8bq.h -- C ABI of libfp8bq.so: blockwise W8A8 FP8 quantization and
 * block-scaled FP8 GEMMs for AMD Instinct MI355X (gfx950).
 *
 * The operations are the linear-layer hot path of FP8 rollout in LLM
 * reinforcement learning as described on the page "FP8-RL: A Practical and
 * Stable Low-Precision Stack for LLM Reinforcement Learning" (paper-graph-ui
 * summary; cited below as [FP8-RL summary]):
 *   - §3.4.2 Phase 2 step 2: per RL step, every 128x128 block of each
 *     quantized BF16 weight matrix gets a scale from its maximum absolute
 *     value, is divided by that scale and rounded to the nearest E4M3 value;
 *   - §3.4.1 "Static vs. Dynamic Quantization" and §3.4.2 Phase 3:
 *     activations are quantized on the fly per token in 1x128 tiles, the
 *     FP8 x FP8 product is accumulated in FP32 and converted back to BF16;
 *   - §3.4.1 "Quantization Scope": MoE expert layers (fc1/fc2) use the same
 *     scheme, which makes the expert GEMMs a ragged grouped GEMM.
 * The [128, 128] weight / [1, 128] activation granularity is also the one of
 * the news page "How FP8 Reinforcement Learning Accelerates LLMs Without
 * Crashing", section "End-to-End Precision Recipes Across Generation and
 * Training Engines".
 *
 * Number formats
 *   BF16 : uint16_t bit patterns (upper half of an IEEE binary32).
 *   E4M3 : uint8_t codes, OCP "e4m3fn": 1 sign, 4 exponent bits (bias 7),
 *          3 mantissa bits, no infinity, 0x7F/0xFF = NaN, max +-448
 *          ([FP8-RL summary] §3.4.1 "Quantization Format and Granularity").
 *          Encoding is round-to-nearest-even with saturation at +-448; the
 *          library never writes 0x7F/0xFF.
 *   Scales: IEEE float32, one per tile: s = fl32(amax / 448.0f).  A tile
 *          whose amax is 0 gets s = 0 and codes 0x00 / 0x80 (the sign of
 *          each input zero).  Quantized value: q = E4M3(fl32(x / s)) with
 *          the IEEE float32 quotient.  FP32 denormals are never flushed.
 *
 * Conventions (all functions)
 *   - Every tensor pointer is a DEVICE pointer to row-major, contiguous
 *     memory on the current HIP device, aligned to 16 bytes.  The caller
 *     allocates and frees every buffer; the library keeps no pointer.
 *     Outputs must not overlap inputs.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default
 *     stream).  Calls enqueue work and return without waiting; results are
 *     ready when the stream reaches that point.
 *   - Arguments are checked before anything is enqueued.  On error nothing
 *     is enqueued and a non-zero fp8bq_status is returned.  A zero-sized
 *     problem is a successful no-op.  No C++ exception crosses the ABI.
 *   - Quantizer and GEMM inputs must be finite (NaN / Inf input gives
 *     unspecified codes).
 *   - Functions are thread-safe; ordering follows the stream.
 */
#ifndef FP8BQ_H
#define FP8BQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int fp8bq_status;

enum {
  FP8BQ_OK = 0,
  FP8BQ_ERR_NULL_PTR = 1,   /* a required pointer is NULL while its size is > 0 */
  FP8BQ_ERR_BAD_SHAPE = 2,  /* negative size, GEMM K % 128 != 0 or K > 2^22, size overflow */
  FP8BQ_ERR_MISALIGNED = 3, /* a tensor pointer is not 16-byte aligned */
  FP8BQ_ERR_LAUNCH = 4,     /* the HIP runtime rejected a kernel launch */
  FP8BQ_ERR_DEVICE = 5,     /* the current device is not gfx950, or no device */
  FP8BQ_ERR_BAD_ARG = 6,    /* an invalid scalar argument or option combination */
  FP8BQ_ERR_WORKSPACE = 7,  /* the workspace is missing, misaligned or smaller than the call needs */
  FP8BQ_ERR_SCRATCH = 8     /* the call needs more than the library's static scratch (FP8BQ_SCRATCH_BYTES) */
};

/* Static, human-readable text for a status code (host function). */
const char* fp8bq_status_string(fp8bq_status s);

/*
 * quantize_weight_blockwise -- per-step re-quantization of BF16 weights.
 * [FP8-RL summary] §3.4.1 formula W^_ij = round(W_ij / scale_ij) with one
 * scale per 128x128 block chosen so the block maximum maps to 448, applied
 * per RL step as in §3.4.2 Phase 2 step 2.
 *
 *   w_bf16  [batch][N][K]  BF16 input (N = out features, K = in features)
 *   w_fp8   [batch][N][K]  E4M3 output
 *   w_scale [batch][ceil(N/128)][ceil(K/128)]  float32 output
 *   batch, N, K >= 0.  Blocks are aligned at (0, 0); edge blocks of an N or
 *   K that is not a multiple of 128 are partial (their amax covers the
 *   in-bounds elements).  The batch dimension quantizes `batch` matrices of
 *   the same shape in one call (e.g. the same projection of every layer).
 */
fp8bq_status quantize_weight_blockwise(const uint16_t* w_bf16, uint8_t* w_fp8, float* w_scale,
                                       int64_t batch, int64_t N, int64_t K, void* stream);

/*
 * quantize_weights_blockwise_multi -- quantize_weight_blockwise of several
 * matrices of any shapes in one launch (a weight sync re-quantizes many
 * parameter tensors per RL step; one launch avoids a ramp and a tail per
 * tensor).  Each matrix gets exactly the codes and scales
 * quantize_weight_blockwise gives it.
 *   descs  HOST array of `count` descriptors (read during the call only):
 *          w_bf16 [N][K] BF16, w_fp8 [N][K] E4M3, w_scale
 *          [ceil(N/128)][ceil(K/128)] float32, N, K >= 0, each validated as
 *          in quantize_weight_blockwise (empty matrices are skipped).
 *   0 <= count <= FP8BQ_MAX_WEIGHT_DESCS; the matrices must not overlap.
 */
#define FP8BQ_MAX_WEIGHT_DESCS 48
typedef struct {
  const uint16_t* w_bf16;
  uint8_t* w_fp8;
  float* w_scale;
  int64_t N;
  int64_t K;
} fp8bq_weight_desc;

fp8bq_status quantize_weights_blockwise_multi(const fp8bq_weight_desc* descs, int64_t count, void* stream);

/*
 * quantize_weight_blockwise_frag / quantize_weights_blockwise_frag_multi --
 * the same re-quantization ([FP8-RL summary] §3.4.1 formula for W^, §3.4.2
 * Phase 2 step 2), with the codes written in the MFMA fragment order that
 * gemm_w8a8_blockscaled_frag reads (the pages fix the values and scales,
 * not the byte layout of the quantized weights; a weight that is
 * re-quantized every step can be stored the way the GEMM reads it).
 *   Fragment order of an [N][K] code matrix (N % 16 == 0, K % 128 == 0):
 *   code (n, k) at byte
 *     ((n/16 * (K/128) + k/128) * 2 + (k%128)/64) * 1024
 *       + (((k%64)/16) * 16 + n%16) * 16 + k%16,
 *   i.e. one 2 KB unit per 16 rows and 128-wide K-block, in it lane
 *   l = 16 c + r of the 16x16x128 FP8 MFMA finds its operand bytes at l*16
 *   (k = 16 c ..) and 1024 + l*16 (k = 64 + 16 c ..).  Same layout as the
 *   activations of quantize_act_per_token_group_frag.
 *   Arguments, scales and errors as for quantize_weight_blockwise /
 *   quantize_weights_blockwise_multi, plus FP8BQ_ERR_BAD_SHAPE unless every
 *   matrix has N % 16 == 0 and K % 128 == 0.  Each matrix gets exactly the
 *   row-major codes permuted into that order, and the same scales.
 */
fp8bq_status quantize_weight_blockwise_frag(const uint16_t* w_bf16, uint8_t* w_fp8_frag, float* w_scale,
                                            int64_t batch, int64_t N, int64_t K, void* stream);
fp8bq_status quantize_weights_blockwise_frag_multi(const fp8bq_weight_desc* descs, int64_t count, void* stream);

/*
 * quantize_act_per_token_group -- dynamic per-token 1x128 quantization of
 * BF16 activations ([FP8-RL summary] §3.4.1, "1 x 128 tiles for
 * activations", and §3.4.2 Phase 3, scales computed on the fly).
 *
 *   x_bf16  [M][K]  BF16 input (M tokens)
 *   x_fp8   [M][K]  E4M3 output
 *   x_scale [M][ceil(K/128)]  float32 output, token-major
 *   M, K >= 0.  Group g of token m covers columns [128 g, min(K, 128 g + 128)).
 */
fp8bq_status quantize_act_per_token_group(const uint16_t* x_bf16, uint8_t* x_fp8, float* x_scale,
                                          int64_t M, int64_t K, void* stream);

/*
 * quantize_acts_per_token_group_multi -- quantize_act_per_token_group of
 * several activations of any shapes in one launch (a decode step quantizes
 * the small inputs of several linears per layer; at a few MB each, one
 * launch per activation is latency-bound).  Each activation gets exactly the
 * codes and scales quantize_act_per_token_group gives it.
 *   descs  HOST array of `count` descriptors (read during the call only):
 *          x_bf16 [M][K] BF16, x_fp8 [M][K] E4M3, x_scale [M][ceil(K/128)]
 *          float32, M, K >= 0, each validated as in
 *          quantize_act_per_token_group (empty ones are skipped).
 *   0 <= count <= FP8BQ_MAX_ACT_DESCS; outputs must not overlap.
 */
#define FP8BQ_MAX_ACT_DESCS 16
typedef struct {
  const uint16_t* x_bf16;
  uint8_t* x_fp8;
  float* x_scale;
  int64_t M;
  int64_t K;
} fp8bq_act_desc;

fp8bq_status quantize_acts_per_token_group_multi(const fp8bq_act_desc* descs, int64_t count, void* stream);

/*
 * quantize_acts_per_token_group_frag_multi -- quantize_act_per_token_group_frag
 * of several activations in one launch (the decode step's inputs of the
 * fragment-order GEMMs).  Same descriptors and limits as
 * quantize_acts_per_token_group_multi, codes in fragment order; each
 * activation needs M % 16 == 0 and K % 128 == 0 (FP8BQ_ERR_BAD_SHAPE
 * otherwise) and gets exactly the codes and scales
 * quantize_act_per_token_group_frag gives it.
 */
fp8bq_status quantize_acts_per_token_group_frag_multi(const fp8bq_act_desc* descs, int64_t count, void* stream);

/*
 * gemm_w8a8_blockscaled -- y = dequant(A) * dequant(W)^T in FP32, stored as
 * BF16 ([FP8-RL summary] §3.4.2 Phase 3: FP8 matrix multiplication,
 * accumulated in FP32, converted back to BF16).
 *
 *   a_fp8   [M][K]  E4M3 activations      a_scale [M][K/128]          float32
 *   w_fp8   [N][K]  E4M3 weights          w_scale [ceil(N/128)][K/128] float32
 *   y_bf16  [M][N]  BF16 output (round to nearest even)
 *   y[m][n] = sum_k (a_scale[m][k/128] * dec(a[m][k])) * (w_scale[n/128][k/128] * dec(w[n][k]))
 *   M, N >= 0; 0 <= K <= 2^22 and K % 128 == 0 (the kernels address a
 *   256-row operand panel with 32-bit offsets).  The summation order is
 *   unspecified (results agree with the exact value to FP32 accumulation
 *   error before the BF16 rounding).
 *   The tile kernel is chosen per shape by a cost model over the device's
 *   CU count; gemm_w8a8_blockscaled_tile runs a named one.
 */
fp8bq_status gemm_w8a8_blockscaled(const uint8_t* a_fp8, const float* a_scale, const uint8_t* w_fp8,
                                   const float* w_scale, uint16_t* y_bf16, int64_t M, int64_t N, int64_t K,
                                   void* stream);

/*
 * Tile kernels of the GEMMs, for tests and diagnostics (the *_tile entry
 * points).  FP8BQ_TILE_AUTO is the choice the plain entry points make.
 *   dense:   SKINNY64, SKINNY48, SKINNY96 (K split over the 4 waves of a
 *            64 / 48 / 96 x 64 tile), WIDE (256 x 256), DECODE_PANEL
 *            (128 x 256), DEEP (256 x 128, three stages), PANEL192 (192 x 128)
 *   grouped: WIDE, DECODE_PANEL, DEEP (one workgroup per tile),
 *            DEEP_PERSISTENT (one workgroup per CU; the default, used for
 *            G <= 1024 only, above that the per-tile DEEP kernel runs)
 */
enum {
  FP8BQ_TILE_AUTO = 0,
  FP8BQ_TILE_SKINNY64 = 1,
  FP8BQ_TILE_SKINNY48 = 2,
  FP8BQ_TILE_WIDE = 3,
  FP8BQ_TILE_DECODE_PANEL = 4,
  FP8BQ_TILE_DEEP = 5,
  FP8BQ_TILE_PANEL192 = 6,
  FP8BQ_TILE_DEEP_PERSISTENT = 7,
  FP8BQ_TILE_SKINNY96 = 8
};

/*
 * gemm_w8a8_blockscaled_tile -- gemm_w8a8_blockscaled with the tile kernel
 * named by `tile` (a dense FP8BQ_TILE_* value; DEEP_PERSISTENT is grouped
 * only).  Same contract and the same result bits for a given tile; another
 * tile may sum in another order.  An unknown tile is FP8BQ_ERR_BAD_ARG.
 */
fp8bq_status gemm_w8a8_blockscaled_tile(const uint8_t* a_fp8, const float* a_scale, const uint8_t* w_fp8,
                                        const float* w_scale, uint16_t* y_bf16, int64_t M, int64_t N, int64_t K,
                                        int tile, void* stream);

/*
 * gemm_w8a8_blockscaled_splitk -- gemm_w8a8_blockscaled for few activation
 * rows, with K split over more workgroups ([FP8-RL summary] §3.4.2 Phase
 * 3: every decode step runs the FP8 GEMMs of each layer on a few hundred
 * tokens).  With M <= 256 every activation row fits one 256-row panel, so
 * each weight byte is read by one workgroup; when the 128-row weight tiles
 * are too few to fill the CUs, K is split into S <= 8 pieces of whole
 * K-blocks, each piece's FP32 partial tile goes to the workspace, and a
 * second kernel sums the S partials in piece order and rounds once to
 * BF16.  The result is deterministic (fixed pieces, fixed order) and meets
 * the contract of gemm_w8a8_blockscaled (only the FP32 summation order
 * differs).  Shapes that do not split run gemm_w8a8_blockscaled itself and
 * need no workspace.
 *   a_fp8 ... M, N, K  as for gemm_w8a8_blockscaled
 *   workspace        DEVICE memory of workspace_bytes bytes, 16-byte
 *                    aligned, owned by the caller; its contents on entry do
 *                    not matter and are overwritten; it must not be used by
 *                    other work until the stream has passed this call
 *   workspace_bytes  at least what gemm_w8a8_blockscaled_splitk_workspace
 *                    gives for (M, N, K) (S * M * N * 4 bytes; at most
 *                    32 MiB on a 256-CU device), else FP8BQ_ERR_WORKSPACE
 */
fp8bq_status gemm_w8a8_blockscaled_splitk(const uint8_t* a_fp8, const float* a_scale, const uint8_t* w_fp8,
                                          const float* w_scale, uint16_t* y_bf16, int64_t M, int64_t N, int64_t K,
                                          void* workspace, int64_t workspace_bytes, void* stream);

/*
 * gemm_w8a8_blockscaled_splitk_workspace -- the workspace bytes
 * gemm_w8a8_blockscaled_splitk needs for (M, N, K) on the current device
 * (the split depends on its CU count), written to *bytes (0: no split).
 * The shape is checked as in gemm_w8a8_blockscaled.  Host only; launches
 * nothing.
 */
fp8bq_status gemm_w8a8_blockscaled_splitk_workspace(int64_t M, int64_t N, int64_t K, int64_t* bytes);

/*
 * gemm_w8a8_blockscaled_splitk_noalloc -- gemm_w8a8_blockscaled_splitk for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops or harnesses that forbid hipMalloc): no workspace argument;
 * the partial tiles go to a static device array of FP8BQ_SCRATCH_BYTES that
 * the library holds on each GPU it runs on until the process ends.  The
 * call itself allocates nothing (no hipMalloc / hipFree, no allocating
 * library routine).  Same kernels and the same result bits as
 * gemm_w8a8_blockscaled_splitk.
 *   Arguments as for gemm_w8a8_blockscaled.  A shape whose split needs more
 *   than FP8BQ_SCRATCH_BYTES (see gemm_w8a8_blockscaled_splitk_workspace)
 *   returns FP8BQ_ERR_SCRATCH and enqueues nothing; with the split rule on a
 *   256-CU device that never happens (S * M * N * 4 <= 32 MiB).
 *   All calls on one GPU share the array: calls that overlap on one GPU (on
 *   different streams, or from different threads without ordering) race
 *   and give unspecified output.  Calls ordered on one stream are safe.
 */
#define FP8BQ_SCRATCH_BYTES (32 * 1024 * 1024)
fp8bq_status gemm_w8a8_blockscaled_splitk_noalloc(const uint8_t* a_fp8, const float* a_scale, const uint8_t* w_fp8,
                                                  const float* w_scale, uint16_t* y_bf16, int64_t M, int64_t N,
                                                  int64_t K, void* stream);

/*
 * quantize_act_per_token_group_frag -- quantize_act_per_token_group with
 * the codes written in the MFMA fragment order that
 * gemm_w8a8_blockscaled_afrag reads ([FP8-RL summary] §3.4.1 "1 × 128 tiles
 * for activations"; §3.4.2 Phase 3).  Same codes and scales, another byte
 * order:
 *   x_bf16      [M][K] BF16, row-major (as for quantize_act_per_token_group)
 *   x_fp8_frag  M * K bytes: code (m, k) at
 *               ((m/16 * K/128 + k/128) * 2 + (k%128)/64) * 1024
 *               + (((k%64)/16) * 16 + m%16) * 16 + k%16
 *               (per 16 rows and K-block, 2 KB: the two 16-byte halves of
 *               each lane's 16x16x128 MFMA operand, lane-major)
 *   x_scale     [M][K/128] float32, token-major (as for the row-major form)
 *   Requires M % 16 == 0 and K % 128 == 0 (FP8BQ_ERR_BAD_SHAPE otherwise);
 *   the other conventions are those of quantize_act_per_token_group.
 */
fp8bq_status quantize_act_per_token_group_frag(const uint16_t* x_bf16, uint8_t* x_fp8_frag, float* x_scale,
                                               int64_t M, int64_t K, void* stream);

/*
 * gemm_w8a8_blockscaled_afrag -- gemm_w8a8_blockscaled on activation codes
 * in the fragment order of quantize_act_per_token_group_frag
 * ([FP8-RL summary] §3.4.2 Phase 3).  Each load of an activation operand is
 * then a contiguous 1 KB piece of a fragment unit.  Same result bits as
 * gemm_w8a8_blockscaled on the row-major codes (same per-element order).
 *   a_fp8_frag  M * K bytes in fragment order; a_scale [M][K/128]
 *   w_fp8 [N][K], w_scale [ceil(N/128)][K/128], y_bf16 [M][N] as for
 *   gemm_w8a8_blockscaled.
 *   Requires M % 16 == 0 and K % 128 == 0 (K <= 2^22); FP8BQ_ERR_BAD_SHAPE
 *   otherwise.  The tile is chosen per shape as for gemm_w8a8_blockscaled
 *   (few activation rows: K split over the waves of a 64- or 48-row tile
 *   that loads the fragments straight into registers; more rows: the panel
 *   tiles, which keep the fragment order in their LDS ring), and the output
 *   is bit-identical to gemm_w8a8_blockscaled's on the row-major codes.
 *   This is the library's path for activations with M % 16 == 0 and
 *   K % 128 == 0: on the Qwen3-8B layer shapes it is faster than
 *   gemm_w8a8_blockscaled at both decode (M = 256) and prefill (M = 8192)
 *   sizes.
 */
fp8bq_status gemm_w8a8_blockscaled_afrag(const uint8_t* a_fp8_frag, const float* a_scale, const uint8_t* w_fp8,
                                         const float* w_scale, uint16_t* y_bf16, int64_t M, int64_t N, int64_t K,
                                         void* stream);

/*
 * gemm_w8a8_blockscaled_frag -- gemm_w8a8_blockscaled_afrag with the weight
 * codes in fragment order as well (quantize_weight_blockwise_frag), the
 * library's fastest form: every operand load is a contiguous 1 KB piece of
 * a fragment unit.  Same result, bit for bit, as gemm_w8a8_blockscaled on
 * the row-major codes; same arguments and errors as
 * gemm_w8a8_blockscaled_afrag, plus FP8BQ_ERR_BAD_SHAPE unless N % 16 == 0.
 */
fp8bq_status gemm_w8a8_blockscaled_frag(const uint8_t* a_fp8_frag, const float* a_scale, const uint8_t* w_fp8_frag,
                                        const float* w_scale, uint16_t* y_bf16, int64_t M, int64_t N, int64_t K,
                                        void* stream);

/*
 * grouped_gemm_w8a8_blockscaled -- the MoE expert form: rows
 * [group_offsets[e], group_offsets[e+1]) of A are multiplied with expert
 * e's weights ([FP8-RL summary] §3.4.1 "Quantization Scope", fc1/fc2 of
 * each expert quantized like the dense linears).
 *
 *   a_fp8   [M_total][K], a_scale [M_total][K/128]
 *   w_fp8   [G][N][K],    w_scale [G][ceil(N/128)][K/128]
 *   group_offsets  DEVICE int32 [G+1], non-decreasing, [0] = 0, [G] = M_total
 *   y_bf16  [M_total][N]
 *   Empty groups are allowed.  G == 0 with M_total * N > 0 is
 *   FP8BQ_ERR_BAD_SHAPE.  The offsets are read on the device only (no
 *   host synchronisation); offsets that break the stated contract give
 *   unspecified output rows but never an out-of-bounds access: every row
 *   index is clamped to [0, M_total).  M_total + 128 * G must fit in int32;
 *   K as for gemm_w8a8_blockscaled.
 *   For G <= 1024 one workgroup per CU runs the expert tiles in turn (the
 *   launch does not depend on how the rows are spread); for more experts,
 *   one workgroup per tile.  grouped_gemm_w8a8_blockscaled_tile runs a
 *   named tile kernel.
 *   Debug mode: with FP8BQ_CHECK_OFFSETS=1 in the environment (read once,
 *   at the first grouped GEMM call of the process) every grouped call first
 *   runs fp8bq_check_group_offsets and returns its error, launching
 *   nothing.  This applies to grouped_gemm_w8a8_blockscaled_gather too.
 */
fp8bq_status grouped_gemm_w8a8_blockscaled(const uint8_t* a_fp8, const float* a_scale, const uint8_t* w_fp8,
                                           const float* w_scale, const int32_t* group_offsets, uint16_t* y_bf16,
                                           int64_t M_total, int64_t N, int64_t K, int64_t G, void* stream);

/*
 * grouped_gemm_w8a8_blockscaled_gather -- the grouped GEMM with its
 * activation rows gathered: output row m (expert e owns rows
 * [group_offsets[e], group_offsets[e+1]) as above) multiplies row
 * a_rows[m] / a_row_div of a_fp8 with expert e's weights.  With a_rows the
 * sorted_pair of moe_sort_by_expert and a_row_div = k, the MoE fc1 reads the
 * token-major FP8 activations (quantize_act_per_token_group of the tokens)
 * directly, and no per-pair copy of them is made ([FP8-RL summary] §3.4.1
 * "Quantization Scope", MoE fc1 / fc2).
 *   a_fp8 [M_a][K], a_scale [M_a][K/128]; a_rows [M_total] int32 (entries
 *   that are negative or name a row >= M_a give a zero activation row);
 *   a_row_div >= 1; w_fp8, w_scale, group_offsets and y_bf16 [M_total][N]
 *   as in grouped_gemm_w8a8_blockscaled.  M_a * K < 2^31; K as for
 *   gemm_w8a8_blockscaled.
 */
fp8bq_status grouped_gemm_w8a8_blockscaled_gather(const uint8_t* a_fp8, const float* a_scale, int64_t M_a,
                                                  const int32_t* a_rows, int64_t a_row_div, const uint8_t* w_fp8,
                                                  const float* w_scale, const int32_t* group_offsets,
                                                  uint16_t* y_bf16, int64_t M_total, int64_t N, int64_t K, int64_t G,
                                                  void* stream);

/*
 * grouped_gemm_w8a8_blockscaled_gather_silu -- the MoE fc1 GEMM with the
 * gated activation and its quantization in the epilogue ([FP8-RL summary]
 * §3.4.1 "Quantization Scope": fc1 gives gate and up, multiplied element-wise
 * before fc2; "Static vs. Dynamic Quantization": the nonlinearity in higher
 * precision, the activations quantized on the fly in 1x128 tiles).  Gives
 * exactly the codes and scales of
 *   silu_mul_quantize_act(grouped_gemm_w8a8_blockscaled_gather(...))
 * without storing the BF16 fc1 output [M_total][2F]: each gate and up value
 * is rounded to BF16 as that output would be, h = SiLU(gate) * up is rounded
 * to BF16 from its exact value, and h is quantized per row in groups of 128
 * columns.
 *   a_fp8, a_scale, M_a, a_rows, a_row_div, group_offsets, M_total, K, G as
 *   in grouped_gemm_w8a8_blockscaled_gather, with K > 0 and G <= 1024;
 *   w_fp8 [G][2F][K] E4M3 with rows [gate (F); up (F)] per expert, w_scale
 *   [G][2F/128][K/128]; outputs h_fp8 [M_total][F] E4M3 and h_scale
 *   [M_total][F/128] float32.  F % 128 == 0 and (F + 128) * K < 2^31;
 *   FP8BQ_ERR_BAD_SHAPE otherwise.  All pointers 16-byte aligned.
 */
fp8bq_status grouped_gemm_w8a8_blockscaled_gather_silu(const uint8_t* a_fp8, const float* a_scale, int64_t M_a,
                                                       const int32_t* a_rows, int64_t a_row_div, const uint8_t* w_fp8,
                                                       const float* w_scale, const int32_t* group_offsets,
                                                       uint8_t* h_fp8, float* h_scale, int64_t M_total, int64_t F,
                                                       int64_t K, int64_t G, void* stream);

/*
 * grouped_gemm_w8a8_blockscaled_tile -- the grouped GEMM (plain when a_rows
 * is NULL, then a_fp8 has M_total rows and M_a / a_row_div are ignored;
 * gathered otherwise, as grouped_gemm_w8a8_blockscaled_gather) with the
 * tile kernel named by `tile`: FP8BQ_TILE_AUTO, WIDE, DECODE_PANEL, DEEP or
 * DEEP_PERSISTENT.  Same contract and the same result bits for a given
 * tile.  Another tile value is FP8BQ_ERR_BAD_ARG.  For tests and
 * diagnostics.
 */
fp8bq_status grouped_gemm_w8a8_blockscaled_tile(const uint8_t* a_fp8, const float* a_scale, int64_t M_a,
                                                const int32_t* a_rows, int64_t a_row_div, const uint8_t* w_fp8,
                                                const float* w_scale, const int32_t* group_offsets,
                                                uint16_t* y_bf16, int64_t M_total, int64_t N, int64_t K, int64_t G,
                                                int tile, void* stream);

/*
 * fp8bq_check_group_offsets -- host check of the grouped GEMMs' offsets
 * contract (the debug mode above): copies group_offsets (DEVICE int32
 * [G+1]) to the host on `stream`, waits for the copy, and returns
 * FP8BQ_ERR_BAD_SHAPE unless [0] = 0, the offsets are non-decreasing and
 * [G] = M_total.  Synchronous; launches no kernel.  G >= 1.
 */
fp8bq_status fp8bq_check_group_offsets(const int32_t* group_offsets, int64_t G, int64_t M_total, void* stream);

/*
 * fp8bq_encode_e4m3 -- the library's float32 -> E4M3 conversion on its own
 * ([FP8-RL summary] §3.4.1 "Quantization Format and Granularity"; round to
 * nearest even, sign of zero kept), so that it can be checked over every
 * float32 input:
 *   method 0: the hardware conversion exactly as the quantizers apply it to
 *             their quotients (defined for |v| < 464, the range every
 *             quantizer quotient lies in);
 *   method 1: saturating encoder: clamp to +-448, then the hardware
 *             conversion (any finite v);
 *   method 2: integer-bit encoder (any finite v).
 *   in [n] float32, out [n] uint8, n >= 0.  Other methods: FP8BQ_ERR_BAD_SHAPE.
 */
fp8bq_status fp8bq_encode_e4m3(const float* in, uint8_t* out, int64_t n, int method, void* stream);

/*
 * token_importance_weights -- per-token rollout-correction weights of FP8
 * rollouts ([FP8-RL summary] §3.4.3 "Train-Inference Mismatch and
 * Importance-Sampling Correction").  The weight of a sampled token is the
 * ratio of the training policy's probability to the FP8 rollout policy's,
 *     w = exp(logp_train - logp_rollout),
 * and it multiplies the token's advantage in the policy loss.
 *   mode FP8BQ_IW_TIS: truncated importance sampling, w limited to [1/C, C]
 *                      (C = 2 in the page's experiments);
 *   mode FP8BQ_IW_MIS: masked importance sampling (only named on the page;
 *                      this library's reading): a token whose weight lies
 *                      outside [1/C, C] gets 0, the others keep w limited to
 *                      [1/C, C].  The in/out decision is exact in float32:
 *                      kept iff |fl32(logp_train - logp_rollout)| <= fl32(ln C).
 *
 *   logp_train    [n] float32  log-probability of each sampled token under
 *                              the training (full-precision) policy
 *   logp_rollout  [n] float32  the same under the FP8 rollout policy
 *   mask          [n] uint8 or NULL: 0 = padding (w = 0, and w * A = 0),
 *                 non-zero = a generated token.  NULL: every token counts.
 *   advantages    [n] float32 or NULL: per-token advantage A
 *   weights       [n] float32 output w
 *   weighted_adv  [n] float32 output w * A (+0 wherever w == 0); must be
 *                 non-NULL exactly when `advantages` is.
 *   0 <= n <= 2^40 (a [responses][max_len] batch is n = responses * max_len).
 *   C >= 1 (C = +inf gives untruncated weights); a NaN C, C < 1, another
 *   mode, or only one of advantages / weighted_adv: FP8BQ_ERR_BAD_ARG.
 * Error: w carries the error of one float32 exp (the difference of the log
 * probabilities is kept exactly), then the clip; a NaN log-probability gives
 * NaN under TIS and 0 under MIS; logp_train = -inf gives 1/C under TIS.
 * Unlike the quantizers, infinite and NaN inputs are defined here.
 */
enum { FP8BQ_IW_TIS = 0, FP8BQ_IW_MIS = 1 };

fp8bq_status token_importance_weights(const float* logp_train, const float* logp_rollout, const uint8_t* mask,
                                      const float* advantages, float* weights, float* weighted_adv, int64_t n,
                                      float C, int mode, void* stream);

/*
 * FP8 training operands ([FP8-RL summary] §3.4.5 "End-to-End FP8 RL": the
 * trainer's forward and backward GEMMs also run in FP8).  With the §3.4.1
 * rule applied in the layout each GEMM reduces over: forward x W^T takes x
 * in 1x128 groups along K and W in 128x128 blocks; dgrad dy W takes W^T
 * ([K][N]) in 128x128 blocks; wgrad dy^T x takes x^T and dy^T in 1x128
 * groups along the tokens.  Both layouts come from one read of the BF16
 * tensor.
 */

/*
 * quantize_weight_blockwise_dual -- W and W^T in 128x128 blocks.  W^T's
 * blocks are W's blocks transposed: wt_fp8 is w_fp8 transposed, wt_scale is
 * w_scale transposed (the codes of quantize_weight_blockwise).
 *   w_bf16 [batch][N][K]; w_fp8 [batch][N][K] and w_scale
 *   [batch][ceil(N/128)][ceil(K/128)], or both NULL (W^T only);
 *   wt_fp8 [batch][K][N], wt_scale [batch][ceil(K/128)][ceil(N/128)].
 *   K % 8 == 0, batch <= 65535.
 */
fp8bq_status quantize_weight_blockwise_dual(const uint16_t* w_bf16, uint8_t* w_fp8, float* w_scale, uint8_t* wt_fp8,
                                            float* wt_scale, int64_t batch, int64_t N, int64_t K, void* stream);

/*
 * quantize_act_dual -- x in 1x128 groups along K (exactly
 * quantize_act_per_token_group) and x^T in 1x128 groups along M: row k of
 * xt_fp8 is channel k of x quantized in groups of 128 consecutive tokens.
 *   x_bf16 [M][K]; x_fp8 [M][K] and x_scale [M][ceil(K/128)], or both NULL
 *   (x^T only); xt_fp8 [K][M], xt_scale [K][ceil(M/128)].  K % 8 == 0.
 */
fp8bq_status quantize_act_dual(const uint16_t* x_bf16, uint8_t* x_fp8, float* x_scale, uint8_t* xt_fp8,
                               float* xt_scale, int64_t M, int64_t K, void* stream);

/*
 * MoE expert-FFN glue around grouped_gemm_w8a8_blockscaled ([FP8-RL
 * summary] §3.4.1 "Quantization Scope": the MoE expert layers fc1 / fc2 are
 * FP8 W8A8 linears like the dense ones, and the gated MLP multiplies the gate
 * and up activations element-wise before the down projection; §3.4.1
 * "Static vs. Dynamic Quantization": activations are quantized on the fly in
 * 1x128 tiles, the nonlinearity stays in higher precision).  One MoE layer:
 *   moe_sort_by_expert -> moe_gather_quantize_act -> grouped GEMM (fc1)
 *   -> silu_mul_quantize_act -> grouped GEMM (fc2) -> moe_combine.
 * A routing "pair" p = t * k + j is slot j of token t.
 */

/*
 * moe_sort_by_expert -- rows grouped by expert for the grouped GEMM.
 *   topk_ids       [T][k] int32, the experts each token is routed to
 *   group_offsets  [E+1] int32 output: expert e owns rows
 *                  [group_offsets[e], group_offsets[e+1]); [0] = 0 and
 *                  [E] = the number of pairs whose id is in [0, E)
 *   sorted_pair    [T*k] int32 output: row r holds pair sorted_pair[r];
 *                  entries from [E] on are left untouched
 *   pair_row       [T*k] int32 output: the row of pair p, or -1 when its id
 *                  is outside [0, E)
 * Rows of one expert keep pair order (by token, for distinct ids per
 * token).  Deterministic, no atomics.  T, k >= 0, T * k < 2^31, E >= 1
 * (group_offsets is written even when T * k == 0).
 */
fp8bq_status moe_sort_by_expert(const int32_t* topk_ids, int64_t T, int64_t k, int64_t E, int32_t* group_offsets,
                                int32_t* sorted_pair, int32_t* pair_row, void* stream);

/*
 * moe_gather_quantize_act -- the fc1 input rows: row r is token
 * sorted_pair[r] / k of x, quantized in 1x128 per-token groups exactly as
 * quantize_act_per_token_group quantizes that token (so the codes equal
 * quantizing x and copying rows).  Rows whose pair is negative or names a
 * token >= T are written as zero codes with scale 0.
 *   x_bf16  [T][K] BF16, sorted_pair [rows] int32 (moe_sort_by_expert)
 *   a_fp8   [rows][K] E4M3 output, a_scale [rows][K/128] float32 output
 *   rows, T >= 0, k >= 1, K >= 0 and K % 128 == 0.
 */
fp8bq_status moe_gather_quantize_act(const uint16_t* x_bf16, const int32_t* sorted_pair, int64_t rows, int64_t T,
                                     int64_t k, int64_t K, uint8_t* a_fp8, float* a_scale, void* stream);

/*
 * silu_mul_quantize_act -- the fc2 input from the fc1 output: per row, with
 * gate = columns [0, F) and up = columns [F, 2F),
 *   h = BF16( SiLU(gate) * up ),  SiLU(g) = g / (1 + exp(-g)),
 * correctly rounded (round to nearest even) from the exact value, then
 * quantized in 1x128 groups exactly as quantize_act_per_token_group
 * quantizes a BF16 [M][F] tensor.
 *   y_bf16 [M][2F] BF16; h_fp8 [M][F] E4M3 output; h_scale [M][ceil(F/128)]
 *   float32 output; h_bf16 [M][F] BF16 output of h itself, or NULL.
 *   M >= 0, F >= 0, F % 8 == 0.  Inputs must be finite and every h must be
 *   finite (below the BF16 maximum).
 */
fp8bq_status silu_mul_quantize_act(const uint16_t* y_bf16, int64_t M, int64_t F, uint8_t* h_fp8, float* h_scale,
                                   uint16_t* h_bf16, void* stream);

/*
 * moe_combine -- each token's output is the routing-weighted sum of its
 * expert rows: out[t] = sum_j topk_weights[t][j] * y[pair_row[t*k + j]],
 * accumulated in float32 (fused multiply-add in slot order j = 0..k-1) and
 * rounded once to BF16 (nearest even).  Slots whose row is outside
 * [0, M_rows) contribute nothing.
 *   y_bf16 [M_rows][H] BF16 (the fc2 output), pair_row [T*k] int32,
 *   topk_weights [T][k] float32, out_bf16 [T][H] BF16 output.
 *   T, k, M_rows >= 0, H >= 0, H % 8 == 0, T * k < 2^31.
 */
fp8bq_status moe_combine(const uint16_t* y_bf16, const int32_t* pair_row, const float* topk_weights, int64_t T,
                         int64_t k, int64_t H, int64_t M_rows, uint16_t* out_bf16, void* stream);

/*
 * FP8 KV cache ([FP8-RL summary] §3.4.4 "KV-Cache Quantization"): K and V are
 * stored as 1-byte E4M3 values.  The weights change every RL step, so at the
 * start of each rollout the per-layer or per-head scales are recomputed from
 * the K and V of its first forward pass (kv_scale_calibrate) and then used
 * for every cache write of the rollout (kv_cache_write_fp8).
 * Layouts: K / V of T tokens [T][H][D] BF16 (H KV heads of D elements); the
 * caches [S][H][D] E4M3 (S token slots); scales float32 [H] (per_head = 1)
 * or [1] (per_head = 0).  D % 8 == 0, H * D <= 8192.  V takes part when
 * v_scale is non-NULL (then its other pointers are required as for K);
 * otherwise its pointers must all be NULL.
 */

/*
 * kv_scale_calibrate -- s = fl32(amax / 448) per KV head (or per layer), with
 * amax = max |x| over all T tokens, for K and for V (the tile rule of the
 * linear layers, §3.4.1).  T == 0 gives s = 0.  Deterministic.
 */
fp8bq_status kv_scale_calibrate(const uint16_t* k_bf16, const uint16_t* v_bf16, int64_t T, int64_t H, int64_t D,
                                int per_head, float* k_scale, float* v_scale, void* stream);

/*
 * kv_cache_write_fp8 -- token t's K and V, quantized with the fixed scales
 * as q = E4M3(fl32(x / s)) (round to nearest even), are stored in slot
 * slot_mapping[t] of the caches.  Quotients beyond the E4M3 range (values
 * above the calibrated amax) saturate to +-448; with s = 0 non-zero values
 * give +-448 and zeros keep their sign.  Tokens whose slot is outside
 * [0, S) (padding) store nothing; slots of the other tokens must differ.
 *   slot_mapping [T] int32; 0 <= S < 2^31.
 */
fp8bq_status kv_cache_write_fp8(const uint16_t* k_bf16, const uint16_t* v_bf16, const int32_t* slot_mapping,
                                const float* k_scale, const float* v_scale, int per_head, uint8_t* k_cache,
                                uint8_t* v_cache, int64_t T, int64_t H, int64_t D, int64_t S, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8BQ_H */
