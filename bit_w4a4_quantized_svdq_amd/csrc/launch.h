// launch.h -- internal launchers of the libsvdq HIP kernels (argument
// checks are done by the C ABI layer before these are called).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

// Epilogue parameters of the grouped QKV layer: per-head RMSNorm and rotary
// embedding of the Q and K heads (128 channels each; columns Q | K | V).
struct QkNormRope {
    const uint16_t *q_w;   // bf16 [128], norm weight of the Q heads
    const uint16_t *k_w;   // bf16 [128], norm weight of the K heads
    const float *cos;      // fp32 [M, 64], the rows' rotary angles
    const float *sin;      // fp32 [M, 64]
    float eps;
    int qk_cols;           // 2 * heads * 128: the Q and K columns
};

// precision: 0 int4 (nibbles), 1 NVFP4, 2 int4 codes in the FP6 layout
hipError_t launch_quantize_act(int precision, bool gelu, int M, int K, int rank, const void *x,
                               const void *smooth, const void *lora_down, void *act_codes,
                               void *act_scales, float *lora_act, hipStream_t stream);
hipError_t launch_gelu_bf16(int64_t n, const void *in, void *out, hipStream_t stream);
size_t lowrank_workspace_bytes(int N, int K, int r);
// Fixed per-device scratch of the allocation-free low-rank entry point: its
// size, and its device address on the current device.
constexpr size_t LOWRANK_SCRATCH_BYTES = size_t(32) << 20;
hipError_t lowrank_scratch(void **ptr);
hipError_t launch_lowrank_factors(int N, int K, int r, const void *W, const void *s, uint64_t seed,
                                  void *workspace, void *up, void *down, hipStream_t stream);
hipError_t launch_smooth_factors(int M, int N, int K, const void *x, const void *W, void *s, hipStream_t stream);
hipError_t launch_quantize_weight(int precision, int N, int K, int rank, const void *W, const void *s,
                                  const void *up, const void *down, void *codes, void *scales,
                                  hipStream_t stream);

// int4 GEMM; packed: wgt_codes is the blob of launch_pack_weight_int4
hipError_t launch_gemm_w4a4_int4(bool packed, int M, int N, int K, int rank, const void *act_codes,
                                 const void *act_scales, const void *wgt_codes,
                                 const void *wgt_scales, float alpha, const float *lora_act,
                                 const void *lora_up, const void *bias, void *out,
                                 hipStream_t stream);
// offline re-encoding of int4 weights for the packed GEMM: blob = codes
// [N, K/2] in the packed layout, then bf16 [N][2][K/64] correction planes;
// invalid (optional) counts the -8 codes, which the layout cannot hold
size_t packed_weight_bytes(int N, int K);
hipError_t launch_pack_weight_int4(int N, int K, const void *wgt_codes, const void *wgt_scales, void *blob,
                                   int32_t *invalid, hipStream_t stream);
// int4 GEMM on the FP6 layout of both operands (launch_pack_weight_fp6 for
// the weight, the activation step's precision 2 for the activations)
size_t fp6_weight_bytes(int N, int K);
hipError_t launch_pack_weight_fp6(int N, int K, const void *wgt_codes, void *blob, hipStream_t stream);
hipError_t launch_gemm_w4a4_fp6(int M, int N, int K, int rank, const void *act_codes, const void *act_scales,
                                const void *wgt_codes, const void *wgt_scales, float alpha, const float *lora_act,
                                const void *lora_up, const void *bias, void *out, hipStream_t stream);
hipError_t launch_gemm_w4a4_fp6_qk(int M, int N, int K, int rank, const void *act_codes, const void *act_scales,
                                   const void *wgt_codes, const void *wgt_scales, float alpha,
                                   const float *lora_act, const void *lora_up, const void *bias,
                                   const QkNormRope &qk, void *out, hipStream_t stream);
hipError_t launch_group_sums_fp6(int M, int N, int K, const void *act_codes, const void *wgt_codes, int32_t *G,
                                 hipStream_t stream);
// the FP6 GEMM of a GELU MLP's up projection with the down layer's activation
// step in its epilogue (workspace: gelu_quant_workspace_bytes)
size_t gelu_quant_workspace_bytes(int M, int N, int rank_next);
hipError_t launch_gemm_w4a4_fp6_gelu_quant(int M, int N, int K, int rank, const void *act_codes,
                                           const void *act_scales, const void *wgt_codes, const void *wgt_scales,
                                           float alpha, const float *lora_act, const void *lora_up,
                                           const void *bias, int rank_next, const void *smooth_next,
                                           const void *lora_down_next, void *next_codes, void *next_scales,
                                           float *next_lora_act, void *workspace, void *out, hipStream_t stream);
hipError_t launch_gemm_w4a4_nvfp4_qk(int M, int N, int K, int rank, const void *act_codes,
                                     const void *act_scales, const void *wgt_codes,
                                     const void *wgt_scales, float alpha, const float *lora_act,
                                     const void *lora_up, const void *bias, const QkNormRope &qk,
                                     void *out, hipStream_t stream);
hipError_t launch_gemm_w4a4_int4_qk(bool packed, int M, int N, int K, int rank, const void *act_codes,
                                    const void *act_scales, const void *wgt_codes,
                                    const void *wgt_scales, float alpha, const float *lora_act,
                                    const void *lora_up, const void *bias, const QkNormRope &qk,
                                    void *out, hipStream_t stream);

hipError_t launch_gemm_w4a4_nvfp4(int M, int N, int K, int rank, const void *act_codes,
                                  const void *act_scales, const void *wgt_codes,
                                  const void *wgt_scales, float alpha, const float *lora_act,
                                  const void *lora_up, const void *bias, void *out,
                                  hipStream_t stream);

hipError_t launch_group_sums_int4(bool packed, int M, int N, int K, const void *act_codes,
                                  const void *wgt_codes, int32_t *G, hipStream_t stream);

// The AWQ layer for one row of x (K a multiple of 512, at most 4096):
// whole-line weight loads, dot products on the vector ALU.
bool awq_gemv_lines_applies(int M, int N, int K);
hipError_t launch_awq_gemv_lines(int M, int N, int K, const void *x, const void *codes, const void *scales,
                                 const void *zeros, const void *bias, void *out, hipStream_t stream);
// The same whole-line stream for up to 8 rows of x with the products on the
// matrix cores (K a multiple of 512, at most 4096, x within the LDS budget).
bool awq_gemv_lines_mfma_applies(int M, int N, int K);
hipError_t launch_awq_gemv_lines_mfma(int M, int N, int K, const void *x, const void *codes, const void *scales,
                                      const void *zeros, const void *bias, void *out, hipStream_t stream);
// plain read, contiguous or in the GEMV's access pattern (a measurement hook)
int64_t stream_read_spans(int64_t bytes);
hipError_t launch_stream_read(const void *src, int64_t bytes, bool lines, uint32_t *out, hipStream_t stream);
hipError_t launch_awq_gemv(int M, int N, int K, const void *x, const void *codes,
                           const void *scales, const void *zeros, const void *bias, void *out,
                           hipStream_t stream);

// The AWQ layer in the GEMM regime (awq_gemm_applies): K a multiple of 512,
// at least AWQ_GEMM_MIN_M rows of x and at least AWQ_GEMM_MIN_TILES 32 x 32
// output tiles (the GEMV's blocks); the GEMV otherwise.  Measured at K = 3072:
// the GEMM takes ~53 us for any grid up to about one block per CU and
// ~0.15 us per 128 x 128 tile beyond; the GEMV ~27 us up to ~400 of its
// tiles and ~0.072 us per tile beyond; both scale with K.
constexpr int AWQ_GEMM_MIN_M = 32;
constexpr long long AWQ_GEMM_MIN_TILES = 576;
bool awq_gemm_applies(int M, int N, int K);
hipError_t launch_awq_gemm(int M, int N, int K, const void *x, const void *codes,
                           const void *scales, const void *zeros, const void *bias, void *out,
                           hipStream_t stream);

}  // namespace svdq
