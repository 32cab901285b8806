// launch.h -- internal launchers of the libsvdq HIP kernels (argument
// checks are done by the C ABI layer before these are called).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

hipError_t launch_quantize_act(int precision, int M, int K, int rank, const void *x,
                               const void *smooth, const void *lora_down, void *act_codes,
                               void *act_scales, float *lora_act, hipStream_t stream);

hipError_t launch_gemm_w4a4_int4(int M, int N, int K, int rank, const void *act_codes,
                                 const void *act_scales, const void *wgt_codes,
                                 const void *wgt_scales, float alpha, const float *lora_act,
                                 const void *lora_up, const void *bias, void *out,
                                 hipStream_t stream);

hipError_t launch_gemm_w4a4_nvfp4(int M, int N, int K, int rank, const void *act_codes,
                                  const void *act_scales, const void *wgt_codes,
                                  const void *wgt_scales, float alpha, const float *lora_act,
                                  const void *lora_up, const void *bias, void *out,
                                  hipStream_t stream);

hipError_t launch_group_sums_int4(int M, int N, int K, const void *act_codes,
                                  const void *wgt_codes, int32_t *G, hipStream_t stream);

hipError_t launch_awq_gemv(int M, int N, int K, const void *x, const void *codes,
                           const void *scales, const void *zeros, const void *bias, void *out,
                           hipStream_t stream);

}  // namespace svdq
