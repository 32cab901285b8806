// Stand-ins for what the C ABI layer calls below it, for the host sanitizer
// run: the HIP runtime's device query (a device whose architecture name the
// driver chooses) and the kernels' launchers, which record the call instead
// of launching anything.
#include <cstdio>
#include <cstring>

#include "../../bit_w4a4_quantized_svdq_amd/csrc/launch.h"
#include "stub_log.h"

StubLog g_stub;

extern "C" {
hipError_t hipGetDevice(int *dev) {
    *dev = g_stub.device;
    return hipSuccess;
}
hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_t *prop, int) {
    std::memset(prop, 0, sizeof *prop);
    std::snprintf(prop->gcnArchName, sizeof prop->gcnArchName, "%s", g_stub.arch);
    return hipSuccess;
}
const char *hipGetErrorString(hipError_t) { return "stub error"; }
}

namespace svdq {
static hipError_t rec(const char *name, long long a, long long b, long long c) {
    g_stub.calls++;
    std::snprintf(g_stub.last, sizeof g_stub.last, "%s", name);
    g_stub.a = a; g_stub.b = b; g_stub.c = c;
    return g_stub.result;
}
hipError_t launch_quantize_act(int precision, bool gelu, int M, int K, int rank, const void *, const void *,
                               const void *, void *, void *, float *, hipStream_t) {
    return rec(gelu ? "quantize_act_gelu" : "quantize_act", M, K, rank + 1000 * precision);
}
hipError_t launch_gelu_bf16(int64_t n, const void *, void *, hipStream_t) { return rec("gelu_bf16", n, 0, 0); }
size_t lowrank_workspace_bytes(int N, int K, int r) { return (size_t)(N + K) * (size_t)(r + 8) * 8u; }
hipError_t launch_lowrank_factors(int N, int K, int r, const void *, const void *, uint64_t, void *, void *,
                                  void *, hipStream_t) {
    return rec("lowrank_factors", N, K, r);
}
hipError_t lowrank_scratch(void **ptr) {
    *ptr = (void *)(uintptr_t)0x200000;   // a fake, aligned device address
    return g_stub.result;
}
hipError_t launch_smooth_factors(int M, int N, int K, const void *, const void *, void *, hipStream_t) {
    return rec("smooth_factors", M, N, K);
}
hipError_t launch_quantize_weight(int precision, int N, int K, int rank, const void *, const void *,
                                  const void *, const void *, void *, void *, hipStream_t) {
    return rec("quantize_weight", N, K, rank + 1000 * precision);
}
hipError_t launch_gemm_w4a4_int4(bool packed, int M, int N, int K, int, const void *, const void *, const void *,
                                 const void *, float, const float *, const void *, const void *, void *,
                                 hipStream_t) {
    return rec(packed ? "gemm_int4_packed" : "gemm_int4", M, N, K);
}
size_t packed_weight_bytes(int N, int K) { return (size_t)N * (K / 2) + (size_t)N * 4 * (K / 64); }
hipError_t launch_pack_weight_int4(int N, int K, const void *, const void *, void *, int32_t *invalid,
                                   hipStream_t) {
    return rec("pack_weight_int4", N, K, invalid != nullptr);
}
hipError_t launch_gemm_w4a4_nvfp4(int M, int N, int K, int, const void *, const void *, const void *,
                                  const void *, float, const float *, const void *, const void *, void *,
                                  hipStream_t) {
    return rec("gemm_nvfp4", M, N, K);
}
hipError_t launch_gemm_w4a4_int4_qk(bool packed, int M, int N, int K, int, const void *, const void *,
                                    const void *, const void *, float, const float *, const void *, const void *,
                                    const QkNormRope &qk, void *, hipStream_t) {
    return rec(packed ? "gemm_int4_packed_qk" : "gemm_int4_qk", M, N, qk.qk_cols);
}
hipError_t launch_gemm_w4a4_nvfp4_qk(int M, int N, int K, int, const void *, const void *, const void *,
                                     const void *, float, const float *, const void *, const void *,
                                     const QkNormRope &qk, void *, hipStream_t) {
    return rec("gemm_nvfp4_qk", M, N, qk.qk_cols);
}
hipError_t launch_group_sums_int4(bool packed, int M, int N, int K, const void *, const void *, int32_t *,
                                  hipStream_t) {
    return rec(packed ? "group_sums_packed" : "group_sums", M, N, K);
}
hipError_t launch_awq_gemv(int M, int N, int K, const void *, const void *, const void *, const void *,
                           const void *, void *, hipStream_t) {
    return rec("awq_gemv", M, N, K);
}
size_t fp6_weight_bytes(int N, int K) { return (size_t)((N + 127) / 128) * (size_t)((K / 64 + 1) / 2) * 12288u; }
hipError_t launch_pack_weight_fp6(int N, int K, const void *, void *, hipStream_t) {
    return rec("pack_weight_fp6", N, K, 0);
}
hipError_t launch_gemm_w4a4_fp6(int M, int N, int K, int, const void *, const void *, const void *, const void *,
                                float, const float *, const void *, const void *, void *, hipStream_t) {
    return rec("gemm_fp6", M, N, K);
}
hipError_t launch_gemm_w4a4_fp6_qk(int M, int N, int, int, const void *, const void *, const void *, const void *,
                                   float, const float *, const void *, const void *, const QkNormRope &qk, void *,
                                   hipStream_t) {
    return rec("gemm_fp6_qk", M, N, qk.qk_cols);
}
size_t gelu_quant_workspace_bytes(int M, int N, int rank_next) {
    return (size_t)((N + 127) / 128) * (size_t)M * (size_t)rank_next * 4u;
}
hipError_t launch_gemm_w4a4_fp6_gelu_quant(int M, int N, int K, int, const void *, const void *, const void *,
                                           const void *, float, const float *, const void *, const void *,
                                           int rank_next, const void *, const void *, void *, void *, float *,
                                           void *, void *, hipStream_t) {
    return rec("gemm_fp6_gelu_quant", M, N, K + rank_next);
}
hipError_t launch_group_sums_fp6(int M, int N, int K, const void *, const void *, int32_t *, hipStream_t) {
    return rec("group_sums_fp6", M, N, K);
}
hipError_t launch_stream_read(const void *, int64_t bytes, bool lines, uint32_t *, hipStream_t) {
    return rec("stream_read", (int)(bytes >> 20), lines, 0);
}
bool awq_gemm_applies(int M, int N, int K) {
    return K % 512 == 0 && M >= AWQ_GEMM_MIN_M &&
           (long long)((M + 31) / 32) * ((N + 31) / 32) >= AWQ_GEMM_MIN_TILES;
}
hipError_t launch_awq_gemm(int M, int N, int K, const void *, const void *, const void *, const void *,
                           const void *, void *, hipStream_t) {
    return rec("awq_gemm", M, N, K);
}
}  // namespace svdq
