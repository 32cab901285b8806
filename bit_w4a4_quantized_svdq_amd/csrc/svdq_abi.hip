// svdq_abi.hip -- the C ABI of libsvdq (declared in include/svdq.h): host-side
// argument checks, a per-device architecture check, and dispatch to the
// gfx950 kernels.  Every check runs before anything is enqueued.
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <cstdint>

#include "../../include/svdq.h"
#include "launch.h"

namespace {

thread_local char g_last_error[256] = "";

svdq_status fail(svdq_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int64_t kMaxMN = int64_t(1) << 24;
constexpr int64_t kMaxK = int64_t(1) << 16;

// 0 = unknown, 1 = gfx950, 2 = other; one slot per device ordinal.
std::atomic<int> g_arch_ok[64];

svdq_status check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(SVDQ_ERR_HIP, "hipGetDevice failed");
    if (dev < 0 || dev >= 64) return fail(SVDQ_ERR_UNSUPPORTED, "device ordinal %d out of range", dev);
    int v = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return fail(SVDQ_ERR_HIP, "hipGetDeviceProperties failed");
        v = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_arch_ok[dev].store(v, std::memory_order_relaxed);
    }
    if (v != 1) return fail(SVDQ_ERR_UNSUPPORTED, "libsvdq runs on gfx950 (MI355X) only");
    return SVDQ_OK;
}

svdq_status check_shape(int64_t M, int64_t N, int64_t K, int32_t rank) {
    if (M < 0 || N < 0 || M > kMaxMN || N > kMaxMN)
        return fail(SVDQ_ERR_INVALID_ARG, "M and N must be in [0, 2^24] (M=%lld N=%lld)",
                    (long long)M, (long long)N);
    if (K <= 0 || K % 64 != 0 || K > kMaxK)
        return fail(SVDQ_ERR_INVALID_ARG, "K must be a positive multiple of 64 up to 2^16 (K=%lld)",
                    (long long)K);
    if (rank < 0 || rank > 128 || rank % 16 != 0)
        return fail(SVDQ_ERR_INVALID_ARG, "rank must be a multiple of 16 in [0, 128] (rank=%d)", rank);
    return SVDQ_OK;
}

svdq_status check_ptr(const void *p, const char *name, bool may_be_null) {
    if (!p) return may_be_null ? SVDQ_OK : fail(SVDQ_ERR_INVALID_ARG, "%s must not be NULL", name);
    if (!aligned16(p)) return fail(SVDQ_ERR_INVALID_ARG, "%s must be 16-byte aligned", name);
    return SVDQ_OK;
}

// The kernels use one-dimensional grids of (M/tm) * (N/tn) blocks.
svdq_status check_grid(int64_t M, int64_t N, int64_t tm, int64_t tn) {
    const int64_t blocks = ((M + tm - 1) / tm) * ((N + tn - 1) / tn);
    if (blocks > INT32_MAX)
        return fail(SVDQ_ERR_INVALID_ARG, "problem too large: %lld thread blocks", (long long)blocks);
    return SVDQ_OK;
}

#define SVDQ_TRY(expr)                      \
    do {                                    \
        svdq_status _st = (expr);           \
        if (_st != SVDQ_OK) return _st;     \
    } while (0)

svdq_status launched(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(SVDQ_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
    g_last_error[0] = '\0';
    return SVDQ_OK;
}

}  // namespace

extern "C" {

static svdq_status quantize_act_common(bool gelu, const char *name, int32_t precision, int64_t M,
                                       int64_t K, int32_t rank, const void *x, const void *smooth,
                                       const void *lora_down, void *act_codes, void *act_scales,
                                       float *lora_act, void *stream)
{
    if (precision != SVDQ_INT4 && precision != SVDQ_NVFP4 && precision != SVDQ_INT4_FP6)
        return fail(SVDQ_ERR_UNSUPPORTED, "precision must be SVDQ_INT4, SVDQ_NVFP4 or SVDQ_INT4_FP6 (got %d)",
                    precision);
    SVDQ_TRY(check_shape(M, 1, K, rank));
    SVDQ_TRY(check_ptr(x, "x", false));
    SVDQ_TRY(check_ptr(smooth, "smooth", true));
    SVDQ_TRY(check_ptr(lora_down, "lora_down", rank == 0));
    SVDQ_TRY(check_ptr(act_codes, "act_codes", false));
    SVDQ_TRY(check_ptr(act_scales, "act_scales", false));
    SVDQ_TRY(check_ptr(lora_act, "lora_act", rank == 0));
    if (M == 0) return SVDQ_OK;
    SVDQ_TRY(check_device());
    const int kernel_prec = precision == SVDQ_INT4_FP6 ? 2 : precision;
    return launched(svdq::launch_quantize_act(kernel_prec, gelu, (int)M, (int)K, rank, x, smooth, lora_down,
                                              act_codes, act_scales, lora_act, (hipStream_t)stream),
                    name);
}

svdq_status svdq_quantize_act(int32_t precision, int64_t M, int64_t K, int32_t rank,
                              const void *x, const void *smooth, const void *lora_down,
                              void *act_codes, void *act_scales, float *lora_act, void *stream)
{
    return quantize_act_common(false, "svdq_quantize_act", precision, M, K, rank, x, smooth, lora_down,
                               act_codes, act_scales, lora_act, stream);
}

svdq_status svdq_gelu_quantize_act(int32_t precision, int64_t M, int64_t K, int32_t rank,
                                   const void *x, const void *smooth, const void *lora_down,
                                   void *act_codes, void *act_scales, float *lora_act, void *stream)
{
    return quantize_act_common(true, "svdq_gelu_quantize_act", precision, M, K, rank, x, smooth,
                               lora_down, act_codes, act_scales, lora_act, stream);
}

svdq_status svdq_smooth_factors(int64_t M, int64_t N, int64_t K, const void *x, const void *W, void *smooth,
                                void *stream)
{
    SVDQ_TRY(check_shape(M, N, K, 0));
    SVDQ_TRY(check_ptr(x, "x", false));
    SVDQ_TRY(check_ptr(W, "W", false));
    SVDQ_TRY(check_ptr(smooth, "smooth", false));
    SVDQ_TRY(check_device());
    return launched(svdq::launch_smooth_factors((int)M, (int)N, (int)K, x, W, smooth, (hipStream_t)stream),
                    "svdq_smooth_factors");
}

int64_t svdq_lowrank_workspace_bytes(int64_t N, int64_t K, int32_t rank)
{
    if (check_shape(1, N, K, rank) != SVDQ_OK || rank < 16 || N < rank + 8 || K < rank + 8) return -1;
    return (int64_t)svdq::lowrank_workspace_bytes((int)N, (int)K, rank);
}

svdq_status svdq_lowrank_factors(int64_t N, int64_t K, int32_t rank, const void *W, const void *smooth,
                                 uint64_t seed, void *workspace, int64_t workspace_bytes, void *lora_up,
                                 void *lora_down, void *stream)
{
    SVDQ_TRY(check_shape(1, N, K, rank));
    if (rank < 16)
        return fail(SVDQ_ERR_INVALID_ARG, "rank must be at least 16 (got %d)", rank);
    if (N < rank + 8 || K < rank + 8)
        return fail(SVDQ_ERR_INVALID_ARG, "N and K must be at least rank + 8 (got N=%lld, K=%lld)", (long long)N,
                    (long long)K);
    SVDQ_TRY(check_ptr(W, "W", false));
    SVDQ_TRY(check_ptr(smooth, "smooth", true));
    SVDQ_TRY(check_ptr(workspace, "workspace", false));
    SVDQ_TRY(check_ptr(lora_up, "lora_up", false));
    SVDQ_TRY(check_ptr(lora_down, "lora_down", false));
    const int64_t need = (int64_t)svdq::lowrank_workspace_bytes((int)N, (int)K, rank);
    if (workspace_bytes < need)
        return fail(SVDQ_ERR_INVALID_ARG, "workspace too small: %lld bytes, %lld needed", (long long)workspace_bytes,
                    (long long)need);
    SVDQ_TRY(check_device());
    return launched(svdq::launch_lowrank_factors((int)N, (int)K, rank, W, smooth, seed, workspace, lora_up, lora_down,
                                                 (hipStream_t)stream),
                    "svdq_lowrank_factors");
}

svdq_status svdq_lowrank_factors_noalloc(int64_t N, int64_t K, int32_t rank, const void *W, const void *smooth,
                                         uint64_t seed, void *lora_up, void *lora_down, void *stream)
{
    SVDQ_TRY(check_shape(1, N, K, rank));
    if (rank < 16)
        return fail(SVDQ_ERR_INVALID_ARG, "rank must be at least 16 (got %d)", rank);
    if (N < rank + 8 || K < rank + 8)
        return fail(SVDQ_ERR_INVALID_ARG, "N and K must be at least rank + 8 (got N=%lld, K=%lld)", (long long)N,
                    (long long)K);
    SVDQ_TRY(check_ptr(W, "W", false));
    SVDQ_TRY(check_ptr(smooth, "smooth", true));
    SVDQ_TRY(check_ptr(lora_up, "lora_up", false));
    SVDQ_TRY(check_ptr(lora_down, "lora_down", false));
    const size_t need = svdq::lowrank_workspace_bytes((int)N, (int)K, rank);
    if (need > svdq::LOWRANK_SCRATCH_BYTES)
        return fail(SVDQ_ERR_INVALID_ARG,
                    "N=%lld K=%lld rank=%d needs %zu bytes of scratch, more than the fixed %zu; "
                    "use svdq_lowrank_factors with a workspace", (long long)N, (long long)K, rank, need,
                    svdq::LOWRANK_SCRATCH_BYTES);
    SVDQ_TRY(check_device());
    void *ws = nullptr;
    const hipError_t e = svdq::lowrank_scratch(&ws);
    if (e != hipSuccess)
        return fail(SVDQ_ERR_HIP, "svdq_lowrank_factors_noalloc: scratch address lookup failed: %s",
                    hipGetErrorString(e));
    return launched(svdq::launch_lowrank_factors((int)N, (int)K, rank, W, smooth, seed, ws, lora_up, lora_down,
                                                 (hipStream_t)stream),
                    "svdq_lowrank_factors_noalloc");
}

svdq_status svdq_quantize_weight(int32_t precision, int64_t N, int64_t K, int32_t rank, const void *W,
                                 const void *smooth, const void *lora_up, const void *lora_down,
                                 void *wgt_codes, void *wgt_scales, void *stream)
{
    if (precision != SVDQ_INT4 && precision != SVDQ_NVFP4)
        return fail(SVDQ_ERR_UNSUPPORTED, "precision must be SVDQ_INT4 or SVDQ_NVFP4 (got %d)", precision);
    SVDQ_TRY(check_shape(1, N, K, rank));
    SVDQ_TRY(check_ptr(W, "W", false));
    SVDQ_TRY(check_ptr(smooth, "smooth", true));
    SVDQ_TRY(check_ptr(lora_up, "lora_up", rank == 0));
    SVDQ_TRY(check_ptr(lora_down, "lora_down", rank == 0));
    SVDQ_TRY(check_ptr(wgt_codes, "wgt_codes", false));
    SVDQ_TRY(check_ptr(wgt_scales, "wgt_scales", false));
    if (N == 0) return SVDQ_OK;
    SVDQ_TRY(check_device());
    return launched(svdq::launch_quantize_weight(precision, (int)N, (int)K, rank, W, smooth, lora_up, lora_down,
                                                 wgt_codes, wgt_scales, (hipStream_t)stream),
                    "svdq_quantize_weight");
}

svdq_status svdq_debug_gelu_bf16(int64_t n, const void *x, void *out, void *stream)
{
    if (n < 0 || n > ((int64_t)1 << 36)) return fail(SVDQ_ERR_INVALID_ARG, "n out of range (got %lld)", (long long)n);
    SVDQ_TRY(check_ptr(x, "x", false));
    SVDQ_TRY(check_ptr(out, "out", false));
    if (n == 0) return SVDQ_OK;
    SVDQ_TRY(check_device());
    return launched(svdq::launch_gelu_bf16(n, x, out, (hipStream_t)stream), "svdq_debug_gelu_bf16");
}

svdq_status svdq_gemm_w4a4_qk_norm_rope(int32_t precision, int64_t M, int64_t N, int64_t K, int32_t rank,
                                        const void *act_codes, const void *act_scales,
                                        const void *wgt_codes, const void *wgt_scales, float alpha,
                                        const float *lora_act, const void *lora_up, const void *bias,
                                        const void *q_norm_weight, const void *k_norm_weight, float eps,
                                        const float *rope_cos, const float *rope_sin, void *out,
                                        void *stream)
{
    if (precision != SVDQ_INT4 && precision != SVDQ_NVFP4 && precision != SVDQ_INT4_PACKED &&
        precision != SVDQ_INT4_FP6)
        return fail(SVDQ_ERR_UNSUPPORTED,
                    "precision must be SVDQ_INT4, SVDQ_NVFP4, SVDQ_INT4_PACKED or SVDQ_INT4_FP6 (got %d)", precision);
    SVDQ_TRY(check_shape(M, N, K, rank));
    if (N % 384 != 0)
        return fail(SVDQ_ERR_INVALID_ARG, "N must be 3 * heads * 128 (got %lld)", (long long)N);
    if (!(eps >= 0.0f) || eps > 3.0e38f)
        return fail(SVDQ_ERR_INVALID_ARG, "eps must be finite and >= 0");
    SVDQ_TRY(check_ptr(act_codes, "act_codes", false));
    SVDQ_TRY(check_ptr(act_scales, "act_scales", false));
    SVDQ_TRY(check_ptr(wgt_codes, "wgt_codes", false));
    SVDQ_TRY(check_ptr(wgt_scales, "wgt_scales", false));
    SVDQ_TRY(check_ptr(lora_act, "lora_act", rank == 0));
    SVDQ_TRY(check_ptr(lora_up, "lora_up", rank == 0));
    SVDQ_TRY(check_ptr(bias, "bias", true));
    SVDQ_TRY(check_ptr(q_norm_weight, "q_norm_weight", false));
    SVDQ_TRY(check_ptr(k_norm_weight, "k_norm_weight", false));
    SVDQ_TRY(check_ptr(rope_cos, "rope_cos", false));
    SVDQ_TRY(check_ptr(rope_sin, "rope_sin", false));
    SVDQ_TRY(check_ptr(out, "out", false));
    if (M == 0) return SVDQ_OK;
    SVDQ_TRY(check_grid(M, N, 128, 128));
    SVDQ_TRY(check_device());
    svdq::QkNormRope qk;
    qk.q_w = (const uint16_t *)q_norm_weight;
    qk.k_w = (const uint16_t *)k_norm_weight;
    qk.cos = rope_cos;
    qk.sin = rope_sin;
    qk.eps = eps;
    qk.qk_cols = (int)(2 * (N / 3));
    const hipError_t e = precision == SVDQ_INT4_FP6
        ? svdq::launch_gemm_w4a4_fp6_qk((int)M, (int)N, (int)K, rank, act_codes, act_scales, wgt_codes, wgt_scales,
                                        alpha, lora_act, lora_up, bias, qk, out, (hipStream_t)stream)
        : precision != SVDQ_NVFP4
        ? svdq::launch_gemm_w4a4_int4_qk(precision == SVDQ_INT4_PACKED, (int)M, (int)N, (int)K, rank, act_codes,
                                         act_scales, wgt_codes, wgt_scales, alpha, lora_act, lora_up, bias, qk, out,
                                         (hipStream_t)stream)
        : svdq::launch_gemm_w4a4_nvfp4_qk((int)M, (int)N, (int)K, rank, act_codes, act_scales, wgt_codes,
                                          wgt_scales, alpha, lora_act, lora_up, bias, qk, out, (hipStream_t)stream);
    return launched(e, "svdq_gemm_w4a4_qk_norm_rope");
}

int64_t svdq_gelu_quantize_workspace_bytes(int64_t M, int64_t N, int32_t rank_next)
{
    if (check_shape(M, 1, N, rank_next) != SVDQ_OK) return -1;
    return (int64_t)svdq::gelu_quant_workspace_bytes((int)M, (int)N, rank_next);
}

svdq_status svdq_gemm_w4a4_gelu_quantize(int32_t precision, int64_t M, int64_t N, int64_t K, int32_t rank,
                                         const void *act_codes, const void *act_scales,
                                         const void *wgt_codes, const void *wgt_scales, float alpha,
                                         const float *lora_act, const void *lora_up, const void *bias,
                                         int32_t rank_next, const void *smooth_next, const void *lora_down_next,
                                         void *next_codes, void *next_scales, float *next_lora_act,
                                         void *workspace, int64_t workspace_bytes, void *out, void *stream)
{
    if (precision != SVDQ_INT4_FP6)
        return fail(SVDQ_ERR_UNSUPPORTED, "svdq_gemm_w4a4_gelu_quantize takes SVDQ_INT4_FP6 only (got %d)",
                    precision);
    SVDQ_TRY(check_shape(M, N, K, rank));
    if (N == 0 || N % 64 != 0 || N > kMaxK || rank_next < 0 || rank_next > 128 || rank_next % 16 != 0)
        return fail(SVDQ_ERR_INVALID_ARG,
                    "N must be a positive multiple of 64 up to 2^16 and rank_next a multiple of 16 in [0, 128] "
                    "(N=%lld rank_next=%d)", (long long)N, rank_next);
    SVDQ_TRY(check_ptr(act_codes, "act_codes", false));
    SVDQ_TRY(check_ptr(act_scales, "act_scales", false));
    SVDQ_TRY(check_ptr(wgt_codes, "wgt_codes", false));
    SVDQ_TRY(check_ptr(wgt_scales, "wgt_scales", false));
    SVDQ_TRY(check_ptr(lora_act, "lora_act", rank == 0));
    SVDQ_TRY(check_ptr(lora_up, "lora_up", rank == 0));
    SVDQ_TRY(check_ptr(bias, "bias", true));
    SVDQ_TRY(check_ptr(smooth_next, "smooth_next", true));
    SVDQ_TRY(check_ptr(lora_down_next, "lora_down_next", rank_next == 0));
    SVDQ_TRY(check_ptr(next_codes, "next_codes", false));
    SVDQ_TRY(check_ptr(next_scales, "next_scales", false));
    SVDQ_TRY(check_ptr(next_lora_act, "next_lora_act", rank_next == 0));
    const int64_t need = (int64_t)svdq::gelu_quant_workspace_bytes((int)M, (int)N, rank_next);
    SVDQ_TRY(check_ptr(workspace, "workspace", need == 0));
    SVDQ_TRY(check_ptr(out, "out", true));
    if (workspace_bytes < need)
        return fail(SVDQ_ERR_INVALID_ARG, "workspace too small: %lld bytes, %lld needed", (long long)workspace_bytes,
                    (long long)need);
    if (M == 0) return SVDQ_OK;
    SVDQ_TRY(check_grid(M, N, 128, 128));
    SVDQ_TRY(check_device());
    return launched(svdq::launch_gemm_w4a4_fp6_gelu_quant((int)M, (int)N, (int)K, rank, act_codes, act_scales,
                                                          wgt_codes, wgt_scales, alpha, lora_act, lora_up, bias,
                                                          rank_next, smooth_next, lora_down_next, next_codes,
                                                          next_scales, next_lora_act, workspace, out,
                                                          (hipStream_t)stream),
                    "svdq_gemm_w4a4_gelu_quantize");
}

svdq_status svdq_gemm_w4a4(int32_t precision, int64_t M, int64_t N, int64_t K, int32_t rank,
                           const void *act_codes, const void *act_scales, const void *wgt_codes,
                           const void *wgt_scales, float alpha, const float *lora_act,
                           const void *lora_up, const void *bias, void *out, void *stream)
{
    if (precision != SVDQ_INT4 && precision != SVDQ_NVFP4 && precision != SVDQ_INT4_PACKED &&
        precision != SVDQ_INT4_FP6)
        return fail(SVDQ_ERR_UNSUPPORTED,
                    "precision must be SVDQ_INT4, SVDQ_NVFP4, SVDQ_INT4_PACKED or SVDQ_INT4_FP6 (got %d)", precision);
    SVDQ_TRY(check_shape(M, N, K, rank));
    SVDQ_TRY(check_ptr(act_codes, "act_codes", false));
    SVDQ_TRY(check_ptr(act_scales, "act_scales", false));
    SVDQ_TRY(check_ptr(wgt_codes, "wgt_codes", false));
    SVDQ_TRY(check_ptr(wgt_scales, "wgt_scales", false));
    SVDQ_TRY(check_ptr(lora_act, "lora_act", rank == 0));
    SVDQ_TRY(check_ptr(lora_up, "lora_up", rank == 0));
    SVDQ_TRY(check_ptr(bias, "bias", true));
    SVDQ_TRY(check_ptr(out, "out", false));
    if (M == 0 || N == 0) return SVDQ_OK;
    SVDQ_TRY(check_grid(M, N, 128, 128));
    SVDQ_TRY(check_device());
    hipError_t e = precision == SVDQ_INT4_FP6
        ? svdq::launch_gemm_w4a4_fp6((int)M, (int)N, (int)K, rank, act_codes, act_scales, wgt_codes, wgt_scales,
                                     alpha, lora_act, lora_up, bias, out, (hipStream_t)stream)
        : precision != SVDQ_NVFP4
        ? svdq::launch_gemm_w4a4_int4(precision == SVDQ_INT4_PACKED, (int)M, (int)N, (int)K, rank, act_codes,
                                      act_scales, wgt_codes, wgt_scales, alpha, lora_act, lora_up, bias, out,
                                      (hipStream_t)stream)
        : svdq::launch_gemm_w4a4_nvfp4((int)M, (int)N, (int)K, rank, act_codes, act_scales, wgt_codes,
                                       wgt_scales, alpha, lora_act, lora_up, bias, out, (hipStream_t)stream);
    return launched(e, "svdq_gemm_w4a4");
}

svdq_status awq_gemv_w4a16(int64_t M, int64_t N, int64_t K, int32_t group_size, const void *x,
                           const void *wgt_codes, const void *wgt_scales, const void *wgt_zeros,
                           const void *bias, void *out, void *stream)
{
    if (group_size != 64)
        return fail(SVDQ_ERR_UNSUPPORTED, "awq_w4a16 supports group_size 64 only (got %d)", group_size);
    SVDQ_TRY(check_shape(M, N, K, 0));
    SVDQ_TRY(check_ptr(x, "x", false));
    SVDQ_TRY(check_ptr(wgt_codes, "wgt_codes", false));
    SVDQ_TRY(check_ptr(wgt_scales, "wgt_scales", false));
    SVDQ_TRY(check_ptr(wgt_zeros, "wgt_zeros", false));
    SVDQ_TRY(check_ptr(bias, "bias", true));
    SVDQ_TRY(check_ptr(out, "out", false));
    if (M == 0 || N == 0) return SVDQ_OK;
    SVDQ_TRY(check_grid(M, N, 64, 16));
    SVDQ_TRY(check_device());
    const hipError_t e = svdq::awq_gemm_applies((int)M, (int)N, (int)K)
        ? svdq::launch_awq_gemm((int)M, (int)N, (int)K, x, wgt_codes, wgt_scales, wgt_zeros, bias, out,
                                (hipStream_t)stream)
        : svdq::launch_awq_gemv((int)M, (int)N, (int)K, x, wgt_codes, wgt_scales, wgt_zeros, bias, out,
                                (hipStream_t)stream);
    return launched(e, "awq_gemv_w4a16");
}

// layout: 0 nibbles, 1 packed weight (fp8 formulation), 2 FP6 layout of both operands
static svdq_status group_sums_common(int layout, const char *name, int64_t M, int64_t N, int64_t K,
                                     const void *act_codes, const void *wgt_codes, int32_t *G, void *stream)
{
    SVDQ_TRY(check_shape(M, N, K, 0));
    SVDQ_TRY(check_ptr(act_codes, "act_codes", false));
    SVDQ_TRY(check_ptr(wgt_codes, layout == 1 ? "packed_weight" : layout == 2 ? "fp6_weight" : "wgt_codes", false));
    SVDQ_TRY(check_ptr(G, "G", false));
    if (M == 0 || N == 0) return SVDQ_OK;
    SVDQ_TRY(check_grid(M, N, 128, 128));
    SVDQ_TRY(check_device());
    const hipError_t e = layout == 2
        ? svdq::launch_group_sums_fp6((int)M, (int)N, (int)K, act_codes, wgt_codes, G, (hipStream_t)stream)
        : svdq::launch_group_sums_int4(layout == 1, (int)M, (int)N, (int)K, act_codes, wgt_codes, G,
                                       (hipStream_t)stream);
    return launched(e, name);
}

svdq_status svdq_debug_group_sums(int64_t M, int64_t N, int64_t K, const void *act_codes,
                                  const void *wgt_codes, int32_t *G, void *stream)
{
    return group_sums_common(0, "svdq_debug_group_sums", M, N, K, act_codes, wgt_codes, G, stream);
}

svdq_status svdq_debug_group_sums_packed(int64_t M, int64_t N, int64_t K, const void *act_codes,
                                         const void *packed_weight, int32_t *G, void *stream)
{
    return group_sums_common(1, "svdq_debug_group_sums_packed", M, N, K, act_codes, packed_weight, G, stream);
}

svdq_status svdq_debug_group_sums_fp6(int64_t M, int64_t N, int64_t K, const void *act_codes,
                                      const void *fp6_weight, int32_t *G, void *stream)
{
    return group_sums_common(2, "svdq_debug_group_sums_fp6", M, N, K, act_codes, fp6_weight, G, stream);
}

int64_t svdq_fp6_codes_bytes(int64_t rows, int64_t K)
{
    if (check_shape(rows, 1, K, 0) != SVDQ_OK) return -1;
    return (int64_t)svdq::fp6_weight_bytes((int)rows, (int)K);
}

svdq_status svdq_pack_weight_fp6(int64_t N, int64_t K, const void *wgt_codes, void *fp6_weight, void *stream)
{
    SVDQ_TRY(check_shape(1, N, K, 0));
    SVDQ_TRY(check_ptr(wgt_codes, "wgt_codes", false));
    SVDQ_TRY(check_ptr(fp6_weight, "fp6_weight", false));
    if (N == 0) return SVDQ_OK;
    SVDQ_TRY(check_device());
    return launched(svdq::launch_pack_weight_fp6((int)N, (int)K, wgt_codes, fp6_weight, (hipStream_t)stream),
                    "svdq_pack_weight_fp6");
}

int64_t svdq_packed_weight_bytes(int64_t N, int64_t K)
{
    if (check_shape(1, N, K, 0) != SVDQ_OK) return -1;
    return (int64_t)svdq::packed_weight_bytes((int)N, (int)K);
}

svdq_status svdq_pack_weight_int4(int64_t N, int64_t K, const void *wgt_codes, const void *wgt_scales,
                                  void *packed_weight, int32_t *invalid_codes, void *stream)
{
    SVDQ_TRY(check_shape(1, N, K, 0));
    SVDQ_TRY(check_ptr(wgt_codes, "wgt_codes", false));
    SVDQ_TRY(check_ptr(wgt_scales, "wgt_scales", false));
    SVDQ_TRY(check_ptr(packed_weight, "packed_weight", false));
    if (invalid_codes && ((uintptr_t)invalid_codes & 3u))
        return fail(SVDQ_ERR_INVALID_ARG, "invalid_codes must be 4-byte aligned");
    if (N == 0) return SVDQ_OK;
    SVDQ_TRY(check_device());
    return launched(svdq::launch_pack_weight_int4((int)N, (int)K, wgt_codes, wgt_scales, packed_weight, invalid_codes,
                                                  (hipStream_t)stream),
                    "svdq_pack_weight_int4");
}

svdq_status svdq_debug_stream_read(const void *src, int64_t bytes, int32_t pattern, uint32_t *out, void *stream)
{
    if (bytes < 0 || bytes > ((int64_t)1 << 40)) return fail(SVDQ_ERR_INVALID_ARG, "bytes out of range");
    if (pattern != 0 && pattern != 1) return fail(SVDQ_ERR_INVALID_ARG, "pattern must be 0 or 1");
    SVDQ_TRY(check_ptr(src, "src", false));
    if (!out || ((uintptr_t)out & 3u)) return fail(SVDQ_ERR_INVALID_ARG, "out must be a 4-byte aligned pointer");
    if (bytes == 0) return SVDQ_OK;
    SVDQ_TRY(check_device());
    return launched(svdq::launch_stream_read(src, bytes, pattern == 1, out, (hipStream_t)stream), "svdq_debug_stream_read");
}

const char *svdq_status_string(svdq_status s)
{
    switch (s) {
        case SVDQ_OK: return "SVDQ_OK";
        case SVDQ_ERR_INVALID_ARG: return "SVDQ_ERR_INVALID_ARG: an argument failed the host-side checks";
        case SVDQ_ERR_UNSUPPORTED: return "SVDQ_ERR_UNSUPPORTED: precision, group size or device not supported";
        case SVDQ_ERR_HIP: return "SVDQ_ERR_HIP: a HIP runtime call or kernel launch failed";
    }
    return "unknown svdq_status";
}

const char *svdq_last_error(void) { return g_last_error; }

int32_t svdq_abi_version(void) { return 11; }

}  // extern "C"
