// Drives every entry point of include/svdq.h through the host-compiled C ABI
// layer (abi_host.cpp + hip_stubs.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer: a valid call must reach the right launcher
// with the caller's sizes; each invalid argument must be rejected with the
// documented status before any launcher runs; an unsupported device and a
// failed launch must come back as statuses with a message.  Prints
// "abi sanitize ok" and exits 0 when every expectation holds.
#include <cstdio>
#include <cstring>

#include "../../include/svdq.h"
#include "stub_log.h"

static int failures = 0;

#define EXPECT(cond, ...)                                             \
    do {                                                              \
        if (!(cond)) {                                                \
            std::fprintf(stderr, "line %d: ", __LINE__);              \
            std::fprintf(stderr, __VA_ARGS__);                        \
            std::fprintf(stderr, " (last error: %s)\n", svdq_last_error()); \
            ++failures;                                               \
        }                                                             \
    } while (0)

// fake, 16-byte aligned device addresses (never dereferenced)
static void *const P = (void *)(uintptr_t)0x100000;
static void *const MIS = (void *)(uintptr_t)0x100008;
static float *const F = (float *)P;
static int32_t *const I = (int32_t *)P;

static void expect_launch(svdq_status st, const char *name, long long a, long long b, long long c) {
    EXPECT(st == SVDQ_OK, "%s: status %d", name, (int)st);
    EXPECT(g_stub.calls == 1 && std::strcmp(g_stub.last, name) == 0, "%s: launcher %s called %d times",
           name, g_stub.last, g_stub.calls);
    EXPECT(g_stub.a == a && g_stub.b == b && g_stub.c == c, "%s: sizes %lld %lld %lld", name, g_stub.a,
           g_stub.b, g_stub.c);
    g_stub.calls = 0;
    g_stub.last[0] = '\0';
}

static void expect_reject(svdq_status st, svdq_status want, const char *what) {
    EXPECT(st == want, "%s: status %d, expected %d", what, (int)st, (int)want);
    EXPECT(g_stub.calls == 0, "%s: a launcher ran (%s)", what, g_stub.last);
    EXPECT(std::strlen(svdq_last_error()) > 0, "%s: no error message", what);
    g_stub.calls = 0;
}

static void expect_noop(svdq_status st, const char *what) {
    EXPECT(st == SVDQ_OK && g_stub.calls == 0, "%s: status %d, %d launches", what, (int)st, g_stub.calls);
    g_stub.calls = 0;
}

int main() {
    const svdq_status INV = SVDQ_ERR_INVALID_ARG, UNS = SVDQ_ERR_UNSUPPORTED;

    // ---- activation step (plain and GELU-fed)
    for (int gelu = 0; gelu < 2; ++gelu) {
        auto qa = gelu ? svdq_gelu_quantize_act : svdq_quantize_act;
        const char *name = gelu ? "quantize_act_gelu" : "quantize_act";
        expect_launch(qa(SVDQ_INT4, 4096, 3072, 32, P, P, P, P, P, F, nullptr), name, 4096, 3072, 32);
        expect_launch(qa(SVDQ_NVFP4, 33, 4160, 0, P, nullptr, nullptr, P, P, nullptr, nullptr), name, 33, 4160, 1000);
        expect_noop(qa(SVDQ_INT4, 0, 64, 16, P, P, P, P, P, F, nullptr), "quantize M=0");
        expect_reject(qa(2, 4, 64, 16, P, P, P, P, P, F, nullptr), UNS, "precision 2");
        expect_launch(qa(SVDQ_INT4_FP6, 4096, 3072, 32, P, P, P, P, P, F, nullptr), name, 4096, 3072, 2032);
        expect_reject(qa(SVDQ_INT4_FP6, 4, 96, 16, P, P, P, P, P, F, nullptr), INV, "fp6 K % 64");
        expect_reject(qa(4, 4, 64, 16, P, P, P, P, P, F, nullptr), UNS, "precision 4");
        expect_reject(qa(SVDQ_INT4, -1, 64, 16, P, P, P, P, P, F, nullptr), INV, "M < 0");
        expect_reject(qa(SVDQ_INT4, (1ll << 24) + 1, 64, 16, P, P, P, P, P, F, nullptr), INV, "M > 2^24");
        expect_reject(qa(SVDQ_INT4, 4, 96, 16, P, P, P, P, P, F, nullptr), INV, "K % 64");
        expect_reject(qa(SVDQ_INT4, 4, 0, 16, P, P, P, P, P, F, nullptr), INV, "K = 0");
        expect_reject(qa(SVDQ_INT4, 4, (1 << 16) + 64, 16, P, P, P, P, P, F, nullptr), INV, "K > 2^16");
        expect_reject(qa(SVDQ_INT4, 4, 64, 24, P, P, P, P, P, F, nullptr), INV, "rank 24");
        expect_reject(qa(SVDQ_INT4, 4, 64, 144, P, P, P, P, P, F, nullptr), INV, "rank 144");
        expect_reject(qa(SVDQ_INT4, 4, 64, 16, nullptr, P, P, P, P, F, nullptr), INV, "x NULL");
        expect_reject(qa(SVDQ_INT4, 4, 64, 16, MIS, P, P, P, P, F, nullptr), INV, "x misaligned");
        expect_reject(qa(SVDQ_INT4, 4, 64, 16, P, MIS, P, P, P, F, nullptr), INV, "smooth misaligned");
        expect_reject(qa(SVDQ_INT4, 4, 64, 16, P, P, nullptr, P, P, F, nullptr), INV, "lora_down NULL");
        expect_reject(qa(SVDQ_INT4, 4, 64, 16, P, P, P, nullptr, P, F, nullptr), INV, "codes NULL");
        expect_reject(qa(SVDQ_INT4, 4, 64, 16, P, P, P, P, MIS, F, nullptr), INV, "scales misaligned");
        expect_reject(qa(SVDQ_INT4, 4, 64, 16, P, P, P, P, P, nullptr, nullptr), INV, "lora_act NULL");
    }

    // ---- W4A4 GEMM
    expect_launch(svdq_gemm_w4a4(SVDQ_INT4, 4096, 12288, 3072, 32, P, P, P, P, 1.0f, F, P, P, P, nullptr),
                  "gemm_int4", 4096, 12288, 3072);
    expect_launch(svdq_gemm_w4a4(SVDQ_NVFP4, 5, 70, 4160, 0, P, P, P, P, 0.5f, nullptr, nullptr, nullptr, P,
                                 nullptr),
                  "gemm_nvfp4", 5, 70, 4160);
    expect_noop(svdq_gemm_w4a4(SVDQ_INT4, 7, 0, 64, 0, P, P, P, P, 1.0f, nullptr, nullptr, nullptr, P, nullptr),
                "gemm N=0");
    expect_reject(svdq_gemm_w4a4(7, 4, 64, 64, 0, P, P, P, P, 1.0f, nullptr, nullptr, nullptr, P, nullptr), UNS,
                  "gemm precision");
    expect_reject(svdq_gemm_w4a4(SVDQ_INT4, 4, -64, 64, 0, P, P, P, P, 1.0f, nullptr, nullptr, nullptr, P, nullptr),
                  INV, "gemm N < 0");
    expect_reject(svdq_gemm_w4a4(SVDQ_INT4, 4, 64, 64, 16, P, P, P, P, 1.0f, nullptr, P, nullptr, P, nullptr), INV,
                  "gemm lora_act NULL");
    expect_reject(svdq_gemm_w4a4(SVDQ_INT4, 4, 64, 64, 16, P, P, P, P, 1.0f, F, nullptr, nullptr, P, nullptr), INV,
                  "gemm lora_up NULL");
    expect_reject(svdq_gemm_w4a4(SVDQ_INT4, 4, 64, 64, 0, P, P, P, P, 1.0f, nullptr, nullptr, MIS, P, nullptr), INV,
                  "gemm bias misaligned");
    expect_reject(svdq_gemm_w4a4(SVDQ_INT4, 4, 64, 64, 0, P, P, nullptr, P, 1.0f, nullptr, nullptr, nullptr, P,
                                 nullptr),
                  INV, "gemm wgt_codes NULL");
    expect_reject(svdq_gemm_w4a4(SVDQ_INT4, 4, 64, 64, 0, P, P, P, P, 1.0f, nullptr, nullptr, nullptr, MIS,
                                 nullptr),
                  INV, "gemm out misaligned");

    expect_launch(svdq_gemm_w4a4(SVDQ_INT4_PACKED, 4096, 12288, 3072, 32, P, P, P, P, 1.0f, F, P, P, P, nullptr),
                  "gemm_int4_packed", 4096, 12288, 3072);
    expect_launch(svdq_gemm_w4a4(SVDQ_INT4_FP6, 4096, 12288, 3072, 32, P, P, P, P, 1.0f, F, P, P, P, nullptr),
                  "gemm_fp6", 4096, 12288, 3072);
    expect_reject(svdq_gemm_w4a4(SVDQ_INT4_FP6, 4, 64, 64, 16, P, P, P, P, 1.0f, nullptr, P, nullptr, P, nullptr),
                  INV, "gemm fp6 lora_act NULL");
    expect_reject(svdq_gemm_w4a4(4, 4, 64, 64, 0, P, P, P, P, 1.0f, nullptr, nullptr, nullptr, P, nullptr), UNS,
                  "gemm precision 4");

    // ---- FP6 layout of int4 weights
    EXPECT(svdq_fp6_codes_bytes(12288, 3072) == 12288ll * 3072 * 3 / 4, "fp6 bytes");
    EXPECT(svdq_fp6_codes_bytes(130, 4160) == 2ll * 33 * 12288, "fp6 bytes, padded tile and pair");
    EXPECT(svdq_fp6_codes_bytes(8, 100) == -1, "fp6 bytes, K % 64");
    expect_launch(svdq_pack_weight_fp6(12288, 3072, P, P, nullptr), "pack_weight_fp6", 12288, 3072, 0);
    expect_noop(svdq_pack_weight_fp6(0, 64, P, P, nullptr), "pack fp6 N=0");
    expect_reject(svdq_pack_weight_fp6(5, 64, nullptr, P, nullptr), INV, "pack fp6 codes NULL");
    expect_reject(svdq_pack_weight_fp6(5, 64, P, MIS, nullptr), INV, "pack fp6 out misaligned");
    expect_launch(svdq_debug_group_sums_fp6(130, 384, 3072, P, P, I, nullptr), "group_sums_fp6", 130, 384, 3072);
    expect_reject(svdq_debug_group_sums_fp6(130, 384, 3072, P, nullptr, I, nullptr), INV,
                  "group sums fp6 weight NULL");

    // ---- the up GEMM with the next layer's activation step (FP6 only)
    {
        const int64_t need = svdq_gelu_quantize_workspace_bytes(4096, 12288, 32);
        EXPECT(need == 96ll * 4096 * 32 * 4, "gelu-quantize workspace bytes");
        EXPECT(svdq_gelu_quantize_workspace_bytes(4, 100, 32) == -1, "gelu-quantize workspace, N % 64");
        auto gq = [&](int32_t prec, int64_t N, int32_t rn, int64_t wb, void *work) {
            return svdq_gemm_w4a4_gelu_quantize(prec, 4096, N, 3072, 32, P, P, P, P, 1.0f, F, P, P, rn, P,
                                                rn ? P : nullptr, P, P, rn ? F : nullptr, work, wb, nullptr, nullptr);
        };
        expect_launch(gq(SVDQ_INT4_FP6, 12288, 32, need, P), "gemm_fp6_gelu_quant", 4096, 12288, 3072 + 32);
        expect_reject(gq(SVDQ_INT4, 12288, 32, need, P), UNS, "gelu-quantize int4 nibbles");
        expect_reject(gq(SVDQ_INT4_FP6, 12288, 32, need - 1, P), INV, "gelu-quantize workspace too small");
        expect_reject(gq(SVDQ_INT4_FP6, 12288, 32, need, nullptr), INV, "gelu-quantize workspace NULL");
        expect_reject(gq(SVDQ_INT4_FP6, 12300, 32, need, P), INV, "gelu-quantize N % 64");
        expect_reject(gq(SVDQ_INT4_FP6, 12288, 24, need, P), INV, "gelu-quantize rank_next 24");
    }

    // ---- packed int4 weights
    EXPECT(svdq_packed_weight_bytes(12288, 3072) == 12288ll * 1536 + 12288ll * 4 * 48, "packed bytes");
    EXPECT(svdq_packed_weight_bytes(8, 100) == -1, "packed bytes, K % 64");
    expect_launch(svdq_pack_weight_int4(12288, 3072, P, P, P, I, nullptr), "pack_weight_int4", 12288, 3072, 1);
    expect_launch(svdq_pack_weight_int4(5, 64, P, P, P, nullptr, nullptr), "pack_weight_int4", 5, 64, 0);
    expect_noop(svdq_pack_weight_int4(0, 64, P, P, P, nullptr, nullptr), "pack N=0");
    expect_reject(svdq_pack_weight_int4(5, 64, nullptr, P, P, nullptr, nullptr), INV, "pack codes NULL");
    expect_reject(svdq_pack_weight_int4(5, 64, P, P, MIS, nullptr, nullptr), INV, "pack blob misaligned");
    expect_reject(svdq_pack_weight_int4(5, 64, P, P, P, (int32_t *)((char *)P + 2), nullptr), INV,
                  "pack counter misaligned");
    expect_launch(svdq_debug_group_sums_packed(130, 384, 3072, P, P, I, nullptr), "group_sums_packed", 130, 384,
                  3072);
    expect_reject(svdq_debug_group_sums_packed(130, 384, 3072, P, nullptr, I, nullptr), INV,
                  "group sums packed weight NULL");

    // ---- grouped QKV GEMM with QK norm + rotary embedding
    const float *Fc = F;
    expect_launch(svdq_gemm_w4a4_qk_norm_rope(SVDQ_INT4, 4096, 9216, 3072, 32, P, P, P, P, 1.0f, Fc, P, P, P, P,
                                              1e-6f, Fc, Fc, P, nullptr),
                  "gemm_int4_qk", 4096, 9216, 6144);
    expect_launch(svdq_gemm_w4a4_qk_norm_rope(SVDQ_INT4_PACKED, 4096, 9216, 3072, 32, P, P, P, P, 1.0f, Fc, P, P, P,
                                              P, 1e-6f, Fc, Fc, P, nullptr),
                  "gemm_int4_packed_qk", 4096, 9216, 6144);
    expect_launch(svdq_gemm_w4a4_qk_norm_rope(SVDQ_INT4_FP6, 4096, 9216, 3072, 32, P, P, P, P, 1.0f, Fc, P, P, P,
                                              P, 1e-6f, Fc, Fc, P, nullptr),
                  "gemm_fp6_qk", 4096, 9216, 6144);
    expect_launch(svdq_gemm_w4a4_qk_norm_rope(SVDQ_NVFP4, 3, 384, 256, 0, P, P, P, P, 1.0f, nullptr, nullptr,
                                              nullptr, P, P, 0.0f, Fc, Fc, P, nullptr),
                  "gemm_nvfp4_qk", 3, 384, 256);
    expect_reject(svdq_gemm_w4a4_qk_norm_rope(SVDQ_INT4, 3, 320, 256, 0, P, P, P, P, 1.0f, nullptr, nullptr,
                                              nullptr, P, P, 0.0f, Fc, Fc, P, nullptr),
                  INV, "qk N not 3*heads*128");
    expect_reject(svdq_gemm_w4a4_qk_norm_rope(SVDQ_INT4, 3, 384, 256, 0, P, P, P, P, 1.0f, nullptr, nullptr,
                                              nullptr, P, P, -1.0f, Fc, Fc, P, nullptr),
                  INV, "qk eps < 0");
    expect_reject(svdq_gemm_w4a4_qk_norm_rope(SVDQ_INT4, 3, 384, 256, 0, P, P, P, P, 1.0f, nullptr, nullptr,
                                              nullptr, P, P, __builtin_nanf(""), Fc, Fc, P, nullptr),
                  INV, "qk eps NaN");
    expect_reject(svdq_gemm_w4a4_qk_norm_rope(SVDQ_INT4, 3, 384, 256, 0, P, P, P, P, 1.0f, nullptr, nullptr,
                                              nullptr, nullptr, P, 0.0f, Fc, Fc, P, nullptr),
                  INV, "qk q weight NULL");
    expect_reject(svdq_gemm_w4a4_qk_norm_rope(SVDQ_INT4, 3, 384, 256, 0, P, P, P, P, 1.0f, nullptr, nullptr,
                                              nullptr, P, P, 0.0f, Fc, nullptr, P, nullptr),
                  INV, "qk sin NULL");

    // ---- AWQ W4A16: the GEMV and, for many rows, the GEMM
    expect_launch(awq_gemv_w4a16(1, 18432, 3072, 64, P, P, P, P, nullptr, P, nullptr), "awq_gemv", 1, 18432, 3072);
    expect_launch(awq_gemv_w4a16(4096, 18432, 3072, 64, P, P, P, P, P, P, nullptr), "awq_gemm", 4096, 18432, 3072);
    expect_launch(awq_gemv_w4a16(4096, 64, 3072, 64, P, P, P, P, P, P, nullptr), "awq_gemv", 4096, 64, 3072);
    expect_noop(awq_gemv_w4a16(0, 64, 64, 64, P, P, P, P, nullptr, P, nullptr), "awq M=0");
    expect_reject(awq_gemv_w4a16(1, 64, 64, 128, P, P, P, P, nullptr, P, nullptr), UNS, "awq group 128");
    expect_reject(awq_gemv_w4a16(1, 64, 100, 64, P, P, P, P, nullptr, P, nullptr), INV, "awq K % 64");
    expect_reject(awq_gemv_w4a16(1, 64, 64, 64, P, P, nullptr, P, nullptr, P, nullptr), INV, "awq scales NULL");
    expect_reject(awq_gemv_w4a16(1, 64, 64, 64, P, P, P, MIS, nullptr, P, nullptr), INV, "awq zeros misaligned");

    // ---- debug entry points
    expect_launch(svdq_debug_group_sums(130, 384, 12288, P, P, I, nullptr), "group_sums", 130, 384, 12288);
    expect_reject(svdq_debug_group_sums(130, 384, 12288, P, P, nullptr, nullptr), INV, "group sums G NULL");
    expect_launch(svdq_debug_gelu_bf16(65536, P, P, nullptr), "gelu_bf16", 65536, 0, 0);
    expect_noop(svdq_debug_gelu_bf16(0, P, P, nullptr), "gelu n=0");
    expect_reject(svdq_debug_gelu_bf16(-1, P, P, nullptr), INV, "gelu n < 0");
    expect_launch(svdq_debug_stream_read(P, 64 << 20, 1, (uint32_t *)I, nullptr), "stream_read", 64, 1, 0);
    expect_launch(svdq_debug_stream_read(P, 64 << 20, 0, (uint32_t *)I, nullptr), "stream_read", 64, 0, 0);
    expect_noop(svdq_debug_stream_read(P, 0, 0, (uint32_t *)I, nullptr), "stream read 0 bytes");
    expect_reject(svdq_debug_stream_read(P, -1, 0, (uint32_t *)I, nullptr), INV, "stream read bytes < 0");
    expect_reject(svdq_debug_stream_read(P, 4096, 2, (uint32_t *)I, nullptr), INV, "stream read pattern 2");
    expect_reject(svdq_debug_stream_read(P, 4096, 0, nullptr, nullptr), INV, "stream read out NULL");

    // ---- offline preparation
    expect_launch(svdq_smooth_factors(4096, 12288, 3072, P, P, P, nullptr), "smooth_factors", 4096, 12288, 3072);
    expect_reject(svdq_smooth_factors(4096, 12288, 3000, P, P, P, nullptr), INV, "smooth K % 64");
    const int64_t ws = svdq_lowrank_workspace_bytes(12288, 3072, 32);
    EXPECT(ws > 0, "workspace bytes %lld", (long long)ws);
    EXPECT(svdq_lowrank_workspace_bytes(12288, 3072, 8) == -1, "workspace for rank 8");
    EXPECT(svdq_lowrank_workspace_bytes(30, 3072, 32) == -1, "workspace for N < rank + 8");
    expect_launch(svdq_lowrank_factors(12288, 3072, 32, P, P, 7, P, ws, P, P, nullptr), "lowrank_factors", 12288,
                  3072, 32);
    expect_reject(svdq_lowrank_factors(12288, 3072, 32, P, P, 7, P, ws - 1, P, P, nullptr), INV,
                  "lowrank workspace too small");
    expect_reject(svdq_lowrank_factors(12288, 3072, 0, P, P, 7, P, ws, P, P, nullptr), INV, "lowrank rank 0");
    expect_reject(svdq_lowrank_factors(36, 3072, 32, P, P, 7, P, ws, P, P, nullptr), INV, "lowrank N < rank + 8");
    expect_launch(svdq_lowrank_factors_noalloc(12288, 3072, 32, P, P, 7, P, P, nullptr), "lowrank_factors", 12288,
                  3072, 32);
    expect_launch(svdq_lowrank_factors_noalloc(3072, 12288, 32, P, nullptr, 7, P, P, nullptr), "lowrank_factors",
                  3072, 12288, 32);
    expect_reject(svdq_lowrank_factors_noalloc(65536, 65536, 128, P, P, 7, P, P, nullptr), INV,
                  "lowrank noalloc beyond the fixed scratch");
    expect_reject(svdq_lowrank_factors_noalloc(12288, 3072, 32, P, P, 7, nullptr, P, nullptr), INV,
                  "lowrank noalloc lora_up NULL");
    expect_launch(svdq_quantize_weight(SVDQ_NVFP4, 3072, 3072, 32, P, P, P, P, P, P, nullptr), "quantize_weight",
                  3072, 3072, 1032);
    expect_reject(svdq_quantize_weight(SVDQ_INT4, 64, 64, 16, P, P, nullptr, P, P, P, nullptr), INV,
                  "quantize_weight lora_up NULL");

    // ---- a launch that fails: status SVDQ_ERR_HIP and a message
    g_stub.result = hipErrorInvalidValue;
    svdq_status st = svdq_gemm_w4a4(SVDQ_INT4, 4, 64, 64, 0, P, P, P, P, 1.0f, nullptr, nullptr, nullptr, P, nullptr);
    EXPECT(st == SVDQ_ERR_HIP && std::strstr(svdq_last_error(), "svdq_gemm_w4a4") != nullptr,
           "failed launch: status %d", (int)st);
    g_stub.result = hipSuccess;
    g_stub.calls = 0;

    // ---- a device that is not gfx950 (a second ordinal, so the first one's cached answer stays)
    g_stub.device = 1;
    g_stub.arch = "gfx942:sramecc+:xnack-";
    expect_reject(svdq_gemm_w4a4(SVDQ_INT4, 4, 64, 64, 0, P, P, P, P, 1.0f, nullptr, nullptr, nullptr, P, nullptr),
                  UNS, "gfx942 device");
    g_stub.device = 64;
    expect_reject(svdq_gemm_w4a4(SVDQ_INT4, 4, 64, 64, 0, P, P, P, P, 1.0f, nullptr, nullptr, nullptr, P, nullptr),
                  UNS, "device ordinal 64");
    g_stub.device = 0;

    // ---- status strings
    for (int s = 0; s < 4; ++s)
        EXPECT(std::strncmp(svdq_status_string((svdq_status)s), "SVDQ_", 5) == 0, "status string %d", s);
    EXPECT(std::strstr(svdq_status_string((svdq_status)99), "unknown") != nullptr, "unknown status string");
    EXPECT(svdq_abi_version() > 0, "abi version");

    if (failures) {
        std::fprintf(stderr, "%d expectation(s) failed\n", failures);
        return 1;
    }
    std::printf("abi sanitize ok\n");
    return 0;
}
