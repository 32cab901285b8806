// gemm_w4a4_nvfp4.hip -- SVDQuant W4A4 GEMM, NVFP4 variant (E2M1 codes,
// E4M3 scales per 16 along K; "Nunchaku Lite" docs, "Supported quantization
// types": svdq_w4a4 nvfp4 group 16), with the low-rank up-projection and the
// bias in the epilogue.
//
// Mapping to CDNA4.  The block-scaled FP4 matrix instructions of gfx950
// take one power-of-two (E8M0) scale per 32 elements; NVFP4 carries one
// E4M3 scale (4-bit significand, not a power of two) per 16 elements, so no
// exact mapping onto them exists.  Instead both operands are dequantized
// exactly: an E2M1 value (at most 2 significant bits) times an E4M3 scale
// (at most 4) has at most 6 significant bits and lies in [2^-10, 2688], so
// it is exactly an fp16 normal number.  gfx950's v_cvt_scalef32_pk_f16_fp4
// turns one byte (two E2M1 codes) into two fp16 values (its scale operand
// only contributes a power of two, so it is left at 1), and one packed fp16
// multiply applies the group scale: one vector instruction per element.
// The block dequantizes each 64-wide K slice of its A and B tiles once into
// LDS, and the waves run v_mfma_f32_32x32x16_f16 on it with fp32
// accumulation (products are exact; only the fp32 sum rounds).  alpha
// multiplies the 4-bit term at the end.
#include "device_common.h"
#include "gemm_epilogue.h"
#include "launch.h"

namespace svdq {

constexpr int NV_BM = 128, NV_BN = 128, NV_BK = 64, NV_THREADS = 256;
constexpr int NV_LDS_STRIDE = NV_BK + 8;   // fp16 elements per LDS row (+16 B against bank conflicts)

typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(NV_THREADS)
void gemm_w4a4_nvfp4_kernel(int M, int N, int K, int rank,
                            const uint8_t *__restrict__ act_codes,
                            const uint8_t *__restrict__ act_scales,
                            const uint8_t *__restrict__ wgt_codes,
                            const uint8_t *__restrict__ wgt_scales, float alpha,
                            const float *__restrict__ lora_act,
                            const uint16_t *__restrict__ lora_up,
                            const uint16_t *__restrict__ bias, uint16_t *__restrict__ out)
{
    __shared__ __attribute__((aligned(16))) uint16_t s_a[NV_BM * NV_LDS_STRIDE];   // fp16 bits
    __shared__ __attribute__((aligned(16))) uint16_t s_b[NV_BN * NV_LDS_STRIDE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, h = lane >> 5;
    const int nbn = (N + NV_BN - 1) / NV_BN;
    const int m0 = (int)(blockIdx.x / nbn) * NV_BM, n0 = (int)(blockIdx.x % nbn) * NV_BN;
    const size_t rowbytes = (size_t)(K >> 1);
    const int NG16 = K >> 4;

    // dequant duty: thread t handles row t/2 of both tiles, K half (t%2)*32 .. +32
    const int d_row = tid >> 1, d_half = tid & 1;
    const int am = m0 + d_row, bn = n0 + d_row;
    const bool a_ok = am < M, b_ok = bn < N;
    const uint8_t *a_cp = act_codes + (size_t)(a_ok ? am : 0) * rowbytes + 16 * d_half;
    const uint8_t *b_cp = wgt_codes + (size_t)(b_ok ? bn : 0) * rowbytes + 16 * d_half;
    const uint8_t *a_sp = act_scales + (size_t)(a_ok ? am : 0) * NG16 + 2 * d_half;
    const uint8_t *b_sp = wgt_scales + (size_t)(b_ok ? bn : 0) * NG16 + 2 * d_half;

    v4u ra, rb;
    uint32_t sa0, sa1, sb0, sb1;
    auto gload = [&](int kb) {
        const int kbyte = kb * (NV_BK / 2), kgrp = kb * (NV_BK / 16);
        ra = a_ok ? *(const v4u *)(a_cp + kbyte) : v4u{0u, 0u, 0u, 0u};
        rb = b_ok ? *(const v4u *)(b_cp + kbyte) : v4u{0u, 0u, 0u, 0u};
        sa0 = a_ok ? a_sp[kgrp] : 0u;
        sa1 = a_ok ? a_sp[kgrp + 1] : 0u;
        sb0 = b_ok ? b_sp[kgrp] : 0u;
        sb1 = b_ok ? b_sp[kgrp + 1] : 0u;
    };
    auto dequant_store = [&](const v4u &codes, uint32_t s0, uint32_t s1, uint16_t *dst) {
        // the two group scales as fp16 (every E4M3 value is an fp16 normal)
        const _Float16 f0 = (_Float16)e4m3_decode(s0), f1 = (_Float16)e4m3_decode(s1);
        v4u o[4];
#pragma unroll
        for (int wdx = 0; wdx < 4; ++wdx) {          // dword wdx holds k = 8*wdx .. 8*wdx+7
            const v2h f = wdx < 2 ? v2h{f0, f0} : v2h{f1, f1};
            // byte p: k = 8*wdx + 2p (low nibble), 8*wdx + 2p + 1 (high nibble)
            o[wdx][0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes[wdx], 1.0f, 0) * f);
            o[wdx][1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes[wdx], 1.0f, 1) * f);
            o[wdx][2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes[wdx], 1.0f, 2) * f);
            o[wdx][3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes[wdx], 1.0f, 3) * f);
        }
        uint16_t *d = dst + d_row * NV_LDS_STRIDE + 32 * d_half;
#pragma unroll
        for (int q = 0; q < 4; ++q) *(v4u *)(d + 8 * q) = o[q];
    };

    v16f acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

    const int KB = K / NV_BK;
    gload(0);
    for (int kb = 0; kb < KB; ++kb) {
        __syncthreads();                              // previous slice fully consumed
        dequant_store(ra, sa0, sa1, s_a);
        dequant_store(rb, sb0, sb1, s_b);
        __syncthreads();
        if (kb + 1 < KB) gload(kb + 1);
#pragma unroll
        for (int ks = 0; ks < NV_BK / 16; ++ks) {
            v8h av[2], bv[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                av[t] = *(const v8h *)(s_a + (wm * 64 + t * 32 + l32) * NV_LDS_STRIDE + 16 * ks + 8 * h);
                bv[t] = *(const v8h *)(s_b + (wn * 64 + t * 32 + l32) * NV_LDS_STRIDE + 16 * ks + 8 * h);
            }
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[a], bv[b], acc[a][b], 0, 0, 0);
        }
    }

    gemm_epilogue(acc, alpha, M, N, rank, m0, n0, wm, wn, lane, lora_act, lora_up, bias, out);
}

hipError_t launch_gemm_w4a4_nvfp4(int M, int N, int K, int rank, const void *act_codes,
                                  const void *act_scales, const void *wgt_codes,
                                  const void *wgt_scales, float alpha, const float *lora_act,
                                  const void *lora_up, const void *bias, void *out,
                                  hipStream_t stream)
{
    dim3 grid(((N + NV_BN - 1) / NV_BN) * ((M + NV_BM - 1) / NV_BM)), block(NV_THREADS);
    hipLaunchKernelGGL(gemm_w4a4_nvfp4_kernel, grid, block, 0, stream, M, N, K, rank,
                       (const uint8_t *)act_codes, (const uint8_t *)act_scales,
                       (const uint8_t *)wgt_codes, (const uint8_t *)wgt_scales, alpha, lora_act,
                       (const uint16_t *)lora_up, (const uint16_t *)bias, (uint16_t *)out);
    return hipGetLastError();
}

}  // namespace svdq
