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
// it is exactly a bf16.  The block dequantizes each 64-wide K slice of its
// A and B tiles once into LDS, and the waves run v_mfma_f32_32x32x16_bf16
// on it with fp32 accumulation (products are exact; only the fp32 sum
// rounds).  alpha multiplies the 4-bit term at the end.
#include "device_common.h"
#include "launch.h"

namespace svdq {

constexpr int NV_BM = 128, NV_BN = 128, NV_BK = 64, NV_THREADS = 256;
constexpr int NV_LDS_STRIDE = NV_BK + 8;   // bf16 elements per LDS row (+16 B against bank conflicts)

// E2M1 code (bit 3 = sign) -> fp32
__device__ __forceinline__ float e2m1_decode(uint32_t c) {
    const uint32_t m = c & 7u;
    uint32_t bits = (m >= 2u) ? ((((m >> 1) + 126u) << 23) | ((m & 1u) << 22)) : (m ? 0x3F000000u : 0u);
    return __uint_as_float(bits | ((c & 8u) << 28));
}

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
    __shared__ __attribute__((aligned(16))) uint16_t s_a[NV_BM * NV_LDS_STRIDE];
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
        const float f0 = e4m3_decode(s0), f1 = e4m3_decode(s1);
        v4u o[4];
#pragma unroll
        for (int wdx = 0; wdx < 4; ++wdx) {          // dword wdx holds k = 8*wdx .. 8*wdx+7
            const float f = wdx < 2 ? f0 : f1;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t lo = __float_as_uint(e2m1_decode((codes[wdx] >> (8 * p)) & 15u) * f) >> 16;
                const uint32_t hi = __float_as_uint(e2m1_decode((codes[wdx] >> (8 * p + 4)) & 15u) * f) >> 16;
                o[wdx][p] = lo | (hi << 16);
            }
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
            v8bf av[2], bv[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                av[t] = *(const v8bf *)(s_a + (wm * 64 + t * 32 + l32) * NV_LDS_STRIDE + 16 * ks + 8 * h);
                bv[t] = *(const v8bf *)(s_b + (wn * 64 + t * 32 + l32) * NV_LDS_STRIDE + 16 * ks + 8 * h);
            }
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[a], bv[b], acc[a][b], 0, 0, 0);
        }
    }

    if (alpha != 1.0f) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[a][b][i] *= alpha;
    }

    // low-rank up-projection: t split into bf16 hi + lo, exact products
    for (int s = 0; s < rank; s += 16) {
        v8bf thi[2], tlo[2], up[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int rrow = m0 + wm * 64 + t * 32 + l32;
            v4u hv = v4u{0u, 0u, 0u, 0u}, lv = hv;
            if (rrow < M) {
                const float *tp = lora_act + (size_t)rrow * rank + s + 8 * h;
                v4f t0 = *(const v4f *)tp, t1 = *(const v4f *)(tp + 4);
                float tv[8] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    uint32_t h0 = f32_to_bf16_rne(tv[2 * p]), h1 = f32_to_bf16_rne(tv[2 * p + 1]);
                    uint32_t l0 = f32_to_bf16_rne(tv[2 * p] - __uint_as_float(h0 << 16));
                    uint32_t l1 = f32_to_bf16_rne(tv[2 * p + 1] - __uint_as_float(h1 << 16));
                    hv[p] = h0 | (h1 << 16);
                    lv[p] = l0 | (l1 << 16);
                }
            }
            thi[t] = __builtin_bit_cast(v8bf, hv);
            tlo[t] = __builtin_bit_cast(v8bf, lv);
            const int ucol = n0 + wn * 64 + t * 32 + l32;
            v4u uv = ucol < N ? *(const v4u *)(lora_up + (size_t)ucol * rank + s + 8 * h) : v4u{0u, 0u, 0u, 0u};
            up[t] = __builtin_bit_cast(v8bf, uv);
        }
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(thi[a], up[b], acc[a][b], 0, 0, 0);
                acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tlo[a], up[b], acc[a][b], 0, 0, 0);
            }
    }

#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int col = n0 + wn * 64 + b * 32 + l32;
        if (col >= N) continue;
        const float bv = bias ? bf16_to_f32(bias[col]) : 0.0f;
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int rowi = m0 + wm * 64 + a * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
                if (rowi < M) out[(size_t)rowi * N + col] = (uint16_t)f32_to_bf16_rne(acc[a][b][i] + bv);
            }
    }
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
