// gemm_w4a4_int4.hip -- second fused step of the SVDQuant W4A4 layer, int4
// variant (group 64, bf16 scales; "Nunchaku Lite" docs, "Supported
// quantization types"), on gfx950 matrix cores:
//   y = alpha * sum_g G_g * sx_g * sw_g  +  lora_act . lora_up^T  +  bias,
//   G_g[m,n] = sum_{k in group g} qa[m,k] * qw[n,k]   (exact integers)
// with the low-rank up-projection and the bias fused into the epilogue
// (blog "Hugging Face integrates Nunchaku 4-bit diffusion inference into
// Diffusers", "SVDQuant and the Nunchaku engine").
//
// Operands.  CDNA4 has no int4 matrix instruction, so a packed nibble is
// placed in the high half of a byte: (d << 4) & 0xF0F0F0F0 gives the even
// nibbles of a dword as int8 = 16*code, d & 0xF0F0F0F0 the odd ones.  Two
// bit operations turn 8 codes into 8 int8 lanes, and v_mfma_i32_32x32x32_i8
// then returns 256 * G exactly (|256 G| <= 2^20).  A dot product does not
// depend on the order of k as long as both operands use the same order, so
// the even/odd split is applied to A and B alike.
//
// Tiling: 256 threads, 128x128 output tile, 4 waves of 64x64 (2x2 tiles of
// 32x32).  One K-step is one group of 64.  Fragments stream from global
// memory straight into registers, one group ahead.  Group scales are staged
// in LDS as fp32, 8 groups at a time, with 2^-8 * alpha folded into the
// weight scale.  Per group and output: one cvt, one mul, one fma (VALU).
#include "device_common.h"
#include "launch.h"

namespace svdq {

constexpr int G4_BM = 128, G4_BN = 128, G4_THREADS = 256, G4_SCHUNK = 8;

// 32x32 MFMA accumulator layout: lane l, register i -> row 8*(i/4) + 4*(l/32) + i%4, col l%32.

template <bool GROUP_SUMS>
__global__ __launch_bounds__(G4_THREADS)
void gemm_w4a4_int4_kernel(int M, int N, int K, int rank,
                           const uint8_t *__restrict__ act_codes,
                           const uint16_t *__restrict__ act_scales,
                           const uint8_t *__restrict__ wgt_codes,
                           const uint16_t *__restrict__ wgt_scales, float alpha,
                           const float *__restrict__ lora_act,
                           const uint16_t *__restrict__ lora_up,
                           const uint16_t *__restrict__ bias,
                           uint16_t *__restrict__ out, int32_t *__restrict__ gsum)
{
    __shared__ float s_sx[2][G4_SCHUNK][G4_BM];
    __shared__ float s_sw[2][G4_SCHUNK][G4_BN];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, h = lane >> 5;
    const int nbn = (N + G4_BN - 1) / G4_BN;
    const int m0 = (int)(blockIdx.x / nbn) * G4_BM, n0 = (int)(blockIdx.x % nbn) * G4_BN;
    const int NG = K >> 6;
    const size_t rowbytes = (size_t)(K >> 1);

    // rows this lane loads fragments for (clamped; out-of-range rows are zeroed)
    int arow[2], brow[2];
    bool aok[2], bok[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        arow[t] = m0 + wm * 64 + t * 32 + l32;
        brow[t] = n0 + wn * 64 + t * 32 + l32;
        aok[t] = arow[t] < M;
        bok[t] = brow[t] < N;
        if (!aok[t]) arow[t] = 0;
        if (!bok[t]) brow[t] = 0;
    }
    const uint8_t *ap[2], *bp[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        ap[t] = act_codes + (size_t)arow[t] * rowbytes + 16 * h;
        bp[t] = wgt_codes + (size_t)brow[t] * rowbytes + 16 * h;
    }

    // scale staging: thread t < 128 loads A row m0+t, t >= 128 loads B row n0+t-128
    const bool s_is_a = tid < G4_BM;
    const int s_r = s_is_a ? tid : tid - G4_BM;
    const int s_row = (s_is_a ? m0 : n0) + s_r;
    const bool s_ok = s_row < (s_is_a ? M : N);
    const uint16_t *s_src = (s_is_a ? act_scales : wgt_scales) + (size_t)(s_ok ? s_row : 0) * NG;
    const float s_mul = s_is_a ? 1.0f : alpha * 0.00390625f;   // alpha * 2^-8 on the weight side
    uint16_t s_reg[G4_SCHUNK];
    auto load_scales = [&](int c) {
#pragma unroll
        for (int i = 0; i < G4_SCHUNK; ++i) {
            int g = c * G4_SCHUNK + i;
            s_reg[i] = (s_ok && g < NG) ? s_src[g] : (uint16_t)0;
        }
    };
    auto store_scales = [&](int buf) {
#pragma unroll
        for (int i = 0; i < G4_SCHUNK; ++i) {
            float v = bf16_to_f32(s_reg[i]) * s_mul;
            if (s_is_a) s_sx[buf][i][s_r] = v;
            else s_sw[buf][i][s_r] = v;
        }
    };

    v16f acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

    v4u fa[2], fb[2];
    auto load_frags = [&](int g) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            fa[t] = aok[t] ? *(const v4u *)(ap[t] + (size_t)g * 32) : v4u{0u, 0u, 0u, 0u};
            fb[t] = bok[t] ? *(const v4u *)(bp[t] + (size_t)g * 32) : v4u{0u, 0u, 0u, 0u};
        }
    };

    if (!GROUP_SUMS) {
        load_scales(0);
        store_scales(0);
        if (NG > G4_SCHUNK) load_scales(1);
    }
    load_frags(0);
    __syncthreads();

    for (int g = 0; g < NG; ++g) {
        v4u ca[2] = {fa[0], fa[1]}, cb[2] = {fb[0], fb[1]};
        if (g + 1 < NG) load_frags(g + 1);

        v4i alo[2], ahi[2], blo[2], bhi[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                alo[t][i] = (int)((ca[t][i] << 4) & 0xF0F0F0F0u);
                ahi[t][i] = (int)(ca[t][i] & 0xF0F0F0F0u);
                blo[t][i] = (int)((cb[t][i] << 4) & 0xF0F0F0F0u);
                bhi[t][i] = (int)(cb[t][i] & 0xF0F0F0F0u);
            }
        }
        v16i G[2][2];
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                v16i z = {};
                z = __builtin_amdgcn_mfma_i32_32x32x32_i8(alo[a], blo[b], z, 0, 0, 0);
                G[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ahi[a], bhi[b], z, 0, 0, 0);
            }

        if constexpr (GROUP_SUMS) {
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const int col = n0 + wn * 64 + b * 32 + l32;
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int rowi = m0 + wm * 64 + a * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
                        if (rowi < M && col < N)
                            gsum[((size_t)rowi * N + col) * NG + g] = G[a][b][i] >> 8;
                    }
                }
        } else {
            const int buf = (g / G4_SCHUNK) & 1, gi = g % G4_SCHUNK;
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                float sx[16];
                const float *sxp = &s_sx[buf][gi][wm * 64 + a * 32 + 4 * h];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    v4f v = *(const v4f *)(sxp + 8 * q);
                    sx[4 * q + 0] = v[0];
                    sx[4 * q + 1] = v[1];
                    sx[4 * q + 2] = v[2];
                    sx[4 * q + 3] = v[3];
                }
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const float sw = s_sw[buf][gi][wn * 64 + b * 32 + l32];
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        acc[a][b][i] = __builtin_fmaf((float)G[a][b][i], sx[i] * sw, acc[a][b][i]);
                }
            }
            // chunk boundary: publish the next chunk of scales
            if (gi == G4_SCHUNK - 1 && g + 1 < NG) {
                const int c_next = g / G4_SCHUNK + 1;
                store_scales(c_next & 1);
                __syncthreads();
                if ((c_next + 1) * G4_SCHUNK < NG) load_scales(c_next + 1);
            }
        }
    }

    if constexpr (!GROUP_SUMS) {
        // ---- low-rank up-projection on the matrix cores: acc += t . up^T.
        // t (fp32) is split into bf16 hi + lo (t - hi is exact in fp32), the
        // up factor is bf16, products are exact in fp32.
        for (int s = 0; s < rank; s += 16) {
            v8bf thi[2], tlo[2], up[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int rrow = m0 + wm * 64 + t * 32 + l32;
                v4u hv, lv;
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
                } else {
                    hv = v4u{0u, 0u, 0u, 0u};
                    lv = hv;
                }
                thi[t] = __builtin_bit_cast(v8bf, hv);
                tlo[t] = __builtin_bit_cast(v8bf, lv);
                const int ucol = n0 + wn * 64 + t * 32 + l32;
                v4u uv = ucol < N ? *(const v4u *)(lora_up + (size_t)ucol * rank + s + 8 * h)
                                  : v4u{0u, 0u, 0u, 0u};
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

        // ---- bias and the bf16 store
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
                    if (rowi < M)
                        out[(size_t)rowi * N + col] = (uint16_t)f32_to_bf16_rne(acc[a][b][i] + bv);
                }
        }
    }
}

hipError_t launch_gemm_w4a4_int4(int M, int N, int K, int rank, const void *act_codes,
                                 const void *act_scales, const void *wgt_codes,
                                 const void *wgt_scales, float alpha, const float *lora_act,
                                 const void *lora_up, const void *bias, void *out,
                                 hipStream_t stream)
{
    dim3 grid(((N + G4_BN - 1) / G4_BN) * ((M + G4_BM - 1) / G4_BM)), block(G4_THREADS);
    hipLaunchKernelGGL((gemm_w4a4_int4_kernel<false>), grid, block, 0, stream, M, N, K, rank,
                       (const uint8_t *)act_codes, (const uint16_t *)act_scales,
                       (const uint8_t *)wgt_codes, (const uint16_t *)wgt_scales, alpha, lora_act,
                       (const uint16_t *)lora_up, (const uint16_t *)bias, (uint16_t *)out,
                       (int32_t *)nullptr);
    return hipGetLastError();
}

hipError_t launch_group_sums_int4(int M, int N, int K, const void *act_codes,
                                  const void *wgt_codes, int32_t *G, hipStream_t stream)
{
    dim3 grid(((N + G4_BN - 1) / G4_BN) * ((M + G4_BM - 1) / G4_BM)), block(G4_THREADS);
    hipLaunchKernelGGL((gemm_w4a4_int4_kernel<true>), grid, block, 0, stream, M, N, K, 0,
                       (const uint8_t *)act_codes, (const uint16_t *)nullptr,
                       (const uint8_t *)wgt_codes, (const uint16_t *)nullptr, 1.0f,
                       (const float *)nullptr, (const uint16_t *)nullptr,
                       (const uint16_t *)nullptr, (uint16_t *)nullptr, G);
    return hipGetLastError();
}

}  // namespace svdq
