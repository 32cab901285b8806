// prepare_weight.hip -- the offline preparation of an SVDQuant W4A4 layer's
// weight on gfx950 (blog "Hugging Face integrates Nunchaku 4-bit diffusion
// inference into Diffusers", section "SVDQuant and the Nunchaku engine":
// activation outliers migrate into the weights, the hardest part of each
// weight is kept in a small 16-bit low-rank branch, the residual is
// quantized to 4 bits).  Two of its three steps are exact and here:
//
//  * smoothing factors from calibration activations x [M,K] and the weight
//    W [N,K] (both bf16):
//        s[k] = RNE_bf16( sqrt( max_m |x[m,k]| / max_n |W[n,k]| ) ),
//    fp64 quotient and square root (each correctly rounded), 1 when either
//    maximum is 0.  The maxima are exact whatever the order: they are taken
//    on the magnitude bits of the bf16 values.
//  * the 4-bit residual, given the rank-r branch (lora_up [N,r], lora_down
//    [r,K], bf16):
//        R[n,k] = fl32( W[n,k] s[k] - sum_{j ascending} up[n,j] down[j,k] ),
//    accumulated in fp64 without fused multiply-adds (so that every partial
//    sum is the one an fp64 loop in that order gives), then quantized per row
//    and group like the activations but from fp32 values with IEEE fp32
//    division: int4 g64 (scale RNE_bf16(absmax/7), code RNE(R/scale) clamped
//    to [-8,7]) or NVFP4 g16 (E4M3 scale of absmax/6, E2M1 code of R/scale by
//    exact comparisons with the E2M1 midpoints, ties to the even code).
//
// Layout: one wave per 64 consecutive weights of a row; lane = weight; the
// branch's lora_down rows are read as 128 contiguous bytes per wave.
#include "device_common.h"
#include "launch.h"

namespace svdq {

// ---- smoothing factors: block = 128 columns (two per lane), 16 waves split
// the rows, four independent row loads in flight per step
constexpr int SF_WAVES = 16;

__device__ __forceinline__ void colmax_rows(const uint16_t *__restrict__ p, int rows, int K, int c, int wave,
                                            uint32_t &m0, uint32_t &m1)
{
    for (int r = wave; r < rows; r += 4 * SF_WAVES) {
        uint32_t v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int rr = r + u * SF_WAVES;
            v[u] = rr < rows ? *(const uint32_t *)(p + (size_t)rr * K + c) : 0u;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            m0 = max(m0, v[u] & 0x7FFFu);
            m1 = max(m1, (v[u] >> 16) & 0x7FFFu);
        }
    }
}

__global__ __launch_bounds__(SF_WAVES * 64) void smooth_factors_kernel(int M, int N, int K,
                                                                        const uint16_t *__restrict__ x,
                                                                        const uint16_t *__restrict__ W,
                                                                        uint16_t *__restrict__ s)
{
    __shared__ uint32_t part[2][SF_WAVES][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = blockIdx.x * 128 + 2 * lane;          // this lane's column pair
    const bool ok = c < K;                               // K is a multiple of 64: both or neither
    uint32_t mx0 = 0, mx1 = 0, mw0 = 0, mw1 = 0;         // max magnitude bits of the two columns
    if (ok) {
        colmax_rows(x, M, K, c, wave, mx0, mx1);
        colmax_rows(W, N, K, c, wave, mw0, mw1);
    }
    part[0][wave][lane] = mx0 | (mx1 << 16);
    part[1][wave][lane] = mw0 | (mw1 << 16);
    __syncthreads();
    if (wave == 0 && ok) {
        uint32_t ax[2] = {0, 0}, aw[2] = {0, 0};
        for (int w = 0; w < SF_WAVES; ++w)
            for (int hh = 0; hh < 2; ++hh) {
                ax[hh] = max(ax[hh], (part[0][w][lane] >> (16 * hh)) & 0xFFFFu);
                aw[hh] = max(aw[hh], (part[1][w][lane] >> (16 * hh)) & 0xFFFFu);
            }
        uint32_t out = 0;
        for (int hh = 0; hh < 2; ++hh) {
            const double a = (double)__uint_as_float(ax[hh] << 16), b = (double)__uint_as_float(aw[hh] << 16);
            const uint32_t sb = (a == 0.0 || b == 0.0) ? 0x3F80u : f64_to_bf16_rne(__builtin_sqrt(a / b));
            out |= sb << (16 * hh);
        }
        *(uint32_t *)(s + c) = out;
    }
}

// ---- residual of one weight (fp64, no contraction, j ascending) -> fp32
__device__ __forceinline__ float residual_at(int n, int k, int K, int rank, const uint16_t *__restrict__ W,
                                             const uint16_t *__restrict__ s, const uint16_t *__restrict__ up,
                                             const uint16_t *__restrict__ down)
{
    const double w = (double)bf16_to_f32(W[(size_t)n * K + k]) * (s ? (double)bf16_to_f32(s[k]) : 1.0);
    double lr = 0.0;
    for (int j = 0; j < rank; ++j)
        lr += (double)bf16_to_f32(up[(size_t)n * rank + j]) * (double)bf16_to_f32(down[(size_t)j * K + k]);
    return (float)(w - lr);
}

// max over the 16 lanes of each DPP row (magnitudes as non-negative floats)
__device__ __forceinline__ float max16(float v) {
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x124, 0xF, 0xF, true)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xF, 0xF, true)));
    return v;
}

// E2M1 code (magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 -> 0..7) of an fp32, round
// to nearest with ties to the even code, saturating at 6; the sign bit is
// kept (a negative value that rounds to 0 gives 0x8).
__device__ __forceinline__ uint32_t e2m1_code(float v) {
    const float a = fabsf(v);
    const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                       (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
    return c | ((__float_as_uint(v) >> 28) & 8u);
}

// ---- residual + quantization: one wave per 64 weights of a row
template <int PREC>
__global__ __launch_bounds__(256) void quantize_weight_kernel(int N, int K, int rank, const uint16_t *__restrict__ W,
                                                              const uint16_t *__restrict__ s,
                                                              const uint16_t *__restrict__ up,
                                                              const uint16_t *__restrict__ down,
                                                              uint8_t *__restrict__ codes, void *__restrict__ scales)
{
    const int lane = threadIdx.x & 63;
    const long long seg = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);   // 64-weight segment
    const int segs_per_row = K >> 6;
    if (seg >= (long long)N * segs_per_row) return;                        // whole waves: no barrier follows
    const int n = (int)(seg / segs_per_row), g64 = (int)(seg % segs_per_row);
    const int k = g64 * 64 + lane;
    const float R = residual_at(n, k, K, rank, W, s, up, down);
    uint32_t code;
    if constexpr (PREC == 0) {
        // int4, group 64: the wave is the group
        float a = max16(fabsf(R));
        a = fmaxf(a, shfl_xor_f(a, 16));
        a = fmaxf(a, shfl_xor_f(a, 32));
        const uint32_t sbits = f32_to_bf16_rne(a / 7.0f);
        const float sb = __uint_as_float(sbits << 16);
        float q = 0.0f;
        if (sb != 0.0f) q = __builtin_amdgcn_fmed3f(__builtin_rintf(R / sb), -8.0f, 7.0f);
        code = (uint32_t)(int)q & 15u;
        if (lane == 0) ((uint16_t *)scales)[(size_t)n * (K >> 6) + g64] = (uint16_t)sbits;
    } else {
        // NVFP4, group 16: a DPP row of 16 lanes is a group
        const float a = max16(fabsf(R));
        const uint32_t se = e4m3_encode_nonneg(a / 6.0f);
        const float d = e4m3_decode_nonneg(se);
        code = d == 0.0f ? 0u : e2m1_code(R / d);
        if ((lane & 15) == 0) ((uint8_t *)scales)[(size_t)n * (K >> 4) + g64 * 4 + (lane >> 4)] = (uint8_t)se;
    }
    // even lane k: the byte of weights k (low nibble) and k+1 (high nibble)
    const uint32_t next = (uint32_t)__shfl_down((int)code, 1, 64);
    if ((lane & 1) == 0) codes[(size_t)n * (K >> 1) + (k >> 1)] = (uint8_t)(code | (next << 4));
}

hipError_t launch_smooth_factors(int M, int N, int K, const void *x, const void *W, void *s, hipStream_t stream)
{
    hipLaunchKernelGGL(smooth_factors_kernel, dim3((K + 127) / 128), dim3(SF_WAVES * 64), 0, stream, M, N, K,
                       (const uint16_t *)x, (const uint16_t *)W, (uint16_t *)s);
    return hipGetLastError();
}

hipError_t launch_quantize_weight(int precision, int N, int K, int rank, const void *W, const void *s,
                                  const void *up, const void *down, void *codes, void *scales,
                                  hipStream_t stream)
{
    const long long segs = (long long)N * (K >> 6);
    const dim3 grid((unsigned)((segs + 3) / 4)), block(256);
    if (precision == 0)
        hipLaunchKernelGGL(quantize_weight_kernel<0>, grid, block, 0, stream, N, K, rank, (const uint16_t *)W,
                           (const uint16_t *)s, (const uint16_t *)up, (const uint16_t *)down, (uint8_t *)codes, scales);
    else
        hipLaunchKernelGGL(quantize_weight_kernel<1>, grid, block, 0, stream, N, K, rank, (const uint16_t *)W,
                           (const uint16_t *)s, (const uint16_t *)up, (const uint16_t *)down, (uint8_t *)codes, scales);
    return hipGetLastError();
}

}  // namespace svdq
