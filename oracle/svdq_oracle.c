/*
 * svdq_oracle.c -- plain CPU reference ("the oracle") for the SVDQuant W4A4
 * linear layer and its AWQ-style W4A16 sibling.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file.  Only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or constant
 * with the HIP kernels; its number codecs are written here from the format
 * definitions.
 *
 * Sources (web pages, cited by title and section):
 *   [DOC]  "Nunchaku Lite" -- Diffusers quantization documentation:
 *          "Supported quantization types" table (svdq_w4a4 nvfp4 g16,
 *          svdq_w4a4 int4 g64, awq_w4a16 int4 g64) and the
 *          "NunchakuLiteQuantizationConfig" section (compute_dtype bfloat16,
 *          precision / group_size / rank).
 *   [JA]   "Hugging Face integrates Nunchaku 4-bit diffusion inference into
 *          Diffusers" (Japanese blog), section "SVDQuant and the Nunchaku
 *          engine": activation outliers are migrated into the weights, the
 *          hardest part of each weight is kept in a small 16-bit low-rank
 *          branch, the residual is quantized to 4 bits; the engine fuses the
 *          low-rank down-projection into the quantize kernel and the
 *          up-projection into the 4-bit compute kernel.
 *   [TH]   "Bringing Nunchaku 4-bit diffusion inference to Diffusers" (Thai
 *          blog), section "Background: SVDQuant and Nunchaku": same method.
 *
 * The pages give no formula, so every rounding point below is a stated
 * reading (listed again where it is used):
 *   - bf16 is the 16-bit type (compute_dtype in [DOC]); rounding is IEEE
 *     round-to-nearest-even (RNE) everywhere.
 *   - int4 (g=64): scale = group absmax / 7 (fp32 divide) rounded to bf16;
 *     code = RNE(v / scale) clamped to [-8, 7]; zero scale gives zero codes.
 *   - NVFP4 (g=16): E2M1 codes with E4M3 group scales; scale = absmax / 6
 *     rounded to E4M3 with saturation; per-tensor scale 1.
 *   - the smoothed activation x/s is rounded to bf16 before both the
 *     low-rank branch and the quantizer.
 *   - the low-rank activation t = x_hat . L1^T is kept in fp32.
 *   - outputs are rounded once, from fp64, to bf16.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math (IEEE binary32/64, no FTZ).
 * All arithmetic that the method performs in fp32 is written with float
 * operands so that C's rules (FLT_EVAL_METHOD == 0 on x86-64) give exactly
 * one IEEE rounding per operation.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#if !defined(FLT_EVAL_METHOD) || FLT_EVAL_METHOD != 0
#error "the oracle needs FLT_EVAL_METHOD == 0 (SSE arithmetic)"
#endif

#define EXPORT __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ */
/* O-0  number formats                                                       */
/* ------------------------------------------------------------------------ */

/* bf16 -> f32 is exact: a bf16 is the top half of an IEEE binary32. */
EXPORT float oracle_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Encode a value that is exactly representable as a positive finite bf16. */
static uint16_t bf16_encode_exact(double r)
{
    if (r < ldexp(1.0, -126)) {                 /* subnormal: r = m * 2^-133 */
        return (uint16_t)(r / ldexp(1.0, -133));
    }
    int e;
    frexp(r, &e);                               /* r in [2^(e-1), 2^e) */
    int ex = e - 1;
    uint32_t mant = (uint32_t)(r / ldexp(1.0, ex - 7)) - 128u;
    return (uint16_t)(((uint32_t)(ex + 127) << 7) | mant);
}

/* Round a double to the nearest bf16, ties to even, in one step.
 * bf16: 8-bit significand, exponent range of binary32 (min normal 2^-126,
 * subnormal spacing 2^-133, largest finite (2 - 2^-7) * 2^127).
 * NaN maps to the quiet NaN 0x7FC0 (sign kept). */
EXPORT uint16_t oracle_f64_to_bf16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v)) return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(v);
    if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);
    int ex = e - 1;                             /* a in [2^ex, 2^(ex+1)) */
    if (ex < -126) ex = -126;                   /* fixed spacing below 2^-126 */
    double spacing = ldexp(1.0, ex - 7);
    double q = nearbyint(a / spacing);          /* exact scaling, then RNE */
    double r = q * spacing;
    if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u);   /* overflow */
    if (r == 0.0) return sign;
    return (uint16_t)(sign | bf16_encode_exact(r));
}

EXPORT uint16_t oracle_f32_to_bf16(float v) { return oracle_f64_to_bf16((double)v); }

/* E4M3 ("FN" variant of the OCP 8-bit float): 1 sign, 4 exponent (bias 7),
 * 3 mantissa bits; no infinity; S.1111.111 is NaN; largest finite 448;
 * min normal 2^-6; subnormal spacing 2^-9. */
EXPORT float oracle_e4m3_to_f32(uint8_t b)
{
    int sign = (b >> 7) & 1;
    int field = (b >> 3) & 15;
    int mant = b & 7;
    double v;
    if (field == 15 && mant == 7) return NAN;
    if (field == 0) v = mant * ldexp(1.0, -9);
    else v = (8 + mant) * ldexp(1.0, field - 10);
    return (float)(sign ? -v : v);
}

/* RNE to E4M3; magnitudes at or above 448 saturate to 448 (the encoding
 * has no infinity).  NaN maps to 0x7F. */
EXPORT uint8_t oracle_f32_to_e4m3(float v)
{
    uint8_t sign = signbit(v) ? 0x80u : 0u;
    if (isnan(v)) return 0x7Fu;
    double a = fabs((double)v);
    if (a >= 448.0) return (uint8_t)(sign | 0x7Eu);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);
    int ex = e - 1;
    if (ex < -6) ex = -6;
    double spacing = ldexp(1.0, ex - 3);
    double r = nearbyint(a / spacing) * spacing;
    if (r == 0.0) return sign;
    if (r < ldexp(1.0, -6)) return (uint8_t)(sign | (uint8_t)(r / ldexp(1.0, -9)));
    frexp(r, &e);
    ex = e - 1;
    uint8_t mant = (uint8_t)((uint32_t)(r / ldexp(1.0, ex - 3)) - 8u);
    return (uint8_t)(sign | ((ex + 7) << 3) | mant);
}

/* E2M1 (OCP 4-bit float): 1 sign, 2 exponent (bias 1), 1 mantissa bit.
 * Magnitude codes 0..7 are 0, 0.5, 1, 1.5, 2, 3, 4, 6; bit 3 is the sign. */
EXPORT float oracle_e2m1_to_f32(uint8_t c)
{
    static const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    float m = mag[c & 7];
    return (c & 8) ? -m : m;
}

/* RNE to E2M1 with saturation at 6.  The decision points between adjacent
 * magnitudes are their midpoints; on a midpoint the code with the even
 * mantissa bit (the even code index) wins.  Sign is kept, so a negative
 * value that rounds to zero gives the code 0x8. */
EXPORT uint8_t oracle_f32_to_e2m1(float v)
{
    uint8_t sign = signbit(v) ? 8u : 0u;
    float a = fabsf(v);
    uint8_t m;
    if (a <= 0.25f) m = 0;          /* midpoint 0.25: tie to code 0 (even) */
    else if (a < 0.75f) m = 1;      /* midpoint 0.75: tie to code 2 (even) */
    else if (a <= 1.25f) m = 2;     /* midpoint 1.25: tie to code 2 */
    else if (a < 1.75f) m = 3;      /* midpoint 1.75: tie to code 4 */
    else if (a <= 2.5f) m = 4;      /* midpoint 2.5 : tie to code 4 */
    else if (a < 3.5f) m = 5;       /* midpoint 3.5 : tie to code 6 */
    else if (a <= 5.0f) m = 6;      /* midpoint 5   : tie to code 6 */
    else m = 7;                     /* 6 and above (saturating) */
    return (uint8_t)(sign | m);
}

/* ------------------------------------------------------------------------ */
/* packed 4-bit layout: row-major, element k of a row in byte k/2, the even  */
/* element in the low nibble.                                                */
/* ------------------------------------------------------------------------ */
static void put_nibble(uint8_t *row, int64_t k, uint8_t nib)
{
    uint8_t *b = &row[k >> 1];
    if (k & 1) *b = (uint8_t)((*b & 0x0Fu) | (uint8_t)(nib << 4));
    else *b = (uint8_t)((*b & 0xF0u) | (nib & 0x0Fu));
}

static uint8_t get_nibble(const uint8_t *row, int64_t k)
{
    uint8_t b = row[k >> 1];
    return (k & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 0x0Fu);
}

/* two's-complement nibble -> int in [-8, 7] */
static int sext4(uint8_t nib) { return (nib & 8) ? (int)nib - 16 : (int)nib; }

EXPORT void oracle_unpack_int4(int64_t rows, int64_t K, const uint8_t *codes, int8_t *out)
{
    for (int64_t m = 0; m < rows; ++m)
        for (int64_t k = 0; k < K; ++k)
            out[m * K + k] = (int8_t)sext4(get_nibble(codes + m * (K / 2), k));
}

EXPORT void oracle_unpack_u4(int64_t rows, int64_t K, const uint8_t *codes, uint8_t *out)
{
    for (int64_t m = 0; m < rows; ++m)
        for (int64_t k = 0; k < K; ++k)
            out[m * K + k] = get_nibble(codes + m * (K / 2), k);
}

/* ------------------------------------------------------------------------ */
/* O-2 / O-3 / O-4  offline weight preparation                               */
/* ------------------------------------------------------------------------ */

/* Smoothing factors that migrate activation outliers into the weights
 * ([JA] "SVDQuant and the Nunchaku engine"):
 *   s[k] = RNE_bf16( sqrt( max_m |x[m,k]| / max_n |W[n,k]| ) ), in fp64,
 * and s[k] = 1 when either maximum is zero.  The layer then uses x/s and
 * W*s, whose product equals x W^T. */
EXPORT void oracle_smooth_factors(int64_t M, int64_t N, int64_t K,
                                  const uint16_t *x, const uint16_t *W, uint16_t *s)
{
    for (int64_t k = 0; k < K; ++k) {
        double ax = 0.0, aw = 0.0;
        for (int64_t m = 0; m < M; ++m) {
            double a = fabs((double)oracle_bf16_to_f32(x[m * K + k]));
            if (a > ax) ax = a;
        }
        for (int64_t n = 0; n < N; ++n) {
            double a = fabs((double)oracle_bf16_to_f32(W[n * K + k]));
            if (a > aw) aw = a;
        }
        s[k] = (ax == 0.0 || aw == 0.0) ? (uint16_t)0x3F80u : oracle_f64_to_bf16(sqrt(ax / aw));
    }
}

/* Residual after the low-rank branch, fp64, rounded once to fp32:
 *   R[n,k] = W[n,k]*s[k] - sum_j up[n,j]*down[j,k].
 * The rounded (bf16) factors are used, so the 4-bit residual absorbs their
 * rounding error. */
EXPORT void oracle_svdq_residual(int64_t N, int64_t K, int32_t rank,
                                 const uint16_t *W, const uint16_t *s,
                                 const uint16_t *lora_up, const uint16_t *lora_down,
                                 float *R)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            double w = (double)oracle_bf16_to_f32(W[n * K + k]) * (double)oracle_bf16_to_f32(s[k]);
            double lr = 0.0;
            for (int32_t j = 0; j < rank; ++j)
                lr += (double)oracle_bf16_to_f32(lora_up[n * rank + j]) *
                      (double)oracle_bf16_to_f32(lora_down[(int64_t)j * K + k]);
            R[n * K + k] = (float)(w - lr);
        }
}

/* ------------------------------------------------------------------------ */
/* O-6  int4 group quantizer (group 64), rows of fp32 values                 */
/* ------------------------------------------------------------------------ */
/* For each row and each group of 64 consecutive elements:
 *   a   = max |v|                        (exact)
 *   s_f = a / 7                          (fp32, correctly rounded)
 *   s_b = RNE_bf16(s_f)                  (the stored scale)
 *   q   = 0 if s_b == 0, else clamp(RNE(v / s_b), -8, 7)   (fp32 divide)
 * Codes are taken against the stored bf16 scale, so q * s_b is the
 * dequantized value. */
EXPORT void oracle_quantize_int4(int64_t rows, int64_t K, const float *v,
                                 uint8_t *codes, uint16_t *scales)
{
    const int64_t G = 64;
    for (int64_t m = 0; m < rows; ++m) {
        const float *row = v + m * K;
        uint8_t *crow = codes + m * (K / 2);
        for (int64_t g = 0; g < K / G; ++g) {
            float a = 0.0f;
            for (int64_t k = g * G; k < (g + 1) * G; ++k) {
                float x = fabsf(row[k]);
                if (x > a) a = x;
            }
            float s_f = a / 7.0f;
            uint16_t s_b = oracle_f32_to_bf16(s_f);
            float sb = oracle_bf16_to_f32(s_b);
            scales[m * (K / G) + g] = s_b;
            for (int64_t k = g * G; k < (g + 1) * G; ++k) {
                int q = 0;
                if (sb != 0.0f) {
                    float r = nearbyintf(row[k] / sb);
                    if (r > 7.0f) r = 7.0f;
                    if (r < -8.0f) r = -8.0f;
                    q = (int)r;
                }
                put_nibble(crow, k, (uint8_t)(q & 0xF));
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* O-7  NVFP4 group quantizer (group 16)                                     */
/* ------------------------------------------------------------------------ */
/* For each row and group of 16:
 *   a   = max |v|
 *   s_f = a / 6                          (fp32; 6 is the largest E2M1 value)
 *   s_e = E4M3_RNE_sat(s_f / g_tensor), g_tensor = 1
 *   d   = dec(s_e); if d == 0 all codes are 0x0
 *   c   = E2M1_RNE_sat(v / d)            (fp32 divide)            */
EXPORT void oracle_quantize_nvfp4(int64_t rows, int64_t K, const float *v,
                                  uint8_t *codes, uint8_t *scales)
{
    const int64_t G = 16;
    for (int64_t m = 0; m < rows; ++m) {
        const float *row = v + m * K;
        uint8_t *crow = codes + m * (K / 2);
        for (int64_t g = 0; g < K / G; ++g) {
            float a = 0.0f;
            for (int64_t k = g * G; k < (g + 1) * G; ++k) {
                float x = fabsf(row[k]);
                if (x > a) a = x;
            }
            float s_f = a / 6.0f;
            uint8_t s_e = oracle_f32_to_e4m3(s_f / 1.0f);
            float d = oracle_e4m3_to_f32(s_e);
            scales[m * (K / G) + g] = s_e;
            for (int64_t k = g * G; k < (g + 1) * G; ++k) {
                uint8_t c = (d == 0.0f) ? 0u : oracle_f32_to_e2m1(row[k] / d);
                put_nibble(crow, k, c);
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* O-5 / O-8 / O-6,7  runtime activation path (first fused step)            */
/* ------------------------------------------------------------------------ */

/* x_hat[m,k] = RNE_bf16( f32(x[m,k]) / f32(s[k]) ), fp32 divide.
 * smooth == NULL means s = 1. */
EXPORT void oracle_smooth_act(int64_t M, int64_t K, const uint16_t *x,
                              const uint16_t *smooth, uint16_t *xhat)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            float xv = oracle_bf16_to_f32(x[m * K + k]);
            float sv = smooth ? oracle_bf16_to_f32(smooth[k]) : 1.0f;
            xhat[m * K + k] = oracle_f32_to_bf16(xv / sv);
        }
}

/* Low-rank down-projection t = x_hat . L1^T, summed in fp64 and rounded
 * once to fp32.  lora_down is [rank, K]. */
EXPORT void oracle_lowrank_down(int64_t M, int64_t K, int32_t rank,
                                const uint16_t *xhat, const uint16_t *lora_down, float *t)
{
    for (int64_t m = 0; m < M; ++m)
        for (int32_t j = 0; j < rank; ++j) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += (double)oracle_bf16_to_f32(xhat[m * K + k]) *
                       (double)oracle_bf16_to_f32(lora_down[(int64_t)j * K + k]);
            t[m * rank + j] = (float)acc;
        }
}

/* The activation half of the layer: smooth, low-rank down-projection and
 * group quantization of the same bf16 x_hat.  precision 0 = int4 (codes
 * [M,K/2], bf16 scales [M,K/64]); 1 = NVFP4 (codes [M,K/2], E4M3 scales
 * [M,K/16]).  xhat_scratch is [M,K] bf16, vals_scratch is [M,K] fp32. */
EXPORT void oracle_svdq_quantize_act(int32_t precision, int64_t M, int64_t K, int32_t rank,
                                     const uint16_t *x, const uint16_t *smooth,
                                     const uint16_t *lora_down,
                                     uint8_t *act_codes, void *act_scales, float *lora_act,
                                     uint16_t *xhat_scratch, float *vals_scratch)
{
    oracle_smooth_act(M, K, x, smooth, xhat_scratch);
    if (rank > 0) oracle_lowrank_down(M, K, rank, xhat_scratch, lora_down, lora_act);
    for (int64_t i = 0; i < M * K; ++i) vals_scratch[i] = oracle_bf16_to_f32(xhat_scratch[i]);
    if (precision == 0)
        oracle_quantize_int4(M, K, vals_scratch, act_codes, (uint16_t *)act_scales);
    else
        oracle_quantize_nvfp4(M, K, vals_scratch, act_codes, (uint8_t *)act_scales);
}

/* ------------------------------------------------------------------------ */
/* O-9  int4 W4A4 GEMM with low-rank up-projection and bias                  */
/* ------------------------------------------------------------------------ */

/* Integer group sums G[m,n,g] = sum_{k in group g} qx[m,k]*qw[n,k]. */
EXPORT void oracle_group_sums_int4(int64_t M, int64_t N, int64_t K,
                                   const uint8_t *act_codes, const uint8_t *wgt_codes, int32_t *G)
{
    const int64_t NG = K / 64;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            for (int64_t g = 0; g < NG; ++g) {
                int32_t acc = 0;
                for (int64_t k = g * 64; k < (g + 1) * 64; ++k)
                    acc += sext4(get_nibble(act_codes + m * (K / 2), k)) *
                           sext4(get_nibble(wgt_codes + n * (K / 2), k));
                G[(m * N + n) * NG + g] = acc;
            }
}

/* Low-rank up-projection plus bias for one output, fp64. */
static double lowrank_up_plus_bias(int64_t m, int64_t n, int32_t rank,
                                   const float *lora_act, const uint16_t *lora_up,
                                   const uint16_t *bias)
{
    double acc = 0.0;
    for (int32_t j = 0; j < rank; ++j)
        acc += (double)lora_act[m * rank + j] * (double)oracle_bf16_to_f32(lora_up[n * rank + j]);
    if (bias) acc += (double)oracle_bf16_to_f32(bias[n]);
    return acc;
}

/* y[m,n] = RNE_bf16( alpha * sum_g G[m,n,g]*sx[m,g]*sw[n,g]
 *                    + sum_j t[m,j]*up[n,j] + bias[n] ), all in fp64.
 * act_* and wgt_* point at row 0 of the rows to compute; out is [M,N]. */
static void gemm_int4(int64_t M, int64_t N, int64_t K, int32_t rank,
                      const uint8_t *act_codes, const uint16_t *act_scales,
                      const uint8_t *wgt_codes, const uint16_t *wgt_scales, float alpha,
                      const float *lora_act, const uint16_t *lora_up, const uint16_t *bias,
                      uint16_t *out)
{
    const int64_t NG = K / 64;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t g = 0; g < NG; ++g) {
                int32_t gs = 0;
                for (int64_t k = g * 64; k < (g + 1) * 64; ++k)
                    gs += sext4(get_nibble(act_codes + m * (K / 2), k)) *
                          sext4(get_nibble(wgt_codes + n * (K / 2), k));
                acc += (double)gs * (double)oracle_bf16_to_f32(act_scales[m * NG + g]) *
                       (double)oracle_bf16_to_f32(wgt_scales[n * NG + g]);
            }
            double y = (double)alpha * acc + lowrank_up_plus_bias(m, n, rank, lora_act, lora_up, bias);
            out[m * N + n] = oracle_f64_to_bf16(y);
        }
}

/* ------------------------------------------------------------------------ */
/* O-10  NVFP4 W4A4 GEMM                                                      */
/* ------------------------------------------------------------------------ */
/* y = RNE_bf16( alpha * sum_k dec(cx)dec(sx)dec(cw)dec(sw) + t.up + bias ),
 * fp64. */
static void gemm_nvfp4(int64_t M, int64_t N, int64_t K, int32_t rank,
                       const uint8_t *act_codes, const uint8_t *act_scales,
                       const uint8_t *wgt_codes, const uint8_t *wgt_scales, float alpha,
                       const float *lora_act, const uint16_t *lora_up, const uint16_t *bias,
                       uint16_t *out)
{
    const int64_t NG = K / 16;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double a = (double)oracle_e2m1_to_f32(get_nibble(act_codes + m * (K / 2), k)) *
                           (double)oracle_e4m3_to_f32(act_scales[m * NG + k / 16]);
                double b = (double)oracle_e2m1_to_f32(get_nibble(wgt_codes + n * (K / 2), k)) *
                           (double)oracle_e4m3_to_f32(wgt_scales[n * NG + k / 16]);
                acc += a * b;
            }
            double y = (double)alpha * acc + lowrank_up_plus_bias(m, n, rank, lora_act, lora_up, bias);
            out[m * N + n] = oracle_f64_to_bf16(y);
        }
}

/* The second fused step of the layer ([JA] "SVDQuant and the Nunchaku
 * engine": 4-bit compute with the low-rank up-projection).  out is [M,N]
 * bf16; bias may be NULL; rank may be 0 (lora_act / lora_up unused). */
EXPORT void oracle_svdq_gemm_w4a4(int32_t precision, int64_t M, int64_t N, int64_t K, int32_t rank,
                                  const uint8_t *act_codes, const void *act_scales,
                                  const uint8_t *wgt_codes, const void *wgt_scales, float alpha,
                                  const float *lora_act, const uint16_t *lora_up,
                                  const uint16_t *bias, uint16_t *out)
{
    if (precision == 0)
        gemm_int4(M, N, K, rank, act_codes, (const uint16_t *)act_scales, wgt_codes,
                  (const uint16_t *)wgt_scales, alpha, lora_act, lora_up, bias, out);
    else
        gemm_nvfp4(M, N, K, rank, act_codes, (const uint8_t *)act_scales, wgt_codes,
                   (const uint8_t *)wgt_scales, alpha, lora_act, lora_up, bias, out);
}

/* ------------------------------------------------------------------------ */
/* O-11  AWQ-style W4A16 (int4 weight-only, group 64)                        */
/* ------------------------------------------------------------------------ */
/* Offline, per weight row n and group of 64 ([DOC] "Supported quantization
 * types": awq_w4a16 int4 g64; asymmetric unsigned codes with a zero point):
 *   lo = min(0, min w), hi = max(0, max w)    over f32(W)
 *   s  = RNE_bf16((hi - lo) / 15)             (fp32 divide)
 *   if s == 0: z = 0, q = 0
 *   else z = clamp(RNE(-lo / s), 0, 15), q = clamp(RNE(w / s) + z, 0, 15)
 * z is stored as bf16 (an exact small integer). */
EXPORT void oracle_awq_quantize_weight(int64_t N, int64_t K, const uint16_t *W,
                                       uint8_t *codes, uint16_t *scales, uint16_t *zeros)
{
    const int64_t G = 64, NG = K / 64;
    for (int64_t n = 0; n < N; ++n) {
        uint8_t *crow = codes + n * (K / 2);
        for (int64_t g = 0; g < NG; ++g) {
            float lo = 0.0f, hi = 0.0f;
            for (int64_t k = g * G; k < (g + 1) * G; ++k) {
                float w = oracle_bf16_to_f32(W[n * K + k]);
                if (w < lo) lo = w;
                if (w > hi) hi = w;
            }
            uint16_t s_b = oracle_f32_to_bf16((hi - lo) / 15.0f);
            float s = oracle_bf16_to_f32(s_b);
            float z = 0.0f;
            if (s != 0.0f) {
                z = nearbyintf(-lo / s);
                if (z < 0.0f) z = 0.0f;
                if (z > 15.0f) z = 15.0f;
            }
            scales[n * NG + g] = s_b;
            zeros[n * NG + g] = oracle_f32_to_bf16(z);
            for (int64_t k = g * G; k < (g + 1) * G; ++k) {
                float q = 0.0f;
                if (s != 0.0f) {
                    q = nearbyintf(oracle_bf16_to_f32(W[n * K + k]) / s) + z;
                    if (q < 0.0f) q = 0.0f;
                    if (q > 15.0f) q = 15.0f;
                }
                put_nibble(crow, k, (uint8_t)q);
            }
        }
    }
}

/* Runtime, y[m,n] = RNE_bf16( sum_k x[m,k]*(q[n,k]-z[n,g])*s[n,g] + bias[n] ),
 * fp64.  out is [M,N]; bias may be NULL. */
EXPORT void oracle_awq_gemv_w4a16(int64_t M, int64_t N, int64_t K, int32_t group_size,
                                  const uint16_t *x, const uint8_t *codes,
                                  const uint16_t *scales, const uint16_t *zeros,
                                  const uint16_t *bias, uint16_t *out)
{
    const int64_t NG = K / group_size;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                int64_t g = k / group_size;
                double w = ((double)get_nibble(codes + n * (K / 2), k) -
                            (double)oracle_bf16_to_f32(zeros[n * NG + g])) *
                           (double)oracle_bf16_to_f32(scales[n * NG + g]);
                acc += (double)oracle_bf16_to_f32(x[m * K + k]) * w;
            }
            if (bias) acc += (double)oracle_bf16_to_f32(bias[n]);
            out[m * N + n] = oracle_f64_to_bf16(acc);
        }
}

/* ------------------------------------------------------------------------ */
/* array forms of the codecs (the Python wrapper calls these)               */
/* ------------------------------------------------------------------------ */
EXPORT void oracle_bf16_to_f32_array(int64_t n, const uint16_t *in, float *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_to_f32(in[i]);
}
EXPORT void oracle_f32_to_bf16_array(int64_t n, const float *in, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_bf16(in[i]);
}
EXPORT void oracle_f64_to_bf16_array(int64_t n, const double *in, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_bf16(in[i]);
}
EXPORT void oracle_e4m3_to_f32_array(int64_t n, const uint8_t *in, float *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_to_f32(in[i]);
}
EXPORT void oracle_f32_to_e4m3_array(int64_t n, const float *in, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_e4m3(in[i]);
}
EXPORT void oracle_e2m1_to_f32_array(int64_t n, const uint8_t *in, float *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e2m1_to_f32(in[i]);
}
EXPORT void oracle_f32_to_e2m1_array(int64_t n, const float *in, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_e2m1(in[i]);
}

/* ------------------------------------------------------------------------ */
/* O-12  GELU (tanh form) on bf16 values                                     */
/* ------------------------------------------------------------------------ */
/* The original engine runs the MLP's GELU fused into its kernels ([DOC]
 * "Fused kernels": a fused GELU kernel for the MLP).  The pages name neither
 * the GELU variant nor its precision; readings:
 *   - the tanh form, gelu(y) = y/2 * (1 + tanh( sqrt(2/pi) * (y + 0.044715 y^3) )),
 *     the variant of the DiT feed-forward blocks this layer serves;
 *   - input and output are bf16 (compute_dtype): the result is the exact
 *     function value rounded once to bf16 (RNE);
 *   - non-finite inputs: +inf -> +inf, -inf -> -0 (the limit), NaN -> NaN.
 * Evaluation in fp64 as y / (1 + exp(-2u)), u = sqrt(2/pi) (y + 0.044715 y^3):
 * the same function (1 + tanh u = 2 / (1 + e^{-2u})) without the cancellation
 * of 1 + tanh u for large negative u.  Ties: the exact value is a bf16
 * rounding midpoint only in the limit of tiny |y|, where
 * gelu(y) = y/2 + (y tanh u)/2 and the second term is positive but below
 * fp64's resolution; so when the fp64 value lands exactly on a midpoint the
 * exact value lies above it, and the tie goes toward +infinity. */
static double gelu_tanh_f64(double y)
{
    const double c = 0.79788456080286535588;   /* sqrt(2/pi) */
    const double u = c * (y + 0.044715 * y * y * y);
    return y / (1.0 + exp(-2.0 * u));
}

EXPORT uint16_t oracle_gelu_tanh_bf16(uint16_t h)
{
    const double y = (double)oracle_bf16_to_f32(h);
    if (isnan(y)) return (uint16_t)((h & 0x8000u) | 0x7FC0u);
    if (isinf(y)) return y > 0 ? (uint16_t)0x7F80u : (uint16_t)0x8000u;
    if (y == 0.0) return h;                       /* gelu(+-0) = +-0 */
    const double v = gelu_tanh_f64(y);
    const double a = fabs(v);
    if (a < ldexp(1.0, -126)) {
        /* bf16 subnormal range: spacing 2^-133, scaling exact */
        const double s = a / ldexp(1.0, -133);
        double q = nearbyint(s);
        if (s - floor(s) == 0.5) q = v > 0 ? ceil(s) : floor(s);   /* tie toward +infinity */
        const uint16_t sign = signbit(v) ? 0x8000u : 0u;   /* -0 when exp(-2u) overflowed */
        return (uint16_t)(sign | (uint16_t)q);    /* q = 128 is the least normal, encoded alike */
    }
    return oracle_f64_to_bf16(v);
}

EXPORT void oracle_gelu_tanh_bf16_array(int64_t n, const uint16_t *in, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_gelu_tanh_bf16(in[i]);
}

/* ------------------------------------------------------------------------ */
/* O-13  per-head RMSNorm + rotary embedding of the Q and K projections      */
/* ------------------------------------------------------------------------ */
/* The original engine fuses the grouped Q, K, V projection with RMSNorm and
 * RoPE ([DOC] "Fused kernels").  The pages give neither the head size nor the
 * rotary layout; readings:
 *   - heads of D = 128 channels; the N = 3 H D output columns are Q | K | V,
 *     head h of Q at columns h D .. h D + 127 (likewise K, V);
 *   - RMSNorm of each (row, Q or K head) over its D channels with its own
 *     bf16 weight w (one for Q, one for K, shared by the heads):
 *       n_j = y_j * w_j / sqrt( (1/D) sum_i y_i^2 + eps );
 *   - the rotary embedding turns each adjacent channel pair (2i, 2i+1) of n
 *     by the row's angle for pair i, given as cos/sin (fp32 [M, D/2], the
 *     caller's positions and frequencies):
 *       out_2i   = n_2i cos_i - n_2i+1 sin_i
 *       out_2i+1 = n_2i+1 cos_i + n_2i sin_i;
 *   - y is the layer's bf16 output (the unfused path's stored value); the
 *     result is computed in fp64 and rounded once to bf16; V is unchanged. */
EXPORT void oracle_qk_norm_rope(int64_t M, int64_t N, const uint16_t *y, const uint16_t *q_w,
                                const uint16_t *k_w, double eps, const float *rope_cos,
                                const float *rope_sin, uint16_t *out)
{
    const int64_t D = 128, HD = N / 3;
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t *yr = y + m * N;
        uint16_t *orow = out + m * N;
        for (int64_t c = 2 * HD; c < N; ++c) orow[c] = yr[c];          /* V */
        for (int64_t c0 = 0; c0 < 2 * HD; c0 += D) {                    /* Q and K heads */
            const uint16_t *w = c0 < HD ? q_w : k_w;
            double ss = 0.0;
            for (int64_t j = 0; j < D; ++j) {
                const double v = (double)oracle_bf16_to_f32(yr[c0 + j]);
                ss += v * v;
            }
            const double r = 1.0 / sqrt(ss / (double)D + eps);
            for (int64_t i = 0; i < D / 2; ++i) {
                const double n0 = (double)oracle_bf16_to_f32(yr[c0 + 2 * i]) * r * (double)oracle_bf16_to_f32(w[2 * i]);
                const double n1 = (double)oracle_bf16_to_f32(yr[c0 + 2 * i + 1]) * r * (double)oracle_bf16_to_f32(w[2 * i + 1]);
                const double cs = (double)rope_cos[m * (D / 2) + i], sn = (double)rope_sin[m * (D / 2) + i];
                orow[c0 + 2 * i] = oracle_f64_to_bf16(n0 * cs - n1 * sn);
                orow[c0 + 2 * i + 1] = oracle_f64_to_bf16(n1 * cs + n0 * sn);
            }
        }
    }
}
