/*
 * svdq.h -- C ABI of the MI355X (gfx950) SVDQuant W4A4 / AWQ W4A16 layer
 * library (libsvdq.so).
 *
 * The layer ("Nunchaku Lite" Diffusers docs, table "Supported quantization
 * types"; blog "Hugging Face integrates Nunchaku 4-bit diffusion inference
 * into Diffusers", section "SVDQuant and the Nunchaku engine"):
 *   W4A4:  y = alpha * Q(x / s) . Q(R)^T  +  (x/s . L1^T) . L2^T  +  bias
 *          where s migrates activation outliers into the weights, L1 / L2
 *          are the 16-bit low-rank branch (rank r) and R is the 4-bit
 *          residual.  The computation is two calls: svdq_quantize_act
 *          (smooth, low-rank down-projection, group quantization: one pass
 *          over x) and svdq_gemm_w4a4 (4-bit GEMM with the low-rank
 *          up-projection and bias in its epilogue).
 *   W4A16: y = x . dequant(q, s, z)^T + bias, int4 weights in groups of 64
 *          with bf16 scales and zero points (awq_gemv_w4a16).
 *
 * Conventions for every call
 *  - All tensor pointers are DEVICE pointers owned by the caller; the
 *    library never allocates, frees or synchronizes.  Work is enqueued on
 *    `stream` (a hipStream_t; NULL is the null stream) and is asynchronous.
 *  - Layouts are row-major and dense.  bf16 values are IEEE binary16-brain
 *    bit patterns.  "codes" are packed 4-bit values: [rows, K/2] bytes,
 *    element k of a row in byte k/2, even k in the low nibble.
 *  - int4 codes are two's complement in [-8, 7]; int4 group size 64 with
 *    bf16 scales.  NVFP4 codes are E2M1 (bit 3 = sign), group size 16 with
 *    E4M3 ("FN" variant) scales.  AWQ codes are unsigned in [0, 15].
 *  - Argument checks run on the host before anything is enqueued; a failed
 *    check returns SVDQ_ERR_INVALID_ARG or SVDQ_ERR_UNSUPPORTED and
 *    enqueues nothing.  Requirements: pointers 16-byte aligned; K a
 *    positive multiple of 64; M >= 0 and N >= 0 (zero-sized calls return
 *    SVDQ_OK and enqueue nothing); rank a multiple of 16 in [0, 128];
 *    M, N <= 2^24 and K <= 2^16; the current device is gfx950.
 *  - A launch failure returns SVDQ_ERR_HIP.  Faults inside a kernel surface
 *    at the caller's next synchronization.  Outputs must not alias inputs.
 *    Calls keep no state besides a per-device architecture check; they may
 *    be made from several threads.  Non-finite inputs, and finite ones whose
 *    smoothed value x/smooth overflows, give unspecified (but memory-safe)
 *    outputs.
 */
#ifndef SVDQ_H
#define SVDQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum svdq_status {
    SVDQ_OK = 0,
    SVDQ_ERR_INVALID_ARG = 1,
    SVDQ_ERR_UNSUPPORTED = 2,
    SVDQ_ERR_HIP = 3
} svdq_status;

/* precision of the W4A4 layer ("Supported quantization types" table).
 * SVDQ_INT4_PACKED is int4 with the weight in the packed form written by
 * svdq_pack_weight_int4; its activations are int4's.  SVDQ_INT4_FP6 is int4
 * (the same codes and scales) with both operands' codes in the FP6 tiled layout:
 * the activations from svdq_quantize_act / svdq_gelu_quantize_act called
 * with SVDQ_INT4_FP6, the weight from svdq_pack_weight_fp6 (the GEMM's
 * fastest path).
 *
 * FP6 tiled layout of int4 codes [rows, K] (svdq_fp6_codes_bytes(rows, K)
 * bytes): per row and group of 64, two 192-bit strings, one per half h of
 * the group; field j of a string (bits 6j .. 6j+5) is the E2M3 encoding (sign
 * bit 5, two exponent bits with bias 1, three mantissa bits) of q/2 for
 * channel 64g + 32h + j, exact for every q in [-8, 7] (a zero code is +0).
 * Bits are numbered from the least significant bit of word 0 of a string.
 * A row's group g is three 16-byte chunks: c = 0: words 0-3 of h0, c = 1:
 * words 0-3 of h1, c = 2: words 4-5 of h0 then words 4-5 of h1, the two
 * halves of chunk 2 swapped (h1's words first) when s(r) = 1.  Rows are
 * stored in tiles of 128 (the last one padded) and groups in pairs (the last
 * one padded when K/64 is odd); with p = r % 128, rot(r) = ((p >> 2) xor
 * (p >> 3)) & 1 and s(r) = ((p >> 3) xor (p >> 4)) & 1, chunk c of group g
 * of row r is at byte
 *   ((r / 128) * ceil(K/128) + g / 2) * 12288 + p * 96
 *     + 16 * ((3 * (g % 2) + c + rot(r)) mod 6),
 * so each (tile, pair) is one contiguous 12 KB block: the GEMM's LDS stage,
 * copied with whole cache lines (rot and s place the 16 rows whose
 * fragments one LDS cycle serves on distinct banks).  Padding is never written or needed: the
 * GEMM only multiplies it into outputs it does not store, or by a zero scale. */
enum {
    SVDQ_INT4 = 0 /* group 64, bf16 scales */,
    SVDQ_NVFP4 = 1 /* group 16, E4M3 scales */,
    SVDQ_INT4_PACKED = 2 /* int4, weight from svdq_pack_weight_int4 (GEMM calls only) */,
    SVDQ_INT4_FP6 = 3 /* int4, codes of both operands in the FP6 tiled layout */
};

/*
 * svdq_quantize_act -- first step of the W4A4 layer: one pass over x.
 *   x_hat[m,k]  = RNE_bf16( x[m,k] / smooth[k] )        (fp32 quotient)
 *   lora_act    = x_hat . lora_down^T                    (fp32, [M, rank])
 *   int4 : per row and group of 64, scale = RNE_bf16(absmax/7),
 *          code = RNE(x_hat/scale) (ties to even), zero scale -> zero codes
 *   nvfp4: per row and group of 16, scale = E4M3_RNE_sat(absmax/6),
 *          code = E2M1_RNE_sat(x_hat/scale), zero scale -> zero codes
 * The method fuses the low-rank down-projection into the quantize kernel
 * ("SVDQuant and the Nunchaku engine").  Codes and scales are bit-exact
 * against the rule above; lora_act is an fp32 sum in unspecified order.
 *
 *   precision  SVDQ_INT4, SVDQ_NVFP4 or SVDQ_INT4_FP6 (int4's codes and
 *              scales, the codes written in the FP6 tiled layout)
 *   x          bf16 [M, K]
 *   smooth     bf16 [K] smoothing factors; NULL means 1
 *   lora_down  bf16 [rank, K]; ignored (may be NULL) when rank == 0
 *   act_codes  out: u8 [M, K/2]; SVDQ_INT4_FP6: the FP6 tiled layout,
 *              svdq_fp6_codes_bytes(M, K) bytes
 *   act_scales out: int4 bf16 [M, K/64]; nvfp4 u8 (E4M3) [M, K/16]
 *   lora_act   out: fp32 [M, rank]; ignored (may be NULL) when rank == 0
 */
svdq_status svdq_quantize_act(int32_t precision, int64_t M, int64_t K, int32_t rank,
                              const void *x, const void *smooth, const void *lora_down,
                              void *act_codes, void *act_scales, float *lora_act,
                              void *stream);

/*
 * svdq_gelu_quantize_act -- svdq_quantize_act of GELU(x), for the layer that
 * consumes a GELU MLP's up projection: x is that projection's bf16 output
 * and the GELU runs inside this step, so it makes no pass of its own over
 * the intermediate ("Nunchaku Lite" docs, "Fused kernels": the original
 * engine's MLP uses a fused GELU).  GELU is the tanh form,
 *   gelu(y) = y/2 * (1 + tanh( sqrt(2/pi) * (y + 0.044715 y^3) )),
 * rounded once to bf16 from its exact value (bit-exact for every bf16 y;
 * +inf -> +inf, -inf -> -0, NaN -> quiet NaN).  Arguments, layouts, checks
 * and results are those of svdq_quantize_act with x replaced by GELU(x).
 */
svdq_status svdq_gelu_quantize_act(int32_t precision, int64_t M, int64_t K, int32_t rank,
                                   const void *x, const void *smooth, const void *lora_down,
                                   void *act_codes, void *act_scales, float *lora_act,
                                   void *stream);

/*
 * svdq_gemm_w4a4 -- second step: 4-bit GEMM with the fused low-rank
 * up-projection and bias ("SVDQuant and the Nunchaku engine": the
 * up-projection is fused into the 4-bit compute kernel).
 *   y[m,n] = RNE_bf16( alpha * sum_k deq(act)[m,k] * deq(wgt)[n,k]
 *                      + sum_j lora_act[m,j] * lora_up[n,j] + bias[n] )
 * deq is code * group scale.  The sum is fp32 in unspecified order.
 *
 *   precision  SVDQ_INT4, SVDQ_NVFP4, SVDQ_INT4_PACKED (the activations
 *              then come from svdq_quantize_act with SVDQ_INT4) or
 *              SVDQ_INT4_FP6 (activations from svdq_quantize_act with
 *              SVDQ_INT4_FP6)
 *   act_codes, act_scales  as written by svdq_quantize_act ([M, ...])
 *   wgt_codes  u8 [N, K/2] (int4 or E2M1 codes of the 4-bit residual);
 *              SVDQ_INT4_PACKED: the svdq_pack_weight_int4 blob of them
 *              (svdq_packed_weight_bytes(N, K) bytes); SVDQ_INT4_FP6: the
 *              svdq_pack_weight_fp6 form (svdq_fp6_codes_bytes(N, K) bytes)
 *   wgt_scales int4 bf16 [N, K/64]; nvfp4 u8 (E4M3) [N, K/16]
 *   alpha      scale of the 4-bit term (per-tensor; 1.0f for int4)
 *   lora_act   fp32 [M, rank]; lora_up bf16 [N, rank]; ignored when rank == 0
 *   bias       bf16 [N] or NULL
 *   out        out: bf16 [M, N]
 */
svdq_status svdq_gemm_w4a4(int32_t precision, int64_t M, int64_t N, int64_t K, int32_t rank,
                           const void *act_codes, const void *act_scales,
                           const void *wgt_codes, const void *wgt_scales, float alpha,
                           const float *lora_act, const void *lora_up, const void *bias,
                           void *out, void *stream);

/*
 * svdq_gemm_w4a4_qk_norm_rope -- svdq_gemm_w4a4 of a grouped QKV projection
 * with per-head RMSNorm and rotary embedding of Q and K in the epilogue (the
 * original engine fuses the QKV projection with RMSNorm and RoPE: "Nunchaku
 * Lite" docs, "Fused kernels").  Heads are 128 channels; the N = 3 H 128
 * output columns are Q | K | V, head h of Q at columns 128h .. 128h + 127.
 * With y the bf16 output svdq_gemm_w4a4 would write, for each row and each Q
 * or K head:
 *   n_j = y_j * w_j / sqrt( (1/128) sum_i y_i^2 + eps )   (w = q or k weight)
 *   out_2i   = RNE_bf16( n_2i cos[m,i] - n_2i+1 sin[m,i] )
 *   out_2i+1 = RNE_bf16( n_2i+1 cos[m,i] + n_2i sin[m,i] ),   i < 64,
 * computed in fp32; V columns are y.  Arguments as for svdq_gemm_w4a4, plus:
 *   precision      SVDQ_INT4, SVDQ_NVFP4, SVDQ_INT4_PACKED or SVDQ_INT4_FP6
 *   N              a multiple of 384
 *   q_norm_weight  bf16 [128]; k_norm_weight bf16 [128]
 *   eps            finite, >= 0
 *   rope_cos, rope_sin  fp32 [M, 64]: each row's rotary angle per channel pair
 */
svdq_status svdq_gemm_w4a4_qk_norm_rope(int32_t precision, int64_t M, int64_t N, int64_t K, int32_t rank,
                                        const void *act_codes, const void *act_scales,
                                        const void *wgt_codes, const void *wgt_scales, float alpha,
                                        const float *lora_act, const void *lora_up, const void *bias,
                                        const void *q_norm_weight, const void *k_norm_weight, float eps,
                                        const float *rope_cos, const float *rope_sin, void *out,
                                        void *stream);

/*
 * svdq_gemm_w4a4_gelu_quantize -- the up projection of a GELU MLP with the
 * down layer's activation step in its epilogue, so that the [M, N] bf16
 * intermediate is not written ("Nunchaku Lite" docs, "Fused kernels": the
 * original engine runs the MLP's GELU fused into its kernels).  Int4 in the
 * FP6 layout only.  With y the bf16 output svdq_gemm_w4a4(SVDQ_INT4_FP6, ...)
 * would write, the outputs are exactly what svdq_gelu_quantize_act(
 * SVDQ_INT4_FP6, y, smooth_next, lora_down_next, ...) writes: the same codes
 * and scales bit for bit; next_lora_act equal up to fp32 summation order
 * (here: partial sums over 128-column tiles, added in tile order, so a given
 * shape gives the same bits on every run).
 *   precision       SVDQ_INT4_FP6 (input operands and output codes)
 *   M, N, K, rank, act_codes ... bias   as for svdq_gemm_w4a4; N <= 65536
 *   rank_next       rank of the down layer (0 or a multiple of 16 up to 128)
 *   smooth_next     bf16 [N] or NULL (s = 1): the down layer's smoothing
 *   lora_down_next  bf16 [rank_next, N]; NULL iff rank_next == 0
 *   next_codes      out: the FP6 tiled layout of [M, N] (svdq_fp6_codes_bytes(M, N))
 *   next_scales     out: bf16 [M, N/64]
 *   next_lora_act   out: fp32 [M, rank_next]; NULL iff rank_next == 0
 *   workspace       device memory of at least
 *                   svdq_gelu_quantize_workspace_bytes(M, N, rank_next) bytes
 *                   (ceil(N/128) * M * rank_next * 4: the fp32 low-rank
 *                   partials of the 128-column tiles), owned by the caller;
 *                   its contents need no initialisation and are scratch
 *                   (calls that share a workspace must be ordered, e.g. on
 *                   one stream); may be NULL when that size is 0
 *   out             bf16 [M, N], or NULL: where given, also receives y
 * Two kernels are enqueued on `stream` (one when rank_next is 0).
 */
int64_t svdq_gelu_quantize_workspace_bytes(int64_t M, int64_t N, int32_t rank_next);   /* -1 if invalid */
svdq_status svdq_gemm_w4a4_gelu_quantize(int32_t precision, int64_t M, int64_t N, int64_t K, int32_t rank,
                                         const void *act_codes, const void *act_scales,
                                         const void *wgt_codes, const void *wgt_scales, float alpha,
                                         const float *lora_act, const void *lora_up, const void *bias,
                                         int32_t rank_next, const void *smooth_next, const void *lora_down_next,
                                         void *next_codes, void *next_scales, float *next_lora_act,
                                         void *workspace, int64_t workspace_bytes, void *out, void *stream);

/*
 * awq_gemv_w4a16 -- int4 weight-only layer with bf16 activations, for the
 * memory-bound, precision-sensitive layers (adaptive-norm modulation;
 * "Nunchaku Lite" docs, awq_w4a16 int4 group 64).
 *   y[m,n] = RNE_bf16( sum_k x[m,k] * (q[n,k] - z[n,k/64]) * s[n,k/64] + bias[n] )
 * The sum is fp32 in unspecified order.  Any M works.  Small M runs as a
 * GEMV that streams the weights once per 32 rows of x; when K is a multiple
 * of 512, M >= 32 and ceil(M/32) * ceil(N/32) >= 576 it runs as a tiled
 * matrix-core GEMM (bf16 products over 128 x 128 output tiles, codes unpacked
 * in registers).  Both paths give the same result up to fp32 summation order.
 *
 *   group_size must be 64
 *   x          bf16 [M, K]
 *   wgt_codes  u8 [N, K/2], unsigned codes 0..15
 *   wgt_scales bf16 [N, K/64]
 *   wgt_zeros  bf16 [N, K/64], integer values 0..15
 *   bias       bf16 [N] or NULL
 *   out        out: bf16 [M, N]
 */
svdq_status awq_gemv_w4a16(int64_t M, int64_t N, int64_t K, int32_t group_size,
                           const void *x, const void *wgt_codes, const void *wgt_scales,
                           const void *wgt_zeros, const void *bias, void *out, void *stream);

/*
 * Offline weight preparation ("SVDQuant and the Nunchaku engine": activation
 * outliers migrate into the weights, the hardest part of each weight stays
 * in a 16-bit low-rank branch, the residual is quantized to 4 bits).
 *
 * svdq_smooth_factors -- smoothing factors from calibration activations:
 *   smooth[k] = RNE_bf16( sqrt( max_m |x[m,k]| / max_n |W[n,k]| ) )
 * (fp64 quotient and square root), 1 when either maximum is 0.
 *   x       bf16 [M, K] calibration activations (M >= 0)
 *   W       bf16 [N, K] the layer's weight
 *   smooth  out: bf16 [K]
 */
svdq_status svdq_smooth_factors(int64_t M, int64_t N, int64_t K, const void *x, const void *W, void *smooth,
                                void *stream);

/*
 * svdq_lowrank_factors -- the 16-bit low-rank branch of the smoothed weight
 * W_hat = W diag(smooth): approximately its top-rank singular triplets, as
 *   lora_up[n,j] = RNE_bf16(U[n,j]),  lora_down[j,k] = RNE_bf16(sigma_j V[k,j]),
 * each left vector's largest-magnitude entry positive.  Randomized subspace
 * iteration (a Gaussian sketch of rank + 8 columns drawn from `seed`, two
 * power iterations, CholeskyQR2 bases, a small Jacobi eigendecomposition):
 * the residual norm is close to, not equal to, the optimal one; results
 * depend on `seed` and are repeatable for a given seed and device.
 *   W          bf16 [N, K]; smooth bf16 [K] or NULL (= 1)
 *   rank       multiple of 16 in [16, 128]; N, K >= rank + 8
 *   workspace  device scratch of at least svdq_lowrank_workspace_bytes(N, K,
 *              rank) bytes, owned by the caller; contents on return unspecified
 *   lora_up    out: bf16 [N, rank]; lora_down out: bf16 [rank, K]
 */
int64_t svdq_lowrank_workspace_bytes(int64_t N, int64_t K, int32_t rank);   /* -1 if invalid */
svdq_status svdq_lowrank_factors(int64_t N, int64_t K, int32_t rank, const void *W, const void *smooth,
                                 uint64_t seed, void *workspace, int64_t workspace_bytes, void *lora_up,
                                 void *lora_down, void *stream);

/*
 * svdq_lowrank_factors_noalloc -- svdq_lowrank_factors for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same kernels and results (bit
 * for bit, for the same arguments and seed), with the workspace taken from a
 * fixed scratch array that the library holds on each device from its load
 * until the process ends.  The call allocates and frees nothing.
 *   arguments  as svdq_lowrank_factors, without workspace / workspace_bytes
 *   limit      svdq_lowrank_workspace_bytes(N, K, rank) <= 32 MiB, e.g. every
 *              layer of a 3072-wide DiT block at rank 32 (about 14 MB), or
 *              N, K <= 16384 at rank 32; larger shapes return
 *              SVDQ_ERR_INVALID_ARG (use svdq_lowrank_factors)
 *   sharing    all calls on one device use that device's one array, which
 *              keeps the last call's contents: calls that overlap on a device
 *              (several streams or threads) race and must be serialized by
 *              the caller; nothing in it needs clearing between calls
 */
svdq_status svdq_lowrank_factors_noalloc(int64_t N, int64_t K, int32_t rank, const void *W, const void *smooth,
                                         uint64_t seed, void *lora_up, void *lora_down, void *stream);

/*
 * svdq_quantize_weight -- the 4-bit residual of the smoothed weight after the
 * low-rank branch, and its group quantization:
 *   R[n,k] = fl32( W[n,k] smooth[k] - sum_{j=0..rank-1} up[n,j] down[j,k] )
 * (fp64 sum in ascending j, one rounding), then per row and group, from the
 * fp32 values: int4 g64 -- scale RNE_bf16(absmax/7), code RNE(R/scale)
 * clamped to [-8,7]; NVFP4 g16 -- scale E4M3_RNE_sat(absmax/6), code
 * E2M1_RNE_sat(R/scale); fp32 IEEE division, zero scale -> zero codes.
 *   W          bf16 [N, K]; smooth bf16 [K] or NULL (= 1)
 *   lora_up    bf16 [N, rank]; lora_down bf16 [rank, K]; ignored when rank == 0
 *   wgt_codes  out: u8 [N, K/2]; wgt_scales out: int4 bf16 [N, K/64], nvfp4 u8 [N, K/16]
 */
svdq_status svdq_quantize_weight(int32_t precision, int64_t N, int64_t K, int32_t rank, const void *W,
                                 const void *smooth, const void *lora_up, const void *lora_down,
                                 void *wgt_codes, void *wgt_scales, void *stream);

/*
 * svdq_pack_weight_int4 -- offline re-encoding of an int4 weight for the
 * int4 GEMM's fast path (precision SVDQ_INT4_PACKED).  The matrix cores of
 * gfx950 take E4M3 bytes and return fp32; the packed codes turn into exact
 * E4M3 values with two masks and a rotate per 8 codes, so the GEMM spends no
 * integer-to-float conversion per output and group.  The blob holds
 *   - the codes, still 4 bits each ([N, K/2] bytes), in sign-magnitude form
 *     and a fixed bit permutation within each dword (documented in the
 *     source, pack_weight.hip);
 *   - bf16 [N][2][K/64]: per row and group, hi + lo = -8 * scale * (sum of
 *     the group's codes), the weight-only factor of the correction for the
 *     activations' +8 offset in that GEMM.
 *   wgt_codes     u8 [N, K/2] two's complement int4 codes (svdq_gemm_w4a4's)
 *   wgt_scales    bf16 [N, K/64]
 *   packed_weight out: u8 [svdq_packed_weight_bytes(N, K)], device
 *   invalid_codes out (device int32, may be NULL): the number of codes equal
 *                 to -8, which the packed form cannot hold (written as 0);
 *                 the int4 group quantizer never produces them.  Set by
 *                 the call's own kernels (no clearing needed).
 * The weight's scales stay a separate argument of the GEMM.
 */
int64_t svdq_packed_weight_bytes(int64_t N, int64_t K);   /* N*K/2 + 4*N*(K/64); -1 if invalid */
svdq_status svdq_pack_weight_int4(int64_t N, int64_t K, const void *wgt_codes, const void *wgt_scales,
                                  void *packed_weight, int32_t *invalid_codes, void *stream);

/*
 * svdq_pack_weight_fp6 -- offline re-encoding of an int4 weight for the
 * SVDQ_INT4_FP6 GEMM: the codes in the FP6 tiled layout (see the
 * precision enum).
 * gfx950's block-scaled matrix instruction takes E2M3 operands at twice its
 * FP8 rate and returns fp32, and every int4 code is an exact E2M3 value
 * (q/2), so the GEMM feeds both operands to the matrix cores as they are
 * stored.  Every code, -8 included, has an exact form.
 *   wgt_codes   u8 [N, K/2] two's complement int4 codes (svdq_gemm_w4a4's)
 *   fp6_weight  out: u8 [svdq_fp6_codes_bytes(N, K)], device
 * The weight's scales stay a separate argument of the GEMM.
 */
/* bytes of [rows, K] int4 codes in the FP6 tiled layout:
 * ceil(rows/128) * ceil(K/128) * 12288; -1 if rows or K is invalid */
int64_t svdq_fp6_codes_bytes(int64_t rows, int64_t K);
svdq_status svdq_pack_weight_fp6(int64_t N, int64_t K, const void *wgt_codes, void *fp6_weight, void *stream);

/*
 * svdq_debug_group_sums -- test hook on the int4 GEMM's own device code
 * path (operand unpacking and integer matrix-core products): writes the
 * exact integer group sums
 *   G[m,n,g] = sum_{k in group g} qa[m,k] * qw[n,k]      int32 [M, N, K/64]
 * Not needed to run the layer.
 */
svdq_status svdq_debug_group_sums(int64_t M, int64_t N, int64_t K, const void *act_codes,
                                  const void *wgt_codes, int32_t *G, void *stream);

/*
 * svdq_debug_group_sums_packed -- the same integer group sums G [M, N, K/64]
 * from the main loop of the SVDQ_INT4_PACKED GEMM (fp8 matrix-core products
 * of the offset activation codes and the packed weight, minus the offset's
 * share): packed_weight is the blob of svdq_pack_weight_int4.
 */
svdq_status svdq_debug_group_sums_packed(int64_t M, int64_t N, int64_t K, const void *act_codes,
                                         const void *packed_weight, int32_t *G, void *stream);

/*
 * svdq_debug_group_sums_fp6 -- the same integer group sums G [M, N, K/64]
 * from the main loop of the SVDQ_INT4_FP6 GEMM (E2M3 matrix-core products):
 * act_codes in the FP6 tiled layout (svdq_quantize_act with SVDQ_INT4_FP6),
 * fp6_weight from svdq_pack_weight_fp6.
 */
svdq_status svdq_debug_group_sums_fp6(int64_t M, int64_t N, int64_t K, const void *act_codes,
                                      const void *fp6_weight, int32_t *G, void *stream);

/*
 * svdq_debug_gelu_bf16 -- test hook on the GELU of svdq_gelu_quantize_act
 * (the same table and rules): out[i] = GELU(x[i]) for n bf16 values.
 *   x, out     bf16 [n], device, 16-byte aligned; 0 <= n <= 2^36
 * Not needed to run the layer.
 */
svdq_status svdq_debug_gelu_bf16(int64_t n, const void *x, void *out, void *stream);

/*
 * svdq_debug_stream_read -- a measurement hook, not needed to run a layer:
 * reads `bytes` of device memory at `src` in spans of 12288 bytes, one span
 * per wave, with 12 loads of 16 bytes per lane all in flight before any use.
 * pattern 0 reads a span contiguously (1 KB per load instruction), pattern 1
 * in the AWQ GEMV's weight pattern (rows of 1536 bytes, 8 lanes per 128-byte
 * line, 8 rows per load instruction).  out (device, uint32, ceil(bytes /
 * 12288) entries, caller-owned) receives the xor of each span's whole
 * 16-byte chunks (a tail shorter than 16 bytes is not read).  Its time is
 * the ceiling the GEMV's HBM rate is compared with.
 * Errors: SVDQ_ERR_INVALID_ARG for bytes < 0, a pattern other than 0 or 1,
 * a NULL or misaligned src (16 bytes) or out (4 bytes); bytes == 0 is a no-op.
 */
svdq_status svdq_debug_stream_read(const void *src, int64_t bytes, int32_t pattern, uint32_t *out, void *stream);

/* Static, human-readable text for a status code (never NULL). */
const char *svdq_status_string(svdq_status s);

/* Text of the last argument-check failure on the calling thread ("" if none). */
const char *svdq_last_error(void);

/* ABI version of this header: 10 (1 plus svdq_gelu_quantize_act, svdq_debug_gelu_bf16,
 * svdq_gemm_w4a4_qk_norm_rope, svdq_smooth_factors, svdq_quantize_weight,
 * svdq_lowrank_workspace_bytes, svdq_lowrank_factors,
 * svdq_lowrank_factors_noalloc, then SVDQ_INT4_PACKED with
 * svdq_packed_weight_bytes, svdq_pack_weight_int4 and
 * svdq_debug_group_sums_packed, then svdq_debug_stream_read, then
 * SVDQ_INT4_FP6 with svdq_fp6_codes_bytes, svdq_pack_weight_fp6 and
 * svdq_debug_group_sums_fp6, in the FP6 tiled layout). */
int32_t svdq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SVDQ_H */
