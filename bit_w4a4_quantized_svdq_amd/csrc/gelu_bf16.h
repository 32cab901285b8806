// gelu_bf16.h -- GELU (tanh form) of bf16 values, rounded once to bf16, for
// the activation step of a layer fed by a GELU MLP's up projection ("Nunchaku
// Lite" docs, section "Fused kernels": the original engine runs the MLP's
// GELU fused into its kernels).
//
//   gelu(y) = y/2 * (1 + tanh( sqrt(2/pi) * (y + 0.044715 y^3) ))
//
// A bf16 input has 65536 possible values, so the rounded result is made
// exact by construction rather than by a careful fp32 evaluation:
//  * |y| in [2^-14, 32): a table of 2 x 19 x 128 results in LDS, computed by
//    each block in fp64 as y / (1 + exp(-2u)) -- the same function, free of
//    the cancellation in 1 + tanh u.  Over the whole input range no exact
//    result comes within 2^-13 of a bf16 spacing of a rounding midpoint,
//    while the fp64 error stays below 2^-36 spacings, so the fp64 value
//    rounds to the correctly rounded result.
//  * |y| >= 32: y for y > 0 (the correction is below 1e-400 relative) and -0
//    for y < 0 (|gelu(y)| far under half the least subnormal); +inf -> +inf,
//    -inf -> -0 (the limit), NaN -> the quiet NaN 0x7FC0 with the sign.
//  * |y| < 2^-14: gelu(y) = y/2 + y tanh(u)/2, and the second term is
//    positive and below 2^-14 of the first, under half a spacing: the result
//    is y/2 -- exact (an exponent decrement) while y/2 is normal, and for the
//    two lowest binades a half-spacing value rounded toward +infinity.
//
// Fast path: two values per dword, their table slots formed with packed
// 16-bit integer operations.  Inputs outside the table's range land on a
// sentinel slot (0x7FFF: bits 14 and 13 both set, which no result below 32
// in magnitude has); when any lane of the wave meets one, the whole group is
// redone with the exact rules (a wave-uniform branch).
#pragma once

#include <stdint.h>

#include "device_common.h"

namespace svdq {

constexpr int GELU_E_LO = 113;                                // 2^-14
constexpr int GELU_E_HI = 131;                                // [16, 32)
constexpr int GELU_SPAN = (GELU_E_HI - GELU_E_LO + 1) * 128;  // results per sign
constexpr int GELU_STRIDE = GELU_SPAN + 1;                    // plus the sentinel slot
constexpr int GELU_TAB = 2 * GELU_STRIDE;                     // 4866 entries, 9.5 KB
constexpr uint32_t GELU_SENTINEL = 0x7FFFu;

// Table slot i: sign i / GELU_STRIDE; slot GELU_SPAN of each sign is the
// sentinel, the others hold magnitude bits (GELU_E_LO << 7) + i % GELU_STRIDE.
__device__ inline uint16_t gelu_table_entry(int i)
{
    const int j = i % GELU_STRIDE;
    if (j == GELU_SPAN) return (uint16_t)GELU_SENTINEL;
    const uint32_t neg = i >= GELU_STRIDE ? 0x8000u : 0u;
    const uint32_t mag = (uint32_t)(GELU_E_LO << 7) + (uint32_t)j;
    const double y = (double)__uint_as_float((neg | mag) << 16);
    const double u = 0.79788456080286535588 * (y + 0.044715 * y * y * y);   // sqrt(2/pi)
    const double v = y / (1.0 + exp(-2.0 * u));
    return (uint16_t)f64_to_bf16_rne(v);   // the sign comes from the bits: v may be -0
}

// Fill a block's table (tid, nthreads: the block's threads); the caller's
// next barrier publishes it.
__device__ inline void gelu_table_fill(uint16_t *tab, int tid, int nthreads)
{
    for (int i = tid; i < GELU_TAB; i += nthreads) tab[i] = gelu_table_entry(i);
}

// GELU of one bf16 by the exact rules (bits in the low half of h, high half 0).
__device__ inline uint32_t gelu_bf16_exact(uint32_t h, const uint16_t *tab)
{
    const uint32_t mag = h & 0x7FFFu, neg = h & 0x8000u;
    const uint32_t ti = mag - (uint32_t)(GELU_E_LO << 7);
    if (ti < (uint32_t)GELU_SPAN) return tab[ti + (neg ? (uint32_t)GELU_STRIDE : 0u)];
    if (mag < (uint32_t)(GELU_E_LO << 7))
        return (mag >> 7) >= 2 ? h - 0x80u : (neg | ((mag + (neg ? 0u : 1u)) >> 1));
    return mag > 0x7F80u ? (neg | 0x7FC0u) : (neg ? 0x8000u : h);
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Table lookups of two packed bf16 (sentinels for inputs outside the range).
__device__ __forceinline__ uint32_t gelu_lookup2(uint32_t w, const uint16_t *tab)
{
    const u16x2 m = __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu);
    u16x2 ti = m - (u16x2)(unsigned short)(GELU_E_LO << 7);                  // wraps below the range
    ti = __builtin_elementwise_min(ti, (u16x2)(unsigned short)GELU_SPAN);    // the sentinel slot
    const u16x2 s = __builtin_bit_cast(u16x2, w) >> (unsigned short)15;
    const u16x2 idx = s * (u16x2)(unsigned short)GELU_STRIDE + ti;
    const uint32_t id = __builtin_bit_cast(uint32_t, idx);
    return (uint32_t)tab[id & 0xFFFFu] | ((uint32_t)tab[id >> 16] << 16);
}

// GELU of 16 packed bf16 in place (the quantize kernel's slice of a group).
__device__ __forceinline__ void gelu_bf16x16(v4u (&x)[2], const uint16_t *tab)
{
    v4u r[2];
    uint32_t flag = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t v = gelu_lookup2(x[j][p], tab);
            r[j][p] = v;
            flag |= v & (v << 1);   // bits 14 and 13 of a half both set: a sentinel
        }
    if (__builtin_expect(__any((flag & 0x40004000u) != 0u), 0)) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t w = x[j][p];
                r[j][p] = gelu_bf16_exact(w & 0xFFFFu, tab) | (gelu_bf16_exact(w >> 16, tab) << 16);
            }
    }
    x[0] = r[0];
    x[1] = r[1];
}

}  // namespace svdq
