// gelu_bf16.h -- GELU (tanh form) of bf16 values, rounded once to bf16, for
// the activation step of a layer fed by a GELU MLP's up projection ("Nunchaku
// Lite" docs, section "Fused kernels": the original engine runs the MLP's
// GELU fused into its kernels).
//
//   gelu(y) = y/2 * (1 + tanh( sqrt(2/pi) * (y + 0.044715 y^3) ))
//
// A bf16 input has 65536 possible values, so the rounded result is made
// exact by construction rather than by a careful fp32 evaluation:
//  * |y| in [2^-14, 128): a table of 2 x 21 x 128 results (gelu_table.h:
//    built at compile time, copied into LDS by each block), computed in fp64
//    as y / (1 + exp(-2u)) -- the same function, free of the
//    cancellation in 1 + tanh u.  Over the whole input range no exact
//    result comes within 2^-13 of a bf16 spacing of a rounding midpoint,
//    while the fp64 error stays below 2^-36 spacings, so the fp64 value
//    rounds to the correctly rounded result (from 32 on, exp(-2u) is 0 or
//    infinity in fp64 and the entries are exactly y and -0, as below).
//  * |y| >= 32: y for y > 0 (the correction is below 1e-400 relative) and -0
//    for y < 0 (|gelu(y)| far under half the least subnormal); +inf -> +inf,
//    -inf -> -0 (the limit), NaN -> the quiet NaN 0x7FC0 with the sign.
//    The table covers this rule up to 128, the range a GELU MLP's
//    pre-activations reach, so the selects below are rarely needed.
//  * |y| < 2^-14: gelu(y) = y/2 + y tanh(u)/2, and the second term is
//    positive and below 2^-14 of the first, under half a spacing: the result
//    is y/2 -- exact (an exponent decrement) while y/2 is normal, and for the
//    two lowest binades a half-spacing value rounded toward +infinity.
//
// Fast path: two values per dword, their table slots formed with packed
// 16-bit integer operations.  Inputs outside the table's range land on a
// sentinel slot (0x7FFF) and raise a tracked slot maximum (one packed max per
// pair); when any lane of the wave has an input of 128 or more in magnitude,
// the pairs get the |y| >= 32 rule by selects, and when any has a NaN or an
// input below 2^-14, the whole group is redone with the exact rules
// (wave-uniform branches).
#pragma once

#include <stdint.h>

#include "device_common.h"
#include "gelu_table.h"

namespace svdq {

// The table (gelu_table.h) as constant device data, built by the compiler;
// each translation unit that includes this header holds its own copy.
static __device__ const std::array<uint16_t, GELU_TAB_PAD> g_gelu_table __attribute__((aligned(16))) =
    make_gelu_table();

// Copy the table into a block's LDS (16-byte aligned, GELU_TAB_PAD entries;
// tid, nthreads: the block's threads, 16 bytes per thread and step); the
// caller's next barrier publishes it.
__device__ inline void gelu_table_fill(uint16_t *tab, int tid, int nthreads)
{
    const v4u *src = (const v4u *)g_gelu_table.data();
    for (int i = tid; i < GELU_TAB_PAD / 8; i += nthreads) ((v4u *)tab)[i] = src[i];
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

// Table lookups of two packed bf16 (the sentinel for inputs outside the
// range), keeping in tmax the largest unclamped slot index seen (one packed
// max): a half of tmax at or above GELU_SPAN means an input outside the
// table's range.
__device__ __forceinline__ uint32_t gelu_lookup2_track(uint32_t w, const uint16_t *tab, u16x2 &tmax)
{
    const u16x2 m = __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu);
    u16x2 ti = m - (u16x2)(unsigned short)(GELU_E_LO << 7);
    tmax = __builtin_elementwise_max(tmax, ti);
    ti = __builtin_elementwise_min(ti, (u16x2)(unsigned short)GELU_SPAN);
    const u16x2 s = __builtin_bit_cast(u16x2, w) >> (unsigned short)15;
    const u16x2 idx = s * (u16x2)(unsigned short)GELU_STRIDE + ti;
    const uint32_t id = __builtin_bit_cast(uint32_t, idx);
    return (uint32_t)tab[id & 0xFFFFu] | ((uint32_t)tab[id >> 16] << 16);
}

// Unclamped slot index of +-infinity: inputs whose index lies in
// [GELU_SPAN, GELU_TI_INF] are 128 <= |y| <= infinity; above it lie NaNs and,
// wrapped around, the inputs below 2^-14.
constexpr uint32_t GELU_TI_INF = 0x7F80u - (uint32_t)(GELU_E_LO << 7);

// The exact rule for |y| >= 32 applied to a looked-up pair: y for y >= 32
// (+infinity included), -0 for y <= -32; other halves keep the table's
// result.  Valid when no input of the pair is a NaN or below 2^-14.
__device__ __forceinline__ uint32_t gelu_fix_big2(uint32_t g, uint32_t w)
{
    const float y0 = bf16_lo(w), y1 = bf16_hi(w);
    uint32_t lo = g & 0xFFFFu, hi = g >> 16;
    lo = y0 >= 32.0f ? (w & 0xFFFFu) : (y0 <= -32.0f ? 0x8000u : lo);
    hi = y1 >= 32.0f ? (w >> 16) : (y1 <= -32.0f ? 0x8000u : hi);
    return lo | (hi << 16);
}

// GELU of n packed pairs in place after gelu_lookup2_track (g: looked-up
// results, w: inputs, tmax: the tracked slot maximum; every lane of the wave
// takes part, the branches are wave-uniform): inputs of 128 and above in
// magnitude take gelu_fix_big2, a NaN or an input below 2^-14 anywhere in
// the wave sends all n pairs through the exact rules.
template <int n>
__device__ __forceinline__ void gelu_resolve(uint32_t (&g)[n], const uint32_t (&w)[n], u16x2 tmax,
                                             const uint16_t *tab)
{
    const uint32_t tm = tmax[0] > tmax[1] ? tmax[0] : tmax[1];
    if (__builtin_expect(__any(tm > GELU_TI_INF), 0)) {
#pragma unroll
        for (int p = 0; p < n; ++p)
            g[p] = gelu_bf16_exact(w[p] & 0xFFFFu, tab) | (gelu_bf16_exact(w[p] >> 16, tab) << 16);
    } else if (__any(tm >= (uint32_t)GELU_SPAN)) {
#pragma unroll
        for (int p = 0; p < n; ++p) g[p] = gelu_fix_big2(g[p], w[p]);
    }
}

// GELU of 16 packed bf16 in place (the quantize kernel's slice of a group).
__device__ __forceinline__ void gelu_bf16x16(v4u (&x)[2], const uint16_t *tab)
{
    uint32_t w[8], r[8];
    u16x2 tmax = (u16x2)(unsigned short)0;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            w[4 * j + p] = x[j][p];
            r[4 * j + p] = gelu_lookup2_track(x[j][p], tab, tmax);
        }
    gelu_resolve(r, w, tmax, tab);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int p = 0; p < 4; ++p) x[j][p] = r[4 * j + p];
}

}  // namespace svdq
