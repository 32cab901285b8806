// device_common.h -- small gfx950 device helpers shared by the HIP kernels of
// libsvdq (bf16 / E4M3 bit manipulation, MFMA operand vector types, wave
// reductions).  Internal to the HIP library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

// address-space-qualified pointers for global_load_lds (global -> LDS copies)
typedef __attribute__((address_space(1))) const void *gptr_t;
typedef __attribute__((address_space(3))) void *lptr_t;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest even; NaN -> quiet NaN with the sign kept.
// Overflow rounds to infinity and subnormals round on the same grid as
// normals because bf16 shares binary32's exponent field.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x0040u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Two fp32 -> two bf16 (lo in bits 0..15), round to nearest even, with the
// gfx950 conversion instruction (v_cvt_pk_bf16_f32, one vector instruction
// for both values).  Finite results equal pack_bf16x2's; a NaN input gives a
// quiet NaN of the same sign.
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f{lo, hi}), v2bf));
}

// fp64 -> bf16, round to nearest even, in one step (bf16: 8-bit significand,
// binary32's exponent range, subnormal spacing 2^-133).  NaN -> quiet NaN
// with the sign; overflow -> infinity.
__device__ inline uint32_t f64_to_bf16_rne(double v) {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t sign = (uint32_t)(b >> 48) & 0x8000u;
    const uint64_t m = b & 0x7FFFFFFFFFFFFFFFull;
    if (m > 0x7FF0000000000000ull) return sign | 0x7FC0u;
    const double a = __longlong_as_double((long long)m);
    if (a < 0x1p-126) return sign | (uint32_t)__builtin_rint(a * 0x1p133);   // exact scaling; 128 -> least normal
    const uint64_t r = m + 0x00000FFFFFFFFFFFull + ((m >> 45) & 1u);       // round at bit 45
    const int64_t e = (int64_t)(r >> 52) - 1023 + 127;
    if (e >= 255) return sign | 0x7F80u;
    return sign | ((uint32_t)e << 7) | (uint32_t)((r >> 45) & 0x7Fu);
}

// Largest-magnitude reduction across lanes xor-distance `mask` (wave64).
__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
    return __shfl_xor(v, mask, kWave);
}

// max(v, v of lane l ^ 16) and max(v, v of lane l ^ 32) on the vector ALU:
// v_permlane16_swap exchanges rows 1 and 3 of 16 lanes of its first operand
// with rows 0 and 2 of its second, v_permlane32_swap the upper 32 lanes of
// the first with the lower 32 of the second; with v in both operands every
// lane ends up with its own value in one result and its partner's in the
// other (no LDS round trip, as a cross-lane shuffle would take).
__device__ __forceinline__ float max_xor16(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto s = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto s = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}

// max(m, |a|, |b|) in one v_max3_f32 (the values are finite; fp32 denormals
// are preserved by the kernels' float mode)
__device__ __forceinline__ float max3_abs(float m, float a, float b) {
#if defined(__HIP_DEVICE_COMPILE__)
    float r;
    asm("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(r) : "v"(m), "v"(a), "v"(b));
    return r;
#else
    return fmaxf(m, fmaxf(fabsf(a), fabsf(b)));
#endif
}

// E4M3 ("FN") encode of a non-negative finite fp32, round to nearest even,
// saturating at 448 (the format has no infinity).
__device__ __forceinline__ uint32_t e4m3_encode_nonneg(float v) {
    if (!(v < 448.0f)) return 0x7Eu;                 // also catches +inf
    if (v < 0.015625f) {                              // below 2^-6: spacing 2^-9
        return (uint32_t)__builtin_rintf(v * 512.0f); // exact scaling; 8 -> 0x08
    }
    uint32_t u = __float_as_uint(v);
    uint32_t e = (u >> 23) - 127u + 7u;               // biased E4M3 exponent, >= 1
    uint32_t mant = u & 0x7FFFFFu;
    uint32_t m = mant >> 20;
    uint32_t rem = mant & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (m & 1u))) ++m;
    if (m == 8u) { m = 0u; ++e; }
    uint32_t code = (e << 3) | m;
    return code > 0x7Eu ? 0x7Eu : code;
}

// E4M3 ("FN") decode of a non-NaN code with the sign bit clear.
__device__ __forceinline__ float e4m3_decode_nonneg(uint32_t c) {
    uint32_t f = (c >> 3) & 15u, m = c & 7u;
    if (f == 0u) return (float)m * 0.001953125f;      // m * 2^-9, exact
    return __uint_as_float(((f + 120u) << 23) | (m << 20));
}

// E4M3 ("FN") decode with the sign bit.
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
    const float v = e4m3_decode_nonneg(c & 0x7Fu);
    return (c & 0x80u) ? -v : v;
}

// FP6 tiled layout of int4 codes (the FP6 GEMM's operands): byte offset of
// 16-byte chunk c (0..2: [h0 dwords 0-3 | h1 dwords 0-3 | h0 dwords 4-5,
// h1 dwords 4-5], the halves of chunk 2 swapped when fp6_half_swap(row)) of
// group g of row r.  Rows form tiles of 128, groups pairs; (tile, pair) is
// a contiguous 12 KB block of 128 rows x 96 bytes, the GEMM's LDS stage
// image, and a row's six chunks sit rotated by fp6_rot(row) positions.  With
// 64 LDS banks of 4 bytes, one LDS cycle serves 16 lanes' 16-byte fragments
// (16 consecutive rows, 96 bytes apart) or 32 lanes' 8-byte pieces; the
// rotation puts those 16 rows on distinct banks (rows r and r + 8 would
// share them with a rotation by bit 2 alone), and the swap does the same for
// the 8-byte pieces of 32 rows.  NP = pairs per row (ceil(K/128)).
constexpr int FP6_TILE_ROWS = 128;
constexpr int FP6_PAIR_BYTES = FP6_TILE_ROWS * 96;      // 12 KB
__host__ __device__ __forceinline__ int fp6_rot(int row) { return ((row >> 2) ^ (row >> 3)) & 1; }
__host__ __device__ __forceinline__ int fp6_half_swap(int row) { return ((row >> 3) ^ (row >> 4)) & 1; }
__host__ __device__ __forceinline__ size_t fp6_tiled_chunk(int row, int g, int c, int NP) {
    const int t = row >> 7, rho = row & 127, s = g >> 1;
    const int slot = (3 * (g & 1) + c + fp6_rot(rho)) % 6;
    return ((size_t)t * NP + s) * FP6_PAIR_BYTES + (size_t)rho * 96 + 16 * slot;
}
__host__ __device__ __forceinline__ size_t fp6_tiled_bytes(int rows, int K) {
    return (size_t)((rows + FP6_TILE_ROWS - 1) / FP6_TILE_ROWS) * (size_t)((K / 64 + 1) / 2) * FP6_PAIR_BYTES;
}

}  // namespace svdq
