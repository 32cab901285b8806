// gelu_table.h -- the GELU (tanh form) table of the bf16 GELU step
// (gelu_bf16.h), as compile-time data: plain C++20, no HIP, so the same
// header also builds the table on the host for its CPU test.
//
// Slot i: sign i / GELU_STRIDE; slot GELU_SPAN of each sign is the sentinel
// (0x7FFF), the others hold the result for the bf16 magnitude bits
// (GELU_E_LO << 7) + i % GELU_STRIDE, i.e. |y| in [2^-14, 128):
//   gelu(y) = y / (1 + exp(-2u)),  u = sqrt(2/pi) (y + 0.044715 y^3),
// the tanh form without the cancellation in 1 + tanh u, evaluated in fp64
// and rounded once to bf16 (nearest, ties to even).  No exact result lies
// within 2^-13 of a bf16 spacing of a rounding midpoint (the oracle's margin
// check), so any fp64 evaluation with a relative error far below 2^-21
// rounds to the correctly rounded result; the exp below errs by about
// 1e-15.  From |y| = 32 on, exp(-2u) is below 2^-700 or above 2^700 and the
// entries are exactly y (y > 0) and -0 (y < 0).
#pragma once

#include <array>
#include <bit>
#include <cstdint>

namespace svdq {

constexpr int GELU_E_LO = 113;                                // 2^-14
constexpr int GELU_E_HI = 133;                                // [64, 128)
constexpr int GELU_SPAN = (GELU_E_HI - GELU_E_LO + 1) * 128;  // results per sign
constexpr int GELU_STRIDE = GELU_SPAN + 1;                    // plus the sentinel slot
constexpr int GELU_TAB = 2 * GELU_STRIDE;                     // 5378 entries, 10.5 KB
constexpr int GELU_TAB_PAD = (GELU_TAB + 7) / 8 * 8;          // whole 16-byte pieces (zeros after)
constexpr uint32_t GELU_SENTINEL = 0x7FFFu;

namespace gelu_detail {

// 2^k for -1022 <= k <= 1023, from the exponent field
constexpr double pow2(int k) { return std::bit_cast<double>((uint64_t)(k + 1023) << 52); }

// exp(x) for |x| <= 700 (the caller saturates beyond): x = k ln2 + r with
// |r| <= ln2/2, ln2 split as a 32-bit head (k * head is exact for |k| < 2^20)
// and a tail that carries the head's error and the double's own; exp(r) by
// its power series (30 terms: the remainder is below 1e-30).
constexpr double exp_small(double x) {
    constexpr double ln2 = 0.6931471805599453;                  // ln 2 rounded to double
    constexpr double ln2_err = 2.3190468138462996e-17;          // ln 2 - ln2 (from ln 2's expansion)
    constexpr double head = std::bit_cast<double>(std::bit_cast<uint64_t>(ln2) & ~((uint64_t(1) << 21) - 1));
    constexpr double tail = (ln2 - head) + ln2_err;
    const double kd = x / ln2;
    const int k = (int)(kd >= 0.0 ? kd + 0.5 : kd - 0.5);
    const double r = (x - k * head) - k * tail;
    double term = 1.0, sum = 1.0;
    for (int n = 1; n <= 30; ++n) {
        term *= r / n;
        sum += term;
    }
    return sum * pow2(k);
}

// fp64 -> bf16 bits, round to nearest even (finite values and zeros)
constexpr uint16_t f64_to_bf16(double v) {
    const uint64_t b = std::bit_cast<uint64_t>(v);
    const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
    const double a = v < 0.0 ? -v : v;
    if (a < 0x1p-126) {                                          // bf16 subnormals: spacing 2^-133
        const double s = a * 0x1p133;                            // exact
        double fl = (double)(uint64_t)s;
        const double fr = s - fl;
        if (fr > 0.5 || (fr == 0.5 && ((uint64_t)fl & 1u))) fl += 1.0;
        return (uint16_t)(sign | (uint16_t)(uint64_t)fl);       // 128 -> the least normal
    }
    const uint64_t m = b & 0x7FFFFFFFFFFFFFFFull;
    const uint64_t r = m + 0x00000FFFFFFFFFFFull + ((m >> 45) & 1u);   // round at bit 45
    const int64_t e = (int64_t)(r >> 52) - 1023 + 127;
    if (e >= 255) return (uint16_t)(sign | 0x7F80u);
    return (uint16_t)(sign | ((uint32_t)e << 7) | (uint32_t)((r >> 45) & 0x7Fu));
}

}  // namespace gelu_detail

constexpr uint16_t gelu_table_entry(int i) {
    const int j = i % GELU_STRIDE;
    if (j == GELU_SPAN) return (uint16_t)GELU_SENTINEL;
    const bool neg = i >= GELU_STRIDE;
    const uint32_t mag = (uint32_t)(GELU_E_LO << 7) + (uint32_t)j;
    const double a = (double)std::bit_cast<float>(mag << 16);
    const double y = neg ? -a : a;
    const double u = 0.79788456080286535588 * (y + 0.044715 * y * y * y);   // sqrt(2/pi)
    const double x = -2.0 * u;
    double v;
    if (x < -700.0) v = y;                          // 1 + exp(x) == 1 in fp64
    else if (x > 700.0) v = neg ? -0.0 : 0.0;       // y / (1 + exp(x)): far below half the least bf16
    else v = y / (1.0 + gelu_detail::exp_small(x));
    return gelu_detail::f64_to_bf16(v);
}

constexpr std::array<uint16_t, GELU_TAB_PAD> make_gelu_table() {
    std::array<uint16_t, GELU_TAB_PAD> t{};
    for (int i = 0; i < GELU_TAB; ++i) t[i] = gelu_table_entry(i);
    return t;
}

}  // namespace svdq
