// gemv_w4a16_awq.hip -- AWQ-style int4 weight-only layer with bf16
// activations on gfx950 ("Nunchaku Lite" docs, "Supported quantization
// types": awq_w4a16 int4 group 64, used for memory-bound, precision-
// sensitive layers such as the adaptive-norm modulation projections):
//   y[m,n] = sum_k x[m,k] * (q[n,k] - z[g,n]) * s[g,n] + bias[n].
//
// The kernel is an HBM stream of the packed weights.  A block owns 16
// weight rows and its 4 waves split K into quarters; each wave keeps four
// groups of loads in flight (codes, scales, zero points and x for the next
// groups while it computes the current one), and the quarter sums are added
// in LDS at the end.  Scales and zero points are stored group-major
// ([K/64, N]), so the four consecutive rows a lane accumulates share one
// 8-byte load.
//
// Arithmetic on the matrix cores, with the weights as the A operand of
// v_mfma_f32_16x16x32_bf16 (16 weight rows) and x as B (16 activation
// columns, zero beyond M):
//  * a code q in 0..15 becomes the bf16 value 128 + q by OR-ing it into the
//    bit pattern 0x4300 (bf16 128 has a unit mantissa step), so unpacking is
//    one and-or per pair of codes;
//  * sum_{k in g} (q - z) x = sum (128 + q) x - (128 + z) sum x, and sum x
//    comes from a second MFMA against an all-ones operand;
//  * the group scale multiplies the group's partial sum in fp32.
// Codes are paired (p, p+4) inside a dword; x is permuted to the same k
// order (a dot product only needs A and B in the same order).
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace svdq {

constexpr int AW_ROWS = 16, AW_WAVES = 4, AW_MT = 4, AW_DEPTH = 4;

template <int MT, bool VEC_SZ>
__global__ __launch_bounds__(AW_WAVES * 64)
void awq_gemv_kernel(int M, int N, int K, const uint16_t *__restrict__ x,
                     const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
                     const uint16_t *__restrict__ zeros, const uint16_t *__restrict__ bias,
                     uint16_t *__restrict__ out)
{
    __shared__ float s_part[AW_WAVES][MT][AW_ROWS * 16];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c16 = lane & 15;          // A: weight row within the tile; B/C: activation column
    const int kq = lane >> 4;           // 16-element slice of the group
    const int nbn = (N + AW_ROWS - 1) / AW_ROWS;
    const int n0 = (int)(blockIdx.x % nbn) * AW_ROWS;
    const int mbase = (int)(blockIdx.x / nbn) * (16 * AW_MT);
    const int NG = K >> 6;
    const int g_begin = (NG * wave) / AW_WAVES, g_end = (NG * (wave + 1)) / AW_WAVES;
    const int ng = g_end - g_begin;

    // Rows past N and columns past M read clamped, valid data: they only feed
    // outputs that are never stored.
    const uint8_t *cp = codes + (size_t)min(n0 + c16, N - 1) * (size_t)(K >> 1) + 8 * kq;
    const uint16_t *xp[MT];
    bool xok[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const int m = mbase + t * 16 + c16;
        xok[t] = m < M;
        xp[t] = x + (size_t)min(m, M - 1) * (size_t)K + 16 * kq;
    }
    // C rows (weight rows) held by this lane: n0 + 4*kq + i, i = 0..3
    const int nq = n0 + 4 * kq;
    int nrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) nrow[i] = min(nq + i, N - 1);
    const int nq_vec = min(nq, N - 4);   // 8-byte loads: stays inside the group row (N >= 4)

    const v8bf ones = __builtin_bit_cast(v8bf, v4u{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
    v4f yacc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) yacc[t] = v4f{0.f, 0.f, 0.f, 0.f};

    // load ring, AW_DEPTH groups deep; slot indices are compile-time constants
    v2u rw[AW_DEPTH], rs[AW_DEPTH], rz[AW_DEPTH];
    v4u rx[AW_DEPTH][MT][2];
    auto load = [&](int g, auto slot_c) __attribute__((always_inline)) {
        constexpr int S = decltype(slot_c)::value;
        rw[S] = *(const v2u *)(cp + (size_t)g * 32);
        if constexpr (VEC_SZ) {
            rs[S] = *(const v2u *)(scales + (size_t)g * N + nq_vec);
            rz[S] = *(const v2u *)(zeros + (size_t)g * N + nq_vec);
        } else {
            const uint16_t *sg = scales + (size_t)g * N, *zg = zeros + (size_t)g * N;
            rs[S] = v2u{(uint32_t)sg[nrow[0]] | ((uint32_t)sg[nrow[1]] << 16),
                        (uint32_t)sg[nrow[2]] | ((uint32_t)sg[nrow[3]] << 16)};
            rz[S] = v2u{(uint32_t)zg[nrow[0]] | ((uint32_t)zg[nrow[1]] << 16),
                        (uint32_t)zg[nrow[2]] | ((uint32_t)zg[nrow[3]] << 16)};
        }
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int s = 0; s < 2; ++s) rx[S][t][s] = *(const v4u *)(xp[t] + (size_t)g * 64 + 8 * s);
        // Keep the loads here, between the computations of the ring slots: the
        // compiler would otherwise sink them to their use or batch them.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    auto compute = [&](auto slot_c) __attribute__((always_inline)) {
        constexpr int S = decltype(slot_c)::value;
        __builtin_amdgcn_sched_barrier(0);
        v4u a[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const uint32_t d = rw[S][s];
#pragma unroll
            for (int j = 0; j < 4; ++j) a[s][j] = ((d >> (4 * j)) & 0x000F000Fu) | 0x43004300u;
        }
        float sc[4], zc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t sw = rs[S][i >> 1], zw = rz[S][i >> 1];
            sc[i] = (i & 1) ? bf16_hi(sw) : bf16_lo(sw);
            zc[i] = 128.0f + ((i & 1) ? bf16_hi(zw) : bf16_lo(zw));
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            v4u xv[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                v4u raw = rx[S][t][s];
                if (!xok[t]) raw = v4u{0u, 0u, 0u, 0u};
                xv[s][0] = __builtin_amdgcn_perm(raw[2], raw[0], 0x05040100u);
                xv[s][1] = __builtin_amdgcn_perm(raw[2], raw[0], 0x07060302u);
                xv[s][2] = __builtin_amdgcn_perm(raw[3], raw[1], 0x05040100u);
                xv[s][3] = __builtin_amdgcn_perm(raw[3], raw[1], 0x07060302u);
            }
            v4f q = v4f{0.f, 0.f, 0.f, 0.f}, xs = q;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const v8bf b = __builtin_bit_cast(v8bf, xv[s]);
                q = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a[s]), b, q, 0, 0, 0);
                xs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, b, xs, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                yacc[t][i] = __builtin_fmaf(sc[i], __builtin_fmaf(-zc[i], xs[i], q[i]), yacc[t][i]);
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;

    // Loads are unconditional (the group index is clamped to the wave's last
    // group; surplus loads read valid memory and are never used) so that the
    // compiler can count the loads in flight exactly and wait only for the
    // group about to be used.
    if (ng > 0) {
        const int g_last = g_end - 1;
        load(min(g_begin + 0, g_last), I0{});
        load(min(g_begin + 1, g_last), I1{});
        load(min(g_begin + 2, g_last), I2{});
        load(min(g_begin + 3, g_last), I3{});
        const int nfull = ng & ~(AW_DEPTH - 1);
        for (int i = 0; i < nfull; i += AW_DEPTH) {
            const int g = g_begin + i;
            compute(I0{});
            load(min(g + 4, g_last), I0{});
            compute(I1{});
            load(min(g + 5, g_last), I1{});
            compute(I2{});
            load(min(g + 6, g_last), I2{});
            compute(I3{});
            load(min(g + 7, g_last), I3{});
        }
        const int rem = ng - nfull;     // groups nfull.. sit in slots 0.. already
        if (rem > 0) compute(I0{});
        if (rem > 1) compute(I1{});
        if (rem > 2) compute(I2{});
    }

#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_part[wave][t][(4 * kq + i) * 16 + c16] = yacc[t][i];
    __syncthreads();
    for (int idx = threadIdx.x; idx < MT * AW_ROWS * 16; idx += blockDim.x) {
        const int t = idx / (AW_ROWS * 16), e = idx % (AW_ROWS * 16);
        const int nr = e >> 4, mc = e & 15;
        const int n = n0 + nr, m = mbase + t * 16 + mc;
        if (n < N && m < M) {
            float s = 0.0f;
#pragma unroll
            for (int w = 0; w < AW_WAVES; ++w) s += s_part[w][t][e];
            if (bias) s += bf16_to_f32(bias[n]);
            out[(size_t)m * N + n] = (uint16_t)f32_to_bf16_rne(s);
        }
    }
}

template <bool V>
static void launch_mt(int mt, dim3 grid, dim3 block, hipStream_t stream, int M, int N, int K,
                      const uint16_t *xp, const uint8_t *cp, const uint16_t *sp, const uint16_t *zp,
                      const uint16_t *bp, uint16_t *op)
{
    switch (mt) {
        case 1: hipLaunchKernelGGL((awq_gemv_kernel<1, V>), grid, block, 0, stream, M, N, K, xp, cp, sp, zp, bp, op); break;
        case 2: hipLaunchKernelGGL((awq_gemv_kernel<2, V>), grid, block, 0, stream, M, N, K, xp, cp, sp, zp, bp, op); break;
        case 3: hipLaunchKernelGGL((awq_gemv_kernel<3, V>), grid, block, 0, stream, M, N, K, xp, cp, sp, zp, bp, op); break;
        default: hipLaunchKernelGGL((awq_gemv_kernel<4, V>), grid, block, 0, stream, M, N, K, xp, cp, sp, zp, bp, op); break;
    }
}

hipError_t launch_awq_gemv(int M, int N, int K, const void *x, const void *codes,
                           const void *scales, const void *zeros, const void *bias, void *out,
                           hipStream_t stream)
{
    const int col_tiles = (M + 15) / 16;
    const int mt = col_tiles >= AW_MT ? AW_MT : col_tiles;
    dim3 grid(((N + AW_ROWS - 1) / AW_ROWS) * ((M + 16 * AW_MT - 1) / (16 * AW_MT))), block(AW_WAVES * 64);
    const uint16_t *xp = (const uint16_t *)x, *sp = (const uint16_t *)scales,
                   *zp = (const uint16_t *)zeros, *bp = (const uint16_t *)bias;
    const uint8_t *cp = (const uint8_t *)codes;
    uint16_t *op = (uint16_t *)out;
    // 8-byte scale/zero loads need every group row of N entries to keep 4 consecutive rows 8-byte aligned
    if (N % 4 == 0)
        launch_mt<true>(mt, grid, block, stream, M, N, K, xp, cp, sp, zp, bp, op);
    else
        launch_mt<false>(mt, grid, block, stream, M, N, K, xp, cp, sp, zp, bp, op);
    return hipGetLastError();
}

}  // namespace svdq
