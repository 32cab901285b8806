// pack_weight.hip -- offline re-encoding of an int4 SVDQuant weight (codes
// two's complement, group 64, bf16 scales; "Nunchaku Lite" docs, "Supported
// quantization types") for the int4 GEMM's fp8 formulation.  The codes keep
// 4 bits each (same [N, K/2] bytes); they are written in sign-magnitude form
// in a bit layout that turns into E4M3 bytes with two masks and a rotate.
// Per weight row and group, the code sum Sw gives the correction plane
// -8 sw Sw (the share of the activations' +8 offset) as two bf16 values.
//
// Blob layout (row-major, all offsets multiples of 16 bytes):
//   bytes [0, N*K/2):  packed codes, row n at n*K/2, group g at 32g within it;
//       in the group, byte 4*(4h + i) + e of dword (h, i) (h = K-half, i =
//       0..3, e = 0..3) holds, with k = 64g + 32h + 8i + 2e:
//         bits 0-2  |q[k]|          bit 7  sign of q[k]
//         bits 4-6  |q[k+1]|        and bit 3 of byte (e+1) mod 4 of the
//                                   same dword holds the sign of q[k+1];
//   then bf16 [N][2][K/64]: for row n, the hi plane [K/64] followed by the lo
//       plane [K/64], hi + lo = -8 * sw[n,g] * sum_{k in g} q[n,k] (the
//       product is exact in fp32; hi = RNE_bf16 of it, lo = RNE_bf16 of the
//       remainder).
// A code -8 has no sign-magnitude 4-bit form; it is written as -0 and counted.
// The FP6 layout at the end of the file holds every code, -8 included.
#include "device_common.h"
#include "launch.h"

namespace svdq {

size_t packed_weight_bytes(int N, int K) { return (size_t)N * (K / 2) + (size_t)N * 2 * (K / 64) * 2; }

__device__ __forceinline__ int sext4(uint32_t v) { return (int)(v << 28) >> 28; }

__global__ void pack_zero_kernel(int32_t *invalid) { *invalid = 0; }

// one thread per (weight row, group of 64 codes)
__global__ __launch_bounds__(256) void pack_int4_kernel(int N, int NG, const uint8_t *__restrict__ codes,
                                                        const uint16_t *__restrict__ scales,
                                                        uint8_t *__restrict__ blob, int32_t *__restrict__ invalid)
{
    const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
    if (t >= (long long)N * NG) return;
    const int n = (int)(t / NG), g = (int)(t % NG);
    const size_t off = (size_t)n * NG * 32 + (size_t)g * 32;
    const v4u d0 = *(const v4u *)(codes + off), d1 = *(const v4u *)(codes + off + 16);
    const uint32_t in[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
    uint32_t pk[8];
    int sum = 0, bad = 0;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        uint32_t p = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int qe = sext4(in[w] >> (8 * e)), qo = sext4(in[w] >> (8 * e + 4));
            bad += (qe == -8) + (qo == -8);
            sum += qe + qo;
            p |= ((uint32_t)(qe < 0 ? -qe : qe) & 7u) << (8 * e) | (uint32_t)(qe < 0) << (8 * e + 7);
            p |= ((uint32_t)(qo < 0 ? -qo : qo) & 7u) << (8 * e + 4) | (uint32_t)(qo < 0) << (8 * ((e + 1) & 3) + 3);
        }
        pk[w] = p;
    }
    *(v4u *)(blob + off) = v4u{pk[0], pk[1], pk[2], pk[3]};
    *(v4u *)(blob + off + 16) = v4u{pk[4], pk[5], pk[6], pk[7]};
    uint16_t *corr = (uint16_t *)(blob + (size_t)N * NG * 32) + (size_t)n * 2 * NG;
    const float c = -8.0f * (float)sum * bf16_to_f32(scales[(size_t)n * NG + g]);   // exact: 12 x 8 bits
    const uint32_t hi = f32_to_bf16_rne(c);
    const uint32_t lo = f32_to_bf16_rne(c - bf16_to_f32((uint16_t)hi));            // remainder exact
    corr[g] = (uint16_t)hi;
    corr[NG + g] = (uint16_t)lo;
    if (bad && invalid) atomicAdd(invalid, bad);
}

// ---------------------------------------------------------------------------
// FP6 tiled layout of int4 codes (the FP6 GEMM's weight operand, the same
// layout as the FP6 output of the activation step; fp6_tiled_chunk): per row
// n and group g two 192-bit strings, one per K-half h, field j (bits 6j ..
// 6j+5) = E2M3 code of q[n, 64g + 32h + j] / 2, as three 16-byte chunks
// [h0 dwords 0-3 | h1 dwords 0-3 | h0 dwords 4-5, h1 dwords 4-5] (the last
// chunk's halves swapped when fp6_half_swap(n)) placed by row tile, group
// pair and rotation.  Every code in [-8, 7] has an exact
// form: |q|/2 = 0, 0.5 (E2M3 subnormal 4/8), then 1 .. 4 in steps of 0.5
// (normal, three mantissa bits).
size_t fp6_weight_bytes(int N, int K) { return fp6_tiled_bytes(N, K); }

// E2M3 bits of |q| / 2 for |q| = 0 .. 8 (sign: bit 5)
__constant__ uint8_t kE2M3Half[9] = {0, 4, 8, 12, 16, 18, 20, 22, 24};

// one thread per (weight row, group of 64 codes)
__global__ __launch_bounds__(256) void pack_fp6_kernel(int N, int NG, const uint8_t *__restrict__ codes,
                                                       uint8_t *__restrict__ blob)
{
    const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
    if (t >= (long long)N * NG) return;
    const int n = (int)(t / NG), g = (int)(t % NG);
    const size_t off = (size_t)n * NG * 32 + (size_t)g * 32;
    const v4u d0 = *(const v4u *)(codes + off), d1 = *(const v4u *)(codes + off + 16);
    const uint32_t in[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
    uint32_t dw[2][6];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        uint64_t bits[3] = {0, 0, 0};
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const int k = 32 * h + j;                                  // channel within the group
            const int q = sext4(in[k >> 3] >> (4 * (k & 7)));
            const uint64_t f = (uint64_t)(kE2M3Half[q < 0 ? -q : q] | (q < 0 ? 32u : 0u));
            const int b = 6 * j;
            bits[b >> 6] |= f << (b & 63);
            if ((b & 63) > 58) bits[(b >> 6) + 1] |= f >> (64 - (b & 63));
        }
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            dw[h][2 * i] = (uint32_t)bits[i];
            dw[h][2 * i + 1] = (uint32_t)(bits[i] >> 32);
        }
    }
    const int NP = (NG + 1) >> 1;
    *(v4u *)(blob + fp6_tiled_chunk(n, g, 0, NP)) = v4u{dw[0][0], dw[0][1], dw[0][2], dw[0][3]};
    *(v4u *)(blob + fp6_tiled_chunk(n, g, 1, NP)) = v4u{dw[1][0], dw[1][1], dw[1][2], dw[1][3]};
    const int sw = fp6_half_swap(n);
    *(v4u *)(blob + fp6_tiled_chunk(n, g, 2, NP)) = v4u{dw[sw][4], dw[sw][5], dw[sw ^ 1][4], dw[sw ^ 1][5]};
}

hipError_t launch_pack_weight_fp6(int N, int K, const void *wgt_codes, void *blob, hipStream_t stream)
{
    const int NG = K / 64;
    const long long n = (long long)N * NG;
    hipLaunchKernelGGL(pack_fp6_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, N, NG,
                       (const uint8_t *)wgt_codes, (uint8_t *)blob);
    return hipGetLastError();
}

hipError_t launch_pack_weight_int4(int N, int K, const void *wgt_codes, const void *wgt_scales, void *blob,
                                   int32_t *invalid, hipStream_t stream)
{
    const int NG = K / 64;
    if (invalid) hipLaunchKernelGGL(pack_zero_kernel, dim3(1), dim3(1), 0, stream, invalid);
    const long long n = (long long)N * NG;
    hipLaunchKernelGGL(pack_int4_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, N, NG,
                       (const uint8_t *)wgt_codes, (const uint16_t *)wgt_scales, (uint8_t *)blob, invalid);
    return hipGetLastError();
}

}  // namespace svdq
