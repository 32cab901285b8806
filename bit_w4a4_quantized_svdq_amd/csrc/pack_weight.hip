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
