// gemm_common.h -- pieces shared by the two W4A4 GEMM kernels (int4 and
// NVFP4): tile rasterization, copy/barrier helpers, and the epilogue
// y = post * acc + bias + t . up^T, rounded to bf16 and stored.  The
// low-rank up-projection is the second half of the 16-bit branch of the
// SVDQuant layer, fused into the 4-bit GEMM (blog "Hugging Face integrates
// Nunchaku 4-bit diffusion inference into Diffusers", "SVDQuant and the
// Nunchaku engine").  Internal to the HIP library.
//
// Tile geometry (both kernels): 256 threads own a 128x128 output tile at
// (m0, n0); wave w covers rows 64*(w/2) .. +63 and columns 64*(w%2) .. +63 as
// 2x2 tiles of 32x32 in the MFMA accumulator layout (lane l, register i ->
// row 8*(i/4) + 4*(l/32) + i%4, column l%32).
#pragma once

#include "device_common.h"

namespace svdq {

// Block -> (M-tile, N-tile).  Hardware dispatches block b to XCD b % 8; give
// each XCD a contiguous range of tile ids, and order tile ids by groups of
// group_m M-tiles so that neighbouring tiles share A rows and B rows.
__device__ __forceinline__ void tile_of_block(int b, int nbm, int nbn, int group_m, int &bm, int &bn) {
    const int nb = nbm * nbn;
    const int x = b & 7, local = b >> 3;
    const int q = nb >> 3, r = nb & 7;
    const int t = (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + local;
    const int per_group = group_m * nbn;
    const int first_m = (t / per_group) * group_m;
    const int gm = min(nbm - first_m, group_m);
    const int within = t % per_group;
    bm = first_m + within % gm;
    bn = within / gm;
}

// The optimizer forgets what x holds: x is (re)defined at this point, so
// nothing computed from it can be hoisted above, and a value that reaches it
// must be complete here.
template <typename T>
__device__ __forceinline__ void opaque(T &x) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" : "+v"(x));
#endif
}

__device__ __forceinline__ void wait_vmcnt(int n) {
    // s_waitcnt with vmcnt = n (0 <= n <= 7); expcnt and lgkmcnt left unconstrained
    switch (n) {
        case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
        case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
        case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
        case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
        case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
        case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
        case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
        default: __builtin_amdgcn_s_waitcnt(0x0F77); break;
    }
}

// Workgroup barrier without the full memory fence of __syncthreads() (which
// would also wait for every copy still in flight).  Callers wait for the
// copies they need with wait_vmcnt() first.  The empty asm statements keep
// the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ void gemm_epilogue(v16f (&acc)[2][2], float post, int M, int N, int rank,
                                              int m0, int n0, int wm, int wn, int lane,
                                              const float *__restrict__ lora_act,
                                              const uint16_t *__restrict__ lora_up,
                                              const uint16_t *__restrict__ bias,
                                              uint16_t *__restrict__ out)
{
    const int l32 = lane & 31, h = lane >> 5;
    const bool rows_full = m0 + 128 <= M;                          // block-uniform
    const bool tile_full = rows_full && n0 + 128 <= N;
    float bv[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int col = n0 + wn * 64 + b * 32 + l32;
        bv[b] = (bias && col < N) ? bf16_to_f32(bias[col]) : 0.0f;
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][b][i] = __builtin_fmaf(acc[a][b][i], post, bv[b]);

    // ---- low-rank up-projection on the matrix cores: acc += t . up^T.
    // t (fp32) is split into bf16 hi + lo (t - hi is exact in fp32), the up
    // factor is bf16, products are exact in fp32.
    for (int s = 0; s < rank; s += 16) {
        v8bf thi[2], tlo[2], up[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int rrow = m0 + wm * 64 + t * 32 + l32;
            v4f t0 = v4f{0.f, 0.f, 0.f, 0.f}, t1 = t0;
            if (rows_full || rrow < M) {
                const float *tp = lora_act + (size_t)rrow * rank + s + 8 * h;
                t0 = *(const v4f *)tp;
                t1 = *(const v4f *)(tp + 4);
            }
            const float tv[8] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
            v4u hv, lv;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t hb = pack_bf16x2_rne(tv[2 * p], tv[2 * p + 1]);
                hv[p] = hb;
                lv[p] = pack_bf16x2_rne(tv[2 * p] - bf16_lo(hb), tv[2 * p + 1] - bf16_hi(hb));
            }
            thi[t] = __builtin_bit_cast(v8bf, hv);
            tlo[t] = __builtin_bit_cast(v8bf, lv);
            const int ucol = n0 + wn * 64 + t * 32 + l32;
            v4u uv = ucol < N ? *(const v4u *)(lora_up + (size_t)ucol * rank + s + 8 * h)
                              : v4u{0u, 0u, 0u, 0u};
            up[t] = __builtin_bit_cast(v8bf, uv);
        }
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(thi[a], up[b], acc[a][b], 0, 0, 0);
                acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tlo[a], up[b], acc[a][b], 0, 0, 0);
            }
    }

    // ---- bf16 store.  Registers i, i+1 (i even) of a lane are rows r, r+1 of
    // one column: one packed conversion, two 2-byte stores.
    if (tile_full && N <= (1 << 22)) {
        // whole tile in range: buffer stores; the row offset of each store is
        // block-uniform (scalar register), only the column part is per lane
        const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(out + (size_t)m0 * N + n0), (short)0, 128 * N * 2, 0x00020000);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int voff = (4 * h * N + wn * 64 + b * 32 + l32) * 2;
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int i = 0; i < 16; i += 2) {
                    const int row = wm * 64 + a * 32 + 8 * (i >> 2) + (i & 3);
                    const uint32_t pk = pack_bf16x2_rne(acc[a][b][i], acc[a][b][i + 1]);
                    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)pk, ro, voff, row * N * 2, 0);
                    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(pk >> 16), ro, voff, (row + 1) * N * 2, 0);
                }
        }
    } else {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int col = n0 + wn * 64 + b * 32 + l32;
            if (col >= N) continue;
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int i = 0; i < 16; i += 2) {
                    const int rowi = m0 + wm * 64 + a * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
                    const uint32_t pk = pack_bf16x2_rne(acc[a][b][i], acc[a][b][i + 1]);
                    if (rowi < M) out[(size_t)rowi * N + col] = (uint16_t)pk;
                    if (rowi + 1 < M) out[(size_t)(rowi + 1) * N + col] = (uint16_t)(pk >> 16);
                }
        }
    }
}

}  // namespace svdq
