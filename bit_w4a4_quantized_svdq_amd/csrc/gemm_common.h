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
#include "launch.h"

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

// acc <- post * acc + bias + t . up^T (fp32, in the accumulator layout)
__device__ __forceinline__ void gemm_epilogue_sum(v16f (&acc)[2][2], float post, int M, int N, int rank,
                                                  int m0, int n0, int wm, int wn, int lane,
                                                  const float *__restrict__ lora_act,
                                                  const uint16_t *__restrict__ lora_up,
                                                  const uint16_t *__restrict__ bias)
{
    const int l32 = lane & 31, h = lane >> 5;
    const bool rows_full = m0 + 128 <= M;                          // block-uniform
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
}

// Round the accumulators to bf16 and store the tile.  Registers i, i+1 (i
// even) of a lane are rows r, r+1 of one column: one packed conversion, two
// 2-byte stores.
__device__ __forceinline__ void gemm_epilogue_store(v16f (&acc)[2][2], int M, int N, int m0, int n0,
                                                    int wm, int wn, int lane, uint16_t *__restrict__ out)
{
    const int l32 = lane & 31, h = lane >> 5;
    const bool tile_full = m0 + 128 <= M && n0 + 128 <= N;          // block-uniform
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

__device__ __forceinline__ void gemm_epilogue(v16f (&acc)[2][2], float post, int M, int N, int rank,
                                              int m0, int n0, int wm, int wn, int lane,
                                              const float *__restrict__ lora_act,
                                              const uint16_t *__restrict__ lora_up,
                                              const uint16_t *__restrict__ bias,
                                              uint16_t *__restrict__ out)
{
    gemm_epilogue_sum(acc, post, M, N, rank, m0, n0, wm, wn, lane, lora_act, lora_up, bias);
    gemm_epilogue_store(acc, M, N, m0, n0, wm, wn, lane, out);
}

// ---------------------------------------------------------------------------
// Grouped QKV layer: per-head RMSNorm and rotary embedding of Q and K in the
// epilogue (the original engine fuses the QKV projection with RMSNorm and
// RoPE -- "Nunchaku Lite" docs, "Fused kernels").  Heads are 128 channels,
// one N-tile; the output columns are Q | K | V.  For a Q or K head:
//   n_j = y_j w_j / sqrt(mean_i y_i^2 + eps),   y = the layer's bf16 output,
//   (out_2i, out_2i+1) = (n_2i c_i - n_2i+1 s_i, n_2i+1 c_i + n_2i s_i),
// with the row's angles c_i = cos, s_i = sin (fp32 [M, 64]); fp32 arithmetic,
// one rounding to bf16.  V heads are stored as they are.
constexpr int QK_ROWB = 128 * 2 + 16;          // LDS bytes per staged row (padded)
constexpr int QK_SMEM = 128 * QK_ROWB;         // 34 KB

// Called by all 256 threads of a block whose tile is a Q or K head, after the
// main loop (smem: at least QK_SMEM bytes, free once every wave is past it).
__device__ __forceinline__ void gemm_epilogue_qk(v16f (&acc)[2][2], int M, int m0, int n0, int wm, int wn,
                                                 int lane, const QkNormRope &qk, uint8_t *smem, int N,
                                                 uint16_t *__restrict__ out)
{
    const int l32 = lane & 31, h = lane >> 5;
    __syncthreads();   // every wave is done with the operand stages
    // y = RNE_bf16(acc) -> LDS, row-major
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int col = wn * 64 + b * 32 + l32;
#pragma unroll
            for (int i = 0; i < 16; i += 2) {
                const int row = wm * 64 + a * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
                const uint32_t pk = pack_bf16x2_rne(acc[a][b][i], acc[a][b][i + 1]);
                *(uint16_t *)(smem + row * QK_ROWB + col * 2) = (uint16_t)pk;
                *(uint16_t *)(smem + (row + 1) * QK_ROWB + col * 2) = (uint16_t)(pk >> 16);
            }
        }
    __syncthreads();
    // Row pass: wave w takes rows 32w .. 32w+31, two per step; lane l works on
    // row 2*step + l/32 and its channels 4*(l%32) .. +3 (rotation pairs
    // 2*(l%32), +1).  Every load and store of a step covers whole rows.
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int c4 = l32;
    const v2u w2 = *(const v2u *)((n0 < (qk.qk_cols >> 1) ? qk.q_w : qk.k_w) + 4 * c4);
    const float w0 = bf16_lo(w2[0]), w1 = bf16_hi(w2[0]), w2f = bf16_lo(w2[1]), w3 = bf16_hi(w2[1]);
#pragma unroll 4
    for (int st = 0; st < 16; ++st) {
        const int r = wave * 32 + 2 * st + h;
        const int grow = min(m0 + r, M - 1);   // rows past M: clamped reads, nothing stored
        const v2u yv = *(const v2u *)(smem + r * QK_ROWB + 8 * c4);
        const v2f cv = *(const v2f *)(qk.cos + (size_t)grow * 64 + 2 * c4);
        const v2f sv = *(const v2f *)(qk.sin + (size_t)grow * 64 + 2 * c4);
        const float y0 = bf16_lo(yv[0]), y1 = bf16_hi(yv[0]), y2 = bf16_lo(yv[1]), y3 = bf16_hi(yv[1]);
        float ss = __builtin_fmaf(y0, y0, __builtin_fmaf(y1, y1, __builtin_fmaf(y2, y2, y3 * y3)));
        // sum over the 32 lanes of the row: within each 16-lane row by DPP, then across the two
        ss += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, ss), 0xB1, 0xF, 0xF, true));
        ss += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, ss), 0x4E, 0xF, 0xF, true));
        ss += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, ss), 0x124, 0xF, 0xF, true));
        ss += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, ss), 0x128, 0xF, 0xF, true));
        ss += shfl_xor_f(ss, 16);
        const float rr = 1.0f / __builtin_sqrtf(__builtin_fmaf(ss, 1.0f / 128.0f, qk.eps));
        const float n0v = y0 * rr * w0, n1v = y1 * rr * w1, n2v = y2 * rr * w2f, n3v = y3 * rr * w3;
        const v2u o = v2u{pack_bf16x2_rne(__builtin_fmaf(n0v, cv[0], -n1v * sv[0]), __builtin_fmaf(n1v, cv[0], n0v * sv[0])),
                          pack_bf16x2_rne(__builtin_fmaf(n2v, cv[1], -n3v * sv[1]), __builtin_fmaf(n3v, cv[1], n2v * sv[1]))};
        if (m0 + r < M) *(v2u *)(out + (size_t)(m0 + r) * N + n0 + 4 * c4) = o;
    }
}

// The epilogue with or without the grouped QKV layer's per-head norm/rotary
// step (QK: Q and K head tiles take gemm_epilogue_qk, the others the plain store).
template <bool QK>
__device__ __forceinline__ void gemm_epilogue_any(v16f (&acc)[2][2], float post, int M, int N, int rank, int m0,
                                                  int n0, int wm, int wn, int lane,
                                                  const float *__restrict__ lora_act,
                                                  const uint16_t *__restrict__ lora_up,
                                                  const uint16_t *__restrict__ bias, uint16_t *__restrict__ out,
                                                  const QkNormRope &qk, uint8_t *smem)
{
    gemm_epilogue_sum(acc, post, M, N, rank, m0, n0, wm, wn, lane, lora_act, lora_up, bias);
    if (QK && n0 < qk.qk_cols)   // block-uniform
        gemm_epilogue_qk(acc, M, m0, n0, wm, wn, lane, qk, smem, N, out);
    else
        gemm_epilogue_store(acc, M, N, m0, n0, wm, wn, lane, out);
}

}  // namespace svdq
