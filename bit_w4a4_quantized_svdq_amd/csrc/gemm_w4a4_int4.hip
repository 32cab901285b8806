// gemm_w4a4_int4.hip -- second fused step of the SVDQuant W4A4 layer, int4
// variant (group 64, bf16 scales; "Nunchaku Lite" docs, "Supported
// quantization types"), on gfx950 matrix cores:
//   y = alpha * sum_g G_g * sx_g * sw_g  +  lora_act . lora_up^T  +  bias,
//   G_g[m,n] = sum_{k in group g} qa[m,k] * qw[n,k]   (exact integers)
// with the low-rank up-projection and the bias fused into the epilogue
// (blog "Hugging Face integrates Nunchaku 4-bit diffusion inference into
// Diffusers", "SVDQuant and the Nunchaku engine").
//
// Integer products.  CDNA4 has no int4 matrix instruction, so a packed
// nibble is placed in the high half of a byte: (d << 4) & 0xF0F0F0F0 gives
// the even nibbles of a dword as int8 = 16*code, d & 0xF0F0F0F0 the odd
// ones.  Two bit operations turn 8 codes into 8 int8 lanes, and two
// v_mfma_i32_32x32x32_i8 return 256 * G_g exactly (|256 G| <= 2^20).  A dot
// product does not depend on the order of k as long as both operands use the
// same order, so the even/odd split is applied to A and B alike.
//
// Group scales.  Every output needs acc += G_g * (sx_g * sw_g) once per
// group, and on CDNA4 the vector ALU is the scarce unit (one 32x32 tile-group
// of int8 matrix work is about as long as 16 vector instructions).  The
// scale outer product P_g = sx_g (x) sw_g is therefore formed on the matrix
// core as well: an fp32 v_mfma_f32_32x32x2 with sx (A) and sw (B) in both k
// slots, i.e. P_g = 2 sx_g (x) sw_g (each operand is one register, and
// lanes 32..63 read the same scales as lanes 0..31).  A product of two bf16
// values is exact in fp32 and doubling is exact, so P_g is exact and lands in
// the same 32x32 accumulator layout as G_g.  The vector ALU then does one
// int->float conversion and one fma per output and group.  The factor 2^-9
// (2^-8 from the 16*code operands, 1/2 from P) and alpha are applied once at
// the end.
//
// Data movement.  256 threads own a 128x128 output tile (4 waves of 64x64,
// each 2x2 tiles of 32x32); one K-step is one group of 64.  A 4-stage ring in
// LDS is filled with global_load_lds (global memory straight to LDS, no
// registers): per group 4 KB of A codes and 4 KB of B codes; the scales of 8
// groups at a time into a two-slot ring.  Codes sit in LDS as
// [half][row][16 B], so the 16-byte fragment reads of a wave are contiguous
// and free of bank conflicts.  One barrier per group separates the consumers
// of a stage from its next refill.  Blocks are
// mapped to tiles so that each XCD (own L2) walks a contiguous band of tiles
// in groups of 8 M-tiles, keeping the A and B tiles in flight L2-resident.
#include "device_common.h"
#include "launch.h"

namespace svdq {

constexpr int G4_BM = 128, G4_BN = 128, G4_THREADS = 256, G4_STAGES = 4;
constexpr int G4_CODES = G4_BM * 32;                   // bytes of A (or B) codes per group
constexpr int G4_STAGE = 2 * G4_CODES;                 // one group of A and B codes: 8 KB
// Scales travel 8 groups at a time: each row's 8 consecutive bf16 scales are
// 16 contiguous bytes, so one 16-byte copy per lane moves 64 rows' scales for
// 8 groups (a copy of one 2-byte scale per lane per group would touch 64
// separate cache lines for 128 bytes).  Two 8-group slots alternate.
// A slot holds [A rows | B rows][8 groups x 2 B] when the row length K/64 is
// a multiple of 8 (16-byte aligned rows); otherwise each group's scales are
// copied one 2-byte value per lane (zero-extended to a dword) into
// [group][A rows | B rows][4 B].
constexpr int G4_SC_GROUPS = 8;
constexpr int G4_SC_SLOT = G4_SC_GROUPS * (G4_BM + G4_BN) * 4;   // 8 KB (the larger layout)
constexpr int G4_SC = G4_STAGES * G4_STAGE;            // offset of the two scale slots
constexpr int G4_SMEM = G4_SC + 2 * G4_SC_SLOT;        // 48 KB
constexpr int G4_GROUP_M = 8;                          // M-tiles per raster group

// 32x32 MFMA accumulator layout: lane l, register i -> row 8*(i/4) + 4*(l/32) + i%4, col l%32.

__device__ __forceinline__ void unpack_i8(const v4u &c, v4i &lo, v4i &hi) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lo[i] = (int)((c[i] << 4) & 0xF0F0F0F0u);
        hi[i] = (int)(c[i] & 0xF0F0F0F0u);
    }
}

// Block -> (M-tile, N-tile).  Hardware dispatches block b to XCD b % 8; give
// each XCD a contiguous range of tile ids, and order tile ids by groups of
// G4_GROUP_M M-tiles so that neighbouring tiles share A rows and B rows.
__device__ __forceinline__ void tile_of_block(int b, int nbm, int nbn, int &bm, int &bn) {
    const int nb = nbm * nbn;
    const int x = b & 7, local = b >> 3;
    const int q = nb >> 3, r = nb & 7;
    const int t = (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + local;
    const int per_group = G4_GROUP_M * nbn;
    const int first_m = (t / per_group) * G4_GROUP_M;
    const int gm = min(nbm - first_m, G4_GROUP_M);
    const int within = t % per_group;
    bm = first_m + within % gm;
    bn = within / gm;
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

// SC16: scales copied 8 groups per 16-byte copy (K/64 a multiple of 8)
template <bool GROUP_SUMS, bool SC16>
__global__ __launch_bounds__(G4_THREADS, 2)
void gemm_w4a4_int4_kernel(int M, int N, int K, int rank,
                           const uint8_t *__restrict__ act_codes,
                           const uint16_t *__restrict__ act_scales,
                           const uint8_t *__restrict__ wgt_codes,
                           const uint16_t *__restrict__ wgt_scales, float alpha,
                           const float *__restrict__ lora_act,
                           const uint16_t *__restrict__ lora_up,
                           const uint16_t *__restrict__ bias,
                           uint16_t *__restrict__ out, int32_t *__restrict__ gsum)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[G4_SMEM];
    // global_load_lds per wave for group g: 2 for the codes, plus the scales
    // (every group, or the first group of each 8 with SC16)
    auto loads_of = [](int g) { return GROUP_SUMS ? 2 : (SC16 ? 2 + ((g & 7) == 0) : 3); };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, h = lane >> 5;
    const int nbm = (M + G4_BM - 1) / G4_BM, nbn = (N + G4_BN - 1) / G4_BN;
    int bm, bn;
    tile_of_block((int)blockIdx.x, nbm, nbn, bm, bn);
    const int m0 = bm * G4_BM, n0 = bn * G4_BN;
    const int NG = K >> 6;
    const size_t rowbytes = (size_t)(K >> 1);

    // Producer role.  Wave w copies LDS chunk w (1 KB) of the A codes and of the
    // B codes of every group: chunk j = half (j/2), rows 64*(j%2) .. +63, lane l
    // -> row 64*(j%2) + l.  Rows past M (columns past N) read a clamped, valid
    // row: they only feed outputs that are never stored.  Waves 0,1 also copy
    // the A scales of rows 64w .. 64w+63, waves 2,3 the B scales (8 groups
    // per copy with SC16).
    const int p_half = wave >> 1, p_row = 64 * (wave & 1) + lane;
    const uint8_t *pa = act_codes + (size_t)min(m0 + p_row, M - 1) * rowbytes + 16 * p_half;
    const uint8_t *pb = wgt_codes + (size_t)min(n0 + p_row, N - 1) * rowbytes + 16 * p_half;
    const bool ps_is_a = wave < 2;
    const int ps_row = 64 * (wave & 1) + lane;
    const uint16_t *ps = nullptr;
    if constexpr (!GROUP_SUMS)
        ps = ps_is_a ? act_scales + (size_t)min(m0 + ps_row, M - 1) * NG
                     : wgt_scales + (size_t)min(n0 + ps_row, N - 1) * NG;
    auto issue = [&](int g) {
        uint8_t *st = smem + (g % G4_STAGES) * G4_STAGE;
        __builtin_amdgcn_global_load_lds((gptr_t)(pa + (size_t)g * 32), (lptr_t)(st + wave * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((gptr_t)(pb + (size_t)g * 32), (lptr_t)(st + G4_CODES + wave * 1024),
                                         16, 0, 0);
        if constexpr (!GROUP_SUMS) {
            uint8_t *slot = smem + G4_SC + ((g >> 3) & 1) * G4_SC_SLOT;
            if constexpr (SC16) {
                if ((g & 7) == 0)   // rows' scales of groups g .. g+7: [A rows | B rows][16 B]
                    __builtin_amdgcn_global_load_lds((gptr_t)(ps + g),
                        (lptr_t)(slot + (ps_is_a ? 0 : G4_BM * 16) + 1024 * (wave & 1)), 16, 0, 0);
            } else {                // group g's scales: [g % 8][A rows | B rows][4 B]
                __builtin_amdgcn_global_load_lds((gptr_t)(ps + g),
                    (lptr_t)(slot + (g & 7) * (4 * (G4_BM + G4_BN)) + (ps_is_a ? 0 : 4 * G4_BM) + 256 * (wave & 1)),
                    2, 0, 0);
            }
        }
    };

    v16f acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

    // consumer offsets inside a stage
    int a_off[2], b_off[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        a_off[t] = h * (G4_CODES / 2) + (wm * 64 + t * 32 + l32) * 16;
        b_off[t] = G4_CODES + h * (G4_CODES / 2) + (wn * 64 + t * 32 + l32) * 16;
    }

    for (int g = 0; g < G4_STAGES - 1 && g < NG; ++g) issue(g);

    for (int g = 0; g < NG; ++g) {
        // this wave's copies of group g have landed once at most the copies of
        // the groups issued after it are still in flight
        const int newer = min(G4_STAGES - 2, NG - 1 - g);
        int newer_loads = 0;
        for (int j = 1; j <= newer; ++j) newer_loads += loads_of(g + j);
        wait_vmcnt(newer_loads);
        // Workgroup barrier without the full memory fence of __syncthreads()
        // (which would also wait for the copies still in flight): every wave
        // has waited for its own copies of g, so after the barrier all of g is
        // in LDS, and every wave has finished reading the stage of g-1.  The
        // empty asm statements keep the compiler from moving LDS accesses
        // across the barrier.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (g + G4_STAGES - 1 < NG) issue(g + G4_STAGES - 1);

        const uint8_t *st = smem + (g % G4_STAGES) * G4_STAGE;
        v4u fa[2], fb[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            fa[t] = *(const v4u *)(st + a_off[t]);
            fb[t] = *(const v4u *)(st + b_off[t]);
        }
        v4i alo[2], ahi[2], blo[2], bhi[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            unpack_i8(fa[t], alo[t], ahi[t]);
            unpack_i8(fb[t], blo[t], bhi[t]);
        }

        if constexpr (GROUP_SUMS) {
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    v16i G = {};
                    G = __builtin_amdgcn_mfma_i32_32x32x32_i8(alo[a], blo[b], G, 0, 0, 0);
                    G = __builtin_amdgcn_mfma_i32_32x32x32_i8(ahi[a], bhi[b], G, 0, 0, 0);
                    const int col = n0 + wn * 64 + b * 32 + l32;
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int rowi = m0 + wm * 64 + a * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
                        if (rowi < M && col < N) gsum[((size_t)rowi * N + col) * NG + g] = G[i] >> 8;
                    }
                }
        } else {
            // P-MFMA operands: this lane's row scale as fp32 (a bf16 is the top
            // half of an fp32), the same value in both k slots
            const uint8_t *slot = smem + G4_SC + ((g >> 3) & 1) * G4_SC_SLOT;
            float pa_op[2], pb_op[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int ra = wm * 64 + t * 32 + l32, rb = wn * 64 + t * 32 + l32;
                uint32_t sa, sb;
                if constexpr (SC16) {
                    sa = *(const uint16_t *)(slot + ra * 16 + (g & 7) * 2);
                    sb = *(const uint16_t *)(slot + G4_BM * 16 + rb * 16 + (g & 7) * 2);
                } else {
                    const uint8_t *gs = slot + (g & 7) * (4 * (G4_BM + G4_BN));
                    sa = *(const uint32_t *)(gs + ra * 4) & 0xFFFFu;
                    sb = *(const uint32_t *)(gs + 4 * G4_BM + rb * 4) & 0xFFFFu;
                }
                pa_op[t] = __uint_as_float(sa << 16);
                pb_op[t] = __uint_as_float(sb << 16);
            }
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    v16i G = {};
                    G = __builtin_amdgcn_mfma_i32_32x32x32_i8(alo[a], blo[b], G, 0, 0, 0);
                    G = __builtin_amdgcn_mfma_i32_32x32x32_i8(ahi[a], bhi[b], G, 0, 0, 0);
                    v16f P = {};
                    P = __builtin_amdgcn_mfma_f32_32x32x2f32(pa_op[a], pb_op[b], P, 0, 0, 0);   // 2 sx sw
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        acc[a][b][i] = __builtin_fmaf((float)G[i], P[i], acc[a][b][i]);
                    if (b == 1) __builtin_amdgcn_sched_barrier(0);   // at most 2 tiles of G, P live
                }
        }
    }

    if constexpr (!GROUP_SUMS) {
        const float post = alpha * 0.001953125f;           // alpha * 2^-9
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[a][b][i] *= post;

        // ---- low-rank up-projection on the matrix cores: acc += t . up^T.
        // t (fp32) is split into bf16 hi + lo (t - hi is exact in fp32), the
        // up factor is bf16, products are exact in fp32.
        for (int s = 0; s < rank; s += 16) {
            v8bf thi[2], tlo[2], up[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int rrow = m0 + wm * 64 + t * 32 + l32;
                v4u hv = v4u{0u, 0u, 0u, 0u}, lv = hv;
                if (rrow < M) {
                    const float *tp = lora_act + (size_t)rrow * rank + s + 8 * h;
                    v4f t0 = *(const v4f *)tp, t1 = *(const v4f *)(tp + 4);
                    float tv[8] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        uint32_t h0 = f32_to_bf16_rne(tv[2 * p]), h1 = f32_to_bf16_rne(tv[2 * p + 1]);
                        uint32_t l0 = f32_to_bf16_rne(tv[2 * p] - __uint_as_float(h0 << 16));
                        uint32_t l1 = f32_to_bf16_rne(tv[2 * p + 1] - __uint_as_float(h1 << 16));
                        hv[p] = h0 | (h1 << 16);
                        lv[p] = l0 | (l1 << 16);
                    }
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

        // ---- bias and the bf16 store
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int col = n0 + wn * 64 + b * 32 + l32;
            if (col >= N) continue;
            const float bv = bias ? bf16_to_f32(bias[col]) : 0.0f;
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int rowi = m0 + wm * 64 + a * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
                    if (rowi < M)
                        out[(size_t)rowi * N + col] = (uint16_t)f32_to_bf16_rne(acc[a][b][i] + bv);
                }
        }
    }
}

hipError_t launch_gemm_w4a4_int4(int M, int N, int K, int rank, const void *act_codes,
                                 const void *act_scales, const void *wgt_codes,
                                 const void *wgt_scales, float alpha, const float *lora_act,
                                 const void *lora_up, const void *bias, void *out,
                                 hipStream_t stream)
{
    dim3 grid(((N + G4_BN - 1) / G4_BN) * ((M + G4_BM - 1) / G4_BM)), block(G4_THREADS);
    if ((K >> 6) % G4_SC_GROUPS == 0)
        hipLaunchKernelGGL((gemm_w4a4_int4_kernel<false, true>), grid, block, 0, stream, M, N, K, rank,
                           (const uint8_t *)act_codes, (const uint16_t *)act_scales,
                           (const uint8_t *)wgt_codes, (const uint16_t *)wgt_scales, alpha, lora_act,
                           (const uint16_t *)lora_up, (const uint16_t *)bias, (uint16_t *)out,
                           (int32_t *)nullptr);
    else
        hipLaunchKernelGGL((gemm_w4a4_int4_kernel<false, false>), grid, block, 0, stream, M, N, K, rank,
                           (const uint8_t *)act_codes, (const uint16_t *)act_scales,
                           (const uint8_t *)wgt_codes, (const uint16_t *)wgt_scales, alpha, lora_act,
                           (const uint16_t *)lora_up, (const uint16_t *)bias, (uint16_t *)out,
                           (int32_t *)nullptr);
    return hipGetLastError();
}

hipError_t launch_group_sums_int4(int M, int N, int K, const void *act_codes,
                                  const void *wgt_codes, int32_t *G, hipStream_t stream)
{
    dim3 grid(((N + G4_BN - 1) / G4_BN) * ((M + G4_BM - 1) / G4_BM)), block(G4_THREADS);
    hipLaunchKernelGGL((gemm_w4a4_int4_kernel<true, false>), grid, block, 0, stream, M, N, K, 0,
                       (const uint8_t *)act_codes, (const uint16_t *)nullptr,
                       (const uint8_t *)wgt_codes, (const uint16_t *)nullptr, 1.0f,
                       (const float *)nullptr, (const uint16_t *)nullptr,
                       (const uint16_t *)nullptr, (uint16_t *)nullptr, G);
    return hipGetLastError();
}

}  // namespace svdq
