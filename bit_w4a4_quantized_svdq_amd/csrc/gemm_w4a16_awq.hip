// gemm_w4a16_awq.hip -- the AWQ int4 weight-only layer with bf16 activations
// ("Nunchaku Lite" docs, "Supported quantization types": awq_w4a16 int4
// group 64) in the GEMM regime, i.e. many rows of x at once (a whole image's
// tokens through a weight-only layer):
//   y[m,n] = sum_k x[m,k] * (q[n,k] - z[n,g]) * s[n,g] + bias[n],   g = k/64.
// The GEMV kernel streams the weights once per 32 rows of x; from a few
// hundred rows on, this kernel, which reads every weight once per 128 rows
// and keeps the matrix core busy, is faster.
//
// Arithmetic (bf16 matrix core, fp32 accumulation):
//   * a code q in 0..15 becomes the bf16 value 128 + q by OR-ing it into the
//     bit pattern 0x4300 (bf16 128 has a unit mantissa step), so the B
//     operand is built with integer bit operations only;
//   * per group, T = sum_k x (128 + q) - (128 + z) X with X = sum_k x over the
//     group's 64 k of the row; the correction -(128 + z) (x) X is a rank-1
//     product formed by a two-block bf16 MFMA (X in three exact bf16 pieces,
//     -(128 + z) exact) and enters the group's MFMA chain as its C input;
//   * y += s * T once per output and group on the vector ALU.
// The correction is about 16 times the result, so fp32 rounding costs ~2^-20
// relative, far below the bf16 output's 2^-9.
//
// Data movement: 256 threads own a 128x128 output tile (4 waves of 64x64);
// one K-step is one group.  A 3-stage LDS ring is filled by buffer loads that
// write LDS directly: per group 16 KB of x (128 rows x 128 B, eight lanes per
// row; the 16-byte chunk c of row r stored at c ^ (r & 7), so that 8 rows
// read at one k offset fall on distinct banks) and 4 KB of codes
// ([half][row][16 B]).  Scales and zero points travel 8 groups (16 B per row)
// per copy into a two-slot ring.  After each group lands, one LDS pass of all
// 256 threads forms X for the block's rows (v_dot2_f32_bf16 against (1, 1))
// and stores its bf16 pieces; a barrier separates that pass from the MFMAs.
// A lane's codes cover k = 32h .. 32h+31 of the group (h = lane/32) and MFMA
// step j its k = 32h + 8j .. +7; the x fragments use the same k.
#include "device_common.h"
#include "gemm_common.h"
#include "launch.h"

namespace svdq {
typedef short v4s __attribute__((ext_vector_type(4)));
typedef float v32f __attribute__((ext_vector_type(32)));

constexpr int AG_BM = 128, AG_BN = 128, AG_THREADS = 256, AG_STAGES = 3;
constexpr int AG_X = AG_BM * 128;                   // x of one group: 16 KB
constexpr int AG_W = AG_BN * 32;                    // codes of one group: 4 KB
constexpr int AG_STAGE = AG_X + AG_W;
constexpr int AG_SZ_SLOT = 2 * AG_BN * 16;          // [scale rows | zero rows][8 groups x bf16]
constexpr int AG_XS_SLOT = AG_BM * 8;               // X pieces of one group: [row][4 x bf16]
constexpr int AG_SZ = AG_STAGES * AG_STAGE;
constexpr int AG_XS = AG_SZ + 2 * AG_SZ_SLOT;
constexpr int AG_SMEM = AG_XS + 2 * AG_XS_SLOT;     // 70 KB: two blocks per CU

__global__ __launch_bounds__(AG_THREADS, 2)
void awq_gemm_kernel(int M, int N, int K, const uint16_t *__restrict__ x,
                     const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
                     const uint16_t *__restrict__ zeros, const uint16_t *__restrict__ bias,
                     uint16_t *__restrict__ out)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[AG_SMEM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, h = lane >> 5;
    const int nbm = (M + AG_BM - 1) / AG_BM, nbn = (N + AG_BN - 1) / AG_BN;
    int bm, bn;
    tile_of_block((int)blockIdx.x, nbm, nbn, 8, bm, bn);
    const int m0 = bm * AG_BM, n0 = bn * AG_BN;
    const int NG = K >> 6;
    const int rows_a = min(AG_BM, M - m0), rows_b = min(AG_BN, N - n0);

    // x copies: wave w issues instructions w, w+4, w+8, w+12 (8 rows x 128 B
    // each): lane i -> row 8q + i/8, LDS slot i%8 holding chunk (i%8) ^ (row & 7).
    // Rows past M read a clamped valid row (their outputs are never stored).
    uint32_t xa_off[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int r = 8 * (wave + 4 * u) + (lane >> 3);
        xa_off[u] = (uint32_t)(min(r, rows_a - 1) * K * 2 + 16 * ((lane & 7) ^ (r & 7)));
    }
    // code copies: wave w copies LDS chunk w (1 KB): half w/2, rows 64*(w%2) + lane
    const int p_row = 64 * (wave & 1) + lane;
    const uint32_t cb_off = (uint32_t)(min(p_row, rows_b - 1) * (K >> 1) + 16 * (wave >> 1));
    // scales (waves 0,1) and zero points (waves 2,3) of 8 groups: 16 B per row
    const bool sz_is_s = wave < 2;
    const uint32_t sz_off = (uint32_t)(min(p_row, rows_b - 1) * NG * 2);
    const __amdgpu_buffer_rsrc_t rsx = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(x + (size_t)m0 * K), (short)0, rows_a * K * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(codes + (size_t)n0 * (K >> 1)), (short)0, rows_b * (K >> 1), 0x00020000);
    const __amdgpu_buffer_rsrc_t rsz = __builtin_amdgcn_make_buffer_rsrc(
        (void *)((sz_is_s ? scales : zeros) + (size_t)n0 * NG), (short)0, rows_b * NG * 2, 0x00020000);
    auto issue_group = [&](int g) {
        uint8_t *st = smem + (g % AG_STAGES) * AG_STAGE;
#pragma unroll
        for (int u = 0; u < 4; ++u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsx, (lptr_t)(st + (wave + 4 * u) * 1024), 16, xa_off[u], g * 128, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsc, (lptr_t)(st + AG_X + wave * 1024), 16, cb_off, g * 32, 0, 0);
    };
    auto issue_chunk = [&](int c, int slot) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsz,
            (lptr_t)(smem + AG_SZ + slot * AG_SZ_SLOT + (sz_is_s ? 0 : AG_BN * 16) + 1024 * (wave & 1)),
            16, sz_off, c * 2, 0, 0);
    };

    v32f acc[2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int i = 0; i < 32; ++i) acc[a][i] = 0.0f;

    // X pass: thread t sums half t%2 (chunks 4*(t%2) .. +3) of row t/2
    const int xr = tid >> 1, xh = tid & 1;
    // consumer offsets
    int a_row[2], b_off[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        a_row[t] = wm * 64 + t * 32 + l32;
        b_off[t] = AG_X + h * (AG_W / 2) + (wn * 64 + t * 32 + l32) * 16;
    }
    const uint32_t ones = 0x3F803F80u;   // bf16 (1, 1)

    // per group: X pieces into slot `xs`
    auto x_pass = [&](const uint8_t *st, uint8_t *xs) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const v4u d = *(const v4u *)(st + xr * 128 + 16 * ((4 * xh + i) ^ (xr & 7)));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t w = d[e];   // a scalar copy: bit_cast of a vector element misbehaves in this compiler
                s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, w), __builtin_bit_cast(v2bf, ones), s, false);
            }
        }
        s += shfl_xor_f(s, 1);
        if (xh == 0) {
            // three bf16 pieces whose exact sum is s to within 2^-24 relative
            const uint32_t hi = __float_as_uint(s) & 0xFFFF0000u;
            const float r1 = s - __uint_as_float(hi);
            const uint32_t mid = __float_as_uint(r1) & 0xFFFF0000u;
            const float r2 = r1 - __uint_as_float(mid);
            const uint32_t lo = pack_bf16x2_rne(r2, 0.0f);
            *(v2u *)(xs + xr * 8) = v2u{(hi >> 16) | mid, lo};
        }
    };

    auto compute = [&](const uint8_t *st, const uint8_t *sz, const uint8_t *xs, int j) {
        // B operands of both column tiles: (128 + q) as bf16, natural k pairs
        v4u bop[2][4];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const v4u w = *(const v4u *)(st + b_off[b]);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const uint32_t L = w[s] & 0x0F0F0F0Fu, H = (w[s] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
                for (int d = 0; d < 4; ++d)
                    bop[b][s][d] = __builtin_amdgcn_perm(H, L, 0x0C000C00u | ((uint32_t)(4 + d) << 16) | (uint32_t)d) | 0x43004300u;
            }
        }
        // this lane's column (two-block layout: lane l -> column wn*64 + l): -(128 + z) in k slots 0..2
        const float zc = -(128.0f + bf16_to_f32(*(const uint16_t *)(sz + (AG_BN + wn * 64 + lane) * 16 + 2 * j)));
        const uint32_t zb = __float_as_uint(zc) >> 16;   // exact: an integer of at most 8 bits
        const v4s cb = __builtin_bit_cast(v4s, v2u{zb | (zb << 16), zb});
        float sc[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) sc[b] = bf16_to_f32(*(const uint16_t *)(sz + (wn * 64 + b * 32 + l32) * 16 + 2 * j));
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            const v4s xp = __builtin_bit_cast(v4s, *(const v2u *)(xs + a_row[a] * 8));
            v32f C = {};
            C = __builtin_amdgcn_mfma_f32_32x32x4bf16_1k(xp, cb, C, 0, 0, 0);
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                v16f T;
#pragma unroll
                for (int i = 0; i < 16; ++i) T[i] = C[16 * b + i];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const v4u xa = *(const v4u *)(st + a_row[a] * 128 + 16 * ((4 * h + s) ^ (a_row[a] & 7)));
                    T = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, xa),
                                                                 __builtin_bit_cast(v8bf, bop[b][s]), T, 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[a][16 * b + i] = __builtin_fmaf(sc[b], T[i], acc[a][16 * b + i]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Per wave, a group costs 5 copies (x 4, codes 1) and a chunk of 8 groups
    // one more (scales or zero points, issued in the chunk's second
    // iteration).  Before group g's first barrier at most group g+1's copies
    // may be in flight, plus the chunk copy when it was issued after them.
    issue_chunk(0, 0);
    issue_group(0);
    issue_group(1);
    for (int c = 0; c < NG; c += 8) {
        const bool last = c + 8 == NG;
        const int par = (c >> 3) & 1;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int g = c + j;
            __builtin_amdgcn_sched_barrier(0);
            if (last && j == 7) wait_vmcnt(0);
            else if (!last && j == 2) wait_vmcnt(6);
            else wait_vmcnt(5);
            lds_barrier();
            if (!last || j < 6) issue_group(g + 2);
            if (!last && j == 1) issue_chunk(c + 8, par ^ 1);
            const uint8_t *st = smem + (g % AG_STAGES) * AG_STAGE;
            uint8_t *xs = smem + AG_XS + (j & 1) * AG_XS_SLOT;
            x_pass(st, xs);
            // the X pieces are LDS stores of this wave: complete them, then the barrier
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt unconstrained
            lds_barrier();
            compute(st, smem + AG_SZ + par * AG_SZ_SLOT, xs, j);
#pragma unroll
            for (int a = 0; a < 2; ++a) opaque(acc[a]);
        }
    }

    v16f acc4[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc4[a][b][i] = acc[a][16 * b + i];
    gemm_epilogue(acc4, 1.0f, M, N, 0, m0, n0, wm, wn, lane, nullptr, nullptr, bias, out);
}

bool awq_gemm_applies(int M, int N, int K)
{
    const long long tiles = (long long)((M + 31) / 32) * (long long)((N + 31) / 32);
    return K % 512 == 0 && M >= AWQ_GEMM_MIN_M && tiles >= AWQ_GEMM_MIN_TILES;
}

hipError_t launch_awq_gemm(int M, int N, int K, const void *x, const void *codes, const void *scales,
                           const void *zeros, const void *bias, void *out, hipStream_t stream)
{
    dim3 grid(((N + AG_BN - 1) / AG_BN) * ((M + AG_BM - 1) / AG_BM)), block(AG_THREADS);
    hipLaunchKernelGGL(awq_gemm_kernel, grid, block, 0, stream, M, N, K, (const uint16_t *)x,
                       (const uint8_t *)codes, (const uint16_t *)scales, (const uint16_t *)zeros,
                       (const uint16_t *)bias, (uint16_t *)out);
    return hipGetLastError();
}

}  // namespace svdq
