// gemm_w4a4_fp6.hip -- second fused step of the SVDQuant W4A4 layer, int4
// variant (group 64, bf16 scales; "Nunchaku Lite" docs, "Supported
// quantization types"), with both operands' codes held as E2M3 values:
//   y = alpha * sum_g X_g * (sx_g (x) sw_g)  +  lora_act . lora_up^T  +  bias,
//   X_g[m,n] = sum_{k in group g} qa[m,k] * qw[n,k]   (exact integers)
// with the low-rank up-projection and the bias fused into the epilogue (blog
// "Hugging Face integrates Nunchaku 4-bit diffusion inference into
// Diffusers", "SVDQuant and the Nunchaku engine").
//
// Operands.  Both sides arrive in the FP6 tiled layout (activation step
// with the FP6 output, weights re-encoded once by svdq_pack_weight_fp6;
// fp6_tiled_chunk): per row and group two 192-bit strings, one per K-half,
// field j = E2M3 code of q/2 for channel 32h + j, as 16-byte chunks [h0
// dw0-3 | h1 dw0-3 | h0 dw4-5, h1 dw4-5].  Every int4 code is exact in E2M3 (q/2 in
// {0, +-0.5, ..., +-4}), so v_mfma_scale_f32_32x32x64_f8f6f4 in its FP6 form
// with E8M0 block scales 2^1 on both sides returns X_g exactly in fp32, at
// the FP6/FP4 rate (half the cycles of the FP8 form) and with no conversion
// on the vector ALU: a lane's 24 bytes are the instruction's operand as they
// are (one 16-byte and one 8-byte LDS read).
//
// Group scales.  P_g = sx_g (x) sw_g of a 32x32 tile comes from a bf16
// v_mfma_f32_32x32x16 in which only one k slot pairs two non-zero values (a
// product of two bf16 values is exact in fp32), and the vector ALU does
// acc += X_g * P_g, one fma per output and group.  A lane holds the bf16
// pairs (groups 2s, 2s+1) of one A row (lanes 0-31: row l of the wave's first
// row tile, lanes 32-63: of the second) and of its two B columns l % 32.  The
// A operand of row tile a keeps the pair only in the lanes of half a (k = 0,
// 1 or k = 8, 9), the B operand of group 2s + gg keeps only that group's half
// of the pair (k = gg and 8 + gg): the one k slot where both are non-zero is
// 8a + gg.  Every other product is a finite scale times zero.
// The scales are read from global memory straight into registers (8 bytes =
// 4 groups per load when K/64 is a multiple of 4, else 2 bytes per group),
// so LDS holds only codes.
//
// Data movement.  256 threads own a 128x128 output tile (4 waves of 64x64,
// each 2x2 tiles of 32x32).  Stages hold two groups: 96 bytes of each of the
// tile's 128 A rows and 128 B rows (24 KB), written by buffer loads straight
// into LDS; two stages alternate (48 KB, three blocks per CU).  In the tiled
// layout a stage's 12 KB of one operand is one contiguous block already in
// the LDS arrangement, so 12 copies of 1 KB (whole cache lines, lane i at
// byte 16i) fill it: row r's chunk c sits in slot (c + fp6_rot(r)) mod 6 of
// its 96 bytes and the two 8-byte halves of its last chunk are swapped when
// fp6_half_swap(r), so the 16 rows whose 16-byte fragments one LDS cycle
// serves, and the 32 rows whose 8-byte pieces it serves, fall on distinct
// banks (64 banks of 4 bytes).  One barrier per stage; the copies of
// stage s+1 go out right after it and land while stage s is computed.  Rows
// past M (columns past N) of the last tile, and the second group of the last
// pair when K/64 is odd, are padding the producers never write: they hold
// some E2M3 values, all finite, which only feed outputs that are not stored,
// or are multiplied by a zero scale.
// Blocks are mapped to tiles so that each XCD walks a contiguous band of
// tiles in groups of 8 M-tiles (tile_of_block).
//
// Epilogue: acc * alpha + bias, the low-rank up-projection on the matrix
// core, bf16 stores (gemm_common.h); the grouped QKV layer's per-head
// RMSNorm + rotary step when QK.
#include <utility>

#include "device_common.h"
#include "gemm_common.h"
#include "launch.h"

namespace svdq {
typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int F6_BM = 128, F6_BN = 128, F6_THREADS = 256;
constexpr int F6_GB = 48;                                // bytes per row and group
constexpr int F6_ROWB = 2 * F6_GB;                       // bytes per row and stage (two groups)
constexpr int F6_OPER = F6_BM * F6_ROWB;                 // 12 KB of one operand per stage
constexpr int F6_STAGE = 2 * F6_OPER;                    // 24 KB
constexpr int F6_SMEM = 2 * F6_STAGE;                    // 48 KB
constexpr int F6_COPIES = F6_OPER / 1024;                // 12 copies of 1 KB per operand and stage
constexpr int F6_GROUP_M = 8;                            // M-tiles per raster group
static_assert(F6_SMEM >= QK_SMEM, "the QK epilogue stages a 128-row tile in the operand LDS");
static_assert(F6_COPIES % 4 == 0, "every wave issues the same number of copies");

// LDS slot (16-byte unit within a row's 96 bytes) of the row's chunk c
__device__ __forceinline__ int f6_slot(int row, int c) { return (c + fp6_rot(row)) % 6; }

// X = sum_k qa_k * qw_k over one group: FP6 (E2M3) operands holding q/2,
// block scales 2^1 * 2^1 (E8M0 128): exact integers in fp32
__device__ __forceinline__ v16f mfma_group_fp6(const v8i &a, const v8i &b) {
    constexpr int kFp6 = 2;                  // format code of E2M3 for both operands
    constexpr int kScale2p1 = 127 + 1;
    const v16f z = {};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, z, kFp6, kFp6, 0, kScale2p1, 0, kScale2p1);
}

// s_waitcnt vmcnt(0) (expcnt, lgkmcnt unconstrained)
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// SC4: K/64 a multiple of 4 (scales of 4 groups per 8-byte load);
// GROUP_SUMS: write X_g (int32 [M][N][K/64]) instead of the layer's output;
// QK: grouped QKV layer (gemm_epilogue_qk for the Q and K heads)
template <bool GROUP_SUMS, bool SC4, bool QK>
__global__ __launch_bounds__(F6_THREADS, GROUP_SUMS ? 2 : 3)
void gemm_w4a4_fp6_kernel(int M, int N, int K, int rank,
                          const uint8_t *__restrict__ act_codes,
                          const uint16_t *__restrict__ act_scales,
                          const uint8_t *__restrict__ wgt_codes,
                          const uint16_t *__restrict__ wgt_scales, float alpha,
                          const float *__restrict__ lora_act,
                          const uint16_t *__restrict__ lora_up,
                          const uint16_t *__restrict__ bias,
                          uint16_t *__restrict__ out, int32_t *__restrict__ gsum,
                          QkNormRope qk)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[F6_SMEM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, h = lane >> 5;
    const int nbm = (M + F6_BM - 1) / F6_BM, nbn = (N + F6_BN - 1) / F6_BN;
    int bm, bn;
    tile_of_block((int)blockIdx.x, nbm, nbn, F6_GROUP_M, bm, bn);
    const int m0 = bm * F6_BM, n0 = bn * F6_BN;
    const int NG = K >> 6;
    const int NP = (NG + 1) >> 1;                           // stages (pairs of groups)
    const int tile_bytes = NP * FP6_PAIR_BYTES;             // one 128-row tile of an operand

    // ---- producer: copy q = wave + 4u (u = 0, 1, 2) of each operand moves
    // bytes 1024q .. 1024q + 1023 of the stage's 12 KB block (lane i: 16i)
    static_assert(F6_OPER == FP6_PAIR_BYTES, "a stage holds one pair of the tiled layout");
    const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(act_codes + (size_t)bm * tile_bytes), (short)0, tile_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(wgt_codes + (size_t)bn * tile_bytes), (short)0, tile_bytes, 0x00020000);
    const uint32_t c_off = (uint32_t)(1024 * wave + 16 * lane);
    // groups 2s, 2s+1 into stage `buf`
    auto issue_pair = [&](int s, int buf) {
        uint8_t *st = smem + buf * F6_STAGE;
#pragma unroll
        for (int u = 0; u < F6_COPIES / 4; ++u) {
            const int q = wave + 4 * u;
            const int soff = s * F6_OPER + 4096 * u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lptr_t)(st + q * 1024), 16, c_off, soff, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lptr_t)(st + F6_OPER + q * 1024), 16, c_off, soff, 0, 0);
        }
    };

    // ---- consumer: fragment offsets of group gg of a stage (tile t adds 32
    // rows = 3072 bytes; B adds a wave-uniform delta: rotation and swap
    // depend on row bits 2-4 only).  The 16-byte piece of group 1 sits 48
    // bytes after that of group 0 (the rotation is at most 1), the 8-byte
    // piece wraps for rotated rows and is the second half of its chunk for
    // h = 1, or for h = 0 in swapped rows.
    const int ra = wm * 64 + l32;
    const int a16 = ra * F6_ROWB + 16 * f6_slot(ra, h);
    const int a8_0 = ra * F6_ROWB + 16 * f6_slot(ra, 2) + 8 * (h ^ fp6_half_swap(ra));
    const int a8_1 = ra * F6_ROWB + 16 * f6_slot(ra, 5) + 8 * (h ^ fp6_half_swap(ra));
    const int bdelta = F6_OPER + (wn - wm) * 64 * F6_ROWB;

    // ---- scales: lanes 0-31 the A row l of the first tile, 32-63 of the
    // second; every lane the B columns l % 32 of both tiles.  Rows past M /
    // columns past N read the last valid one (their outputs are not stored).
    // (byte offsets into the scale tensors, read through buffer descriptors)
    uint32_t sa_off = 0u, sb_off[2] = {0u, 0u};
    __amdgpu_buffer_rsrc_t rss_a = rsa, rss_b = rsb;
    if constexpr (!GROUP_SUMS) {
        // over the block's rows / columns, like the code descriptors
        rss_a = __builtin_amdgcn_make_buffer_rsrc((void *)(act_scales + (size_t)m0 * NG), (short)0,
                                                  min(F6_BM, M - m0) * NG * 2, 0x00020000);
        rss_b = __builtin_amdgcn_make_buffer_rsrc((void *)(wgt_scales + (size_t)n0 * NG), (short)0,
                                                  min(F6_BN, N - n0) * NG * 2, 0x00020000);
        sa_off = (uint32_t)(min(wm * 64 + h * 32 + l32, M - 1 - m0) * NG * 2);
#pragma unroll
        for (int b = 0; b < 2; ++b) sb_off[b] = (uint32_t)(min(wn * 64 + b * 32 + l32, N - 1 - n0) * NG * 2);
    }
    // A operands keep the pair in the lanes of their row tile's half
    const uint32_t lanes_a1 = h ? 0xFFFFFFFFu : 0u;

    v16f acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

    // One group: fragments of group gg of the stage at st; pa: the P-MFMA A
    // operands of the stage (row tiles 0, 1), sb0, sb1: the B columns' bf16
    // pairs, g the group's index (group sums mode)
    auto compute = [&](const uint8_t *st, auto ggc, const v8bf (&pa)[2], uint32_t sb0, uint32_t sb1, int g) {
        constexpr int gg = decltype(ggc)::value;
        const int a8 = gg ? a8_1 : a8_0;
        v8i B[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const v4u qb = *(const v4u *)(st + bdelta + a16 + 48 * gg + t * 32 * F6_ROWB);
            const v2u db = *(const v2u *)(st + bdelta + a8 + t * 32 * F6_ROWB);
            B[t] = v8i{(int)qb[0], (int)qb[1], (int)qb[2], (int)qb[3], (int)db[0], (int)db[1], 0, 0};
        }
        // P-MFMA B operands: this group's half of the pair
        constexpr uint32_t half = gg ? 0xFFFF0000u : 0x0000FFFFu;
        v8bf pb[2];
        if constexpr (!GROUP_SUMS) {
            pb[0] = __builtin_bit_cast(v8bf, v4u{sb0 & half, 0u, 0u, 0u});
            pb[1] = __builtin_bit_cast(v8bf, v4u{sb1 & half, 0u, 0u, 0u});
        }
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            const v4u qa = *(const v4u *)(st + a16 + 48 * gg + a * 32 * F6_ROWB);
            const v2u da = *(const v2u *)(st + a8 + a * 32 * F6_ROWB);
            const v8i A = v8i{(int)qa[0], (int)qa[1], (int)qa[2], (int)qa[3], (int)da[0], (int)da[1], 0, 0};
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const v16f X = mfma_group_fp6(A, B[b]);
                if constexpr (GROUP_SUMS) {
                    const int col = n0 + wn * 64 + b * 32 + l32;
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int rowi = m0 + wm * 64 + a * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
                        if (g < NG && rowi < M && col < N) gsum[((size_t)rowi * N + col) * NG + g] = (int)X[i];
                    }
                } else {
                    const v16f z = {};
                    const v16f P = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[a], pb[b], z, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[a][b][i] = __builtin_fmaf(X[i], P[i], acc[a][b][i]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // the group's accumulation completes here (otherwise the unrolled
        // groups' products would be kept live and summed later)
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b) opaque(acc[a][b]);
    };

    // stage s (groups 2s, 2s+1) from buffer B (compile-time), scales as the
    // bf16 pairs of its two groups
    auto stage = [&](int s, auto bc, uint32_t sa, uint32_t sb0, uint32_t sb1) {
        constexpr int B = decltype(bc)::value;
        __builtin_amdgcn_sched_barrier(0);                    // stages stay in program order
        wait_vmcnt0();
        lds_barrier();
        if (s + 1 < NP) issue_pair(s + 1, B ^ 1);
        const uint8_t *st = smem + B * F6_STAGE;
        const v8bf pa[2] = {__builtin_bit_cast(v8bf, v4u{sa & ~lanes_a1, 0u, 0u, 0u}),
                            __builtin_bit_cast(v8bf, v4u{sa & lanes_a1, 0u, 0u, 0u})};
        compute(st, std::integral_constant<int, 0>{}, pa, sb0, sb1, 2 * s);
        compute(st, std::integral_constant<int, 1>{}, pa, sb0, sb1, 2 * s + 1);
    };

    issue_pair(0, 0);
    if constexpr (SC4) {
        // chunks of 4 groups (2 stages): the next chunk's scales are loaded at
        // the start of a chunk, two register sets alternating (the group sums
        // mode runs the same loop without scales)
        v2u sc[2][3] = {};
        auto load_sc = [&](int c, int set) {
            if constexpr (!GROUP_SUMS) {
                sc[set][0] = __builtin_bit_cast(v2u, __builtin_amdgcn_raw_buffer_load_b64(rss_a, sa_off, 2 * c, 0));
                sc[set][1] = __builtin_bit_cast(v2u, __builtin_amdgcn_raw_buffer_load_b64(rss_b, sb_off[0], 2 * c, 0));
                sc[set][2] = __builtin_bit_cast(v2u, __builtin_amdgcn_raw_buffer_load_b64(rss_b, sb_off[1], 2 * c, 0));
            }
        };
        load_sc(0, 0);
        auto chunk = [&](int c, auto setc) {
            constexpr int S = decltype(setc)::value;
            stage(c >> 1, std::integral_constant<int, 0>{}, sc[S][0][0], sc[S][1][0], sc[S][2][0]);
            if (c + 4 < NG) load_sc(c + 4, S ^ 1);
            stage((c >> 1) + 1, std::integral_constant<int, 1>{}, sc[S][0][1], sc[S][1][1], sc[S][2][1]);
        };
        for (int c = 0; c < NG; c += 8) {
            chunk(c, std::integral_constant<int, 0>{});
            if (c + 4 < NG) chunk(c + 4, std::integral_constant<int, 1>{});
        }
    } else {
        // any K/64: scales of a stage's two groups as 2-byte loads (zero past
        // the last group), loaded one stage ahead
        uint32_t sv[2][3];
        auto load_sv = [&](int s, int set) {
            const int g0 = 2 * s, g1 = 2 * s + 1;
            if constexpr (!GROUP_SUMS) {
                const uint16_t *sa_row = act_scales + (size_t)m0 * NG + sa_off / 2;
                sv[set][0] = (uint32_t)sa_row[g0] | (g1 < NG ? (uint32_t)sa_row[g1] << 16 : 0u);
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const uint16_t *sb_col = wgt_scales + (size_t)n0 * NG + sb_off[b] / 2;
                    sv[set][1 + b] = (uint32_t)sb_col[g0] | (g1 < NG ? (uint32_t)sb_col[g1] << 16 : 0u);
                }
            } else {
                sv[set][0] = sv[set][1] = sv[set][2] = 0u;
            }
        };
        load_sv(0, 0);
        for (int s = 0; s < NP; s += 2) {
            if (s + 1 < NP) load_sv(s + 1, 1);
            stage(s, std::integral_constant<int, 0>{}, sv[0][0], sv[0][1], sv[0][2]);
            if (s + 1 < NP) {
                if (s + 2 < NP) load_sv(s + 2, 0);
                stage(s + 1, std::integral_constant<int, 1>{}, sv[1][0], sv[1][1], sv[1][2]);
            }
        }
    }

    if constexpr (!GROUP_SUMS) {
        if constexpr (QK) {
            gemm_epilogue_sum(acc, alpha, M, N, rank, m0, n0, wm, wn, lane, lora_act, lora_up, bias);
            if (n0 < qk.qk_cols)   // block-uniform: a Q or K head
                gemm_epilogue_qk(acc, M, m0, n0, wm, wn, lane, qk, smem, N, out);
            else
                gemm_epilogue_store(acc, M, N, m0, n0, wm, wn, lane, out);
        } else {
            gemm_epilogue(acc, alpha, M, N, rank, m0, n0, wm, wn, lane, lora_act, lora_up, bias, out);
        }
    }
}

template <bool GROUP_SUMS, bool QK>
static hipError_t launch_fp6(int M, int N, int K, int rank, const void *act_codes, const void *act_scales,
                             const void *wgt_codes, const void *wgt_scales, float alpha, const float *lora_act,
                             const void *lora_up, const void *bias, void *out, int32_t *G, const QkNormRope &qk,
                             hipStream_t stream)
{
    dim3 grid(((N + F6_BN - 1) / F6_BN) * ((M + F6_BM - 1) / F6_BM)), block(F6_THREADS);
#define F6_LAUNCH(SC)                                                                                             \
    hipLaunchKernelGGL((gemm_w4a4_fp6_kernel<GROUP_SUMS, SC, QK>), grid, block, 0, stream, M, N, K, rank,        \
                       (const uint8_t *)act_codes, (const uint16_t *)act_scales, (const uint8_t *)wgt_codes,     \
                       (const uint16_t *)wgt_scales, alpha, lora_act, (const uint16_t *)lora_up,                  \
                       (const uint16_t *)bias, (uint16_t *)out, G, qk)
    if ((K >> 6) % 4 == 0)
        F6_LAUNCH(true);
    else
        F6_LAUNCH(false);
#undef F6_LAUNCH
    return hipGetLastError();
}

hipError_t launch_gemm_w4a4_fp6(int M, int N, int K, int rank, const void *act_codes, const void *act_scales,
                                const void *wgt_codes, const void *wgt_scales, float alpha, const float *lora_act,
                                const void *lora_up, const void *bias, void *out, hipStream_t stream)
{
    const QkNormRope none{};
    return launch_fp6<false, false>(M, N, K, rank, act_codes, act_scales, wgt_codes, wgt_scales, alpha, lora_act,
                                    lora_up, bias, out, nullptr, none, stream);
}

hipError_t launch_gemm_w4a4_fp6_qk(int M, int N, int K, int rank, const void *act_codes, const void *act_scales,
                                   const void *wgt_codes, const void *wgt_scales, float alpha,
                                   const float *lora_act, const void *lora_up, const void *bias,
                                   const QkNormRope &qk, void *out, hipStream_t stream)
{
    return launch_fp6<false, true>(M, N, K, rank, act_codes, act_scales, wgt_codes, wgt_scales, alpha, lora_act,
                                   lora_up, bias, out, nullptr, qk, stream);
}

// the GEMM's own main loop (same stages, copies and matrix instructions)
// writing X_g instead of accumulating
hipError_t launch_group_sums_fp6(int M, int N, int K, const void *act_codes, const void *wgt_codes, int32_t *G,
                                 hipStream_t stream)
{
    const QkNormRope none{};
    return launch_fp6<true, false>(M, N, K, 0, act_codes, nullptr, wgt_codes, nullptr, 1.0f, nullptr, nullptr,
                                   nullptr, nullptr, G, none, stream);
}

}  // namespace svdq
