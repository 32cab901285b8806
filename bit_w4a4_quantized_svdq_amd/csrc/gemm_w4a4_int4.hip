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
// group, and on CDNA4 the vector ALU is the scarce unit here (the loop is
// bound by vector instructions, not by the matrix core).  The scale outer
// product P_g = sx_g (x) sw_g is therefore formed on the matrix core as well:
// a bf16 v_mfma_f32_32x32x4_2b (two 32x32 blocks) whose only non-zero k slot
// holds sx (A: lane -> row, the same rows for both blocks) and sw (B: lane l
// -> column l of the wave's 64), i.e. P_g for the tiles (a,0) and (a,1) of a
// wave in one instruction.  A product of two bf16 values is exact in fp32, so
// P_g is exact and lands in the same 32x32 accumulator layout as G_g.  The
// vector ALU then does one int->float conversion and one fma per output and
// group.  The factor 2^-8 (from the 16*code operands) and alpha are applied
// once at the end.
//
// Data movement.  256 threads own a 128x128 output tile (4 waves of 64x64,
// each 2x2 tiles of 32x32); one K-step is one group of 64.  A 4-stage ring in
// LDS is filled with buffer loads that write LDS directly (no registers):
// per group 4 KB of A codes and 4 KB of B codes; the scales of 8 groups at a
// time into a two-slot ring.  Buffer descriptors hold the block's base, so a
// copy costs one scalar offset and one 32-bit lane offset.  Codes sit in LDS
// as [half][row][16 B], so the 16-byte fragment reads of a wave are
// contiguous and free of bank conflicts.  One barrier per group separates the
// consumers of a stage from its next refill.  When K/64 is a multiple of 8
// the loop runs in chunks of 8 groups (the scale-copy period) with every wait
// count and LDS offset a compile-time constant.  Blocks are mapped to tiles so
// that each XCD (own L2) walks a contiguous band of tiles in groups of 8
// M-tiles, keeping the A and B tiles in flight L2-resident.
//
// Epilogue.  acc * 2^-8 * alpha + bias in one fma, the low-rank up-projection
// on the matrix core (t split into bf16 hi + lo), packed hardware bf16
// conversion, and for a tile fully inside the output, 2-byte buffer stores
// whose row offsets are scalar.
#include "device_common.h"
#include "gemm_common.h"
#include "launch.h"

namespace svdq {
typedef short v4s __attribute__((ext_vector_type(4)));
typedef float v32f __attribute__((ext_vector_type(32)));

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
    for (int i = 0; i < 4; i += 2) {
        const uint64_t w = ((uint64_t)c[i + 1] << 32 | c[i]) << 4;   // one 64-bit shift for two dwords
        lo[i] = (int)((uint32_t)w & 0xF0F0F0F0u);
        lo[i + 1] = (int)((uint32_t)(w >> 32) & 0xF0F0F0F0u);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) hi[i] = (int)(c[i] & 0xF0F0F0F0u);
}

// SC16: scales copied 8 groups per 16-byte copy (K/64 a multiple of 8)
// QK: grouped QKV layer, per-head RMSNorm + rotary embedding of Q and K in
// the epilogue (gemm_epilogue_qk)
template <bool GROUP_SUMS, bool SC16, bool QK = false>
__global__ __launch_bounds__(G4_THREADS, GROUP_SUMS ? 2 : 3)
void gemm_w4a4_int4_kernel(int M, int N, int K, int rank,
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
    static_assert(G4_SMEM >= QK_SMEM, "the QK epilogue stages a 128-row tile in the operand LDS");
    __shared__ __attribute__((aligned(16))) uint8_t smem[G4_SMEM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, h = lane >> 5;
    const int nbm = (M + G4_BM - 1) / G4_BM, nbn = (N + G4_BN - 1) / G4_BN;
    int bm, bn;
    tile_of_block((int)blockIdx.x, nbm, nbn, G4_GROUP_M, bm, bn);
    const int m0 = bm * G4_BM, n0 = bn * G4_BN;
    const int NG = K >> 6;
    const int rowbytes = K >> 1;

    // Producer role.  Wave w copies LDS chunk w (1 KB) of the A codes and of the
    // B codes of every group: chunk j = half (j/2), rows 64*(j%2) .. +63, lane l
    // -> row 64*(j%2) + l.  Rows past M (columns past N) read a clamped, valid
    // row: they only feed outputs that are never stored.  Waves 0,1 also copy
    // the A scales of rows 64w .. 64w+63, waves 2,3 the B scales (8 groups
    // per copy with SC16).  Addresses are a block-uniform base (scalar
    // registers, advanced per group) plus a 32-bit per-lane offset; with
    // K <= 2^16 a block's 128 rows span less than 4 MB.
    const int p_half = wave >> 1, p_row = 64 * (wave & 1) + lane;
    const uint8_t *pa_base = act_codes + (size_t)m0 * rowbytes;
    const uint8_t *pb_base = wgt_codes + (size_t)n0 * rowbytes;
    const uint32_t pa_off = (uint32_t)(min(p_row, M - 1 - m0) * rowbytes + 16 * p_half);
    const uint32_t pb_off = (uint32_t)(min(p_row, N - 1 - n0) * rowbytes + 16 * p_half);
    const bool ps_is_a = wave < 2;
    const uint16_t *ps_base = nullptr;
    if constexpr (!GROUP_SUMS)
        ps_base = ps_is_a ? act_scales + (size_t)m0 * NG : wgt_scales + (size_t)n0 * NG;
    // buffer descriptors over the block's rows (uniform, scalar registers)
    const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
        (void *)pa_base, (short)0, min(G4_BM, M - m0) * rowbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
        (void *)pb_base, (short)0, min(G4_BN, N - n0) * rowbytes, 0x00020000);
    __amdgpu_buffer_rsrc_t rss = rsa;
    if constexpr (!GROUP_SUMS)
        rss = __builtin_amdgcn_make_buffer_rsrc((void *)ps_base, (short)0,
                                                 (ps_is_a ? min(G4_BM, M - m0) : min(G4_BN, N - n0)) * NG * 2,
                                                 0x00020000);
    auto issue_codes = [&](int g, int stage) {
        uint8_t *st = smem + stage * G4_STAGE + wave * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lptr_t)st, 16, pa_off, g * 32, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lptr_t)(st + G4_CODES), 16, pb_off, g * 32, 0, 0);
    };
    // The byte offset of this lane's scale row is that of the same clamped
    // row's codes divided by 16: pa_off / 16 (waves 0,1: row * K/2) or
    // (pb_off - 16) / 16 (waves 2,3: row * K/2 + 16).  It is derived where it
    // is used (opaque() keeps it from being hoisted into one more long-lived
    // register).
    // rows' scales of groups g .. g+7 into slot `slot`: [A rows | B rows][16 B]
    auto issue_scales8 = [&](int g, int slot) {
        uint32_t oa = pa_off, ob = pb_off;
        opaque(oa);
        opaque(ob);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rss,
            (lptr_t)(smem + G4_SC + slot * G4_SC_SLOT + (ps_is_a ? 0 : G4_BM * 16) + 1024 * (wave & 1)),
            16, (ps_is_a ? oa : ob - 16) >> 4, g * 2, 0, 0);
    };
    // group g's scales: [g % 8][A rows | B rows][4 B] (zero-extended 2-byte copies)
    auto issue_scales1 = [&](int g) {
        uint32_t oa = pa_off, ob = pb_off;
        opaque(oa);
        opaque(ob);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rss,
            (lptr_t)(smem + G4_SC + ((g >> 3) & 1) * G4_SC_SLOT + (g & 7) * (4 * (G4_BM + G4_BN)) +
                     (ps_is_a ? 0 : 4 * G4_BM) + 256 * (wave & 1)), 2, (ps_is_a ? oa : ob - 16) >> 4, g * 2, 0, 0);
    };

    v16f acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

    // consumer offsets inside a stage and inside a scale slot
    int a_off[2], b_off[2], sa_off[2], sb_off[2];
    // 2-block P operand B: lane l carries column wn*64 + l (block l/32)
    const int sb2_off = SC16 ? G4_BM * 16 + (wn * 64 + lane) * 16 : 4 * G4_BM + (wn * 64 + lane) * 4;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        a_off[t] = h * (G4_CODES / 2) + (wm * 64 + t * 32 + l32) * 16;
        b_off[t] = G4_CODES + h * (G4_CODES / 2) + (wn * 64 + t * 32 + l32) * 16;
        sa_off[t] = SC16 ? (wm * 64 + t * 32 + l32) * 16 : (wm * 64 + t * 32 + l32) * 4;
        sb_off[t] = SC16 ? G4_BM * 16 + (wn * 64 + t * 32 + l32) * 16 : 4 * G4_BM + (wn * 64 + t * 32 + l32) * 4;
    }

    // lds_barrier(): every wave has waited for its own copies of the group
    // about to be read, so after it all of that group is in LDS, and every
    // wave has finished reading the stage that the next copy overwrites.

    // One group: fragments from the stage at `st`, scales from `sc` (this
    // group's column of a scale slot), G_g on the integer matrix core.
    auto compute = [&](const uint8_t *st, const uint8_t *sc, int g) {
        v4u fa[2], fb[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            fa[t] = *(const v4u *)(st + a_off[t]);
            fb[t] = *(const v4u *)(st + b_off[t]);
        }
        v4i alo[2], ahi[2], blo[2], bhi[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) unpack_i8(fb[t], blo[t], bhi[t]);
        if constexpr (GROUP_SUMS) {
#pragma unroll
            for (int t = 0; t < 2; ++t) unpack_i8(fa[t], alo[t], ahi[t]);
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
            v4s pa_op[2], pb_op;
            {
                uint32_t sa[2], sb;
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    sa[t] = SC16 ? *(const uint16_t *)(sc + sa_off[t]) : *(const uint32_t *)(sc + sa_off[t]) & 0xFFFFu;
                sb = SC16 ? *(const uint16_t *)(sc + sb2_off) : *(const uint32_t *)(sc + sb2_off) & 0xFFFFu;
#pragma unroll
                for (int t = 0; t < 2; ++t) pa_op[t] = __builtin_bit_cast(v4s, v2u{sa[t], 0u});
                pb_op = __builtin_bit_cast(v4s, v2u{sb, 0u});
            }
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                unpack_i8(fa[a], alo[a], ahi[a]);   // the second row tile's operands only when needed
                // two 32x32 blocks: P for tiles (a,0) and (a,1)
                v32f P = {};
                P = __builtin_amdgcn_mfma_f32_32x32x4bf16_1k(pa_op[a], pb_op, P, 0, 0, 0);
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    v16i G = {};
                    G = __builtin_amdgcn_mfma_i32_32x32x32_i8(alo[a], blo[b], G, 0, 0, 0);
                    G = __builtin_amdgcn_mfma_i32_32x32x32_i8(ahi[a], bhi[b], G, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        acc[a][b][i] = __builtin_fmaf((float)G[i], P[16 * b + i], acc[a][b][i]);
                }
                __builtin_amdgcn_sched_barrier(0);   // at most 2 tiles of G, P live
            }
        }
    };

    if constexpr (SC16 && !GROUP_SUMS) {
        // K/64 is a multiple of 8: the loop runs over chunks of 8 groups, the
        // period of the scale copies, so that every wait count and every LDS
        // offset below is a compile-time constant.  Per wave, group g costs
        // two copies (codes), plus one (scales) when g % 8 == 0; waiting until
        // at most the copies of the two groups issued after g are in flight
        // means that g has landed.
        issue_codes(0, 0);
        issue_scales8(0, 0);
        issue_codes(1, 1);
        issue_codes(2, 2);
        for (int c = 0; c < NG; c += G4_SC_GROUPS) {
            const bool last = c + G4_SC_GROUPS == NG;
            const int par = (c >> 3) & 1;
            const uint8_t *slot = smem + G4_SC + par * G4_SC_SLOT;
#pragma unroll
            for (int j = 0; j < G4_SC_GROUPS; ++j) {
                __builtin_amdgcn_sched_barrier(0);            // groups stay in program order
                if (j < 6) wait_vmcnt(4);                   // groups c+j+1, c+j+2: codes only
                else if (j == 6) { if (last) wait_vmcnt(2); else wait_vmcnt(5); }
                else { if (last) wait_vmcnt(0); else wait_vmcnt(5); }
                lds_barrier();
                if (j < 5) {
                    issue_codes(c + j + 3, (j + 3) & 3);
                } else if (!last) {
                    issue_codes(c + j + 3, (j + 3) & 3);
                    if (j == 5) issue_scales8(c + G4_SC_GROUPS, par ^ 1);
                }
                compute(smem + (j & 3) * G4_STAGE, slot + 2 * j, c + j);
                // the group's accumulation completes here, before the next
                // barrier (otherwise the unrolled groups' products would be
                // kept live and summed later)
#pragma unroll
                for (int a = 0; a < 2; ++a)
#pragma unroll
                    for (int b = 0; b < 2; ++b) opaque(acc[a][b]);
            }
        }
    } else {
        // general loop: any K/64, and the group-sum mode (no scales)
        auto loads_of = [](int g) { return GROUP_SUMS ? 2 : 3; };
        auto issue = [&](int g) {
            issue_codes(g, g % G4_STAGES);
            if constexpr (!GROUP_SUMS) issue_scales1(g);
        };
        for (int g = 0; g < G4_STAGES - 1 && g < NG; ++g) issue(g);
        for (int g = 0; g < NG; ++g) {
            const int newer = min(G4_STAGES - 2, NG - 1 - g);
            wait_vmcnt(newer * loads_of(g));
            lds_barrier();
            if (g + G4_STAGES - 1 < NG) issue(g + G4_STAGES - 1);
            compute(smem + (g % G4_STAGES) * G4_STAGE,
                    smem + G4_SC + ((g >> 3) & 1) * G4_SC_SLOT + (g & 7) * (4 * (G4_BM + G4_BN)), g);
        }
    }

    if constexpr (!GROUP_SUMS) {
        // acc = 2^8 * sum_g G_g sx_g sw_g (the codes entered as 16*code)
        if constexpr (QK) {
            gemm_epilogue_sum(acc, alpha * 0.00390625f, M, N, rank, m0, n0, wm, wn, lane, lora_act, lora_up, bias);
            if (n0 < qk.qk_cols)   // block-uniform: a Q or K head
                gemm_epilogue_qk(acc, M, m0, n0, wm, wn, lane, qk, smem, N, out);
            else
                gemm_epilogue_store(acc, M, N, m0, n0, wm, wn, lane, out);
        } else {
            gemm_epilogue(acc, alpha * 0.00390625f, M, N, rank, m0, n0, wm, wn, lane, lora_act, lora_up, bias, out);
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
                           (int32_t *)nullptr, QkNormRope{});
    else
        hipLaunchKernelGGL((gemm_w4a4_int4_kernel<false, false>), grid, block, 0, stream, M, N, K, rank,
                           (const uint8_t *)act_codes, (const uint16_t *)act_scales,
                           (const uint8_t *)wgt_codes, (const uint16_t *)wgt_scales, alpha, lora_act,
                           (const uint16_t *)lora_up, (const uint16_t *)bias, (uint16_t *)out,
                           (int32_t *)nullptr, QkNormRope{});
    return hipGetLastError();
}

hipError_t launch_gemm_w4a4_int4_qk(int M, int N, int K, int rank, const void *act_codes,
                                    const void *act_scales, const void *wgt_codes,
                                    const void *wgt_scales, float alpha, const float *lora_act,
                                    const void *lora_up, const void *bias, const QkNormRope &qk,
                                    void *out, hipStream_t stream)
{
    dim3 grid(((N + G4_BN - 1) / G4_BN) * ((M + G4_BM - 1) / G4_BM)), block(G4_THREADS);
    if ((K >> 6) % G4_SC_GROUPS == 0)
        hipLaunchKernelGGL((gemm_w4a4_int4_kernel<false, true, true>), grid, block, 0, stream, M, N, K, rank,
                           (const uint8_t *)act_codes, (const uint16_t *)act_scales,
                           (const uint8_t *)wgt_codes, (const uint16_t *)wgt_scales, alpha, lora_act,
                           (const uint16_t *)lora_up, (const uint16_t *)bias, (uint16_t *)out,
                           (int32_t *)nullptr, qk);
    else
        hipLaunchKernelGGL((gemm_w4a4_int4_kernel<false, false, true>), grid, block, 0, stream, M, N, K, rank,
                           (const uint8_t *)act_codes, (const uint16_t *)act_scales,
                           (const uint8_t *)wgt_codes, (const uint16_t *)wgt_scales, alpha, lora_act,
                           (const uint16_t *)lora_up, (const uint16_t *)bias, (uint16_t *)out,
                           (int32_t *)nullptr, qk);
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
                       (const uint16_t *)nullptr, (uint16_t *)nullptr, G, QkNormRope{});
    return hipGetLastError();
}

}  // namespace svdq
