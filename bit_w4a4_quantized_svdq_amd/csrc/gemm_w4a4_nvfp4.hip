// gemm_w4a4_nvfp4.hip -- SVDQuant W4A4 GEMM, NVFP4 variant (E2M1 codes,
// E4M3 scales per 16 along K; "Nunchaku Lite" docs, "Supported quantization
// types": svdq_w4a4 nvfp4 group 16), with the low-rank up-projection and the
// bias in the epilogue.
//
// Mapping to CDNA4.  The block-scaled FP4 matrix instructions of gfx950
// take one power-of-two (E8M0) scale per 32 elements; NVFP4 carries one
// E4M3 scale (4-bit significand, not a power of two) per 16 elements, so no
// exact mapping onto them exists.  Instead both operands are dequantized
// exactly: an E2M1 value (at most 2 significant bits) times an E4M3 scale
// (at most 4) has at most 6 significant bits and lies in [2^-10, 2688], so
// it is exactly an fp16 normal number.  gfx950's v_cvt_scalef32_pk_f16_fp4
// turns one byte (two E2M1 codes) into two fp16 values (its scale operand
// only contributes a power of two, so it is left at 1), and one packed fp16
// multiply applies the group scale: one vector instruction per element.
// v_cvt_scalef32_pk_f16_fp8 turns two E4M3 scale bytes into fp16 (exact for
// all 256 codes).  The products in v_mfma_f32_32x32x16_f16 are exact; only
// the fp32 accumulation rounds.  alpha multiplies the 4-bit term at the end.
//
// Data movement follows the int4 kernel: 256 threads own a 128x128 output
// tile (4 waves of 64x64); one K-step is a 64-wide slice (4 scale groups).
// A 4-stage LDS ring is filled with buffer loads that write LDS directly:
// per slice 4 KB of A codes and 4 KB of B codes as [half][row][16 B], so a
// lane's 16-byte fragment holds 32 consecutive k of one row.  Each wave
// dequantizes its own fragments in registers (each element is converted by
// the two waves that share its row or column) and feeds them to the matrix
// core: per slice and wave 128 vector instructions against 16 MFMAs.  A
// dot product does not depend on the order of k, so lane half h takes k =
// 32h .. 32h+31 of the slice and MFMA step s its k = 32h + 8s .. +7, for A
// and B alike.
//
// Copies.  A copy instruction moves 64 lanes x 16 bytes; the vector memory
// path handles it per distinct cache line, so 16 bytes from each of 64 rows
// (one slice) costs four times the address work of 64 bytes from each of 16
// rows.  When K is a multiple of 512 (the main path) a stage therefore holds
// two slices, 64 bytes of every row, the scales travel 8 slices (32 bytes per
// row) at a time, and two stages alternate with one barrier per stage.
// Otherwise a 4-stage ring of single slices is used: when K is a multiple of
// 256 its scales travel 4 slices at a time (16 bytes per row) with
// compile-time wait counts, else each slice's 4 scale bytes per row are
// copied on their own.
#include "device_common.h"
#include "gemm_common.h"
#include "launch.h"

namespace svdq {

constexpr int NV_BM = 128, NV_BN = 128, NV_THREADS = 256, NV_STAGES = 4;
constexpr int NV_CODES = NV_BM * 32;                  // bytes of A (or B) codes per slice
constexpr int NV_STAGE = 2 * NV_CODES;                // 8 KB
constexpr int NV_SC_SLICES = 4;                       // slices per 16-byte scale copy
constexpr int NV_SC_SLOT = (NV_BM + NV_BN) * 16;      // 4 KB: [A rows | B rows][16 B]
constexpr int NV_SC = NV_STAGES * NV_STAGE;           // offset of the two scale slots
constexpr int NV_SMEM = NV_SC + 2 * NV_SC_SLOT;       // 40 KB
constexpr int NV_GROUP_M = 8;

typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// SC4: scales copied 4 slices (16 bytes per row) at a time (K a multiple of 256)
// QK: grouped QKV layer, per-head RMSNorm + rotary embedding of Q and K in
// the epilogue (gemm_epilogue_qk)
template <bool SC4, bool QK = false>
__global__ __launch_bounds__(NV_THREADS, 2)
void gemm_w4a4_nvfp4_kernel(int M, int N, int K, int rank,
                            const uint8_t *__restrict__ act_codes,
                            const uint8_t *__restrict__ act_scales,
                            const uint8_t *__restrict__ wgt_codes,
                            const uint8_t *__restrict__ wgt_scales, float alpha,
                            const float *__restrict__ lora_act,
                            const uint16_t *__restrict__ lora_up,
                            const uint16_t *__restrict__ bias, uint16_t *__restrict__ out,
                            QkNormRope qk)
{
    static_assert(NV_SMEM >= QK_SMEM, "the QK epilogue stages a 128-row tile in the operand LDS");
    __shared__ __attribute__((aligned(16))) uint8_t smem[NV_SMEM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, h = lane >> 5;
    const int nbm = (M + NV_BM - 1) / NV_BM, nbn = (N + NV_BN - 1) / NV_BN;
    int bm, bn;
    tile_of_block((int)blockIdx.x, nbm, nbn, NV_GROUP_M, bm, bn);
    const int m0 = bm * NV_BM, n0 = bn * NV_BN;
    const int NS = K >> 6;                            // slices
    const int rowbytes = K >> 1;
    const int NG16 = K >> 4;                          // scale bytes per row

    // Producer role (as in the int4 kernel): wave w copies LDS chunk w (1 KB)
    // of the A and of the B codes of every slice, lane l -> row 64*(w%2) + l,
    // half w/2; rows past M (columns past N) read a clamped valid row whose
    // outputs are never stored.  Waves 0,1 copy the A scales of their 64
    // rows, waves 2,3 the B scales.
    const int p_half = wave >> 1, p_row = 64 * (wave & 1) + lane;
    const uint8_t *pa_base = act_codes + (size_t)m0 * rowbytes;
    const uint8_t *pb_base = wgt_codes + (size_t)n0 * rowbytes;
    const uint32_t pa_off = (uint32_t)(min(p_row, M - 1 - m0) * rowbytes + 16 * p_half);
    const uint32_t pb_off = (uint32_t)(min(p_row, N - 1 - n0) * rowbytes + 16 * p_half);
    const bool ps_is_a = wave < 2;
    const uint8_t *ps_base = ps_is_a ? act_scales + (size_t)m0 * NG16 : wgt_scales + (size_t)n0 * NG16;
    const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
        (void *)pa_base, (short)0, min(NV_BM, M - m0) * rowbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
        (void *)pb_base, (short)0, min(NV_BN, N - n0) * rowbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rss = __builtin_amdgcn_make_buffer_rsrc(
        (void *)ps_base, (short)0, (ps_is_a ? min(NV_BM, M - m0) : min(NV_BN, N - n0)) * NG16, 0x00020000);
    auto issue_codes = [&](int g, int stage) {
        uint8_t *st = smem + stage * NV_STAGE + wave * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lptr_t)st, 16, pa_off, g * 32, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lptr_t)(st + NV_CODES), 16, pb_off, g * 32, 0, 0);
    };
    // This lane's scale row starts at byte row * K/16 = (its code offset) / 8
    // (waves 2,3 copy the second code half: subtract its 16 bytes first).
    // Scales of slices g .. g+3 into slot `slot`: [A rows | B rows][16 B].
    auto issue_scales4 = [&](int g, int slot) {
        uint32_t oa = pa_off, ob = pb_off;
        opaque(oa);
        opaque(ob);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rss,
            (lptr_t)(smem + NV_SC + slot * NV_SC_SLOT + (ps_is_a ? 0 : NV_BM * 16) + 1024 * (wave & 1)),
            16, (ps_is_a ? oa : ob - 16) >> 3, g * 4, 0, 0);
    };
    // Scales of slice g alone into entry g % 4 of a ring of 1 KB entries,
    // each [A rows | B rows][4 B] (one entry per code stage in flight).
    auto issue_scales1 = [&](int g) {
        uint32_t oa = pa_off, ob = pb_off;
        opaque(oa);
        opaque(ob);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rss,
            (lptr_t)(smem + NV_SC + (g % NV_STAGES) * 1024 + (ps_is_a ? 0 : NV_BM * 4) + 256 * (wave & 1)),
            4, (ps_is_a ? oa : ob - 16) >> 3, g * 4, 0, 0);
    };

    v16f acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

    // consumer offsets: fragments in a stage, scale pairs in a slot
    int a_off[2], b_off[2], sa_off[2], sb_off[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int ra = wm * 64 + t * 32 + l32, rb = wn * 64 + t * 32 + l32;
        a_off[t] = h * (NV_CODES / 2) + ra * 16;
        b_off[t] = NV_CODES + h * (NV_CODES / 2) + rb * 16;
        // the lane's two groups of a slice are 2h, 2h+1: one 2-byte read
        sa_off[t] = (SC4 ? ra * 16 : ra * 4) + 2 * h;
        sb_off[t] = (SC4 ? (NV_BM + rb) * 16 : (NV_BM + rb) * 4) + 2 * h;
    }

    // one slice: dequantize this wave's fragments step by step and run the MFMAs
    auto compute = [&](const uint8_t *st, const uint8_t *sc) {
        v4u fa[2], fb[2];
        v2h sa[2], sb[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            fa[t] = *(const v4u *)(st + a_off[t]);
            fb[t] = *(const v4u *)(st + b_off[t]);
            // two E4M3 scales -> fp16 {group 2h, group 2h+1}
            sa[t] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(*(const uint16_t *)(sc + sa_off[t]), 1.0f, false);
            sb[t] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(*(const uint16_t *)(sc + sb_off[t]), 1.0f, false);
        }
        // dword s of a fragment: k = 32h + 8s .. +7, group 2h + s/2
        auto deq = [](uint32_t c, v2h sc2, int s) {
            const v2h f = (s < 2) ? v2h{sc2[0], sc2[0]} : v2h{sc2[1], sc2[1]};
            v4u o;
            o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 0) * f);
            o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 1) * f);
            o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 2) * f);
            o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 3) * f);
            return __builtin_bit_cast(v8h, o);
        };
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            v8h av[2], bv[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                av[t] = deq(fa[t][s], sa[t], s);
                bv[t] = deq(fb[t][s], sb[t], s);
            }
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[a], bv[b], acc[a][b], 0, 0, 0);
        }
    };

    if constexpr (SC4) {
        // Per wave, slice g costs two copies (codes), plus one (scales) when
        // g % 4 == 0; waiting until at most the copies of the two slices
        // issued after g are in flight means that g has landed.
        issue_codes(0, 0);
        issue_scales4(0, 0);
        issue_codes(1, 1);
        issue_codes(2, 2);
        for (int c = 0; c < NS; c += NV_SC_SLICES) {
            const bool last = c + NV_SC_SLICES == NS;
            const int par = (c >> 2) & 1;
            const uint8_t *slot = smem + NV_SC + par * NV_SC_SLOT;
#pragma unroll
            for (int j = 0; j < NV_SC_SLICES; ++j) {
                __builtin_amdgcn_sched_barrier(0);            // slices stay in program order
                if (j < 2) wait_vmcnt(4);                     // slices c+j+1, c+j+2: codes only
                else if (j == 2) { if (last) wait_vmcnt(2); else wait_vmcnt(5); }
                else { if (last) wait_vmcnt(0); else wait_vmcnt(5); }
                lds_barrier();
                if (j == 0) {
                    issue_codes(c + 3, 3);
                } else if (!last) {
                    issue_codes(c + j + 3, (j + 3) & 3);
                    if (j == 1) issue_scales4(c + NV_SC_SLICES, par ^ 1);
                }
                compute(smem + j * NV_STAGE, slot + 4 * j);
                // the slice's accumulation completes before the next barrier
#pragma unroll
                for (int a = 0; a < 2; ++a)
#pragma unroll
                    for (int b = 0; b < 2; ++b) opaque(acc[a][b]);
            }
        }
    } else {
        auto issue = [&](int g) {
            issue_codes(g, g % NV_STAGES);
            issue_scales1(g);
        };
        for (int g = 0; g < NV_STAGES - 1 && g < NS; ++g) issue(g);
        for (int g = 0; g < NS; ++g) {
            const int newer = min(NV_STAGES - 2, NS - 1 - g);
            wait_vmcnt(3 * newer);
            lds_barrier();
            if (g + NV_STAGES - 1 < NS) issue(g + NV_STAGES - 1);
            compute(smem + (g % NV_STAGES) * NV_STAGE, smem + NV_SC + (g % NV_STAGES) * 1024);
        }
    }

    gemm_epilogue_any<QK>(acc, alpha, M, N, rank, m0, n0, wm, wn, lane, lora_act, lora_up, bias, out, qk, smem);
}

// Main path (K a multiple of 512): a stage holds two slices, 64 bytes of
// every row, so each copy instruction reads 16 rows x 64 B (four lanes per
// row).  Within a row's 64 bytes the four 16-byte chunks are stored in the
// order c ^ co_swz(row), co_swz(row) = ((row >> 1) & 3) ^ ((row >> 3) & 1):
// the 16 consecutive rows whose 16-byte fragments one LDS cycle serves (64
// banks of 4 bytes) then fall on distinct banks, and so do any 8 of them
// that are consecutive.  (The swizzle (row >> 1) & 3 alone leaves rows r
// and r + 8 on the same banks: the LDS bank-conflict counter read 74 % of
// the LDS-active cycles with it.)
constexpr int CO_ROWB = 64;                               // bytes per row and stage
constexpr int CO_CODES = NV_BM * CO_ROWB;                 // 8 KB of A (or B) codes per stage
constexpr int CO_STAGE = 2 * CO_CODES;                    // 16 KB
constexpr int CO_SC_ROWB = 32;                            // scale bytes per row and chunk (8 slices)
constexpr int CO_SC_SLOT = (NV_BM + NV_BN) * CO_SC_ROWB;  // 8 KB
constexpr int CO_SC = 2 * CO_STAGE;
constexpr int CO_SMEM = CO_SC + 2 * CO_SC_SLOT;           // 48 KB

__device__ __forceinline__ int co_swz(int row) { return ((row >> 1) & 3) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int co_chunk_slot(int row, int c) { return c ^ co_swz(row); }

template <bool QK = false>
__global__ __launch_bounds__(NV_THREADS, 2)
void gemm_w4a4_nvfp4_co_kernel(int M, int N, int K, int rank,
                               const uint8_t *__restrict__ act_codes,
                               const uint8_t *__restrict__ act_scales,
                               const uint8_t *__restrict__ wgt_codes,
                               const uint8_t *__restrict__ wgt_scales, float alpha,
                               const float *__restrict__ lora_act,
                               const uint16_t *__restrict__ lora_up,
                               const uint16_t *__restrict__ bias, uint16_t *__restrict__ out,
                               QkNormRope qk)
{
    static_assert(CO_SMEM >= QK_SMEM, "the QK epilogue stages a 128-row tile in the operand LDS");
    __shared__ __attribute__((aligned(16))) uint8_t smem[CO_SMEM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, h = lane >> 5;
    const int nbm = (M + NV_BM - 1) / NV_BM, nbn = (N + NV_BN - 1) / NV_BN;
    int bm, bn;
    tile_of_block((int)blockIdx.x, nbm, nbn, NV_GROUP_M, bm, bn);
    const int m0 = bm * NV_BM, n0 = bn * NV_BN;
    const int NP = K >> 7;                            // stages of two slices
    const int rowbytes = K >> 1;
    const int NG16 = K >> 4;
    const int rows_a = min(NV_BM, M - m0), rows_b = min(NV_BN, N - n0);

    // copies of codes: wave w issues instructions w and w + 4 of A and of B
    // (16 rows each); lane i -> row 16q + i/4, LDS slot i % 4, chunk c.
    uint32_t ca_off[2], cb_off[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int q = wave + 4 * u, r = 16 * q + (lane >> 2), c = co_chunk_slot(r, lane & 3);
        ca_off[u] = (uint32_t)(min(r, rows_a - 1) * rowbytes + 16 * c);
        cb_off[u] = (uint32_t)(min(r, rows_b - 1) * rowbytes + 16 * c);
    }
    // copies of scales: 256 rows [A | B] x 32 B per chunk; wave w issues
    // instructions 2w, 2w+1 (32 rows each): lane i -> row 32q + i/2, half i%2
    const bool ps_is_a = wave < 2;
    uint32_t s_off[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int q = 2 * wave + u, r = 32 * q + (lane >> 1) - (ps_is_a ? 0 : NV_BM);
        s_off[u] = (uint32_t)(min(r, (ps_is_a ? rows_a : rows_b) - 1) * NG16 + 16 * (lane & 1));
    }
    const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(act_codes + (size_t)m0 * rowbytes), (short)0, rows_a * rowbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(wgt_codes + (size_t)n0 * rowbytes), (short)0, rows_b * rowbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rss = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(ps_is_a ? act_scales + (size_t)m0 * NG16 : wgt_scales + (size_t)n0 * NG16), (short)0,
        (ps_is_a ? rows_a : rows_b) * NG16, 0x00020000);
    auto issue_codes = [&](int p) {
        uint8_t *st = smem + (p & 1) * CO_STAGE;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lptr_t)(st + (wave + 4 * u) * 1024), 16, ca_off[u], p * CO_ROWB, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lptr_t)(st + CO_CODES + (wave + 4 * u) * 1024), 16, cb_off[u], p * CO_ROWB, 0, 0);
        }
    };
    auto issue_scales = [&](int ch) {
        uint8_t *sl = smem + CO_SC + (ch & 1) * CO_SC_SLOT;
#pragma unroll
        for (int u = 0; u < 2; ++u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rss, (lptr_t)(sl + (2 * wave + u) * 1024), 16, s_off[u], ch * CO_SC_ROWB, 0, 0);
    };

    v16f acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

    // consumer offsets: for slice-in-stage s, fragment of tile t at
    // row * 64 + 16 * slot(row, 2s + h); scale pair at row * 32 + 4 * slice + 2h
    int a_row[2], b_row[2], a_sw[2], b_sw[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        a_row[t] = wm * 64 + t * 32 + l32;
        b_row[t] = wn * 64 + t * 32 + l32;
        a_sw[t] = co_swz(a_row[t]);
        b_sw[t] = co_swz(b_row[t]);
    }

    auto deq = [](uint32_t c, v2h sc2, int s) {
        const v2h f = (s < 2) ? v2h{sc2[0], sc2[0]} : v2h{sc2[1], sc2[1]};
        v4u o;
        o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 0) * f);
        o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 1) * f);
        o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 2) * f);
        o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 3) * f);
        return __builtin_bit_cast(v8h, o);
    };
    // slice si (0, 1) of the stage at st; its scales at slice index ss of slot sc
    auto compute = [&](const uint8_t *st, const uint8_t *sc, int si, int ss) {
        v4u fa[2], fb[2];
        v2h sa[2], sb[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            fa[t] = *(const v4u *)(st + a_row[t] * CO_ROWB + 16 * ((2 * si + h) ^ a_sw[t]));
            fb[t] = *(const v4u *)(st + CO_CODES + b_row[t] * CO_ROWB + 16 * ((2 * si + h) ^ b_sw[t]));
            sa[t] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(
                *(const uint16_t *)(sc + a_row[t] * CO_SC_ROWB + 4 * ss + 2 * h), 1.0f, false);
            sb[t] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(
                *(const uint16_t *)(sc + (NV_BM + b_row[t]) * CO_SC_ROWB + 4 * ss + 2 * h), 1.0f, false);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            v8h av[2], bv[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                av[t] = deq(fa[t][s], sa[t], s);
                bv[t] = deq(fb[t][s], sb[t], s);
            }
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[a], bv[b], acc[a][b], 0, 0, 0);
        }
    };

    // Stage p: wait for its copies (issued one iteration earlier), barrier
    // (every wave is past stage p-1, whose buffer receives stage p+1), issue
    // stage p+1 and, at the first stage of a scale chunk, the next chunk's
    // scales into the other slot (its previous chunk is finished).  Only the
    // copies of that chunk may still be in flight at the next wait.
    issue_scales(0);
    issue_codes(0);
    for (int p = 0; p < NP; ++p) {
        __builtin_amdgcn_sched_barrier(0);
        if ((p & 3) == 1 && (p >> 2) + 1 < (NP >> 2)) wait_vmcnt(2);
        else wait_vmcnt(0);
        lds_barrier();
        if (p + 1 < NP) issue_codes(p + 1);
        if ((p & 3) == 0 && (p >> 2) + 1 < (NP >> 2)) issue_scales((p >> 2) + 1);
        const uint8_t *st = smem + (p & 1) * CO_STAGE;
        const uint8_t *sc = smem + CO_SC + ((p >> 2) & 1) * CO_SC_SLOT;
        compute(st, sc, 0, 2 * (p & 3));
        compute(st, sc, 1, 2 * (p & 3) + 1);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b) opaque(acc[a][b]);
    }

    gemm_epilogue_any<QK>(acc, alpha, M, N, rank, m0, n0, wm, wn, lane, lora_act, lora_up, bias, out, qk, smem);
}

template <bool QK>
static hipError_t launch_nvfp4(int M, int N, int K, int rank, const void *act_codes, const void *act_scales,
                               const void *wgt_codes, const void *wgt_scales, float alpha, const float *lora_act,
                               const void *lora_up, const void *bias, const QkNormRope &qk, void *out,
                               hipStream_t stream)
{
    dim3 grid(((N + NV_BN - 1) / NV_BN) * ((M + NV_BM - 1) / NV_BM)), block(NV_THREADS);
    if (K % 512 == 0)
        hipLaunchKernelGGL((gemm_w4a4_nvfp4_co_kernel<QK>), grid, block, 0, stream, M, N, K, rank,
                           (const uint8_t *)act_codes, (const uint8_t *)act_scales,
                           (const uint8_t *)wgt_codes, (const uint8_t *)wgt_scales, alpha, lora_act,
                           (const uint16_t *)lora_up, (const uint16_t *)bias, (uint16_t *)out, qk);
    else if (K % 256 == 0)
        hipLaunchKernelGGL((gemm_w4a4_nvfp4_kernel<true, QK>), grid, block, 0, stream, M, N, K, rank,
                           (const uint8_t *)act_codes, (const uint8_t *)act_scales,
                           (const uint8_t *)wgt_codes, (const uint8_t *)wgt_scales, alpha, lora_act,
                           (const uint16_t *)lora_up, (const uint16_t *)bias, (uint16_t *)out, qk);
    else
        hipLaunchKernelGGL((gemm_w4a4_nvfp4_kernel<false, QK>), grid, block, 0, stream, M, N, K, rank,
                           (const uint8_t *)act_codes, (const uint8_t *)act_scales,
                           (const uint8_t *)wgt_codes, (const uint8_t *)wgt_scales, alpha, lora_act,
                           (const uint16_t *)lora_up, (const uint16_t *)bias, (uint16_t *)out, qk);
    return hipGetLastError();
}

hipError_t launch_gemm_w4a4_nvfp4(int M, int N, int K, int rank, const void *act_codes,
                                  const void *act_scales, const void *wgt_codes,
                                  const void *wgt_scales, float alpha, const float *lora_act,
                                  const void *lora_up, const void *bias, void *out,
                                  hipStream_t stream)
{
    return launch_nvfp4<false>(M, N, K, rank, act_codes, act_scales, wgt_codes, wgt_scales, alpha, lora_act,
                               lora_up, bias, QkNormRope{}, out, stream);
}

hipError_t launch_gemm_w4a4_nvfp4_qk(int M, int N, int K, int rank, const void *act_codes,
                                     const void *act_scales, const void *wgt_codes,
                                     const void *wgt_scales, float alpha, const float *lora_act,
                                     const void *lora_up, const void *bias, const QkNormRope &qk,
                                     void *out, hipStream_t stream)
{
    return launch_nvfp4<true>(M, N, K, rank, act_codes, act_scales, wgt_codes, wgt_scales, alpha, lora_act,
                              lora_up, bias, qk, out, stream);
}

}  // namespace svdq
