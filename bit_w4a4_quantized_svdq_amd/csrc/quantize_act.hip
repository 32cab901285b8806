// quantize_act.hip -- first fused step of the SVDQuant W4A4 layer on gfx950:
// smoothing, 16-bit low-rank down-projection and per-group 4-bit
// quantization in one pass over the activations (blog "Hugging Face
// integrates Nunchaku 4-bit diffusion inference into Diffusers", section
// "SVDQuant and the Nunchaku engine": the low-rank down-projection is fused
// into the quantize kernel so the 16-bit branch adds no extra pass over x).
//
// Work split: a block owns 16 rows; its 8 waves take the K-groups of 64 in
// turn (wave w: groups w, w+8, ...).  Lane l of a wave holds row l%16 and the
// 8-element slices 8*(l/16) and 32+8*(l/16) of the group -- exactly the
// A-operand layout of v_mfma_f32_16x16x32_bf16, so the smoothed bf16 values
// feed the matrix core for x_hat . L1^T straight from registers, and the same
// registers give the group absmax (a max over the 4 lanes of a row).  x is
// read from HBM once.
//
// Exactness (codes and scales must equal the reference rule bit for bit):
//  * x_hat = RNE_bf16(fl32(x / s)) is computed as RNE_bf16(x * fl32(1/s)).
//    Both operands are bf16 (8-bit significands), so a quotient that is not
//    itself a bf16 midpoint lies at least 2^-17 (relative) from every
//    midpoint, far beyond the 2^-23 error of the product; a quotient can only
//    BE a midpoint when the result is below 2^-126 (a bf16 subnormal), and
//    such lanes (fp32-subnormal products) are recomputed with IEEE division,
//    as are channels whose 1/s would leave fp32's normal range.
//  * Group scales: absmax * fl32(1/7) (int4) and absmax * fl32(1/6) (NVFP4)
//    give, after the scale's own rounding to bf16 resp. E4M3, the same
//    result as the division for every bf16 absmax (checked exhaustively).
//  * int4: q = RNE(x_hat / scale).  The quotient is formed as one Newton
//    step on the hardware reciprocal inv (v_rcp_f32, within 1 ulp):
//    qe = x*inv; r = fma(-qe, scale, x) is exact; q = fma(r, inv, qe) is
//    within ~2^-45 (relative) of the exact quotient, so it IS the exact value
//    whenever the exact quotient is a half-integer, while a non-tie quotient
//    of two bf16 values is at least 2^-10 from a half-integer.  Rounding to
//    the nearest integer (ties to even) then happens in an fp32 add of 2^23
//    (or in v_rndne_f32), and byte permutes pack the nibbles.
//  * NVFP4: the E2M1 code of v = x_hat/d is rint(min(2|v|, |v|+2, |v|/2+4))
//    clamped to 7 -- the piecewise-linear map that sends the E2M1 grid
//    {0,.5,1,1.5,2,3,4,6} onto 0..7, so round-to-nearest-even on it gives the
//    nearest value with ties to the even code.  v comes from the same Newton
//    step; ties are exact and non-ties stay 2^-11 (relative) away.
//
// FP6 tiled layout (PREC 2, int4 codes for the FP6 GEMM): the same codes q
// in [-8, 7], written as E2M3 values q/2 (exact: every integer up to 8 has
// at most three significant bits) in the operand layout of the gfx950
// block-scaled matrix instruction.  Per row and group of 64, two 192-bit
// strings, one per K-half h: field j (bits 6j .. 6j+5) is the code of
// channel 32h + j; as three 16-byte chunks [h0 dwords 0-3 | h1 dwords 0-3 |
// h0 dwords 4-5, h1 dwords 4-5], so a GEMM lane reads its 24 bytes as one
// 16-byte and one 8-byte piece.  Rows are stored in tiles of 128 and groups
// in pairs, each (tile, pair) a contiguous 12 KB image of the GEMM's LDS
// stage (fp6_tiled_chunk): the GEMM copies it with whole-line loads.
// A lane converts its 16 codes with one v_cvt_scalef32_2xpk16_fp6_f32 (two
// 16-value sources whose fields interleave: field 2i from the first, 2i+1
// from the second; the scale divides, so 2.0 turns q into q/2), giving its
// 48 bits of each half; two lane swaps (v_permlane16_swap,
// v_permlane32_swap) gather a whole half string in each lane, and one store
// per lane writes a 16- or 8-byte piece.
//
// GELU variant (a layer fed by a GELU MLP's up projection): x is first
// mapped through GELU (tanh form) of bf16 to bf16, exact by construction
// (gelu_bf16.h: a 10.5 KB table built at compile time, which each block
// copies into LDS, plus exact rules outside the table's range); everything
// after it is unchanged.
#include <type_traits>

#include "device_common.h"
#include "gelu_bf16.h"
#include "launch.h"

namespace svdq {

constexpr int QA_ROWS = 16;          // rows per block (one MFMA row tile)
// waves per block: 16 (four per SIMD) for ranks up to 16, else 8 (the
// low-rank partials of all waves are reduced in LDS), and 12 at rank 17-32
// for the GELU variants and NVFP4.  Both int4 outputs (nibbles and the FP6
// layout) take the same count, so that their low-rank sums agree bit for bit.  A block's time is the latency of its waves' group
// sequences (one block per CU), so more waves per block shorten it where the
// registers allow: at rank 32 the GELU variants fit 12 waves (3 per SIMD,
// 168 registers) without spilling.  Measured at 4096 rows against 8 waves
// (int4 nibbles / NVFP4 / FP6 codes): K = 12288 51.1 / 56.0 / 52.2 against
// 53.0 / 63.0 / 57.1 us, K = 3072 18.4 / 19.9 / 18.8 against 19.2 / 21.6 /
// 19.8 us.  Without GELU, with the whole-line x loads: NVFP4 at K = 3072
// 14.0 against 14.7 us, at K = 12288 43.0 against 45.5 us; the FP6 variant
// spilled at 12 waves (14.6 against 13.7 us), so both int4 variants keep 8
// (nibbles: 12.7 either way at K = 3072, 40.8 against 41.7 at K = 12288).
// 16 waves at rank 32 (128 registers) spill.
template <int PREC, int RT, bool GELU> constexpr int qa_waves() {
    return RT <= 1 && !GELU ? 16 : (RT == 2 && (GELU || PREC == 1) ? 12 : 8);
}
// K-groups whose 1/s is staged in LDS at a time: 8 channels per thread
template <int PREC, int RT, bool GELU> constexpr int qa_chunk() { return qa_waves<PREC, RT, GELU>() * 8; }
constexpr int QA_XDEPTH = 2;         // x slices in flight per wave (groups ahead)
// Whole-line x loads (8- and 12-wave blocks): a group's 16 rows x 128 bytes are
// loaded as 8 rows x 128 B per instruction (lane i: row 8j + i/8, 16-byte
// chunk i % 8), so every load instruction moves whole cache lines, and one
// LDS pass per wave puts them into the MFMA layout (lane l: row l % 16,
// chunks l/16 and l/16 + 4).  Loading the MFMA layout directly touches each
// line with two instructions (64 of its 128 bytes each); the vector memory
// path is what this kernel waits on.  Measured against the direct loads
// (same outputs byte for byte): 14.2 against 15.5 us at K = 3072 and 43.8
// against 50.1 us at K = 12288 (4096 rows, rank 32, FP6 codes); the
// GELU-fed step was 2 % slower with it and keeps the direct loads, as do
// ranks above 64 (whose three-slot low-rank ring would spill).
template <int PREC, int RT, bool GELU> constexpr bool qa_lds_x() {
    return (qa_waves<PREC, RT, GELU>() == 8 || qa_waves<PREC, RT, GELU>() == 12) && RT <= 4 && !GELU;
}
constexpr int QA_XSLOT = QA_ROWS * 128;      // bytes of one group's x slice
constexpr int QA_PERIOD = 3;         // unroll period: a multiple of both ring sizes (3, and 3 or 1)

__device__ __forceinline__ float v4u_elem(const v4u &v, int e) {
    // element e (0..7) of 8 packed bf16
    uint32_t w = v[e >> 1];
    return (e & 1) ? bf16_hi(w) : bf16_lo(w);
}

struct F16 { float v[16]; };

// Eight quotients clamped to [-8, 7], rounded to the nearest integer (ties
// to even) and packed as two's-complement nibbles, element e in nibble e.
// Even elements: the fp32 add of 2^23 + 8 rounds and leaves q + 8 in the low
// byte; odd ones are rounded first, then 16 q + 2^23 + 128 leaves 16 (q + 8)
// in the low byte.  Byte permutes gather the low bytes, and the final xor
// turns q + 8 into q mod 16.
__device__ __forceinline__ uint32_t pack_int4_word(const float (&q)[8]) {
    uint32_t t[8];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        t[e] = __float_as_uint(q[e] + 8388616.0f);                                             // 2^23 + 8
        t[e + 1] = __float_as_uint(__builtin_fmaf(__builtin_rintf(q[e + 1]), 16.0f, 8388736.0f));   // 2^23 + 128
    }
    // v_perm_b32: selector bytes 0-3 pick bytes of the second operand, 4-7 of the first, 0x0C gives 0
    const uint32_t lo = __builtin_amdgcn_perm(t[2], t[0], 0x0C0C0400u) | __builtin_amdgcn_perm(t[6], t[4], 0x04000C0Cu);
    const uint32_t hi = __builtin_amdgcn_perm(t[3], t[1], 0x0C0C0400u) | __builtin_amdgcn_perm(t[7], t[5], 0x04000C0Cu);
    return (lo | hi) ^ 0x88888888u;
}

// Rare paths, kept out of line so that the unrolled main loop stays small.
// Smoothing by IEEE fp32 division, for lanes whose fast product is an fp32
// subnormal and for channels whose 1/s leaves fp32's normal range.
__device__ __noinline__ F16 smooth_exact(v4u x0, v4u x1, const uint16_t *__restrict__ smooth, int kbase) {
    F16 r;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const float xv = v4u_elem(e < 8 ? x0 : x1, e & 7);
        const int k = kbase + (e >> 3) * 32 + (e & 7);
        const float s = smooth ? bf16_to_f32(smooth[k]) : 1.0f;
        r.v[e] = xv / s;
    }
    return r;
}

// int4 codes of a group whose bf16 scale is tiny or zero: IEEE division
// (a zero scale gives zero codes).  Returns the two packed code words.
__device__ __noinline__ v2u int4_codes_exact(F16 xh, float sb) {
    v2u word = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const float q = sb == 0.0f ? 0.0f : __builtin_amdgcn_fmed3f(__builtin_rintf(xh.v[e] / sb), -8.0f, 7.0f);
        const uint32_t nib = __float_as_uint(q + 8388624.0f) & 15u;
        word[e >> 3] |= nib << (4 * (e & 7));
    }
    return word;
}

// The int4 codes of a group whose bf16 scale is tiny or zero, as floats:
// IEEE division, rounded to the nearest integer (ties to even), clamped.
__device__ __noinline__ F16 int4_q_exact(F16 xh, float sb) {
    F16 q;
#pragma unroll
    for (int e = 0; e < 16; ++e)
        q.v[e] = sb == 0.0f ? 0.0f : __builtin_amdgcn_fmed3f(__builtin_rintf(xh.v[e] / sb), -8.0f, 7.0f);
    return q;
}

typedef float v16f_q __attribute__((ext_vector_type(16)));

// The 16 codes of one lane (q[0..7]: channels 8kq..8kq+7 of group g's
// first K-half, q[8..15]: the same of the second), integers in [-8, 7] held
// as floats, into the group's three chunks of the FP6 tiled layout, here in
// the block's LDS image of it: [pair][16 rows][96 bytes], row r's chunk c of
// group g (g even: chunks 0-2, odd: 3-5) at slot (c + fp6_rot(rho)) mod 6,
// the halves of its last chunk swapped when fp6_half_swap(rho); rho = the
// row's index in its 128-row tile (a block's 16 rows start at a multiple of
// 16 there, so rho = 16 * (block % 8) + r).  Lanes kq = 0..3 of a row are
// lanes r + 16 kq; every lane of the wave takes part (the swaps are
// wave-wide).
__device__ __forceinline__ void store_fp6_group(const float (&q)[16], uint8_t *img, int r, int rho, int g_local,
                                                int kq) {
    v16f_q a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = q[2 * i];
        b[i] = q[2 * i + 1];
        a[8 + i] = 0.0f;
        b[8 + i] = 0.0f;
    }
    // fields 2i = a[i], 2i+1 = b[i]: fields 0..7 = q[0..7], 8..15 = q[8..15], values q/2
    const auto f = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(a, b, 2.0f);
    const uint32_t f0 = f[0], f1 = f[1], f2 = f[2];
    // this lane's 48 bits of each half: X (first half), Y (second half)
    uint32_t x0 = f0, x1 = f1 & 0xFFFFu;
    uint32_t y0 = (f1 >> 16) | (f2 << 16), y1 = f2 >> 16;
    // rows 1, 3 of 16 lanes (kq odd) swap X with rows 0, 2 (kq even) swapping
    // Y: kq even then holds (own X, partner's X) = 96 bits of the first half,
    // kq odd (partner's Y, own Y) = 96 bits of the second
    {
        const auto s0 = __builtin_amdgcn_permlane16_swap(x0, y0, false, false);
        const auto s1 = __builtin_amdgcn_permlane16_swap(x1, y1, false, false);
        x0 = s0[0]; y0 = s0[1];
        x1 = s1[0]; y1 = s1[1];
    }
    uint32_t v[3] = {x0, (x1 & 0xFFFFu) | (y0 << 16), (y0 >> 16) | (y1 << 16)};
    // kq 0, 1 hold bits 0..95 of their half, kq 2, 3 bits 96..191: the upper
    // 32 lanes swap with the lower 32, after which every lane has the whole
    // 192-bit string of its half as (first, second) = (d, s)
    uint32_t d[3], sr[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const auto w = __builtin_amdgcn_permlane32_swap(v[i], v[i], false, false);
        d[i] = w[0];
        sr[i] = w[1];
    }
    const int half = kq & 1, rot = fp6_rot(rho), sw = fp6_half_swap(rho);
    uint8_t *rowimg = img + (g_local >> 1) * (16 * 96) + r * 96;
    const int c0 = 3 * (g_local & 1);
    if (kq < 2) *(v4u *)(rowimg + 16 * ((c0 + half + rot) % 6)) = v4u{d[0], d[1], d[2], sr[0]};
    else *(v2u *)(rowimg + 16 * ((c0 + 2 + rot) % 6) + 8 * (half ^ sw)) = v2u{sr[1], sr[2]};
}

template <int PREC, int RT, bool GELU>
__global__ __launch_bounds__((qa_waves<PREC, RT, GELU>() * 64))
void quantize_act_kernel(int M, int K, const uint16_t *__restrict__ x,
                         const uint16_t *__restrict__ smooth,
                         const uint16_t *__restrict__ lora_down,
                         uint8_t *__restrict__ codes, void *__restrict__ scales,
                         float *__restrict__ lora_act)
{
    constexpr int QA_WAVES = qa_waves<PREC, RT, GELU>();
    constexpr bool LDSX = qa_lds_x<PREC, RT, GELU>();
    // low-rank slices (L2 resident): loaded per group, or one group ahead
    // when x comes through LDS (so that waiting for them never waits for
    // the newest x copies)
    constexpr int LSLOTS = LDSX ? 3 : 1;
    constexpr int QA_CHUNK = qa_chunk<PREC, RT, GELU>();
    constexpr int SINV = QA_CHUNK * 64 / (QA_WAVES * 64);   // 1/s channels per thread per chunk
    static_assert(SINV == 4 || SINV == 8, "1/s staging: 8 or 16 bytes of bf16 per thread");
    __shared__ float s_inv[QA_CHUNK * 64];
    __shared__ float s_part[RT > 0 ? QA_WAVES * QA_ROWS * RT * 16 : 1];
    __shared__ __attribute__((aligned(16))) uint16_t s_gelu[GELU ? GELU_TAB_PAD : 8];
    // The chunk's codes and scales are staged in LDS and written out once per
    // chunk with whole-line stores: storing each lane's 2 to 16 bytes as the
    // groups are done costs one memory request per piece, and the vector
    // memory path is what this kernel waits on.
    //   PREC 2: [pair][16 rows][96 B], the FP6 tiled layout of these rows;
    //   PREC 0/1: [16 rows][QA_OROW bytes] packed nibbles, row-major;
    //   scales: [16 rows][QA_SROW bytes] (bf16 per group; NVFP4 4 E4M3 bytes).
    constexpr int QA_OROW = QA_CHUNK * 32 + 16;        // +16: rows 0 and 8 share banks only
    constexpr int QA_OUT = PREC == 2 ? QA_CHUNK / 2 * 16 * 96 : QA_ROWS * QA_OROW;
    constexpr int QA_SROW = QA_CHUNK * (PREC == 1 ? 4 : 2) + 4;
    __shared__ __attribute__((aligned(16))) uint8_t s_out[QA_OUT];
    __shared__ __attribute__((aligned(16))) uint8_t s_osc[QA_ROWS * QA_SROW];
    // per wave one [16 rows][128 B] slice; row rl's 16-byte chunk c at
    // position c ^ ((rl >> 1) & 7), so that the 16 rows one LDS cycle
    // serves fall on distinct banks
    __shared__ __attribute__((aligned(16))) uint8_t s_xr[LDSX ? QA_WAVES * QA_XSLOT : 16];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (scalar)
    const int r = lane & 15;
    const int kq = lane >> 4;
    const int row = blockIdx.x * QA_ROWS + r;
    const int NG = K >> 6;
    const size_t xrow_off = (size_t)min(row, M - 1) * (size_t)K;   // rows past M: clamped, results not stored
    // whole-line loads of x: lane i of load j takes chunk i % 8 of row
    // 8j + i/8 (clamped to a valid row) and puts it at its LDS position
    size_t xl_off[2] = {0, 0};
    int xl_pos[2] = {0, 0};
    if constexpr (LDSX) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int rl = 8 * j + (lane >> 3);
            xl_off[j] = (size_t)min(blockIdx.x * QA_ROWS + rl, M - 1) * (size_t)K + 8 * (lane & 7);
            xl_pos[j] = rl * 128 + 16 * ((lane & 7) ^ ((rl >> 1) & 7));
        }
    }

    v4f acc[RT > 0 ? RT : 1];
#pragma unroll
    for (int t = 0; t < (RT > 0 ? RT : 1); ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int c0 = 0; c0 < NG; c0 += QA_CHUNK) {
        const int cg = min(QA_CHUNK, NG - c0);
        int unsafe = 0;

        // This wave's groups in the chunk: g_i = c0 + wave + i * QA_WAVES.  x
        // slices stream QA_XDEPTH groups ahead and the low-rank factor slices
        // (L2 resident) one group ahead, in register rings with compile-time
        // slots.  The loop body is one unroll period; a partial last period
        // runs the same body with its surplus steps skipped, so that the
        // kernel stays small enough for the instruction cache.
        const int n_w = wave < cg ? (cg - wave + QA_WAVES - 1) / QA_WAVES : 0;
        v4u xring[QA_XDEPTH + 1][2];
        v4u lring[LSLOTS][RT > 0 ? RT : 1][2];
        auto load_x = [&](int i, auto slot_c) __attribute__((always_inline)) {
            constexpr int S = decltype(slot_c)::value;
            if constexpr (LDSX) {
                const int kg = (c0 + wave + i * QA_WAVES) * 64;
                xring[S][0] = *(const v4u *)(x + xl_off[0] + kg);
                xring[S][1] = *(const v4u *)(x + xl_off[1] + kg);
            } else {
                const int kb = (c0 + wave + i * QA_WAVES) * 64 + 8 * kq;
                xring[S][0] = *(const v4u *)(x + xrow_off + kb);
                xring[S][1] = *(const v4u *)(x + xrow_off + kb + 32);
            }
            asm volatile("" ::: "memory");   // keep the loads here, ahead of their use
            __builtin_amdgcn_sched_barrier(0);
        };
        auto load_l = [&](int i, auto slot_c) __attribute__((always_inline)) {
            constexpr int S = decltype(slot_c)::value;
            const int kb = (c0 + wave + i * QA_WAVES) * 64 + 8 * kq;
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                const uint16_t *lp = lora_down + (size_t)(t * 16 + r) * (size_t)K + kb;
                lring[S][t][0] = *(const v4u *)lp;
                lring[S][t][1] = *(const v4u *)(lp + 32);
            }
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
        };
        auto process = [&](int i, const v4u (&xin)[2], const v4u (&lr)[RT > 0 ? RT : 1][2]) __attribute__((always_inline)) {
            v4u xr[2] = {xin[0], xin[1]};
            if constexpr (GELU) gelu_bf16x16(xr, s_gelu);
            const int g = c0 + wave + i * QA_WAVES;
            const int kbase = g * 64 + 8 * kq;
            const float *inv = s_inv + (g - c0) * 64 + 8 * kq;

            // ---- smoothing: v = x * (1/s), then RNE to bf16
            float xh[16];
            int bad = 0;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                float xv = v4u_elem(xr[e >> 3], e & 7);
                float v = xv * inv[(e >> 3) * 32 + (e & 7)];
                bad |= __builtin_amdgcn_class(v, 0x90) ? 1 : 0;   // fp32 subnormal
                xh[e] = v;
            }
            if (__builtin_expect(unsafe | __any(bad), 0)) {
                const F16 ex = smooth_exact(xr[0], xr[1], smooth, kbase);   // IEEE fp32 division
#pragma unroll
                for (int e = 0; e < 16; ++e) xh[e] = ex.v[e];
            }
            // RNE to bf16 two at a time (v_cvt_pk_bf16_f32; fp32 subnormals are
            // kept, so it equals the scalar rule for every finite value)
            v4u ah[2];
            float amax = 0.0f;
            float amax_j[2] = {0.0f, 0.0f};
#pragma unroll
            for (int j = 0; j < 2; ++j) {
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const uint32_t pk = pack_bf16x2_rne(xh[8 * j + 2 * p], xh[8 * j + 2 * p + 1]);
                    ah[j][p] = pk;
                    xh[8 * j + 2 * p] = bf16_lo(pk);
                    xh[8 * j + 2 * p + 1] = bf16_hi(pk);
                    amax_j[j] = max3_abs(amax_j[j], xh[8 * j + 2 * p], xh[8 * j + 2 * p + 1]);
                }
            }

            // ---- low-rank down-projection on the matrix cores
#pragma unroll
            for (int t = 0; t < RT; ++t) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(v8bf, ah[j]), __builtin_bit_cast(v8bf, lr[t][j]),
                        acc[t], 0, 0, 0);
                }
            }

            if constexpr (PREC == 2) {
                // ---- int4 codes in the FP6 layout: the same scale and codes
                amax = fmaxf(amax_j[0], amax_j[1]);
                amax = max_xor32(max_xor16(amax));
                const float s_f = amax * (1.0f / 7.0f);
                const uint32_t sbits = f32_to_bf16_rne(s_f);
                const float sb = __uint_as_float(sbits << 16);
                float q[16];
                if (__builtin_expect(__any(sb < 0x1p-100f), 0)) {
                    F16 xv;
#pragma unroll
                    for (int e = 0; e < 16; ++e) xv.v[e] = xh[e];
                    const F16 qe = int4_q_exact(xv, sb);
#pragma unroll
                    for (int e = 0; e < 16; ++e) q[e] = qe.v[e];
                } else {
                    const float inv_s = __builtin_amdgcn_rcpf(sb);
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const float xv = xh[e];
                        const float qe = xv * inv_s;
                        const float rr = __builtin_fmaf(-qe, sb, xv);
                        const float qc = __builtin_fmaf(rr, inv_s, qe);
                        q[e] = __builtin_rintf(__builtin_amdgcn_fmed3f(qc, -8.0f, 7.0f));
                    }
                }
                // a zero code is +0 in the layout (rint keeps the sign of -0.4)
#pragma unroll
                for (int e = 0; e < 16; ++e) q[e] += 0.0f;
                store_fp6_group(q, s_out, r, 16 * (blockIdx.x & 7) + r, g - c0, kq);
                if (kq == 0) *(uint16_t *)(s_osc + r * QA_SROW + 2 * (g - c0)) = (uint16_t)sbits;
            } else if constexpr (PREC == 0) {
                // ---- int4, group 64: absmax over the row's 4 lanes
                amax = fmaxf(amax_j[0], amax_j[1]);
                amax = max_xor32(max_xor16(amax));
                // fl32(amax / 7) and fl32(amax * fl32(1/7)) round to the same bf16
                // for every bf16 amax (checked exhaustively)
                const float s_f = amax * (1.0f / 7.0f);
                const uint32_t sbits = f32_to_bf16_rne(s_f);
                const float sb = __uint_as_float(sbits << 16);
                uint32_t word[2] = {0u, 0u};
                if (__builtin_expect(__any(sb < 0x1p-100f), 0)) {
                    F16 xv;
#pragma unroll
                    for (int e = 0; e < 16; ++e) xv.v[e] = xh[e];
                    const v2u w = int4_codes_exact(xv, sb);
                    word[0] = w[0];
                    word[1] = w[1];
                } else {
                    // a reciprocal within 1 ulp suffices: the Newton step below
                    // leaves an error of ~2^-45 relative, so half-integer quotients
                    // come out exact and others stay far from a tie
                    const float inv_s = __builtin_amdgcn_rcpf(sb);
#pragma unroll
                    for (int w = 0; w < 2; ++w) {
                        float qv[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float xv = xh[8 * w + e];
                            float qe = xv * inv_s;
                            float rr = __builtin_fmaf(-qe, sb, xv);
                            float qc = __builtin_fmaf(rr, inv_s, qe);
                            qv[e] = __builtin_amdgcn_fmed3f(qc, -8.0f, 7.0f);
                        }
                        word[w] = pack_int4_word(qv);
                    }
                }
                {
                    uint8_t *cp = s_out + r * QA_OROW + (g - c0) * 32 + 4 * kq;
                    *(uint32_t *)cp = word[0];
                    *(uint32_t *)(cp + 16) = word[1];
                    if (kq == 0) *(uint16_t *)(s_osc + r * QA_SROW + 2 * (g - c0)) = (uint16_t)sbits;
                }
            } else {
                // ---- NVFP4, group 16: lanes kq and kq^1 share a group within step j
                uint32_t word[2] = {0u, 0u};
                uint32_t sc[2];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    float a = max_xor16(amax_j[j]);
                    const float s_f = a * (1.0f / 6.0f);   // same E4M3 code as fl32(a / 6) for every bf16 a
                    const uint32_t se = e4m3_encode_nonneg(s_f);
                    const float d = e4m3_decode_nonneg(se);
                    sc[j] = se;
                    if (d != 0.0f) {
                        const float inv_d = __builtin_amdgcn_rcpf(d);
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            float xv = xh[8 * j + e];
                            float qe = xv * inv_d;
                            float rr = __builtin_fmaf(-qe, d, xv);
                            float v = fabsf(__builtin_fmaf(rr, inv_d, qe));
                            float f = fminf(fminf(2.0f * v, v + 2.0f), __builtin_fmaf(v, 0.5f, 4.0f));
                            f = fminf(f, 7.0f);
                            uint32_t m = __float_as_uint(f + 8388608.0f) & 7u;      // + 2^23
                            uint32_t sgn = (__float_as_uint(xv) >> 28) & 8u;
                            word[j] |= (m | sgn) << (4 * e);
                        }
                    }
                }
                {
                    uint8_t *cp = s_out + r * QA_OROW + (g - c0) * 32 + 4 * kq;
                    *(uint32_t *)cp = word[0];
                    *(uint32_t *)(cp + 16) = word[1];
                    if ((kq & 1) == 0) {
                        uint8_t *sp = s_osc + r * QA_SROW + (g - c0) * 4 + (kq >> 1);
                        sp[0] = (uint8_t)sc[0];
                        sp[2] = (uint8_t)sc[1];
                    }
                }
            }
        };
        // Loads are unconditional (the index is clamped to the wave's last
        // group; surplus loads read valid memory and are never used) so that
        // the compiler can count the loads in flight exactly.
        const int i_last = n_w - 1;
        constexpr int XR = QA_XDEPTH + 1;                 // x ring slots
        auto step = [&](int i, auto q_c) __attribute__((always_inline)) {
            constexpr int Q = decltype(q_c)::value;       // i % QA_PERIOD
            constexpr int XS = Q % XR, LS = Q % LSLOTS;
            if constexpr (LDSX) {
                // issue order per step: the low-rank slices of group i+1, then
                // the x slice of group i+2, so that waiting for group i's slices
                // (issued before the x slice of group i+1) never waits for the
                // newest x loads
                load_l(min(i + 1, i_last), std::integral_constant<int, (LS + 1) % 3>{});
                load_x(min(i + QA_XDEPTH, i_last), std::integral_constant<int, (XS + QA_XDEPTH) % XR>{});
                // into the MFMA layout through this wave's LDS slice (a wave's LDS
                // accesses run in order: the previous group's reads are done)
                uint8_t *sw = s_xr + wave * QA_XSLOT;
                *(v4u *)(sw + xl_pos[0]) = xring[XS][0];
                *(v4u *)(sw + xl_pos[1]) = xring[XS][1];
                const uint8_t *sl = sw + r * 128;
                const int fr = (r >> 1) & 7;
                const v4u xl[2] = {*(const v4u *)(sl + 16 * (kq ^ fr)), *(const v4u *)(sl + 16 * ((kq + 4) ^ fr))};
                process(i, xl, lring[LS]);
                return;
            }
            load_x(min(i + QA_XDEPTH, i_last), std::integral_constant<int, (XS + QA_XDEPTH) % XR>{});
            if constexpr (LSLOTS == 3) {
                load_l(min(i + 1, i_last), std::integral_constant<int, (LS + 1) % 3>{});
                process(i, xring[XS], lring[LS]);
            } else {
                load_l(i, std::integral_constant<int, 0>{});
                process(i, xring[XS], lring[0]);
            }
        };
        if (n_w > 0) {
            if constexpr (LDSX) {
                static_assert(QA_XDEPTH == 2, "the wait count assumes two x slices ahead");
                load_x(0, std::integral_constant<int, 0>{});
                load_l(0, std::integral_constant<int, 0>{});
                load_x(min(1, i_last), std::integral_constant<int, 1>{});
            } else {
                [&]<int... P>(std::integer_sequence<int, P...>) __attribute__((always_inline)) {
                    (load_x(min(P, i_last), std::integral_constant<int, P>{}), ...);
                }(std::make_integer_sequence<int, QA_XDEPTH>{});
                if constexpr (LSLOTS == 3) load_l(0, std::integral_constant<int, 0>{});
            }
        }
        // the GELU table, copied into LDS while the first slices are on their
        // way (published by the barrier below, before the first group is processed)
        if constexpr (GELU) {
            if (c0 == 0) gelu_table_fill(s_gelu, threadIdx.x, QA_WAVES * 64);
        }
        // 1/s of the chunk's channels (IEEE division), staged in LDS: thread t
        // takes channels SINV*t .. +SINV-1 with one load, issued after the
        // first x slices so that both latencies overlap.
        {
            const int i0 = threadIdx.x * SINV;
            if (i0 < cg * 64) {
                v4u sv = v4u{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};   // s = 1
                if (smooth) {
                    if constexpr (SINV == 8) {
                        sv = *(const v4u *)(smooth + (size_t)c0 * 64 + i0);
                    } else {
                        const v2u s2 = *(const v2u *)(smooth + (size_t)c0 * 64 + i0);
                        sv[0] = s2[0];
                        sv[1] = s2[1];
                    }
                }
                v4f inv[2];
#pragma unroll
                for (int e = 0; e < SINV; ++e) {
                    const float sf = v4u_elem(sv, e);
                    const float as = fabsf(sf);
                    const bool ok = (as >= 0x1p-64f) && (as <= 0x1p64f);
                    inv[e >> 2][e & 3] = ok ? 1.0f / sf : 0.0f;
                    unsafe |= ok ? 0 : 1;
                }
                *(v4f *)(s_inv + i0) = inv[0];
                if constexpr (SINV == 8) *(v4f *)(s_inv + i0 + 4) = inv[1];
            }
        }
        unsafe = __syncthreads_or(unsafe);
        if (n_w > 0) {
            for (int i = 0; i < n_w; i += QA_PERIOD)
                [&]<int... P>(std::integer_sequence<int, P...>) __attribute__((always_inline)) {
                    ((i + P < n_w ? step(i + P, std::integral_constant<int, P>{}) : void()), ...);
                }(std::make_integer_sequence<int, QA_PERIOD>{});
        }
        __syncthreads();

        // ---- the chunk's codes and scales: LDS -> global, consecutive threads
        // on consecutive bytes (rows past M are not written, and neither is
        // the second group of a last pair when K/64 is odd: FP6 padding)
        const int T = QA_WAVES * 64;
        const int row0 = blockIdx.x * QA_ROWS;
        const int rows = min(QA_ROWS, M - row0);
        if constexpr (PREC == 2) {
            const int NP = (NG + 1) >> 1, np = (cg + 1) >> 1;
            for (int idx = threadIdx.x; idx < np * 96; idx += T) {
                const int pl = idx / 96, rem = idx - pl * 96, rr = rem / 6, slot = rem - rr * 6;
                const int c = (slot + 6 - fp6_rot(rr)) % 6;              // the chunk held in this slot
                if (rr < rows && c0 + 2 * pl + c / 3 < NG) {
                    const int grow = row0 + rr;
                    const size_t off = ((size_t)(grow >> 7) * NP + (c0 >> 1) + pl) * FP6_PAIR_BYTES +
                                       (size_t)(grow & 127) * 96 + 16 * slot;
                    *(v4u *)(codes + off) = *(const v4u *)(s_out + idx * 16);
                }
            }
        } else {
            const int per_row = cg * 2;                                    // 16-byte pieces of a row
            for (int idx = threadIdx.x; idx < rows * per_row; idx += T) {
                const int rr = idx / per_row, pc = idx - rr * per_row;
                *(v4u *)(codes + (size_t)(row0 + rr) * (size_t)(K >> 1) + (size_t)c0 * 32 + 16 * pc) =
                    *(const v4u *)(s_out + rr * QA_OROW + 16 * pc);
            }
        }
        if constexpr (PREC == 1) {
            for (int idx = threadIdx.x; idx < rows * cg; idx += T) {
                const int rr = idx / cg, gl = idx - rr * cg;
                *(uint32_t *)((uint8_t *)scales + (size_t)(row0 + rr) * (size_t)(K >> 4) + (size_t)(c0 + gl) * 4) =
                    *(const uint32_t *)(s_osc + rr * QA_SROW + 4 * gl);
            }
        } else {
            for (int idx = threadIdx.x; idx < rows * cg; idx += T) {
                const int rr = idx / cg, gl = idx - rr * cg;
                ((uint16_t *)scales)[(size_t)(row0 + rr) * NG + c0 + gl] =
                    *(const uint16_t *)(s_osc + rr * QA_SROW + 2 * gl);
            }
        }
    }

    if constexpr (RT > 0) {
        // ---- reduce the low-rank partials of the 8 waves and write fp32
        // MFMA 16x16 output layout: lane l holds column l%16, rows 4*(l/16)+i.
        float *mine = s_part + wave * (QA_ROWS * RT * 16);
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                mine[(4 * kq + i) * (RT * 16) + t * 16 + r] = acc[t][i];
        __syncthreads();
        const int total = QA_ROWS * RT * 16;
        for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
            float s = 0.0f;
#pragma unroll
            for (int w = 0; w < QA_WAVES; ++w) s += s_part[w * total + idx];
            const int rr = idx / (RT * 16);
            const int orow = blockIdx.x * QA_ROWS + rr;
            if (orow < M) lora_act[(size_t)orow * (RT * 16) + (idx % (RT * 16))] = s;
        }
    }
}

template <int PREC, bool GELU>
static hipError_t launch_prec(int M, int K, int rank, const void *x, const void *smooth,
                              const void *lora_down, void *codes, void *scales, float *lora_act,
                              hipStream_t st)
{
    dim3 grid((M + QA_ROWS - 1) / QA_ROWS);
    const uint16_t *xp = (const uint16_t *)x, *sp = (const uint16_t *)smooth,
                   *lp = (const uint16_t *)lora_down;
    uint8_t *cp = (uint8_t *)codes;
#define QA_CASE(RTV)                                                                            \
    case RTV:                                                                                   \
        hipLaunchKernelGGL((quantize_act_kernel<PREC, RTV, GELU>), grid, dim3((qa_waves<PREC, RTV, GELU>() * 64)), 0, st, \
                           M, K, xp, sp, lp, cp, scales, lora_act);                             \
        break;
    switch (rank / 16) {
        QA_CASE(0) QA_CASE(1) QA_CASE(2) QA_CASE(3) QA_CASE(4)
        QA_CASE(5) QA_CASE(6) QA_CASE(7) QA_CASE(8)
        default: return hipErrorInvalidValue;
    }
#undef QA_CASE
    return hipGetLastError();
}

hipError_t launch_quantize_act(int precision, bool gelu, int M, int K, int rank, const void *x,
                               const void *smooth, const void *lora_down, void *act_codes,
                               void *act_scales, float *lora_act, hipStream_t stream)
{
    if (precision == 0)
        return gelu ? launch_prec<0, true>(M, K, rank, x, smooth, lora_down, act_codes, act_scales, lora_act, stream)
                    : launch_prec<0, false>(M, K, rank, x, smooth, lora_down, act_codes, act_scales, lora_act, stream);
    if (precision == 2)
        return gelu ? launch_prec<2, true>(M, K, rank, x, smooth, lora_down, act_codes, act_scales, lora_act, stream)
                    : launch_prec<2, false>(M, K, rank, x, smooth, lora_down, act_codes, act_scales, lora_act, stream);
    return gelu ? launch_prec<1, true>(M, K, rank, x, smooth, lora_down, act_codes, act_scales, lora_act, stream)
                : launch_prec<1, false>(M, K, rank, x, smooth, lora_down, act_codes, act_scales, lora_act, stream);
}

// The GELU of n bf16 values through the quantize kernel's own code
// (gelu_bf16x16: table, sentinel check and fallback), 16 values per thread;
// a test hook.
__global__ __launch_bounds__(256) void gelu_bf16_kernel(int64_t n, const uint16_t *__restrict__ in,
                                                        uint16_t *__restrict__ out)
{
    __shared__ __attribute__((aligned(16))) uint16_t tab[GELU_TAB_PAD];
    gelu_table_fill(tab, threadIdx.x, 256);
    __syncthreads();
    const int64_t base = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 16;
    v4u x[2];
    if (base + 16 <= n) {
        x[0] = *(const v4u *)(in + base);
        x[1] = *(const v4u *)(in + base + 8);
    } else {
        // the tail (and lanes past n): zeros beyond n, nothing stored there
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
            const uint32_t lo = base + e < n ? in[base + e] : 0u;
            const uint32_t hi = base + e + 1 < n ? in[base + e + 1] : 0u;
            x[e >> 3][(e >> 1) & 3] = lo | (hi << 16);
        }
    }
    gelu_bf16x16(x, tab);   // every lane takes part: the fallback's branch is wave-uniform
    if (base + 16 <= n) {
        *(v4u *)(out + base) = x[0];
        *(v4u *)(out + base + 8) = x[1];
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const uint32_t w = x[e >> 3][(e >> 1) & 3];
            if (base + e < n) out[base + e] = (uint16_t)((e & 1) ? (w >> 16) : (w & 0xFFFFu));
        }
    }
}

hipError_t launch_gelu_bf16(int64_t n, const void *in, void *out, hipStream_t stream)
{
    const int64_t blocks = (n + 16 * 256 - 1) / (16 * 256);
    hipLaunchKernelGGL(gelu_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       n, (const uint16_t *)in, (uint16_t *)out);
    return hipGetLastError();
}

}  // namespace svdq
