// gemv_w4a16_lines.hip -- the AWQ-style int4 weight-only layer ("Nunchaku
// Lite" docs, "Supported quantization types": awq_w4a16 int4 group 64, the
// memory-bound modulation projections) for up to eight rows of x:
//   y[m,n] = sum_k x[m,k] * (q[n,k] - z[n,g]) * s[n,g] + bias[n].
// Two kernels: one row on the vector ALU, two to eight on the matrix cores.
//
// At a few rows the layer is a pure HBM stream of the packed weights,
// and the matrix-core GEMV (gemv_w4a16_awq.hip) spends most of its time on
// the shape of its loads: a lane there owns one weight row, so each load
// instruction touches 32 rows x 32 bytes.  Here a wave owns 8 weight rows
// and lane l reads 16-byte chunk l%8 + 8j of row l/8: every load instruction
// covers 8 whole 128-byte lines, and each lane keeps AL_AHEAD chunk loads in
// flight ahead of the chunk it works on (about 7 MB over the whole grid at
// this shape, enough to keep HBM streaming).  The dot products run on the
// vector ALU (v_dot2_f32_bf16, two products per instruction): about 75
// vector instructions per chunk and lane, which the stream has to hide.
// Measured at 3072 -> 18432 over 16 rotating weight copies: with all of a
// lane's loads issued at once (the whole matrix requested at the start)
// 9.6 us, since most chunks then land near the end and their arithmetic
// runs after the stream; 3 ahead 8.6 us (1 ahead 9.3, 2 ahead 8.65, 4
// ahead 8.7); the same kernel without the arithmetic 7.4 us.
//
// Order of work in a block (4 waves, 32 weight rows):
//   1. each thread issues its loads of x and of the block's scales and zero
//      points, then its first AL_AHEAD weight chunks;
//   2. it waits for the first two only (loads complete in order), stores x
//      into LDS in the pair order of the unpacked codes together with the
//      sums of x over every 32-code chunk, and the scales and zero points;
//   3. after one barrier, chunk j is used as soon as it lands, after the
//      load of chunk j + AL_AHEAD has gone out.
// Arithmetic (as in the matrix-core GEMV): a code q in 0..15 becomes the bf16
// value 128 + q by placing it under the byte 0x43 (v_perm_b32), so
// sum (q - z) x = sum (128 + q) x - (128 + z) sum x per chunk, and the group
// scale multiplies the chunk's sum in fp32.  Each lane adds its chunks in
// order; the 8 lanes of a row are summed at the end (xor shuffles 1, 2, 4).
#include "device_common.h"
#include "launch.h"

namespace svdq {

constexpr int AL_WAVES = 4, AL_THREADS = AL_WAVES * 64;   // 3 and 6 measured slower at K = 3072
constexpr int AL_ROWS = AL_WAVES * 8;               // weight rows per block
constexpr int AL_MAX_K = 4096;                      // K / 256 <= 16 chunk loads per lane
constexpr int AL_AHEAD = 3;                         // chunk loads in flight ahead of the one in use

// one row of x (the template takes more, but from two rows on the
// matrix-core kernel below is faster: 9.9 against 11.6 us at two rows)
bool awq_gemv_lines_applies(int M, int N, int K) {
    return M == 1 && N >= 1 && K % 512 == 0 && K <= AL_MAX_K;
}

// LDS: x [MR][K/8][16 B] (pair order), sum of x per chunk [MR][K/32] fp32,
// scales and zero points [AL_ROWS][K/64] as (s | z << 16)
__host__ __device__ constexpr size_t al_lds_bytes(int MR, int K) {
    return (size_t)MR * K * 2 + (size_t)MR * (K / 32) * 4 + (size_t)AL_ROWS * (K / 64) * 4;
}

template <int MR, int NL>
__global__ __launch_bounds__(AL_THREADS)
void awq_gemv_lines_kernel(int N, int K, const uint16_t *__restrict__ x, const uint8_t *__restrict__ codes,
                           const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
                           const uint16_t *__restrict__ bias, uint16_t *__restrict__ out)
{
    extern __shared__ __align__(16) uint8_t al_smem[];
    const int NG = K >> 6, NC = K >> 5;              // groups, 32-code chunks per row
    uint8_t *s_x = al_smem;                          // [MR][K/8] x 16 B
    float *s_sum = (float *)(al_smem + (size_t)MR * K * 2);   // [MR][NC]
    uint32_t *s_sz = (uint32_t *)(s_sum + MR * NC);           // [AL_ROWS][NG]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n0 = blockIdx.x * AL_ROWS;

    // ---- 1. loads: x pieces (8 bf16 each), scale / zero pieces, weight chunks
    const int xpieces = MR * (K >> 3);               // 16-byte pieces of x
    constexpr int XP = (MR * AL_MAX_K / 8 + AL_THREADS - 1) / AL_THREADS;   // pieces per thread, at most
    v4u xr[XP];
#pragma unroll
    for (int i = 0; i < XP; ++i) {
        const int p = tid + i * AL_THREADS;
        if (p < xpieces) xr[i] = *(const v4u *)(x + (size_t)p * 8);
    }
    const int spr = NG >> 3;                          // 16-byte pieces per row of scales (NG % 8 == 0)
    const int spieces = AL_ROWS * spr;
    constexpr int SP = (AL_ROWS * (AL_MAX_K / 512) + AL_THREADS - 1) / AL_THREADS;
    v4u sr[SP], zr[SP];
#pragma unroll
    for (int i = 0; i < SP; ++i) {
        const int p = tid + i * AL_THREADS;
        if (p < spieces) {
            const int row = min(n0 + p / spr, N - 1);   // rows past N: a valid row, never stored
            const size_t off = (size_t)row * NG + (size_t)(p % spr) * 8;
            sr[i] = *(const v4u *)(scales + off);
            zr[i] = *(const v4u *)(zeros + off);
        }
    }
    const int row = min(n0 + wave * 8 + (lane >> 3), N - 1);
    // this row's bias, used only at the end; loaded unconditionally (a load
    // under a branch is waited for at the join), from the scales when there is
    // no bias (N <= N * K / 64 of them)
    const uint32_t braw = (bias ? bias : scales)[row];
    const int c0 = lane & 7;
    const uint8_t *wrow = codes + (size_t)row * (size_t)(K >> 1) + 16 * c0;
    v4u wr[NL];
    constexpr int AH = AL_AHEAD < NL ? AL_AHEAD : NL;
#pragma unroll
    for (int j = 0; j < AH; ++j) wr[j] = *(const v4u *)(wrow + 128 * j);

    // ---- 2. wait for x and the scales (issued first), stage them in LDS
    __builtin_amdgcn_s_waitcnt((AH & 15) | ((AH >> 4) << 14) | 0x0F70);   // vmcnt(AH)
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < XP; ++i) {
        const int p = tid + i * AL_THREADS;
        const bool ok = p < xpieces;
        const v4u w = ok ? xr[i] : v4u{0u, 0u, 0u, 0u};
        // (x0,x2) (x4,x6) (x1,x3) (x5,x7): the order the codes unpack in
        const v4u o = {__builtin_amdgcn_perm(w[1], w[0], 0x05040100u), __builtin_amdgcn_perm(w[3], w[2], 0x05040100u),
                       __builtin_amdgcn_perm(w[1], w[0], 0x07060302u), __builtin_amdgcn_perm(w[3], w[2], 0x07060302u)};
        if (ok) *(v4u *)(s_x + (size_t)p * 16) = o;
        // sum over the piece, then over the 4 pieces of a chunk (lanes 4q .. 4q+3)
        float s = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) s += bf16_lo(w[e]) + bf16_hi(w[e]);
        s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0xB1, 0xF, 0xF, true));
        s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0x4E, 0xF, 0xF, true));
        if (ok && (p & 3) == 0) s_sum[p >> 2] = s;   // chunk p/4 of the flattened [MR][NC]
    }
#pragma unroll
    for (int i = 0; i < SP; ++i) {
        const int p = tid + i * AL_THREADS;
        if (p < spieces) {
            const int r = p / spr, g8 = (p % spr) * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t sv = (e & 1) ? sr[i][e >> 1] >> 16 : sr[i][e >> 1] & 0xFFFFu;
                const uint32_t zv = (e & 1) ? zr[i][e >> 1] >> 16 : zr[i][e >> 1] & 0xFFFFu;
                s_sz[r * NG + g8 + e] = sv | zv << 16;
            }
        }
    }
    __syncthreads();

    // ---- 3. the weight chunks, each as soon as it has landed
    const uint32_t k43 = 0x43434343u;
    const uint32_t *szrow = s_sz + (wave * 8 + (lane >> 3)) * NG;
    float y[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) y[m] = 0.0f;
    auto chunk = [&](auto jc) {
        constexpr int j = decltype(jc)::value;
        __builtin_amdgcn_sched_barrier(0);           // chunks stay in order (registers: one chunk's x at a time)
        if constexpr (j + AH < NL) wr[j + AH] = *(const v4u *)(wrow + 128 * (j + AH));
        // loads issued after chunk j's: up to chunk j + AH
        constexpr int newer = (j + AH < NL ? j + AH : NL - 1) - j;
        __builtin_amdgcn_s_waitcnt((newer & 15) | ((newer >> 4) << 14) | 0x0F70);   // vmcnt(newer)
        asm volatile("" ::: "memory");
        const int c = c0 + 8 * j;                    // chunk of the row: codes 32c .. 32c+31
        v2bf pq[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = wr[j][i] & 0x0F0F0F0Fu, hi = (wr[j][i] >> 4) & 0x0F0F0F0Fu;
            pq[4 * i + 0] = __builtin_bit_cast(v2bf, __builtin_amdgcn_perm(k43, lo, 0x04010400u));
            pq[4 * i + 1] = __builtin_bit_cast(v2bf, __builtin_amdgcn_perm(k43, lo, 0x04030402u));
            pq[4 * i + 2] = __builtin_bit_cast(v2bf, __builtin_amdgcn_perm(k43, hi, 0x04010400u));
            pq[4 * i + 3] = __builtin_bit_cast(v2bf, __builtin_amdgcn_perm(k43, hi, 0x04030402u));
        }
        const uint32_t sz = szrow[c >> 1];
        const float sc = __uint_as_float(sz << 16), zp = 128.0f + __uint_as_float(sz & 0xFFFF0000u);
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            const v4u *xp = (const v4u *)(s_x + ((size_t)m * (K >> 3) + 4 * c) * 16);
            float t0 = 0.0f, t1 = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // elements copied to scalars before the bit casts: this clang
                // miscompiles a bit cast of an element of a vector value
                const v4u xv = xp[i];
                const uint32_t x0 = xv[0], x1 = xv[1], x2 = xv[2], x3 = xv[3];
                t0 = __builtin_amdgcn_fdot2_f32_bf16(pq[4 * i + 0], __builtin_bit_cast(v2bf, x0), t0, false);
                t1 = __builtin_amdgcn_fdot2_f32_bf16(pq[4 * i + 1], __builtin_bit_cast(v2bf, x1), t1, false);
                t0 = __builtin_amdgcn_fdot2_f32_bf16(pq[4 * i + 2], __builtin_bit_cast(v2bf, x2), t0, false);
                t1 = __builtin_amdgcn_fdot2_f32_bf16(pq[4 * i + 3], __builtin_bit_cast(v2bf, x3), t1, false);
            }
            // sum_chunk (q - z) x = sum (128 + q) x - (128 + z) sum x
            const float part = __builtin_fmaf(-zp, s_sum[m * NC + c], t0 + t1);
            y[m] = __builtin_fmaf(sc, part, y[m]);
            asm volatile("" : "+v"(y[m]));           // the chunk's sum is complete here
        }
    };
    [&]<int... J>(std::integer_sequence<int, J...>) { (chunk(std::integral_constant<int, J>{}), ...); }(
        std::make_integer_sequence<int, NL>{});

    // ---- 4. the 8 lanes of a row, then bias and the bf16 store
    const int orow = n0 + wave * 8 + (lane >> 3);
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        float v = y[m];
        v += __shfl_xor(v, 1, 64);
        v += __shfl_xor(v, 2, 64);
        v += __shfl_xor(v, 4, 64);
        if (c0 == 0 && orow < N) {
            if (bias) v += __uint_as_float(braw << 16);
            out[(size_t)m * N + orow] = (uint16_t)f32_to_bf16_rne(v);
        }
    }
}

// The same whole-line weight stream with the products on the matrix cores,
// for up to 8 rows of x.  v_mfma_f32_16x16x32_bf16 wants 16 A rows that
// share their k slots; a whole-line load gives 8 weight rows, so each A row
// is one half of a weight row's 128-byte line: lane l takes row a = l%16 =
// (weight row a/2, half h = a%2) and chunk 4h + l/16 of that line, i.e. the 8
// lanes of a weight row cover its line and every load instruction 8 whole
// lines.  The B columns are (row m of x, half) pairs, b = 2m + h', holding x
// at the code positions of half h'; D[a][b] is a product of weight-row half
// h with x of half h', wanted only for h = h' (the other half of D is not
// used, the matrix cores have room to spare).  Per load instruction: one
// MFMA per dword of the lanes' 16 bytes, 4 in all, for any M up to 8.
//
// An MFMA adds 32 k slots, 8 from each lane group l/16 (the 4 chunks of a
// half line, two groups of 64 codes); one v_permlane32_swap per dword pair
// trades dwords 2, 3 of lane groups 0, 1 for dwords 0, 1 of lane groups 2, 3
// (same row, chunks two apart), after which dwords 0, 1 of every lane hold
// codes of the first group of its half and dwords 2, 3 of the second.  The
// code positions of MFMA i in lane group q, within the half, are
// 64 (i/2) + 8 (i%2) + {0, 32, 16, 48}[q] + (0 2 4 6 1 3 5 7), the same in
// x's LDS copy.  Each group's two MFMAs give P = sum (128 + q) x; lane l
// keeps the entries of D in its own half, rows 2 (l/16) and 2 (l/16) + 1 at
// column l%16, and adds s (P - (128 + z) sum x); the two halves of a row are
// added at the end (xor shuffle 1).
//
// Measured at 3072 -> 18432 over 16 rotating weight copies (2, 3, 4, 5, 8 rows
// of x): 9.9-10.6, 11.1, 11.5, 12.0, 13.1-13.3 us, against 11.6, 15.2, 15.5,
// 16.0, 17.5 us for the vector-ALU kernel (two rows) and the one-row-per-lane
// matrix-core GEMV (three and more).  Also tried: lanes loading 64 bytes of
// 16 weight rows, which feed the MFMA without the half-row trick, 11.1-12.4
// us for 1-5 rows (that load pattern alone reads 7% slower than whole lines,
// and the K split it needs adds an LDS reduction); 16-block 4x4x4 MFMAs,
// whose A operand fits whole-line loads directly, 10.4-12.0 us for 2-4 rows
// but 15.3-16.4 for 5-8 (twice the MFMAs and x reads).  At eight rows of x the
// 8-wave block matters: with 4 waves (576 blocks of 67 KB LDS, two per CU)
// 17.7 us.  At one row the vector-ALU kernel stays ahead (8.2-8.7 against
// 9.5-10.1 us).
constexpr int LQ_MAX_K = 4096, LQ_MAX_M = 8;
constexpr int LQ_AHEAD = 3;                          // load instructions in flight ahead of the one in use

// x in LDS: row m at m * stride, its 16-byte piece P (8 values, pair order)
// at 16 (P + P/16): the pieces of the two halves of a line, which one read
// instruction takes for the same m, sit 4 banks apart, and the row stride is
// 2 pieces mod 16 so that the 8 rows read together fall on distinct banks
__host__ __device__ constexpr int lq_xstride(int K) {
    return 16 * (K / 8 + K / 128 + ((2 - (K / 8 + K / 128)) & 15));
}
// LDS: x, sum of x per group [M][K/64] fp32, (scale, 128 + zero) fp32 pairs
// [K/64 groups][8 W rows]
__host__ __device__ constexpr size_t lq_lds_bytes(int W, int M, int K) {
    return (size_t)M * lq_xstride(K) + (size_t)M * (K / 64) * 4 + (size_t)(K / 64) * (8 * W) * 8;
}

// waves per block: 8 when x is large (its staging is then shared by 64 rows)
static int lq_waves(int M) { return M > 4 ? 8 : 4; }

// at most 80 KB of LDS per block: two blocks per CU (gfx950 has 160 KB)
bool awq_gemv_lines_mfma_applies(int M, int N, int K) {
    return M >= 1 && M <= LQ_MAX_M && N >= 1 && K % 512 == 0 && K <= LQ_MAX_K &&
           lq_lds_bytes(lq_waves(M), M, K) <= 80 * 1024;
}

template <int W, int MB, int NL>
__global__ __launch_bounds__(W * 64)
void awq_gemv_lines_mfma_kernel(int M, int N, int K, const uint16_t *__restrict__ x,
                                const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
                                const uint16_t *__restrict__ zeros, const uint16_t *__restrict__ bias,
                                uint16_t *__restrict__ out)
{
    extern __shared__ __align__(16) uint8_t lq_smem[];
    constexpr int LQ_THREADS = W * 64, LQ_ROWS = W * 8;
    const int NG = K >> 6, KP = K >> 3;              // groups, 16-byte pieces per row of x
    const int xstride = lq_xstride(K);
    uint8_t *s_x = lq_smem;
    float *s_sum = (float *)(lq_smem + (size_t)M * xstride);  // [M][NG]
    v2f *s_sz = (v2f *)(s_sum + (size_t)M * NG);             // [NG][LQ_ROWS]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n0 = blockIdx.x * LQ_ROWS;
    const int q = lane >> 4, a = lane & 15, hb = lane & 1;   // lane group; A row / B column; half

    // ---- 1. loads: x pieces, scale / zero pieces, bias, weight lines.  x has
    // M * K / 8 pieces, a multiple of 64, so the guards are uniform over a
    // wave (a load under a per-lane branch is waited for at the join).
    const int xpieces = M * KP;
    constexpr int XP = (MB * LQ_MAX_K / 8 + LQ_THREADS - 1) / LQ_THREADS;
    v4u xr[XP];
#pragma unroll
    for (int i = 0; i < XP; ++i)
        if (i * LQ_THREADS + wave * 64 < xpieces) xr[i] = *(const v4u *)(x + (size_t)(tid + i * LQ_THREADS) * 8);
    const int spr = NG >> 3;                         // 16-byte pieces per row of scales
    const int spieces = LQ_ROWS * spr;
    constexpr int SP = (LQ_ROWS * (LQ_MAX_K / 512) + LQ_THREADS - 1) / LQ_THREADS;
    v4u sr[SP], zr[SP];
#pragma unroll
    for (int i = 0; i < SP; ++i) {
        const int p = tid + i * LQ_THREADS;
        if (p < spieces) {
            const int row = min(n0 + p / spr, N - 1);   // rows past N: a valid row, never stored
            const size_t off = (size_t)row * NG + (size_t)(p % spr) * 8;
            sr[i] = *(const v4u *)(scales + off);
            zr[i] = *(const v4u *)(zeros + off);
        }
    }
    // the bias of this lane's two output rows, used only at the end; from
    // the scales when there is no bias (N * K / 64 of them cover N rows)
    const int orow0 = n0 + wave * 8 + 2 * q;
    const uint16_t *bsrc = bias ? bias : scales;
    const uint32_t braw0 = bsrc[min(orow0, N - 1)], braw1 = bsrc[min(orow0 + 1, N - 1)];
    const int row = min(n0 + wave * 8 + (a >> 1), N - 1);
    const uint8_t *wrow = codes + (size_t)row * (size_t)(K >> 1) + 16 * (4 * hb + q);
    v4u wr[NL];
    constexpr int AH = LQ_AHEAD < NL ? LQ_AHEAD : NL;
#pragma unroll
    for (int j = 0; j < AH; ++j) wr[j] = *(const v4u *)(wrow + 128 * j);

    // ---- 2. wait for everything but the weight lines, stage x (pair order,
    // with the sums over each group) and the scales in LDS
    __builtin_amdgcn_s_waitcnt((AH & 15) | ((AH >> 4) << 14) | 0x0F70);   // vmcnt(AH)
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < XP; ++i) {
        if (i * LQ_THREADS + wave * 64 >= xpieces) continue;
        const int p = tid + i * LQ_THREADS;
        const int m = p / KP, pc = p - m * KP;
        const v4u w = xr[i];
        // (x0,x2) (x4,x6) (x1,x3) (x5,x7): the order the codes unpack in
        const v4u o = {__builtin_amdgcn_perm(w[1], w[0], 0x05040100u), __builtin_amdgcn_perm(w[3], w[2], 0x05040100u),
                       __builtin_amdgcn_perm(w[1], w[0], 0x07060302u), __builtin_amdgcn_perm(w[3], w[2], 0x07060302u)};
        *(v4u *)(s_x + (size_t)m * xstride + 16 * (pc + (pc >> 4))) = o;
        float sm = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) sm += bf16_lo(w[e]) + bf16_hi(w[e]);
        sm += __shfl_xor(sm, 1, 64);                 // the 8 pieces of a group: lanes 8t .. 8t+7
        sm += __shfl_xor(sm, 2, 64);
        sm += __shfl_xor(sm, 4, 64);
        if ((p & 7) == 0) s_sum[p >> 3] = sm;        // group p/8 of the flattened [M][NG]
    }
#pragma unroll
    for (int i = 0; i < SP; ++i) {
        const int p = tid + i * LQ_THREADS;
        if (p < spieces) {
            const int rr = p / spr, g8 = (p % spr) * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t sv = (e & 1) ? sr[i][e >> 1] >> 16 : sr[i][e >> 1] & 0xFFFFu;
                const uint32_t zv = (e & 1) ? zr[i][e >> 1] >> 16 : zr[i][e >> 1] & 0xFFFFu;
                s_sz[(g8 + e) * LQ_ROWS + rr] = v2f{__uint_as_float(sv << 16), 128.0f + __uint_as_float(zv << 16)};
            }
        }
    }
    __syncthreads();

    // ---- 3. the weight lines, each as soon as it has landed
    const uint32_t k43 = 0x43434343u;
    const int mc = min(a >> 1, M - 1);               // row of x in this lane's B column
    // piece offset of MFMA i's x within a half line: 8 (i/2) + (i%2) + {0, 4, 2, 6}[q]
    const int qp = ((q & 1) << 2) | ((q & 2) >> 0);
    const uint8_t *xb = s_x + (size_t)mc * xstride;
    const float *sxl = s_sum + (size_t)mc * NG + 2 * hb;
    const v2f *szl = s_sz + wave * 8 + 2 * q;
    float y0 = 0.0f, y1 = 0.0f;
    auto line = [&](auto jc) __attribute__((always_inline)) {
        constexpr int j = decltype(jc)::value;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (j + AH < NL) wr[j + AH] = *(const v4u *)(wrow + 128 * (j + AH));
        constexpr int newer = (j + AH < NL ? j + AH : NL - 1) - j;
        __builtin_amdgcn_s_waitcnt((newer & 15) | ((newer >> 4) << 14) | 0x0F70);   // vmcnt(newer)
        asm volatile("" ::: "memory");
        // dwords 0, 1 of lanes 32..63 <-> dwords 2, 3 of lanes 0..31
        const auto s02 = __builtin_amdgcn_permlane32_swap(wr[j][0], wr[j][2], false, false);
        const auto s13 = __builtin_amdgcn_permlane32_swap(wr[j][1], wr[j][3], false, false);
        const uint32_t d[4] = {s02[0], s13[0], s02[1], s13[1]};
        v4u av[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = d[i] & 0x0F0F0F0Fu, hi = (d[i] >> 4) & 0x0F0F0F0Fu;
            av[i] = v4u{__builtin_amdgcn_perm(k43, lo, 0x04010400u), __builtin_amdgcn_perm(k43, lo, 0x04030402u),
                        __builtin_amdgcn_perm(k43, hi, 0x04010400u), __builtin_amdgcn_perm(k43, hi, 0x04030402u)};
        }
        const int pbase = 32 * j + 16 * hb + qp;     // piece of MFMA 0 in this lane's half
        const v2f sx = *(const v2f *)(sxl + 4 * j);  // sums of x over the half's two groups
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            v4f pacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int i = 2 * g; i < 2 * g + 2; ++i) {
                const int pc = pbase + 8 * (i >> 1) + (i & 1);
                const v4u xv = *(const v4u *)(xb + 16 * (pc + (pc >> 4)));
                pacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, av[i]),
                                                               __builtin_bit_cast(v8bf, xv), pacc, 0, 0, 0);
            }
            // D rows 4q .. 4q+3 = (weight row 2q + r/2, half r%2): this lane's half is r = hb, hb + 2
            const float p0 = hb ? pacc[1] : pacc[0], p1 = hb ? pacc[3] : pacc[2];
            const v4f sz = *(const v4f *)(szl + (4 * j + 2 * hb + g) * LQ_ROWS);   // rows 2q, 2q+1
            const float sxg = g ? sx[1] : sx[0];
            y0 = __builtin_fmaf(sz[0], __builtin_fmaf(-sz[1], sxg, p0), y0);
            y1 = __builtin_fmaf(sz[2], __builtin_fmaf(-sz[3], sxg, p1), y1);
        }
    };
    [&]<int... J>(std::integer_sequence<int, J...>) { (line(std::integral_constant<int, J>{}), ...); }(
        std::make_integer_sequence<int, NL>{});

    // ---- 4. the two halves of each row, then bias and the bf16 store
    y0 += __shfl_xor(y0, 1, 64);
    y1 += __shfl_xor(y1, 1, 64);
    const int m = a >> 1;
    if (hb == 0 && m < M) {
        if (orow0 < N) {
            float v = y0;
            if (bias) v += __uint_as_float(braw0 << 16);
            out[(size_t)m * N + orow0] = (uint16_t)f32_to_bf16_rne(v);
        }
        if (orow0 + 1 < N) {
            float v = y1;
            if (bias) v += __uint_as_float(braw1 << 16);
            out[(size_t)m * N + orow0 + 1] = (uint16_t)f32_to_bf16_rne(v);
        }
    }
}

// A plain read of `bytes` of device memory, the ceiling the weight stream is
// measured against.  Each wave reads a 12 KB span with 12 loads of 16 bytes
// per lane, all issued before any use, either in the GEMV's pattern (rows
// of 1536 bytes, 8 lanes per 128-byte line: lane l takes row l/8, chunk
// l%8 + 8j; LINES) or contiguously (lane l takes 16 l + 1024 j).  The xor
// of the span's words goes to out[span] (a plain store per wave: one shared
// atomic would serialize thousands of waves), so that no load is dropped.
constexpr int SR_LOADS = 12;
constexpr int SR_SPAN = 64 * SR_LOADS * 16;   // bytes per wave
template <bool LINES>
__global__ __launch_bounds__(256) void stream_read_kernel(const uint8_t *__restrict__ src, int64_t bytes,
                                                          uint32_t *__restrict__ out)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t base = wave * SR_SPAN +
                         (LINES ? (int64_t)(lane >> 3) * (SR_LOADS * 128) + 16 * (lane & 7) : 16 * lane);
    constexpr int step = LINES ? 128 : 1024;
    v4u r[SR_LOADS];
#pragma unroll
    for (int j = 0; j < SR_LOADS; ++j) {
        const int64_t off = base + (int64_t)step * j;
        r[j] = off + 16 <= bytes ? *(const v4u *)(src + off) : v4u{0u, 0u, 0u, 0u};
    }
    uint32_t acc = 0u;
#pragma unroll
    for (int j = 0; j < SR_LOADS; ++j) acc ^= r[j][0] ^ r[j][1] ^ r[j][2] ^ r[j][3];
    acc ^= __shfl_xor(acc, 32, 64);
    acc ^= __shfl_xor(acc, 16, 64);
    acc ^= __shfl_xor(acc, 8, 64);
    acc ^= __shfl_xor(acc, 4, 64);
    acc ^= __shfl_xor(acc, 2, 64);
    acc ^= __shfl_xor(acc, 1, 64);
    if (lane == 0 && wave * SR_SPAN < bytes) out[wave] = acc;
}

int64_t stream_read_spans(int64_t bytes) { return (bytes + SR_SPAN - 1) / SR_SPAN; }

hipError_t launch_stream_read(const void *src, int64_t bytes, bool lines, uint32_t *out, hipStream_t stream)
{
    const int64_t blocks = (stream_read_spans(bytes) + 3) / 4;
    if (lines)
        hipLaunchKernelGGL(stream_read_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           (const uint8_t *)src, bytes, out);
    else
        hipLaunchKernelGGL(stream_read_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           (const uint8_t *)src, bytes, out);
    return hipGetLastError();
}

template <int MR>
static hipError_t launch_lines_mr(int N, int K, const uint16_t *xp, const uint8_t *cp, const uint16_t *sp,
                                  const uint16_t *zp, const uint16_t *bp, uint16_t *op, hipStream_t stream)
{
    const dim3 grid((N + AL_ROWS - 1) / AL_ROWS), block(AL_THREADS);
    const size_t lds = al_lds_bytes(MR, K);
#define AL_CASE(NLV)                                                                                        \
    case NLV:                                                                                               \
        hipLaunchKernelGGL((awq_gemv_lines_kernel<MR, NLV>), grid, block, lds, stream, N, K, xp, cp, sp, zp, bp, op); \
        break;
    switch (K / 256) {
        AL_CASE(2) AL_CASE(4) AL_CASE(6) AL_CASE(8) AL_CASE(10) AL_CASE(12) AL_CASE(14) AL_CASE(16)
        default: return hipErrorInvalidValue;
    }
#undef AL_CASE
    return hipGetLastError();
}

template <int W, int MB>
static hipError_t launch_lines_mfma_mb(int M, int N, int K, const uint16_t *xp, const uint8_t *cp,
                                       const uint16_t *sp, const uint16_t *zp, const uint16_t *bp, uint16_t *op,
                                       hipStream_t stream)
{
    const dim3 grid((N + 8 * W - 1) / (8 * W)), block(64 * W);
    const size_t lds = lq_lds_bytes(W, M, K);
#define LQ_CASE(NLV)                                                                                          \
    case NLV:                                                                                                 \
        hipLaunchKernelGGL((awq_gemv_lines_mfma_kernel<W, MB, NLV>), grid, block, lds, stream, M, N, K, xp, cp, \
                           sp, zp, bp, op);                                                                   \
        break;
    switch (K / 256) {
        LQ_CASE(2) LQ_CASE(4) LQ_CASE(6) LQ_CASE(8) LQ_CASE(10) LQ_CASE(12) LQ_CASE(14) LQ_CASE(16)
        default: return hipErrorInvalidValue;
    }
#undef LQ_CASE
    return hipGetLastError();
}

hipError_t launch_awq_gemv_lines_mfma(int M, int N, int K, const void *x, const void *codes, const void *scales,
                                      const void *zeros, const void *bias, void *out, hipStream_t stream)
{
    const uint16_t *xp = (const uint16_t *)x, *sp = (const uint16_t *)scales, *zp = (const uint16_t *)zeros,
                   *bp = (const uint16_t *)bias;
    const uint8_t *cp = (const uint8_t *)codes;
    uint16_t *op = (uint16_t *)out;
    if (!awq_gemv_lines_mfma_applies(M, N, K)) return hipErrorInvalidValue;
    if (M <= 2) return launch_lines_mfma_mb<4, 2>(M, N, K, xp, cp, sp, zp, bp, op, stream);
    if (M <= 4) return launch_lines_mfma_mb<4, 4>(M, N, K, xp, cp, sp, zp, bp, op, stream);
    return launch_lines_mfma_mb<8, 8>(M, N, K, xp, cp, sp, zp, bp, op, stream);
}

hipError_t launch_awq_gemv_lines(int M, int N, int K, const void *x, const void *codes, const void *scales,
                                 const void *zeros, const void *bias, void *out, hipStream_t stream)
{
    const uint16_t *xp = (const uint16_t *)x, *sp = (const uint16_t *)scales, *zp = (const uint16_t *)zeros,
                   *bp = (const uint16_t *)bias;
    const uint8_t *cp = (const uint8_t *)codes;
    uint16_t *op = (uint16_t *)out;
    if (!awq_gemv_lines_applies(M, N, K)) return hipErrorInvalidValue;
    return launch_lines_mr<1>(N, K, xp, cp, sp, zp, bp, op, stream);
}

}  // namespace svdq
