// gemv_w4a16_lines.hip -- the AWQ-style int4 weight-only layer ("Nunchaku
// Lite" docs, "Supported quantization types": awq_w4a16 int4 group 64, the
// memory-bound modulation projections) for one or two rows of x:
//   y[m,n] = sum_k x[m,k] * (q[n,k] - z[n,g]) * s[n,g] + bias[n].
//
// At one or two rows the layer is a pure HBM stream of the packed weights,
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

bool awq_gemv_lines_applies(int M, int N, int K) {
    return M >= 1 && M <= 2 && N >= 1 && K % 512 == 0 && K <= AL_MAX_K;
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
            if (bias) v += bf16_to_f32(bias[orow]);
            out[(size_t)m * N + orow] = (uint16_t)f32_to_bf16_rne(v);
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

hipError_t launch_awq_gemv_lines(int M, int N, int K, const void *x, const void *codes, const void *scales,
                                 const void *zeros, const void *bias, void *out, hipStream_t stream)
{
    const uint16_t *xp = (const uint16_t *)x, *sp = (const uint16_t *)scales, *zp = (const uint16_t *)zeros,
                   *bp = (const uint16_t *)bias;
    const uint8_t *cp = (const uint8_t *)codes;
    uint16_t *op = (uint16_t *)out;
    return M == 1 ? launch_lines_mr<1>(N, K, xp, cp, sp, zp, bp, op, stream)
                  : launch_lines_mr<2>(N, K, xp, cp, sp, zp, bp, op, stream);
}

}  // namespace svdq
