// gemv_w4a16_awq.hip -- AWQ-style int4 weight-only layer with bf16
// activations on gfx950 ("Nunchaku Lite" docs, "Supported quantization
// types": awq_w4a16 int4 group 64, used for memory-bound, precision-
// sensitive layers such as the adaptive-norm modulation projections):
//   y[m,n] = sum_k x[m,k] * (q[n,k] - z[n,g]) * s[n,g] + bias[n].
//
// The kernel is an HBM stream of the packed weights, so it is built around
// having a wave's whole share of the weights in flight at once:
//  * Weights are the B operand of v_mfma_f32_32x32x16_bf16: lane l owns
//    weight row n0 + l%32 and the half l/32 of each 64-code group, i.e. one
//    16-byte load per lane per group, and one scale and zero point per lane
//    per group.  Eight groups (a K-part at K = 3072) are in flight per lane
//    before anything waits.
//  * x is the A operand (rows m).  A block copies its M-tile of x global ->
//    LDS (global_load_lds) and waits for it before any weight load goes out,
//    so later waits are for exactly the group about to be used and each
//    group is processed as soon as its codes land.  One pass over LDS then
//    permutes x in place to the order the codes unpack in and forms the
//    per-group sums of x.  Lanes whose row m lies past M read the last real
//    row (their results are never stored).
//  * A block is one 32-row weight tile and 6 waves, one per K-part; the part
//    sums are added through LDS at the end.  Small blocks keep the work per
//    SIMD even (the kernel is balanced between compute and HBM), and a whole
//    layer's grid is resident on the chip at once.
//
// Arithmetic: a code q in 0..15 becomes the bf16 value 128 + q by OR-ing it
// into the bit pattern 0x4300 (bf16 128 has a unit mantissa step), so one
// and-or unpacks two codes; sum_{k in g} (q - z) x = sum (128 + q) x -
// (128 + z) sum x; the group scale multiplies the group's sum in fp32.
// Codes unpack in pairs (p, p+4) of a dword and x is staged in the same
// order (a dot product only needs A and B in one order).
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace svdq {

constexpr int AW_KP = 6;                 // waves per block, one K-part each
constexpr int AW_THREADS = AW_KP * 64;
constexpr int AW_TILE_N = 32;            // weight rows per block (one MFMA tile)
constexpr int AW_XBYTES = 64 * 1024;     // LDS for one K-chunk of x (without row padding)
constexpr int AW_MAXCG = 64;             // groups per K-chunk at most
constexpr int AW_XPAD = 16;              // bytes of padding per staged x row (bank spread)

// Groups of one K-chunk: as many as fit in AW_XBYTES for Mt rows, a multiple
// of 8 (a row is staged in whole 1 KB copies of 8 groups, so its LDS stride
// must hold them all); with 8-byte scale loads (VEC) a multiple of 4 * AW_KP
// so every K-part starts on a multiple of 4 groups.
__host__ __device__ inline int aw_chunk_groups(int Mt, bool vec) {
    int cg = AW_XBYTES / (Mt * 128);
    if (cg > AW_MAXCG) cg = AW_MAXCG;
    cg -= cg % 8;
    return vec ? cg - cg % (4 * AW_KP) : cg;
}

// (m, q) = divmod(idx, d) for idx < 2^12 and 1 <= d <= 2^9: the fp32 estimate
// is off by at most one, which one correction step removes.
__device__ __forceinline__ void aw_divmod(int idx, int d, float rd, int &m, int &q) {
    m = (int)((float)idx * rd);
    q = idx - m * d;
    if (q >= d) { ++m; q -= d; }
    if (q < 0) { --m; q += d; }
}

__host__ __device__ constexpr int aw_xs_bytes(int MR) { return (AW_MAXCG * MR + 8) * 4; }

// Memory instructions one load_quad issues: four 16-byte code loads, plus
// one 8-byte scale and one 8-byte zero-point load (VEC) or four 2-byte loads
// of each.
__host__ __device__ constexpr int aw_quad_loads(bool vec) { return vec ? 6 : 12; }

// s_waitcnt vmcnt(N) (N < 64: low 4 bits in [3:0], high 2 bits in [15:14]);
// expcnt and lgkmcnt unconstrained
template <int N>
__device__ __forceinline__ void aw_wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit count");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

__device__ __forceinline__ void aw_lds_barrier() {
    // LDS traffic done, then the workgroup barrier; outstanding global loads
    // (the weight stream) stay in flight.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt unconstrained
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int MR, bool VEC>
__global__ __launch_bounds__(AW_THREADS) __attribute__((amdgpu_waves_per_eu(5, 5)))
void awq_gemv_kernel(int M, int N, int K, const uint16_t *__restrict__ x,
                     const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
                     const uint16_t *__restrict__ zeros, const uint16_t *__restrict__ bias,
                     uint16_t *__restrict__ out)
{
    // C registers in use: rows 8*(i/4) + 4*h + i%4 (h = lane/32), those < MR
    constexpr int NI = MR >= 8 ? MR / 2 : MR;
    // Dynamic LDS (sized by the launcher): the sums of x [group][row] plus
    // spare slots, then the x chunk (rows padded) plus one 16-byte surplus
    // slot; after the last chunk the x area holds the per-wave sums.
    extern __shared__ __align__(16) uint8_t aw_smem[];
    float *s_xs = (float *)aw_smem;
    uint8_t *s_x = aw_smem + aw_xs_bytes(MR);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar registers
    const int part = wave;   // this wave's K-part
    const int c32 = lane & 31, h = lane >> 5;
    const int NG = K >> 6;
    const int nbt = (N + AW_TILE_N - 1) / AW_TILE_N;
    const int bt = (int)(blockIdx.x % nbt), mt = (int)(blockIdx.x / nbt);
    const int m0 = mt * MR;
    const int Mt = min(MR, M - m0);
    const int nt0 = bt * AW_TILE_N;
    // Weight-side loads address from this tile's first row (a wave-uniform base
    // in scalar registers) plus a 32-bit lane offset.  Rows past N read row N-1
    // (their outputs are never stored).
    const int nl = min(c32, N - 1 - nt0);
    const uint8_t *cbase = codes + (size_t)nt0 * (size_t)(K >> 1);
    const uint8_t *sbase = (const uint8_t *)(scales + (size_t)nt0 * NG);
    const uint8_t *zbase = (const uint8_t *)(zeros + (size_t)nt0 * NG);
    const uint32_t coff = (uint32_t)(nl * (K >> 1) + 16 * h);   // bytes: this lane's row and half
    const uint32_t soff = (uint32_t)(nl * NG * 2);              // bytes: this lane's row of scales
    const uint16_t *xt = x + (size_t)m0 * (size_t)K;

    const int cg_max = aw_chunk_groups(Mt, VEC);
    const int xstride = cg_max * 128 + AW_XPAD;           // bytes per staged row
    const int arow = min(c32, Mt - 1) * xstride + 64 * h;  // this lane's A row and half

    float y[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) y[i] = 0.0f;
    // The nibble mask lives in a register so that each unpack is one
    // v_and_or_b32 (a VOP3 instruction cannot take two literal constants).
    uint32_t nib_mask = 0x000F000Fu;
    asm volatile("" : "+v"(nib_mask));

    // code ring: 2 quads of 4 groups; scale/zero ring: one 4-group word pair per quad
    v4u rc[2][4];
    v2u rs[2], rz[2];
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;

    for (int cb = 0; cb < NG; cb += cg_max) {
        const int cg = min(cg_max, NG - cb);
        // ---- this wave's groups of the chunk (two quads of codes = 8 groups in flight)
        const int gs = cb + (cg * part) / AW_KP, ge = cb + (cg * (part + 1)) / AW_KP;
        const int nw = ge - gs;
        const int nq = (nw + 3) >> 2;
        auto load_quad = [&](int Q, auto slot_c) __attribute__((always_inline)) {
            constexpr int S = decltype(slot_c)::value;
            // groups are clamped to the wave's last (surplus copies are never used)
            const int g4 = gs + 4 * min(Q, nq - 1);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                rc[S][j] = *(const v4u *)(cbase + coff + (uint32_t)min(g4 + j, ge - 1) * 32u);
            if constexpr (VEC) {
                rs[S] = *(const v2u *)(sbase + soff + (uint32_t)g4 * 2u);
                rz[S] = *(const v2u *)(zbase + soff + (uint32_t)g4 * 2u);
            } else {
                uint32_t sv[4], zv[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t o = soff + (uint32_t)min(g4 + j, ge - 1) * 2u;
                    sv[j] = *(const uint16_t *)(sbase + o);
                    zv[j] = *(const uint16_t *)(zbase + o);
                }
                rs[S] = v2u{sv[0] | (sv[1] << 16), sv[2] | (sv[3] << 16)};
                rz[S] = v2u{zv[0] | (zv[1] << 16), zv[2] | (zv[3] << 16)};
            }
            asm volatile("" ::: "memory");   // keep the loads here, ahead of their use
            __builtin_amdgcn_sched_barrier(0);
        };
        const int P = Mt * cg * 8, cg8 = cg * 8;
        // one 16-byte piece of x: permuted in place to the codes' pair order
        // (p, p+4) and summed; the 8 pieces of a group sit in 8 consecutive lanes
        auto stage_piece = [&](const v4u &r, int idx, int m, int q) __attribute__((always_inline)) {
            v4u pr;
            pr[0] = __builtin_amdgcn_perm(r[2], r[0], 0x05040100u);
            pr[1] = __builtin_amdgcn_perm(r[2], r[0], 0x07060302u);
            pr[2] = __builtin_amdgcn_perm(r[3], r[1], 0x05040100u);
            pr[3] = __builtin_amdgcn_perm(r[3], r[1], 0x07060302u);
            float sx = 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) sx += bf16_lo(r[e]) + bf16_hi(r[e]);
            sx += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, sx), 0xB1, 0xF, 0xF, true));
            sx += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, sx), 0x4E, 0xF, 0xF, true));
            sx += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, sx), 0x141, 0xF, 0xF, true));
            // surplus pieces and the 7 non-leading lanes of each group's sum write to spare slots
            const bool ok = idx < P;
            const int xo = ok ? m * xstride + q * 16 : Mt * xstride;
            const int so = (ok && (q & 7) == 0) ? (q >> 3) * MR + m : AW_MAXCG * MR;
            *(v4u *)(s_x + xo) = pr;
            s_xs[so] = sx;
        };
        const float rcg8 = 1.0f / (float)cg8;
        // ---- x first: the chunk is copied global -> LDS (row m: cg*128 bytes
        // in 1 KB copies; a last partial copy reads clamped, valid elements of
        // the row into the rest of the row's stride), then the first two quads
        // of codes go out behind it.  Memory operations complete in order, so
        // waiting until at most those quads' loads are outstanding means this
        // wave's copies have landed, while the codes stay in flight; no copy
        // is pending after the barrier, so every later wait on the codes is
        // for exactly the group about to be used.
        const int per_row = (cg + 7) >> 3, copies = Mt * per_row;
        for (int j = wave; j < copies; j += AW_KP) {
            const int m = j / per_row, pc = j - m * per_row;
            const int e = min(cb * 64 + pc * 512 + lane * 8, K - 8);
            __builtin_amdgcn_global_load_lds((gptr_t)(xt + (size_t)m * K + e),
                                             (lptr_t)(s_x + m * xstride + pc * 1024), 16, 0, 0);
        }
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        if (nw > 0) {
            load_quad(0, I0{});
            load_quad(1, I1{});
            aw_wait_vmcnt<2 * aw_quad_loads(VEC)>();
        } else {
            aw_wait_vmcnt<0>();
        }
        aw_lds_barrier();
        for (int i0 = 0; i0 < P; i0 += AW_THREADS) {
            const int idx = i0 + tid;
            int m, q;
            aw_divmod(min(idx, P - 1), cg8, rcg8, m, q);
            stage_piece(*(const v4u *)(s_x + m * xstride + q * 16), idx, m, q);
        }
        aw_lds_barrier();

        // ---- the wave's groups: 4 MFMAs per group, then the group epilogue
        auto group = [&](int g, const v4u &cw, uint32_t sw, uint32_t zw, bool hi16)
            __attribute__((always_inline)) {
            __builtin_amdgcn_sched_barrier(0);   // one group's operands live at a time
            const int gl = g - cb;
            v16f c = {};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // one step's fragments at a time (registers are the occupancy limit)
                const v4u a = *(const v4u *)(s_x + arow + gl * 128 + 16 * j);
                const uint32_t d = cw[j];
                v4u b;
#pragma unroll
                for (int p = 0; p < 4; ++p) b[p] = ((d >> (4 * p)) & nib_mask) | 0x43004300u;
                c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a),
                                                            __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
            const float sc = hi16 ? bf16_hi(sw) : bf16_lo(sw);
            const float zc = 128.0f + (hi16 ? bf16_hi(zw) : bf16_lo(zw));
            if constexpr (NI >= 4) {
#pragma unroll
                for (int ib = 0; ib < NI / 4; ++ib) {
                    const v4f xs = *(const v4f *)(s_xs + gl * MR + 8 * ib + 4 * h);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        y[4 * ib + i] = __builtin_fmaf(sc, __builtin_fmaf(-zc, xs[i], c[4 * ib + i]),
                                                       y[4 * ib + i]);
                }
            } else {
                // rows 4h + i: only h = 0 holds real rows; h = 1 reads spare entries
#pragma unroll
                for (int i = 0; i < NI; ++i)
                    y[i] = __builtin_fmaf(sc, __builtin_fmaf(-zc, s_xs[gl * MR + 4 * h + i], c[i]), y[i]);
            }
        };
        auto quad = [&](int Q, auto slot_c) __attribute__((always_inline)) {
            constexpr int S = decltype(slot_c)::value;
            __builtin_amdgcn_sched_barrier(0);
            const int g0 = gs + 4 * Q;
            // groups past the wave's last one are surplus loads: skipped
            group(g0, rc[S][0], rs[S][0], rz[S][0], false);
            if (g0 + 1 < ge) group(g0 + 1, rc[S][1], rs[S][0], rz[S][0], true);
            if (g0 + 2 < ge) group(g0 + 2, rc[S][2], rs[S][1], rz[S][1], false);
            if (g0 + 3 < ge) group(g0 + 3, rc[S][3], rs[S][1], rz[S][1], true);
        };
        // Quads beyond the first two reload the ring as it drains (K-parts
        // longer than 8 groups).
        if (nw > 0) {
            const int nfull = nq & ~1;
            for (int Q = 0; Q < nfull; Q += 2) {
                quad(Q, I0{});
                if (Q + 2 < nq) load_quad(Q + 2, I0{});
                quad(Q + 1, I1{});
                if (Q + 3 < nq) load_quad(Q + 3, I1{});
            }
            if (nfull < nq) quad(nfull, I0{});
        }
        aw_lds_barrier();   // the next chunk (or the final sums) overwrites s_x
    }

    // ---- add the K-parts through LDS, then bias, round, store
    float *s_part = (float *)s_x;   // per-wave sums [wave][MR][32], over the staged x
    float *mine = s_part + wave * (MR * 32);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int row = 8 * (i / 4) + 4 * h + (i % 4);
        if (row < MR) mine[row * 32 + c32] = y[i];
    }
    __syncthreads();
    for (int r = tid; r < MR * 32; r += AW_THREADS) {
        const int m = r >> 5, nn = r & 31;
        const int on = nt0 + nn;
        if (m < Mt && on < N) {
            float s = 0.0f;
#pragma unroll
            for (int pp = 0; pp < AW_KP; ++pp) s += s_part[pp * (MR * 32) + r];
            if (bias) s += bf16_to_f32(bias[on]);
            out[(size_t)(m0 + m) * N + on] = (uint16_t)f32_to_bf16_rne(s);
        }
    }
}

template <int MR>
static void launch_mr(bool vec, dim3 grid, hipStream_t stream, int M, int N, int K,
                      const uint16_t *xp, const uint8_t *cp, const uint16_t *sp, const uint16_t *zp,
                      const uint16_t *bp, uint16_t *op)
{
    // LDS: sums of x, then max(x chunk + surplus slot, per-wave sums); the
    // block with the most rows of x (min(M, MR)) sets the size
    const int Mt = M < MR ? M : MR;
    const int cg = aw_chunk_groups(Mt, vec);
    const int xbytes = Mt * (cg * 128 + AW_XPAD) + 16;
    const int pbytes = AW_KP * MR * 32 * 4;
    const size_t lds = (size_t)aw_xs_bytes(MR) + (size_t)(xbytes > pbytes ? xbytes : pbytes);
    if (vec)
        hipLaunchKernelGGL((awq_gemv_kernel<MR, true>), grid, dim3(AW_THREADS), lds, stream, M, N, K,
                           xp, cp, sp, zp, bp, op);
    else
        hipLaunchKernelGGL((awq_gemv_kernel<MR, false>), grid, dim3(AW_THREADS), lds, stream, M, N, K,
                           xp, cp, sp, zp, bp, op);
}

hipError_t launch_awq_gemv(int M, int N, int K, const void *x, const void *codes,
                           const void *scales, const void *zeros, const void *bias, void *out,
                           hipStream_t stream)
{
    // up to 8 rows of x: the whole-line streams of gemv_w4a16_lines.hip
    if (awq_gemv_lines_applies(M, N, K))
        return launch_awq_gemv_lines(M, N, K, x, codes, scales, zeros, bias, out, stream);
    if (awq_gemv_lines_mfma_applies(M, N, K))
        return launch_awq_gemv_lines_mfma(M, N, K, x, codes, scales, zeros, bias, out, stream);
    const int MR = M <= 2 ? 2 : (M <= 8 ? 8 : (M <= 16 ? 16 : 32));
    const int nmt = (M + MR - 1) / MR;
    const int Mt = M < MR ? M : MR;   // rows of the largest M-tile
    dim3 grid(((N + AW_TILE_N - 1) / AW_TILE_N) * nmt);
    const uint16_t *xp = (const uint16_t *)x, *sp = (const uint16_t *)scales,
                   *zp = (const uint16_t *)zeros, *bp = (const uint16_t *)bias;
    const uint8_t *cp = (const uint8_t *)codes;
    uint16_t *op = (uint16_t *)out;
    // 8-byte scale/zero loads need every K-part to start on a multiple of 4
    // groups, i.e. chunks of a multiple of 4 * AW_KP groups.  From 22 rows of x
    // on no such chunk fits the LDS budget (the rounding leaves 0 groups per
    // chunk, and the chunk loop would never advance): those tiles take the
    // 2-byte loads, which take any chunk of 8k groups (16 for 32 rows).
    // Smaller tiles of the same launch get at least as many groups.
    const bool vec = ((K >> 6) % (4 * AW_KP)) == 0 && aw_chunk_groups(Mt, true) > 0;
    switch (MR) {
        case 2: launch_mr<2>(vec, grid, stream, M, N, K, xp, cp, sp, zp, bp, op); break;
        case 8: launch_mr<8>(vec, grid, stream, M, N, K, xp, cp, sp, zp, bp, op); break;
        case 16: launch_mr<16>(vec, grid, stream, M, N, K, xp, cp, sp, zp, bp, op); break;
        default: launch_mr<32>(vec, grid, stream, M, N, K, xp, cp, sp, zp, bp, op); break;
    }
    return hipGetLastError();
}

}  // namespace svdq
