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
// RMSNorm + rotary step (EPI_QK); or, for the up projection of a GELU MLP,
// the next layer's whole activation step (EPI_GQ, below).
#include <utility>

#include "device_common.h"
#include "gelu_bf16.h"
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
constexpr int EPI_PLAIN = 0, EPI_QK = 1, EPI_GQ = 2;
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

// ---------------------------------------------------------------------------
// EPI_GQ: the up projection of a GELU MLP with the down layer's activation
// step in its epilogue ("Nunchaku Lite" docs, "Fused kernels": the original
// engine runs the MLP's GELU fused into its kernels), so the [M, N] bf16
// intermediate is never written.  For every output y (the layer's bf16
// result, the value svdq_gemm_w4a4 would store):
//   h = GELU_tanh(y) rounded to bf16 (the table of gelu_bf16.h),
//   x_hat = RNE_bf16(h / s_next[n])             (the next layer's smoothing),
// then per row and group of 64 columns the int4 rule (scale = absmax/7 as
// bf16, q = RNE(x_hat / scale)) with the codes written in the FP6 tiled
// layout, and the low-rank partial x_hat . lora_down_next^T over the block's
// 128 columns, one fp32 [M, rank_next] slice per column tile; a second
// kernel sums the slices in column-tile order (deterministic).
// The arithmetic is that of the activation step (quantize_act.hip): the
// smoothing as x * fl(1/s) with IEEE division for fp32-subnormal products
// and channels whose 1/s leaves fp32's normal range, the scale as
// absmax * fl(1/7), the quotient by one Newton step on v_rcp_f32.
// Work split: the accumulators pass through GELU and the smoothing in the
// MFMA layout (a lane's two columns share one 1/s each), x_hat goes to a
// row-major LDS tile, then thread t quantizes row t/2, group t%2 of the tile
// -- 64 values, 48 bytes of codes, all three 16-byte chunks of one (row,
// group) -- and wave w runs rows 32w..32w+31 of the low-rank partial on the
// matrix core.  Rows past M and groups past N are not written.
struct GeluQuantNext {
    const uint16_t *smooth;      // bf16 [N] or NULL (s = 1)
    const uint16_t *lora_down;   // bf16 [rank, N]
    int rank;                    // 0 or a multiple of 16 up to 128
    uint8_t *codes;              // FP6 tiled layout of [M, N]
    uint16_t *scales;            // bf16 [M, N/64]
    float *partial;              // fp32 [ceil(N/128)][M][rank]
};
constexpr int GQ_TAB_BYTES = GELU_TAB_PAD * 2;
constexpr int GQ_INV_OFF = GQ_TAB_BYTES;                 // float [128]: 1/s of the tile's columns
constexpr int GQ_ROWB = 128 * 2 + 16;                    // x_hat tile row (bf16, padded)
constexpr int GQ_TILE_OFF = GQ_INV_OFF + 128 * 4;
constexpr int GQ_SMEM = GQ_TILE_OFF + 128 * GQ_ROWB;
static_assert(F6_SMEM >= GQ_SMEM, "the GELU-quantize epilogue uses the operand LDS");
static_assert(GQ_TILE_OFF % 16 == 0, "16-byte LDS rows");

// lora_act[i] = sum over column tiles b of partial[b][i], in a fixed order:
// four threads share 4 consecutive values, thread j summing the tiles
// b = j, j + 4, j + 8, ... in turn, then the four sums are added as
// ((s0 + s1) + s2) + s3 -- the same bits on every run.
__global__ __launch_bounds__(256) void gq_partial_sum_kernel(int64_t n, int nparts, const float *__restrict__ part,
                                                             float *__restrict__ lora_act) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int j = (int)(t & 3);
    const int64_t i = (t >> 2) * 4;
    v4f s = v4f{0.f, 0.f, 0.f, 0.f};
    if (i < n) {
#pragma unroll 6
        for (int b = j; b < nparts; b += 4) {
            const v4f v = *(const v4f *)(part + (size_t)b * (size_t)n + i);
            s = v4f{s[0] + v[0], s[1] + v[1], s[2] + v[2], s[3] + v[3]};
        }
    }
    v4f o[4];
    o[0] = s;
#pragma unroll
    for (int d = 1; d < 4; ++d)
#pragma unroll
        for (int c = 0; c < 4; ++c) o[d][c] = __shfl_down(s[c], d, 64);
    if (j == 0 && i < n) {
        v4f r = o[0];
#pragma unroll
        for (int d = 1; d < 4; ++d) r = v4f{r[0] + o[d][0], r[1] + o[d][1], r[2] + o[d][2], r[3] + o[d][3]};
        *(v4f *)(lora_act + i) = r;
    }
}

// What the epilogue reads from global memory, loaded before the layer's
// own epilogue sum so that the latency of these loads overlaps it: this
// thread's pieces of the GELU table, the smoothing factor of column tid
// (tid < 128), and this lane's low-rank operand for the first 32 ranks.
struct GqPrefetch {
    v4u tab[3];
    uint32_t smooth;
    v4u down[8];
};
constexpr int GQ_TAB_CHUNKS = GQ_TAB_BYTES / 16;
static_assert(GQ_TAB_CHUNKS <= 3 * F6_THREADS, "three table pieces per thread");

__device__ __forceinline__ void gq_prefetch(GqPrefetch &pf, const GeluQuantNext &gq, int N, int n0, int tid,
                                            int lane) {
#pragma unroll
    for (int u = 0; u < 3; ++u) {
        const int i = tid + u * F6_THREADS;
        if (i < GQ_TAB_CHUNKS) pf.tab[u] = ((const v4u *)g_gelu_table.data())[i];
    }
    pf.smooth = 0x3F80u;                                  // bf16 1.0
    if (tid < 128 && gq.smooth && n0 + tid < N) pf.smooth = gq.smooth[n0 + tid];
    const int l32 = lane & 31, h = lane >> 5;
    const bool jok = l32 < gq.rank;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        const int k = 16 * ks + 8 * h;
        pf.down[ks] = (jok && n0 + k < N) ? *(const v4u *)(gq.lora_down + (size_t)l32 * (size_t)N + n0 + k)
                                          : v4u{0u, 0u, 0u, 0u};
    }
}

// Called by all 256 threads after gemm_epilogue_sum (acc = the fp32 result
// before its rounding to bf16).
__device__ __forceinline__ void gemm_epilogue_gelu_quant(v16f (&acc)[2][2], int M, int N, int m0, int n0, int wm,
                                                         int wn, int lane, const GeluQuantNext &gq,
                                                         const GqPrefetch &pf, uint8_t *smem)
{
    const int tid = threadIdx.x;
    const int l32 = lane & 31, h = lane >> 5;
    uint16_t *tab = (uint16_t *)smem;
    float *s_inv = (float *)(smem + GQ_INV_OFF);
    uint8_t *xt = smem + GQ_TILE_OFF;
    __syncthreads();   // every wave is done with the operand stages
#pragma unroll
    for (int u = 0; u < 3; ++u) {
        const int i = tid + u * F6_THREADS;
        if (i < GQ_TAB_CHUNKS) ((v4u *)smem)[i] = pf.tab[u];
    }
    int unsafe = 0;
    if (tid < 128) {
        const float sf = bf16_to_f32((uint16_t)pf.smooth);
        const float as = fabsf(sf);
        const bool ok = (as >= 0x1p-64f) && (as <= 0x1p64f);
        s_inv[tid] = ok ? 1.0f / sf : 0.0f;
        unsafe = ok ? 0 : 1;
    }
    unsafe = __syncthreads_or(unsafe);

    // ---- y -> GELU -> smoothing -> x_hat (bf16) into the LDS tile
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int c = wn * 64 + b * 32 + l32;             // column within the tile
        const bool col_ok = n0 + c < N;
        const float iv = s_inv[c];
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            uint32_t y[8], g[8];
            u16x2 tmax = (u16x2)(unsigned short)0;
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                y[p] = pack_bf16x2_rne(acc[a][b][2 * p], acc[a][b][2 * p + 1]);
                g[p] = gelu_lookup2_track(y[p], tab, tmax);
            }
            gelu_resolve(g, y, tmax, tab);
            float v[16];
            int bad = 0;
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                v[2 * p] = bf16_lo(g[p]) * iv;
                v[2 * p + 1] = bf16_hi(g[p]) * iv;
                bad |= __builtin_amdgcn_class(v[2 * p], 0x90) | __builtin_amdgcn_class(v[2 * p + 1], 0x90);
            }
            if (__builtin_expect(unsafe | __any(bad), 0)) {
                const float sf = (gq.smooth && col_ok) ? bf16_to_f32(gq.smooth[n0 + c]) : 1.0f;
#pragma unroll
                for (int p = 0; p < 8; ++p) {
                    v[2 * p] = bf16_lo(g[p]) / sf;
                    v[2 * p + 1] = bf16_hi(g[p]) / sf;
                }
            }
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const uint32_t xh = col_ok ? pack_bf16x2_rne(v[2 * p], v[2 * p + 1]) : 0u;
                const int row = wm * 64 + a * 32 + 8 * (p >> 1) + 4 * h + 2 * (p & 1);
                *(uint16_t *)(xt + row * GQ_ROWB + 2 * c) = (uint16_t)xh;
                *(uint16_t *)(xt + (row + 1) * GQ_ROWB + 2 * c) = (uint16_t)(xh >> 16);
            }
        }
    }
    __syncthreads();

    // ---- group quantization: thread t takes row t/2, group t%2 of the tile
    {
        const int r = tid >> 1, gh = tid & 1;
        const int grow = m0 + r, gcol = n0 + 64 * gh;
        const uint8_t *xr = xt + r * GQ_ROWB + 128 * gh;
        float q[64];
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const v4u xv = *(const v4u *)(xr + 16 * j);
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                q[8 * j + 2 * p] = bf16_lo(xv[p]);
                q[8 * j + 2 * p + 1] = bf16_hi(xv[p]);
                amax = max3_abs(amax, q[8 * j + 2 * p], q[8 * j + 2 * p + 1]);
            }
        }
        const uint32_t sbits = f32_to_bf16_rne(amax * (1.0f / 7.0f));
        const float sb = __uint_as_float(sbits << 16);
        if (__builtin_expect(sb < 0x1p-100f, 0)) {
            // tiny or zero scale: IEEE division (a zero scale gives zero codes)
#pragma unroll
            for (int e = 0; e < 64; ++e)
                q[e] = sb == 0.0f ? 0.0f
                                  : (__builtin_amdgcn_fmed3f(q[e] / sb, -8.0f, 7.0f) + 12582912.0f) - 12582912.0f;
        } else {
            // |x_hat| <= absmax and sb >= (absmax / 7)(1 - 2^-8), so |q| <= 7.03
            // rounds into [-7, 7]: no clamp.  Rounding to the nearest integer
            // (ties to even) by adding and subtracting 1.5 * 2^23, which also
            // gives +0 for every zero code (the layout's zero).
            const float inv = __builtin_amdgcn_rcpf(sb);
#pragma unroll
            for (int e = 0; e < 64; ++e) {
                const float qe = q[e] * inv;
                const float rr = __builtin_fmaf(-qe, sb, q[e]);
                const float qc = __builtin_fmaf(rr, inv, qe);
                q[e] = (qc + 12582912.0f) - 12582912.0f;
            }
        }
        // the two 192-bit strings (channels 32hh + j in field j, values q/2)
        uint32_t hs[2][6];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            v16f fa, fb;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                fa[i] = q[32 * hh + 2 * i];
                fb[i] = q[32 * hh + 2 * i + 1];
            }
            const auto f = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(fa, fb, 2.0f);
#pragma unroll
            for (int d = 0; d < 6; ++d) hs[hh][d] = f[d];
        }
        if (grow < M && gcol < N) {
            const int g = gcol >> 6;
            const int NP = ((N >> 6) + 1) >> 1;
            const bool sw = fp6_half_swap(r);
            *(v4u *)(gq.codes + fp6_tiled_chunk(grow, g, 0, NP)) = v4u{hs[0][0], hs[0][1], hs[0][2], hs[0][3]};
            *(v4u *)(gq.codes + fp6_tiled_chunk(grow, g, 1, NP)) = v4u{hs[1][0], hs[1][1], hs[1][2], hs[1][3]};
            *(v4u *)(gq.codes + fp6_tiled_chunk(grow, g, 2, NP)) =
                sw ? v4u{hs[1][4], hs[1][5], hs[0][4], hs[0][5]} : v4u{hs[0][4], hs[0][5], hs[1][4], hs[1][5]};
            gq.scales[(size_t)grow * (size_t)(N >> 6) + g] = (uint16_t)sbits;
        }
    }

    // ---- low-rank partial of the block's columns: wave w, rows 32w..32w+31
    if (gq.rank > 0) {
        const int w = tid >> 6;
        float *pp = gq.partial + (size_t)(n0 >> 7) * (size_t)M * (size_t)gq.rank;
        for (int rc = 0; rc < gq.rank; rc += 32) {
            const int j = rc + l32;
            const bool jok = j < gq.rank;
            v16f t = {};
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const int k = 16 * ks + 8 * h;
                const v4u av = *(const v4u *)(xt + (32 * w + l32) * GQ_ROWB + 2 * k);
                v4u bv = pf.down[ks];                        // ranks 0..31: loaded up front
                if (rc > 0)
                    bv = (jok && n0 + k < N) ? *(const v4u *)(gq.lora_down + (size_t)j * (size_t)N + n0 + k)
                                             : v4u{0u, 0u, 0u, 0u};
                t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, av),
                                                           __builtin_bit_cast(v8bf, bv), t, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = m0 + 32 * w + 8 * (i >> 2) + 4 * h + (i & 3);
                if (jok && row < M) pp[(size_t)row * (size_t)gq.rank + j] = t[i];
            }
        }
    }
}

// SC4: K/64 a multiple of 4 (scales of 4 groups per 8-byte load);
// GROUP_SUMS: write X_g (int32 [M][N][K/64]) instead of the layer's output;
// EPI: EPI_PLAIN, EPI_QK (grouped QKV layer: gemm_epilogue_qk for the Q and K
// heads) or EPI_GQ (the next layer's activation step, gemm_epilogue_gelu_quant;
// out, if not NULL, also receives the layer's output)
template <bool GROUP_SUMS, bool SC4, int EPI>
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
                          QkNormRope qk, GeluQuantNext gq)
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
        if constexpr (EPI == EPI_QK) {
            gemm_epilogue_sum(acc, alpha, M, N, rank, m0, n0, wm, wn, lane, lora_act, lora_up, bias);
            if (n0 < qk.qk_cols)   // block-uniform: a Q or K head
                gemm_epilogue_qk(acc, M, m0, n0, wm, wn, lane, qk, smem, N, out);
            else
                gemm_epilogue_store(acc, M, N, m0, n0, wm, wn, lane, out);
        } else if constexpr (EPI == EPI_GQ) {
            GqPrefetch pf;
            gq_prefetch(pf, gq, N, n0, tid, lane);
            gemm_epilogue_sum(acc, alpha, M, N, rank, m0, n0, wm, wn, lane, lora_act, lora_up, bias);
            if (out) gemm_epilogue_store(acc, M, N, m0, n0, wm, wn, lane, out);
            gemm_epilogue_gelu_quant(acc, M, N, m0, n0, wm, wn, lane, gq, pf, smem);
        } else {
            gemm_epilogue(acc, alpha, M, N, rank, m0, n0, wm, wn, lane, lora_act, lora_up, bias, out);
        }
    }
}

template <bool GROUP_SUMS, int EPI>
static hipError_t launch_fp6(int M, int N, int K, int rank, const void *act_codes, const void *act_scales,
                             const void *wgt_codes, const void *wgt_scales, float alpha, const float *lora_act,
                             const void *lora_up, const void *bias, void *out, int32_t *G, const QkNormRope &qk,
                             const GeluQuantNext &gq, hipStream_t stream)
{
    dim3 grid(((N + F6_BN - 1) / F6_BN) * ((M + F6_BM - 1) / F6_BM)), block(F6_THREADS);
#define F6_LAUNCH(SC)                                                                                             \
    hipLaunchKernelGGL((gemm_w4a4_fp6_kernel<GROUP_SUMS, SC, EPI>), grid, block, 0, stream, M, N, K, rank,       \
                       (const uint8_t *)act_codes, (const uint16_t *)act_scales, (const uint8_t *)wgt_codes,     \
                       (const uint16_t *)wgt_scales, alpha, lora_act, (const uint16_t *)lora_up,                  \
                       (const uint16_t *)bias, (uint16_t *)out, G, qk, gq)
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
    const GeluQuantNext no_gq{};
    return launch_fp6<false, EPI_PLAIN>(M, N, K, rank, act_codes, act_scales, wgt_codes, wgt_scales, alpha,
                                        lora_act, lora_up, bias, out, nullptr, none, no_gq, stream);
}

hipError_t launch_gemm_w4a4_fp6_qk(int M, int N, int K, int rank, const void *act_codes, const void *act_scales,
                                   const void *wgt_codes, const void *wgt_scales, float alpha,
                                   const float *lora_act, const void *lora_up, const void *bias,
                                   const QkNormRope &qk, void *out, hipStream_t stream)
{
    const GeluQuantNext no_gq{};
    return launch_fp6<false, EPI_QK>(M, N, K, rank, act_codes, act_scales, wgt_codes, wgt_scales, alpha, lora_act,
                                     lora_up, bias, out, nullptr, qk, no_gq, stream);
}

// Workspace of the GELU-quantize form: the low-rank partials
// [ceil(N/128)][M][rank_next] (fp32).
size_t gelu_quant_workspace_bytes(int M, int N, int rank_next)
{
    return (size_t)((N + F6_BN - 1) / F6_BN) * (size_t)M * (size_t)rank_next * 4u;
}

hipError_t launch_gemm_w4a4_fp6_gelu_quant(int M, int N, int K, int rank, const void *act_codes,
                                           const void *act_scales, const void *wgt_codes, const void *wgt_scales,
                                           float alpha, const float *lora_act, const void *lora_up,
                                           const void *bias, int rank_next, const void *smooth_next,
                                           const void *lora_down_next, void *next_codes, void *next_scales,
                                           float *next_lora_act, void *workspace, void *out, hipStream_t stream)
{
    float *partial = (float *)workspace;
    GeluQuantNext gq;
    gq.smooth = (const uint16_t *)smooth_next;
    gq.lora_down = (const uint16_t *)lora_down_next;
    gq.rank = rank_next;
    gq.codes = (uint8_t *)next_codes;
    gq.scales = (uint16_t *)next_scales;
    gq.partial = partial;
    const QkNormRope none{};
    const hipError_t e = launch_fp6<false, EPI_GQ>(M, N, K, rank, act_codes, act_scales, wgt_codes, wgt_scales, alpha, lora_act,
                                  lora_up, bias, out, nullptr, none, gq, stream);
    if (e != hipSuccess || rank_next == 0) return e;
    const int64_t n = (int64_t)M * rank_next;
    const int64_t blocks = (n + 255) / 256;          // four threads per 4 values
    hipLaunchKernelGGL(gq_partial_sum_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, n,
                       (N + F6_BN - 1) / F6_BN, (const float *)partial, next_lora_act);
    return hipGetLastError();
}

// the GEMM's own main loop (same stages, copies and matrix instructions)
// writing X_g instead of accumulating
hipError_t launch_group_sums_fp6(int M, int N, int K, const void *act_codes, const void *wgt_codes, int32_t *G,
                                 hipStream_t stream)
{
    const QkNormRope none{};
    const GeluQuantNext no_gq{};
    return launch_fp6<true, EPI_PLAIN>(M, N, K, 0, act_codes, nullptr, wgt_codes, nullptr, 1.0f, nullptr, nullptr,
                                       nullptr, nullptr, G, none, no_gq, stream);
}

}  // namespace svdq
