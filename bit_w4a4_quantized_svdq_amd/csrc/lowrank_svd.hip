// lowrank_svd.hip -- the 16-bit low-rank branch of a smoothed weight on
// gfx950: the top-r singular triplets of W_hat = W diag(s) (blog "Hugging Face
// integrates Nunchaku 4-bit diffusion inference into Diffusers", section
// "SVDQuant and the Nunchaku engine": the hardest part of each weight is kept
// in a small 16-bit low-rank branch), as
//     lora_up[n,j] = RNE_bf16(U[n,j]),  lora_down[j,k] = RNE_bf16(sigma_j V[k,j]),
// signs canonical (each left vector's largest-magnitude entry positive).
//
// Method: randomized subspace iteration (range finder with a Gaussian sketch
// of l = r + 8 columns and two power iterations), every basis re-orthonormal-
// ized by CholeskyQR2 (fp64 Gram matrices); then B = Q^T W_hat, whose small
// l x l Gram matrix B B^T is diagonalized by parallel (round-robin) Jacobi in
// fp64 within one workgroup; U = Q E, Sigma V^T = E^T B.  The result is an
// approximation of the exact truncated SVD: its residual norm is within a
// small factor of the Eckart-Young optimum, closer the faster the spectrum
// decays.
//
// Kernels: a tiled fp32 product (W_hat or an fp32 basis against an l-column
// block, plain or transposed), fp64 Gram partials + reduction, and three
// single-workgroup steps (Cholesky with triangular inverse, Jacobi, final sort
// and signs).  All scratch lives in a caller-provided workspace, or, for
// callers that cannot allocate, in this file's fixed device array `scratch`.
#include <algorithm>
#include <mutex>

#include "device_common.h"
#include "launch.h"

namespace svdq {

constexpr int SV_OVERSAMPLE = 8;
constexpr int SV_MAXL = 128 + SV_OVERSAMPLE;   // largest l
constexpr int SV_JC = (SV_MAXL + 15) / 16;       // output columns per thread (stride 16)
constexpr int SV_GROWS = 256;                    // rows per Gram partial

// ---------------------------------------------------------------- products
// out[i][c] = sum_t A(i,t) X[t][c]  (i < I, c < L, t < T), fp32 accumulation.
//   !TRANS: A(i,t) = a[i*T + t] * s[t]   (a: [I x T] row-major)
//   TRANS:  A(i,t) = a[t*I + i] * s[i]   (a: [T x I] row-major)
// s == nullptr means 1.  Block: 64 output rows, all L columns; thread: 4 rows
// x ceil(L/16) columns.  blockIdx.y takes the reduction slice [y*tsplit,
// (y+1)*tsplit) and writes its partial sums to out + y*I*L (summed afterwards
// in slice order by sv_sum_kernel).
template <typename TA, bool TRANS>
__global__ __launch_bounds__(256) void sv_product_kernel(int I, int T, int L, const TA *__restrict__ a,
                                                         const uint16_t *__restrict__ s,
                                                         const float *__restrict__ X, float *__restrict__ out,
                                                         int tsplit)
{
    const int tb = blockIdx.y * tsplit, te = min(T, tb + tsplit);
    out += (size_t)blockIdx.y * I * L;
    __shared__ float As[32][64];
    __shared__ float Xs[32][SV_MAXL];
    const int tid = threadIdx.x, ri = tid >> 4, cg = tid & 15;
    const int i0 = blockIdx.x * 64;
    float acc[4][SV_JC];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < SV_JC; ++j) acc[u][j] = 0.0f;
    auto aval = [&](int i, int t) -> float {
        if (i >= I || t >= te) return 0.0f;
        float v;
        if constexpr (sizeof(TA) == 2) v = bf16_to_f32(TRANS ? a[(size_t)t * I + i] : a[(size_t)i * T + t]);
        else v = TRANS ? a[(size_t)t * I + i] : a[(size_t)i * T + t];
        if (s) v *= bf16_to_f32(s[TRANS ? i : t]);
        return v;
    };
    for (int t0 = tb; t0 < te; t0 += 32) {
        __syncthreads();
        if constexpr (sizeof(TA) == 2) {
            // bf16 W: 8 consecutive elements of a row of `a` per thread, one
            // 16-byte load (and one of s).  The chunk is wholly inside or
            // outside: I (TRANS) resp. T and the slice bounds (!TRANS) are
            // multiples of 8, and a and s are 16-byte aligned.
            const int tt = TRANS ? tid >> 3 : (tid & 3) * 8, ii = TRANS ? (tid & 7) * 8 : tid >> 2;
            const int i = i0 + ii, t = t0 + tt;
            float v[8];
            if (i < I && t < te) {
                const v4u w = *(const v4u *)(TRANS ? a + (size_t)t * I + i : a + (size_t)i * T + t);
                const v4u sc = s ? *(const v4u *)(s + (TRANS ? i : t)) : v4u{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    v[2 * q] = bf16_lo(w[q]) * bf16_lo(sc[q]);
                    v[2 * q + 1] = bf16_hi(w[q]) * bf16_hi(sc[q]);
                }
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q) v[q] = 0.0f;
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                if constexpr (TRANS) As[tt][ii + q] = v[q];
                else As[tt + q][ii] = v[q];
            }
        } else {
            for (int e = tid; e < 32 * 64; e += 256) {
                const int tt = TRANS ? e >> 6 : e & 31, ii = TRANS ? e & 63 : e >> 5;   // contiguous along a's rows
                As[tt][ii] = aval(i0 + ii, t0 + tt);
            }
        }
        for (int e = tid; e < 32 * L; e += 256) {
            const int tt = e / L, c = e - tt * L;
            Xs[tt][c] = t0 + tt < te ? X[(size_t)(t0 + tt) * L + c] : 0.0f;
        }
        __syncthreads();
#pragma unroll 4
        for (int tt = 0; tt < 32; ++tt) {
            float av[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) av[u] = As[tt][4 * ri + u];
#pragma unroll
            for (int j = 0; j < SV_JC; ++j) {
                const int c = cg + 16 * j;
                const float xv = c < L ? Xs[tt][c] : 0.0f;
#pragma unroll
                for (int u = 0; u < 4; ++u) acc[u][j] = __builtin_fmaf(av[u], xv, acc[u][j]);
            }
        }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int i = i0 + 4 * ri + u;
        if (i >= I) continue;
#pragma unroll
        for (int j = 0; j < SV_JC; ++j) {
            const int c = cg + 16 * j;
            if (c < L) out[(size_t)i * L + c] = acc[u][j];
        }
    }
}

// out[e] = sum_{y < S} part[y*n + e], in slice order
__global__ __launch_bounds__(256) void sv_sum_kernel(int S, long long n, const float *__restrict__ part,
                                                     float *__restrict__ out)
{
    const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
    if (e >= n) return;
    float v = 0.0f;
    for (int y = 0; y < S; ++y) v += part[(size_t)y * n + e];
    out[e] = v;
}

// ---------------------------------------------------------------- Gram matrices
// part[b] = sum over rows r in block b's range of X[r]^T X[r] (upper triangle, fp64)
__global__ __launch_bounds__(256) void sv_gram_partial_kernel(int R, int L, const float *__restrict__ X,
                                                              double *__restrict__ part)
{
    __shared__ float Xs[64][SV_MAXL];
    const int r0 = blockIdx.x * SV_GROWS;
    const int npair = L * (L + 1) / 2;
    double acc[(SV_MAXL * (SV_MAXL + 1) / 2 + 255) / 256];
    constexpr int NP = (SV_MAXL * (SV_MAXL + 1) / 2 + 255) / 256;
#pragma unroll
    for (int q = 0; q < NP; ++q) acc[q] = 0.0;
    for (int rc = 0; rc < SV_GROWS; rc += 64) {
        __syncthreads();
        for (int e = threadIdx.x; e < 64 * L; e += 256) {
            const int rr = e / L, c = e - rr * L;
            const int r = r0 + rc + rr;
            Xs[rr][c] = r < R ? X[(size_t)r * L + c] : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < NP; ++q) {
            const int p = threadIdx.x + 256 * q;
            if (p >= npair) continue;
            // pair p -> (i, j), i <= j, row-major over the upper triangle
            int i = 0, rem = p;
            while (rem >= L - i) { rem -= L - i; ++i; }
            const int j = i + rem;
            double sacc = 0.0;
            for (int rr = 0; rr < 64; ++rr) sacc += (double)Xs[rr][i] * (double)Xs[rr][j];
            acc[q] += sacc;
        }
    }
#pragma unroll
    for (int q = 0; q < NP; ++q) {
        const int p = threadIdx.x + 256 * q;
        if (p < npair) part[(size_t)blockIdx.x * npair + p] = acc[q];
    }
}

// G = sum of the partials, as a full symmetric L x L matrix.  32 lanes per
// entry: lane l adds partials l, l+32, ... in order, then a fixed butterfly
// over the 32 lanes (the same order on every run).
constexpr int SV_RED_PAIRS = 8;   // entries per 256-thread block
__global__ __launch_bounds__(256) void sv_gram_reduce_kernel(int nb, int L, const double *__restrict__ part,
                                                             double *__restrict__ G)
{
    const int npair = L * (L + 1) / 2;
    const int p = blockIdx.x * SV_RED_PAIRS + (threadIdx.x >> 5), l = threadIdx.x & 31;
    double s = 0.0;
    if (p < npair)
        for (int b = l; b < nb; b += 32) s += part[(size_t)b * npair + p];
    for (int o = 16; o > 0; o >>= 1) s += __shfl_xor(s, o, 32);
    if (p < npair && l == 0) {
        int i = 0, rem = p;
        while (rem >= L - i) { rem -= L - i; ++i; }
        const int j = i + rem;
        G[i * L + j] = s;
        G[j * L + i] = s;
    }
}

// ---------------------------------------------------------------- CholeskyQR step
// G (L x L, fp64) -> T = L^{-T} (upper triangular, fp32) for X <- X T, where
// G + delta I = L L^T; delta = 1e-13 trace / L (1e-300 for a zero matrix)
// keeps a rank-deficient basis from breaking down.  Both steps are written
// so that every thread of the block has work at every column: the factor by
// right-looking elimination (scale column j, then a rank-1 update of the
// trailing lower triangle), the inverse by column-oriented forward
// substitution (row j of L^{-1} is final once divided by L[j][j], and is
// then eliminated from the rows below).  IN_LDS: the factor and the inverse
// in LDS (2 L^2 doubles); else in global memory (Lg, Xg).
template <bool IN_LDS>
__global__ __launch_bounds__(256) void sv_chol_inv_kernel(int L, const double *__restrict__ Gg, double *__restrict__ Lg,
                                                          double *__restrict__ Xg, float *__restrict__ Tout)
{
    extern __shared__ double sv_dyn[];
    __shared__ double shift;
    __shared__ double diag[SV_MAXL];
    double *A = Lg, *Xi = Xg;   // A: G + delta I, factored in place (strict lower triangle; diagonal in diag[])
    if constexpr (IN_LDS) {
        A = sv_dyn;
        Xi = sv_dyn + L * L;
    }
    const int tid = threadIdx.x;
    for (int e = tid; e < L * L; e += 256) {
        A[e] = Gg[e];
        Xi[e] = (e / L == e % L) ? 1.0 : 0.0;
    }
    __syncthreads();
    if (tid == 0) {
        double tr = 0.0;
        for (int i = 0; i < L; ++i) tr += A[i * L + i];
        shift = tr > 0.0 ? 1e-13 * tr / L : 1e-300;
    }
    __syncthreads();
    for (int i = tid; i < L; i += 256) A[i * L + i] += shift;
    __syncthreads();
    // The diagonal of the factor goes to diag[] (every thread computes it from
    // the untouched A[j][j]), so a column needs two barriers, not three.
    for (int j = 0; j < L; ++j) {
        const double d = A[j * L + j];
        const double djj = __builtin_sqrt(d > 0.0 ? d : shift);
        if (tid == 0) diag[j] = djj;
        for (int i = j + 1 + tid; i < L; i += 256) A[i * L + j] /= djj;
        __syncthreads();
        const int m = L - 1 - j;   // trailing block: rows and columns j+1 .. L-1
        for (int e = tid; e < m * m; e += 256) {
            const int i = j + 1 + e / m, k = j + 1 + e % m;
            if (k <= i) A[i * L + k] -= A[i * L + j] * A[k * L + j];
        }
        __syncthreads();
    }
    // Rows of L^{-1} are kept undivided: row j's final value is Xi[j][:] /
    // diag[j], formed by every thread that eliminates it (one barrier per row).
    for (int j = 0; j < L; ++j) {
        const double ljj = diag[j];
        const int m = L - 1 - j, w = j + 1;   // rows j+1 .. L-1, columns 0 .. j
        for (int e = tid; e < m * w; e += 256) {
            const int i = j + 1 + e / w, c = e % w;
            Xi[i * L + c] -= A[i * L + j] * (Xi[j * L + c] / ljj);
        }
        __syncthreads();
    }
    // T[c][i] = (L^{-1})[i][c]
    for (int e = tid; e < L * L; e += 256) {
        const int i = e / L, c = e - i * L;
        Tout[c * L + i] = (float)(Xi[i * L + c] / diag[i]);
    }
}

// ---------------------------------------------------------------- Jacobi
// Symmetric C (L x L, fp64, even L) -> eigenvalues on its diagonal and
// eigenvectors in the columns of E, by cyclic parallel Jacobi: each step
// rotates L/2 disjoint pairs (round-robin pairing), at most 40 sweeps.
// Round robin: index 0 stays in place and the other L-1 rotate by one place
// per step, so after s steps place i >= 1 holds 1 + ((i - 1 - s) mod (L-1));
// step s pairs the indices at places k and L-1-k.
// C and E live in (dynamic) LDS when IN_LDS (2 L^2 doubles), else in global memory.
template <bool IN_LDS>
__global__ __launch_bounds__(256) void sv_jacobi_kernel(int L, double *__restrict__ Cg, double *__restrict__ Eg)
{
    constexpr bool in_lds = IN_LDS;
    extern __shared__ double sv_dyn[];
    __shared__ double cs[SV_MAXL / 2], sn[SV_MAXL / 2];
    __shared__ int pp[SV_MAXL / 2], qq[SV_MAXL / 2];
    __shared__ double roff[SV_MAXL], rtot[SV_MAXL];
    __shared__ double off, tot;
    double *C = in_lds ? sv_dyn : Cg;
    double *E = in_lds ? sv_dyn + L * L : Eg;
    if (in_lds)
        for (int e = threadIdx.x; e < L * L; e += 256) C[e] = Cg[e];
    for (int e = threadIdx.x; e < L * L; e += 256) E[e] = (e / L == e % L) ? 1.0 : 0.0;
    const int H = L / 2;
    auto place = [L](int i, int step) { return i == 0 ? 0 : 1 + (i - 1 - step % (L - 1) + (L - 1)) % (L - 1); };
    __syncthreads();
    for (int sweep = 0; sweep < 40; ++sweep) {
        // squared off-diagonal and diagonal mass: one row per thread, rows added in order
        for (int i = threadIdx.x; i < L; i += 256) {
            double o = 0.0, t = 0.0;
            for (int j = 0; j < L; ++j) {
                const double v = C[i * L + j] * C[i * L + j];
                if (i == j) t += v; else o += v;
            }
            roff[i] = o;
            rtot[i] = t;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            double o = 0.0, t = 0.0;
            for (int i = 0; i < L; ++i) {
                o += roff[i];
                t += rtot[i];
            }
            off = o;
            tot = t;
        }
        __syncthreads();
        if (!(off > 1e-30 * tot)) break;   // block-uniform
        for (int step = 0; step < L - 1; ++step) {
            // pairs (place k, place L-1-k)
            for (int k = threadIdx.x; k < H; k += 256) {
                int p = place(k, step), q = place(L - 1 - k, step);
                if (p > q) { const int t = p; p = q; q = t; }
                const double apq = C[p * L + q], app = C[p * L + p], aqq = C[q * L + q];
                double c = 1.0, s = 0.0;
                if (apq != 0.0) {
                    const double tau = (aqq - app) / (2.0 * apq);
                    const double t = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + __builtin_sqrt(1.0 + tau * tau));
                    c = 1.0 / __builtin_sqrt(1.0 + t * t);
                    s = t * c;
                }
                cs[k] = c; sn[k] = s; pp[k] = p; qq[k] = q;
            }
            __syncthreads();
            // rows: C[p,:], C[q,:]
            for (int e = threadIdx.x; e < H * L; e += 256) {
                const int k = e / L, col = e - k * L;
                const int p = pp[k], q = qq[k];
                const double c = cs[k], s = sn[k];
                const double xp = C[p * L + col], xq = C[q * L + col];
                C[p * L + col] = c * xp - s * xq;
                C[q * L + col] = s * xp + c * xq;
            }
            __syncthreads();
            // columns: C[:,p], C[:,q] and E[:,p], E[:,q]
            for (int e = threadIdx.x; e < H * L; e += 256) {
                const int k = e / L, row = e - k * L;
                const int p = pp[k], q = qq[k];
                const double c = cs[k], s = sn[k];
                const double xp = C[row * L + p], xq = C[row * L + q];
                C[row * L + p] = c * xp - s * xq;
                C[row * L + q] = s * xp + c * xq;
                const double ep = E[row * L + p], eq = E[row * L + q];
                E[row * L + p] = c * ep - s * eq;
                E[row * L + q] = s * ep + c * eq;
            }
            __syncthreads();
        }
    }
    if (in_lds) {
        __syncthreads();
        for (int e = threadIdx.x; e < L * L; e += 256) {
            Cg[e] = C[e];
            Eg[e] = E[e];
        }
    }
}

// Top-r eigenvectors (eigenvalues descending) as an fp32 L x r block.
__global__ __launch_bounds__(256) void sv_select_kernel(int L, int r, const double *__restrict__ C,
                                                        const double *__restrict__ E, float *__restrict__ Er)
{
    __shared__ int order[SV_MAXL];
    __shared__ double dg[SV_MAXL];
    for (int i = threadIdx.x; i < L; i += 256) dg[i] = C[i * L + i];
    __syncthreads();
    // rank of eigenvalue i in descending order, ties to the lower index
    for (int i = threadIdx.x; i < L; i += 256) {
        const double v = dg[i];
        int rank = 0;
        for (int j = 0; j < L; ++j) rank += (dg[j] > v || (dg[j] == v && j < i)) ? 1 : 0;
        order[rank] = i;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < L * r; e += 256) {
        const int i = e / r, j = e - i * r;
        Er[e] = (float)E[i * L + order[j]];
    }
}

// sign[j] = +1 or -1 so that column j's largest-magnitude entry (first on ties) is positive
__global__ __launch_bounds__(256) void sv_sign_kernel(int N, int r, const float *__restrict__ U, float *__restrict__ sign)
{
    __shared__ float bv[256];
    __shared__ int bi[256];
    const int j = blockIdx.x;
    float best = -1.0f;
    int at = 0x7FFFFFFF;
    for (int n = threadIdx.x; n < N; n += 256) {
        const float v = fabsf(U[(size_t)n * r + j]);
        if (v > best) { best = v; at = n; }
    }
    bv[threadIdx.x] = best;
    bi[threadIdx.x] = at;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int t = 1; t < 256; ++t)
            if (bv[t] > best || (bv[t] == best && bi[t] < at)) { best = bv[t]; at = bi[t]; }
        sign[j] = (at < N && U[(size_t)at * r + j] < 0.0f) ? -1.0f : 1.0f;
    }
}

__global__ __launch_bounds__(256) void sv_write_kernel(int N, int K, int r, const float *__restrict__ U,
                                                       const float *__restrict__ D, const float *__restrict__ sign,
                                                       uint16_t *__restrict__ up, uint16_t *__restrict__ down)
{
    const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
    if (e < (long long)N * r) {
        const int j = (int)(e % r);
        up[e] = (uint16_t)f32_to_bf16_rne(U[e] * sign[j]);
    }
    if (e < (long long)K * r) {
        const int k = (int)(e / r), j = (int)(e % r);
        down[(size_t)j * K + k] = (uint16_t)f32_to_bf16_rne(D[e] * sign[j]);
    }
}

// Gaussian sketch: Box-Muller on two 53-bit uniforms from a SplitMix64 hash of (seed, index)
__device__ __forceinline__ uint64_t sv_mix(uint64_t z) {
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
__global__ __launch_bounds__(256) void sv_gauss_kernel(long long n, uint64_t seed, float *__restrict__ out)
{
    const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
    if (e >= n) return;
    const uint64_t h1 = sv_mix(seed ^ sv_mix(2 * (uint64_t)e)), h2 = sv_mix(seed ^ sv_mix(2 * (uint64_t)e + 1));
    const double u1 = ((double)(h1 >> 11) + 1.0) * 0x1p-53, u2 = (double)(h2 >> 11) * 0x1p-53;
    out[e] = (float)(__builtin_sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2));
}

// ---------------------------------------------------------------- host side
struct SvWork {
    float *Z, *Y, *Y2, *U, *D, *T, *Er, *sign, *ppart;
    double *part, *G, *Lw, *E;
};

// reduction slices of a product with I output rows: enough blocks to fill the chip
static int sv_slices(int I) {
    const int nb = (I + 63) / 64;
    const int S = (512 + nb - 1) / nb;
    return S < 1 ? 1 : (S > 8 ? 8 : S);
}

static size_t sv_layout(int N, int K, int r, char *base, SvWork *w)
{
    const int L = r + SV_OVERSAMPLE;
    const int R = N > K ? N : K;
    const int nb = (R + SV_GROWS - 1) / SV_GROWS;
    size_t off = 0;
    auto take = [&](size_t bytes) { char *p = base ? base + off : nullptr; off += (bytes + 255) & ~(size_t)255; return p; };
    // the three bases trade places during the iteration: each holds max(N, K) rows
    float *Z = (float *)take((size_t)R * L * 4), *Y = (float *)take((size_t)R * L * 4),
          *Y2 = (float *)take((size_t)R * L * 4), *U = (float *)take((size_t)N * r * 4),
          *D = (float *)take((size_t)K * r * 4), *T = (float *)take((size_t)L * L * 4),
          *Er = (float *)take((size_t)L * r * 4), *sign = (float *)take((size_t)r * 4);
    const size_t pp = (size_t)std::max((size_t)sv_slices(N) * N, (size_t)sv_slices(K) * K) * L;
    float *ppart = (float *)take(pp * 4);
    double *part = (double *)take((size_t)nb * L * (L + 1) / 2 * 8), *G = (double *)take((size_t)L * L * 8),
           *Lw = (double *)take((size_t)L * L * 8), *E = (double *)take((size_t)L * L * 8);
    if (w) *w = SvWork{Z, Y, Y2, U, D, T, Er, sign, ppart, part, G, Lw, E};
    return off;
}

size_t lowrank_workspace_bytes(int N, int K, int r) { return sv_layout(N, K, r, nullptr, nullptr); }

// ------------------------------------------------ fixed scratch (no allocation)
// The workspace of the allocation-free entry point: one array per device,
// resident from the library's load until the process ends.  In host code the
// name `scratch` is a host-side handle, not a device address; kernels get the
// address that hipGetSymbolAddress returns for the current device.  Every
// call shares its device's array: calls that overlap on one device race.
// Nothing in it needs to start at zero (every kernel of the branch writes
// each scratch element before reading it), so it is never cleared.
static __device__ __align__(256) char scratch[LOWRANK_SCRATCH_BYTES];

hipError_t lowrank_scratch(void **ptr)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {   // once per device, with that device current
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

#define SV_TRY(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) return e_; } while (0)

// out = W_hat X (trans false: I = N, T = K) or W_hat^T X (trans true: I = K, T = N),
// split over the reduction when the rows alone would leave the chip idle
static hipError_t sv_wprod(bool trans, int I, int T, int L, const uint16_t *W, const uint16_t *s, const float *X,
                           float *out, float *ppart, hipStream_t st)
{
    const int S0 = sv_slices(I);
    int tsplit = ((T + S0 - 1) / S0 + 31) & ~31;
    const int S = (T + tsplit - 1) / tsplit;
    float *dst = S > 1 ? ppart : out;
    const dim3 grid((I + 63) / 64, S);
    if (trans)
        hipLaunchKernelGGL((sv_product_kernel<uint16_t, true>), grid, dim3(256), 0, st, I, T, L, W, s, X, dst, tsplit);
    else
        hipLaunchKernelGGL((sv_product_kernel<uint16_t, false>), grid, dim3(256), 0, st, I, T, L, W, s, X, dst, tsplit);
    if (S > 1) {
        const long long n = (long long)I * L;
        hipLaunchKernelGGL(sv_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, S, n, ppart, out);
    }
    return hipGetLastError();
}

// X (R x L) <- orthonormal basis of its columns: CholeskyQR2
static hipError_t sv_orth(int R, int L, float *&X, float *&Xtmp, const SvWork &w, hipStream_t st)
{
    const int nb = (R + SV_GROWS - 1) / SV_GROWS;
    for (int pass = 0; pass < 2; ++pass) {
        hipLaunchKernelGGL(sv_gram_partial_kernel, dim3(nb), dim3(256), 0, st, R, L, X, w.part);
        hipLaunchKernelGGL(sv_gram_reduce_kernel, dim3((L * (L + 1) / 2 + SV_RED_PAIRS - 1) / SV_RED_PAIRS), dim3(256), 0, st, nb, L, w.part, w.G);
        if (2 * L * L * 8 <= 62 * 1024)
            hipLaunchKernelGGL(sv_chol_inv_kernel<true>, dim3(1), dim3(256), 2 * L * L * 8, st, L, w.G, w.Lw, w.E, w.T);
        else
            hipLaunchKernelGGL(sv_chol_inv_kernel<false>, dim3(1), dim3(256), 0, st, L, w.G, w.Lw, w.E, w.T);
        hipLaunchKernelGGL((sv_product_kernel<float, false>), dim3((R + 63) / 64), dim3(256), 0, st, R, L, L, X,
                           (const uint16_t *)nullptr, w.T, Xtmp, L);
        float *t = X; X = Xtmp; Xtmp = t;
        SV_TRY(hipGetLastError());
    }
    return hipSuccess;
}

hipError_t launch_lowrank_factors(int N, int K, int r, const void *W, const void *s, uint64_t seed,
                                  void *workspace, void *up, void *down, hipStream_t st)
{
    const int L = r + SV_OVERSAMPLE;
    SvWork w;
    sv_layout(N, K, r, (char *)workspace, &w);
    const uint16_t *Wb = (const uint16_t *)W, *sb = (const uint16_t *)s;
    // sketch and range: Y = W_hat Omega
    hipLaunchKernelGGL(sv_gauss_kernel, dim3((unsigned)(((long long)K * L + 255) / 256)), dim3(256), 0, st,
                       (long long)K * L, seed, w.Z);
    SV_TRY(sv_wprod(false, N, K, L, Wb, sb, w.Z, w.Y, w.ppart, st));
    float *Y = w.Y, *Ytmp = w.Y2, *Z = w.Z;
    SV_TRY(sv_orth(N, L, Y, Ytmp, w, st));
    for (int it = 0; it < 2; ++it) {
        // Z = W_hat^T Y, orthonormalized; Y = W_hat Z, orthonormalized
        SV_TRY(sv_wprod(true, K, N, L, Wb, sb, Y, Z, w.ppart, st));
        float *Zt = Ytmp;   // every basis buffer has room for max(N, K) rows
        SV_TRY(sv_orth(K, L, Z, Zt, w, st));
        Ytmp = Zt;
        SV_TRY(sv_wprod(false, N, K, L, Wb, sb, Z, Y, w.ppart, st));
        SV_TRY(sv_orth(N, L, Y, Ytmp, w, st));
    }
    // Z = W_hat^T Q (= B^T); C = B B^T = Z^T Z; eigenvectors E
    SV_TRY(sv_wprod(true, K, N, L, Wb, sb, Y, Z, w.ppart, st));
    const int nbk = (K + SV_GROWS - 1) / SV_GROWS;
    hipLaunchKernelGGL(sv_gram_partial_kernel, dim3(nbk), dim3(256), 0, st, K, L, Z, w.part);
    hipLaunchKernelGGL(sv_gram_reduce_kernel, dim3((L * (L + 1) / 2 + SV_RED_PAIRS - 1) / SV_RED_PAIRS), dim3(256), 0, st, nbk, L, w.part, w.G);
    if (2 * L * L * 8 <= 62 * 1024)
        hipLaunchKernelGGL(sv_jacobi_kernel<true>, dim3(1), dim3(256), 2 * L * L * 8, st, L, w.G, w.E);
    else
        hipLaunchKernelGGL(sv_jacobi_kernel<false>, dim3(1), dim3(256), 0, st, L, w.G, w.E);
    hipLaunchKernelGGL(sv_select_kernel, dim3(1), dim3(256), 0, st, L, r, w.G, w.E, w.Er);
    // U = Q E_r (N x r), D = B^T E_r = Z E_r (K x r) = V Sigma
    hipLaunchKernelGGL((sv_product_kernel<float, false>), dim3((N + 63) / 64), dim3(256), 0, st, N, L, r, Y,
                       (const uint16_t *)nullptr, w.Er, w.U, L);
    hipLaunchKernelGGL((sv_product_kernel<float, false>), dim3((K + 63) / 64), dim3(256), 0, st, K, L, r, Z,
                       (const uint16_t *)nullptr, w.Er, w.D, L);
    hipLaunchKernelGGL(sv_sign_kernel, dim3(r), dim3(256), 0, st, N, r, w.U, w.sign);
    const long long m = (long long)(N > K ? N : K) * r;
    hipLaunchKernelGGL(sv_write_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, st, N, K, r, w.U, w.D, w.sign,
                       (uint16_t *)up, (uint16_t *)down);
    return hipGetLastError();
}

}  // namespace svdq
