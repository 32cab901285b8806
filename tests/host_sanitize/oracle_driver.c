/* Host AddressSanitizer / UndefinedBehaviorSanitizer run of the CPU oracle.
 *
 * Compiles oracle/svdq_oracle.c into this program (test infrastructure: the
 * oracle is only ever used by the tests, the smoke check and the CPU
 * baseline) and calls every exported function on small inputs whose buffers
 * are heap blocks of exactly the documented sizes, with the edge values the
 * parity tests use: all bf16 / E4M3 / E2M1 codes, NaN, infinities,
 * subnormals, zero groups, ragged shapes, rank 0 and NULL bias.  Any
 * out-of-bounds access or undefined behaviour aborts the run (built with
 * -fno-sanitize-recover=all); a clean run prints "oracle sanitize ok". */
#include "../../oracle/svdq_oracle.c"

#include <stdio.h>
#include <stdlib.h>

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {             /* splitmix64 */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static double uniform(void) { return (double)(next_u64() >> 11) * 0x1p-53; }
static double normal(void) {
    double u = uniform(), v = uniform();
    if (u < 1e-300) u = 1e-300;
    return sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v);
}
static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}
static uint16_t *bf16_array(int64_t n, double sigma) {
    uint16_t *a = xmalloc((size_t)n * sizeof *a);
    for (int64_t i = 0; i < n; ++i) a[i] = oracle_f64_to_bf16(normal() * sigma);
    return a;
}

static void codecs(void) {
    float *f = xmalloc(65536 * sizeof *f);
    uint16_t *h = xmalloc(65536 * sizeof *h), *g = xmalloc(65536 * sizeof *g);
    for (int i = 0; i < 65536; ++i) h[i] = (uint16_t)i;
    oracle_bf16_to_f32_array(65536, h, f);
    oracle_f32_to_bf16_array(65536, f, g);
    oracle_gelu_tanh_bf16_array(65536, h, g);
    double *d = xmalloc(8 * sizeof *d);
    const double dv[8] = {0.0, -0.0, 1.0 + 0x1p-8, 1e300, -1e-300, INFINITY, -INFINITY, NAN};
    for (int i = 0; i < 8; ++i) d[i] = dv[i];
    oracle_f64_to_bf16_array(8, d, g);
    uint8_t *b = xmalloc(256), *c = xmalloc(256);
    for (int i = 0; i < 256; ++i) b[i] = (uint8_t)i;
    oracle_e4m3_to_f32_array(256, b, f);
    oracle_f32_to_e4m3_array(256, f, c);
    oracle_e2m1_to_f32_array(256, b, f);
    oracle_f32_to_e2m1_array(256, f, c);
    float *e = xmalloc(12 * sizeof *e);
    const float ev[12] = {0.0f, -0.0f, 0.25f, 0.75f, 5.0f, 7.0f, 464.0f, 1e30f, -1e-45f, INFINITY, -INFINITY, NAN};
    for (int i = 0; i < 12; ++i) e[i] = ev[i];
    oracle_f32_to_e4m3_array(12, e, c);
    oracle_f32_to_e2m1_array(12, e, c);
    free(f); free(h); free(g); free(d); free(b); free(c); free(e);
}

static void layer(int32_t prec, int64_t M, int64_t N, int64_t K, int32_t rank, int with_bias) {
    uint16_t *x = bf16_array(M * K, 1.0), *W = bf16_array(N * K, 0.02);
    for (int64_t k = 0; k < K; k += 7) x[k] = 0;               /* zero and tiny channels */
    if (M > 1) for (int64_t k = 0; k < 64 && k < K; ++k) x[K + k] = 0;   /* an all-zero group */
    uint16_t *s = xmalloc((size_t)K * sizeof *s);
    oracle_smooth_factors(M, N, K, x, W, s);
    uint16_t *up = rank ? bf16_array(N * rank, 0.3) : NULL, *down = rank ? bf16_array(rank * K, 0.3) : NULL;
    float *R = xmalloc((size_t)(N * K) * sizeof *R);
    oracle_svdq_residual(N, K, rank, W, s, up, down, R);
    const int64_t sgroups = prec == 0 ? K / 64 : K / 16;
    const size_t ssize = prec == 0 ? 2 : 1;
    uint8_t *wc = xmalloc((size_t)(N * K / 2));
    void *ws = xmalloc((size_t)(N * sgroups) * ssize);
    if (prec == 0) oracle_quantize_int4(N, K, R, wc, ws);
    else oracle_quantize_nvfp4(N, K, R, wc, ws);
    uint8_t *ac = xmalloc((size_t)(M * K / 2));
    void *as = xmalloc((size_t)(M * sgroups) * ssize);
    float *t = rank ? xmalloc((size_t)(M * rank) * sizeof(float)) : NULL;
    uint16_t *xh = xmalloc((size_t)(M * K) * sizeof *xh);
    float *vals = xmalloc((size_t)(M * K) * sizeof *vals);
    oracle_svdq_quantize_act(prec, M, K, rank, x, s, down, ac, as, t, xh, vals);
    uint16_t *bias = with_bias ? bf16_array(N, 1.0) : NULL;
    uint16_t *out = xmalloc((size_t)(M * N) * sizeof *out);
    oracle_svdq_gemm_w4a4(prec, M, N, K, rank, ac, as, wc, ws, prec ? 0.5f : 1.0f, t, up, bias, out);
    if (prec == 0) {
        int32_t *G = xmalloc((size_t)(M * N * (K / 64)) * sizeof *G);
        oracle_group_sums_int4(M, N, K, ac, wc, G);
        int8_t *u = xmalloc((size_t)(M * K));
        oracle_unpack_int4(M, K, ac, u);
        free(G); free(u);
    }
    free(x); free(W); free(s); free(up); free(down); free(R); free(wc); free(ws); free(ac); free(as);
    free(t); free(xh); free(vals); free(bias); free(out);
}

static void awq(int64_t M, int64_t N, int64_t K, int with_bias) {
    uint16_t *x = bf16_array(M * K, 1.0), *W = bf16_array(N * K, 0.02);
    for (int64_t k = 0; k < 64; ++k) W[k] = 0;                  /* a zero group: scale 0 */
    uint8_t *codes = xmalloc((size_t)(N * K / 2));
    uint16_t *sc = xmalloc((size_t)(N * K / 64) * sizeof *sc), *z = xmalloc((size_t)(N * K / 64) * sizeof *z);
    oracle_awq_quantize_weight(N, K, W, codes, sc, z);
    uint8_t *u = xmalloc((size_t)(N * K));
    oracle_unpack_u4(N, K, codes, u);
    uint16_t *bias = with_bias ? bf16_array(N, 1.0) : NULL;
    uint16_t *out = xmalloc((size_t)(M * N) * sizeof *out);
    oracle_awq_gemv_w4a16(M, N, K, 64, x, codes, sc, z, bias, out);
    free(x); free(W); free(codes); free(sc); free(z); free(u); free(bias); free(out);
}

static void qk(int64_t M, int64_t heads) {
    const int64_t N = 3 * heads * 128;
    uint16_t *y = bf16_array(M * N, 1.0), *qw = bf16_array(128, 1.0), *kw = bf16_array(128, 1.0);
    for (int64_t n = 0; n < N; ++n) y[n] = 0;                   /* a zero row: eps keeps it finite */
    float *c = xmalloc((size_t)(M * 64) * sizeof *c), *sn = xmalloc((size_t)(M * 64) * sizeof *sn);
    for (int64_t i = 0; i < M * 64; ++i) { c[i] = (float)cos(0.1 * (double)i); sn[i] = (float)sin(0.1 * (double)i); }
    uint16_t *out = xmalloc((size_t)(M * N) * sizeof *out);
    oracle_qk_norm_rope(M, N, y, qw, kw, 1e-6, c, sn, out);
    free(y); free(qw); free(kw); free(c); free(sn); free(out);
}

int main(void) {
    codecs();
    for (int prec = 0; prec < 2; ++prec) {
        layer(prec, 1, 64, 64, 0, 0);
        layer(prec, 33, 130, 192, 16, 1);
        layer(prec, 5, 7, 256, 32, 0);
        layer(prec, 2, 48, 64, 48, 1);                            /* rank above K/2 */
    }
    awq(1, 5, 64, 1);
    awq(3, 33, 192, 0);
    qk(3, 1);
    qk(2, 2);
    printf("oracle sanitize ok\n");
    return 0;
}
