/* Host sanitizer driver for the C oracle (test infrastructure).
 *
 * Built together with oracle/convrot_oracle.c under AddressSanitizer and
 * UndefinedBehaviorSanitizer by tests/test_oracle_sanitized.py, it walks every
 * oracle entry point over small shapes (several Hadamard blocks, ragged row
 * counts, both input types and output types, the error paths) so that an out
 * of bounds access, a leak or undefined arithmetic in the checker itself fails
 * the test.  The values are checked by the pin tests; here only the return
 * codes and a few invariants are. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_num_threads(void);
float oracle_bf16_to_f32(uint16_t h);
uint16_t oracle_f32_to_bf16(float f);
int oracle_fwht_f32(float *v, int64_t K, int b);
int oracle_rowquant(const float *v, int64_t K, int b, int8_t *q, float *s);
int oracle_rotate_quantize_rows(const void *src, int dtype, int64_t rows, int64_t K,
                                int64_t ld, int b, int8_t *q, float *s);
int oracle_prepare_weights_in_major(const void *src, int dtype, int64_t N, int64_t K, int b,
                                    int8_t *q, float *s);
int oracle_gemm_i32(const int8_t *qx, const int8_t *qw, int64_t M, int64_t N, int64_t K,
                    int32_t *acc);
int oracle_dequant(const int32_t *acc, const float *sx, const float *sw, const float *bias,
                   int64_t M, int64_t N, int out_dtype, void *out);
int oracle_linear_forward(const uint16_t *X, int64_t M, int64_t K, int b, const int8_t *qw,
                          const float *sw, int64_t N, const float *bias, int out_dtype,
                          void *out);
int oracle_lowrank_forward(const uint16_t *X, int64_t M, int64_t K, int b, const int8_t *qa,
                           const float *sa, int64_t r, const int8_t *qb, const float *sb,
                           int64_t N, const float *bias, int out_dtype, void *out,
                           uint16_t *h_out);
double oracle_gelu_f64(double z);
void oracle_gelu_bf16(const uint16_t *u, int64_t n, uint16_t *g);
int oracle_mlp_forward(const uint16_t *X, int64_t M, int64_t K, int b, const int8_t *qu,
                       const float *su, int64_t F, const float *bias_up, const int8_t *qd,
                       const float *sd, int64_t N, const float *bias_down, int out_dtype,
                       void *out, uint16_t *u_out, uint16_t *g_out);

enum { F32 = 0, BF16 = 1 };

static uint64_t state = 0x9e3779b97f4a7c15ull;
static float frand(void)  /* xorshift64*, uniform in [-1, 1) */
{
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    return (float)((state * 0x2545f4914f6cdd1dull) >> 40) / (float)(1 << 23) - 1.0f;
}

static int fails = 0;
#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++fails;                                                      \
        }                                                                 \
    } while (0)

static void *xmalloc(size_t n) { void *p = malloc(n ? n : 1); if (!p) abort(); return p; }

static void linear_case(int64_t M, int64_t K, int64_t N, int b)
{
    float *W = xmalloc(sizeof(float) * N * K);
    uint16_t *X = xmalloc(sizeof(uint16_t) * M * K);
    for (int64_t i = 0; i < N * K; ++i) W[i] = 0.02f * frand();
    for (int64_t i = 0; i < M * K; ++i) X[i] = oracle_f32_to_bf16(3.0f * frand());
    int8_t *qw = xmalloc(N * K), *qwi = xmalloc(N * K);
    float *sw = xmalloc(sizeof(float) * N), *swi = xmalloc(sizeof(float) * N);
    CHECK(oracle_rotate_quantize_rows(W, F32, N, K, K, b, qw, sw) == 0);
    /* the same weights stored input-major give the same codes */
    float *Wt = xmalloc(sizeof(float) * N * K);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) Wt[k * N + n] = W[n * K + k];
    CHECK(oracle_prepare_weights_in_major(Wt, F32, N, K, b, qwi, swi) == 0);
    CHECK(memcmp(qw, qwi, N * K) == 0 && memcmp(sw, swi, sizeof(float) * N) == 0);
    float *bias = xmalloc(sizeof(float) * N);
    for (int64_t n = 0; n < N; ++n) bias[n] = 0.01f * frand();
    uint16_t *yb = xmalloc(sizeof(uint16_t) * M * N);
    float *yf = xmalloc(sizeof(float) * M * N);
    CHECK(oracle_linear_forward(X, M, K, b, qw, sw, N, bias, BF16, yb) == 0);
    CHECK(oracle_linear_forward(X, M, K, b, qw, sw, N, NULL, F32, yf) == 0);
    int8_t *qx = xmalloc(M * K);
    float *sx = xmalloc(sizeof(float) * M);
    int32_t *acc = xmalloc(sizeof(int32_t) * M * N);
    CHECK(oracle_rotate_quantize_rows(X, BF16, M, K, K, b, qx, sx) == 0);
    CHECK(oracle_gemm_i32(qx, qw, M, N, K, acc) == 0);
    CHECK(oracle_dequant(acc, sx, sw, bias, M, N, BF16, yb) == 0);
    free(W); free(Wt); free(X); free(qw); free(qwi); free(sw); free(swi); free(bias);
    free(yb); free(yf); free(qx); free(sx); free(acc);
}

int main(void)
{
    /* FWHT and the quantiser on every block size, including b = 1 */
    for (int b = 1; b <= 256; b *= 2) {
        const int64_t K = 2 * b;
        float *v = xmalloc(sizeof(float) * K);
        int8_t *q = xmalloc(K);
        float s;
        for (int64_t k = 0; k < K; ++k) v[k] = frand();
        CHECK(oracle_fwht_f32(v, K, b) == 0);
        CHECK(oracle_rowquant(v, K, b, q, &s) == 0);
        memset(v, 0, sizeof(float) * K);
        CHECK(oracle_rowquant(v, K, b, q, &s) == 0 && s == 0.0f);
        free(v); free(q);
    }
    /* error paths */
    float dummy[8] = {0};
    int8_t qd[8];
    float sd[1];
    CHECK(oracle_fwht_f32(dummy, 8, 3) != 0);
    CHECK(oracle_rotate_quantize_rows(dummy, F32, 1, 8, 4, 4, qd, sd) != 0);   /* ld < K */
    CHECK(oracle_gemm_i32(qd, qd, 1, 1, 200000, NULL) != 0);                 /* K bound */

    linear_case(3, 256, 16, 128);
    linear_case(17, 512, 48, 64);
    linear_case(5, 768, 32, 256);
    linear_case(0, 256, 16, 128);

    /* low-rank and MLP chains */
    {
        const int64_t M = 9, K = 512, r = 128, N = 64, F = 256;
        const int b = 128;
        uint16_t *X = xmalloc(sizeof(uint16_t) * M * K);
        for (int64_t i = 0; i < M * K; ++i) X[i] = oracle_f32_to_bf16(frand());
        float *A = xmalloc(sizeof(float) * r * K), *B = xmalloc(sizeof(float) * N * r);
        for (int64_t i = 0; i < r * K; ++i) A[i] = 0.02f * frand();
        for (int64_t i = 0; i < N * r; ++i) B[i] = 0.02f * frand();
        int8_t *qa = xmalloc(r * K), *qb = xmalloc(N * r);
        float *sa = xmalloc(sizeof(float) * r), *sb = xmalloc(sizeof(float) * N);
        CHECK(oracle_rotate_quantize_rows(A, F32, r, K, K, b, qa, sa) == 0);
        CHECK(oracle_rotate_quantize_rows(B, F32, N, r, r, b, qb, sb) == 0);
        uint16_t *y = xmalloc(sizeof(uint16_t) * M * N), *h = xmalloc(sizeof(uint16_t) * M * r);
        CHECK(oracle_lowrank_forward(X, M, K, b, qa, sa, r, qb, sb, N, NULL, BF16, y, h) == 0);
        CHECK(oracle_lowrank_forward(X, M, K, b, qa, sa, 100, qb, sb, N, NULL, BF16, y, h) != 0);
        float *Wu = xmalloc(sizeof(float) * F * K), *Wd = xmalloc(sizeof(float) * N * F);
        for (int64_t i = 0; i < F * K; ++i) Wu[i] = 0.02f * frand();
        for (int64_t i = 0; i < N * F; ++i) Wd[i] = 0.02f * frand();
        int8_t *qu = xmalloc(F * K), *qdn = xmalloc(N * F);
        float *su = xmalloc(sizeof(float) * F), *sdn = xmalloc(sizeof(float) * N);
        CHECK(oracle_rotate_quantize_rows(Wu, F32, F, K, K, b, qu, su) == 0);
        CHECK(oracle_rotate_quantize_rows(Wd, F32, N, F, F, b, qdn, sdn) == 0);
        uint16_t *u = xmalloc(sizeof(uint16_t) * M * F), *g = xmalloc(sizeof(uint16_t) * M * F);
        CHECK(oracle_mlp_forward(X, M, K, b, qu, su, F, NULL, qdn, sdn, N, NULL, BF16, y, u, g)
              == 0);
        free(X); free(A); free(B); free(qa); free(qb); free(sa); free(sb); free(y); free(h);
        free(Wu); free(Wd); free(qu); free(qdn); free(su); free(sdn); free(u); free(g);
    }
    /* GELU over every bf16 pattern */
    {
        uint16_t *u = xmalloc(sizeof(uint16_t) * 65536), *g = xmalloc(sizeof(uint16_t) * 65536);
        for (int i = 0; i < 65536; ++i) u[i] = (uint16_t)i;
        oracle_gelu_bf16(u, 65536, g);
        CHECK(g[0] == 0);                                   /* GELU(+0) = +0 */
        CHECK(oracle_gelu_f64(0.0) == 0.0);
        free(u); free(g);
    }
    printf("sanitized oracle walk: %d failed checks, %d threads\n", fails, oracle_num_threads());
    return fails ? 1 : 0;
}
