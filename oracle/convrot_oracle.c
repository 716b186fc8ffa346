/*
 * convrot_oracle.c -- plain CPU oracle for the ConvRot W8A8 INT8 linear.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no code,
 * header or constant with the HIP library and must never sit on the product
 * path.
 *
 * What it computes (sources, all read as descriptions, none copied):
 *  - "HyperFlow H3 Flash" card as summarised on the lehuy.net article
 *    ("Cach nen hoat dong", second bullet): the linear layers are INT8 W8A8
 *    behind a block-diagonal Hadamard rotation.
 *  - MiniMax-H3-Rung-Omega README, "Technical Architecture Overview", Floor 1:
 *    the activation is rotated (ConvRot) and then quantised row by row
 *    (rowwise INT8 quantise) in front of the projection.
 *  - PulpCut "MiniMax H3 - pruned INT8 ConvRot - input-major", section
 *    "Input-major checkpoint": weights are INT8 codes with one F32 scale per
 *    output channel, stored [output, input] (or [input, output] after an
 *    exact transpose).
 *  - HyperFlow H3 Flash MLX card, "Where the weights come from": dequantising
 *    the int8 weights and undoing their Hadamard rotation is exact, so the
 *    stored weights are W.R^T for an orthogonal R.
 *  - HyperFlow H3 Flash card, "Choose a Weight Format" table: the INT8
 *    package is W8A8 and also holds low-rank factorised linears;
 *    "Standalone Transformer (AutoModel)": low-rank ranks get padded to a
 *    multiple of 64.
 *  - MiniMax-H3-Rung-Omega README, "Technical Architecture Overview", item 1:
 *    a rotation by the regular ("DC-balanced") orthogonal Hadamard
 *    H_256 = H_4 (x) H_4 (x) H_4 (x) H_4 on 256-element blocks, offered here as
 *    the second rotation kind (orders 64 and 256).
 *
 * Readings taken where the pages are silent (each listed in the design notes):
 *  R1 Sylvester Hadamard in natural order, unnormalised; 1/sqrt(b) is folded
 *     into the scale.
 *  R2 Butterfly stages in ascending stride h = 1, 2, 4, ..., b/2, in fp32.
 *  R3 Symmetric range [-127, 127]; code = rint(v * (127/amax)) with a
 *     correctly rounded fp32 reciprocal-by-division; scale =
 *     (amax/127) * fp32(1/sqrt(b)).  A zero row gives codes 0 and scale 0.
 *  R4 Dequant: ((float)acc * s_x) * s_w, then + bias; no fused multiply-add.
 *  R5 bf16 outputs are round-to-nearest-even of the fp32 value.
 *  R6 Low-rank: bf16 intermediate, requantised with the same block b along r.
 *  R7 MLP pair: g = bf16(GELU_erf(float(u))) with GELU evaluated in fp64.
 *  R8 Regular rotation: H_4 = J - 2I (diagonal -1, every other entry +1, so
 *     every row sums to 2), applied along the base-4 digits of the index in
 *     ascending order; a group (v0, v1, v2, v3) becomes S - 2 v_j with
 *     S = (v0 + v1) + (v2 + v3), in fp32.  The scale folds 1/sqrt(b) as in R1.
 *  R9 bf16 low-rank comparison variant (the HyperFlow H3 Flash card, "INT8
 *     convrot in ComfyUI": there the low-rank linears stay bf16): each
 *     product is the exact sum over K rounded once to fp32, the bias added in
 *     fp32, then bf16 by round to nearest even; no rotation, no quantisation.
 * R10 SwiGLU MLP (MiniMax-H3-Rung-Omega README, "Technical Architecture
 *     Overview", Floor 1: SwiGLU, ConvRot64 and the rowwise INT8 quantise
 *     fused in front of MLP.fc2).  fc1 is one linear with 2F outputs whose
 *     bf16 result holds the gate in columns [0, F) and the up projection in
 *     [F, 2F); g = bf16(s * u) with s = fp32(silu(gate)), silu(z) =
 *     z / (1 + exp(-z)) evaluated in fp64 on the bf16 gate and rounded once
 *     to fp32, s * u one fp32 multiply; fc2 rotates g with its own block
 *     (64 for ConvRot64) and quantises it per token.
 *
 * Precision: every step that decides an INT8 code is evaluated in fp32 (the
 * precision the GPU kernels take those decisions in), with the butterfly order
 * of R2.  Build with -ffp-contract=off and without -ffast-math.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_EINVAL (-1)
#define OR_ENONFINITE (-2)

/* dtype tags used by this oracle only */
#define OR_F32 0
#define OR_BF16 1

/* Threads an OpenMP region of this library uses (for reporting). */
int oracle_num_threads(void) { return omp_get_max_threads(); }

/* Set the threads of later OpenMP regions (n >= 1; for timing on one core). */
void oracle_set_num_threads(int n)
{
    if (n >= 1)
        omp_set_num_threads(n);
}

/* ------------------------------------------------------------------ */
/* bf16 <-> fp32                                                       */
/* ------------------------------------------------------------------ */

/* bf16 is the top half of an IEEE binary32; widening is exact. */
float oracle_bf16_to_f32(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round-to-nearest-even narrowing of binary32 to bfloat16 (R5).
 * Written from the definition: pick the nearer of the two bf16 neighbours,
 * the one with an even last mantissa bit on a tie. */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if (isnan(f))
        return (uint16_t)(((u >> 16) & 0x8000u) | 0x7fc0u);
    uint32_t lower = u & 0xffff0000u;          /* truncated toward zero   */
    uint32_t rest = u & 0x0000ffffu;           /* discarded low half      */
    uint32_t keep = lower >> 16;
    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u)))
        keep += 1u;                            /* away from zero in magnitude */
    return (uint16_t)keep;
}

/* ------------------------------------------------------------------ */
/* O1: blockwise fast Walsh-Hadamard transform (R1, R2)                */
/* ------------------------------------------------------------------ */

static int is_pow2(long long b) { return b >= 1 && (b & (b - 1)) == 0; }

/* In place on v[0..K): each length-b block becomes H_b . block, where H_b is
 * the Sylvester matrix H_1 = [1], H_2k = [[H_k, H_k], [H_k, -H_k]]. */
int oracle_fwht_f32(float *v, int64_t K, int b)
{
    if (!is_pow2(b) || K < 0 || K % b != 0)
        return OR_EINVAL;
    for (int64_t j0 = 0; j0 < K; j0 += b) {
        float *blk = v + j0;
        for (int h = 1; h < b; h *= 2) {
            for (int i = 0; i < b; ++i) {
                if ((i & h) == 0) {
                    float a = blk[i];
                    float c = blk[i + h];
                    blk[i] = a + c;
                    blk[i + h] = a - c;
                }
            }
        }
    }
    return OR_OK;
}

static int is_pow4(long long b) { return is_pow2(b) && (b & 0x55555555LL) != 0; }

/* In place on v[0..K): each length-b block (b a power of 4) becomes
 * (H_4 (x) ... (x) H_4) . block with the regular H_4 = J - 2I of R8: for each
 * base-4 digit of the index, lowest first, every group of four elements that
 * differ only in that digit (v_j at digit value j) becomes S - 2 v_j with
 * S = (v0 + v1) + (v2 + v3).  2 v_j is exact, so each output is one rounding
 * of S - 2 v_j. */
int oracle_fwht_regular_f32(float *v, int64_t K, int b)
{
    if (!is_pow4(b) || K < 0 || K % b != 0)
        return OR_EINVAL;
    for (int64_t j0 = 0; j0 < K; j0 += b) {
        float *blk = v + j0;
        for (int h = 1; h < b; h *= 4) {
            for (int i = 0; i < b; ++i) {
                if ((i / h) % 4 != 0)
                    continue;
                float a0 = blk[i], a1 = blk[i + h], a2 = blk[i + 2 * h], a3 = blk[i + 3 * h];
                float S = (a0 + a1) + (a2 + a3);
                blk[i] = S - 2.0f * a0;
                blk[i + h] = S - 2.0f * a1;
                blk[i + 2 * h] = S - 2.0f * a2;
                blk[i + 3 * h] = S - 2.0f * a3;
            }
        }
    }
    return OR_OK;
}

/* Rotation kinds: 0 = the Sylvester blocks of R1, 1 = the regular blocks of
 * R8. */
#define OR_ROT_SYLVESTER 0
#define OR_ROT_REGULAR 1

int oracle_rotate_f32(float *v, int64_t K, int b, int rot)
{
    if (rot == OR_ROT_SYLVESTER)
        return oracle_fwht_f32(v, K, b);
    if (rot == OR_ROT_REGULAR)
        return oracle_fwht_regular_f32(v, K, b);
    return OR_EINVAL;
}

/* The fp32 value of 1/sqrt(b), rounded once from double. */
float oracle_inv_sqrt_b(int b) { return (float)(1.0 / sqrt((double)b)); }

/* ------------------------------------------------------------------ */
/* O2: symmetric rowwise INT8 quantisation of a rotated row (R3)       */
/* ------------------------------------------------------------------ */

int oracle_rowquant(const float *v, int64_t K, int b, int8_t *q, float *s)
{
    float amax = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        if (!isfinite(v[k]))
            return OR_ENONFINITE;
        float a = fabsf(v[k]);
        if (a > amax)
            amax = a;
    }
    if (amax == 0.0f) {
        for (int64_t k = 0; k < K; ++k)
            q[k] = 0;
        *s = 0.0f;
        return OR_OK;
    }
    float inv = 127.0f / amax;
    for (int64_t k = 0; k < K; ++k) {
        float t = rintf(v[k] * inv);
        if (t > 127.0f) t = 127.0f;
        if (t < -127.0f) t = -127.0f;
        q[k] = (int8_t)t;
    }
    float step = amax / 127.0f;
    *s = step * oracle_inv_sqrt_b(b);
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* O3 / O4: rotate-then-quantise over the rows of a matrix              */
/* ------------------------------------------------------------------ */

/* Rows of `src` (fp32 or bf16, row stride `ld` elements) -> codes [rows, K]
 * and one scale per row, rotated with rotation kind `rot`.  Rows are
 * independent; OpenMP splits them. */
int oracle_rotate_quantize_rows_rot(const void *src, int dtype, int64_t rows,
                                    int64_t K, int64_t ld, int b, int rot, int8_t *q,
                                    float *s)
{
    if (!is_pow2(b) || K <= 0 || K % b != 0 || rows < 0 || ld < K)
        return OR_EINVAL;
    if (rot != OR_ROT_SYLVESTER && (rot != OR_ROT_REGULAR || !is_pow4(b)))
        return OR_EINVAL;
    if (dtype != OR_F32 && dtype != OR_BF16)
        return OR_EINVAL;
    int bad = 0;
#pragma omp parallel
    {
        float *row = (float *)malloc(sizeof(float) * (size_t)K);
#pragma omp for schedule(static)
        for (int64_t m = 0; m < rows; ++m) {
            for (int64_t k = 0; k < K; ++k) {
                if (dtype == OR_F32)
                    row[k] = ((const float *)src)[m * ld + k];
                else
                    row[k] = oracle_bf16_to_f32(((const uint16_t *)src)[m * ld + k]);
            }
            oracle_rotate_f32(row, K, b, rot);
            if (oracle_rowquant(row, K, b, q + m * K, s + m) != OR_OK) {
#pragma omp atomic write
                bad = 1;
            }
        }
        free(row);
    }
    return bad ? OR_ENONFINITE : OR_OK;
}

int oracle_rotate_quantize_rows(const void *src, int dtype, int64_t rows,
                                int64_t K, int64_t ld, int b, int8_t *q,
                                float *s)
{
    return oracle_rotate_quantize_rows_rot(src, dtype, rows, K, ld, b, OR_ROT_SYLVESTER, q, s);
}

/* O3 for an input-major [K, N] weight: row n of W is column n. */
int oracle_prepare_weights_in_major_rot(const void *src, int dtype, int64_t N,
                                        int64_t K, int b, int rot, int8_t *q, float *s)
{
    if (!is_pow2(b) || K <= 0 || K % b != 0 || N < 0)
        return OR_EINVAL;
    if (dtype != OR_F32 && dtype != OR_BF16)
        return OR_EINVAL;
    float *tmp = (float *)malloc(sizeof(float) * (size_t)N * (size_t)K);
    if (!tmp)
        return OR_EINVAL;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n)
            tmp[n * K + k] = (dtype == OR_F32)
                                 ? ((const float *)src)[k * N + n]
                                 : oracle_bf16_to_f32(((const uint16_t *)src)[k * N + n]);
    int rc = oracle_rotate_quantize_rows_rot(tmp, OR_F32, N, K, K, b, rot, q, s);
    free(tmp);
    return rc;
}

int oracle_prepare_weights_in_major(const void *src, int dtype, int64_t N,
                                    int64_t K, int b, int8_t *q, float *s)
{
    return oracle_prepare_weights_in_major_rot(src, dtype, N, K, b, OR_ROT_SYLVESTER, q, s);
}

/* ------------------------------------------------------------------ */
/* O5: exact INT8 x INT8 -> INT32 contraction                           */
/* ------------------------------------------------------------------ */

/* acc[m, n] = sum_k qx[m, k] * qw[n, k].  |acc| <= K * 127^2 fits int32 for
 * K <= 133144; larger K is refused. */
int oracle_gemm_i32(const int8_t *qx, const int8_t *qw, int64_t M, int64_t N,
                    int64_t K, int32_t *acc)
{
    if (M < 0 || N < 0 || K <= 0 || K > 133144)
        return OR_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const int8_t *a = qx + m * K;
        for (int64_t n = 0; n < N; ++n) {
            const int8_t *w = qw + n * K;
            int32_t sum = 0;
            for (int64_t k = 0; k < K; ++k)
                sum += (int32_t)a[k] * (int32_t)w[k];
            acc[m * N + n] = sum;
        }
    }
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* O6 / O7: dequantise, add bias, narrow (R4, R5)                       */
/* ------------------------------------------------------------------ */

static float dequant_one(int32_t acc, float sx, float sw, const float *bias,
                         int64_t n)
{
    float y = (float)acc;      /* int32 -> fp32, round to nearest even */
    y = y * sx;
    y = y * sw;
    if (bias)
        y = y + bias[n];
    return y;
}

int oracle_dequant(const int32_t *acc, const float *sx, const float *sw,
                   const float *bias, int64_t M, int64_t N, int out_dtype,
                   void *out)
{
    if (M < 0 || N < 0 || (out_dtype != OR_F32 && out_dtype != OR_BF16))
        return OR_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            float y = dequant_one(acc[m * N + n], sx[m], sw[n], bias, n);
            if (out_dtype == OR_F32)
                ((float *)out)[m * N + n] = y;
            else
                ((uint16_t *)out)[m * N + n] = oracle_f32_to_bf16(y);
        }
    }
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* Whole linear: O4 -> O5 -> O6/O7                                     */
/* ------------------------------------------------------------------ */

/* X is bf16 [M, K]; qw/sw are the prepared weights [N, K] / [N], rotated
 * with kind `rot` (the activations get the same rotation). */
int oracle_linear_forward_rot(const uint16_t *X, int64_t M, int64_t K, int b, int rot,
                              const int8_t *qw, const float *sw, int64_t N,
                              const float *bias, int out_dtype, void *out)
{
    if (M == 0)
        return OR_OK;
    int8_t *qx = (int8_t *)malloc((size_t)M * (size_t)K);
    float *sx = (float *)malloc(sizeof(float) * (size_t)M);
    int32_t *acc = (int32_t *)malloc(sizeof(int32_t) * (size_t)M * (size_t)N);
    int rc = OR_EINVAL;
    if (qx && sx && acc) {
        rc = oracle_rotate_quantize_rows_rot(X, OR_BF16, M, K, K, b, rot, qx, sx);
        if (rc == OR_OK)
            rc = oracle_gemm_i32(qx, qw, M, N, K, acc);
        if (rc == OR_OK)
            rc = oracle_dequant(acc, sx, sw, bias, M, N, out_dtype, out);
    }
    free(qx);
    free(sx);
    free(acc);
    return rc;
}

int oracle_linear_forward(const uint16_t *X, int64_t M, int64_t K, int b,
                          const int8_t *qw, const float *sw, int64_t N,
                          const float *bias, int out_dtype, void *out)
{
    return oracle_linear_forward_rot(X, M, K, b, OR_ROT_SYLVESTER, qw, sw, N, bias,
                                     out_dtype, out);
}

/* ------------------------------------------------------------------ */
/* O8: low-rank chain (R6)                                             */
/* ------------------------------------------------------------------ */

/* h = bf16(linear(X; A)) with A [r, K] and no bias, then
 * y = linear(h; B) with B [N, r] and the bias.  If h_out is not NULL the bf16
 * intermediate is returned too. */
int oracle_lowrank_forward_rot(const uint16_t *X, int64_t M, int64_t K, int b, int rot,
                               const int8_t *qa, const float *sa, int64_t r,
                               const int8_t *qb, const float *sb, int64_t N,
                               const float *bias, int out_dtype, void *out,
                               uint16_t *h_out)
{
    if (r <= 0 || r % b != 0)
        return OR_EINVAL;
    if (M == 0)
        return OR_OK;
    uint16_t *h = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)M * (size_t)r);
    if (!h)
        return OR_EINVAL;
    int rc = oracle_linear_forward_rot(X, M, K, b, rot, qa, sa, r, NULL, OR_BF16, h);
    if (rc == OR_OK)
        rc = oracle_linear_forward_rot(h, M, r, b, rot, qb, sb, N, bias, out_dtype, out);
    if (rc == OR_OK && h_out)
        memcpy(h_out, h, sizeof(uint16_t) * (size_t)M * (size_t)r);
    free(h);
    return rc;
}

int oracle_lowrank_forward(const uint16_t *X, int64_t M, int64_t K, int b,
                           const int8_t *qa, const float *sa, int64_t r,
                           const int8_t *qb, const float *sb, int64_t N,
                           const float *bias, int out_dtype, void *out,
                           uint16_t *h_out)
{
    return oracle_lowrank_forward_rot(X, M, K, b, OR_ROT_SYLVESTER, qa, sa, r, qb, sb, N,
                                      bias, out_dtype, out, h_out);
}

/* ------------------------------------------------------------------ */
/* O9: MLP pair with an erf GELU between the projections (R7)          */
/* ------------------------------------------------------------------ */

/* GELU(z) = z/2 * (1 + erf(z / sqrt 2)), evaluated in fp64. */
double oracle_gelu_f64(double z) { return 0.5 * z * (1.0 + erf(z / sqrt(2.0))); }

/* g = bf16(GELU(float(u))) elementwise; u and g are bf16. */
void oracle_gelu_bf16(const uint16_t *u, int64_t n, uint16_t *g)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        double z = (double)oracle_bf16_to_f32(u[i]);
        g[i] = oracle_f32_to_bf16((float)oracle_gelu_f64(z));
    }
}

/* u = bf16(linear(X; W_up, bias_up)); g = GELU(u); y = linear(g; W_down,
 * bias_down).  u_out / g_out, when not NULL, receive the intermediates. */
int oracle_mlp_forward_rot(const uint16_t *X, int64_t M, int64_t K, int b, int rot,
                           const int8_t *qu, const float *su, int64_t F,
                           const float *bias_up, const int8_t *qd, const float *sd,
                           int64_t N, const float *bias_down, int out_dtype,
                           void *out, uint16_t *u_out, uint16_t *g_out)
{
    if (F <= 0 || F % b != 0)
        return OR_EINVAL;
    if (M == 0)
        return OR_OK;
    size_t n = (size_t)M * (size_t)F;
    uint16_t *u = (uint16_t *)malloc(sizeof(uint16_t) * n);
    uint16_t *g = (uint16_t *)malloc(sizeof(uint16_t) * n);
    int rc = OR_EINVAL;
    if (u && g) {
        rc = oracle_linear_forward_rot(X, M, K, b, rot, qu, su, F, bias_up, OR_BF16, u);
        if (rc == OR_OK) {
            oracle_gelu_bf16(u, (int64_t)n, g);
            rc = oracle_linear_forward_rot(g, M, F, b, rot, qd, sd, N, bias_down,
                                           out_dtype, out);
        }
        if (rc == OR_OK && u_out)
            memcpy(u_out, u, sizeof(uint16_t) * n);
        if (rc == OR_OK && g_out)
            memcpy(g_out, g, sizeof(uint16_t) * n);
    }
    free(u);
    free(g);
    return rc;
}

int oracle_mlp_forward(const uint16_t *X, int64_t M, int64_t K, int b,
                       const int8_t *qu, const float *su, int64_t F,
                       const float *bias_up, const int8_t *qd, const float *sd,
                       int64_t N, const float *bias_down, int out_dtype,
                       void *out, uint16_t *u_out, uint16_t *g_out)
{
    return oracle_mlp_forward_rot(X, M, K, b, OR_ROT_SYLVESTER, qu, su, F, bias_up, qd, sd, N,
                                  bias_down, out_dtype, out, u_out, g_out);
}

/* ------------------------------------------------------------------ */
/* R9: the bf16 low-rank comparison variant                            */
/* ------------------------------------------------------------------ */

/* out[m, n] = bf16(fp32(sum_k x[m, k] w[n, k]) (+ bias[n])) for bf16 x [M, K]
 * and w [N, K].  The sum is taken in fp64: a product of two bf16 values is
 * exact there, and so are sums of them over the exponent ranges used. */
static void bf16_linear(const uint16_t *x, const uint16_t *w, int64_t M, int64_t N,
                        int64_t K, const float *bias, uint16_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += (double)oracle_bf16_to_f32(x[m * K + k]) *
                       (double)oracle_bf16_to_f32(w[n * K + k]);
            float y = (float)acc;
            if (bias)
                y += bias[n];
            out[m * N + n] = oracle_f32_to_bf16(y);
        }
    }
}

/* h = bf16(X . A^T) [M, r], then y = bf16(h . B^T + bias) [M, N]; h_out, when
 * not NULL, receives h. */
int oracle_lowrank_bf16_forward(const uint16_t *X, int64_t M, int64_t K, const uint16_t *A,
                                int64_t r, const uint16_t *B, int64_t N, const float *bias,
                                uint16_t *y, uint16_t *h_out)
{
    if (M < 0 || K <= 0 || r <= 0 || N <= 0)
        return OR_EINVAL;
    if (M == 0)
        return OR_OK;
    uint16_t *h = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)M * (size_t)r);
    if (!h)
        return OR_EINVAL;
    bf16_linear(X, A, M, r, K, NULL, h);
    bf16_linear(h, B, M, N, r, bias, y);
    if (h_out)
        memcpy(h_out, h, sizeof(uint16_t) * (size_t)M * (size_t)r);
    free(h);
    return OR_OK;
}


/* ------------------------------------------------------------------ */
/* R10: SwiGLU MLP                                                     */
/* ------------------------------------------------------------------ */

/* silu(z) = z * sigmoid(z) = z / (1 + exp(-z)), evaluated in fp64. */
double oracle_silu_f64(double z) { return z / (1.0 + exp(-z)); }

/* The fp32 activation of one bf16 gate value: the fp64 evaluation rounded
 * once to fp32. */
float oracle_silu_f32(uint16_t a) { return (float)oracle_silu_f64((double)oracle_bf16_to_f32(a)); }

/* g [M, F] from the fc1 output gu [M, 2F] (gate = columns [0, F), up =
 * columns [F, 2F)): g = bf16(silu_f32(gate) * up), one fp32 product. */
void oracle_swiglu_bf16(const uint16_t *gu, int64_t M, int64_t F, uint16_t *g)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t j = 0; j < F; ++j) {
            float sg = oracle_silu_f32(gu[m * 2 * F + j]);
            float up = oracle_bf16_to_f32(gu[m * 2 * F + F + j]);
            float p = sg * up;
            g[m * F + j] = oracle_f32_to_bf16(p);
        }
    }
}

/* gu = bf16(linear(X; W_gu, bias_gu)) with W_gu [2F, K] rotated with block
 * b_up, g = swiglu(gu), y = linear(g; W_down, bias_down) with W_down [N, F]
 * rotated with block b_down.  gu_out / g_out, when not NULL, receive the
 * intermediates. */
int oracle_swiglu_mlp_forward_rot(const uint16_t *X, int64_t M, int64_t K, int b_up,
                                  int b_down, int rot, const int8_t *qgu, const float *sgu,
                                  int64_t F, const float *bias_gu, const int8_t *qd,
                                  const float *sd, int64_t N, const float *bias_down,
                                  int out_dtype, void *out, uint16_t *gu_out, uint16_t *g_out)
{
    if (F <= 0 || F % b_down != 0)
        return OR_EINVAL;
    if (M == 0)
        return OR_OK;
    size_t n = (size_t)M * (size_t)F;
    uint16_t *gu = (uint16_t *)malloc(sizeof(uint16_t) * 2 * n);
    uint16_t *g = (uint16_t *)malloc(sizeof(uint16_t) * n);
    int rc = OR_EINVAL;
    if (gu && g) {
        rc = oracle_linear_forward_rot(X, M, K, b_up, rot, qgu, sgu, 2 * F, bias_gu, OR_BF16, gu);
        if (rc == OR_OK) {
            oracle_swiglu_bf16(gu, M, F, g);
            rc = oracle_linear_forward_rot(g, M, F, b_down, rot, qd, sd, N, bias_down,
                                           out_dtype, out);
        }
        if (rc == OR_OK && gu_out)
            memcpy(gu_out, gu, sizeof(uint16_t) * 2 * n);
        if (rc == OR_OK && g_out)
            memcpy(g_out, g, sizeof(uint16_t) * n);
    }
    free(gu);
    free(g);
    return rc;
}
