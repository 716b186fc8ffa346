/*
 * A C program that drives libconvrot.so through its C ABI alone: device
 * buffers from hipMalloc, no Python, no PyTorch.  It prepares a weight, runs
 * one linear forward with bias and fp32 output, and checks the weight codes,
 * the weight scales and every output against the CPU oracle linked beside
 * it, bit for bit.  It also checks that a misaligned pointer is rejected
 * before anything is launched.  Then it prepares low-rank pairs whose rank
 * needs padding (lowrank_convrot_prepare_weights) and runs the low-rank
 * forward with bias: outputs bit for bit against the oracle's chain on the
 * unpadded factors when b divides r, on zero-padded factors otherwise.  Last,
 * the SwiGLU MLP (fc1 prepared interleaved, fc2 with its own block, biases on
 * both), bit for bit against the oracle's chain, after checking that a plain
 * forward refuses the interleaved fc1 weight.
 *
 * Test infrastructure: tests/test_c_abi.py builds it with gcc and runs it.
 * Exit status 0 = every check passed.
 */
#include <hip/hip_runtime_api.h>

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "convrot.h"

/* the oracle's C entry points (oracle/convrot_oracle.c); dtype 0 = F32 */
int oracle_rotate_quantize_rows_rot(const void *src, int dtype, int64_t rows, int64_t K,
                                    int64_t ld, int b, int rot, int8_t *q, float *s);
int oracle_linear_forward(const uint16_t *X, int64_t M, int64_t K, int b, const int8_t *qw,
                          const float *sw, int64_t N, const float *bias, int out_dtype,
                          void *out);
int oracle_lowrank_forward(const uint16_t *X, int64_t M, int64_t K, int b, const int8_t *qa,
                           const float *sa, int64_t r, const int8_t *qb, const float *sb,
                           int64_t N, const float *bias, int out_dtype, void *out,
                           uint16_t *h_out);
int oracle_swiglu_mlp_forward_rot(const uint16_t *X, int64_t M, int64_t K, int b_up,
                                  int b_down, int rot, const int8_t *qgu, const float *sgu,
                                  int64_t F, const float *bias_gu, const int8_t *qd,
                                  const float *sd, int64_t N, const float *bias_down,
                                  int out_dtype, void *out, uint16_t *gu_out, uint16_t *g_out);

#define HIP_OK(x)                                                                  \
    do {                                                                           \
        hipError_t e_ = (x);                                                       \
        if (e_ != hipSuccess) {                                                    \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                \
            return 2;                                                              \
        }                                                                          \
    } while (0)
#define CR_OK(x)                                                                   \
    do {                                                                           \
        int r_ = (x);                                                              \
        if (r_ != CONVROT_OK) {                                                    \
            fprintf(stderr, "%s: %s\n", #x, convrot_status_string(r_));            \
            return 3;                                                              \
        }                                                                          \
    } while (0)

/* 64-bit LCG (Knuth's MMIX constants), uniform in [-1, 1) */
static float uniform(uint64_t *s)
{
    *s = *s * 6364136223846793005ULL + 1442695040888963407ULL;
    return (float)(*s >> 40) * (1.0f / 8388608.0f) - 1.0f;
}

/* fp32 -> bf16 bits, round to nearest even (inputs here are finite) */
static uint16_t to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* byte offset of code (m, k) in the K-tiled layout of the public header */
static int64_t tiled(int64_t m, int64_t k, int64_t K)
{
    return ((m / 16) * (K / 64) + k / 64) * 1024 + (m % 16) * 64 +
           (((k / 16) % 4) ^ ((m / 4) % 4)) * 16 + k % 16;
}

/* One low-rank pair A [r, K], B [N, r] (fp32, seeded), rank r padded by the
 * library; returns the number of fp32 outputs that differ from the oracle
 * (or a negative code on a failed call). */
static int64_t lowrank_case(const uint16_t *X, const void *dX, int64_t M, int64_t K, int64_t r,
                            int64_t N, int b, uint64_t *seed)
{
    const int64_t rp = lowrank_convrot_padded_rank(r, b);
    /* the oracle's factors: unpadded when b divides r, else zero-padded */
    const int64_t ro = (r % b == 0) ? r : rp;
    float *A = calloc((size_t)(ro * K), sizeof(float)), *B = calloc((size_t)(N * ro), sizeof(float));
    float *A0 = malloc(sizeof(float) * r * K), *B0 = malloc(sizeof(float) * N * r);
    float *bias = malloc(sizeof(float) * N), *Y = malloc(sizeof(float) * M * N);
    float *Yref = malloc(sizeof(float) * M * N), *sa = malloc(sizeof(float) * ro);
    float *sb = malloc(sizeof(float) * N);
    int8_t *qa = malloc((size_t)(ro * K)), *qb = malloc((size_t)(N * ro));
    if (!A || !B || !A0 || !B0 || !bias || !Y || !Yref || !sa || !sb || !qa || !qb || rp <= 0)
        return -4;
    for (int64_t i = 0; i < r * K; ++i) A0[i] = A[i] = 0.05f * uniform(seed);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < r; ++j) B0[n * r + j] = B[n * ro + j] = 0.05f * uniform(seed);
    for (int64_t i = 0; i < N; ++i) bias[i] = 0.5f * uniform(seed);

    void *dA, *dB, *dca, *dsa, *dcb, *dsb, *dbias, *dY, *dwp = NULL, *dws;
    const size_t ca = convrot_weights_packed_bytes(rp, K, b), cb = convrot_weights_packed_bytes(N, rp, b);
    const size_t wp = lowrank_convrot_prepare_workspace_bytes(r, K, N, b, CONVROT_F32);
    const size_t wf = lowrank_convrot_workspace_bytes(M, K, rp, N, b);
    if (!ca || !cb || !wf || (rp != r && !wp)) return -5;
    if (hipMalloc(&dA, sizeof(float) * r * K) || hipMalloc(&dB, sizeof(float) * N * r) ||
        hipMalloc(&dca, ca) || hipMalloc(&dsa, 4 * rp) || hipMalloc(&dcb, cb) ||
        hipMalloc(&dsb, 4 * N) || hipMalloc(&dbias, 4 * N) || hipMalloc(&dY, 4 * M * N) ||
        (wp && hipMalloc(&dwp, wp)) || hipMalloc(&dws, wf))
        return -2;
    if (hipMemcpy(dA, A0, sizeof(float) * r * K, hipMemcpyHostToDevice) ||
        hipMemcpy(dB, B0, sizeof(float) * N * r, hipMemcpyHostToDevice) ||
        hipMemcpy(dbias, bias, 4 * N, hipMemcpyHostToDevice))
        return -2;
    convrot_weights wa, wb;
    memset(&wa, 0, sizeof wa);
    memset(&wb, 0, sizeof wb);
    wa.codes = (int8_t *)dca; wa.scale = (float *)dsa;
    wb.codes = (int8_t *)dcb; wb.scale = (float *)dsb;
    int rc = lowrank_convrot_prepare_weights(dA, dB, CONVROT_F32, r, K, N, b, &wa, &wb, dwp, wp,
                                             NULL);
    if (rc == CONVROT_OK && (wa.N != rp || wb.K != rp)) rc = -6;
    if (rc == CONVROT_OK)
        rc = lowrank_convrot_forward(dX, M, &wa, &wb, dbias, dY, CONVROT_F32, dws, wf, NULL);
    if (rc != CONVROT_OK) {
        fprintf(stderr, "low-rank r=%lld b=%d: %s\n", (long long)r, b, convrot_status_string(rc));
        return -3;
    }
    if (hipDeviceSynchronize() || hipMemcpy(Y, dY, 4 * M * N, hipMemcpyDeviceToHost)) return -2;
    if (oracle_rotate_quantize_rows_rot(A, 0, ro, K, K, b, 0, qa, sa) != 0 ||
        oracle_rotate_quantize_rows_rot(B, 0, N, ro, ro, b, 0, qb, sb) != 0 ||
        oracle_lowrank_forward(X, M, K, b, qa, sa, ro, qb, sb, N, bias, 0, Yref, NULL) != 0)
        return -6;
    int64_t bad = 0;
    for (int64_t i = 0; i < M * N; ++i) bad += memcmp(&Y[i], &Yref[i], 4) != 0;
    printf("c-abi low-rank M=%lld K=%lld r=%lld (stored %lld) N=%lld b=%d: %lld outputs differ "
           "from the oracle\n", (long long)M, (long long)K, (long long)r, (long long)rp,
           (long long)N, b, (long long)bad);
    hipFree(dA); hipFree(dB); hipFree(dca); hipFree(dsa); hipFree(dcb); hipFree(dsb);
    hipFree(dbias); hipFree(dY); hipFree(dwp); hipFree(dws);
    free(A); free(B); free(A0); free(B0); free(bias); free(Y); free(Yref); free(sa); free(sb);
    free(qa); free(qb);
    return bad;
}

/* The SwiGLU MLP: fc1 W_gu [2F, K] (gate rows, then up rows) prepared by
 * convrot_swiglu_prepare_weights with block b_up, fc2 W_down [N, F] with its
 * own block b_down, biases on both; returns the number of fp32 outputs that
 * differ from the oracle (or a negative code on a failed call). */
static int64_t swiglu_case(const uint16_t *X, const void *dX, int64_t M, int64_t K, int64_t F,
                           int64_t N, int b_up, int b_down, uint64_t *seed)
{
    float *Wgu = malloc(sizeof(float) * 2 * F * K), *Wd = malloc(sizeof(float) * N * F);
    float *bgu = malloc(sizeof(float) * 2 * F), *bd = malloc(sizeof(float) * N);
    float *Y = malloc(sizeof(float) * M * N), *Yref = malloc(sizeof(float) * M * N);
    float *sgu = malloc(sizeof(float) * 2 * F), *sd = malloc(sizeof(float) * N);
    int8_t *qgu = malloc((size_t)(2 * F * K)), *qd = malloc((size_t)(N * F));
    if (!Wgu || !Wd || !bgu || !bd || !Y || !Yref || !sgu || !sd || !qgu || !qd) return -4;
    for (int64_t i = 0; i < 2 * F * K; ++i) Wgu[i] = 0.05f * uniform(seed);
    for (int64_t i = 0; i < N * F; ++i) Wd[i] = 0.05f * uniform(seed);
    for (int64_t i = 0; i < 2 * F; ++i) bgu[i] = 0.5f * uniform(seed);
    for (int64_t i = 0; i < N; ++i) bd[i] = 0.5f * uniform(seed);

    void *dWgu, *dWd, *dcgu, *dsgu, *dcd, *dsd, *dbgu, *dbd, *dY, *dwp, *dwd = NULL, *dws;
    const size_t cgu = convrot_weights_packed_bytes(2 * F, K, b_up);
    const size_t cd = convrot_weights_packed_bytes(N, F, b_down);
    const size_t wp = convrot_swiglu_prepare_workspace_bytes(F, K, b_up, CONVROT_F32);
    const size_t wd = convrot_prepare_workspace_bytes(N, F, b_down, CONVROT_F32, CONVROT_OUT_MAJOR);
    const size_t wf = convrot_swiglu_mlp_workspace_bytes(M, K, F, N, b_up, b_down);
    if (!cgu || !cd || !wp || !wf) return -5;
    if (hipMalloc(&dWgu, sizeof(float) * 2 * F * K) || hipMalloc(&dWd, sizeof(float) * N * F) ||
        hipMalloc(&dcgu, cgu) || hipMalloc(&dsgu, 8 * F) || hipMalloc(&dcd, cd) ||
        hipMalloc(&dsd, 4 * N) || hipMalloc(&dbgu, 8 * F) || hipMalloc(&dbd, 4 * N) ||
        hipMalloc(&dY, 4 * M * N) || hipMalloc(&dwp, wp) || (wd && hipMalloc(&dwd, wd)) ||
        hipMalloc(&dws, wf))
        return -2;
    if (hipMemcpy(dWgu, Wgu, sizeof(float) * 2 * F * K, hipMemcpyHostToDevice) ||
        hipMemcpy(dWd, Wd, sizeof(float) * N * F, hipMemcpyHostToDevice) ||
        hipMemcpy(dbgu, bgu, 8 * F, hipMemcpyHostToDevice) ||
        hipMemcpy(dbd, bd, 4 * N, hipMemcpyHostToDevice))
        return -2;
    convrot_weights wgu, wdn;
    memset(&wgu, 0, sizeof wgu);
    memset(&wdn, 0, sizeof wdn);
    wgu.codes = (int8_t *)dcgu; wgu.scale = (float *)dsgu;
    wdn.codes = (int8_t *)dcd; wdn.scale = (float *)dsd;
    int rc = convrot_swiglu_prepare_weights(dWgu, CONVROT_F32, NULL, F, K, b_up, &wgu, dwp, wp,
                                            NULL);
    if (rc == CONVROT_OK)
        rc = convrot_linear_prepare_weights(dWd, CONVROT_F32, CONVROT_OUT_MAJOR, NULL, N, F,
                                            b_down, &wdn, dwd, wd, NULL);
    /* the interleaved fc1 weight is not a plain linear weight */
    if (rc == CONVROT_OK &&
        convrot_linear_forward(dX, M, &wgu, NULL, dY, CONVROT_F32, dws, wf, NULL) != CONVROT_ELAYOUT)
        rc = -7;
    if (rc == CONVROT_OK)
        rc = convrot_swiglu_mlp_forward(dX, M, &wgu, (const float *)dbgu, &wdn, (const float *)dbd,
                                        dY, CONVROT_F32, dws, wf, NULL);
    if (rc != CONVROT_OK) {
        fprintf(stderr, "swiglu F=%lld: %s\n", (long long)F,
                rc < -6 ? "a plain forward accepted the fc1 weight" : convrot_status_string(rc));
        return -3;
    }
    if (hipDeviceSynchronize() || hipMemcpy(Y, dY, 4 * M * N, hipMemcpyDeviceToHost)) return -2;
    if (oracle_rotate_quantize_rows_rot(Wgu, 0, 2 * F, K, K, b_up, 0, qgu, sgu) != 0 ||
        oracle_rotate_quantize_rows_rot(Wd, 0, N, F, F, b_down, 0, qd, sd) != 0 ||
        oracle_swiglu_mlp_forward_rot(X, M, K, b_up, b_down, 0, qgu, sgu, F, bgu, qd, sd, N, bd,
                                      0, Yref, NULL, NULL) != 0)
        return -6;
    int64_t bad = 0;
    for (int64_t i = 0; i < M * N; ++i) bad += memcmp(&Y[i], &Yref[i], 4) != 0;
    printf("c-abi swiglu M=%lld K=%lld F=%lld N=%lld b=%d/%d: %lld outputs differ from the "
           "oracle\n", (long long)M, (long long)K, (long long)F, (long long)N, b_up, b_down,
           (long long)bad);
    hipFree(dWgu); hipFree(dWd); hipFree(dcgu); hipFree(dsgu); hipFree(dcd); hipFree(dsd);
    hipFree(dbgu); hipFree(dbd); hipFree(dY); hipFree(dwp); hipFree(dwd); hipFree(dws);
    free(Wgu); free(Wd); free(bgu); free(bd); free(Y); free(Yref); free(sgu); free(sd);
    free(qgu); free(qd);
    return bad;
}

int main(void)
{
    const int64_t M = 300, K = 1024, N = 512;
    const int b = 128;
    uint64_t seed = 12345;

    uint16_t *X = malloc(sizeof(uint16_t) * M * K);
    float *W = malloc(sizeof(float) * N * K), *bias = malloc(sizeof(float) * N);
    float *Y = malloc(sizeof(float) * M * N), *Yref = malloc(sizeof(float) * M * N);
    float *sw = malloc(sizeof(float) * N), *sw_ref = malloc(sizeof(float) * N);
    int8_t *qw_ref = malloc((size_t)(N * K));
    const size_t code_bytes = convrot_weights_packed_bytes(N, K, b);
    int8_t *codes = malloc(code_bytes);
    if (!X || !W || !bias || !Y || !Yref || !sw || !sw_ref || !qw_ref || !codes || !code_bytes)
        return 4;
    for (int64_t i = 0; i < M * K; ++i) X[i] = to_bf16(3.0f * uniform(&seed));
    for (int64_t i = 0; i < N * K; ++i) W[i] = 0.05f * uniform(&seed);
    for (int64_t i = 0; i < N; ++i) bias[i] = 0.01f * uniform(&seed);

    void *dX, *dW, *dcodes, *dscale, *dbias, *dY, *dwsp = NULL, *dwsf;
    const size_t wsp = convrot_prepare_workspace_bytes(N, K, b, CONVROT_F32, CONVROT_OUT_MAJOR);
    const size_t wsf = convrot_linear_workspace_bytes(M, K, N, b);
    HIP_OK(hipMalloc(&dX, sizeof(uint16_t) * M * K));
    HIP_OK(hipMalloc(&dW, sizeof(float) * N * K));
    HIP_OK(hipMalloc(&dcodes, code_bytes));
    HIP_OK(hipMalloc(&dscale, sizeof(float) * N));
    HIP_OK(hipMalloc(&dbias, sizeof(float) * N));
    HIP_OK(hipMalloc(&dY, sizeof(float) * M * N));
    if (wsp) HIP_OK(hipMalloc(&dwsp, wsp));
    HIP_OK(hipMalloc(&dwsf, wsf));
    HIP_OK(hipMemcpy(dX, X, sizeof(uint16_t) * M * K, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dW, W, sizeof(float) * N * K, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dbias, bias, sizeof(float) * N, hipMemcpyHostToDevice));

    convrot_weights w;
    memset(&w, 0, sizeof w);
    w.codes = (int8_t *)dcodes;
    w.scale = (float *)dscale;
    CR_OK(convrot_linear_prepare_weights(dW, CONVROT_F32, CONVROT_OUT_MAJOR, NULL, N, K, b, &w,
                                         dwsp, wsp, NULL));
    /* a misaligned output pointer: rejected, nothing launched */
    if (convrot_linear_forward(dX, M, &w, dbias, (char *)dY + 4, CONVROT_F32, dwsf, wsf, NULL) !=
        CONVROT_EALIGN) {
        fprintf(stderr, "misaligned output not rejected\n");
        return 5;
    }
    CR_OK(convrot_linear_forward(dX, M, &w, dbias, dY, CONVROT_F32, dwsf, wsf, NULL));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(Y, dY, sizeof(float) * M * N, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(codes, dcodes, code_bytes, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(sw, dscale, sizeof(float) * N, hipMemcpyDeviceToHost));

    if (oracle_rotate_quantize_rows_rot(W, 0, N, K, K, b, 0, qw_ref, sw_ref) != 0 ||
        oracle_linear_forward(X, M, K, b, qw_ref, sw_ref, N, bias, 0, Yref) != 0)
        return 6;
    int64_t bad_codes = 0, bad_scales = 0, bad_out = 0;
    for (int64_t n = 0; n < N; ++n) {
        bad_scales += memcmp(&sw[n], &sw_ref[n], 4) != 0;
        for (int64_t k = 0; k < K; ++k) bad_codes += codes[tiled(n, k, K)] != qw_ref[n * K + k];
    }
    for (int64_t i = 0; i < M * N; ++i) bad_out += memcmp(&Y[i], &Yref[i], 4) != 0;
    printf("c-abi forward M=%lld K=%lld N=%lld b=%d: %lld codes, %lld scales, %lld outputs "
           "differ from the oracle\n",
           (long long)M, (long long)K, (long long)N, b, (long long)bad_codes,
           (long long)bad_scales, (long long)bad_out);
    /* low-rank pairs: r = 192 at b = 64 (padded to 256, b divides r) and
     * r = 320 at b = 128 (padded to 384, b does not divide r) */
    const int64_t lr1 = lowrank_case(X, dX, M, K, 192, 272, 64, &seed);
    const int64_t lr2 = lowrank_case(X, dX, M, K, 320, 272, 128, &seed);
    if (lr1 != 0 || lr2 != 0) return lr1 < 0 || lr2 < 0 ? 7 : 1;
    /* the SwiGLU MLP: fc1 b = 128, fc2 ConvRot64 */
    const int64_t sg = swiglu_case(X, dX, M, K, 256, 272, 128, 64, &seed);
    if (sg != 0) return sg < 0 ? 8 : 1;
    hipFree(dX); hipFree(dW); hipFree(dcodes); hipFree(dscale); hipFree(dbias); hipFree(dY);
    hipFree(dwsp); hipFree(dwsf);
    free(X); free(W); free(bias); free(Y); free(Yref); free(sw); free(sw_ref); free(qw_ref);
    free(codes);
    return (bad_codes || bad_scales || bad_out) ? 1 : 0;
}
