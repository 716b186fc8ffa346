/*
 * A C program that drives libconvrot.so through its C ABI alone: device
 * buffers from hipMalloc, no Python, no PyTorch.  It prepares a weight, runs
 * one linear forward with bias and fp32 output, and checks the weight codes,
 * the weight scales and every output against the CPU oracle linked beside
 * it, bit for bit.  It also checks that a misaligned pointer is rejected
 * before anything is launched.
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
    hipFree(dX); hipFree(dW); hipFree(dcodes); hipFree(dscale); hipFree(dbias); hipFree(dY);
    hipFree(dwsp); hipFree(dwsf);
    free(X); free(W); free(bias); free(Y); free(Yref); free(sw); free(sw_ref); free(qw_ref);
    free(codes);
    return (bad_codes || bad_scales || bad_out) ? 1 : 0;
}
