/*
 * The host side of libconvrot.so (argument validation and workspace sizing)
 * driven under AddressSanitizer and UndefinedBehaviorSanitizer: every sizing
 * query over a grid of shapes, extreme ones included, and every validation
 * path that returns before a launch.  Device pointers are fake (never
 * dereferenced); no call here reaches the GPU.
 *
 * Test infrastructure: tests/test_abi_sanitized.py builds the library's host
 * code with the sanitizers, links this program against it and runs it on the
 * CPU.  It prints "N failed checks"; exit status 0 when N is 0.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "convrot.h"

static int failed = 0, checks = 0;

#define EXPECT(call, want)                                                           \
    do {                                                                             \
        int got_ = (call);                                                           \
        ++checks;                                                                    \
        if (got_ != (want)) {                                                        \
            ++failed;                                                                \
            printf("line %d: %s returned %d, expected %d\n", __LINE__, #call, got_,  \
                   (int)(want));                                                     \
        }                                                                            \
    } while (0)

#define FAKE ((void *)(uintptr_t)0x7f0000000000ull)
#define FAKE_ODD ((void *)(uintptr_t)0x7f0000000008ull)

static convrot_weights desc(int64_t N, int64_t K, int block)
{
    convrot_weights d;
    memset(&d, 0, sizeof d);
    d.magic = CONVROT_WEIGHTS_MAGIC;
    d.version = CONVROT_WEIGHTS_VERSION;
    d.N = N;
    d.K = K;
    d.block = block;
    d.codes = (int8_t *)FAKE;
    d.scale = (float *)FAKE;
    return d;
}

int main(void)
{
    /* status strings and version */
    for (int c = -8; c <= 2; ++c) {
        const char *s = convrot_status_string(c);
        ++checks;
        if (!s || !s[0]) { ++failed; printf("empty status string for %d\n", c); }
    }
    EXPECT(convrot_version() >= 100, 1);

    /* sizing: a grid of shapes, extremes included; the queries must not
     * overflow or trap, and must return 0 where the shape is unsupported */
    const int64_t dims[] = {-1, 0, 1, 15, 16, 64, 128, 500, 512, 5376, 21504, 65536, 65664,
                            1 << 20, (int64_t)1 << 31, (int64_t)1 << 40, INT64_MAX};
    const int blocks[] = {0, 32, 64, 100, 128, 256, 512};
    const int nd = sizeof dims / sizeof dims[0], nb = sizeof blocks / sizeof blocks[0];
    size_t acc = 0;
    for (int i = 0; i < nd; ++i)
        for (int j = 0; j < nd; ++j)
            for (int k = 0; k < nb; ++k) {
                acc += convrot_weights_packed_bytes(dims[i], dims[j], blocks[k]);
                acc += convrot_prepare_workspace_bytes(dims[i], dims[j], blocks[k], CONVROT_BF16,
                                                       CONVROT_IN_MAJOR);
                acc += convrot_linear_workspace_bytes(dims[i], dims[j], 512, blocks[k]);
                acc += lowrank_convrot_workspace_bytes(dims[i], dims[j], 512, dims[j], blocks[k]);
                acc += convrot_mlp_workspace_bytes(dims[i], dims[j], 21504, dims[j], blocks[k]);
                acc += lowrank_bf16_workspace_bytes(dims[i], dims[j]);
                acc += lowrank_convrot_prepare_workspace_bytes(dims[i], dims[j], dims[j],
                                                               blocks[k], CONVROT_F32);
                acc += (size_t)lowrank_convrot_padded_rank(dims[i], blocks[k]);
                acc += convrot_swiglu_prepare_workspace_bytes(dims[i], dims[j], blocks[k],
                                                              CONVROT_I8);
                acc += convrot_swiglu_mlp_workspace_bytes(dims[i], dims[j], dims[j], 512,
                                                          blocks[k], 64);
            }
    EXPECT(convrot_weights_packed_bytes(16, 65536 + 128, 128) == 0, 1);
    EXPECT(convrot_weights_packed_bytes(512, 5376, 128) == (size_t)512 * 5376, 1);

    /* forward validation */
    convrot_weights d = desc(512, 512, 128), bad = d;
    const size_t big_ws = (size_t)1 << 30;
    EXPECT(convrot_linear_forward(FAKE, 4, NULL, NULL, FAKE, CONVROT_BF16, FAKE, big_ws, NULL),
           CONVROT_EINVAL);
    EXPECT(convrot_linear_forward(FAKE, -1, &d, NULL, FAKE, CONVROT_BF16, FAKE, big_ws, NULL),
           CONVROT_EINVAL);
    EXPECT(convrot_linear_forward(FAKE, 0, &d, NULL, FAKE, CONVROT_BF16, FAKE, big_ws, NULL),
           CONVROT_OK);
    EXPECT(convrot_linear_forward(NULL, 4, &d, NULL, FAKE, CONVROT_BF16, FAKE, big_ws, NULL),
           CONVROT_EINVAL);
    EXPECT(convrot_linear_forward(FAKE_ODD, 4, &d, NULL, FAKE, CONVROT_BF16, FAKE, big_ws, NULL),
           CONVROT_EALIGN);
    EXPECT(convrot_linear_forward(FAKE, 4, &d, NULL, FAKE, CONVROT_BF16, NULL, big_ws, NULL),
           CONVROT_EWORKSPACE);
    EXPECT(convrot_linear_forward(FAKE, 4, &d, NULL, FAKE, CONVROT_BF16, FAKE, 16, NULL),
           CONVROT_EWORKSPACE);
    EXPECT(convrot_linear_forward(FAKE, 4, &d, NULL, FAKE, CONVROT_I8, FAKE, big_ws, NULL),
           CONVROT_EUNSUPPORTED);
    bad.magic = 0;
    EXPECT(convrot_linear_forward(FAKE, 4, &bad, NULL, FAKE, CONVROT_BF16, FAKE, big_ws, NULL),
           CONVROT_ELAYOUT);
    bad = d;
    bad.version = 9;
    EXPECT(convrot_linear_forward(FAKE, 4, &bad, NULL, FAKE, CONVROT_BF16, FAKE, big_ws, NULL),
           CONVROT_ELAYOUT);
    convrot_weights wide = desc(16, 65536, 128);
    EXPECT(convrot_linear_forward(FAKE, 40000, &wide, NULL, FAKE, CONVROT_BF16, FAKE, big_ws,
                                  NULL),
           CONVROT_EUNSUPPORTED);
    EXPECT(convrot_linear_forward(FAKE, INT64_MAX, &d, NULL, FAKE, CONVROT_BF16, FAKE, big_ws,
                                  NULL),
           CONVROT_EUNSUPPORTED);
    EXPECT(convrot_rotate_quantize(FAKE, CONVROT_BF16, INT64_MAX, 512, 128, 0, (int8_t *)FAKE,
                                   (float *)FAKE, NULL),
           CONVROT_EUNSUPPORTED);
    EXPECT(lowrank_bf16_forward(FAKE, INT64_MAX, 512, FAKE, 64, FAKE, INT64_MAX - 15, NULL, FAKE,
                                FAKE, 1 << 20, NULL),
           CONVROT_EUNSUPPORTED);
    convrot_weights tall = desc(INT64_MAX - 15, 512, 128);
    EXPECT(convrot_linear_forward(FAKE, 4, &tall, NULL, FAKE, CONVROT_BF16, FAKE, big_ws, NULL),
           CONVROT_EUNSUPPORTED);
    convrot_weights huge = desc(INT64_MAX / 2, INT64_MAX / 2, 128);
    EXPECT(convrot_linear_forward(FAKE, 4, &huge, NULL, FAKE, CONVROT_BF16, FAKE, big_ws, NULL)
               != CONVROT_OK, 1);

    /* prepare validation (nothing written on error) */
    convrot_weights out;
    memset(&out, 0, sizeof out);
    out.codes = (int8_t *)FAKE;
    out.scale = (float *)FAKE;
    EXPECT(convrot_linear_prepare_weights(FAKE, CONVROT_F32, CONVROT_OUT_MAJOR, NULL, 512, 512, 32,
                                          &out, NULL, 0, NULL),
           CONVROT_EINVAL);
    EXPECT(convrot_linear_prepare_weights(FAKE, CONVROT_F32, CONVROT_OUT_MAJOR, NULL, 24, 512,
                                          128, &out, NULL, 0, NULL),
           CONVROT_EUNSUPPORTED);
    EXPECT(convrot_linear_prepare_weights(FAKE, CONVROT_I8, CONVROT_OUT_MAJOR, NULL, 512, 512,
                                          128, &out, NULL, 0, NULL),
           CONVROT_EINVAL);
    EXPECT(convrot_linear_prepare_weights(FAKE, CONVROT_F32, 7, NULL, 512, 512, 128, &out, NULL,
                                          0, NULL),
           CONVROT_EINVAL);
    EXPECT(convrot_linear_prepare_weights(FAKE_ODD, CONVROT_F32, CONVROT_OUT_MAJOR, NULL, 512,
                                          512, 128, &out, NULL, 0, NULL),
           CONVROT_EALIGN);
    EXPECT(convrot_linear_prepare_weights(FAKE, CONVROT_F32, CONVROT_IN_MAJOR, NULL, 512, 512,
                                          128, &out, NULL, 0, NULL),
           CONVROT_EWORKSPACE);
    EXPECT(convrot_linear_prepare_weights(FAKE, CONVROT_F32, CONVROT_OUT_MAJOR, NULL, 512,
                                          INT64_MAX, 128, &out, NULL, 0, NULL) != CONVROT_OK, 1);
    EXPECT(out.magic == 0, 1);

    /* low-rank, MLP and the hooks */
    convrot_weights A = desc(256, 512, 128), B = desc(512, 256, 128), Br = desc(512, 384, 128);
    EXPECT(lowrank_convrot_forward(FAKE, 0, &A, &B, NULL, FAKE, CONVROT_BF16, FAKE, big_ws, NULL),
           CONVROT_OK);
    EXPECT(lowrank_convrot_forward(FAKE, 8, &A, &Br, NULL, FAKE, CONVROT_BF16, FAKE, big_ws,
                                   NULL),
           CONVROT_ELAYOUT);
    EXPECT(lowrank_convrot_forward(FAKE, 8, &A, &B, NULL, FAKE, CONVROT_BF16, FAKE, 64, NULL),
           CONVROT_EWORKSPACE);
    EXPECT(convrot_mlp_forward(FAKE, 8, &A, NULL, &Br, NULL, FAKE, CONVROT_BF16, FAKE, big_ws,
                               NULL),
           CONVROT_ELAYOUT);
    EXPECT(convrot_rotate_quantize(FAKE, CONVROT_BF16, 4, 500, 128, 0, (int8_t *)FAKE,
                                   (float *)FAKE, NULL),
           CONVROT_EINVAL);
    EXPECT(convrot_rotate_quantize(FAKE, CONVROT_BF16, 4, 512, 128, 0x200, (int8_t *)FAKE,
                                   (float *)FAKE, NULL),
           CONVROT_EUNSUPPORTED);
    EXPECT(convrot_gemm_i32((const int8_t *)FAKE_ODD, 4, &d, (int32_t *)FAKE, NULL),
           CONVROT_EALIGN);
    EXPECT(convrot_gemm_dequant((const int8_t *)FAKE, (const float *)FAKE, 4, &d, NULL, FAKE,
                                CONVROT_F32, CONVROT_FLAG_GELU, NULL),
           CONVROT_EUNSUPPORTED);
    convrot_weights r640 = desc(640, 512, 128);
    EXPECT(convrot_lowrank_factor1((const int8_t *)FAKE, (const float *)FAKE, 4, &r640,
                                   (int8_t *)FAKE, (float *)FAKE, NULL),
           CONVROT_EUNSUPPORTED);
    EXPECT(convrot_gelu_bf16((const uint16_t *)FAKE, -1, (uint16_t *)FAKE, NULL), CONVROT_EINVAL);
    EXPECT(convrot_gelu_bf16(NULL, 0, NULL, NULL), CONVROT_OK);
    EXPECT(lowrank_bf16_forward(FAKE, 8, 500, FAKE, 64, FAKE, 256, NULL, FAKE, FAKE, 1 << 20,
                                NULL),
           CONVROT_EUNSUPPORTED);
    /* low-rank preparation: rank padding and validation */
    EXPECT(lowrank_convrot_padded_rank(192, 64), 256);
    EXPECT(lowrank_convrot_padded_rank(320, 128), 384);
    EXPECT(lowrank_convrot_padded_rank(320, 256), 512);
    EXPECT(lowrank_convrot_padded_rank(512, 128), 512);
    EXPECT(lowrank_convrot_padded_rank(0, 128), 0);
    EXPECT(lowrank_convrot_prepare_workspace_bytes(512, 5376, 5376, 128, CONVROT_F32) == 0, 1);
    EXPECT(lowrank_convrot_prepare_workspace_bytes(192, 512, 272, 64, CONVROT_BF16) ==
               (size_t)256 * 512 * 2 + (size_t)272 * 256 * 2, 1);
    EXPECT(lowrank_convrot_prepare_workspace_bytes(192, 512, 272, 64, CONVROT_I8) == 0, 1);
    convrot_weights pa = desc(0, 0, 0), pb = desc(0, 0, 0);
    pa.magic = pb.magic = 0;
    EXPECT(lowrank_convrot_prepare_weights(FAKE, FAKE, CONVROT_I8, 192, 512, 272, 64, &pa, &pb,
                                           FAKE, 1 << 20, NULL),
           CONVROT_EUNSUPPORTED);
    EXPECT(lowrank_convrot_prepare_weights(FAKE, FAKE, CONVROT_F32, 192, 512, 272, 64, &pa, &pb,
                                           NULL, 0, NULL),
           CONVROT_EWORKSPACE);
    EXPECT(lowrank_convrot_prepare_weights(FAKE, FAKE, CONVROT_F32, 192, 500, 272, 64, &pa, &pb,
                                           FAKE, 1 << 20, NULL),
           CONVROT_EINVAL);
    EXPECT(lowrank_convrot_prepare_weights(FAKE_ODD, FAKE, CONVROT_F32, 192, 512, 272, 64, &pa,
                                           &pb, FAKE, 1 << 20, NULL),
           CONVROT_EALIGN);
    EXPECT(lowrank_convrot_prepare_weights(FAKE, FAKE, CONVROT_F32, 192, 512, 270, 64, &pa, &pb,
                                           FAKE, 1 << 20, NULL),
           CONVROT_EUNSUPPORTED);
    EXPECT(lowrank_convrot_prepare_weights(NULL, FAKE, CONVROT_F32, 192, 512, 272, 64, &pa, &pb,
                                           FAKE, 1 << 20, NULL),
           CONVROT_EINVAL);
    pb.flags = CONVROT_ROT_REGULAR;
    EXPECT(lowrank_convrot_prepare_weights(FAKE, FAKE, CONVROT_F32, 192, 512, 272, 64, &pa, &pb,
                                           FAKE, 1 << 20, NULL),
           CONVROT_EINVAL);
    EXPECT(pa.magic == 0 && pb.magic == 0, 1);
    /* SwiGLU: preparation, forward, the fused flag and the hooks */
    EXPECT(convrot_swiglu_prepare_workspace_bytes(256, 512, 128, CONVROT_F32) ==
               (size_t)512 * 512 * 4, 1);
    EXPECT(convrot_swiglu_prepare_workspace_bytes(256, 512, 128, CONVROT_I8) ==
               (size_t)512 * 512 + 2048, 1);
    EXPECT(convrot_swiglu_prepare_workspace_bytes(100, 512, 128, CONVROT_F32) == 0, 1);
    EXPECT(convrot_swiglu_mlp_workspace_bytes(8, 512, 256, 272, 128, 100) == 0, 1);
    EXPECT(convrot_swiglu_prepare_weights(FAKE, CONVROT_F32, NULL, 100, 512, 128, &pa, FAKE,
                                          1 << 20, NULL),
           CONVROT_EUNSUPPORTED);
    EXPECT(convrot_swiglu_prepare_weights(FAKE, CONVROT_I8, NULL, 256, 512, 128, &pa, FAKE,
                                          1 << 20, NULL),
           CONVROT_EINVAL);
    EXPECT(convrot_swiglu_prepare_weights(FAKE, CONVROT_F32, NULL, 256, 512, 128, &pa, NULL, 0,
                                          NULL),
           CONVROT_EWORKSPACE);
    EXPECT(convrot_swiglu_prepare_weights(FAKE_ODD, CONVROT_F32, NULL, 256, 512, 128, &pa, FAKE,
                                          1 << 20, NULL),
           CONVROT_EALIGN);
    EXPECT(pa.magic == 0, 1);
    convrot_weights gu = desc(512, 512, 128), dn = desc(272, 256, 64), gu_bad = gu;
    gu.flags = (int32_t)CONVROT_SWIGLU_PAIRS;
    EXPECT(convrot_swiglu_mlp_forward(FAKE, 8, &gu_bad, NULL, &dn, NULL, FAKE, CONVROT_BF16, FAKE,
                                      big_ws, NULL),
           CONVROT_ELAYOUT);                                  /* fc1 not interleaved */
    EXPECT(convrot_swiglu_mlp_forward(FAKE, 8, &gu, NULL, &gu, NULL, FAKE, CONVROT_BF16, FAKE,
                                      big_ws, NULL),
           CONVROT_ELAYOUT);                                  /* fc2 interleaved */
    convrot_weights dn_wide = desc(272, 384, 64);
    EXPECT(convrot_swiglu_mlp_forward(FAKE, 8, &gu, NULL, &dn_wide, NULL, FAKE, CONVROT_BF16,
                                      FAKE, big_ws, NULL),
           CONVROT_ELAYOUT);                                  /* 2F != fc1 outputs */
    EXPECT(convrot_swiglu_mlp_forward(FAKE, INT64_MAX, &gu, NULL, &dn, NULL, FAKE, CONVROT_BF16,
                                      FAKE, big_ws, NULL),
           CONVROT_EUNSUPPORTED);
    EXPECT(convrot_swiglu_mlp_forward(FAKE, 8, &gu, NULL, &dn, NULL, FAKE, CONVROT_BF16, FAKE, 64,
                                      NULL),
           CONVROT_EWORKSPACE);
    EXPECT(convrot_swiglu_mlp_forward(FAKE, 0, &gu, NULL, &dn, NULL, FAKE, CONVROT_BF16, FAKE,
                                      big_ws, NULL),
           CONVROT_OK);
    EXPECT(convrot_linear_forward(FAKE, 4, &gu, NULL, FAKE, CONVROT_BF16, FAKE, big_ws, NULL),
           CONVROT_ELAYOUT);                                  /* interleaved in a plain forward */
    EXPECT(convrot_gemm_dequant((const int8_t *)FAKE, (const float *)FAKE, 4, &d, NULL, FAKE,
                                CONVROT_BF16, CONVROT_FLAG_SWIGLU, NULL),
           CONVROT_ELAYOUT);                                  /* the flag on a plain weight */
    EXPECT(convrot_gemm_dequant((const int8_t *)FAKE, (const float *)FAKE, 4, &gu, NULL, FAKE,
                                CONVROT_F32, CONVROT_FLAG_SWIGLU, NULL),
           CONVROT_EUNSUPPORTED);                             /* bf16 only */
    EXPECT(convrot_swiglu_bf16((const uint16_t *)FAKE, -1, 16, (uint16_t *)FAKE, NULL),
           CONVROT_EINVAL);
    EXPECT(convrot_swiglu_bf16((const uint16_t *)FAKE, 4, 12, (uint16_t *)FAKE, NULL),
           CONVROT_EUNSUPPORTED);
    EXPECT(convrot_swiglu_bf16((const uint16_t *)FAKE_ODD, 4, 16, (uint16_t *)FAKE, NULL),
           CONVROT_EALIGN);
    EXPECT(convrot_swiglu_bf16(NULL, 0, 16, NULL, NULL), CONVROT_OK);
    EXPECT(convrot_silu_f32((const uint16_t *)FAKE, -1, (float *)FAKE, NULL), CONVROT_EINVAL);
    EXPECT(convrot_silu_f32(NULL, 0, NULL, NULL), CONVROT_OK);
    /* the allocation-free forward: a workspace beyond its static array, bad M */
    EXPECT(convrot_linear_forward_noalloc(FAKE, 1 << 20, &d, NULL, FAKE, CONVROT_BF16, NULL),
           CONVROT_EWORKSPACE);
    EXPECT(convrot_linear_forward_noalloc(FAKE, -1, &d, NULL, FAKE, CONVROT_BF16, NULL),
           CONVROT_EINVAL);
    EXPECT(convrot_linear_forward_noalloc(FAKE, 0, &d, NULL, FAKE, CONVROT_BF16, NULL), CONVROT_OK);

    int64_t ops = 0;
    EXPECT(convrot_probe_mfma_i8(0, FAKE, FAKE, &ops, NULL), CONVROT_EINVAL);
    EXPECT(convrot_probe_stream(FAKE, FAKE, 64, 3, NULL), CONVROT_EINVAL);
    EXPECT(convrot_probe_stream(FAKE_ODD, FAKE, 64, 0, NULL), CONVROT_EALIGN);

    printf("%d checks, %d failed checks (sizing sum %zu)\n", checks, failed, acc);
    return failed ? 1 : 0;
}
