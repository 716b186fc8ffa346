// C ABI of libconvrot: argument validation, workspace carving and launch
// sequencing.  Every check runs on the host before any launch; a call that
// fails validation launches nothing.
#include "convrot.h"
#include "common.hpp"

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

namespace convrot {

int device_cu_count()
{
    // one entry per device ordinal; threads racing on a first query store
    // the same value
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
        n = 256;
    if (dev < 64) cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

} // namespace convrot

namespace {

constexpr int64_t kMaxK = 65536;
constexpr int64_t kI32Bound = (int64_t)1 << 31;
constexpr size_t kAlign = 256;

thread_local int g_last_hip_error = 0;

bool log_enabled()
{
    static const bool on = [] {
        const char *e = std::getenv("CONVROT_LOG");
        return e && e[0] == '1';
    }();
    return on;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_block(int b) { return b == 64 || b == 128 || b == 256; }

// Rotation kinds (convrot_weights.flags, convrot_rotate_quantize flags): the
// Sylvester blocks, or CONVROT_ROT_REGULAR, the H_4 Kronecker blocks, which
// exist for b = 64 and 256 only.
bool valid_rotation(uint32_t rot, int b)
{
    if (rot == 0) return true;
    return rot == CONVROT_ROT_REGULAR && (b == 64 || b == 256);
}

bool is_regular(const convrot_weights *W) { return (W->flags & CONVROT_ROT_REGULAR) != 0; }
uint32_t rotation_of(const convrot_weights *W) { return (uint32_t)W->flags & CONVROT_ROT_REGULAR; }
bool is_swiglu_pairs(const convrot_weights *W)
{
    return ((uint32_t)W->flags & CONVROT_SWIGLU_PAIRS) != 0;
}

// fp32 1/sqrt(b), rounded once from double.
float inv_sqrt_block(int b) { return (float)(1.0 / std::sqrt((double)b)); }

int hip_status(hipError_t e)
{
    if (e == hipSuccess) return CONVROT_OK;
    g_last_hip_error = (int)e;
    if (log_enabled())
        std::fprintf(stderr, "[convrot] HIP error %d: %s\n", (int)e, hipGetErrorString(e));
    return CONVROT_EHIP;
}

// Shape rules shared by every projection (K inputs, N outputs, block b).
int check_linear_shape(int64_t N, int64_t K, int block)
{
    if (N <= 0 || K <= 0 || !valid_block(block) || K % block != 0) return CONVROT_EINVAL;
    // N is bounded before the product, so it cannot overflow
    if (K % 128 != 0 || N % 16 != 0 || K > kMaxK || N >= kI32Bound || N * K >= kI32Bound)
        return CONVROT_EUNSUPPORTED;
    return CONVROT_OK;
}

// A prepared descriptor.  `pairs`: whether the weight must (true) or must not
// (false) hold interleaved SwiGLU gate/up rows; a mismatch is ELAYOUT, since
// the outputs of such a weight are not the columns of a plain linear.
int check_weights(const convrot_weights *W, bool pairs = false)
{
    if (!W) return CONVROT_EINVAL;
    if (W->magic != CONVROT_WEIGHTS_MAGIC || W->version != CONVROT_WEIGHTS_VERSION)
        return CONVROT_ELAYOUT;
    if (!W->codes || !W->scale) return CONVROT_EINVAL;
    if (!aligned16(W->codes) || !aligned16(W->scale)) return CONVROT_EALIGN;
    int rc = check_linear_shape(W->N, W->K, W->block);
    const uint32_t extra = (uint32_t)W->flags & ~(CONVROT_ROT_REGULAR | CONVROT_SWIGLU_PAIRS);
    if (rc == CONVROT_OK &&
        (extra != 0 || !valid_rotation(rotation_of(W), W->block) || is_swiglu_pairs(W) != pairs ||
         (pairs && W->N % 32 != 0)))
        return CONVROT_ELAYOUT;
    return rc == CONVROT_EINVAL ? CONVROT_ELAYOUT : rc;
}

// M rows of K: the K-tiled codes hold padded_rows(M) rows, and every byte
// offset the kernels form must fit in 32 bits.
int check_rows(int64_t M, int64_t K)
{
    if (M < 0) return CONVROT_EINVAL;
    // K <= 65536 here; M is bounded before padding and product
    if (M >= kI32Bound || convrot::padded_rows(M) * K >= kI32Bound) return CONVROT_EUNSUPPORTED;
    return CONVROT_OK;
}

int check_out_dtype(int y_dtype)
{
    return (y_dtype == CONVROT_BF16 || y_dtype == CONVROT_F32) ? CONVROT_OK : CONVROT_EUNSUPPORTED;
}

convrot::OutKind out_kind(int y_dtype)
{
    return y_dtype == CONVROT_F32 ? convrot::OutKind::F32 : convrot::OutKind::BF16;
}

// Bump allocator over a caller workspace.
struct Carve {
    char *base;
    size_t used = 0;
    explicit Carve(void *p) : base(static_cast<char *>(p)) {}
    void *take(size_t bytes)
    {
        void *p = base ? base + used : nullptr;
        used += round_up(bytes, kAlign);
        return p;
    }
};

size_t codes_bytes(int64_t M, int64_t K)
{
    return round_up((size_t)convrot::padded_rows(M) * (size_t)K, kAlign);
}
size_t scales_bytes(int64_t M) { return round_up((size_t)M * 4u, kAlign); }

// With CONVROT_LOG=1 the main entry points also print their name, shape and
// status to stderr.
void log_call(const char *name, int64_t M, int64_t N, int64_t K, int rc)
{
    if (log_enabled())
        std::fprintf(stderr, "[convrot] %s M=%lld N=%lld K=%lld -> %s\n", name, (long long)M,
                     (long long)N, (long long)K, convrot_status_string(rc));
}

} // namespace

extern "C" {

const char *convrot_status_string(int status)
{
    switch (status) {
    case CONVROT_OK: return "ok";
    case CONVROT_EINVAL: return "invalid argument";
    case CONVROT_EALIGN: return "pointer not 16-byte aligned";
    case CONVROT_EWORKSPACE: return "workspace missing or too small";
    case CONVROT_ELAYOUT: return "weight descriptor layout/version mismatch";
    case CONVROT_EUNSUPPORTED: return "unsupported shape or dtype";
    case CONVROT_EHIP: return "HIP launch error";
    default: return "unknown status";
    }
}

int convrot_last_hip_error(void) { return g_last_hip_error; }

int convrot_version(void) { return 100; }

size_t convrot_weights_packed_bytes(int64_t N, int64_t K, int block)
{
    if (check_linear_shape(N, K, block) != CONVROT_OK) return 0;
    return (size_t)N * (size_t)K;
}

size_t convrot_prepare_workspace_bytes(int64_t N, int64_t K, int block, int w_dtype,
                                       int layout)
{
    if (check_linear_shape(N, K, block) != CONVROT_OK) return 0;
    if (layout == CONVROT_IN_MAJOR && (w_dtype == CONVROT_F32 || w_dtype == CONVROT_BF16))
        return round_up((size_t)N * (size_t)K * (w_dtype == CONVROT_F32 ? 4u : 2u), kAlign);
    return 0;
}

size_t convrot_linear_workspace_bytes(int64_t M, int64_t K, int64_t N, int block)
{
    if (check_linear_shape(N, K, block) != CONVROT_OK || check_rows(M, K) != CONVROT_OK)
        return 0;
    return codes_bytes(M, K) + scales_bytes(M);
}

size_t lowrank_convrot_workspace_bytes(int64_t M, int64_t K, int64_t r, int64_t N, int block)
{
    if (check_linear_shape(r, K, block) != CONVROT_OK ||
        check_linear_shape(N, r, block) != CONVROT_OK || check_rows(M, K) != CONVROT_OK ||
        check_rows(M, r) != CONVROT_OK)
        return 0;
    return codes_bytes(M, K) + scales_bytes(M) + round_up((size_t)M * (size_t)r * 2u, kAlign) +
           codes_bytes(M, r) + scales_bytes(M);
}

size_t convrot_mlp_workspace_bytes(int64_t M, int64_t K, int64_t F, int64_t N, int block)
{
    if (check_linear_shape(F, K, block) != CONVROT_OK ||
        check_linear_shape(N, F, block) != CONVROT_OK || check_rows(M, K) != CONVROT_OK ||
        check_rows(M, F) != CONVROT_OK)
        return 0;
    return codes_bytes(M, K) + scales_bytes(M) + round_up((size_t)M * (size_t)F * 2u, kAlign) +
           codes_bytes(M, F) + scales_bytes(M);
}

static int prepare_weights_impl(const void *W, int w_dtype, int layout,
                                   const float *src_scale, int64_t N, int64_t K, int block,
                                   convrot_weights *out, void *ws, size_t ws_bytes, void *stream)
{
    if (!W || !out || !out->codes || !out->scale) return CONVROT_EINVAL;
    int rc = check_linear_shape(N, K, block);
    if (rc != CONVROT_OK) return rc;
    if (layout != CONVROT_OUT_MAJOR && layout != CONVROT_IN_MAJOR) return CONVROT_EINVAL;
    if (w_dtype != CONVROT_F32 && w_dtype != CONVROT_BF16 && w_dtype != CONVROT_I8)
        return CONVROT_EUNSUPPORTED;
    const bool import = (w_dtype == CONVROT_I8);
    if (import != (src_scale != nullptr)) return CONVROT_EINVAL;
    const uint32_t rot = (uint32_t)out->flags;
    if (!valid_rotation(rot, block)) return CONVROT_EINVAL;   // SwiGLU pairs: their own entry
    if (!aligned16(W) || !aligned16(out->codes) || !aligned16(out->scale) ||
        (src_scale && !aligned16(src_scale)))
        return CONVROT_EALIGN;
    const size_t need = convrot_prepare_workspace_bytes(N, K, block, w_dtype, layout);
    if (need > 0 && (!ws || ws_bytes < need)) return CONVROT_EWORKSPACE;
    if (ws && !aligned16(ws)) return CONVROT_EALIGN;

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    if (import) {
        e = convrot::launch_tile_codes(static_cast<const int8_t *>(W),
                                       layout == CONVROT_IN_MAJOR, out->codes, N, K, s);
        if (e == hipSuccess)
            e = hipMemcpyAsync(out->scale, src_scale, (size_t)N * 4u, hipMemcpyDeviceToDevice, s);
    } else {
        const convrot::InType in =
            (w_dtype == CONVROT_F32) ? convrot::InType::F32 : convrot::InType::BF16;
        const void *rows = W;
        if (layout == CONVROT_IN_MAJOR) {
            e = convrot::launch_transpose(W, ws, K, N, w_dtype == CONVROT_F32 ? 4 : 2, s);
            rows = ws;
        }
        if (e == hipSuccess)
            e = convrot::launch_rotquant(rows, in, N, K, K, block, rot != 0,
                                         inv_sqrt_block(block), out->codes, out->scale, s);
    }
    rc = hip_status(e);
    if (rc != CONVROT_OK) return rc;
    out->magic = CONVROT_WEIGHTS_MAGIC;
    out->version = CONVROT_WEIGHTS_VERSION;
    out->N = N;
    out->K = K;
    out->block = block;
    out->flags = (int32_t)rot;
    return CONVROT_OK;
}

int convrot_linear_prepare_weights(const void *W, int w_dtype, int layout,
                                   const float *src_scale, int64_t N, int64_t K, int block,
                                   convrot_weights *out, void *ws, size_t ws_bytes, void *stream)
{
    const int rc = prepare_weights_impl(W, w_dtype, layout, src_scale, N, K, block, out, ws,
                                        ws_bytes, stream);
    log_call("convrot_linear_prepare_weights", 0, N, K, rc);
    return rc;
}

// The rank a low-rank pair is stored with: r rounded up to a multiple of 128
// (a multiple of 64, as the checkpoint loader pads ranks, and the
// contraction's K granularity), or of 256 for b = 256 so that whole blocks
// tile the rank.
static int64_t lowrank_rank(int64_t r, int block)
{
    const int64_t m = block == 256 ? 256 : 128;
    return (r + m - 1) / m * m;
}

static bool lowrank_prep_args(int64_t r, int64_t K, int64_t N, int block, int w_dtype)
{
    // r is bounded before it is rounded up, so the rounding cannot overflow
    if (r <= 0 || r > kMaxK || !valid_block(block) ||
        (w_dtype != CONVROT_F32 && w_dtype != CONVROT_BF16))
        return false;
    const int64_t rp = lowrank_rank(r, block);
    return check_linear_shape(rp, K, block) == CONVROT_OK &&
           check_linear_shape(N, rp, block) == CONVROT_OK;
}

int64_t lowrank_convrot_padded_rank(int64_t r, int block)
{
    if (r <= 0 || r > kMaxK || !valid_block(block)) return 0;
    return lowrank_rank(r, block);
}

size_t lowrank_convrot_prepare_workspace_bytes(int64_t r, int64_t K, int64_t N,
                                                          int block, int w_dtype)
{
    if (!lowrank_prep_args(r, K, N, block, w_dtype)) return 0;
    const int64_t rp = lowrank_rank(r, block);
    if (rp == r) return 0;
    const size_t es = w_dtype == CONVROT_F32 ? 4u : 2u;
    return round_up((size_t)rp * (size_t)K * es, kAlign) + round_up((size_t)N * (size_t)rp * es, kAlign);
}

static int lowrank_prepare_impl(const void *A, const void *B, int w_dtype, int64_t r, int64_t K,
                                int64_t N, int block, convrot_weights *outA,
                                convrot_weights *outB, void *ws, size_t ws_bytes, void *stream)
{
    if (!A || !B || !outA || !outB || !outA->codes || !outA->scale || !outB->codes ||
        !outB->scale)
        return CONVROT_EINVAL;
    if (w_dtype != CONVROT_F32 && w_dtype != CONVROT_BF16) return CONVROT_EUNSUPPORTED;
    if (r <= 0 || K <= 0 || N <= 0 || !valid_block(block) || K % block != 0) return CONVROT_EINVAL;
    if (outA->flags != outB->flags || !valid_rotation((uint32_t)outA->flags, block))
        return CONVROT_EINVAL;
    if (!lowrank_prep_args(r, K, N, block, w_dtype)) return CONVROT_EUNSUPPORTED;
    if (!aligned16(A) || !aligned16(B) || (ws && !aligned16(ws))) return CONVROT_EALIGN;
    const int64_t rp = lowrank_rank(r, block);
    const size_t need = lowrank_convrot_prepare_workspace_bytes(r, K, N, block, w_dtype);
    if (need > 0 && (!ws || ws_bytes < need)) return CONVROT_EWORKSPACE;
    const int es = w_dtype == CONVROT_F32 ? 4 : 2;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const void *Ap = A, *Bp = B;
    if (rp != r) {
        // A gains zero rows r .. rp-1, B zero columns r .. rp-1: B' A' = B A,
        // and the zero blocks of A' and the zero columns of B' rotate to zero
        Carve c(ws);
        void *a = c.take((size_t)rp * (size_t)K * es);
        void *b = c.take((size_t)N * (size_t)rp * es);
        hipError_t e = convrot::launch_pad_copy(A, r, K, a, rp, K, es, s);
        if (e == hipSuccess) e = convrot::launch_pad_copy(B, N, r, b, N, rp, es, s);
        const int rc = hip_status(e);
        if (rc != CONVROT_OK) return rc;
        Ap = a;
        Bp = b;
    }
    // the float copies are consumed in stream order, so the workspace may be
    // reused once the stream has passed this call
    int rc = prepare_weights_impl(Ap, w_dtype, CONVROT_OUT_MAJOR, nullptr, rp, K, block, outA,
                                  nullptr, 0, stream);
    if (rc == CONVROT_OK)
        rc = prepare_weights_impl(Bp, w_dtype, CONVROT_OUT_MAJOR, nullptr, N, rp, block, outB,
                                  nullptr, 0, stream);
    return rc;
}

int lowrank_convrot_prepare_weights(const void *A, const void *B, int w_dtype,
                                               int64_t r, int64_t K, int64_t N, int block,
                                               convrot_weights *outA, convrot_weights *outB,
                                               void *ws, size_t ws_bytes, void *stream)
{
    const int rc = lowrank_prepare_impl(A, B, w_dtype, r, K, N, block, outA, outB, ws, ws_bytes,
                                        stream);
    log_call("lowrank_convrot_prepare_weights", r, N, K, rc);
    return rc;
}

static int linear_forward_impl(const void *X, int64_t M, const convrot_weights *W,
                           const float *bias, void *Y, int y_dtype, void *ws, size_t ws_bytes,
                           void *stream)
{
    int rc = check_weights(W);
    if (rc != CONVROT_OK) return rc;
    if ((rc = check_rows(M, W->K)) != CONVROT_OK) return rc;
    if ((rc = check_out_dtype(y_dtype)) != CONVROT_OK) return rc;
    if (M == 0) return CONVROT_OK;
    if (!X || !Y) return CONVROT_EINVAL;
    if (!aligned16(X) || !aligned16(Y) || (bias && !aligned16(bias)) || (ws && !aligned16(ws)))
        return CONVROT_EALIGN;
    const size_t need = convrot_linear_workspace_bytes(M, W->K, W->N, W->block);
    if (!ws || ws_bytes < need) return CONVROT_EWORKSPACE;

    // code regions are K-tiled with padded rows: the last 16-row block spans
    // padded_rows(M) * K bytes, not M * K
    Carve c(ws);
    int8_t *qx = static_cast<int8_t *>(c.take(codes_bytes(M, W->K)));
    float *sx = static_cast<float *>(c.take((size_t)M * 4u));
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = convrot::launch_rotquant(X, convrot::InType::BF16, M, W->K, W->K, W->block,
                                            is_regular(W),
                                            inv_sqrt_block(W->block), qx, sx, s);
    if (e == hipSuccess)
        e = convrot::launch_gemm_i8(qx, W->codes, sx, W->scale, bias, Y, out_kind(y_dtype), M,
                                    W->N, W->K, s);
    return hip_status(e);
}

int convrot_linear_forward(const void *X, int64_t M, const convrot_weights *W,
                           const float *bias, void *Y, int y_dtype, void *ws, size_t ws_bytes,
                           void *stream)
{
    const int rc = linear_forward_impl(X, M, W, bias, Y, y_dtype, ws, ws_bytes, stream);
    log_call("convrot_linear_forward", M, W ? W->N : 0, W ? W->K : 0, rc);
    return rc;
}

// ---------------------------------------------------------------------------
// SwiGLU MLP (MiniMax-H3-Rung-Omega README, "Technical Architecture
// Overview", Floor 1: SwiGLU, ConvRot64 and the rowwise INT8 quantise in front
// of MLP.fc2).  fc1 is one linear with 2F outputs, gate then up; its weight
// rows are stored interleaved (swiglu_src_row) so that the fc1 epilogue holds
// each gate next to its up value and writes g = bf16(silu(gate) * up) alone.
// ---------------------------------------------------------------------------

size_t convrot_swiglu_prepare_workspace_bytes(int64_t F, int64_t K, int block, int w_dtype)
{
    if (F <= 0 || F >= kI32Bound || F % 16 != 0 ||
        check_linear_shape(2 * F, K, block) != CONVROT_OK)
        return 0;
    const size_t es = w_dtype == CONVROT_F32 ? 4u : w_dtype == CONVROT_BF16 ? 2u :
                      w_dtype == CONVROT_I8 ? 1u : 0u;
    if (es == 0) return 0;
    return round_up((size_t)2 * F * (size_t)K * es, kAlign) +
           (w_dtype == CONVROT_I8 ? round_up((size_t)8 * F, kAlign) : 0);
}

static int swiglu_prepare_impl(const void *W, int w_dtype, const float *src_scale, int64_t F,
                               int64_t K, int block, convrot_weights *out, void *ws,
                               size_t ws_bytes, void *stream)
{
    if (!W || !out || !out->codes || !out->scale || F <= 0) return CONVROT_EINVAL;
    if (F >= kI32Bound || F % 16 != 0) return CONVROT_EUNSUPPORTED;
    int rc = check_linear_shape(2 * F, K, block);
    if (rc != CONVROT_OK) return rc;
    if (w_dtype != CONVROT_F32 && w_dtype != CONVROT_BF16 && w_dtype != CONVROT_I8)
        return CONVROT_EUNSUPPORTED;
    const bool import = w_dtype == CONVROT_I8;
    if (import != (src_scale != nullptr)) return CONVROT_EINVAL;
    if (!valid_rotation((uint32_t)out->flags, block)) return CONVROT_EINVAL;
    if (!aligned16(W) || !aligned16(out->codes) || !aligned16(out->scale) ||
        (src_scale && !aligned16(src_scale)) || (ws && !aligned16(ws)))
        return CONVROT_EALIGN;
    const size_t need = convrot_swiglu_prepare_workspace_bytes(F, K, block, w_dtype);
    if (!ws || ws_bytes < need) return CONVROT_EWORKSPACE;
    const int es = w_dtype == CONVROT_F32 ? 4 : w_dtype == CONVROT_BF16 ? 2 : 1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Carve c(ws);
    void *rows = c.take((size_t)2 * F * (size_t)K * es);
    hipError_t e = convrot::launch_swiglu_interleave(W, rows, F, K, es, s);
    const float *scales = nullptr;
    if (import && e == hipSuccess) {
        // the per-output scales follow their rows (rows of one 4-byte scale)
        void *sc = c.take((size_t)8 * F);
        e = convrot::launch_swiglu_interleave(src_scale, sc, F, 1, 4, s);
        scales = static_cast<const float *>(sc);
    }
    rc = hip_status(e);
    if (rc != CONVROT_OK) return rc;
    rc = prepare_weights_impl(rows, w_dtype, CONVROT_OUT_MAJOR, scales, 2 * F, K, block, out,
                              nullptr, 0, stream);
    if (rc == CONVROT_OK) out->flags |= (int32_t)CONVROT_SWIGLU_PAIRS;
    return rc;
}

int convrot_swiglu_prepare_weights(const void *W, int w_dtype, const float *src_scale, int64_t F,
                                   int64_t K, int block, convrot_weights *out, void *ws,
                                   size_t ws_bytes, void *stream)
{
    const int rc = swiglu_prepare_impl(W, w_dtype, src_scale, F, K, block, out, ws, ws_bytes,
                                       stream);
    log_call("convrot_swiglu_prepare_weights", 0, 2 * F, K, rc);
    return rc;
}

size_t convrot_swiglu_mlp_workspace_bytes(int64_t M, int64_t K, int64_t F, int64_t N,
                                          int block_up, int block_down)
{
    if (F <= 0 || F >= kI32Bound || F % 16 != 0 ||
        check_linear_shape(2 * F, K, block_up) != CONVROT_OK ||
        check_linear_shape(N, F, block_down) != CONVROT_OK || check_rows(M, K) != CONVROT_OK ||
        check_rows(M, F) != CONVROT_OK)
        return 0;
    return codes_bytes(M, K) + scales_bytes(M) + round_up((size_t)M * (size_t)F * 2u, kAlign) +
           codes_bytes(M, F) + scales_bytes(M);
}

static int swiglu_forward_impl(const void *X, int64_t M, const convrot_weights *W_gu,
                               const float *bias_gu, const convrot_weights *W_down,
                               const float *bias_down, void *Y, int y_dtype, void *ws,
                               size_t ws_bytes, void *stream)
{
    int rc = check_weights(W_gu, true);
    if (rc != CONVROT_OK) return rc;
    if ((rc = check_weights(W_down)) != CONVROT_OK) return rc;
    if (W_gu->N != 2 * W_down->K || rotation_of(W_gu) != rotation_of(W_down))
        return CONVROT_ELAYOUT;
    const int64_t F = W_down->K;
    if ((rc = check_rows(M, W_gu->K)) != CONVROT_OK) return rc;
    if ((rc = check_rows(M, F)) != CONVROT_OK) return rc;
    if ((rc = check_out_dtype(y_dtype)) != CONVROT_OK) return rc;
    if (M == 0) return CONVROT_OK;
    if (!X || !Y) return CONVROT_EINVAL;
    if (!aligned16(X) || !aligned16(Y) || (bias_gu && !aligned16(bias_gu)) ||
        (bias_down && !aligned16(bias_down)) || (ws && !aligned16(ws)))
        return CONVROT_EALIGN;
    const size_t need = convrot_swiglu_mlp_workspace_bytes(M, W_gu->K, F, W_down->N,
                                                           W_gu->block, W_down->block);
    if (!ws || ws_bytes < need) return CONVROT_EWORKSPACE;

    Carve c(ws);
    int8_t *qx = static_cast<int8_t *>(c.take(codes_bytes(M, W_gu->K)));
    float *sx = static_cast<float *>(c.take((size_t)M * 4u));
    void *g = c.take((size_t)M * (size_t)F * 2u);
    int8_t *qg = static_cast<int8_t *>(c.take(codes_bytes(M, F)));
    float *sg = static_cast<float *>(c.take((size_t)M * 4u));
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = convrot::launch_rotquant(X, convrot::InType::BF16, M, W_gu->K, W_gu->K,
                                            W_gu->block, is_regular(W_gu),
                                            inv_sqrt_block(W_gu->block), qx, sx, s);
    // fc1 with the SwiGLU epilogue: g [M, F] is the only intermediate written
    if (e == hipSuccess)
        e = convrot::launch_gemm_i8(qx, W_gu->codes, sx, W_gu->scale, bias_gu, g,
                                    convrot::OutKind::SWIGLU_BF16, M, W_gu->N, W_gu->K, s);
    if (e == hipSuccess)
        e = convrot::launch_rotquant(g, convrot::InType::BF16, M, F, F, W_down->block,
                                     is_regular(W_down), inv_sqrt_block(W_down->block), qg, sg, s);
    if (e == hipSuccess)
        e = convrot::launch_gemm_i8(qg, W_down->codes, sg, W_down->scale, bias_down, Y,
                                    out_kind(y_dtype), M, W_down->N, F, s);
    return hip_status(e);
}

int convrot_swiglu_mlp_forward(const void *X, int64_t M, const convrot_weights *W_gu,
                               const float *bias_gu, const convrot_weights *W_down,
                               const float *bias_down, void *Y, int y_dtype, void *ws,
                               size_t ws_bytes, void *stream)
{
    const int rc = swiglu_forward_impl(X, M, W_gu, bias_gu, W_down, bias_down, Y, y_dtype, ws,
                                       ws_bytes, stream);
    log_call("convrot_swiglu_mlp_forward", M, W_down ? W_down->N : 0, W_gu ? W_gu->K : 0, rc);
    return rc;
}

int convrot_swiglu_bf16(const uint16_t *gu, int64_t M, int64_t F, uint16_t *g, void *stream)
{
    if (M < 0 || F <= 0) return CONVROT_EINVAL;
    if (F % 8 != 0 || M >= kI32Bound || F >= kI32Bound) return CONVROT_EUNSUPPORTED;
    if (M == 0) return CONVROT_OK;
    if (!gu || !g) return CONVROT_EINVAL;
    if (!aligned16(gu) || !aligned16(g)) return CONVROT_EALIGN;
    return hip_status(convrot::launch_swiglu_bf16(gu, M, F, g, static_cast<hipStream_t>(stream)));
}

int convrot_silu_f32(const uint16_t *a, int64_t n, float *s_out, void *stream)
{
    if (n < 0) return CONVROT_EINVAL;
    if (n == 0) return CONVROT_OK;
    if (!a || !s_out) return CONVROT_EINVAL;
    return hip_status(convrot::launch_silu_f32(a, n, s_out, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
// The allocation-free linear forward: the workspace of convrot_linear_forward
// (the rotated activations' K-tiled codes and row scales) lives in a
// file-scope device array, one copy per device, held until the process ends.
// The array's name is a host-side stand-in in host code: its device address
// is looked up once per device (hipGetSymbolAddress, with that device
// current) and only that address is passed to the kernels.
// ---------------------------------------------------------------------------
static __device__ __align__(256) int8_t scratch[CONVROT_NOALLOC_SCRATCH_BYTES];

static int scratch_ptr(void **out)
{
    static std::atomic<void *> cached[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= 64) return CONVROT_EUNSUPPORTED;
    void *p = cached[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e);
        if (!p || !aligned16(p)) return hip_status(hipErrorInvalidSymbol);
        cached[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return CONVROT_OK;
}

int convrot_linear_forward_noalloc(const void *X, int64_t M, const convrot_weights *W,
                                   const float *bias, void *Y, int y_dtype, void *stream)
{
    int rc = check_weights(W);
    if (rc == CONVROT_OK) rc = check_rows(M, W->K);
    if (rc == CONVROT_OK &&
        convrot_linear_workspace_bytes(M, W->K, W->N, W->block) > CONVROT_NOALLOC_SCRATCH_BYTES)
        rc = CONVROT_EWORKSPACE;   // beyond the static scratch: the caller must use a workspace
    void *ws = nullptr;
    if (rc == CONVROT_OK && M > 0) rc = scratch_ptr(&ws);
    if (rc == CONVROT_OK)
        rc = linear_forward_impl(X, M, W, bias, Y, y_dtype, ws, CONVROT_NOALLOC_SCRATCH_BYTES,
                                 stream);
    log_call("convrot_linear_forward_noalloc", M, W ? W->N : 0, W ? W->K : 0, rc);
    return rc;
}

static int lowrank_forward_impl(const void *X, int64_t M, const convrot_weights *A,
                            const convrot_weights *B, const float *bias, void *Y, int y_dtype,
                            void *ws, size_t ws_bytes, void *stream)
{
    int rc = check_weights(A);
    if (rc != CONVROT_OK) return rc;
    if ((rc = check_weights(B)) != CONVROT_OK) return rc;
    if (A->N != B->K || A->block != B->block || A->flags != B->flags) return CONVROT_ELAYOUT;
    if ((rc = check_rows(M, A->K)) != CONVROT_OK) return rc;
    if ((rc = check_rows(M, A->N)) != CONVROT_OK) return rc;
    if ((rc = check_out_dtype(y_dtype)) != CONVROT_OK) return rc;
    if (M == 0) return CONVROT_OK;
    if (!X || !Y) return CONVROT_EINVAL;
    if (!aligned16(X) || !aligned16(Y) || (bias && !aligned16(bias)) || (ws && !aligned16(ws)))
        return CONVROT_EALIGN;
    const int64_t r = A->N;
    const size_t need = lowrank_convrot_workspace_bytes(M, A->K, r, B->N, A->block);
    if (!ws || ws_bytes < need) return CONVROT_EWORKSPACE;

    Carve c(ws);
    int8_t *qx = static_cast<int8_t *>(c.take(codes_bytes(M, A->K)));
    float *sx = static_cast<float *>(c.take((size_t)M * 4u));
    void *h = c.take((size_t)M * (size_t)r * 2u);
    int8_t *qh = static_cast<int8_t *>(c.take(codes_bytes(M, r)));
    float *sh = static_cast<float *>(c.take((size_t)M * 4u));
    hipStream_t s = static_cast<hipStream_t>(stream);
    const float isb = inv_sqrt_block(A->block);
    hipError_t e = convrot::launch_rotquant(X, convrot::InType::BF16, M, A->K, A->K, A->block,
                                            is_regular(A), isb, qx, sx, s);
    if (!is_regular(A) && convrot::lowrank_f1_fusable(r, A->block)) {
        // a row of H fits one workgroup tile: factor 1 rotates and
        // requantises it in its epilogue, H never reaches memory
        if (e == hipSuccess)
            e = convrot::launch_lowrank_f1(qx, A->codes, sx, A->scale, qh, sh, M, r, A->K,
                                           A->block, isb, s);
    } else {
        if (e == hipSuccess)
            e = convrot::launch_gemm_i8(qx, A->codes, sx, A->scale, nullptr, h,
                                        convrot::OutKind::BF16, M, r, A->K, s);
        if (e == hipSuccess)
            e = convrot::launch_rotquant(h, convrot::InType::BF16, M, r, r, B->block,
                                         is_regular(B), isb, qh, sh, s);
    }
    if (e == hipSuccess)
        e = convrot::launch_gemm_i8(qh, B->codes, sh, B->scale, bias, Y, out_kind(y_dtype), M,
                                    B->N, r, s);
    return hip_status(e);
}

int lowrank_convrot_forward(const void *X, int64_t M, const convrot_weights *A,
                            const convrot_weights *B, const float *bias, void *Y, int y_dtype,
                            void *ws, size_t ws_bytes, void *stream)
{
    const int rc = lowrank_forward_impl(X, M, A, B, bias, Y, y_dtype, ws, ws_bytes, stream);
    log_call("lowrank_convrot_forward", M, B ? B->N : 0, A ? A->K : 0, rc);
    return rc;
}

static int mlp_forward_impl(const void *X, int64_t M, const convrot_weights *W_up,
                        const float *bias_up, const convrot_weights *W_down,
                        const float *bias_down, void *Y, int y_dtype, void *ws, size_t ws_bytes,
                        void *stream)
{
    int rc = check_weights(W_up);
    if (rc != CONVROT_OK) return rc;
    if ((rc = check_weights(W_down)) != CONVROT_OK) return rc;
    if (W_up->N != W_down->K || W_up->block != W_down->block || W_up->flags != W_down->flags)
        return CONVROT_ELAYOUT;
    if ((rc = check_rows(M, W_up->K)) != CONVROT_OK) return rc;
    if ((rc = check_rows(M, W_up->N)) != CONVROT_OK) return rc;
    if ((rc = check_out_dtype(y_dtype)) != CONVROT_OK) return rc;
    if (M == 0) return CONVROT_OK;
    if (!X || !Y) return CONVROT_EINVAL;
    if (!aligned16(X) || !aligned16(Y) || (bias_up && !aligned16(bias_up)) ||
        (bias_down && !aligned16(bias_down)) || (ws && !aligned16(ws)))
        return CONVROT_EALIGN;
    const int64_t F = W_up->N;
    const size_t need = convrot_mlp_workspace_bytes(M, W_up->K, F, W_down->N, W_up->block);
    if (!ws || ws_bytes < need) return CONVROT_EWORKSPACE;

    Carve c(ws);
    int8_t *qx = static_cast<int8_t *>(c.take(codes_bytes(M, W_up->K)));
    float *sx = static_cast<float *>(c.take((size_t)M * 4u));
    void *g = c.take((size_t)M * (size_t)F * 2u);
    int8_t *qg = static_cast<int8_t *>(c.take(codes_bytes(M, F)));
    float *sg = static_cast<float *>(c.take((size_t)M * 4u));
    hipStream_t s = static_cast<hipStream_t>(stream);
    const float isb = inv_sqrt_block(W_up->block);
    // GELU goes where it costs least: for the long rows that the two-rows-
    // per-wave rotquant kernel serves, into that kernel's loads (the up
    // projection writes u with the plain epilogue and g is never stored);
    // otherwise into the up projection's epilogue.  Both give bf16(GELU(u)).
    const bool gelu_on_load = convrot::rotquant_fuses_gelu(F);
    hipError_t e = convrot::launch_rotquant(X, convrot::InType::BF16, M, W_up->K, W_up->K,
                                            W_up->block, is_regular(W_up), isb, qx, sx, s);
    if (e == hipSuccess)
        e = convrot::launch_gemm_i8(qx, W_up->codes, sx, W_up->scale, bias_up, g,
                                    gelu_on_load ? convrot::OutKind::BF16
                                                 : convrot::OutKind::GELU_BF16,
                                    M, F, W_up->K, s);
    if (e == hipSuccess && gelu_on_load) {
        const uint16_t *table = nullptr;
        e = convrot::launch_gelu_table(&table, s);
        if (e == hipSuccess)
            e = convrot::launch_rotquant_gelu(g, M, F, F, W_down->block, is_regular(W_down), isb,
                                              table, qg, sg, s);
    } else if (e == hipSuccess) {
        e = convrot::launch_rotquant(g, convrot::InType::BF16, M, F, F, W_down->block,
                                     is_regular(W_down), isb, qg, sg, s);
    }
    if (e == hipSuccess)
        e = convrot::launch_gemm_i8(qg, W_down->codes, sg, W_down->scale, bias_down, Y,
                                    out_kind(y_dtype), M, W_down->N, F, s);
    return hip_status(e);
}

int convrot_mlp_forward(const void *X, int64_t M, const convrot_weights *W_up,
                        const float *bias_up, const convrot_weights *W_down,
                        const float *bias_down, void *Y, int y_dtype, void *ws, size_t ws_bytes,
                        void *stream)
{
    const int rc = mlp_forward_impl(X, M, W_up, bias_up, W_down, bias_down, Y, y_dtype, ws,
                                    ws_bytes, stream);
    log_call("convrot_mlp_forward", M, W_down ? W_down->N : 0, W_up ? W_up->K : 0, rc);
    return rc;
}

size_t lowrank_bf16_workspace_bytes(int64_t M, int64_t r)
{
    if (M < 0 || r <= 0 || r > kMaxK || M >= kI32Bound || M * 2 * r >= kI32Bound) return 0;
    return round_up((size_t)M * (size_t)r * 2u, kAlign);
}

int lowrank_bf16_forward(const void *X, int64_t M, int64_t K, const void *A, int64_t r,
                         const void *B, int64_t N, const float *bias, void *Y, void *ws,
                         size_t ws_bytes, void *stream)
{
    if (M < 0 || K <= 0 || r <= 0 || N <= 0) return CONVROT_EINVAL;
    if (K % 64 != 0 || r % 64 != 0 || N % 16 != 0 || K > kMaxK || r > kMaxK)
        return CONVROT_EUNSUPPORTED;
    if (M >= kI32Bound || N >= kI32Bound || M * 2 * K >= kI32Bound || M * 2 * r >= kI32Bound ||
        N * 2 * K >= kI32Bound || N * 2 * r >= kI32Bound)
        return CONVROT_EUNSUPPORTED;
    if (M == 0) return CONVROT_OK;
    if (!X || !A || !B || !Y) return CONVROT_EINVAL;
    if (!aligned16(X) || !aligned16(A) || !aligned16(B) || !aligned16(Y) ||
        (bias && !aligned16(bias)) || (ws && !aligned16(ws)))
        return CONVROT_EALIGN;
    if (!ws || ws_bytes < lowrank_bf16_workspace_bytes(M, r)) return CONVROT_EWORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // the operands are bf16: the contraction counts bytes along K
    hipError_t e = convrot::launch_gemm_i8(static_cast<const int8_t *>(X),
                                           static_cast<const int8_t *>(A), nullptr, nullptr,
                                           nullptr, ws, convrot::OutKind::BF16_MM, M, r, 2 * K, s);
    if (e == hipSuccess)
        e = convrot::launch_gemm_i8(static_cast<const int8_t *>(ws),
                                    static_cast<const int8_t *>(B), nullptr, nullptr, bias, Y,
                                    convrot::OutKind::BF16_MM, M, N, 2 * r, s);
    return hip_status(e);
}

int convrot_rotate_quantize(const void *X, int x_dtype, int64_t M, int64_t K, int block,
                            uint32_t flags, int8_t *q, float *s_out, void *stream)
{
    if (M < 0 || K <= 0 || !valid_block(block) || K % block != 0) return CONVROT_EINVAL;
    if ((flags & ~(CONVROT_ROT_REGULAR | CONVROT_FLAG_GELU)) != 0) return CONVROT_EUNSUPPORTED;
    const uint32_t rot = flags & CONVROT_ROT_REGULAR;
    const bool gelu = (flags & CONVROT_FLAG_GELU) != 0;
    if (!valid_rotation(rot, block)) return CONVROT_EINVAL;
    if (x_dtype != CONVROT_F32 && x_dtype != CONVROT_BF16) return CONVROT_EUNSUPPORTED;
    if (gelu && (x_dtype != CONVROT_BF16 || !convrot::rotquant_fuses_gelu(K)))
        return CONVROT_EUNSUPPORTED;
    if (K > kMaxK || check_rows(M, K) != CONVROT_OK) return CONVROT_EUNSUPPORTED;
    if (M == 0) return CONVROT_OK;
    if (!X || !q || !s_out) return CONVROT_EINVAL;
    if (!aligned16(X) || !aligned16(q) || !aligned16(s_out)) return CONVROT_EALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (gelu) {
        const uint16_t *table = nullptr;
        hipError_t e = convrot::launch_gelu_table(&table, s);
        if (e == hipSuccess)
            e = convrot::launch_rotquant_gelu(X, M, K, K, block, rot != 0, inv_sqrt_block(block),
                                              table, q, s_out, s);
        return hip_status(e);
    }
    const convrot::InType in = x_dtype == CONVROT_F32 ? convrot::InType::F32 : convrot::InType::BF16;
    return hip_status(convrot::launch_rotquant(X, in, M, K, K, block, rot != 0,
                                               inv_sqrt_block(block), q, s_out, s));
}

int convrot_gemm_i32(const int8_t *q_x, int64_t M, const convrot_weights *W, int32_t *acc,
                     void *stream)
{
    // any prepared weight, SwiGLU pairs included (columns in packed row order)
    int rc = check_weights(W, W && is_swiglu_pairs(W));
    if (rc != CONVROT_OK) return rc;
    if ((rc = check_rows(M, W->K)) != CONVROT_OK) return rc;
    if (M == 0) return CONVROT_OK;
    if (!q_x || !acc) return CONVROT_EINVAL;
    if (!aligned16(q_x) || !aligned16(acc)) return CONVROT_EALIGN;
    return hip_status(convrot::launch_gemm_i8(q_x, W->codes, nullptr, nullptr, nullptr, acc,
                                              convrot::OutKind::I32, M, W->N, W->K,
                                              static_cast<hipStream_t>(stream)));
}

int convrot_gemm_dequant(const int8_t *q_x, const float *s_x, int64_t M,
                         const convrot_weights *W, const float *bias, void *Y, int y_dtype,
                         uint32_t flags, void *stream)
{
    if ((flags & ~(CONVROT_FLAG_GELU | CONVROT_FLAG_SWIGLU)) != 0 ||
        flags == (CONVROT_FLAG_GELU | CONVROT_FLAG_SWIGLU))
        return CONVROT_EUNSUPPORTED;
    const bool gelu = (flags & CONVROT_FLAG_GELU) != 0;
    const bool swiglu = (flags & CONVROT_FLAG_SWIGLU) != 0;
    int rc = check_weights(W, swiglu);
    if (rc != CONVROT_OK) return rc;
    if ((rc = check_rows(M, W->K)) != CONVROT_OK) return rc;
    if ((rc = check_out_dtype(y_dtype)) != CONVROT_OK) return rc;
    if ((gelu || swiglu) && y_dtype != CONVROT_BF16) return CONVROT_EUNSUPPORTED;
    if (M == 0) return CONVROT_OK;
    if (!q_x || !s_x || !Y) return CONVROT_EINVAL;
    if (!aligned16(q_x) || !aligned16(s_x) || !aligned16(Y) || (bias && !aligned16(bias)))
        return CONVROT_EALIGN;
    return hip_status(convrot::launch_gemm_i8(
        q_x, W->codes, s_x, W->scale, bias, Y,
        swiglu ? convrot::OutKind::SWIGLU_BF16
               : gelu ? convrot::OutKind::GELU_BF16 : out_kind(y_dtype),
        M, W->N, W->K, static_cast<hipStream_t>(stream)));
}

int convrot_lowrank_factor1(const int8_t *q_x, const float *s_x, int64_t M,
                            const convrot_weights *A, int8_t *q_h, float *s_h, void *stream)
{
    int rc = check_weights(A);
    if (rc != CONVROT_OK) return rc;
    if ((rc = check_rows(M, A->K)) != CONVROT_OK) return rc;
    if ((rc = check_rows(M, A->N)) != CONVROT_OK) return rc;
    if (is_regular(A) || !convrot::lowrank_f1_fusable(A->N, A->block))
        return CONVROT_EUNSUPPORTED;
    if (M == 0) return CONVROT_OK;
    if (!q_x || !s_x || !q_h || !s_h) return CONVROT_EINVAL;
    if (!aligned16(q_x) || !aligned16(s_x) || !aligned16(q_h) || !aligned16(s_h))
        return CONVROT_EALIGN;
    return hip_status(convrot::launch_lowrank_f1(q_x, A->codes, s_x, A->scale, q_h, s_h, M,
                                                 A->N, A->K, A->block,
                                                 inv_sqrt_block(A->block),
                                                 static_cast<hipStream_t>(stream)));
}

int convrot_gelu_bf16(const uint16_t *u, int64_t n, uint16_t *g, void *stream)
{
    if (n < 0) return CONVROT_EINVAL;
    if (n == 0) return CONVROT_OK;
    if (!u || !g) return CONVROT_EINVAL;
    return hip_status(convrot::launch_gelu_bf16(u, g, n, static_cast<hipStream_t>(stream)));
}

int convrot_probe_mfma_i8(int64_t iters, const void *seed, void *sink, int64_t *ops,
                          void *stream)
{
    if (iters < 1 || iters > (int64_t(1) << 24) || !seed || !sink || !ops)
        return CONVROT_EINVAL;
    if (!aligned16(seed) || !aligned16(sink)) return CONVROT_EALIGN;
    *ops = convrot::probe_mfma_i8_ops(iters);
    return hip_status(convrot::launch_probe_mfma_i8(iters, static_cast<const int *>(seed),
                                                    static_cast<int *>(sink),
                                                    static_cast<hipStream_t>(stream)));
}

int convrot_probe_stream(const void *src, void *dst, int64_t n16, int mode, void *stream)
{
    if (n16 < 0 || mode < 0 || mode > 2) return CONVROT_EINVAL;
    if (n16 == 0) return CONVROT_OK;
    if ((!src && mode != 2) || !dst) return CONVROT_EINVAL;
    if ((src && !aligned16(src)) || !aligned16(dst)) return CONVROT_EALIGN;
    return hip_status(convrot::launch_probe_stream(src, dst, n16, mode,
                                                   static_cast<hipStream_t>(stream)));
}

} // extern "C"
