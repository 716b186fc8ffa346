/*
 * convrot.h -- C ABI of libconvrot.so: the ConvRot W8A8 INT8 linear layer on
 * AMD Instinct MI355X (gfx950).
 *
 * The method (what every entry point computes):
 *   - Linear layers of the INT8 package are W8A8: INT8 activations times INT8
 *     weights, placed behind a block-diagonal Hadamard rotation (lehuy.net
 *     article on HyperFlow H3 Flash, "Cach nen hoat dong", second bullet).
 *   - The activation row is rotated and then quantised row-wise to INT8 right
 *     in front of the projection (MiniMax-H3-Rung-Omega README, "Technical
 *     Architecture Overview", Floor 1, where rotation and rowwise quantise are
 *     fused ahead of MLP.fc2).
 *   - Weights are stored pre-rotated as INT8 codes with one F32 scale per
 *     output channel, source layout [output, input], and an exact transpose
 *     [input, output] exists (PulpCut MiniMax H3 INT8 ConvRot input-major
 *     README, "Input-major checkpoint").  Dequantising and undoing the
 *     rotation recovers the weights (HyperFlow H3 Flash MLX card, "Where the
 *     weights come from"), so the stored codes approximate W . R^T with R
 *     orthogonal.
 *   - Low-rank factorised linears sit beside the INT8 ones, with ranks padded
 *     to a multiple of 64 (HyperFlow H3 Flash card, "Choose a Weight Format"
 *     and "Standalone Transformer (AutoModel)").
 *
 * Arithmetic fixed by this library (readings where the pages are silent):
 *   R = blockdiag(H_b) / sqrt(b), H_b the Sylvester Hadamard in natural order
 *   (H_1 = [1], H_2k = [[H_k, H_k], [H_k, -H_k]]), b in {64, 128, 256}.
 *   Rotation: fp32 butterflies with strides h = 1, 2, 4, ..., b/2 in that
 *   order (bf16 inputs widen exactly).
 *   Row quantise: amax = max|v|; codes = rint(v * (127/amax)) in [-127, 127]
 *   (fp32, correctly rounded division, round half to even); scale =
 *   (amax/127) * fp32(1/sqrt(b)).  A zero row gives codes 0 and scale 0.
 *   Contraction: exact int32 acc = sum_k qx[m,k] * qw[n,k].
 *   Epilogue: y = ((float)acc * s_x[m]) * s_w[n], then y += bias[n]; no fused
 *   multiply-add; bf16 outputs round to nearest even.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     allocates nothing and keeps no per-call state.  It is re-entrant: calls
 *     on different streams may overlap if they use separate workspaces (the
 *     allocation-free forward below shares one scratch array per device and
 *     is the exception).  Its device state is fixed in size, one copy per
 *     device in the library's code object: two read-only tables, each written
 *     once per device by the first call of a path that reads it -- the
 *     65,536-entry bf16 GELU table (convrot_mlp_forward, CONVROT_FLAG_GELU,
 *     convrot_gelu_bf16) and the 65,536-entry fp32 silu table (the SwiGLU
 *     paths: convrot_swiglu_mlp_forward, CONVROT_FLAG_SWIGLU,
 *     convrot_swiglu_bf16, convrot_silu_f32) -- and the scratch array of
 *     convrot_linear_forward_noalloc.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls are asynchronous on that stream.  The host waits only once per
 *     device and table: the first call of a GELU or SwiGLU path that is not
 *     being recorded into a graph waits for its table fill, so that launches
 *     on any stream may read the table from then on.  Such a call recorded
 *     into a graph before that records the fill too (each replay rewrites the
 *     same values).
 *   - Float matrices (X, Y, weights, intermediates in bf16) are row-major and
 *     dense; bf16 tensors hold raw bfloat16 bits.  INT8 code matrices (the
 *     test hooks' q_x and q_h, prepared weight codes) use the K-tiled layout
 *     below.  Every pointer must be 16-byte aligned.
 *   - Arguments are validated before anything is launched.  A call that
 *     returns an error has launched nothing and written nothing.  Device
 *     faults surface at the caller's next synchronisation.
 *   - Non-finite inputs give unspecified (but memory-safe) results.
 *   - Shape limits: K % 128 == 0, N % 16 == 0, K <= 65536, Mp*K < 2^31 with
 *     Mp = M rounded up to a multiple of 16, N*K < 2^31 (EUNSUPPORTED
 *     otherwise).  M == 0 is a no-op returning OK.  The contraction consumes
 *     K in pairs of 64-byte K-tiles, hence K % 128.  A layer whose K is an
 *     odd multiple of 64 (b = 64) is served exactly by padding K with one
 *     zero block: zero columns of X and W rotate to zero blocks, change no
 *     row amax and add nothing to the INT32 sum.
 *
 * K-tiled INT8 layout of a code matrix with M rows of K codes (K % 64 == 0):
 * rows are padded to Mp (a multiple of 16) and the code (m, k) sits at byte
 *   ((m / 16) * (K / 64) + k / 64) * 1024 + (m % 16) * 64
 *     + (((k / 16) % 4) XOR ((m / 4) % 4)) * 16 + k % 16,
 * i.e. each block of 16 rows is K/64 consecutive 1 KiB tiles of 16 rows x 64
 * codes, with the four 16-byte chunks of a row permuted by its row index.  A
 * GEMM K-step of 16 rows is then one contiguous 1 KiB read that lands in LDS
 * in bank-conflict-free order.  The buffer holds Mp * K bytes; the padding
 * rows are never read into an output.
 */
#ifndef CONVROT_H
#define CONVROT_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define CONVROT_API __attribute__((visibility("default")))
#else
#define CONVROT_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ */
/* status codes, dtypes, layouts                                       */
/* ------------------------------------------------------------------ */

typedef enum convrot_status {
    CONVROT_OK = 0,
    CONVROT_EINVAL = -1,       /* null pointer, bad shape, K % b != 0, bad b */
    CONVROT_EALIGN = -2,       /* a pointer is not 16-byte aligned */
    CONVROT_EWORKSPACE = -3,   /* workspace NULL or smaller than the query */
    CONVROT_ELAYOUT = -4,      /* weight descriptor magic/version/shape mismatch */
    CONVROT_EUNSUPPORTED = -5, /* outside the shape limits, or dtype combination */
    CONVROT_EHIP = -6          /* a HIP launch failed; see convrot_last_hip_error */
} convrot_status;

typedef enum convrot_dtype {
    CONVROT_F32 = 0,
    CONVROT_BF16 = 1,
    CONVROT_I8 = 2,
    CONVROT_I32 = 3
} convrot_dtype;

typedef enum convrot_layout {
    CONVROT_OUT_MAJOR = 0,     /* W stored [N, K]: [output, input] */
    CONVROT_IN_MAJOR = 1       /* W stored [K, N]: [input, output] */
} convrot_layout;

#define CONVROT_WEIGHTS_MAGIC 0x38545243u /* "CRT8" little-endian */

/* Rotation kind, in convrot_weights.flags and in convrot_rotate_quantize's
 * flags.  0: the Sylvester blocks H_b (b in {64, 128, 256}).
 * CONVROT_ROT_REGULAR: the regular ("DC-balanced") orthogonal Hadamard
 * H_4 (x) ... (x) H_4 with H_4 = J - 2I (every row sums to 2), b in {64, 256}
 * (MiniMax-H3-Rung-Omega README, "Technical Architecture Overview", item 1:
 * H_256 = H_4^(x)4).  It is applied along the base-4 digits of the in-block
 * index, lowest first; a group (v0..v3) becomes S - 2 v_j with
 * S = (v0 + v1) + (v2 + v3) in fp32.  The scale folds 1/sqrt(b) either way. */
#define CONVROT_ROT_REGULAR 0x100u
/* Set by convrot_swiglu_prepare_weights (never by the caller): the 2F rows are
 * a SwiGLU fc1's gate and up channels, stored interleaved in 32-row blocks
 * (packed row p holds source row (p/32)*16 + p%32 for p%32 < 16, else
 * F + (p/32)*16 + p%32 - 16).  Only convrot_swiglu_mlp_forward, the
 * CONVROT_FLAG_SWIGLU hook and convrot_gemm_i32 accept such a weight; other
 * entry points return CONVROT_ELAYOUT. */
#define CONVROT_SWIGLU_PAIRS 0x200u
#define CONVROT_WEIGHTS_VERSION 2u

/* Prepared (pre-rotated, quantised, packed) weights of one linear layer.
 * A host struct holding caller-owned device pointers.  `codes` and `scale`
 * must be allocated by the caller before convrot_linear_prepare_weights
 * (sizes: convrot_weights_packed_bytes(N, K, block) and 4*N bytes); the
 * prepare call fills every other field.  The codes are stored K-tiled (N is a
 * multiple of 16, so there are no padding rows); the layout is tagged by
 * magic/version: forward calls reject a descriptor whose tag does not match
 * (CONVROT_ELAYOUT), the way a runtime validates a versioned layout marker
 * before building its pipeline (PulpCut input-major README, "Input-major
 * checkpoint"). */
typedef struct convrot_weights {
    uint32_t magic;            /* CONVROT_WEIGHTS_MAGIC once prepared */
    uint32_t version;          /* CONVROT_WEIGHTS_VERSION */
    int64_t N;                 /* output channels */
    int64_t K;                 /* input channels */
    int32_t block;             /* Hadamard block b the codes were rotated with */
    int32_t flags;             /* rotation kind: 0 or CONVROT_ROT_REGULAR */
    int8_t *codes;             /* device, K-tiled INT8 codes of W . R^T [N, K] */
    float *scale;              /* device, [N] per-output F32 scales */
} convrot_weights;

/* Human-readable name of a status code (static string, never NULL). */
CONVROT_API const char *convrot_status_string(int status);

/* The hipError_t of the most recent CONVROT_EHIP on this thread (0 if none). */
CONVROT_API int convrot_last_hip_error(void);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
CONVROT_API int convrot_version(void);

/* ------------------------------------------------------------------ */
/* sizing queries (host only, no HIP calls)                            */
/* ------------------------------------------------------------------ */

/* Bytes of packed codes for an [N, K] weight (0 for invalid shapes): one
 * INT8 code per weight, as the INT8 checkpoint stores them (PulpCut input-major
 * README, "Input-major checkpoint"), in the K-tiled layout above. */
CONVROT_API size_t convrot_weights_packed_bytes(int64_t N, int64_t K, int block);

/* Workspace for convrot_linear_prepare_weights (0 is a valid answer): the
 * transposed float weights when an input-major [input, output] source is
 * rotated (PulpCut input-major README, "Input-major checkpoint"). */
CONVROT_API size_t convrot_prepare_workspace_bytes(int64_t N, int64_t K, int block,
                                       int w_dtype, int layout);

/* Workspace for convrot_linear_forward: K-tiled INT8 codes (Mp x K bytes) and
 * F32 row scales [M] of the rotated activations, each region 256-byte
 * aligned.  A caller-owned static workspace stands in for per-call
 * allocation (MiniMax-H3-Rung-Omega README, "Technical Architecture
 * Overview", Floor 1: one contiguous workspace instead of per-call mallocs). */
CONVROT_API size_t convrot_linear_workspace_bytes(int64_t M, int64_t K, int64_t N, int block);

/* Workspace for lowrank_convrot_forward (codes of X, bf16 intermediate
 * H [M, r], codes of H, and row scales) -- the low-rank linears of the INT8
 * package (HyperFlow H3 Flash card, "Choose a Weight Format"). */
CONVROT_API size_t lowrank_convrot_workspace_bytes(int64_t M, int64_t K, int64_t r,
                                       int64_t N, int block);

/* Workspace for convrot_mlp_forward (codes of X, the bf16 intermediate u or g [M, F],
 * codes of g, row scales): the MLP whose activation feeds a rotated, rowwise
 * quantised fc2 (MiniMax-H3-Rung-Omega README, "Technical Architecture
 * Overview", Floor 1). */
CONVROT_API size_t convrot_mlp_workspace_bytes(int64_t M, int64_t K, int64_t F, int64_t N,
                                   int block);

/* ------------------------------------------------------------------ */
/* weight preparation (load time)                                      */
/* ------------------------------------------------------------------ */

/* Rotate, quantise and pack one weight matrix: the INT8 codes with one F32
 * scale per output channel, output-major [output, input] or input-major
 * [input, output] at the source (PulpCut input-major README, "Input-major
 * checkpoint"), rotated so that dequantising and undoing the rotation gives
 * the weights back (HyperFlow H3 Flash MLX card, "Where the weights come
 * from").
 *   W         device; F32 or BF16 float weights, or I8 codes that are already
 *             rotated (import mode).  Layout per `layout`:
 *             CONVROT_OUT_MAJOR -> [N, K], CONVROT_IN_MAJOR -> [K, N].
 *   src_scale I8 import only: device [N] per-output scales, copied unchanged;
 *             must be NULL for float weights.
 *   block     Hadamard block b in {64, 128, 256}; K % block == 0.
 *   out       host struct; out->codes and out->scale must point to caller
 *             allocations of convrot_weights_packed_bytes(N, K, block) and 4*N
 *             bytes, and out->flags selects the rotation kind (0 or
 *             CONVROT_ROT_REGULAR; EINVAL for other bits or for the regular
 *             kind at b = 128).  On success every other field is filled in.
 *   ws        device workspace of convrot_prepare_workspace_bytes(...) bytes
 *             (may be NULL when that query returns 0).
 * Float weights: row n of W becomes codes/scale of FWHT_b(W[n, :]) quantised
 * per output channel, i.e. the INT8 image of W . R^T.  Import mode copies the
 * codes (row-major [N, K], or [K, N] for IN_MAJOR) into the K-tiled layout and
 * the scales without changing any value, as the input-major repack does. */
CONVROT_API int convrot_linear_prepare_weights(const void *W, int w_dtype, int layout,
                                   const float *src_scale, int64_t N, int64_t K,
                                   int block, convrot_weights *out, void *ws,
                                   size_t ws_bytes, void *stream);

/* The rank a low-rank pair is stored with (0 for r <= 0, r > 65536 or a bad
 * block): r rounded up to a multiple of 128, or of 256 when b = 256.  The
 * checkpoint loader pads low-rank ranks to a multiple of 64 (HyperFlow H3
 * Flash card, "Standalone Transformer (AutoModel)", pad_lowrank_ranks); 128
 * is such a multiple and the contraction's K granularity, and 256 lets whole
 * blocks tile the rank. */
CONVROT_API int64_t lowrank_convrot_padded_rank(int64_t r, int block);

/* Workspace for lowrank_convrot_prepare_weights: the zero-padded float copies
 * of both factors when the rank needs padding, else 0. */
CONVROT_API size_t lowrank_convrot_prepare_workspace_bytes(int64_t r, int64_t K, int64_t N,
                                                           int block, int w_dtype);

/* Prepare a low-rank pair W ~ B . A (HyperFlow H3 Flash card, "Choose a Weight
 * Format" and "Standalone Transformer (AutoModel)"):
 *   A, B      device float weights (w_dtype CONVROT_F32 or CONVROT_BF16), both
 *             output-major and row-major: A [r, K], B [N, r].
 *   outA      prepared [rp, K] factor, rp = lowrank_convrot_padded_rank(r, b);
 *             outA->codes / outA->scale point to caller allocations of
 *             convrot_weights_packed_bytes(rp, K, b) and 4*rp bytes.
 *   outB      prepared [N, rp] factor; convrot_weights_packed_bytes(N, rp, b)
 *             and 4*N bytes.  outA->flags == outB->flags selects the rotation
 *             kind, as for convrot_linear_prepare_weights.
 *   ws        device workspace of lowrank_convrot_prepare_workspace_bytes(...)
 *             (may be NULL when it is 0); it is read in stream order.
 * The rank is padded with zero rows of A and zero columns of B, which leaves
 * B . A unchanged; their rotated blocks are zero, so when b divides r the
 * forward equals the unpadded chain bit for bit.  Errors as for
 * convrot_linear_prepare_weights (EUNSUPPORTED for other dtypes or for padded
 * shapes outside the limits). */
CONVROT_API int lowrank_convrot_prepare_weights(const void *A, const void *B, int w_dtype,
                                                int64_t r, int64_t K, int64_t N, int block,
                                                convrot_weights *outA, convrot_weights *outB,
                                                void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------ */
/* forward entry points                                                */
/* ------------------------------------------------------------------ */

/* Y = dequant(Q(R x) . Q(W R^T)^T) (+ bias) for every row x of X: the W8A8
 * linear behind a block-diagonal Hadamard rotation (lehuy.net article on
 * HyperFlow H3 Flash, "Cach nen hoat dong", second bullet), the activation
 * rotated and quantised row-wise first (MiniMax-H3-Rung-Omega README,
 * "Technical Architecture Overview", Floor 1).
 *   X       device bf16 [M, W->K] activations.
 *   W       prepared weights (host struct).
 *   bias    device F32 [W->N] or NULL.
 *   Y       device [M, W->N], y_dtype CONVROT_BF16 or CONVROT_F32.
 *   ws      device workspace of convrot_linear_workspace_bytes(M, K, N, b).
 * Rows are independent: forward on a row slice equals the same slice of the
 * full forward, bit for bit. */
CONVROT_API int convrot_linear_forward(const void *X, int64_t M, const convrot_weights *W,
                           const float *bias, void *Y, int y_dtype, void *ws,
                           size_t ws_bytes, void *stream);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): convrot_linear_forward
 * without a workspace argument.  The rotated activations' K-tiled codes and
 * row scales go to a static device array of the library of
 * CONVROT_NOALLOC_SCRATCH_BYTES (32 MiB, one copy per device, held until the
 * process ends) instead of a caller workspace; the call allocates nothing.
 * Shapes whose convrot_linear_workspace_bytes(M, K, N, b) exceed that size
 * return CONVROT_EWORKSPACE (use convrot_linear_forward); M = 4096 at
 * K = 5376 fits.  Every call on a device shares that device's array, so calls
 * on one device that overlap in time (concurrent streams) race and must be
 * ordered by the caller.  Nothing in the array needs to start at zero: each
 * call writes every code and scale it reads.  Otherwise the arguments, the
 * results (bit for bit) and the errors are those of convrot_linear_forward. */
#define CONVROT_NOALLOC_SCRATCH_BYTES (32u << 20)
CONVROT_API int convrot_linear_forward_noalloc(const void *X, int64_t M,
                                               const convrot_weights *W, const float *bias,
                                               void *Y, int y_dtype, void *stream);

/* Low-rank ConvRot linear (HyperFlow H3 Flash card, "Choose a Weight Format":
 * the INT8 package holds W8A8 linears and low-rank factorised ones; both
 * factors are W8A8 here): h = bf16(linear(X; A)) with A [r, K] and no bias,
 * then Y = linear(h; B) with B [N, r] and the bias; h is re-rotated along r
 * with the same block and requantised per token.  Requires A->N == B->K (= r),
 * A->block == B->block, the same rotation kind (A->flags == B->flags) and
 * r % 128 == 0 (pad the rank with zero rows of A and
 * zero columns of B, which leaves the product unchanged). */
CONVROT_API int lowrank_convrot_forward(const void *X, int64_t M, const convrot_weights *A,
                            const convrot_weights *B, const float *bias,
                            void *Y, int y_dtype, void *ws, size_t ws_bytes,
                            void *stream);

/* MLP pair, its activation applied in front of the rotated, rowwise
 * quantised down projection (MiniMax-H3-Rung-Omega README, "Technical
 * Architecture Overview", Floor 1, fuses the activation, ConvRot and the
 * rowwise INT8 quantise ahead of MLP.fc2):
 * u = bf16(linear(X; W_up) + bias_up); g = bf16(GELU(u)) with the
 * erf form of GELU (see convrot_gelu_bf16); Y = linear(g; W_down) + bias_down.
 * Requires W_up->N == W_down->K (= F) and the same block and rotation kind.
 * Where GELU runs depends on F only, never the result: for 6144 < F <= 24576
 * the up projection writes u and the rotate+quantise pass of the down
 * projection applies GELU as it loads u (g is never written); otherwise the
 * up projection's epilogue applies it and writes g (u is never written). */
CONVROT_API int convrot_mlp_forward(const void *X, int64_t M, const convrot_weights *W_up,
                        const float *bias_up, const convrot_weights *W_down,
                        const float *bias_down, void *Y, int y_dtype, void *ws,
                        size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------ */
/* SwiGLU MLP                                                          */
/* ------------------------------------------------------------------ */

/* The SwiGLU MLP of MiniMax-H3-Rung-Omega README, "Technical Architecture
 * Overview", Floor 1 (SwiGLU, ConvRot64 and the rowwise INT8 quantise fused
 * in front of MLP.fc2).  fc1 is one ConvRot linear with 2F outputs, the gate
 * channels [0, F) and the up channels [F, 2F); the activation is
 *   g = bf16(s * u),  s = fp32(silu(gate)),  silu(z) = z / (1 + exp(-z))
 * evaluated in fp64 on the bf16 gate and rounded once to fp32, s * u one fp32
 * multiply on the bf16 up value u, g rounded to nearest even; fc2 is a ConvRot
 * linear on g with its own block (64 for ConvRot64).  fc1's epilogue forms g,
 * so the [M, 2F] fc1 output is never written; g [M, F] is, and fc2's
 * rotate+quantise reads it. */

/* Workspace for convrot_swiglu_prepare_weights: the interleaved copy of the
 * [2F, K] weight (and of its scales when importing codes). */
CONVROT_API size_t convrot_swiglu_prepare_workspace_bytes(int64_t F, int64_t K, int block,
                                                          int w_dtype);

/* Prepare a SwiGLU fc1 weight W [2F, K], output-major, gate rows first:
 * F32/BF16 float weights (rotated and quantised per output channel as by
 * convrot_linear_prepare_weights), or I8 codes with src_scale [2F] (import).
 * The rows are stored interleaved (CONVROT_SWIGLU_PAIRS, set in out->flags
 * beside the rotation kind, which out->flags selects on entry as for
 * convrot_linear_prepare_weights).  out->codes / out->scale: caller
 * allocations of convrot_weights_packed_bytes(2F, K, b) and 8F bytes.
 * F % 16 == 0; ws of convrot_swiglu_prepare_workspace_bytes(F, K, b, w_dtype)
 * bytes (required).  Errors as for convrot_linear_prepare_weights. */
CONVROT_API int convrot_swiglu_prepare_weights(const void *W, int w_dtype,
                                               const float *src_scale, int64_t F, int64_t K,
                                               int block, convrot_weights *out, void *ws,
                                               size_t ws_bytes, void *stream);

/* Workspace for convrot_swiglu_mlp_forward (codes of X, g [M, F] bf16, codes
 * of g, row scales); block_up and block_down are fc1's and fc2's blocks. */
CONVROT_API size_t convrot_swiglu_mlp_workspace_bytes(int64_t M, int64_t K, int64_t F,
                                                      int64_t N, int block_up,
                                                      int block_down);

/* Y = linear(g; W_down) + bias_down with g = swiglu(linear(X; W_gu) + bias_gu).
 *   X        device bf16 [M, K].
 *   W_gu     prepared by convrot_swiglu_prepare_weights (2F x K).
 *   bias_gu  device F32 [2F] in source order (gate biases, then up), or NULL.
 *   W_down   a plain prepared weight [N, F]; its block may differ from W_gu's
 *            (64 for ConvRot64); both must have the same rotation kind.
 *   bias_down device F32 [N] or NULL; Y device [M, N] (BF16 or F32).
 * ELAYOUT if W_gu lacks CONVROT_SWIGLU_PAIRS, W_down has it, W_gu->N != 2F or
 * the rotation kinds differ. */
CONVROT_API int convrot_swiglu_mlp_forward(const void *X, int64_t M, const convrot_weights *W_gu,
                                           const float *bias_gu,
                                           const convrot_weights *W_down,
                                           const float *bias_down, void *Y, int y_dtype,
                                           void *ws, size_t ws_bytes, void *stream);

/* The SwiGLU activation on its own (a test hook and the unfused form): g [M, F]
 * from gu [M, 2F] (gate | up), bf16 device buffers, 16-byte aligned,
 * F % 8 == 0. */
CONVROT_API int convrot_swiglu_bf16(const uint16_t *gu, int64_t M, int64_t F, uint16_t *g,
                                    void *stream);

/* s[i] = fp32(silu(a[i])) for n bf16 values, the s of every SwiGLU path
 * (test hook: lets a test compare every bf16 pattern at fp32 precision). */
CONVROT_API int convrot_silu_f32(const uint16_t *a, int64_t n, float *s, void *stream);

/* ------------------------------------------------------------------ */
/* comparison variant (not the W8A8 path)                              */
/* ------------------------------------------------------------------ */

/* Low-rank linear whose factors stay bf16: no rotation, no quantisation, as
 * in the ComfyUI INT8 convrot copies where the low-rank linears stay bf16
 * (HyperFlow H3 Flash card, "INT8 convrot in ComfyUI").  Kept to compare the
 * W8A8 low-rank path against.  h = bf16(X . A^T) and Y = bf16(h . B^T + bias),
 * each product accumulated in fp32 on the matrix cores, the bias added in
 * fp32, bf16 by round to nearest even.
 *   X bf16 [M, K], A bf16 [r, K], B bf16 [N, r], all row-major device
 *   pointers; bias F32 [N] or NULL; Y bf16 [M, N].
 *   ws: device workspace of lowrank_bf16_workspace_bytes(M, r) bytes (h).
 * K % 64 == 0, r % 64 == 0 (the checkpoint's rank padding), N % 16 == 0,
 * K, r <= 65536 and every matrix under 2^31 bytes (EUNSUPPORTED otherwise). */
CONVROT_API size_t lowrank_bf16_workspace_bytes(int64_t M, int64_t r);
CONVROT_API int lowrank_bf16_forward(const void *X, int64_t M, int64_t K, const void *A,
                         int64_t r, const void *B, int64_t N, const float *bias,
                         void *Y, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------ */
/* test hooks: the stages of the forward path, exported for parity     */
/* tests.  Same validation and error behaviour as the entry points.    */
/* ------------------------------------------------------------------ */

/* Rotate and quantise rows (the rotation and rowwise INT8 quantise of
 * MiniMax-H3-Rung-Omega README, "Technical Architecture Overview", Floor 1;
 * for F32 weight rows, the weight preparation of convrot_linear_prepare_weights):
 * X [M, K] row-major (x_dtype F32 or BF16) -> q
 * K-tiled int8 codes (Mp x K bytes; the padding rows are left as they were)
 * and s [M] F32.  flags: 0 or CONVROT_ROT_REGULAR (the rotation kind), plus
 * optionally CONVROT_FLAG_GELU (defined below): the rows are then
 * bf16(GELU(X)) of bf16 X, as convrot_mlp_forward quantises its intermediate
 * when 6144 < K <= 24576 (the up projection writes X = u with the plain
 * epilogue and the GELU is applied as the rows are loaded).  With the flag,
 * F32 input or K outside that range returns EUNSUPPORTED. */
CONVROT_API int convrot_rotate_quantize(const void *X, int x_dtype, int64_t M, int64_t K,
                            int block, uint32_t flags, int8_t *q, float *s,
                            void *stream);

/* Exact INT32 contraction acc[M, N] (row-major) = q_x . codes(W)^T, q_x the
 * K-tiled codes of M rows (Mp x W->K bytes): the INT8 GEMM of the W8A8 linear
 * (mmh3turbo README, "Why it is fast, and where it is not"). */
CONVROT_API int convrot_gemm_i32(const int8_t *q_x, int64_t M, const convrot_weights *W,
                     int32_t *acc, void *stream);

/* Contraction plus the dequant epilogue from given codes and row scales,
 * per token (s_x) and per output channel (s_w, the checkpoint's per-output
 * F32 scales: PulpCut input-major README, "Input-major checkpoint"):
 * Y = ((float)(q_x . codes(W)^T) * s_x) * s_w (+ bias).  With
 * CONVROT_FLAG_GELU (y_dtype must be BF16) the epilogue writes
 * bf16(GELU(float(bf16(Y)))), the activation the MLP entry point feeds to its
 * down projection. */
#define CONVROT_FLAG_GELU 1u
/* CONVROT_FLAG_SWIGLU (W prepared by convrot_swiglu_prepare_weights, y_dtype
 * BF16): the epilogue writes g = swiglu of the bf16 fc1 outputs, Y [M, W->N/2],
 * as convrot_swiglu_mlp_forward feeds its down projection; the bias is [W->N]
 * in source order. */
#define CONVROT_FLAG_SWIGLU 2u
CONVROT_API int convrot_gemm_dequant(const int8_t *q_x, const float *s_x, int64_t M,
                         const convrot_weights *W, const float *bias, void *Y,
                         int y_dtype, uint32_t flags, void *stream);

/* Factor 1 of the low-rank chain and the requantisation of its output, in
 * one kernel: h = bf16(((float)(q_x . codes(A)^T) * s_x) * s_A) [M, r] with
 * r = A->N, then (q_h, s_h) = rotate_quantize(h) with block A->block, exactly
 * as lowrank_convrot_forward feeds factor 2 (low-rank ConvRot linears: the
 * MLX model card, "Choose a Weight Format").  h itself is never written.
 * q_x (K-tiled, Mp x A->K bytes) and s_x [M] F32 come from
 * convrot_rotate_quantize; q_h (K-tiled, Mp x r bytes; its padding rows get
 * unspecified codes) and s_h [M] F32 are written.  All device pointers,
 * 16-byte aligned.  Supported for the Sylvester rotation with A->block in
 * {64, 128} and r <= 512 (CONVROT_EUNSUPPORTED otherwise;
 * lowrank_convrot_forward then runs the two stages separately). */
CONVROT_API int convrot_lowrank_factor1(const int8_t *q_x, const float *s_x, int64_t M,
                            const convrot_weights *A, int8_t *q_h, float *s_h,
                            void *stream);

/* The activation in front of fc2 (MiniMax-H3-Rung-Omega README, "Technical
 * Architecture Overview", Floor 1), GELU form:
 * g[i] = bf16(GELU(u[i])) for n bf16 values, exactly as the MLP entry point
 * and CONVROT_FLAG_GELU apply it: GELU in its erf form, 0.5 z (1 + erf(z /
 * sqrt 2)), evaluated in fp64 on the bf16 value z, rounded to fp32 and then
 * to bf16 (nearest even).  u and g are device pointers; n >= 0. */
CONVROT_API int convrot_gelu_bf16(const uint16_t *u, int64_t n, uint16_t *g, void *stream);

/* ------------------------------------------------------------------ */
/* measurement probes: ceilings measured on the device, printed by the */
/* benchmark beside the spec peaks.  They compute nothing of the      */
/* method.                                                            */
/* ------------------------------------------------------------------ */

/* INT8 matrix-core rate on operands that change every round: one 256-thread
 * workgroup per compute unit; each wave runs `iters` rounds of 4 x 4
 * v_mfma_i32_32x32x32_i8 (16 x 65536 INT8 operations per round) on fragments
 * seeded from `seed` (4 KiB, device) and remixed after every round.  `sink`
 * (16 bytes, device) is written only if the accumulators fold to one
 * improbable value; it keeps the work from being dropped.  *ops (host)
 * receives the INT8 operations of the launch.  1 <= iters <= 2^24;
 * device pointers 16-byte aligned. */
CONVROT_API int convrot_probe_mfma_i8(int64_t iters, const void *seed, void *sink,
                                      int64_t *ops, void *stream);

/* Streaming probe with no arithmetic, over n16 16-byte items: mode 0 (the
 * rotate+quantise traffic shape) reads item i of src and writes 8 bytes to
 * dst + 8 i (the xor of input words 0 and 1, then of words 2 and 3); mode 1
 * copies the 16 bytes to dst + 16 i; mode 2 reads nothing (src may be NULL)
 * and writes the low 32 bits of i to all four words of dst + 16 i.  Device
 * pointers, 16-byte aligned, not overlapping. */
CONVROT_API int convrot_probe_stream(const void *src, void *dst, int64_t n16, int mode,
                                     void *stream);

#ifdef __cplusplus
}
#endif

#endif /* CONVROT_H */
