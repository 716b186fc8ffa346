// Shared device helpers and launch declarations of libconvrot (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convrot {

// ---------------------------------------------------------------- bf16 ----

// bf16 -> fp32 is exact: the bf16 bits are the top half of the binary32.
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest, ties to even (NaN -> quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return ((u >> 16) & 0x8000u) | 0x7fc0u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

} // namespace convrot

// ------------------------------------------------------ kernel launchers ----
// All launchers assume arguments were validated by the API layer.

namespace convrot {

// ------------------------------------------------ INT8 code layout ----
// Every INT8 code matrix of the library (activation codes, weight codes, the
// low-rank intermediate) is stored K-tiled: rows in blocks of 16, a block as
// K/64 consecutive 1 KiB tiles of 16 rows x 64 bytes, and inside a tile the
// 16-byte chunk c of row r at slot c ^ ((r >> 2) & 3).  The GEMM's copy of one
// 16-row K-tile is then a single contiguous 1 KiB read (8 whole cache lines
// instead of 16 half lines, twice the copy rate on gfx950), and it lands in
// LDS already in the order whose fragment reads are free of bank conflicts.
// Rows are padded to a multiple of 16; the block of rows m0 .. m0+15 starts
// at byte m0 * K as in row-major order.  Requires K % 64 == 0.
__host__ __device__ inline int64_t tiled_offset(int64_t m, int64_t k, int64_t K)
{
    return ((m >> 4) * (K >> 6) + (k >> 6)) * 1024 + (m & 15) * 64 +
           ((((k >> 4) & 3) ^ ((m >> 2) & 3)) << 4) + (k & 15);
}
__host__ __device__ inline int64_t padded_rows(int64_t M) { return (M + 15) & ~int64_t(15); }

enum class InType { F32 = 0, BF16 = 1 };

// Compute units of the current device (queried once; 256 if the query fails).
int device_cu_count();
// BF16_MM: not an INT8 path -- bf16 x bf16 operands, row-major, fp32
// accumulation, y = bf16(acc (+ bias)); used by the bf16 low-rank variant.
// SWIGLU_BF16: the weight rows come in 32-row blocks of 16 gate rows and their
// 16 up rows (convrot_swiglu_prepare_weights); the epilogue writes
// g = bf16(fp32(silu(bf16 gate)) * bf16 up) as an [M, N/2] bf16 matrix.
enum class OutKind { BF16 = 0, F32 = 1, I32 = 2, GELU_BF16 = 3, BF16_MM = 4, SWIGLU_BF16 = 5 };

// Packed row p of a SwiGLU fc1 weight holds source row swiglu_src_row(p, F)
// of the [2F, K] weight (gate rows 0 .. F-1, up rows F .. 2F-1).
__host__ __device__ inline int64_t swiglu_src_row(int64_t p, int64_t F)
{
    const int64_t blk = p >> 5, r = p & 31;
    return r < 16 ? blk * 16 + r : F + blk * 16 + (r - 16);
}

// Rotate (blockwise Sylvester FWHT, or with `regular` the H_4 = J - 2I
// Kronecker blocks for block 64 or 256) + rowwise INT8 quantise.  src rows
// have stride ld elements; q is K-tiled with padded_rows(M) rows (the
// padding rows are not written).
hipError_t launch_rotquant(const void *src, InType in, int64_t M, int64_t K,
                           int64_t ld, int block, bool regular, float inv_sqrt_b, int8_t *q,
                           float *s, hipStream_t stream);

// Rotate and quantise bf16(GELU(u)) for bf16 rows u: the MLP's down-projection
// input, read as the up projection's plain output.  gelu_table holds
// bf16(GELU(x)) for every bf16 pattern x (launch_gelu_table).  Only for rows
// that the two-rows-per-wave kernel serves: rotquant_fuses_gelu(K).
bool rotquant_fuses_gelu(int64_t K);
hipError_t launch_rotquant_gelu(const void *src, int64_t M, int64_t K, int64_t ld, int block,
                                bool regular, float inv_sqrt_b, const uint16_t *gelu_table,
                                int8_t *q, float *s, hipStream_t stream);

// SwiGLU (fc1 output gu [M, 2F] = gate | up): the elementwise g [M, F] =
// bf16(fp32(silu(gate)) * up) (F % 8 == 0, 16-byte aligned buffers);
// fp32(silu(a)) for n bf16 values; and the device address of the silu table
// (fp32 silu of every bf16 pattern, written once per device like the GELU
// table), which the fused SwiGLU epilogue of the GEMM reads.
hipError_t launch_swiglu_bf16(const uint16_t *gu, int64_t M, int64_t F, uint16_t *g,
                              hipStream_t stream);
hipError_t launch_silu_f32(const uint16_t *a, int64_t n, float *out, hipStream_t stream);
hipError_t launch_silu_table(const float **table, hipStream_t stream);

// Factor 1 of the low-rank chain with the requantisation fused in:
// (qh, sh) = rotate+quantise(bf16(((float)(qx . qa^T) * sx) * sa)) along the R
// outputs, for R % 128 == 0, R <= 512 and block 64 or 128 (lowrank_f1_fusable).
bool lowrank_f1_fusable(int64_t R, int block);
hipError_t launch_lowrank_f1(const int8_t *qx, const int8_t *qa, const float *sx,
                             const float *sa, int8_t *qh, float *sh, int64_t M, int64_t R,
                             int64_t K, int block, float inv_sqrt_b, hipStream_t stream);

// g[i] = bf16(GELU(u[i])) for bf16 u, as the MLP's up projection applies it.
hipError_t launch_gelu_bf16(const uint16_t *u, uint16_t *g, int64_t n, hipStream_t stream);
// The device address of the 65,536-entry bf16 GELU table on the current
// device, written on `stream` if it has not been yet: the first such call that
// is not being recorded into a graph waits for the fill once, after which no
// call launches it again on that device.
hipError_t launch_gelu_table(const uint16_t **table, hipStream_t stream);

// INT8 codes [R, C] into the K-tiled layout (R % 16 == 0, C % 64 == 0); the
// source is row-major [R, C] (ld = C) or, with transposed, [C, R].
hipError_t launch_tile_codes(const int8_t *src, bool transposed, int8_t *dst, int64_t R,
                             int64_t C, hipStream_t stream);

// dst [Rd, Cd] (Rd >= R, Cd >= C) = the [R, C] matrix src of 2- or 4-byte
// elements in its top-left corner, zeros elsewhere.
hipError_t launch_pad_copy(const void *src, int64_t R, int64_t C, void *dst, int64_t Rd,
                           int64_t Cd, int elem_bytes, hipStream_t stream);

// Transpose an [R, C] matrix of 1-, 2- or 4-byte elements into [C, R].
hipError_t launch_transpose(const void *src, void *dst, int64_t R, int64_t C,
                            int elem_bytes, hipStream_t stream);

// acc/Y[M, N] = epilogue(qx[M, K] . qw[N, K]^T), both code matrices K-tiled.
// For OutKind::BF16_MM, qx and qw are row-major bf16 matrices, K counts
// their row bytes (2 x elements), and sx, sw are unused.  For
// OutKind::SWIGLU_BF16, Y is [M, N/2] and the bias is indexed by source row
// (swiglu_src_row).
hipError_t launch_gemm_i8(const int8_t *qx, const int8_t *qw, const float *sx,
                          const float *sw, const float *bias, void *Y,
                          OutKind out, int64_t M, int64_t N, int64_t K,
                          hipStream_t stream);

// Copy the rows of a [2F, K] SwiGLU fc1 weight (elem_bytes 1, 2 or 4), or of
// its scales (K = 1, elem_bytes 4), into the interleaved order of
// swiglu_src_row: dst row p = src row swiglu_src_row(p, F).
// K * elem_bytes % 4 == 0.
hipError_t launch_swiglu_interleave(const void *src, void *dst, int64_t F, int64_t K,
                                    int elem_bytes, hipStream_t stream);

// Measurement probes (probes.hip): INT8 MFMA rounds on changing operands, one
// workgroup per CU (probe_mfma_i8_ops: the INT8 operations of one launch),
// and a streaming pass over n16 16-byte items (mode 0: 8 bytes out per item,
// 1: a copy, 2: writes only).
int64_t probe_mfma_i8_ops(int64_t iters);
hipError_t launch_probe_mfma_i8(int64_t iters, const int *seed, int *sink, hipStream_t stream);
hipError_t launch_probe_stream(const void *src, void *dst, int64_t n16, int mode,
                               hipStream_t stream);

} // namespace convrot
