// INT8 x INT8 -> INT32 GEMM on gfx950 matrix cores with a fused dequant
// epilogue:  Y[m, n] = ((float)acc[m, n] * s_x[m]) * s_w[n] (+ bias[n]).
//
// The contraction is the W8A8 projection of a ConvRot linear (lehuy.net
// article on HyperFlow H3 Flash, "Cach nen hoat dong"; the mmh3turbo README,
// "Why it is fast, and where it is not", reports it for K = 5376).  The scales
// are per token (s_x) and per output channel (s_w; PulpCut input-major README,
// "Input-major checkpoint").
//
// Operands: qx [M, K] and qw [N, K], both row-major with K contiguous, so each
// MFMA lane reads 16 consecutive bytes of one row for either operand.
//
// Tiling: a 256-thread workgroup (4 waves, one per SIMD) owns a 256 (n) x 256
// (m) output tile; wave (wn, wm) owns 128 x 128 of it as 4 x 4 tiles of
// v_mfma_i32_32x32x32_i8 (256 int32 accumulators per lane, held in AGPRs).
// The weight tile is the MFMA A operand (rows = n) and the activation tile
// the B operand (columns = m), so an accumulator lane holds 4 consecutive n of
// one m and the epilogue stores 4 outputs per instruction.
// K advances 128 bytes per stage through two LDS stages of 64 KiB each; the
// next stage's global loads are issued before the current stage's MFMAs and
// written to LDS after them, one barrier per stage.
// LDS rows are 128 bytes; the 16-byte chunk c of tile row r lives at slot
// c ^ f(r), f(r) = (r & 7) ^ ((r >> 3) & 1), which keeps both the row-wise
// writes and the column-wise MFMA fragment reads free of bank conflicts.
// Workgroups are renumbered so each of the 8 XCDs walks a contiguous range of
// tiles, grouped 8 tile-rows high, for L2 reuse of both operands.
#include "common.hpp"

namespace convrot {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kTile = 256;     // tile edge in m and in n
constexpr int kBK = 128;       // K bytes per LDS stage
constexpr int kThreads = 256;
constexpr int kStageBytes = kTile * kBK;   // one operand, one stage: 32 KiB
constexpr int kGroup = 8;      // tile-rows per L2 group

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int OUT, bool HAS_BIAS>
__device__ __forceinline__ void store4(void *Y, int64_t off, const v16i &acc, int q,
                                       float sxm, const float4 &swv, const float4 &bv)
{
    if constexpr (OUT == int(OutKind::I32)) {
        int4 o;
        o.x = acc[4 * q + 0]; o.y = acc[4 * q + 1];
        o.z = acc[4 * q + 2]; o.w = acc[4 * q + 3];
        *reinterpret_cast<int4 *>(reinterpret_cast<int32_t *>(Y) + off) = o;
    } else {
        float y[4];
        const float sw4[4] = {swv.x, swv.y, swv.z, swv.w};
        const float b4[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            float f = __fmul_rn(__fmul_rn((float)acc[4 * q + t], sxm), sw4[t]);
            if constexpr (HAS_BIAS) f = __fadd_rn(f, b4[t]);
            y[t] = f;
        }
        if constexpr (OUT == int(OutKind::F32)) {
            *reinterpret_cast<float4 *>(reinterpret_cast<float *>(Y) + off) =
                make_float4(y[0], y[1], y[2], y[3]);
        } else {
            if constexpr (OUT == int(OutKind::GELU_BF16)) {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float u = __uint_as_float(f32_to_bf16_bits(y[t]) << 16);
                    y[t] = gelu_erf(u);
                }
            }
            uint2 o;
            o.x = pack_bf16x2(y[0], y[1]);
            o.y = pack_bf16x2(y[2], y[3]);
            *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(Y) + off) = o;
        }
    }
}

template <int OUT, bool HAS_BIAS>
__global__ __launch_bounds__(kThreads, 1) void gemm_i8_kernel(
    const int8_t *__restrict__ qx, const int8_t *__restrict__ qw,
    const float *__restrict__ sx, const float *__restrict__ sw,
    const float *__restrict__ bias, void *__restrict__ Y, int M, int N, int K,
    int tiles_m, int tiles_n, int tiles_per_xcd)
{
    __shared__ __attribute__((aligned(16))) int8_t smem[2][2][kStageBytes];  // [stage][W|X]

    // ---- tile selection: XCD-contiguous ranges, grouped along m ----
    const int pid = blockIdx.x;
    const int t = (pid & 7) * tiles_per_xcd + (pid >> 3);
    if (t >= tiles_m * tiles_n) return;
    const int width = kGroup * tiles_n;
    const int first_m = (t / width) * kGroup;
    const int gsz = min(tiles_m - first_m, kGroup);
    const int tm = first_m + (t % width) % gsz;
    const int tn = (t % width) / gsz;
    const int m0 = tm * kTile, n0 = tn * kTile;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wn = wave & 1, wm = wave >> 1;

    // ---- global -> LDS copy assignment: 8 rows per thread and operand ----
    const int crow = tid >> 3, cch = tid & 7;
    uint32_t offx[8], offw[8];
#pragma unroll
    for (int l = 0; l < 8; ++l) {
        const int r = crow + 32 * l;
        offx[l] = (uint32_t)min(m0 + r, M - 1) * (uint32_t)K + cch * 16;
        offw[l] = (uint32_t)min(n0 + r, N - 1) * (uint32_t)K + cch * 16;
    }
    const int lds_w = crow * kBK + ((cch ^ swz(crow)) << 4);  // + 4096 * l

    // ---- fragment read assignment ----
    const int l32 = lane & 31, g = lane >> 5;
    const int fx = g ^ swz(l32);
    int foff[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) foff[s] = ((2 * s) ^ fx) << 4;
    const int frow_w = (wn * 128 + l32) * kBK;  // + 4096 * i
    const int frow_x = (wm * 128 + l32) * kBK;  // + 4096 * j

    v16i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

    v4i rw[8], rx[8];
#pragma unroll
    for (int l = 0; l < 8; ++l) {
        rw[l] = *reinterpret_cast<const v4i *>(qw + offw[l]);
        rx[l] = *reinterpret_cast<const v4i *>(qx + offx[l]);
    }
#pragma unroll
    for (int l = 0; l < 8; ++l) {
        *reinterpret_cast<v4i *>(&smem[0][0][lds_w + 4096 * l]) = rw[l];
        *reinterpret_cast<v4i *>(&smem[0][1][lds_w + 4096 * l]) = rx[l];
    }
    __syncthreads();

    const int nk = K / kBK;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            const int8_t *bw = qw + (kt + 1) * kBK;
            const int8_t *bx = qx + (kt + 1) * kBK;
#pragma unroll
            for (int l = 0; l < 8; ++l) {
                rw[l] = *reinterpret_cast<const v4i *>(bw + offw[l]);
                rx[l] = *reinterpret_cast<const v4i *>(bx + offx[l]);
            }
        }
        const int8_t *sw_ = smem[cur][0];
        const int8_t *sx_ = smem[cur][1];
        v4i a[2][4], b[2][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a[0][i] = *reinterpret_cast<const v4i *>(sw_ + frow_w + 4096 * i + foff[0]);
            b[0][i] = *reinterpret_cast<const v4i *>(sx_ + frow_x + 4096 * i + foff[0]);
        }
        // Sub-step s: read the fragments of s+1, then 16 MFMAs on those of s.
        // The scheduling barriers keep each group together so the LDS reads
        // of the next sub-step overlap the current MFMAs.
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int c = s & 1;
            if (s < 3) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    a[c ^ 1][i] = *reinterpret_cast<const v4i *>(sw_ + frow_w + 4096 * i + foff[s + 1]);
                    b[c ^ 1][i] = *reinterpret_cast<const v4i *>(sx_ + frow_x + 4096 * i + foff[s + 1]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[c][i], b[c][j], acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (more) {
#pragma unroll
            for (int l = 0; l < 8; ++l) {
                *reinterpret_cast<v4i *>(&smem[cur ^ 1][0][lds_w + 4096 * l]) = rw[l];
                *reinterpret_cast<v4i *>(&smem[cur ^ 1][1][lds_w + 4096 * l]) = rx[l];
            }
        }
        __syncthreads();
    }

    // ---- epilogue: lane holds n = nb..nb+3 of one m per (i, j, q) ----
    const float4 zero4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int m = m0 + wm * 128 + 32 * j + l32;
        if (m >= M) continue;
        const float sxm = (OUT == int(OutKind::I32)) ? 0.0f : sx[m];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int nb = n0 + wn * 128 + 32 * i + 8 * q + 4 * g;
                if (nb >= N) continue;
                float4 swv = zero4, bv = zero4;
                if constexpr (OUT != int(OutKind::I32)) {
                    swv = *reinterpret_cast<const float4 *>(sw + nb);
                    if constexpr (HAS_BIAS) bv = *reinterpret_cast<const float4 *>(bias + nb);
                }
                store4<OUT, HAS_BIAS>(Y, (int64_t)m * N + nb, acc[i][j], q, sxm, swv, bv);
            }
        }
    }
}

template <int OUT, bool HAS_BIAS>
hipError_t launch_t(const int8_t *qx, const int8_t *qw, const float *sx,
                    const float *sw, const float *bias, void *Y, int64_t M,
                    int64_t N, int64_t K, hipStream_t stream)
{
    const int tiles_m = (int)((M + kTile - 1) / kTile);
    const int tiles_n = (int)((N + kTile - 1) / kTile);
    const int tiles = tiles_m * tiles_n;
    const int per_xcd = (tiles + 7) / 8;
    hipLaunchKernelGGL((gemm_i8_kernel<OUT, HAS_BIAS>), dim3(8 * per_xcd), dim3(kThreads), 0,
                       stream, qx, qw, sx, sw, bias, Y, (int)M, (int)N, (int)K, tiles_m,
                       tiles_n, per_xcd);
    return hipGetLastError();
}

} // namespace

hipError_t launch_gemm_i8(const int8_t *qx, const int8_t *qw, const float *sx,
                          const float *sw, const float *bias, void *Y,
                          OutKind out, int64_t M, int64_t N, int64_t K,
                          hipStream_t stream)
{
    if (M == 0 || N == 0) return hipSuccess;
    const bool hb = bias != nullptr;
    switch (out) {
    case OutKind::I32:
        return launch_t<int(OutKind::I32), false>(qx, qw, sx, sw, bias, Y, M, N, K, stream);
    case OutKind::F32:
        return hb ? launch_t<int(OutKind::F32), true>(qx, qw, sx, sw, bias, Y, M, N, K, stream)
                  : launch_t<int(OutKind::F32), false>(qx, qw, sx, sw, bias, Y, M, N, K, stream);
    case OutKind::BF16:
        return hb ? launch_t<int(OutKind::BF16), true>(qx, qw, sx, sw, bias, Y, M, N, K, stream)
                  : launch_t<int(OutKind::BF16), false>(qx, qw, sx, sw, bias, Y, M, N, K, stream);
    case OutKind::GELU_BF16:
        return hb ? launch_t<int(OutKind::GELU_BF16), true>(qx, qw, sx, sw, bias, Y, M, N, K, stream)
                  : launch_t<int(OutKind::GELU_BF16), false>(qx, qw, sx, sw, bias, Y, M, N, K, stream);
    }
    return hipErrorInvalidValue;
}

} // namespace convrot
