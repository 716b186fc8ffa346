// Measurement probes: the ceilings the benchmark prints beside the spec
// peaks.  They compute nothing of the method.
//
//  - mfma_i8_probe: the INT8 matrix-core rate when the operands change every
//    round, as they do in a GEMM on real data.  The clock under a sustained
//    INT8 MFMA load is power-limited, and random operands draw more power
//    than constant ones, so this rate, not 5.0 POP/s, is what a GEMM can
//    approach on this part.
//  - stream_probe: a streaming kernel with the rotate+quantise traffic shape
//    (16 bytes read, 8 written per item), a plain 16-byte copy, or writes
//    only (the traffic of a GEMM whose output dominates), with no arithmetic:
//    what HBM delivers to that access pattern.
#include "common.hpp"

#include <algorithm>

namespace convrot {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kProbeThreads = 256;
constexpr int kSeedInts = 1024;        // 4 KiB of seed

// Each wave holds 4 A and 4 B fragments of 16 bytes per lane and runs 4 x 4
// v_mfma_i32_32x32x32_i8 per round into 256 accumulators; after each round
// the fragments are remixed (xor of each other), so every MFMA sees operands
// it has not seen before.
__global__ __launch_bounds__(kProbeThreads, 1) void mfma_i8_probe(int64_t iters,
                                                                  const int *__restrict__ seed,
                                                                  int *__restrict__ sink)
{
    const int t = blockIdx.x * kProbeThreads + threadIdx.x;
    v4i a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a[i][e] = seed[(t * 32 + i * 4 + e) % kSeedInts];
            b[i][e] = seed[(t * 32 + 16 + i * 4 + e) % kSeedInts];
        }
    }
    v16i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const v4i na = a[i] ^ b[(i + 1) & 3];
            const v4i nb = b[i] ^ a[(i + 2) & 3];
            a[i] = na;
            b[i] = nb;
        }
    }
    int k = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) k ^= acc[i][j][0] ^ acc[i][j][9];
    if (k == 0x5eed5eed) sink[threadIdx.x & 3] = k;   // keeps the work alive
}

// Grid-stride streaming: item i reads 16 bytes of src (non-temporal) and
// writes 8 (MODE 0: two xors of the input words) or all 16 bytes (MODE 1) to
// dst; MODE 2 reads nothing and writes the item index to all 16 bytes.
template <int MODE>
__global__ __launch_bounds__(kProbeThreads) void stream_probe(const v4i *__restrict__ src,
                                                              void *__restrict__ dst, int64_t n16)
{
    const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
    for (int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x; i < n16; i += stride) {
        if constexpr (MODE == 2) {
            const int lo = (int)i;
            static_cast<v4i *>(dst)[i] = (v4i){lo, lo, lo, lo};
            continue;
        }
        const v4i d = __builtin_nontemporal_load(&src[i]);
        if constexpr (MODE == 0) {
            v2i o;
            o[0] = d[0] ^ d[1];
            o[1] = d[2] ^ d[3];
            static_cast<v2i *>(dst)[i] = o;
        } else {
            static_cast<v4i *>(dst)[i] = d;
        }
    }
}

} // namespace

int64_t probe_mfma_i8_ops(int64_t iters)
{
    return (int64_t)device_cu_count() * (kProbeThreads / 64) * iters * 16 * 65536;
}

hipError_t launch_probe_mfma_i8(int64_t iters, const int *seed, int *sink, hipStream_t stream)
{
    hipLaunchKernelGGL(mfma_i8_probe, dim3(device_cu_count()), dim3(kProbeThreads), 0, stream,
                       iters, seed, sink);
    return hipGetLastError();
}

hipError_t launch_probe_stream(const void *src, void *dst, int64_t n16, int mode,
                               hipStream_t stream)
{
    if (n16 == 0) return hipSuccess;
    // 64 workgroups per CU, each thread walking items a grid apart
    const int64_t blocks = std::min<int64_t>((int64_t)device_cu_count() * 64,
                                             (n16 + kProbeThreads - 1) / kProbeThreads);
    const auto s = static_cast<const v4i *>(src);
    if (mode == 0)
        hipLaunchKernelGGL(stream_probe<0>, dim3((unsigned)blocks), dim3(kProbeThreads), 0,
                           stream, s, dst, n16);
    else if (mode == 1)
        hipLaunchKernelGGL(stream_probe<1>, dim3((unsigned)blocks), dim3(kProbeThreads), 0,
                           stream, s, dst, n16);
    else
        hipLaunchKernelGGL(stream_probe<2>, dim3((unsigned)blocks), dim3(kProbeThreads), 0,
                           stream, s, dst, n16);
    return hipGetLastError();
}

} // namespace convrot
