// INT8 x INT8 -> INT32 GEMM on gfx950 matrix cores with a fused dequant
// epilogue:  Y[m, n] = ((float)acc[m, n] * s_x[m]) * s_w[n] (+ bias[n]).
//
// The contraction is the W8A8 projection of a ConvRot linear (lehuy.net
// article on HyperFlow H3 Flash, "Cach nen hoat dong"; the mmh3turbo README,
// "Why it is fast, and where it is not", reports it for K = 5376).  The scales
// are per token (s_x) and per output channel (s_w; PulpCut input-major README,
// "Input-major checkpoint").
//
// Operands: qx [M, K] and qw [N, K], both in the library's K-tiled code
// layout (blocks of 16 rows stored as 1 KiB tiles of 16 rows x 64 B, chunk c
// of row r at slot c ^ ((r >> 2) & 3)), so each MFMA lane reads 16
// consecutive bytes of one row for either operand.
//
// Tiling: a 256-thread workgroup (4 waves, one per SIMD) owns a 256 (n) x 256
// (m) output tile; wave (wn, wm) owns 128 x 128 of it as 4 x 4 tiles of
// v_mfma_i32_32x32x32_i8 (256 int32 accumulators per lane, held in AGPRs).
// The weight tile is the MFMA A operand (rows = n) and the activation tile
// the B operand (columns = m), so an accumulator lane holds 4 consecutive n of
// one m; in the bf16 epilogue lane pairs exchange halves with
// v_permlane32_swap so that every lane stores 16 contiguous bytes.
//
// Persistent schedule: one workgroup per CU walks a sequence of tiles, and the
// copy stream runs on across tile boundaries, so the next tile's first
// K-tiles land while the current one is dequantised and stored.
//
// K pipeline: K advances 64 bytes per K-tile; S stages of 32 KiB (W and X
// tiles, 256 rows x 64 B each) live in LDS.  Global -> LDS copies use the
// direct-to-LDS buffer load (buffer_load_dwordx4 ... lds: each lane fetches
// 16 bytes and the wave's 1 KiB lands contiguously in LDS), so no registers
// stage the tiles and no LDS write instructions are issued.  In the K-tiled
// layout one copy instruction moves one 16-row tile, a contiguous 1 KiB.  The
// copies of each K-tile are split over the two halves of a step and spread
// between the MFMAs, which keeps the texture-address queue from filling.
// Every wait on a copy is explicit: s_waitcnt vmcnt(n) for this wave's
// copies, then a barrier for the other waves'.
//
// LDS rows are 64 bytes; chunk c (16 B) of tile row r sits at slot
// c ^ f(r), f(r) = (r >> 2) & 3, as in the global layout.  The fragment
// reads (ds_read_b128 of 32 rows x one chunk per half-wave) then run without
// bank conflicts on gfx950: measured with SQ_LDS_BANK_CONFLICT, they take the
// 4 cycles of a linear read, where f(r) = ((r >> 1) ^ (r >> 3)) & 3 took 8
// and no swizzle 16.  Copies of 16 half cache lines per instruction (row-major
// operands) moved half as many bytes per cycle as the contiguous 1 KiB tiles.
//
// Workgroups are renumbered so each of the 8 XCDs walks a contiguous range of
// tiles, grouped 4 tile-rows high, for L2 reuse of both operands (4 rows
// fetch 30% fewer L2 lines than 8 at K = 5376, measured with TCC_EA0_RDREQ).
//
// Also in this file, on the same K loop:
//  - 256 (n) x 128 (m) tiles (TJ = 2), launched for the last tile-rows when
//    a round of 256 x 256 tiles would leave CUs idle (launch_t);
//  - the bf16 x bf16 product of the low-rank comparison variant
//    (OutKind::BF16_MM: v_mfma_f32_32x32x16_bf16, row-major operands);
//  - the low-rank factor 1 with the rotation and requantisation of its
//    output in the epilogue (lowrank_f1_kernel);
//  - the bf16 GELU table of the MLP's up projection, whose epilogue reads the
//    slice with |u| in [2^-31, 2^9) from LDS (20 KiB beside the stages);
//  - the SwiGLU fc1 epilogue (OutKind::SWIGLU_BF16), reading the fp32 silu
//    table's slice with |gate| in [2^-15, 2^8) from LDS (23 KiB).
#include "common.hpp"

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <utility>

namespace convrot {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kTile = 256;     // tile edge in n (and in m for TJ = 4)
constexpr int kBK = 64;        // K bytes per LDS stage
constexpr int kThreads = 256;
constexpr int kGroup = 4;      // tile-rows per L2 group
// buffer resource word 3: raw (untyped) 32-bit data format, no swizzle
constexpr int kRsrcWord3 = 0x00020000;
// rint(t) for |t| < 2^22 lands in the low bits of t + 1.5 * 2^23
constexpr float kMagicRint = 12582912.0f;

__device__ __forceinline__ int swz(int r) { return (r >> 2) & 3; }

// s_waitcnt vmcnt(n) with expcnt/lgkmcnt left unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// s_waitcnt lgkmcnt(0) with vmcnt/expcnt left unconstrained.
__device__ __forceinline__ void wait_lds_reads()
{
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Scheduling-group masks (LLVM AMDGPU sched_group_barrier).
constexpr int kSgMfma = 0x008, kSgVmemRead = 0x020, kSgDsRead = 0x100;

// Order the current scheduling region so that LDS reads and global->LDS
// copies trickle out between matrix instructions instead of blocking issue in
// bursts: the reads take every other MFMA slot from the first, the copies are
// spread evenly from the first slot on, so neither the LDS nor the
// texture-address queue sees the whole wave's requests at once.  (Copies
// spread from the first slot rather than ending at the last gave 0.5-0.9%
// at K = 512, 5376 and 21504: each copy gets a little longer to land.)
template <int MFMAS, int VMEMS, int DSREADS, int K>
__device__ __forceinline__ void interleave_slot()
{
    // reads [RD_LO, RD_HI) and copies [VM_LO, VM_HI) follow MFMA slot K
    constexpr int RD_LO = (K * DSREADS + MFMAS - 1) / MFMAS;
    constexpr int RD_HI = ((K + 1) * DSREADS + MFMAS - 1) / MFMAS;
    constexpr int VM_LO = (K * VMEMS + MFMAS - 1) / MFMAS;
    constexpr int VM_HI = ((K + 1) * VMEMS + MFMAS - 1) / MFMAS;
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
    if constexpr (RD_HI > RD_LO) __builtin_amdgcn_sched_group_barrier(kSgDsRead, RD_HI - RD_LO, 0);
    if constexpr (VM_HI > VM_LO) __builtin_amdgcn_sched_group_barrier(kSgVmemRead, VM_HI - VM_LO, 0);
}

template <int MFMAS, int VMEMS, int DSREADS, int... K>
__device__ __forceinline__ void interleave_all(std::integer_sequence<int, K...>)
{
    (interleave_slot<MFMAS, VMEMS, DSREADS, K>(), ...);
}

template <int MFMAS, int VMEMS, int DSREADS>
__device__ __forceinline__ void interleave()
{
    interleave_all<MFMAS, VMEMS, DSREADS>(std::make_integer_sequence<int, MFMAS>{});
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 with v_cvt_pk_bf16_f32 (round to nearest even).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi)
{
    const bf16x2 p = __builtin_convertvector((f32x2){lo, hi}, bf16x2);
    return __builtin_bit_cast(uint32_t, p);
}


// Dequantise and store a wave's 128 x 128 block.  FULL: the tile lies inside
// [M, N], so no per-lane bounds checks are needed.
// fp32 value of one output: ((float)acc * s_x) * s_w (+ bias).
// For the bf16 x bf16 product (OutKind::BF16_MM) the accumulator already
// holds the fp32 sum: y = acc (+ bias).
template <int OUT, bool HAS_BIAS>
__device__ __forceinline__ float dequant1(int acc, float sxm, float swn, float bn)
{
    float f;
    if constexpr (OUT == int(OutKind::BF16_MM))
        f = __int_as_float(acc);
    else
        f = __fmul_rn(__fmul_rn((float)acc, sxm), swn);
    if constexpr (HAS_BIAS) f = __fadd_rn(f, bn);
    return f;
}

// bf16(GELU(u)) for every bf16 bit pattern u: GELU in its erf form,
// 0.5 z (1 + erf(z / sqrt 2)), evaluated in fp64 on the bf16 value z of the
// up projection's output, then rounded to fp32 and to bf16 (round to nearest
// even both times).  The MLP's up projection looks its outputs up here
// instead of evaluating erf per element.  The table is written once per device
// (launch_gelu_table): the first call of a GELU path that is not being
// recorded into a graph fills it on its stream and waits for the fill, and
// every later launch on any stream reads the finished table.  A call recorded
// into a graph before that records the fill too, and each replay rewrites the
// table with the same values.
__device__ __align__(16) uint16_t g_gelu_bf16[65536];

__global__ __launch_bounds__(256) void gelu_table_kernel()
{
    const uint32_t u = blockIdx.x * 256u + threadIdx.x;
    const double z = (double)__uint_as_float(u << 16);
    const double gd = 0.5 * z * (1.0 + erf(z / sqrt(2.0)));
    g_gelu_bf16[u] = (uint16_t)f32_to_bf16_bits((float)gd);
}

// g[i] = bf16(GELU(u[i])) through the same table (the elementwise form the
// MLP entry point applies inside its up projection).
__global__ __launch_bounds__(256) void gelu_apply_kernel(const uint16_t *__restrict__ u,
                                                         uint16_t *__restrict__ g, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) g[i] = g_gelu_bf16[u[i]];
}

__device__ __forceinline__ uint32_t gelu_pair(uint32_t u2)
{
    return (uint32_t)g_gelu_bf16[u2 & 0xffffu] | ((uint32_t)g_gelu_bf16[u2 >> 16] << 16);
}

// The slice of that table the GEMM epilogue reads from LDS: for each sign the
// patterns with |u| in [2^-31, 2^9), i.e. biased exponents 96..135 (40 x 128
// entries, 10 KiB per sign).  Gathers from LDS cost a fraction of gathers
// through the texture path; a 32-row slab in which any |u| falls outside the
// slice (zero, tiny, huge, inf, NaN) is patched from the full table.
constexpr int kGeluLo = 96 * 128;      // first |u| pattern of the slice
constexpr int kGeluSpan = 40 * 128;    // patterns per sign
__shared__ uint16_t g_gelu_lds[2 * kGeluSpan];

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Offsets of both halves' |u| from the slice start (wrapping below it): a
// half is inside the slice iff its offset is < kGeluSpan.
__device__ __forceinline__ u16x2 gelu_slice_off(uint32_t u2)
{
    return (__builtin_bit_cast(u16x2, u2) & (u16x2)(0x7fff)) - (u16x2)(kGeluLo);
}

// Both halves from the LDS slice (an index clamped into it when outside);
// mx collects the largest offset seen, so that mx < kGeluSpan in both halves
// means every lookup was inside the slice.
__device__ __forceinline__ uint32_t gelu_pair_lds(uint32_t u2, u16x2 &mx)
{
    const u16x2 d = gelu_slice_off(u2);
    mx = __builtin_elementwise_max(mx, d);
    const u16x2 idx = (__builtin_bit_cast(u16x2, u2) >> (u16x2)(15)) * (u16x2)(kGeluSpan) +
                      __builtin_elementwise_min(d, (u16x2)(kGeluSpan - 1));
    return (uint32_t)g_gelu_lds[idx.x] | ((uint32_t)g_gelu_lds[idx.y] << 16);
}

// g = bf16(GELU(u)) for 8 consecutive values per thread (one 16-byte load
// and store), from the LDS slice of the table; a thread holding a value
// outside the slice redoes its 8 values from the full table.  Grid-stride
// over n8 groups; each workgroup fills its LDS slice once.
__global__ __launch_bounds__(256) void gelu_apply8_kernel(const uint4 *__restrict__ u,
                                                          uint4 *__restrict__ g, int64_t n8)
{
    for (int i = threadIdx.x; i < 2 * kGeluSpan; i += 256) {
        const int neg = i >= kGeluSpan;
        g_gelu_lds[i] = g_gelu_bf16[(neg << 15) | (i - neg * kGeluSpan + kGeluLo)];
    }
    __syncthreads();
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += stride) {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(u) + i);
        u16x2 mx = (u16x2)(0);
        uint4 o;
        o.x = gelu_pair_lds(x[0], mx);
        o.y = gelu_pair_lds(x[1], mx);
        o.z = gelu_pair_lds(x[2], mx);
        o.w = gelu_pair_lds(x[3], mx);
        if (mx.x >= kGeluSpan || mx.y >= kGeluSpan) {
            o.x = gelu_pair(x[0]);
            o.y = gelu_pair(x[1]);
            o.z = gelu_pair(x[2]);
            o.w = gelu_pair(x[3]);
        }
        g[i] = o;
    }
}

// Dequantise and store a wave's 128 (n) x 32 TJ (m) block.  FULL: the tile
// lies inside [M, N], so no per-lane bounds checks are needed.
//
// Accumulator layout: lane (l32, g) holds, for sub-tile (i, j) and q = 0..3,
// n = 32 i + 8 q + 4 g + 0..3 of row m = 32 j + l32.  For bf16 outputs the two
// lanes of a row exchange halves with v_permlane32_swap so that each holds
// 8 consecutive columns (16 bytes): the lower lane n = 32 i + 16 p + 0..7, the
// upper lane + 8..15, for q = 2p, 2p + 1.  Rows are the outer loop so the
// 16-byte stores of one 128-byte line leave back to back.
// Copy one accumulator fragment from AGPRs to VGPRs where it is used.  Left
// to itself the compiler copies the whole tile at once after the K loop
// (the values cross basic blocks), which does not fit in 256 VGPRs.
__device__ __forceinline__ v16i acc_frag(const v16i &a)
{
    v16i v;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        int x;
        asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(x) : "a"(a[e]));
        v[e] = x;
    }
    return v;
}

// GELU epilogue, one 32-row slab j of a wave's block: dequantise, round to
// bf16 and look up bf16(GELU(u)) for its 4 x 32 columns in the LDS slice; if
// any lane met a |u| outside it, recompute those pairs from the full table ...
template <int OUT, bool HAS_BIAS, int TJ, int J>
__device__ __forceinline__ void gelu_lookup(const v16i (&acc)[4][TJ],
                                            const float (&sscale)[3][kTile], int wm, int wn,
                                            int l32, int g, uint32_t (&gv)[4][2][2][2])
{
    const int ml = wm * 32 * TJ + 32 * J + l32;
    const float sxm = sscale[0][ml];
    // packed bf16 u of columns 4q .. 4q + 3 of fragment i (two dwords)
    auto u_pair = [&](const v16i &av, int i, int q, int half) {
        const int nl = wn * 128 + 32 * i + 8 * q + 4 * g;
        const float4 swv = *reinterpret_cast<const float4 *>(&sscale[1][nl]);
        const float4 bv = *reinterpret_cast<const float4 *>(&sscale[2][nl]);
        return half == 0 ? cvt_pk_bf16(dequant1<OUT, HAS_BIAS>(av[4 * q + 0], sxm, swv.x, bv.x),
                                       dequant1<OUT, HAS_BIAS>(av[4 * q + 1], sxm, swv.y, bv.y))
                         : cvt_pk_bf16(dequant1<OUT, HAS_BIAS>(av[4 * q + 2], sxm, swv.z, bv.z),
                                       dequant1<OUT, HAS_BIAS>(av[4 * q + 3], sxm, swv.w, bv.w));
    };
    u16x2 mx = (u16x2)(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const v16i av = acc_frag(acc[i][J]);
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                gv[i][p][h][0] = gelu_pair_lds(u_pair(av, i, 2 * p + h, 0), mx);
                gv[i][p][h][1] = gelu_pair_lds(u_pair(av, i, 2 * p + h, 1), mx);
            }
    }
    const bool outside = mx.x >= kGeluSpan || mx.y >= kGeluSpan;
    if (__builtin_amdgcn_ballot_w64(outside)) {
        // rare: only the pairs with a half outside the slice gather from the
        // full table (the others keep their LDS results)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const v16i av = acc_frag(acc[i][J]);
#pragma unroll
            for (int p = 0; p < 2; ++p)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int d = 0; d < 2; ++d) {
                        const uint32_t u2 = u_pair(av, i, 2 * p + h, d);
                        const u16x2 o = gelu_slice_off(u2);
                        if (o.x >= kGeluSpan || o.y >= kGeluSpan) gv[i][p][h][d] = gelu_pair(u2);
                    }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
}

// ... and store them, 16 contiguous bytes per lane (as the bf16 epilogue).
template <int TJ, bool FULL, int J>
__device__ __forceinline__ void gelu_store(void *Y, const uint32_t (&gv)[4][2][2][2], int M,
                                           int N, int m0, int n0, int wm, int wn, int l32,
                                           int g)
{
    const int m = m0 + wm * 32 * TJ + 32 * J + l32;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const auto s0 = __builtin_amdgcn_permlane32_swap(gv[i][p][0][0], gv[i][p][1][0],
                                                             false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(gv[i][p][0][1], gv[i][p][1][1],
                                                             false, false);
            const int nb = n0 + wn * 128 + 32 * i + 16 * p + 8 * g;
            if (!FULL && (m >= M || nb >= N)) continue;
            uint4 o;
            o.x = s0[0]; o.y = s1[0]; o.z = s0[1]; o.w = s1[1];
            *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(Y) + (int64_t)m * N + nb) = o;
        }
    __builtin_amdgcn_sched_barrier(0);
}

// SwiGLU epilogue (MiniMax-H3-Rung-Omega README, "Technical Architecture
// Overview", Floor 1: SwiGLU in front of the rotated, rowwise quantised fc2),
// fused into fc1: the fc1 weight rows come in 32-row blocks of 16 gate rows
// followed by their 16 up rows (swiglu_src_row), so in each 32-row fragment
// lane (l32, g) holds, for token m, gate rows 8q + 4g + r and the matching up
// rows 16 + 8q + 4g + r (q = 0, 1; r = 0..3).  Both are dequantised and
// rounded to bf16 (the fc1 output), then g = bf16(fp32(silu(gate)) * up) is
// formed and only g [M, N/2] is written: 16 columns per fragment, after a
// v_permlane32_swap 8 consecutive ones (16 bytes) per lane.
//
// fp32(silu) comes from the LDS slice of the silu table with |gate| in
// [2^-15, 2^8) (biased exponents 112..134, 11.5 KiB per sign, beside the 128
// KiB of stages); a gate outside it (rare: tiny or huge, zero, inf, NaN) is
// looked up in the full table in memory.
constexpr int kSiluLoE = 112 << 7;     // first |gate| pattern of the slice
constexpr int kSiluSpanE = 23 << 7;    // patterns per sign
__shared__ float g_silu_lds[2 * kSiluSpanE];

template <bool HAS_BIAS, int TJ, bool FULL>
__device__ __forceinline__ void swiglu_epilogue(void *Y, const v16i (&acc)[4][TJ],
                                                const float (&sscale)[3][kTile],
                                                const float *__restrict__ silu_tab, int M,
                                                int N, int m0, int n0, int wm, int wn, int l32,
                                                int g)
{
    const int F = N >> 1;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
        const int ml = wm * 32 * TJ + 32 * j + l32;
        const int m = m0 + ml;
        if (!FULL && m >= M) continue;
        const float sxm = sscale[0][ml];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int nf = n0 + wn * 128 + 32 * i;       // first packed row of the fragment
            if (!FULL && nf >= N) continue;
            const v16i av = acc_frag(acc[i][j]);
            // the fc1 outputs of this lane as packed bf16: [q][dword]
            uint32_t pk[4][2];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int nl = wn * 128 + 32 * i + 8 * q + 4 * g;
                const float4 swv = *reinterpret_cast<const float4 *>(&sscale[1][nl]);
                const float4 bv = *reinterpret_cast<const float4 *>(&sscale[2][nl]);
                pk[q][0] = cvt_pk_bf16(
                    dequant1<int(OutKind::BF16), HAS_BIAS>(av[4 * q + 0], sxm, swv.x, bv.x),
                    dequant1<int(OutKind::BF16), HAS_BIAS>(av[4 * q + 1], sxm, swv.y, bv.y));
                pk[q][1] = cvt_pk_bf16(
                    dequant1<int(OutKind::BF16), HAS_BIAS>(av[4 * q + 2], sxm, swv.z, bv.z),
                    dequant1<int(OutKind::BF16), HAS_BIAS>(av[4 * q + 3], sxm, swv.w, bv.w));
            }
            // fp32 silu of the 8 gates (q = 0, 1), from the LDS slice
            float sv[2][4];
            bool outside = false;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t a = (pk[h][e >> 1] >> (16 * (e & 1))) & 0xffffu;
                    const uint32_t off = (a & 0x7fffu) - (uint32_t)kSiluLoE;
                    outside |= off >= (uint32_t)kSiluSpanE;
                    sv[h][e] = g_silu_lds[(a >> 15) * kSiluSpanE +
                                          min(off, (uint32_t)kSiluSpanE - 1u)];
                }
            if (__builtin_amdgcn_ballot_w64(outside)) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t a = (pk[h][e >> 1] >> (16 * (e & 1))) & 0xffffu;
                        if ((a & 0x7fffu) - (uint32_t)kSiluLoE >= (uint32_t)kSiluSpanE)
                            sv[h][e] = silu_tab[a];
                    }
            }
            // g = bf16(s * up), up rows 16 + (the gate's row): q + 2
            uint32_t d[2][2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t u0 = pk[h + 2][0], u1 = pk[h + 2][1];
                d[h][0] = cvt_pk_bf16(__fmul_rn(sv[h][0], __uint_as_float(u0 << 16)),
                                      __fmul_rn(sv[h][1], __uint_as_float(u0 & 0xffff0000u)));
                d[h][1] = cvt_pk_bf16(__fmul_rn(sv[h][2], __uint_as_float(u1 << 16)),
                                      __fmul_rn(sv[h][3], __uint_as_float(u1 & 0xffff0000u)));
            }
            // lower lanes' q = 1 half <-> upper lanes' q = 0 half: lane g then
            // holds columns 8 g .. 8 g + 7 of the fragment's 16
            const auto s0 = __builtin_amdgcn_permlane32_swap(d[0][0], d[1][0], false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(d[0][1], d[1][1], false, false);
            uint4 o;
            o.x = s0[0]; o.y = s1[0]; o.z = s0[1]; o.w = s1[1];
            *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(Y) + (int64_t)m * F +
                                       (nf >> 1) + 8 * g) = o;
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

template <int OUT, bool HAS_BIAS, int TJ, bool FULL>
__device__ __forceinline__ void epilogue(void *Y, const v16i (&acc)[4][TJ],
                                         const float (&sscale)[3][kTile], int M, int N,
                                         int m0, int n0, int wm, int wn, int l32, int g)
{
    if constexpr (OUT == int(OutKind::GELU_BF16)) {
        // GELU outputs, 32 rows at a time: the table lookups of the next
        // rows are issued before the stores of the current ones, so waiting
        // for a lookup never waits for a store.
        uint32_t ga[4][2][2][2], gb[4][2][2][2];   // [i][p][q - 2p][dword]
        gelu_lookup<OUT, HAS_BIAS, TJ, 0>(acc, sscale, wm, wn, l32, g, ga);
        gelu_lookup<OUT, HAS_BIAS, TJ, 1>(acc, sscale, wm, wn, l32, g, gb);
        gelu_store<TJ, FULL, 0>(Y, ga, M, N, m0, n0, wm, wn, l32, g);
        if constexpr (TJ == 4) {
            gelu_lookup<OUT, HAS_BIAS, TJ, 2>(acc, sscale, wm, wn, l32, g, ga);
            gelu_store<TJ, FULL, 1>(Y, gb, M, N, m0, n0, wm, wn, l32, g);
            gelu_lookup<OUT, HAS_BIAS, TJ, 3>(acc, sscale, wm, wn, l32, g, gb);
            gelu_store<TJ, FULL, 2>(Y, ga, M, N, m0, n0, wm, wn, l32, g);
            gelu_store<TJ, FULL, 3>(Y, gb, M, N, m0, n0, wm, wn, l32, g);
        } else {
            gelu_store<TJ, FULL, 1>(Y, gb, M, N, m0, n0, wm, wn, l32, g);
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
        const int ml = wm * 32 * TJ + 32 * j + l32;
        const int m = m0 + ml;
        if (!FULL && m >= M) continue;
        const float sxm = (OUT == int(OutKind::I32)) ? 0.0f : sscale[0][ml];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const v16i av = OUT == int(OutKind::I32) ? acc[i][j] : acc_frag(acc[i][j]);
            if constexpr (OUT == int(OutKind::I32) || OUT == int(OutKind::F32)) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int nl = wn * 128 + 32 * i + 8 * q + 4 * g;
                    const int nb = n0 + nl;
                    if (!FULL && nb >= N) continue;
                    const int64_t off = (int64_t)m * N + nb;
                    if constexpr (OUT == int(OutKind::I32)) {
                        int4 o;
                        o.x = acc[i][j][4 * q + 0]; o.y = acc[i][j][4 * q + 1];
                        o.z = acc[i][j][4 * q + 2]; o.w = acc[i][j][4 * q + 3];
                        *reinterpret_cast<int4 *>(reinterpret_cast<int32_t *>(Y) + off) = o;
                    } else {
                        const float4 swv = *reinterpret_cast<const float4 *>(&sscale[1][nl]);
                        const float4 bv = *reinterpret_cast<const float4 *>(&sscale[2][nl]);
                        float4 o;
                        o.x = dequant1<OUT, HAS_BIAS>(av[4 * q + 0], sxm, swv.x, bv.x);
                        o.y = dequant1<OUT, HAS_BIAS>(av[4 * q + 1], sxm, swv.y, bv.y);
                        o.z = dequant1<OUT, HAS_BIAS>(av[4 * q + 2], sxm, swv.z, bv.z);
                        o.w = dequant1<OUT, HAS_BIAS>(av[4 * q + 3], sxm, swv.w, bv.w);
                        *reinterpret_cast<float4 *>(reinterpret_cast<float *>(Y) + off) = o;
                    }
                }
            } else {
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    uint32_t d[2][2];   // [q - 2p][dword]
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int q = 2 * p + h;
                        const int nl = wn * 128 + 32 * i + 8 * q + 4 * g;
                        const float4 swv = *reinterpret_cast<const float4 *>(&sscale[1][nl]);
                        const float4 bv = *reinterpret_cast<const float4 *>(&sscale[2][nl]);
                        d[h][0] = cvt_pk_bf16(
                            dequant1<OUT, HAS_BIAS>(av[4 * q + 0], sxm, swv.x, bv.x),
                            dequant1<OUT, HAS_BIAS>(av[4 * q + 1], sxm, swv.y, bv.y));
                        d[h][1] = cvt_pk_bf16(
                            dequant1<OUT, HAS_BIAS>(av[4 * q + 2], sxm, swv.z, bv.z),
                            dequant1<OUT, HAS_BIAS>(av[4 * q + 3], sxm, swv.w, bv.w));
                    }
                    // upper lanes' q = 2p half <-> lower lanes' q = 2p + 1 half
                    const auto s0 = __builtin_amdgcn_permlane32_swap(d[0][0], d[1][0], false, false);
                    const auto s1 = __builtin_amdgcn_permlane32_swap(d[0][1], d[1][1], false, false);
                    const int nb = n0 + wn * 128 + 32 * i + 16 * p + 8 * g;
                    if (!FULL && nb >= N) continue;
                    uint4 o;
                    o.x = s0[0]; o.y = s1[0]; o.z = s0[1]; o.w = s1[1];
                    *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(Y) +
                                               (int64_t)m * N + nb) = o;
                }
            }
            // keep the scheduler from hoisting every accumulator read and
            // scale load of the tile, which would not fit in registers
            __builtin_amdgcn_sched_barrier(0);
        }
    }

}

// Copies of one tile go through buffer resources whose base is the tile's
// first row and whose size ends at the matrix's last row, so rows past the end
// are out of range and read as zero (they only feed outputs that are never
// stored).  Per lane, the offset within a tile is the same for both operands
// and for every tile: copy j of wave w moves rows [(4w + j) 16, +16) x 64 B,
// and lane i takes row + i/4 and the chunk that belongs in slot i & 3 of it.
struct TileSrc {
    __amdgpu_buffer_rsrc_t w, x;
};

template <bool RM = false>
__device__ __forceinline__ TileSrc tile_src(const int8_t *qw, const int8_t *qx, int m0, int n0,
                                            int M, int N, int K)
{
    TileSrc t;
    t.w = __builtin_amdgcn_make_buffer_rsrc((void *)(qw + (int64_t)n0 * K), (short)0,
                                            (N - n0) * K, kRsrcWord3);
    // rows up to the 16-row padding: the last block's tiles hold real rows
    // throughout its K range
    t.x = __builtin_amdgcn_make_buffer_rsrc((void *)(qx + (int64_t)m0 * K), (short)0,
                                            (int)((RM ? M : padded_rows(M)) - m0) * K,
                                            kRsrcWord3);
    return t;
}

// The copy source after a workgroup's last tile: empty ranges, so the copies
// the pipeline issues ahead for a next tile read zeros without memory
// traffic (their LDS stages are never read).
__device__ __forceinline__ TileSrc empty_src(const int8_t *qw, const int8_t *qx)
{
    TileSrc t;
    t.w = __builtin_amdgcn_make_buffer_rsrc((void *)qw, (short)0, 0, kRsrcWord3);
    t.x = __builtin_amdgcn_make_buffer_rsrc((void *)qx, (short)0, 0, kRsrcWord3);
    return t;
}

// Copy j of wave w moves rows [(n w + j) 16, +16) of an operand tile of 64 n
// rows (n = 4 for the 256-row weight tile, TJ for the activation tile): the
// 1 KiB tile of that row block, lane i its i-th 16 bytes.
// RM: row-major operands (the bf16 product): lane i takes row + i/4 and the
// 16-byte chunk (i & 3) ^ f(row) of it, so the LDS tile has the same layout.
template <bool RM = false, int NC>
__device__ __forceinline__ void lane_offsets(int K, int wave, int lane, uint32_t (&voff)[NC])
{
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        if constexpr (RM) {
            const int r = (wave * NC + j) * 16 + (lane >> 2);
            voff[j] = (uint32_t)r * (uint32_t)K + (((lane & 3) ^ swz(r)) << 4);
        } else {
            voff[j] = (uint32_t)((wave * NC + j) * 16) * (uint32_t)K + (uint32_t)lane * 16u;
        }
    }
}

// Half H of K-tile `k` of the copy stream into one stage: the wave's weight
// copies j = H CW/2 .. (H + 1) CW/2 - 1 and its activation copies
// [0, ceil(CX/2)) in half 0, the rest in half 1.
// Below nk the K-tile belongs to the current tile, from nk on to the next one
// (the last tile of a workgroup re-reads its own first K-tiles, which no one
// consumes).
template <int CW, int CX, int H, bool RM = false>
__device__ __forceinline__ void issue_half(const TileSrc &cur, const TileSrc &nxt,
                                           const uint32_t *voffw, const uint32_t *voffx, int k,
                                           int nk, int wave, int8_t *__restrict__ dst_w,
                                           int8_t *__restrict__ dst_x)
{
    const bool next = k >= nk;
    const __amdgpu_buffer_rsrc_t rw = next ? nxt.w : cur.w, rx = next ? nxt.x : cur.x;
    // K-tile k: of a 16-row block (K-tiled), or 64 bytes along the row
    const int soff = (next ? k - nk : k) * (RM ? kBK : 1024);
#pragma unroll
    for (int j = H * CW / 2; j < (H + 1) * CW / 2; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rw, (__attribute__((address_space(3))) void *)(dst_w + (wave * CW + j) * 1024), 16,
            voffw[j], soff, 0, 0);
#pragma unroll
    for (int j = H ? (CX + 1) / 2 : 0; j < (H ? CX : (CX + 1) / 2); ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rx, (__attribute__((address_space(3))) void *)(dst_x + (wave * CX + j) * 1024), 16,
            voffx[j], soff, 0, 0);
}

template <int TJ>
__device__ __forceinline__ void read_frags(const int8_t *__restrict__ sw_,
                                           const int8_t *__restrict__ sx_, int frow_w,
                                           int frow_x, int foff, v4i (&a)[4], v4i (&b)[TJ])
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = *reinterpret_cast<const v4i *>(sw_ + frow_w + 2048 * i + foff);
        if (i < TJ) b[i] = *reinterpret_cast<const v4i *>(sx_ + frow_x + 2048 * i + foff);
    }
}

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// BF: the operands are bf16 (8 per 16-byte fragment) and the accumulators
// hold fp32 bits (v_mfma_f32_32x32x16_bf16, the same fragment shapes).
template <int TJ, bool BF = false>
__device__ __forceinline__ void mfma_block(v16i (&acc)[4][TJ], const v4i (&a)[4],
                                           const v4i (&b)[TJ])
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            if constexpr (BF)
                acc[i][j] = __builtin_bit_cast(
                    v16i, __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                              __builtin_bit_cast(v8bf, a[i]), __builtin_bit_cast(v8bf, b[j]),
                              __builtin_bit_cast(v16f, acc[i][j]), 0, 0, 0));
            else
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], acc[i][j], 0, 0, 0);
        }
}

template <int S, int I>
__device__ __forceinline__ int8_t *pick(int8_t *p0, int8_t *p1, int8_t *p2, int8_t *p3)
{
    constexpr int k = I % S;
    return k == 0 ? p0 : k == 1 ? p1 : k == 2 ? p2 : p3;
}

template <int N1, int N2>
__device__ __forceinline__ void wait_vmcnt_either(bool second)
{
    if (second) wait_vmcnt<N2>();
    else wait_vmcnt<N1>();
}

// The K loop of one tile, in a stream of tiles.  Each LDS stage is a separate
// object reached through its own restrict pointer, and the loop is unrolled
// by the stage count so every access names its stage at compile time: the
// compiler then proves that an LDS read of one stage does not depend on copies
// still landing in another and only waits for copies into the stage read.
// Waiting for the other waves' copies is explicit: each wave retires its own
// copies of the next K-tile, then all meet at a barrier.
//
// Step k (K-tile k, stage k % S) runs the MFMAs of its two 32-byte sub-steps.
// Its first half reads the sub-step-1 fragments and copies the second half of
// stream K-tile k + S - 1 into stage (k - 1) % S (free since step k - 1's
// barrier); its second half, after the barrier, reads the next K-tile's
// sub-step-0 fragments and copies the first half of K-tile k + S into stage
// k % S.  Copies of a K-tile are thus issued in stream order, 8 per wave.
//
// On entry: first == true -> nothing is in flight and every stage is free;
// first == false -> K-tiles 0 .. S-2 of this tile are in flight, issued during
// the previous tile, then (EARLY) K-tile S-1, issued by the caller once
// stage S-1 was free, then EPI younger memory operations per wave (the
// previous tile's stores and this tile's scale loads).  Without EARLY, stage
// S-1 is free and K-tile S-1 is issued here, after the EPI operations.
// Issuing it ahead of the stores gives them one more K-step to complete
// before a wait (vmcnt retires in order) has to cover them.
// On exit: K-tiles 0 .. S-2 of the next tile are in flight.  Requires
// nk % S == 0.
template <int TJ, int CW, int CX, int S, int EPI, bool EARLY, bool BF = false>
__device__ __forceinline__ void k_loop(int8_t *__restrict__ w0, int8_t *__restrict__ w1,
                                       int8_t *__restrict__ w2, int8_t *__restrict__ w3,
                                       int8_t *__restrict__ x0, int8_t *__restrict__ x1,
                                       int8_t *__restrict__ x2, int8_t *__restrict__ x3,
                                       const TileSrc &cur, const TileSrc &nxt,
                                       const uint32_t *voffw, const uint32_t *voffx,
                                       int nk, bool first, int wave, int frow_w, int frow_x,
                                       int foff0, int foff1, v16i (&acc)[4][TJ])
{
    static_assert(S == 2 || S == 4, "stages");
    static_assert(TJ == 1 || TJ == 2 || TJ == 4, "activation sub-tiles per wave");
    static_assert(CW % 2 == 0, "weight copies split evenly over two halves");
    constexpr int C = CW + CX;               // copy instructions per wave per K-tile
    constexpr int CH0 = CW / 2 + (CX + 1) / 2, CH1 = C - CH0;   // ... in each half
    constexpr int MF = 4 * TJ, RD = 4 + TJ;  // MFMAs and LDS reads per half
    static_assert((S - 1) * C + EPI < 64, "vmcnt range");
    v4i a0[4], b0[TJ], a1[4], b1[TJ];
    int8_t *const wl = pick<S, S - 1>(w0, w1, w2, w3), *const xl = pick<S, S - 1>(x0, x1, x2, x3);

    if (first) {
        issue_half<CW, CX, 0, BF>(cur, nxt, voffw, voffx, 0, nk, wave, w0, x0);
        issue_half<CW, CX, 1, BF>(cur, nxt, voffw, voffx, 0, nk, wave, w0, x0);
        if constexpr (S == 4) {
            issue_half<CW, CX, 0, BF>(cur, nxt, voffw, voffx, 1, nk, wave, w1, x1);
            issue_half<CW, CX, 1, BF>(cur, nxt, voffw, voffx, 1, nk, wave, w1, x1);
            issue_half<CW, CX, 0, BF>(cur, nxt, voffw, voffx, 2, nk, wave, w2, x2);
            issue_half<CW, CX, 1, BF>(cur, nxt, voffw, voffx, 2, nk, wave, w2, x2);
        }
    }
    if constexpr (EARLY) {
        if (first) {
            issue_half<CW, CX, 0, BF>(cur, nxt, voffw, voffx, S - 1, nk, wave, wl, xl);
            issue_half<CW, CX, 1, BF>(cur, nxt, voffw, voffx, S - 1, nk, wave, wl, xl);
        }
        wait_vmcnt_either<(S - 1) * C + EPI, (S - 1) * C>(first);
    } else {
        issue_half<CW, CX, 0, BF>(cur, nxt, voffw, voffx, S - 1, nk, wave, wl, xl);
        wait_vmcnt_either<(S - 2) * C + CH0 + EPI, (S - 2) * C + CH0>(first);
    }
    block_barrier();
    read_frags(w0, x0, frow_w, frow_x, foff0, a0, b0);

#define CONVROT_STEP(I)                                                                  \
    do {                                                                                 \
        int8_t *pw_ = pick<S, I + S - 1>(w0, w1, w2, w3), *px_ = pick<S, I + S - 1>(x0, x1, x2, x3); \
        int8_t *cw_ = pick<S, I>(w0, w1, w2, w3), *cx_ = pick<S, I>(x0, x1, x2, x3);      \
        int8_t *nw_ = pick<S, I + 1>(w0, w1, w2, w3), *nx_ = pick<S, I + 1>(x0, x1, x2, x3); \
        wait_lds_reads();                                                                \
        __builtin_amdgcn_sched_barrier(0);                                               \
        read_frags(cw_, cx_, frow_w, frow_x, foff1, a1, b1);                              \
        if (!EARLY || (I) != 0 || kt != 0)                                               \
            issue_half<CW, CX, 1, BF>(cur, nxt, voffw, voffx, kt + (I) + S - 1, nk, wave, pw_, px_); \
        mfma_block<TJ, BF>(acc, a0, b0);                                                         \
        interleave<MF, CH1, RD>();                                                         \
        __builtin_amdgcn_sched_barrier(0);                                               \
        wait_lds_reads();                                                                \
        wait_vmcnt_either<(S - 2) * C, (S - 2) * C + EPI>(                               \
            !first && kt + (I) < (EARLY ? S - 1 : S - 2));                               \
        block_barrier();                                                                 \
        read_frags(nw_, nx_, frow_w, frow_x, foff0, a0, b0);                              \
        issue_half<CW, CX, 0, BF>(cur, nxt, voffw, voffx, kt + (I) + S, nk, wave, cw_, cx_);                 \
        mfma_block<TJ, BF>(acc, a1, b1);                                                         \
        interleave<MF, CH0, RD>();                                                         \
        __builtin_amdgcn_sched_barrier(0);                                               \
    } while (0)

    // nk - 1 steps (K-tiles 0 .. nk-2), S at a time, then the rest in line
    int kt = 0;
    for (; kt + S < nk; kt += S) {
        CONVROT_STEP(0);
        CONVROT_STEP(1);
        if constexpr (S == 4) {
            CONVROT_STEP(2);
            CONVROT_STEP(3);
        }
    }
    CONVROT_STEP(0);
    if constexpr (S == 4) {
        CONVROT_STEP(1);
        CONVROT_STEP(2);
    }
#undef CONVROT_STEP
    // K-tile nk - 1: no barrier, nothing to overwrite but stage S - 2
    {
        wait_lds_reads();
        __builtin_amdgcn_sched_barrier(0);
        read_frags(wl, xl, frow_w, frow_x, foff1, a1, b1);
        issue_half<CW, CX, 1, BF>(cur, nxt, voffw, voffx, nk + S - 2, nk, wave, pick<S, S - 2>(w0, w1, w2, w3),
                      pick<S, S - 2>(x0, x1, x2, x3));
        mfma_block<TJ, BF>(acc, a0, b0);
        interleave<MF, CH1, RD>();
        __builtin_amdgcn_sched_barrier(0);
        mfma_block<TJ, BF>(acc, a1, b1);
    }
}

// Persistent GEMM: one 256-thread workgroup per CU walks a sequence of
// 256 (n) x 256 (m) output tiles; wave (wn, wm) computes 128 x 128 of each in
// 256 AGPR accumulators.  The copy stream runs across tile boundaries, so the
// next tile's first K-tiles land while the current one is dequantised and
// stored, and its stores drain while the next tile computes.
// S: LDS stages of 2 x 16 KiB (4 when nk % 4 == 0, else 2).
template <int OUT, bool HAS_BIAS, int TJ, int S>
__global__ __launch_bounds__(kThreads, 1) void gemm_i8_kernel(
    const int8_t *__restrict__ qx, const int8_t *__restrict__ qw,
    const float *__restrict__ sx, const float *__restrict__ sw,
    const float *__restrict__ bias, void *__restrict__ Y, int M, int N, int K,
    int tiles_m, int tiles_n, int tiles_per_xcd, int wgs_per_xcd,
    const float *__restrict__ silu_tab)
{
    constexpr int TM = 64 * TJ;            // tile edge in m
    constexpr int STGW = kTile * kBK;      // 16 KiB of weights per stage
    constexpr int STGX = TM * kBK;         // 16 or 8 KiB of activations per stage
    constexpr bool MM = OUT == int(OutKind::BF16_MM);   // bf16 operands, row-major
    constexpr bool SWIGLU = OUT == int(OutKind::SWIGLU_BF16);
    constexpr bool BF16_OUT =
        OUT == int(OutKind::BF16) || OUT == int(OutKind::GELU_BF16) || MM;
    constexpr int NSCALE = OUT == int(OutKind::I32) ? 0 : MM ? (HAS_BIAS ? 1 : 0)
                                                             : (HAS_BIAS ? 3 : 2);
    // memory operations per wave between a tile's K-tile S-2 copies and its
    // K-tile S-1 copies: the previous tile's stores (bf16: 4 x TJ x 2 of 16 B;
    // SwiGLU: 4 x TJ) and this tile's scale loads; other outputs drain at the
    // tile boundary
    constexpr int EPI = (BF16_OUT ? 8 * TJ : SWIGLU ? 4 * TJ : 0) + NSCALE;
    __shared__ __attribute__((aligned(1024))) int8_t sw0[STGW], sw1[STGW],
        sw2[S == 4 ? STGW : 16], sw3[S == 4 ? STGW : 16];
    __shared__ __attribute__((aligned(1024))) int8_t sx0[STGX], sx1[STGX],
        sx2[S == 4 ? STGX : 16], sx3[S == 4 ? STGX : 16];
    __shared__ __attribute__((aligned(16))) float sscale[3][kTile];   // s_x, s_w, bias

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave & 1, wm = wave >> 1;
    const int tiles = tiles_m * tiles_n;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int nk = K / kBK;

    // i-th tile of this workgroup (XCD-contiguous ranges, grouped along m),
    // or false past the end
    auto tile_at = [&](int i, int &m0, int &n0) -> bool {
        const int tl = slot + i * wgs_per_xcd;
        const int t = xcd * tiles_per_xcd + tl;
        if (tl >= tiles_per_xcd || t >= tiles) return false;
        const int width = kGroup * tiles_n;
        const int first_m = (t / width) * kGroup;
        const int gsz = min(tiles_m - first_m, kGroup);
        m0 = (first_m + (t % width) % gsz) * TM;
        n0 = ((t % width) / gsz) * kTile;
        return true;
    };

    int m0, n0;
    if (!tile_at(0, m0, n0)) return;
    if constexpr (SWIGLU) {
        // the LDS slice of the silu table (written once per device before any
        // launch that reads it)
        for (int i = threadIdx.x; i < 2 * kSiluSpanE; i += kThreads) {
            const int neg = i >= kSiluSpanE;
            g_silu_lds[i] = silu_tab[(neg << 15) | (i - neg * kSiluSpanE + kSiluLoE)];
        }
        __syncthreads();
    }
    if constexpr (OUT == int(OutKind::GELU_BF16)) {
        // the LDS slice of the GELU table (written once per device before
        // any launch that reads it)
        for (int i = threadIdx.x; i < 2 * kGeluSpan; i += kThreads) {
            const int neg = i >= kGeluSpan;
            g_gelu_lds[i] = g_gelu_bf16[(neg << 15) | (i - neg * kGeluSpan + kGeluLo)];
        }
        __syncthreads();
    }

    const int l32 = lane & 31, g = lane >> 5;
    const int foff0 = ((0 + g) ^ swz(l32)) << 4;
    const int foff1 = ((2 + g) ^ swz(l32)) << 4;
    const int frow_w = (wn * 128 + l32) * kBK;   // + 2048 * i
    const int frow_x = (wm * 32 * TJ + l32) * kBK;   // + 2048 * j

    auto load_scales = [&](int m0_, int n0_, float &a, float &b, float &c) {
        if constexpr (OUT != int(OutKind::I32) && !MM) {
            a = sx[min(m0_ + tid, M - 1)];
            b = sw[min(n0_ + tid, N - 1)];
        }
        if constexpr (OUT != int(OutKind::I32) && HAS_BIAS) {
            const int n = min(n0_ + tid, N - 1);
            // SwiGLU: the bias of the interleaved row's source channel
            c = bias[SWIGLU ? (int)swiglu_src_row(n, N >> 1) : n];
        }
    };

    float sc_x = 0.f, sc_w = 0.f, sc_b = 0.f;
    load_scales(m0, n0, sc_x, sc_w, sc_b);
    uint32_t voffw[4], voffx[TJ];
    lane_offsets<MM>(K, wave, lane, voffw);
    lane_offsets<MM>(K, wave, lane, voffx);
    TileSrc cur = tile_src<MM>(qw, qx, m0, n0, M, N, K);
    int nm0 = m0, nn0 = n0;
    bool more = tile_at(1, nm0, nn0);
    TileSrc nxt = more ? tile_src<MM>(qw, qx, nm0, nn0, M, N, K) : empty_src(qw, qx);

    for (int it = 0;; ++it) {
        v16i acc[4][TJ];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

        k_loop<TJ, 4, TJ, S, EPI, true, MM>(sw0, sw1, sw2, sw3, sx0, sx1, sx2, sx3, cur, nxt,
                                            voffw, voffx, nk, it == 0, wave, frow_w, frow_x,
                                            foff0, foff1, acc);

        if constexpr (OUT != int(OutKind::I32)) {
            sscale[0][tid] = sc_x;
            sscale[1][tid] = sc_w;
            sscale[2][tid] = sc_b;
        }
        // not __syncthreads(): its fence would also wait for the next tile's
        // copies already in flight
        wait_lds_reads();
        block_barrier();
        // stage S-1 is read by no one now: the next tile's K-tile S-1 goes
        // out ahead of this tile's stores (after the last tile: from the empty
        // source, no traffic)
        {
            int8_t *const wl = pick<S, S - 1>(sw0, sw1, sw2, sw3);
            int8_t *const xl = pick<S, S - 1>(sx0, sx1, sx2, sx3);
            issue_half<4, TJ, 0, MM>(cur, nxt, voffw, voffx, nk + S - 1, nk, wave, wl, xl);
            issue_half<4, TJ, 1, MM>(cur, nxt, voffw, voffx, nk + S - 1, nk, wave, wl, xl);
        }
        const bool full = m0 + TM <= M && n0 + kTile <= N;
        if constexpr (SWIGLU) {
            if (full)
                swiglu_epilogue<HAS_BIAS, TJ, true>(Y, acc, sscale, silu_tab, M, N, m0, n0, wm,
                                                    wn, l32, g);
            else
                swiglu_epilogue<HAS_BIAS, TJ, false>(Y, acc, sscale, silu_tab, M, N, m0, n0, wm,
                                                     wn, l32, g);
        } else {
            if (full)
                epilogue<OUT, HAS_BIAS, TJ, true>(Y, acc, sscale, M, N, m0, n0, wm, wn, l32, g);
            else
                epilogue<OUT, HAS_BIAS, TJ, false>(Y, acc, sscale, M, N, m0, n0, wm, wn, l32, g);
        }

        if (!more) break;
        // The next tile's waits count exactly EPI operations issued after its
        // first copies.  A partial tile issues fewer stores (and other outputs
        // more), so drain them: every copy issued so far has then landed.
        if (!(BF16_OUT || SWIGLU) || !full) wait_vmcnt<0>();
        m0 = nm0;
        n0 = nn0;
        cur = nxt;
        load_scales(m0, n0, sc_x, sc_w, sc_b);
        more = tile_at(it + 2, nm0, nn0);
        nxt = more ? tile_src<MM>(qw, qx, nm0, nn0, M, N, K) : empty_src(qw, qx);
        // sscale is rewritten only after the next K loop's barriers
    }
    // No copy may still be writing LDS when the workgroup ends.
    wait_vmcnt<0>();
}

template <int OUT, bool HAS_BIAS, int TJ>
hipError_t launch_tj(const int8_t *qx, const int8_t *qw, const float *sx, const float *sw,
                     const float *bias, void *Y, int64_t M, int64_t N, int64_t K, int cus,
                     hipStream_t stream, const float *silu_tab)
{
    constexpr int TM = 64 * TJ;
    const int tiles_m = (int)((M + TM - 1) / TM);
    const int tiles_n = (int)((N + kTile - 1) / kTile);
    const int tiles = tiles_m * tiles_n;
    const int per_xcd = (tiles + 7) / 8;
    const int wgs_per_xcd = std::max(1, std::min(cus / 8, per_xcd));
    const int nk = (int)(K / kBK);
    const dim3 grid(8 * wgs_per_xcd), block(kThreads);
    if (nk % 4 == 0)
        hipLaunchKernelGGL((gemm_i8_kernel<OUT, HAS_BIAS, TJ, 4>), grid, block, 0, stream, qx, qw,
                           sx, sw, bias, Y, (int)M, (int)N, (int)K, tiles_m, tiles_n, per_xcd,
                           wgs_per_xcd, silu_tab);
    else
        hipLaunchKernelGGL((gemm_i8_kernel<OUT, HAS_BIAS, TJ, 2>), grid, block, 0, stream, qx, qw,
                           sx, sw, bias, Y, (int)M, (int)N, (int)K, tiles_m, tiles_n, per_xcd,
                           wgs_per_xcd, silu_tab);
    return hipGetLastError();
}


// ---------------------------------------------------------------------------
// Factor 1 of the low-rank chain with the requantisation of its output fused
// into the epilogue.  The chain is h = bf16(linear(X; A)) followed by the
// rotate + per-token quantise of h along r (low-rank ConvRot linears: the MLX
// card, "Choose a Weight Format" and "Standalone Transformer"); since a row of
// h has only r <= 512 entries, a 128-token x 512-output tile holds whole rows,
// so the rotation, the row amax and the codes are computed here and h never
// reaches memory.
//
// Wave w owns outputs [128 w, 128 w + 128): one Hadamard block of 128 (or two
// of 64) for each of the tile's 128 tokens.  In the accumulator layout lane
// (l32, g) holds, for token 32 j + l32, the outputs n = 32 i + 8 q + 4 g + r
// (i, q, r = 0..3): index bits 0-1 are r, bit 2 is g, bits 3-4 q, bits 5-6 i.
// Butterfly stages on r, q and i stay in the lane; the stage on g pairs lane
// l32 with lane l32 + 32 through v_permlane32_swap.  Stages run in ascending
// stride, each as (a + b, a - b), exactly the order of the reading.
// ---------------------------------------------------------------------------

// v_accvgpr_write: keep a value in the accumulator registers (the rotated
// outputs wait there between the amax pass and the quantise pass).
__device__ __forceinline__ int to_acc(float v)
{
    int a;
    asm volatile("v_accvgpr_write_b32 %0, %1" : "=a"(a) : "v"(v));
    return a;
}

// One stage of stride H over the 64 values [i][q][r] a lane holds for one token.
template <int H>
__device__ __forceinline__ void f1_stage(float (&v)[4][4][4], int g)
{
    if constexpr (H == 4) {
        // across the lane halves: the lower lane (g = 0) gets a + b, the upper
        // one a - b; an fma by +-1 rounds exactly like the add or subtract
        const float c = g ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const auto pr = __builtin_amdgcn_permlane32_swap(
                        __float_as_int(v[i][q][r]), __float_as_int(v[i][q][r]), false, false);
                    // pr[0]: the lower lane's value, pr[1]: the upper lane's
                    v[i][q][r] = __builtin_fmaf(c, __int_as_float(pr[1]), __int_as_float(pr[0]));
                }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int n = 32 * i + 8 * q + r;   // bit 2 (g) is 0 here
                    if ((n & H) != 0) continue;
                    const int n2 = n + H;
                    float &a = v[i][q][r];
                    float &b = v[n2 >> 5][(n2 >> 3) & 3][n2 & 3];
                    const float s0 = __fadd_rn(a, b), d0 = __fsub_rn(a, b);
                    a = s0;
                    b = d0;
                }
    }
}

template <int BLK, int TJ>
__device__ __forceinline__ void f1_epilogue(v16i (&acc)[4][TJ], const float *s_x,
                                            const float *s_a, float *red, int8_t *qh, float *sh,
                                            int m0, int M, int R, float inv_sqrt_b, int wave,
                                            int l32, int g)
{
    constexpr int TM = 32 * TJ;
    // pass 1: h = bf16(((float)acc * s_x) * s_a), rotated, kept in the
    // accumulators; partial |max| of each token's row
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
        float v[4][4][4];
        const float sxm = s_x[32 * j + l32];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const v16i av = acc_frag(acc[i][j]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 sav =
                    *reinterpret_cast<const float4 *>(&s_a[wave * 128 + 32 * i + 8 * q + 4 * g]);
                const float sa4[4] = {sav.x, sav.y, sav.z, sav.w};
#pragma unroll
                for (int r = 0; r < 4; r += 2) {
                    const uint32_t p = cvt_pk_bf16(
                        __fmul_rn(__fmul_rn((float)av[4 * q + r], sxm), sa4[r]),
                        __fmul_rn(__fmul_rn((float)av[4 * q + r + 1], sxm), sa4[r + 1]));
                    v[i][q][r] = __uint_as_float(p << 16);
                    v[i][q][r + 1] = __uint_as_float(p & 0xffff0000u);
                }
            }
        }
        f1_stage<1>(v, g);
        f1_stage<2>(v, g);
        f1_stage<4>(v, g);
        f1_stage<8>(v, g);
        f1_stage<16>(v, g);
        f1_stage<32>(v, g);
        if constexpr (BLK == 128) f1_stage<64>(v, g);
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    m = fmaxf(m, fabsf(v[i][q][r]));
                    acc[i][j][4 * q + r] = to_acc(v[i][q][r]);
                }
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        if (g == 0) red[wave * TM + 32 * j + l32] = m;
        __builtin_amdgcn_sched_barrier(0);
    }
    wait_lds_reads();
    block_barrier();

    // pass 2: the row amax over the four waves, codes and scales.  The codes
    // go out K-tiled (m0 is a multiple of 16); rows between M and the 16-row
    // padding get codes too, which no reader uses.
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(qh + (int64_t)m0 * R), (short)0, (int)(padded_rows(M) - m0) * R, kRsrcWord3);
    const bool active = wave * 128 < R;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
        const int row = 32 * j + l32;
        const float amax = fmaxf(fmaxf(red[row], red[TM + row]),
                                 fmaxf(red[2 * TM + row], red[3 * TM + row]));
        const float inv = amax > 0.0f ? __fdiv_rn(127.0f, amax) : 0.0f;
        if (wave == 0 && g == 0 && m0 + row < M)
            sh[m0 + row] = __fmul_rn(__fdiv_rn(amax, 127.0f), inv_sqrt_b);
        if (!active) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const v16i av = acc_frag(acc[i][j]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t c[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    c[r] = __float_as_uint(__fadd_rn(__fmul_rn(__int_as_float(av[4 * q + r]), inv),
                                                     kMagicRint));
                const uint32_t w01 = __builtin_amdgcn_perm(c[1], c[0], 0x0c0c0400u);
                const uint32_t w23 = __builtin_amdgcn_perm(c[3], c[2], 0x0c0c0400u);
                __builtin_amdgcn_raw_buffer_store_b32(
                    (int)__builtin_amdgcn_perm(w23, w01, 0x05040100u), qr,
                    (int)tiled_offset(row, wave * 128 + 32 * i + 8 * q + 4 * g, R), 0, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int BLK, int S, int TJ>
__global__ __launch_bounds__(kThreads, 1) void lowrank_f1_kernel(
    const int8_t *__restrict__ qx, const int8_t *__restrict__ qa,
    const float *__restrict__ sx, const float *__restrict__ sa, int8_t *__restrict__ qh,
    float *__restrict__ sh, int M, int R, int K, float inv_sqrt_b)
{
    constexpr int TM = 32 * TJ;             // tokens per tile: 128, 64 or 32
    // activation copies per wave per K-tile: each copy moves one 16-row block,
    // so a 32-token tile is copied as 64 rows (every wave one block) whose
    // upper 32 are never read
    constexpr int CX = TJ >= 2 ? TJ / 2 : 1;
    constexpr int STGW = 512 * kBK;         // 32 KiB of A codes per stage
    constexpr int STGX = 64 * CX * kBK;     // 8 or 4 KiB of activation codes per stage
    constexpr int NSCALE = 3;               // per thread: a token scale, two channel scales
    __shared__ __attribute__((aligned(1024))) int8_t sw0[STGW], sw1[STGW],
        sw2[S == 4 ? STGW : 16], sw3[S == 4 ? STGW : 16];
    __shared__ __attribute__((aligned(1024))) int8_t sx0[STGX], sx1[STGX],
        sx2[S == 4 ? STGX : 16], sx3[S == 4 ? STGX : 16];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, g = lane >> 5;
    const int tiles = (M + TM - 1) / TM;
    const int nk = K / kBK;
    const int foff0 = ((0 + g) ^ swz(l32)) << 4;
    const int foff1 = ((2 + g) ^ swz(l32)) << 4;
    const int frow_w = (wave * 128 + l32) * kBK;   // + 2048 * i
    const int frow_x = l32 * kBK;                  // + 2048 * j
    uint32_t voffw[8], voffx[CX];
    lane_offsets(K, wave, lane, voffw);
    lane_offsets(K, wave, lane, voffx);

    auto src_of = [&](int t) {
        TileSrc ts;
        ts.w = __builtin_amdgcn_make_buffer_rsrc((void *)qa, (short)0, R * K, kRsrcWord3);
        ts.x = __builtin_amdgcn_make_buffer_rsrc((void *)(qx + (int64_t)t * TM * K), (short)0,
                                                 (int)(padded_rows(M) - t * TM) * K, kRsrcWord3);
        return ts;
    };
    float c_x, c_a0, c_a1;
    auto load_scales = [&](int t) {
        c_x = sx[min(t * TM + (tid & (TM - 1)), M - 1)];
        c_a0 = tid < R ? sa[tid] : 0.0f;
        c_a1 = tid + 256 < R ? sa[tid + 256] : 0.0f;
    };

    // epilogue scratch in stage S-1 (free from the end of the K loop until the
    // next tile's first copy into it): token scales, channel scales, row maxima
    int8_t *scratch = pick<S, S - 1>(sw0, sw1, sw2, sw3);
    float *s_x = reinterpret_cast<float *>(scratch);
    float *s_a = s_x + TM;
    float *red = s_a + 512;

    int t = blockIdx.x;                     // grid <= tiles
    load_scales(t);
    TileSrc cur = src_of(t);
    int tn = t + gridDim.x;
    bool more = tn < tiles;
    TileSrc nxt = more ? src_of(tn) : empty_src(qa, qx);

    for (int it = 0;; ++it) {
        v16i acc[4][TJ];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

        k_loop<TJ, 8, CX, S, NSCALE, false>(sw0, sw1, sw2, sw3, sx0, sx1, sx2, sx3, cur, nxt, voffw,
                                   voffx, nk, it == 0, wave, frow_w, frow_x, foff0, foff1, acc);

        // every wave is done reading stage S-1 before it becomes scratch
        wait_lds_reads();
        block_barrier();
        if (tid < TM) s_x[tid] = c_x;
        s_a[tid] = c_a0;
        s_a[tid + 256] = c_a1;
        wait_lds_reads();
        block_barrier();
        f1_epilogue<BLK, TJ>(acc, s_x, s_a, red, qh, sh, t * TM, M, R, inv_sqrt_b, wave, l32, g);
        // the codes drained (so the next tile's waits count exactly) and the
        // scratch read by everyone before the next tile's copies reuse it
        wait_vmcnt<0>();
        wait_lds_reads();
        block_barrier();
        if (!more) break;
        t = tn;
        cur = nxt;
        load_scales(t);
        tn = t + gridDim.x;
        more = tn < tiles;
        nxt = more ? src_of(tn) : empty_src(qa, qx);
    }
    wait_vmcnt<0>();
}

template <int BLK, int TJ>
hipError_t launch_f1_tj(const int8_t *qx, const int8_t *qa, const float *sx, const float *sa,
                        int8_t *qh, float *sh, int64_t M, int64_t R, int64_t K,
                        float inv_sqrt_b, int64_t max_grid, hipStream_t stream)
{
    const int64_t tiles = (M + 32 * TJ - 1) / (32 * TJ);
    const dim3 grid((unsigned)std::min<int64_t>(tiles, max_grid)), block(kThreads);
    if ((K / kBK) % 4 == 0)
        hipLaunchKernelGGL((lowrank_f1_kernel<BLK, 4, TJ>), grid, block, 0, stream, qx, qa, sx,
                           sa, qh, sh, (int)M, (int)R, (int)K, inv_sqrt_b);
    else
        hipLaunchKernelGGL((lowrank_f1_kernel<BLK, 2, TJ>), grid, block, 0, stream, qx, qa, sx,
                           sa, qh, sh, (int)M, (int)R, (int)K, inv_sqrt_b);
    return hipGetLastError();
}

// 128-token tiles, one per CU at a time.  When the last round of them would
// keep at most half the CUs busy, its rows go to a second launch of smaller
// tiles, one per CU: 32-token tiles when they fit in one round (at most a
// quarter of the CUs would hold a 128-token tile), else 64-token tiles.  At
// M = 38656 the 32-token tail makes the low-rank chain 1.2% faster than the
// 64-token one (434 vs 440 us, same outputs).
template <int BLK>
hipError_t launch_f1_blk(const int8_t *qx, const int8_t *qa, const float *sx, const float *sa,
                         int8_t *qh, float *sh, int64_t M, int64_t R, int64_t K,
                         float inv_sqrt_b, hipStream_t stream)
{
    const int64_t cus = device_cu_count();
    const int64_t tiles = (M + 127) / 128;
    const int64_t rounds = (tiles + cus - 1) / cus;
    const int64_t last = tiles - (rounds - 1) * cus;
    if (2 * last > cus)
        return launch_f1_tj<BLK, 4>(qx, qa, sx, sa, qh, sh, M, R, K, inv_sqrt_b, cus, stream);
    const int64_t m1 = (rounds - 1) * cus * 128;   // rows in whole rounds of 128
    if (m1 > 0) {
        const hipError_t e =
            launch_f1_tj<BLK, 4>(qx, qa, sx, sa, qh, sh, m1, R, K, inv_sqrt_b, cus, stream);
        if (e != hipSuccess) return e;
    }
    if (4 * last <= cus)
        return launch_f1_tj<BLK, 1>(qx + m1 * K, qa, sx + m1, sa, qh + m1 * R, sh + m1, M - m1, R,
                                    K, inv_sqrt_b, cus, stream);
    return launch_f1_tj<BLK, 2>(qx + m1 * K, qa, sx + m1, sa, qh + m1 * R, sh + m1, M - m1, R, K,
                                inv_sqrt_b, cus, stream);
}

// 256 x 256 tiles, one per CU at a time.  When the last round of them would
// leave CUs idle, the last tile-rows can go to a second launch of 256 (n) x
// 128 (m) tiles (TJ = 2), which take about 0.6 of a 256 x 256 tile each (they
// move more bytes per MFMA, so a whole launch of them runs at 0.8 of the
// rate), or, for the plain outputs, of 256 x 64 tiles (TJ = 1, about 0.35).
// The split is chosen from these estimates when K >= 1024; it pays when
// tiles are few (M = 4096: 336 tiles for 256 CUs, 10% faster), and at
// M = 38656, N = 16128 the last tile-row as one round of 256 x 64 tiles
// takes about 7 us less than as 256 x 128 ones.  With short K (the low-rank
// factor 2, K = 512) the launch is bound by its output stores and the split
// measured slower.
constexpr double kHalfTileCost = 0.625;   // TJ = 2 tile time / TJ = 4 tile time
constexpr double kQuarterTileCost = 0.35; // TJ = 1 tile time / TJ = 4 tile time
constexpr double kLaunchCost = 0.05;      // a second launch, in tile times

template <int OUT, bool HAS_BIAS>
hipError_t launch_t(const int8_t *qx, const int8_t *qw, const float *sx, const float *sw,
                    const float *bias, void *Y, int64_t M, int64_t N, int64_t K,
                    hipStream_t stream)
{
    if constexpr (OUT == int(OutKind::GELU_BF16)) {
        const uint16_t *table = nullptr;
        const hipError_t e = launch_gelu_table(&table, stream);
        if (e != hipSuccess) return e;
    }
    const float *silu_tab = nullptr;
    if constexpr (OUT == int(OutKind::SWIGLU_BF16)) {
        const hipError_t e = launch_silu_table(&silu_tab, stream);
        if (e != hipSuccess) return e;
    }
    const int cus = device_cu_count();
    const int64_t tm = (M + kTile - 1) / kTile, tn = (N + kTile - 1) / kTile;
    auto rounds = [&](int64_t tiles) { return (double)((tiles + cus - 1) / cus); };
    // quarter tiles (256 (n) x 64 (m), TJ = 1) for the plain outputs
    constexpr bool QUARTER = OUT == int(OutKind::BF16) || OUT == int(OutKind::F32) ||
                             OUT == int(OutKind::I32);
    int64_t best_a = tm;
    bool best_q = false;
    double best = rounds(tm * tn);
    for (int64_t a = tm - 1; K >= 1024 && a >= 0 && a >= tm - 16; --a) {
        const double th = rounds(a * tn) + kHalfTileCost * rounds(2 * (tm - a) * tn) + kLaunchCost;
        const double tq = QUARTER ? rounds(a * tn) + kQuarterTileCost * rounds(4 * (tm - a) * tn) +
                                        kLaunchCost
                                  : 1e30;
        const double t = std::min(th, tq);
        if (t < best - 0.1) {
            best = t;
            best_a = a;
            best_q = tq < th;
        }
    }
    const int64_t m1 = std::min<int64_t>(M, best_a * kTile);
    if (m1 > 0) {
        const hipError_t e =
            launch_tj<OUT, HAS_BIAS, 4>(qx, qw, sx, sw, bias, Y, m1, N, K, cus, stream, silu_tab);
        if (e != hipSuccess || m1 == M) return e;
    }
    constexpr size_t ysize = OUT == int(OutKind::F32) || OUT == int(OutKind::I32) ? 4 : 2;
    // row stride of Y in elements (SwiGLU writes N/2 columns)
    const int64_t ycols = OUT == int(OutKind::SWIGLU_BF16) ? N / 2 : N;
    if constexpr (QUARTER) {
        if (best_q)
            return launch_tj<OUT, HAS_BIAS, 1>(qx + m1 * K, qw, sx ? sx + m1 : nullptr, sw, bias,
                                               static_cast<char *>(Y) + (size_t)(m1 * ycols) * ysize,
                                               M - m1, N, K, cus, stream, silu_tab);
    }
    return launch_tj<OUT, HAS_BIAS, 2>(qx + m1 * K, qw, sx ? sx + m1 : nullptr, sw, bias,
                                       static_cast<char *>(Y) + (size_t)(m1 * ycols) * ysize,
                                       M - m1, N, K, cus, stream, silu_tab);
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
    case OutKind::BF16_MM:
        return hb ? launch_t<int(OutKind::BF16_MM), true>(qx, qw, sx, sw, bias, Y, M, N, K, stream)
                  : launch_t<int(OutKind::BF16_MM), false>(qx, qw, sx, sw, bias, Y, M, N, K, stream);
    case OutKind::SWIGLU_BF16:
        return hb ? launch_t<int(OutKind::SWIGLU_BF16), true>(qx, qw, sx, sw, bias, Y, M, N, K, stream)
                  : launch_t<int(OutKind::SWIGLU_BF16), false>(qx, qw, sx, sw, bias, Y, M, N, K, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gelu_table(const uint16_t **table, hipStream_t stream)
{
    // per device ordinal (each device holds its own copy of the module's
    // globals): the table's device address, and whether it has been written
    static std::atomic<const uint16_t *> cached[64];
    static std::atomic<int> filled[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool known = dev >= 0 && dev < 64;
    const uint16_t *p = known ? cached[dev].load(std::memory_order_relaxed) : nullptr;
    if (!p) {
        void *a = nullptr;
        e = hipGetSymbolAddress(&a, HIP_SYMBOL(g_gelu_bf16));
        if (e != hipSuccess) return e;
        p = static_cast<const uint16_t *>(a);
        // readers copy it in 16-byte pieces
        if (reinterpret_cast<uintptr_t>(p) & 15) return hipErrorInvalidValue;
        if (known) cached[dev].store(p, std::memory_order_relaxed);
    }
    *table = p;
    if (known && filled[dev].load(std::memory_order_acquire)) return hipSuccess;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gelu_table_kernel, dim3(256), dim3(256), 0, stream);
    e = hipGetLastError();
    if (e != hipSuccess || cap != hipStreamCaptureStatusNone || !known) return e;
    // the one wait of the library: once per device, so that launches on other
    // streams may read the table without being ordered after this one
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return e;
    filled[dev].store(1, std::memory_order_release);
    if (std::getenv("CONVROT_LOG") && std::getenv("CONVROT_LOG")[0] == '1')
        std::fprintf(stderr, "[convrot] GELU table written on device %d\n", dev);
    return hipSuccess;
}

hipError_t launch_gelu_bf16(const uint16_t *u, uint16_t *g, int64_t n, hipStream_t stream)
{
    if (n == 0) return hipSuccess;
    const uint16_t *table = nullptr;
    const hipError_t e = launch_gelu_table(&table, stream);
    if (e != hipSuccess) return e;
    // 16-byte aligned buffers: 8 values per thread from the LDS slice, the
    // last n % 8 one per thread; otherwise one per thread throughout
    const bool vec = ((reinterpret_cast<uintptr_t>(u) | reinterpret_cast<uintptr_t>(g)) & 15) == 0;
    const int64_t n8 = vec ? n / 8 : 0;
    if (n8 > 0) {
        const int64_t blocks = std::min<int64_t>((n8 + 255) / 256, (int64_t)device_cu_count() * 4);
        hipLaunchKernelGGL(gelu_apply8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                           reinterpret_cast<const uint4 *>(u), reinterpret_cast<uint4 *>(g), n8);
    }
    const int64_t rest = n - 8 * n8;
    if (rest > 0)
        hipLaunchKernelGGL(gelu_apply_kernel, dim3((unsigned)((rest + 255) / 256)), dim3(256), 0,
                           stream, u + 8 * n8, g + 8 * n8, rest);
    return hipGetLastError();
}

bool lowrank_f1_fusable(int64_t R, int block)
{
    return (block == 64 || block == 128) && R % 128 == 0 && R > 0 && R <= 512;
}

hipError_t launch_lowrank_f1(const int8_t *qx, const int8_t *qa, const float *sx,
                             const float *sa, int8_t *qh, float *sh, int64_t M, int64_t R,
                             int64_t K, int block, float inv_sqrt_b, hipStream_t stream)
{
    if (M == 0) return hipSuccess;
    if (!lowrank_f1_fusable(R, block)) return hipErrorInvalidValue;
    return block == 128
               ? launch_f1_blk<128>(qx, qa, sx, sa, qh, sh, M, R, K, inv_sqrt_b, stream)
               : launch_f1_blk<64>(qx, qa, sx, sa, qh, sh, M, R, K, inv_sqrt_b, stream);
}

} // namespace convrot
