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
//
// K pipeline: K advances 64 bytes per stage; STAGES stages of 32 KiB (W and X
// tiles, 256 rows x 64 B each) live in LDS.  Global -> LDS copies use the
// direct-to-LDS load (global_load_lds_dwordx4: each lane fetches 16 bytes and
// the wave's 1 KiB lands contiguously in LDS), so no registers stage the
// tiles and no LDS write instructions are issued.  Tile kt + STAGES is
// requested as soon as stage kt is consumed, STAGES - 1 tiles ahead of use.
// The compiler does not order LDS reads after these copies, so every wait is
// explicit: s_waitcnt vmcnt(n) for this wave's copies, then a barrier for the
// other waves'.
//
// LDS rows are 64 bytes; chunk c (16 B) of tile row r sits at slot
// c ^ f(r), f(r) = ((r >> 1) ^ (r >> 3)) & 3.  A copy instruction writes 16
// consecutive rows, so lane i fetches chunk (i & 3) ^ f(row) of its row; the
// column-wise MFMA fragment reads (32 rows, one chunk) then hit distinct banks
// for 32- and 64-bank LDS alike.
//
// Workgroups are renumbered so each of the 8 XCDs walks a contiguous range of
// tiles, grouped 8 tile-rows high, for L2 reuse of both operands.
#include "common.hpp"

#include <utility>

namespace convrot {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kTile = 256;     // tile edge in m and in n
constexpr int kBK = 64;        // K bytes per LDS stage
constexpr int kThreads = 256;
constexpr int kGroup = 8;      // tile-rows per L2 group

__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

// s_waitcnt vmcnt(n) with expcnt/lgkmcnt left unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until at most `tiles` stages of this wave's copies (COPIES each) are
// still in flight.
template <int COPIES>
__device__ __forceinline__ void wait_copies(int tiles)
{
    if (tiles >= 3) wait_vmcnt<3 * COPIES>();
    else if (tiles == 2) wait_vmcnt<2 * COPIES>();
    else if (tiles == 1) wait_vmcnt<1 * COPIES>();
    else wait_vmcnt<0>();
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
// a burst: the memory instructions (all LDS reads first, then all copies --
// a read placed after a copy in the same block would get a conservative vmcnt
// wait on that copy) are spread evenly behind the MFMAs.
template <int MFMAS, int VMEMS, int DSREADS, int K>
__device__ __forceinline__ void interleave_slot()
{
    constexpr int TOTAL = VMEMS + DSREADS;
    // memory ops whose share falls in MFMA slot K: ops [LO, HI)
    constexpr int LO = (K * TOTAL + MFMAS - 1) / MFMAS;
    constexpr int HI = ((K + 1) * TOTAL + MFMAS - 1) / MFMAS;
    constexpr int RD_LO = LO < DSREADS ? LO : DSREADS, RD_HI = HI < DSREADS ? HI : DSREADS;
    constexpr int VM_LO = LO > DSREADS ? LO : DSREADS, VM_HI = HI > DSREADS ? HI : DSREADS;
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

__device__ __forceinline__ void copy16(const int8_t *g, int8_t *lds)
{
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(g),
                                     (__attribute__((address_space(3))) void *)(lds), 16, 0, 0);
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
// fp32 value of one output: ((float)acc * s_x) * s_w (+ bias), optionally
// followed by bf16 rounding and GELU (the MLP's up projection).
template <int OUT, bool HAS_BIAS>
__device__ __forceinline__ float dequant1(int acc, float sxm, float swn, float bn)
{
    float f = __fmul_rn(__fmul_rn((float)acc, sxm), swn);
    if constexpr (HAS_BIAS) f = __fadd_rn(f, bn);
    if constexpr (OUT == int(OutKind::GELU_BF16))
        f = gelu_erf(__uint_as_float(f32_to_bf16_bits(f) << 16));
    return f;
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
template <int OUT, bool HAS_BIAS, int TJ, bool FULL>
__device__ __forceinline__ void epilogue(void *Y, const v16i (&acc)[4][TJ],
                                         const float (&sscale)[3][kTile], int M, int N,
                                         int m0, int n0, int wm, int wn, int l32, int g)
{
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
        const int ml = wm * 32 * TJ + 32 * j + l32;
        const int m = m0 + ml;
        if (!FULL && m >= M) continue;
        const float sxm = (OUT == int(OutKind::I32)) ? 0.0f : sscale[0][ml];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
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
                        o.x = dequant1<OUT, HAS_BIAS>(acc[i][j][4 * q + 0], sxm, swv.x, bv.x);
                        o.y = dequant1<OUT, HAS_BIAS>(acc[i][j][4 * q + 1], sxm, swv.y, bv.y);
                        o.z = dequant1<OUT, HAS_BIAS>(acc[i][j][4 * q + 2], sxm, swv.z, bv.z);
                        o.w = dequant1<OUT, HAS_BIAS>(acc[i][j][4 * q + 3], sxm, swv.w, bv.w);
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
                            dequant1<OUT, HAS_BIAS>(acc[i][j][4 * q + 0], sxm, swv.x, bv.x),
                            dequant1<OUT, HAS_BIAS>(acc[i][j][4 * q + 1], sxm, swv.y, bv.y));
                        d[h][1] = cvt_pk_bf16(
                            dequant1<OUT, HAS_BIAS>(acc[i][j][4 * q + 2], sxm, swv.z, bv.z),
                            dequant1<OUT, HAS_BIAS>(acc[i][j][4 * q + 3], sxm, swv.w, bv.w));
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
        }
    }
}

// Per-wave state of the K loop, kept in registers.
template <int TJ>
struct CopyPlan {
    uint32_t offw[4];    // byte offsets of this lane's 16-byte W chunks, per copy
    uint32_t offx[TJ];   // same for X
};

// Direct-to-LDS copies of K-tile `kt` into one stage (wave-uniform LDS bases):
// wave w fills W rows [(4w + j) 16, +16) and X rows [(TJ w + j) 16, +16).
template <int TJ>
__device__ __forceinline__ void issue_stage(const int8_t *qw, const int8_t *qx,
                                            const CopyPlan<TJ> &cp, int kt, int wave,
                                            int8_t *__restrict__ dst_w,
                                            int8_t *__restrict__ dst_x)
{
#pragma unroll
    for (int j = 0; j < 4; ++j)
        copy16(qw + kt * kBK + cp.offw[j], dst_w + (wave * 4 + j) * 1024);
#pragma unroll
    for (int j = 0; j < TJ; ++j)
        copy16(qx + kt * kBK + cp.offx[j], dst_x + (wave * TJ + j) * 1024);
}

template <int TJ>
__device__ __forceinline__ void read_frags(const int8_t *__restrict__ sw_,
                                           const int8_t *__restrict__ sx_, int frow_w,
                                           int frow_x, int foff, v4i (&a)[4], v4i (&b)[TJ])
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const v4i *>(sw_ + frow_w + 2048 * i + foff);
#pragma unroll
    for (int j = 0; j < TJ; ++j)
        b[j] = *reinterpret_cast<const v4i *>(sx_ + frow_x + 2048 * j + foff);
}

template <int TJ>
__device__ __forceinline__ void mfma_block(v16i (&acc)[4][TJ], const v4i (&a)[4],
                                           const v4i (&b)[TJ])
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], acc[i][j], 0, 0, 0);
}

template <int S, int I>
__device__ __forceinline__ int8_t *pick(int8_t *p0, int8_t *p1, int8_t *p2, int8_t *p3)
{
    constexpr int k = I % S;
    return k == 0 ? p0 : k == 1 ? p1 : k == 2 ? p2 : p3;
}

// The K loop over one tile.  Each LDS stage is a separate object reached
// through its own restrict pointer, and the loop is unrolled by the stage
// count so every access names its stage at compile time.  That lets the
// compiler prove that an LDS read of one stage does not depend on copies still
// landing in another, so it only waits (vmcnt) for copies into the stage being
// read.  Waiting for the other waves' copies is explicit: each wave retires
// its own copies of the next K-tile, then all meet at a barrier.
// Requires nk % S == 0.
template <int TJ, int S>
__device__ __forceinline__ void k_loop(int8_t *__restrict__ w0, int8_t *__restrict__ w1,
                                       int8_t *__restrict__ w2, int8_t *__restrict__ w3,
                                       int8_t *__restrict__ x0, int8_t *__restrict__ x1,
                                       int8_t *__restrict__ x2, int8_t *__restrict__ x3,
                                       const int8_t *qw, const int8_t *qx,
                                       const CopyPlan<TJ> &cp, int nk, int wave, int frow_w,
                                       int frow_x, int foff0, int foff1,
                                       v16i (&acc)[4][TJ])
{
    static_assert(S >= 2 && S <= 4, "stages");
    constexpr int COPIES = 4 + TJ;           // copy instructions per wave per K-tile
    constexpr int MF = 4 * TJ;               // MFMAs per sub-step
    constexpr int RD = 4 + TJ;               // fragment reads per sub-step
    v4i a0[4], b0[TJ], a1[4], b1[TJ];

    // prologue: every stage starts free
    issue_stage<TJ>(qw, qx, cp, 0, wave, w0, x0);
    issue_stage<TJ>(qw, qx, cp, min(1, nk - 1), wave, w1, x1);
    if constexpr (S >= 3) issue_stage<TJ>(qw, qx, cp, min(2, nk - 1), wave, w2, x2);
    if constexpr (S >= 4) issue_stage<TJ>(qw, qx, cp, min(3, nk - 1), wave, w3, x3);
    wait_vmcnt<(S - 1) * COPIES>();
    block_barrier();
    read_frags<TJ>(w0, x0, frow_w, frow_x, foff0, a0, b0);

    // One step = the second half of K-tile kt (MFMAs on the sub-step-1
    // fragments, with the reads of tile kt+1's sub-step 0 and the copies of
    // tile kt+S interleaved) and the first half of tile kt+1.
#define CONVROT_STEP(I)                                                                  \
    do {                                                                                 \
        int8_t *cw_ = pick<S, I>(w0, w1, w2, w3), *cx_ = pick<S, I>(x0, x1, x2, x3);      \
        int8_t *nw_ = pick<S, I + 1>(w0, w1, w2, w3), *nx_ = pick<S, I + 1>(x0, x1, x2, x3); \
        wait_lds_reads();                                                                \
        __builtin_amdgcn_sched_barrier(0);                                               \
        read_frags<TJ>(cw_, cx_, frow_w, frow_x, foff1, a1, b1);                          \
        mfma_block<TJ>(acc, a0, b0);                                                     \
        interleave<MF, 0, RD>();                                                         \
        __builtin_amdgcn_sched_barrier(0);                                               \
        wait_lds_reads();                                                                \
        wait_vmcnt<(S - 2) * COPIES>();                                                  \
        block_barrier();                                                                 \
        read_frags<TJ>(nw_, nx_, frow_w, frow_x, foff0, a0, b0);                          \
        issue_stage<TJ>(qw, qx, cp, min(kt + I + S, nk - 1), wave, cw_, cx_);            \
        mfma_block<TJ>(acc, a1, b1);                                                     \
        interleave<MF, COPIES, RD>();                                                    \
        __builtin_amdgcn_sched_barrier(0);                                               \
    } while (0)

    // nk - 1 steps (K-tiles 0 .. nk-2), S at a time, then the rest in line
    int kt = 0;
    for (; kt + S < nk; kt += S) {
        CONVROT_STEP(0);
        CONVROT_STEP(1);
        if constexpr (S >= 3) CONVROT_STEP(2);
        if constexpr (S >= 4) CONVROT_STEP(3);
    }
    // nk is a multiple of S: S - 1 steps remain
    CONVROT_STEP(0);
    if constexpr (S >= 3) CONVROT_STEP(1);
    if constexpr (S >= 4) CONVROT_STEP(2);
#undef CONVROT_STEP
    {
        const int8_t *lw = pick<S, S - 1>(w0, w1, w2, w3), *lx = pick<S, S - 1>(x0, x1, x2, x3);
        wait_lds_reads();
        __builtin_amdgcn_sched_barrier(0);
        read_frags<TJ>(lw, lx, frow_w, frow_x, foff1, a1, b1);
        mfma_block<TJ>(acc, a0, b0);
        interleave<MF, 0, RD>();
        __builtin_amdgcn_sched_barrier(0);
        mfma_block<TJ>(acc, a1, b1);
    }
    // No copy may still be writing LDS when the workgroup moves on.
    wait_vmcnt<0>();
}

// One 256 (n) x 64 TJ (m) output tile per 256-thread workgroup; wave (wn, wm)
// computes 128 (n) x 32 TJ (m).  TJ = 4: 256 AGPR accumulators, one workgroup
// per CU.  TJ = 2: 128 accumulators, two workgroups per CU, so one
// workgroup's barriers and epilogue overlap the other's matrix work.
// S: LDS stages of (256 + 64 TJ) x 64 bytes; nk % S == 0.
template <int OUT, bool HAS_BIAS, int TJ, int S, int OCC>
__global__ __launch_bounds__(kThreads, OCC) void gemm_i8_kernel(
    const int8_t *__restrict__ qx, const int8_t *__restrict__ qw,
    const float *__restrict__ sx, const float *__restrict__ sw,
    const float *__restrict__ bias, void *__restrict__ Y, int M, int N, int K,
    int tiles_m, int tiles_n, int tiles_per_xcd)
{
    constexpr int BM = 64 * TJ;
    constexpr int SW = kTile * kBK;          // W stage bytes
    constexpr int SX = BM * kBK;             // X stage bytes
    __shared__ __attribute__((aligned(1024))) int8_t sw0[SW], sw1[SW], sw2[S >= 3 ? SW : 16],
        sw3[S >= 4 ? SW : 16];
    __shared__ __attribute__((aligned(1024))) int8_t sx0[SX], sx1[SX], sx2[S >= 3 ? SX : 16],
        sx3[S >= 4 ? SX : 16];
    __shared__ __attribute__((aligned(16))) float sscale[3][kTile];   // s_x, s_w, bias

    // ---- tile selection: XCD-contiguous ranges, grouped along m ----
    const int pid = blockIdx.x;
    const int t = (pid & 7) * tiles_per_xcd + (pid >> 3);
    if (t >= tiles_m * tiles_n) return;
    const int width = kGroup * tiles_n;
    const int first_m = (t / width) * kGroup;
    const int gsz = min(tiles_m - first_m, kGroup);
    const int tm = first_m + (t % width) % gsz;
    const int tn = (t % width) / gsz;
    const int m0 = tm * BM, n0 = tn * kTile;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wn = wave & 1, wm = wave >> 1;

    // ---- copy plan: a copy moves 16 rows x 64 B; lane i takes row + i/4 and
    // the chunk that belongs in slot i & 3 of that row ----
    CopyPlan<TJ> cp;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = (wave * 4 + j) * 16 + (lane >> 2);
        cp.offw[j] = (uint32_t)min(n0 + r, N - 1) * (uint32_t)K + (((lane & 3) ^ swz(r)) << 4);
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
        const int r = (wave * TJ + j) * 16 + (lane >> 2);
        cp.offx[j] = (uint32_t)min(m0 + r, M - 1) * (uint32_t)K + (((lane & 3) ^ swz(r)) << 4);
    }

    // ---- fragment read assignment ----
    const int l32 = lane & 31, g = lane >> 5;
    const int foff0 = ((0 + g) ^ swz(l32)) << 4;
    const int foff1 = ((2 + g) ^ swz(l32)) << 4;
    const int frow_w = (wn * 128 + l32) * kBK;       // + 2048 * i
    const int frow_x = (wm * 32 * TJ + l32) * kBK;   // + 2048 * j

    // The tile's scales: plain loads issued ahead of the first K-tile copies,
    // written to LDS before the epilogue.
    float sc_x = 0.f, sc_w = 0.f, sc_b = 0.f;
    if constexpr (OUT != int(OutKind::I32)) {
        sc_x = sx[min(m0 + (tid % BM), M - 1)];
        sc_w = sw[min(n0 + tid, N - 1)];
        if constexpr (HAS_BIAS) sc_b = bias[min(n0 + tid, N - 1)];
    }

    v16i acc[4][TJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

    k_loop<TJ, S>(sw0, sw1, sw2, sw3, sx0, sx1, sx2, sx3, qw, qx, cp, K / kBK, wave, frow_w,
                  frow_x, foff0, foff1, acc);

    if constexpr (OUT != int(OutKind::I32)) {
        if (tid < BM) sscale[0][tid] = sc_x;
        sscale[1][tid] = sc_w;
        sscale[2][tid] = sc_b;
    }
    __syncthreads();

    // ---- epilogue: lane holds n = nb..nb+3 of one m per (i, j, q) ----
    if (m0 + BM <= M && n0 + kTile <= N)
        epilogue<OUT, HAS_BIAS, TJ, true>(Y, acc, sscale, M, N, m0, n0, wm, wn, l32, g);
    else
        epilogue<OUT, HAS_BIAS, TJ, false>(Y, acc, sscale, M, N, m0, n0, wm, wn, l32, g);
}

template <int OUT, bool HAS_BIAS, int TJ, int S, int OCC>
hipError_t launch_cfg(const int8_t *qx, const int8_t *qw, const float *sx, const float *sw,
                      const float *bias, void *Y, int64_t M, int64_t N, int64_t K,
                      hipStream_t stream)
{
    constexpr int BM = 64 * TJ;
    const int tiles_m = (int)((M + BM - 1) / BM);
    const int tiles_n = (int)((N + kTile - 1) / kTile);
    const int tiles = tiles_m * tiles_n;
    const int per_xcd = (tiles + 7) / 8;
    hipLaunchKernelGGL((gemm_i8_kernel<OUT, HAS_BIAS, TJ, S, OCC>), dim3(8 * per_xcd),
                       dim3(kThreads), 0, stream, qx, qw, sx, sw, bias, Y, (int)M, (int)N,
                       (int)K, tiles_m, tiles_n, per_xcd);
    return hipGetLastError();
}

#ifndef CONVROT_GEMM_TJ
#define CONVROT_GEMM_TJ 4
#endif

template <int OUT, bool HAS_BIAS>
hipError_t launch_t(const int8_t *qx, const int8_t *qw, const float *sx, const float *sw,
                    const float *bias, void *Y, int64_t M, int64_t N, int64_t K,
                    hipStream_t stream)
{
    const int nk = (int)(K / kBK);
    if constexpr (CONVROT_GEMM_TJ == 4) {
        if (nk % 4 == 0)
            return launch_cfg<OUT, HAS_BIAS, 4, 4, 1>(qx, qw, sx, sw, bias, Y, M, N, K, stream);
        return launch_cfg<OUT, HAS_BIAS, 4, 2, 1>(qx, qw, sx, sw, bias, Y, M, N, K, stream);
    } else {
        if (nk % 3 == 0)
            return launch_cfg<OUT, HAS_BIAS, 2, 3, 2>(qx, qw, sx, sw, bias, Y, M, N, K, stream);
        return launch_cfg<OUT, HAS_BIAS, 2, 2, 2>(qx, qw, sx, sw, bias, Y, M, N, K, stream);
    }
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
