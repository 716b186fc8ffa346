// Fused rotate + rowwise INT8 quantise for gfx950.
//
// What it computes (per row x of length K, block b):
//   v = blockdiag(H_b) . x  in fp32, butterfly strides h = 1, 2, ..., b/2 in
//       ascending order (Sylvester H_b, natural order, unnormalised), or the
//       regular H_4 Kronecker blocks (rotate_regular, b = 64 or 256);
//   amax = max |v|;  q = rint(v * (127/amax)) in [-127, 127];
//   s = (amax/127) * fp32(1/sqrt(b));  a zero row gives q = 0, s = 0.
// The rotation and the row-wise quantise are the fused prologue of a ConvRot
// projection (MiniMax-H3-Rung-Omega README, "Technical Architecture Overview",
// Floor 1); the block-diagonal Hadamard in front of the W8A8 linears is the
// lehuy.net article's ("Cach nen hoat dong", second bullet).
//
// Data layout in registers.  A wave covers 512 consecutive elements of a row
// per "step": 64 lanes x 8 elements (the pair kernel: 256 elements of each of
// two rows, one per half-wave).  A block of b elements is spread over
// L = b/8 lanes, and lane i of the block holds the 8-element chunk pi(i) of it,
// where pi is the GF(2)-linear map with pi(1)=1, pi(2)=2, pi(4)=7, pi(8)=12,
// pi(16)=16.  With that assignment the partner of every cross-lane butterfly
// stage is a single DPP pattern:
//   chunk bit 0 (h =  8): lane ^ 1   quad_perm:[1,0,3,2]
//   chunk bit 1 (h = 16): lane ^ 2   quad_perm:[2,3,0,1]
//   chunk bit 2 (h = 32): lane ^ 7   row_half_mirror
//   chunk bit 3 (h = 64): lane ^ 15  row_mirror
//   chunk bit 4 (h =128): lane ^ 16  ds_swizzle SWAP16
// so the 8 elements of a lane go through stages h = 1, 2, 4 in registers and
// the remaining stages cost one v_fmac_f32_dpp each.
//
// Sign tracking.  A butterfly needs lo+up in the lower lane and lo-up in the
// upper one.  Every lane instead computes r + c*partner with c = +1 (lower) or
// -1 (upper), one fused multiply-add by +-1, which rounds exactly like the add
// or subtract.  The upper lane then holds -(lo-up); the sign is the same for
// every element of a lane, (-1)^popcount(pi(i)) after all stages, and is
// folded into the quantisation multiplier (negation is exact and rint is odd).
// Hence the codes equal those of the plain butterfly order bit for bit.
//
// Quantise: t = v * inv rounds once (fp32), then t + 1.5*2^23 rounds to an
// integer with ties to even (|t| <= 127.00001 << 2^22), and the code is the low
// byte of that float's bits.  Codes go out in the library's K-tiled layout
// (common.hpp): 8 bytes per lane per step into the row's 16-row block.
#include "common.hpp"

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>

namespace convrot {
namespace {

constexpr int kStep = 512;      // elements per wave step
// cache policy of every input load: nt (streaming), since each input byte
// is read once; measured 8% faster on the M=38656, K=5376 activations read
// right after a GEMM, 2% on the MLP's g
constexpr int kStreamLoad = 2;
constexpr int kTiledStep = 16 * kStep;   // bytes a step spans in a K-tiled row block
constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23

__device__ __forceinline__ int chunk_of_lane(int i)
{
    int c = 0;
    if (i & 1) c ^= 1;
    if (i & 2) c ^= 2;
    if (i & 4) c ^= 7;
    if (i & 8) c ^= 12;
    if (i & 16) c ^= 16;
    return c;
}

// One cross-lane butterfly stage on the 8 registers of a chunk.  The leading
// s_nop covers the VALU-write -> DPP-read hazard of whatever precedes.
#define CR_DPP_STAGE(CTRL, v, c)                                              \
    asm volatile("s_nop 1\n\t"                                                \
                 "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
                 "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
                 "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
                 "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
                 "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
                 "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
                 "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
                 "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf"   \
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]),             \
                   "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7])              \
                 : "v"(c))

template <int STAGE>
__device__ __forceinline__ void cross_stage(float (&v)[8], float c)
{
    if constexpr (STAGE == 0) {
        CR_DPP_STAGE("quad_perm:[1,0,3,2]", v, c);
    } else if constexpr (STAGE == 1) {
        CR_DPP_STAGE("quad_perm:[2,3,0,1]", v, c);
    } else if constexpr (STAGE == 2) {
        CR_DPP_STAGE("row_half_mirror", v, c);
    } else if constexpr (STAGE == 3) {
        CR_DPP_STAGE("row_mirror", v, c);
    } else {
        static_assert(STAGE == 4, "b <= 256");
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float p = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v[j]), 0x401F));
            v[j] = __builtin_fmaf(p, c, v[j]);
        }
    }
}

// Butterflies h = 1, 2, 4 inside one lane's chunk (ascending).
__device__ __forceinline__ void inlane_fwht8(float (&v)[8])
{
#pragma unroll
    for (int h = 1; h < 8; h *= 2) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if ((i & h) == 0) {
                float a = v[i], c = v[i + h];
                v[i] = __fadd_rn(a, c);
                v[i + h] = __fsub_rn(a, c);
            }
        }
    }
}

// d = s + (s of the lane holding the partner chunk of stage STAGE), for the
// regular rotation's pair sums.  fp32 addition is commutative, so both lanes
// of a pair get the same bits.
#define CR_DPP_ADD(CTRL, d, s)                                                \
    asm volatile("s_nop 1\n\t"                                                \
                 "v_add_f32_dpp %0, %8, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
                 "v_add_f32_dpp %1, %9, %9 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
                 "v_add_f32_dpp %2, %10, %10 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
                 "v_add_f32_dpp %3, %11, %11 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
                 "v_add_f32_dpp %4, %12, %12 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
                 "v_add_f32_dpp %5, %13, %13 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
                 "v_add_f32_dpp %6, %14, %14 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
                 "v_add_f32_dpp %7, %15, %15 " CTRL " row_mask:0xf bank_mask:0xf"   \
                 : "=&v"(d[0]), "=&v"(d[1]), "=&v"(d[2]), "=&v"(d[3]),         \
                   "=&v"(d[4]), "=&v"(d[5]), "=&v"(d[6]), "=&v"(d[7])          \
                 : "v"(s[0]), "v"(s[1]), "v"(s[2]), "v"(s[3]),                 \
                   "v"(s[4]), "v"(s[5]), "v"(s[6]), "v"(s[7]))

template <int STAGE>
__device__ __forceinline__ void partner_add(float (&d)[8], const float (&s)[8])
{
    if constexpr (STAGE == 0) {
        CR_DPP_ADD("quad_perm:[1,0,3,2]", d, s);
    } else if constexpr (STAGE == 1) {
        CR_DPP_ADD("quad_perm:[2,3,0,1]", d, s);
    } else if constexpr (STAGE == 2) {
        CR_DPP_ADD("row_half_mirror", d, s);
    } else if constexpr (STAGE == 3) {
        CR_DPP_ADD("row_mirror", d, s);
    } else {
        static_assert(STAGE == 4, "b <= 256");
#pragma unroll
        for (int j = 0; j < 8; ++j)
            d[j] = __fadd_rn(s[j], __int_as_float(__builtin_amdgcn_ds_swizzle(
                                       __float_as_int(s[j]), 0x401F)));
    }
}

// The regular rotation of one chunk: H_4 = J - 2I along every base-4 digit
// of the in-block index, lowest digit first (the Rung-Omega README's
// H_256 = H_4 (x) H_4 (x) H_4 (x) H_4, and its order-64 counterpart).  A group
// (v0, v1, v2, v3) of one digit becomes S - 2 v_j with S = (v0 + v1) + (v2 +
// v3).  Digit 0 lies inside the lane; digit 1 pairs elements e, e + 4 of the
// lane and of the chunk across chunk bit 0; digit d >= 2 is chunk bits
// 2d - 3 and 2d - 2, whose partner lanes are the Sylvester stages' DPP
// patterns.  2 v_j is exact, so each output is one rounding of S - 2 v_j.
template <int B>
__device__ __forceinline__ void rotate_regular(float (&v)[8])
{
#pragma unroll
    for (int g = 0; g < 8; g += 4) {
        const float S = __fadd_rn(__fadd_rn(v[g], v[g + 1]), __fadd_rn(v[g + 2], v[g + 3]));
#pragma unroll
        for (int j = 0; j < 4; ++j) v[g + j] = __fsub_rn(S, 2.0f * v[g + j]);
    }
    {
        float p[8], S[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[i] = __fadd_rn(v[i], v[i + 4]);
            p[i + 4] = p[i];
        }
        partner_add<0>(S, p);
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = __fsub_rn(S[j], 2.0f * v[j]);
    }
    {
        float a[8], S[8];
        partner_add<1>(a, v);
        partner_add<2>(S, a);
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = __fsub_rn(S[j], 2.0f * v[j]);
    }
    if constexpr (B == 256) {
        float a[8], S[8];
        partner_add<3>(a, v);
        partner_add<4>(S, a);
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = __fsub_rn(S[j], 2.0f * v[j]);
    }
}

// Rotation kinds: 0 = Sylvester blocks (butterflies with the sign trick),
// 1 = regular H_4 Kronecker blocks (B = 64 or 256).
template <int B, int ROT, int NSTAGE>
__device__ __forceinline__ void rotate_chunk(float (&v)[8], const float (&csign)[NSTAGE])
{
    if constexpr (ROT == 1) {
        static_assert(B == 64 || B == 256, "regular blocks are powers of 4");
        rotate_regular<B>(v);
    } else {
        inlane_fwht8(v);
        cross_stage<0>(v, csign[0]);
        cross_stage<1>(v, csign[1]);
        cross_stage<2>(v, csign[2]);
        if constexpr (NSTAGE > 3) cross_stage<3>(v, csign[3]);
        if constexpr (NSTAGE > 4) cross_stage<4>(v, csign[4]);
    }
}

// buffer resource word 3: raw (untyped) 32-bit data format, no swizzle
constexpr int kRsrcWord3 = 0x00020000;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));

// One row as a buffer resource of `bytes` bytes: loads past the end read as
// zero and stores past the end are dropped, so a partial last step needs no
// per-lane branches.  A row beyond M gets an empty range.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void *base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes,
                                             kRsrcWord3);
}

// The 8 elements of one chunk at element offset e of the row.
template <int IN>
__device__ __forceinline__ void load_chunk(__amdgpu_buffer_rsrc_t row, int e, float (&v)[8])
{
    if constexpr (IN == int(InType::BF16)) {
        const v4i d = __builtin_amdgcn_raw_buffer_load_b128(row, e * 2, 0, kStreamLoad);
        v[0] = bf16_lo(d[0]); v[1] = bf16_hi(d[0]);
        v[2] = bf16_lo(d[1]); v[3] = bf16_hi(d[1]);
        v[4] = bf16_lo(d[2]); v[5] = bf16_hi(d[2]);
        v[6] = bf16_lo(d[3]); v[7] = bf16_hi(d[3]);
    } else {
        const v4i a = __builtin_amdgcn_raw_buffer_load_b128(row, e * 4, 0, kStreamLoad);
        const v4i c = __builtin_amdgcn_raw_buffer_load_b128(row, e * 4 + 16, 0, kStreamLoad);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[j] = __int_as_float(a[j]);
            v[4 + j] = __int_as_float(c[j]);
        }
    }
}

__device__ __forceinline__ uint32_t code_bits(float v, float inv)
{
    return __float_as_uint(__fadd_rn(__fmul_rn(v, inv), kMagic));
}

__device__ __forceinline__ uint2 quantise_chunk(const float (&v)[8], float inv)
{
    uint32_t c0 = code_bits(v[0], inv), c1 = code_bits(v[1], inv);
    uint32_t c2 = code_bits(v[2], inv), c3 = code_bits(v[3], inv);
    uint32_t c4 = code_bits(v[4], inv), c5 = code_bits(v[5], inv);
    uint32_t c6 = code_bits(v[6], inv), c7 = code_bits(v[7], inv);
    // v_perm_b32: pick the low byte of each code into one dword.
    uint32_t p01 = __builtin_amdgcn_perm(c1, c0, 0x0c0c0400u);
    uint32_t p23 = __builtin_amdgcn_perm(c3, c2, 0x0c0c0400u);
    uint32_t p45 = __builtin_amdgcn_perm(c5, c4, 0x0c0c0400u);
    uint32_t p67 = __builtin_amdgcn_perm(c7, c6, 0x0c0c0400u);
    uint2 r;
    r.x = __builtin_amdgcn_perm(p23, p01, 0x05040100u);
    r.y = __builtin_amdgcn_perm(p67, p45, 0x05040100u);
    return r;
}

__device__ __forceinline__ float wave_max(float m)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        m = fmaxf(m, __shfl_xor(m, off, 64));
    return m;
}

// IN: input type; B: Hadamard block; SPR: wave steps held per wave (an upper
// bound: steps past the end of the row are skipped by a wave-uniform branch);
// RPW: rows per wave (when WPR == 1); WPR: waves per row; NW: waves per WG.
template <int IN, int B, int ROT, int SPR, int RPW, int WPR, int NW>
__global__ __launch_bounds__(NW * 64) void rotquant_kernel(
    const void *__restrict__ src, int64_t M, int K, int64_t ld, float inv_sqrt_b,
    int8_t *__restrict__ q, float *__restrict__ s)
{
    static_assert(RPW == 1 || WPR == 1, "multi-wave rows hold one row per wave");
    static_assert(NW % WPR == 0, "");
    constexpr int LPB = B / 8;
    constexpr int NSTAGE = (B == 64) ? 3 : (B == 128) ? 4 : 5;
    constexpr int GROUPS = NW / WPR;
    constexpr int ESIZE = IN == int(InType::BF16) ? 2 : 4;

    __shared__ float red[NW];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int part = wave % WPR;
    const int grp = wave / WPR;
    const int64_t row0 = ((int64_t)blockIdx.x * GROUPS + grp) * RPW;
    const int li = lane % LPB;
    const int chunk = chunk_of_lane(li);
    const int lane_off = (lane / LPB) * B + chunk * 8;
    const int steps = (K + kStep - 1) / kStep;
    // steps of this wave: part, part + WPR, ... below `steps`
    const int my_steps = (steps - part + WPR - 1) / WPR;

    // codes: the row's 16-row block of the K-tiled layout as the range (so
    // elements past K fall outside it) and this lane's offset in the block
    __amdgpu_buffer_rsrc_t src_row[RPW], q_blk[RPW];
    int q_off[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        const int64_t row = row0 + r;
        const bool in = row < M;
        src_row[r] = row_rsrc(reinterpret_cast<const char *>(src) + (in ? row : 0) * ld * ESIZE,
                              in ? K * ESIZE : 0);
        q_blk[r] = row_rsrc(q + (in ? (row & ~int64_t(15)) : 0) * (int64_t)K, in ? 16 * K : 0);
        q_off[r] = (int)tiled_offset(row & 15, lane_off, K);
    }

    float v[RPW][SPR][8];

    // ---- loads: every chunk of every row this wave owns, all in flight ----
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int t = 0; t < SPR; ++t)
            if (t < my_steps)
                load_chunk<IN>(src_row[r], (part + WPR * t) * kStep + lane_off, v[r][t]);

    float csign[NSTAGE];
#pragma unroll
    for (int k = 0; k < NSTAGE; ++k)
        csign[k] = ((chunk >> k) & 1) ? -1.0f : 1.0f;

    // ---- rotation (wave-uniform control flow: the DPP stages need every
    // lane) and the row's |max| ----
    float m[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        m[r] = 0.0f;
#pragma unroll
        for (int t = 0; t < SPR; ++t) {
            if (t < my_steps) {
                rotate_chunk<B, ROT>(v[r][t], csign);
#pragma unroll
                for (int j = 0; j < 8; ++j) m[r] = fmaxf(m[r], fabsf(v[r][t][j]));
            }
        }
    }

    // the Sylvester sign trick leaves the upper lanes' values negated
    const bool negated = ROT == 0 && (__builtin_popcount(chunk) & 1) != 0;

    // ---- per row: amax, scale, codes ----
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        const int64_t row = row0 + r;
        float mx = wave_max(m[r]);
        if constexpr (WPR > 1) {
            if (lane == 0) red[wave] = mx;
            __syncthreads();
#pragma unroll
            for (int w = 0; w < WPR; ++w) mx = fmaxf(mx, red[grp * WPR + w]);
        }
        const float inv = (mx > 0.0f) ? __fdiv_rn(127.0f, mx) : 0.0f;
        const float invs = negated ? -inv : inv;
        if (part == 0 && lane == 0 && row < M)
            s[row] = __fmul_rn(__fdiv_rn(mx, 127.0f), inv_sqrt_b);
#pragma unroll
        for (int t = 0; t < SPR; ++t) {
            if (t < my_steps) {
                const uint2 c = quantise_chunk(v[r][t], invs);
                __builtin_amdgcn_raw_buffer_store_b64((v2i){(int)c.x, (int)c.y}, q_blk[r],
                                                      (part + WPR * t) * kTiledStep + q_off[r],
                                                      0, 0);
            }
        }
    }
}

template <int IN, int B, int ROT, int SPR, int RPW, int WPR, int NW>
hipError_t launch_cfg(const void *src, int64_t M, int64_t K, int64_t ld,
                      float inv_sqrt_b, int8_t *q, float *s, hipStream_t stream)
{
    constexpr int rows_per_wg = (NW / WPR) * RPW;
    const int64_t grid = (M + rows_per_wg - 1) / rows_per_wg;
    hipLaunchKernelGGL((rotquant_kernel<IN, B, ROT, SPR, RPW, WPR, NW>), dim3((unsigned)grid),
                       dim3(NW * 64), 0, stream, src, M, (int)K, ld, inv_sqrt_b, q, s);
    return hipGetLastError();
}

// Streaming variant for rows split over WPR waves (K > 2048): one persistent
// workgroup per CU walks row groups, and each wave loads the raw input of
// its next group before rotating the current one, so memory and the rotation
// overlap inside the wave as well as across waves.
template <int IN, int B, int ROT, int SPR, int WPR, int NW>
__global__ __launch_bounds__(NW * 64) void rotquant_stream_kernel(
    const void *__restrict__ src, int64_t M, int K, int64_t ld, float inv_sqrt_b,
    int8_t *__restrict__ q, float *__restrict__ s)
{
    static_assert(NW % WPR == 0 && WPR > 1, "");
    constexpr int LPB = B / 8;
    constexpr int NSTAGE = (B == 64) ? 3 : (B == 128) ? 4 : 5;
    constexpr int GROUPS = NW / WPR;
    constexpr int ESIZE = IN == int(InType::BF16) ? 2 : 4;
    constexpr int DW = IN == int(InType::BF16) ? 4 : 8;   // raw dwords per lane per step

    __shared__ float red[2][NW];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int part = wave % WPR;
    const int grp = wave / WPR;
    const int li = lane % LPB;
    const int chunk = chunk_of_lane(li);
    const int lane_off = (lane / LPB) * B + chunk * 8;
    const int steps = (K + kStep - 1) / kStep;
    const int my_steps = (steps - part + WPR - 1) / WPR;
    const int64_t ngroups = (M + GROUPS - 1) / GROUPS;

    float csign[NSTAGE];
#pragma unroll
    for (int k = 0; k < NSTAGE; ++k)
        csign[k] = ((chunk >> k) & 1) ? -1.0f : 1.0f;
    // the Sylvester sign trick leaves the upper lanes' values negated
    const bool negated = ROT == 0 && (__builtin_popcount(chunk) & 1) != 0;

    // Every memory instruction is unconditional (steps past the row end fall
    // outside the buffer range: loads read zero, stores are dropped), so the
    // compiler can count them and wait for the prefetched loads only.
    int raw[SPR][DW];
    auto issue = [&](int64_t gi) {
        const int64_t row = gi * GROUPS + grp;
        const bool in = row < M;
        const __amdgpu_buffer_rsrc_t r = row_rsrc(
            reinterpret_cast<const char *>(src) + (in ? row : 0) * ld * ESIZE, in ? K * ESIZE : 0);
#pragma unroll
        for (int t = 0; t < SPR; ++t) {
            const int e = (part + WPR * t) * kStep + lane_off;
            const v4i a = __builtin_amdgcn_raw_buffer_load_b128(r, e * ESIZE, 0, kStreamLoad);
#pragma unroll
            for (int j = 0; j < 4; ++j) raw[t][j] = a[j];
            if constexpr (DW == 8) {
                const v4i c = __builtin_amdgcn_raw_buffer_load_b128(r, e * ESIZE + 16, 0, kStreamLoad);
#pragma unroll
                for (int j = 0; j < 4; ++j) raw[t][4 + j] = c[j];
            }
        }
    };
    const __amdgpu_buffer_rsrc_t srs = row_rsrc(s, (int)(M * 4 < 0x7fffffff ? M * 4 : 0x7fffffff));

    int64_t gi = blockIdx.x;
    issue(gi);
    {
        // the loop's stores, into an empty range: both ways into the loop
        // then carry the same sequence of memory operations, and the
        // compiler's waits at the top of the loop cover the loads only
        const __amdgpu_buffer_rsrc_t none = row_rsrc(q, 0);
        __builtin_amdgcn_raw_buffer_store_b32(0, none, 0, 0, 0);
#pragma unroll
        for (int t = 0; t < SPR; ++t)
            __builtin_amdgcn_raw_buffer_store_b64((v2i){0, 0}, none, 0, 0, 0);
    }
    int par = 0;
    for (; gi < ngroups; gi += gridDim.x, par ^= 1) {
        const int64_t row = gi * GROUPS + grp;
        float v[SPR][8];
#pragma unroll
        for (int t = 0; t < SPR; ++t) {
            if constexpr (DW == 4) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v[t][2 * j] = bf16_lo((uint32_t)raw[t][j]);
                    v[t][2 * j + 1] = bf16_hi((uint32_t)raw[t][j]);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) v[t][j] = __int_as_float(raw[t][j]);
            }
        }
        // next group; on the last pass a group past the end, whose rows are
        // out of range: its loads read an empty buffer (zeros, no memory
        // traffic) and keep the sequence of memory operations uniform
        issue(gi + gridDim.x);

        float m = 0.0f;
#pragma unroll
        for (int t = 0; t < SPR; ++t) {
            if (t < my_steps) {
                rotate_chunk<B, ROT>(v[t], csign);
#pragma unroll
                for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[t][j]));
            }
        }
        // the row's |max| over its WPR waves; red[] alternates between passes
        // so a fast wave cannot overwrite values a slow one still reads
        float mx = wave_max(m);
        if (lane == 0) red[par][wave] = mx;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < WPR; ++w) mx = fmaxf(mx, red[par][grp * WPR + w]);
        const float inv = (mx > 0.0f) ? __fdiv_rn(127.0f, mx) : 0.0f;
        const float invs = negated ? -inv : inv;
        const bool in = row < M;
        // the scale: one lane per row writes, every other lane's offset is
        // out of range
        __builtin_amdgcn_raw_buffer_store_b32(
            __float_as_int(__fmul_rn(__fdiv_rn(mx, 127.0f), inv_sqrt_b)), srs,
            (part == 0 && lane == 0 && in) ? (int)(row * 4) : 0x7ffffff0, 0, 0);
        const __amdgpu_buffer_rsrc_t qb =
            row_rsrc(q + (in ? (row & ~int64_t(15)) : 0) * (int64_t)K, in ? 16 * K : 0);
        const int q_off = (int)tiled_offset(row & 15, lane_off, K);
#pragma unroll
        for (int t = 0; t < SPR; ++t) {
            const uint2 c = quantise_chunk(v[t], invs);
            __builtin_amdgcn_raw_buffer_store_b64((v2i){(int)c.x, (int)c.y}, qb,
                                                  (part + WPR * t) * kTiledStep + q_off, 0, 0);
        }
    }
}

template <int IN, int B, int ROT, int SPR, int WPR, int NW>
hipError_t launch_stream(const void *src, int64_t M, int64_t K, int64_t ld,
                         float inv_sqrt_b, int8_t *q, float *s, hipStream_t stream)
{
    constexpr int rows_per_wg = NW / WPR;
    const int64_t groups = (M + rows_per_wg - 1) / rows_per_wg;
    const int64_t grid = std::min<int64_t>(groups, device_cu_count());
    hipLaunchKernelGGL((rotquant_stream_kernel<IN, B, ROT, SPR, WPR, NW>), dim3((unsigned)grid),
                       dim3(NW * 64), 0, stream, src, M, (int)K, ld, inv_sqrt_b, q, s);
    return hipGetLastError();
}

// ------------------------------------------------------------- SwiGLU ----
// The activation of the SwiGLU MLP (MiniMax-H3-Rung-Omega README, "Technical
// Architecture Overview", Floor 1: SwiGLU in front of the rotated, rowwise
// quantised fc2): fc1 writes [gate | up] as one bf16 row of 2F values and
// g = bf16(s * up) with s = fp32(silu(gate)), silu(z) = z / (1 + exp(-z))
// evaluated in fp64 on the bf16 gate and rounded once to fp32, s * up one
// fp32 multiply.
//
// g_silu_f32 holds s for every bf16 gate pattern, written once per device
// (launch_silu_table).  Kernels read a slice of it from LDS: for each sign the
// patterns with |z| in [2^-24, 2^8) (biased exponents 103..134, 4096 entries,
// 16 KiB per sign).  Outside the slice s has a closed form, which the
// exhaustive test of every pattern checks: z/2 for |z| < 2^-24 (the next term
// z^2/4 is below half an ulp of z/2), z for z >= 2^8 and -0 for z <= -2^8
// (exp(-|z|) is far below an ulp there; both hold from |z| >= 128 on).
// Non-finite gates give unspecified values.
__device__ __align__(16) float g_silu_f32[65536];

constexpr int kSiluLo = 103 << 7;     // first |z| pattern of the slice
constexpr int kSiluSpan = 32 << 7;    // patterns per sign

__global__ __launch_bounds__(256) void silu_table_kernel()
{
    const uint32_t a = blockIdx.x * 256u + threadIdx.x;
    const double z = (double)__uint_as_float(a << 16);
    g_silu_f32[a] = (float)(z / (1.0 + exp(-z)));
}

// Copy the slice of the table into LDS (every thread of the workgroup takes
// part; the caller synchronises).
__device__ __forceinline__ void load_silu_slice(float *sl, const float *__restrict__ tab,
                                                int nthreads)
{
    for (int i = threadIdx.x; i < 2 * kSiluSpan; i += nthreads) {
        const int neg = i >= kSiluSpan;
        sl[i] = tab[(neg << 15) | (i - neg * kSiluSpan + kSiluLo)];
    }
}

// s = fp32(silu(z)) of the bf16 pattern a (low 16 bits), from the LDS slice or
// the closed forms outside it; branch-free (the index is clamped into the
// slice either way).
__device__ __forceinline__ float silu_of(uint32_t a, const float *sl)
{
    const uint32_t mag = a & 0x7fffu, neg = (a >> 15) & 1u;
    const float z = __uint_as_float(a << 16);
    const uint32_t off = mag - (uint32_t)kSiluLo;      // wraps below the slice
    const float t = sl[neg * kSiluSpan + min(off, (uint32_t)kSiluSpan - 1u)];
    const float out = mag < (uint32_t)kSiluLo ? __fmul_rn(z, 0.5f) : (neg ? -0.0f : z);
    return off < (uint32_t)kSiluSpan ? t : out;
}

typedef __bf16 rq_bf16x2 __attribute__((ext_vector_type(2)));
typedef float rq_f32x2 __attribute__((ext_vector_type(2)));

// Two bf16 gate/up pairs (packed dwords) -> the packed bf16 pair of g.
__device__ __forceinline__ uint32_t swiglu_pair(uint32_t gate2, uint32_t up2, const float *sl)
{
    const float g0 = __fmul_rn(silu_of(gate2 & 0xffffu, sl), bf16_lo(up2));
    const float g1 = __fmul_rn(silu_of(gate2 >> 16, sl), bf16_hi(up2));
    // v_cvt_pk_bf16_f32: round to nearest even
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((rq_f32x2){g0, g1}, rq_bf16x2));
}

// g [M, F] = swiglu of gu [M, 2F], 8 values per thread (16-byte loads of the
// gate and the up halves, one 16-byte store); grid-stride over M * F / 8.
__global__ __launch_bounds__(256) void swiglu_apply8_kernel(const uint4 *__restrict__ gu,
                                                            uint4 *__restrict__ g, int64_t M,
                                                            int64_t F8)
{
    __shared__ float sl[2 * kSiluSpan];
    load_silu_slice(sl, g_silu_f32, 256);
    __syncthreads();
    const int64_t n = M * F8, stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
        const int64_t m = i / F8, j = i % F8;
        const uint4 a = gu[m * 2 * F8 + j], u = gu[m * 2 * F8 + F8 + j];
        uint4 o;
        o.x = swiglu_pair(a.x, u.x, sl);
        o.y = swiglu_pair(a.y, u.y, sl);
        o.z = swiglu_pair(a.z, u.z, sl);
        o.w = swiglu_pair(a.w, u.w, sl);
        g[i] = o;
    }
}

// s[i] = fp32(silu(a[i])) for n bf16 values, through the same slice and
// closed forms as every SwiGLU kernel.
__global__ __launch_bounds__(256) void silu_f32_kernel(const uint16_t *__restrict__ a,
                                                       float *__restrict__ out, int64_t n)
{
    __shared__ float sl[2 * kSiluSpan];
    load_silu_slice(sl, g_silu_f32, 256);
    __syncthreads();
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride)
        out[i] = silu_of(a[i], sl);
}

// Streaming variant for long rows (6144 < K <= 24576): rows are taken in
// pairs, one per half-wave.  A wave step covers 256 elements of each row of
// the pair (32 lanes x 8 elements; a Hadamard block of b <= 256 lies inside
// a half-wave, so the rotation is the same code), and a pair is split over
// WPR = 2..16 waves of at most SPR steps.  Both rows of a pair are
// neighbours in a 16-row block of the K-tiled codes, so a store instruction
// writes 4 K-tiles x 2 rows x 64 B = 4 whole 128-byte lines (one row per wave
// wrote 8 half lines per instruction: 27% slower at K = 21504).  One
// persistent workgroup per CU walks pair groups, and each wave loads the raw
// input of its next group before rotating the current one, so memory and the
// rotation overlap inside the wave as well as across waves.
// ACT = kActGelu (bf16 input only): each loaded value u is replaced by
// bf16(GELU(u)) from the 65,536-entry table gtab (one entry per bf16 pattern)
// before the rotation, so the MLP's intermediate is read once, as u, and g is
// never written.  The table is copied into LDS (128 KiB) when the workgroup
// starts.
constexpr int kActNone = 0, kActGelu = 1;

template <int IN, int B, int ROT, int SPR, int WPR, int NW, int ACT = kActNone>
__global__ __launch_bounds__(NW * 64) void rotquant_pair_kernel(
    const void *__restrict__ src, int64_t M, int K, int64_t ld, float inv_sqrt_b,
    int8_t *__restrict__ q, float *__restrict__ s, const void *__restrict__ gtab)
{
    static_assert(ACT == kActNone || IN == int(InType::BF16), "activations take bf16 input");
    constexpr bool GELU = ACT == kActGelu;
    __shared__ uint16_t tab[GELU ? 65536 : 2];
    if constexpr (GELU) {
        const uint4 *gt = reinterpret_cast<const uint4 *>(gtab);
        uint4 *lt = reinterpret_cast<uint4 *>(tab);
        for (int i = threadIdx.x; i < 65536 / 8; i += NW * 64) lt[i] = gt[i];
        __syncthreads();
    }
    static_assert(NW % WPR == 0 && WPR > 1, "");
    static_assert(B <= 256, "a block lies inside a half-wave");
    constexpr int HS = 256;                   // elements per row per step
    constexpr int LPB = B / 8;
    constexpr int NSTAGE = (B == 64) ? 3 : (B == 128) ? 4 : 5;
    constexpr int PAIRS = NW / WPR;           // row pairs per pass
    constexpr int ESIZE = IN == int(InType::BF16) ? 2 : 4;
    constexpr int DW = IN == int(InType::BF16) ? 4 : 8;   // raw dwords per lane per step

    __shared__ float red[2][NW][2];

    const int lane = threadIdx.x & 63;
    const int half = lane >> 5, hl = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int part = wave % WPR;
    const int grp = wave / WPR;
    const int li = hl % LPB;
    const int chunk = chunk_of_lane(li);
    const int lane_off = (hl / LPB) * B + chunk * 8;   // inside the 256-element step
    const int steps = (K + HS - 1) / HS;
    const int my_steps = (steps - part + WPR - 1) / WPR;
    const int64_t ngroups = (M + 2 * PAIRS - 1) / (2 * PAIRS);

    float csign[NSTAGE];
#pragma unroll
    for (int k = 0; k < NSTAGE; ++k)
        csign[k] = ((chunk >> k) & 1) ? -1.0f : 1.0f;
    // the Sylvester sign trick leaves the upper lanes' values negated
    const bool negated = ROT == 0 && (__builtin_popcount(chunk) & 1) != 0;

    // Every memory instruction is unconditional, so the compiler can count
    // them and wait for the prefetched loads only.  The buffer resources are
    // wave-uniform (a resource that differs between the half-waves costs a
    // loop per instruction): loads go through the pair's rows inside M, the
    // lane's own row reached by its offset, and an element at or past K gets
    // an offset outside every range, so it reads zero; stores go through the
    // pair's 16-row block of codes, and a lane whose row is past M stores
    // outside it (dropped).
    constexpr uint32_t kOut = 0x7f000000u;       // beyond every range used here
    const uint32_t lane_row = (uint32_t)(half * ld * ESIZE);
    auto pair_rsrc = [&](int64_t gi) {
        const int64_t row0 = (gi * PAIRS + grp) * 2;
        const int64_t rows = row0 < M ? (M - row0 < 2 ? M - row0 : 2) : 0;
        return row_rsrc(reinterpret_cast<const char *>(src) + (rows ? row0 : 0) * ld * ESIZE,
                        (int)(rows * ld * ESIZE));
    };
    // byte offset of step t of this lane's row, `skip` elements into the row
    auto step_off = [&](int t, int skip) -> uint32_t {
        const int e = (part + WPR * t) * HS + lane_off;
        return e < K ? lane_row + (uint32_t)((skip + e) * ESIZE) : kOut;
    };

    int raw[SPR][DW];
    auto issue = [&](int64_t gi) {
        const __amdgpu_buffer_rsrc_t r = pair_rsrc(gi);
#pragma unroll
        for (int t = 0; t < SPR; ++t) {
            const uint32_t o = step_off(t, 0);
            const v4i a = __builtin_amdgcn_raw_buffer_load_b128(r, (int)o, 0, kStreamLoad);
#pragma unroll
            for (int j = 0; j < 4; ++j) raw[t][j] = a[j];
            if constexpr (DW == 8) {
                const v4i c = __builtin_amdgcn_raw_buffer_load_b128(r, (int)o + 16, 0, kStreamLoad);
#pragma unroll
                for (int j = 0; j < 4; ++j) raw[t][4 + j] = c[j];
            }
        }
    };
    const __amdgpu_buffer_rsrc_t srs = row_rsrc(s, (int)(M * 4 < 0x7fffffff ? M * 4 : 0x7fffffff));

    int64_t gi = blockIdx.x;
    issue(gi);
    {
        // the loop's stores, into an empty range: both ways into the loop
        // then carry the same sequence of memory operations, and the
        // compiler's waits at the top of the loop cover the loads only
        const __amdgpu_buffer_rsrc_t none = row_rsrc(q, 0);
        __builtin_amdgcn_raw_buffer_store_b32(0, none, 0, 0, 0);
#pragma unroll
        for (int t = 0; t < SPR; ++t)
            __builtin_amdgcn_raw_buffer_store_b64((v2i){0, 0}, none, 0, 0, 0);
    }
    int par = 0;
    for (; gi < ngroups; gi += gridDim.x, par ^= 1) {
        const int64_t row = (gi * PAIRS + grp) * 2 + half;
        float v[SPR][8];
#pragma unroll
        for (int t = 0; t < SPR; ++t) {
            if constexpr (DW == 4) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    uint32_t u = (uint32_t)raw[t][j];
                    if constexpr (GELU)
                        u = (uint32_t)tab[u & 0xffffu] | ((uint32_t)tab[u >> 16] << 16);
                    v[t][2 * j] = bf16_lo(u);
                    v[t][2 * j + 1] = bf16_hi(u);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) v[t][j] = __int_as_float(raw[t][j]);
            }
        }
        // next group; on the last pass a group past the end, whose rows are
        // out of range: its loads read an empty buffer (zeros, no memory
        // traffic) and keep the sequence of memory operations uniform
        issue(gi + gridDim.x);

        float m = 0.0f;
#pragma unroll
        for (int t = 0; t < SPR; ++t) {
            if (t < my_steps) {
                rotate_chunk<B, ROT>(v[t], csign);
#pragma unroll
                for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[t][j]));
            }
        }
        // the row's |max|: over the half-wave, then over its WPR waves; red[]
        // alternates between passes so a fast wave cannot overwrite values a
        // slow one still reads
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1)
            m = fmaxf(m, __shfl_xor(m, off, 64));
        if (hl == 0) red[par][wave][half] = m;
        __syncthreads();
        float mx = 0.0f;
#pragma unroll
        for (int w = 0; w < WPR; ++w) mx = fmaxf(mx, red[par][grp * WPR + w][half]);
        const float inv = (mx > 0.0f) ? __fdiv_rn(127.0f, mx) : 0.0f;
        const float invs = negated ? -inv : inv;
        const bool in = row < M;
        // the scale: one lane per row writes, every other lane's offset is
        // out of range
        __builtin_amdgcn_raw_buffer_store_b32(
            __float_as_int(__fmul_rn(__fdiv_rn(mx, 127.0f), inv_sqrt_b)), srs,
            (part == 0 && hl == 0 && in) ? (int)(row * 4) : 0x7ffffff0, 0, 0);
        const int64_t row0 = row - half;
        const __amdgpu_buffer_rsrc_t qb =
            row_rsrc(q + (row0 < M ? (row0 & ~int64_t(15)) : 0) * (int64_t)K,
                     row0 < M ? 16 * K : 0);
        const uint32_t q_off = in ? (uint32_t)tiled_offset(row & 15, lane_off, K) : kOut;
#pragma unroll
        for (int t = 0; t < SPR; ++t) {
            const uint2 c = quantise_chunk(v[t], invs);
            // step t spans 4 K-tiles of the row block: 4 KiB
            __builtin_amdgcn_raw_buffer_store_b64((v2i){(int)c.x, (int)c.y}, qb,
                                                  (int)((part + WPR * t) * 4096 + q_off), 0, 0);
        }
    }
}

template <int IN, int B, int ROT, int SPR, int WPR, int NW, int ACT = kActNone>
hipError_t launch_pair(const void *src, int64_t M, int64_t K, int64_t ld,
                         float inv_sqrt_b, int8_t *q, float *s, hipStream_t stream,
                         const void *gtab = nullptr)
{
    constexpr int rows_per_wg = 2 * (NW / WPR);
    const int64_t groups = (M + rows_per_wg - 1) / rows_per_wg;
    const int64_t grid = std::min<int64_t>(groups, device_cu_count());
    hipLaunchKernelGGL((rotquant_pair_kernel<IN, B, ROT, SPR, WPR, NW, ACT>),
                       dim3((unsigned)grid), dim3(NW * 64), 0, stream, src, M, (int)K, ld,
                       inv_sqrt_b, q, s, gtab);
    return hipGetLastError();
}

// Rows of up to 4 steps (2048 elements) are held by one wave, several rows
// per wave when they are short.  Rows of up to 6 steps go to the streaming
// kernel, one row over 2 waves of up to 6 steps, 16 waves per CU.  Longer
// rows up to 24576 elements go in pairs to the pair kernel: rows of at most
// 21 steps of 256 elements over 3 waves of 7 steps (12 waves per CU; at
// K = 5376 rotate+quantise of 38656 rows takes 99.7 us where the streaming
// kernel took 107.4 us, back to back on one box), up to 24 steps over 4
// waves of 6, then 8 or 16 waves of 6 (at K = 21504 it takes 0.200 ms where
// one row per wave took 0.244 ms).  Longer rows go to the one-shot kernel
// with 16 waves of up to 8 steps of 512 elements (K <= 65536).
template <int IN, int B, int ROT>
hipError_t launch_b(const void *src, int64_t M, int64_t K, int64_t ld,
                    float inv_sqrt_b, int8_t *q, float *s, hipStream_t stream)
{
    const int64_t steps = (K + kStep - 1) / kStep;
    const int64_t hsteps = (K + 255) / 256;
    if (steps <= 1) return launch_cfg<IN, B, ROT, 1, 8, 1, 4>(src, M, K, ld, inv_sqrt_b, q, s, stream);
    if (steps <= 2) return launch_cfg<IN, B, ROT, 2, 4, 1, 4>(src, M, K, ld, inv_sqrt_b, q, s, stream);
    if (steps <= 4) return launch_cfg<IN, B, ROT, 4, 2, 1, 4>(src, M, K, ld, inv_sqrt_b, q, s, stream);
    if (steps <= 6) return launch_stream<IN, B, ROT, 6, 2, 16>(src, M, K, ld, inv_sqrt_b, q, s, stream);
    if (hsteps <= 21) return launch_pair<IN, B, ROT, 7, 3, 12>(src, M, K, ld, inv_sqrt_b, q, s, stream);
    if (hsteps <= 24) return launch_pair<IN, B, ROT, 6, 4, 16>(src, M, K, ld, inv_sqrt_b, q, s, stream);
    if (hsteps <= 48) return launch_pair<IN, B, ROT, 6, 8, 16>(src, M, K, ld, inv_sqrt_b, q, s, stream);
    if (hsteps <= 96) return launch_pair<IN, B, ROT, 6, 16, 16>(src, M, K, ld, inv_sqrt_b, q, s, stream);
    return launch_cfg<IN, B, ROT, 8, 1, 16, 16>(src, M, K, ld, inv_sqrt_b, q, s, stream);
}

template <int IN>
hipError_t launch_in(const void *src, int64_t M, int64_t K, int64_t ld, int block,
                     bool regular, float inv_sqrt_b, int8_t *q, float *s, hipStream_t stream)
{
    if (regular) {
        switch (block) {
        case 64: return launch_b<IN, 64, 1>(src, M, K, ld, inv_sqrt_b, q, s, stream);
        case 256: return launch_b<IN, 256, 1>(src, M, K, ld, inv_sqrt_b, q, s, stream);
        default: return hipErrorInvalidValue;
        }
    }
    switch (block) {
    case 64: return launch_b<IN, 64, 0>(src, M, K, ld, inv_sqrt_b, q, s, stream);
    case 128: return launch_b<IN, 128, 0>(src, M, K, ld, inv_sqrt_b, q, s, stream);
    case 256: return launch_b<IN, 256, 0>(src, M, K, ld, inv_sqrt_b, q, s, stream);
    default: return hipErrorInvalidValue;
    }
}

// The pair kernel's range, with an activation on load (bf16 rows,
// 6144 < K <= 24576).
template <int B, int ROT, int ACT>
hipError_t launch_act_b(const void *src, int64_t M, int64_t K, int64_t ld, float inv_sqrt_b,
                        int8_t *q, float *s, const void *gtab, hipStream_t stream)
{
    constexpr int BF = int(InType::BF16);
    const int64_t hsteps = (K + 255) / 256;
    if (hsteps <= 48)
        return launch_pair<BF, B, ROT, 6, 8, 16, ACT>(src, M, K, ld, inv_sqrt_b, q, s, stream, gtab);
    return launch_pair<BF, B, ROT, 6, 16, 16, ACT>(src, M, K, ld, inv_sqrt_b, q, s, stream, gtab);
}

template <int ACT>
hipError_t launch_act(const void *src, int64_t M, int64_t K, int64_t ld, int block, bool regular,
                      float inv_sqrt_b, const void *gtab, int8_t *q, float *s,
                      hipStream_t stream)
{
    if (regular) {
        switch (block) {
        case 64: return launch_act_b<64, 1, ACT>(src, M, K, ld, inv_sqrt_b, q, s, gtab, stream);
        case 256: return launch_act_b<256, 1, ACT>(src, M, K, ld, inv_sqrt_b, q, s, gtab, stream);
        default: return hipErrorInvalidValue;
        }
    }
    switch (block) {
    case 64: return launch_act_b<64, 0, ACT>(src, M, K, ld, inv_sqrt_b, q, s, gtab, stream);
    case 128: return launch_act_b<128, 0, ACT>(src, M, K, ld, inv_sqrt_b, q, s, gtab, stream);
    case 256: return launch_act_b<256, 0, ACT>(src, M, K, ld, inv_sqrt_b, q, s, gtab, stream);
    default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------- tile codes ----

// One thread per 16-byte chunk of the K-tiled output: row n, columns
// 16 c .. 16 c + 15, gathered from row-major [R, C] or transposed [C, R] codes.
__global__ __launch_bounds__(256) void tile_codes_kernel(const int8_t *__restrict__ src,
                                                         bool transposed,
                                                         int8_t *__restrict__ dst, int64_t R,
                                                         int64_t C)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t chunks = C / 16;
    if (i >= R * chunks) return;
    const int64_t n = i / chunks, k = (i % chunks) * 16;
    uint32_t w[4];
    if (!transposed) {
        const uint4 v = *reinterpret_cast<const uint4 *>(src + n * C + k);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t x = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b)
                x |= (uint32_t)(uint8_t)src[(k + 4 * j + b) * R + n] << (8 * b);
            w[j] = x;
        }
    }
    *reinterpret_cast<uint4 *>(dst + tiled_offset(n, k, C)) = make_uint4(w[0], w[1], w[2], w[3]);
}

// ------------------------------------------------------------ transpose ----

template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T *__restrict__ src,
                                                        T *__restrict__ dst,
                                                        int64_t R, int64_t C)
{
    __shared__ T tile[32][33];
    const int64_t c0 = (int64_t)blockIdx.x * 32, r0 = (int64_t)blockIdx.y * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8
#pragma unroll
    for (int k = 0; k < 32; k += 8) {
        const int64_t r = r0 + ty + k, c = c0 + tx;
        if (r < R && c < C) tile[ty + k][tx] = src[r * C + c];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 32; k += 8) {
        const int64_t c = c0 + ty + k, r = r0 + tx;
        if (r < R && c < C) dst[c * R + r] = tile[tx][ty + k];
    }
}

// --------------------------------------------------------- padded copy ----

// dst [Rd, Cd] = src [R, C] in its top-left corner, zeros elsewhere
// (grid-stride over the destination).
template <typename T>
__global__ __launch_bounds__(256) void pad_copy_kernel(const T *__restrict__ src, int64_t R,
                                                       int64_t C, T *__restrict__ dst,
                                                       int64_t Rd, int64_t Cd)
{
    const int64_t n = Rd * Cd, stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
        const int64_t r = i / Cd, c = i % Cd;
        dst[i] = (r < R && c < C) ? src[r * C + c] : T(0);
    }
}

// --------------------------------------------------- SwiGLU interleave ----

// dst row p of a [2F, rows of ru units U] SwiGLU fc1 weight (or of its
// per-row scales, one 4-byte unit per row) = src row swiglu_src_row(p, F).
template <typename U>
__global__ __launch_bounds__(256) void swiglu_interleave_kernel(const U *__restrict__ src,
                                                                U *__restrict__ dst, int64_t F,
                                                                int64_t ru)
{
    const int64_t n = 2 * F * ru, stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
        const int64_t p = i / ru, c = i % ru;
        dst[i] = src[swiglu_src_row(p, F) * ru + c];
    }
}

} // namespace

hipError_t launch_rotquant(const void *src, InType in, int64_t M, int64_t K,
                           int64_t ld, int block, bool regular, float inv_sqrt_b, int8_t *q,
                           float *s, hipStream_t stream)
{
    if (M == 0) return hipSuccess;
    if (in == InType::BF16)
        return launch_in<int(InType::BF16)>(src, M, K, ld, block, regular, inv_sqrt_b, q, s,
                                            stream);
    return launch_in<int(InType::F32)>(src, M, K, ld, block, regular, inv_sqrt_b, q, s, stream);
}

bool rotquant_fuses_gelu(int64_t K)
{
    return K > 12 * kStep && K <= 96 * 256;
}

hipError_t launch_rotquant_gelu(const void *src, int64_t M, int64_t K, int64_t ld, int block,
                                bool regular, float inv_sqrt_b, const uint16_t *gelu_table,
                                int8_t *q, float *s, hipStream_t stream)
{
    if (!rotquant_fuses_gelu(K) || !gelu_table) return hipErrorInvalidValue;
    if (M == 0) return hipSuccess;
    return launch_act<kActGelu>(src, M, K, ld, block, regular, inv_sqrt_b, gelu_table, q, s,
                                stream);
}

hipError_t launch_silu_table(const float **table, hipStream_t stream)
{
    // per device ordinal: the table's address, and whether it has been
    // written (the scheme of the GELU table: the first call outside a graph
    // capture fills it and waits once)
    static std::atomic<const float *> cached[64];
    static std::atomic<int> filled[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool known = dev >= 0 && dev < 64;
    const float *p = known ? cached[dev].load(std::memory_order_relaxed) : nullptr;
    if (!p) {
        void *a = nullptr;
        e = hipGetSymbolAddress(&a, HIP_SYMBOL(g_silu_f32));
        if (e != hipSuccess) return e;
        p = static_cast<const float *>(a);
        if (reinterpret_cast<uintptr_t>(p) & 15) return hipErrorInvalidValue;
        if (known) cached[dev].store(p, std::memory_order_relaxed);
    }
    *table = p;
    if (known && filled[dev].load(std::memory_order_acquire)) return hipSuccess;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(silu_table_kernel, dim3(256), dim3(256), 0, stream);
    e = hipGetLastError();
    if (e != hipSuccess || cap != hipStreamCaptureStatusNone || !known) return e;
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return e;
    filled[dev].store(1, std::memory_order_release);
    if (std::getenv("CONVROT_LOG") && std::getenv("CONVROT_LOG")[0] == '1')
        std::fprintf(stderr, "[convrot] silu table written on device %d\n", dev);
    return hipSuccess;
}

hipError_t launch_swiglu_bf16(const uint16_t *gu, int64_t M, int64_t F, uint16_t *g,
                              hipStream_t stream)
{
    if (M == 0 || F == 0) return hipSuccess;
    if (F % 8 != 0 || ((reinterpret_cast<uintptr_t>(gu) | reinterpret_cast<uintptr_t>(g)) & 15))
        return hipErrorInvalidValue;
    const float *table = nullptr;
    const hipError_t e = launch_silu_table(&table, stream);
    if (e != hipSuccess) return e;
    const int64_t n = M * (F / 8);
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, (int64_t)device_cu_count() * 4);
    hipLaunchKernelGGL(swiglu_apply8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const uint4 *>(gu), reinterpret_cast<uint4 *>(g), M,
                       F / 8);
    return hipGetLastError();
}

hipError_t launch_silu_f32(const uint16_t *a, int64_t n, float *out, hipStream_t stream)
{
    if (n == 0) return hipSuccess;
    const float *table = nullptr;
    const hipError_t e = launch_silu_table(&table, stream);
    if (e != hipSuccess) return e;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, (int64_t)device_cu_count() * 4);
    hipLaunchKernelGGL(silu_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a, out, n);
    return hipGetLastError();
}

hipError_t launch_tile_codes(const int8_t *src, bool transposed, int8_t *dst, int64_t R,
                             int64_t C, hipStream_t stream)
{
    const int64_t n = R * (C / 16);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(tile_codes_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       stream, src, transposed, dst, R, C);
    return hipGetLastError();
}

hipError_t launch_transpose(const void *src, void *dst, int64_t R, int64_t C,
                            int elem_bytes, hipStream_t stream)
{
    if (R == 0 || C == 0) return hipSuccess;
    dim3 grid((unsigned)((C + 31) / 32), (unsigned)((R + 31) / 32));
    switch (elem_bytes) {
    case 1:
        hipLaunchKernelGGL(transpose_kernel<int8_t>, grid, dim3(256), 0, stream,
                           (const int8_t *)src, (int8_t *)dst, R, C);
        break;
    case 2:
        hipLaunchKernelGGL(transpose_kernel<uint16_t>, grid, dim3(256), 0, stream,
                           (const uint16_t *)src, (uint16_t *)dst, R, C);
        break;
    case 4:
        hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(256), 0, stream,
                           (const float *)src, (float *)dst, R, C);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_pad_copy(const void *src, int64_t R, int64_t C, void *dst, int64_t Rd,
                           int64_t Cd, int elem_bytes, hipStream_t stream)
{
    const int64_t n = Rd * Cd;
    if (n == 0) return hipSuccess;
    const unsigned grid = (unsigned)std::min<int64_t>((n + 255) / 256, 8 * device_cu_count());
    switch (elem_bytes) {
    case 2:
        hipLaunchKernelGGL(pad_copy_kernel<uint16_t>, dim3(grid), dim3(256), 0, stream,
                           (const uint16_t *)src, R, C, (uint16_t *)dst, Rd, Cd);
        break;
    case 4:
        hipLaunchKernelGGL(pad_copy_kernel<uint32_t>, dim3(grid), dim3(256), 0, stream,
                           (const uint32_t *)src, R, C, (uint32_t *)dst, Rd, Cd);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_swiglu_interleave(const void *src, void *dst, int64_t F, int64_t K,
                                    int elem_bytes, hipStream_t stream)
{
    const int64_t rb = K * elem_bytes;
    if (F == 0) return hipSuccess;
    if (rb % 4 != 0) return hipErrorInvalidValue;
    // rows move in 16-byte units, or 4-byte ones (a row of one scale)
    const int64_t unit = rb % 16 == 0 ? 16 : 4, ru = rb / unit, n = 2 * F * ru;
    const unsigned grid = (unsigned)std::min<int64_t>((n + 255) / 256, 8 * device_cu_count());
    if (unit == 16)
        hipLaunchKernelGGL(swiglu_interleave_kernel<uint4>, dim3(grid), dim3(256), 0, stream,
                           static_cast<const uint4 *>(src), static_cast<uint4 *>(dst), F, ru);
    else
        hipLaunchKernelGGL(swiglu_interleave_kernel<uint32_t>, dim3(grid), dim3(256), 0, stream,
                           static_cast<const uint32_t *>(src), static_cast<uint32_t *>(dst), F,
                           ru);
    return hipGetLastError();
}

} // namespace convrot
