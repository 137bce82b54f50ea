// gemm_mfma16.hip -- MFMA GEMM for fp16/bf16 inputs on gfx950.
//
// The computation is the blocked product of "Chapter 13: The Blocked Matmul
// Kernel" (section 13.1): one workgroup per BM x BN output tile, a K-loop over
// 64-deep chunks, and an fp32 accumulator zeroed once before the loop
// (section 13.3: it is converted to the output dtype once, at the store).
// Ragged M, N and K (section 13.2) are served by the RAGGED instantiation,
// which replaces every slot outside the views by an exact zero; the other
// instantiation is used only when M, N and K are multiples of the tile
// ("Triton from zero, Lesson 4: Block Pointers", homework 3: check only the
// edges a problem actually has).
//
// gfx950 design:
//  * 256 threads = 4 wave64s in a 2 x 2 arrangement; each wave owns a
//    (BM/2) x (BN/2) block of C as 32 x 32 MFMA tiles
//    (v_mfma_f32_32x32x16_{f16,bf16}: A fragment = 8 k-values of one row per
//    lane, B fragment = 8 k-values of one column per lane, 16 fp32 results
//    per lane).  The accumulators live in the AccVGPR file.
//  * Each operand tile is read from global memory with 16-byte loads along
//    its contiguous axis: K for a K-contiguous operand (A row-major, or B
//    given as the transpose of an N x K array), M or N otherwise.
//  * In LDS both tiles are stored "row x k" with k contiguous, so both
//    fragment reads are single ds_read_b128.  An M- or N-contiguous operand
//    is transposed in registers on the way: each thread loads a KB x 8
//    (k x row) block and writes its columns as k-contiguous runs.  Rows are
//    padded by one 16-byte unit (stride 144 B), which spreads 16 consecutive
//    rows over distinct bank groups for the fragment reads.
//  * Two LDS stages: the global loads for chunk k+1 are issued before the
//    MFMAs of chunk k and written to the other stage after them, with one
//    barrier per chunk.
//  * Workgroup ids are remapped so that each XCD (ids congruent mod 8) owns
//    a compact group of tiles, which keeps A rows and B columns in its L2.
#include "launch.h"

namespace dtm {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16 bytes = 8 elements
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BK = 64;
constexpr int ROW_UNITS = BK / 8 + 1;  // 16-byte units per LDS row (8 data + 1 pad)
constexpr int64_t GROUP_M = 4;

template <int IN>
__device__ __forceinline__ floatx16 mfma(const u32x4 &a, const u32x4 &b, const floatx16 &c)
{
    if constexpr (IN == DTM_F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a),
                                                      __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0,
                                                       0);
}

// 16 bytes = 8 consecutive elements at p[0..7]; elements at positions >= valid
// are zero.  `valid` <= 0 gives all zeros without touching memory.  All
// eight valid: one 16-byte copy, which the compiler emits as one dwordx4
// load also where p is only 4-byte aligned (views whose leading dimension is
// even but off a multiple of 8 elements take this form).
__device__ __forceinline__ u32x4 load8_masked(const uint16_t *p, int64_t valid)
{
    if (valid >= 8) {
        u32x4 v;
        __builtin_memcpy(&v, p, sizeof(v));
        return v;
    }
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (e < valid)
            w[e >> 1] |= static_cast<uint32_t>(p[e]) << (16 * (e & 1));
    return u32x4{w[0], w[1], w[2], w[3]};
}

__device__ __forceinline__ uint32_t half_of(const u32x4 &v, int j)
{
    const uint32_t w = (j >> 1) == 0 ? v.x : (j >> 1) == 1 ? v.y : (j >> 1) == 2 ? v.z : v.w;
    return (j & 1) ? (w >> 16) : (w & 0xffffu);
}

// Global -> registers for the R x BK tile of one operand starting at row
// (or column) mn0 and k0; X addresses element (mn, k) at mn*s_mn + k*s_k and
// the operand has ext rows.  Each of the 256 threads holds R/32 16-byte
// units:
//  K-contiguous (KC): unit i is chunk t%8 (k 8c .. 8c+7) of row t/8 + 32 i;
//  otherwise: unit i is k-row KB*g + i (KB = R/32, g = t % (BK/KB)) at rows
//  8c .. 8c+7, c = t / (BK/KB).
// RAGGED: slots outside the view are exact zeros and are never read.
template <int R, bool KC, bool RAGGED>
__device__ __forceinline__ void load_operand(u32x4 (&r)[R / 32], const uint16_t *X, int64_t mn0,
                                             int64_t s_mn, int64_t s_k, int64_t ext,
                                             int64_t K, int64_t k0, int t)
{
    constexpr int UNITS = R / 32;
    if constexpr (KC) {
        const int c = t & 7, row = t >> 3;
#pragma unroll
        for (int i = 0; i < UNITS; ++i) {
            const int64_t mn = mn0 + row + 32 * i;
            const uint16_t *src = X + mn * s_mn + k0 + 8 * c;
            if constexpr (RAGGED)
                r[i] = load8_masked(src, mn < ext ? K - (k0 + 8 * c) : 0);
            else
                r[i] = *reinterpret_cast<const u32x4 *>(src);
        }
    } else {
        constexpr int KB = UNITS, KG = BK / KB;
        const int g = t % KG, c = t / KG;
#pragma unroll
        for (int i = 0; i < KB; ++i) {
            const int64_t k = k0 + KB * g + i;
            const uint16_t *src = X + k * s_k + mn0 + 8 * c;
            if constexpr (RAGGED)
                r[i] = load8_masked(src, k < K ? ext - (mn0 + 8 * c) : 0);
            else
                r[i] = *reinterpret_cast<const u32x4 *>(src);
        }
    }
}

// Registers -> the operand's part of an LDS stage (rows of ROW_UNITS
// 16-byte units, k contiguous).  An M/N-contiguous KB x 8 block is
// transposed on the way, so that its column j becomes a k-contiguous run in
// LDS row 8c + j.
template <int R, bool KC>
__device__ __forceinline__ void store_operand(const u32x4 (&r)[R / 32], u32x4 *s, int t)
{
    constexpr int UNITS = R / 32;
    if constexpr (KC) {
        const int c = t & 7, row = t >> 3;
#pragma unroll
        for (int i = 0; i < UNITS; ++i)
            s[(row + 32 * i) * ROW_UNITS + c] = r[i];
    } else {
        constexpr int KB = UNITS, KG = BK / KB;
        static_assert(KB == 8 || KB == 4, "the transposed block is 8x8 or 4x8");
        const int g = t % KG, c = t / KG;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int n = 8 * c + j;
            if constexpr (KB == 8) {
                u32x4 v;
                v.x = half_of(r[0], j) | (half_of(r[1], j) << 16);
                v.y = half_of(r[2], j) | (half_of(r[3], j) << 16);
                v.z = half_of(r[4], j) | (half_of(r[5], j) << 16);
                v.w = half_of(r[6], j) | (half_of(r[7], j) << 16);
                s[n * ROW_UNITS + g] = v;
            } else {
                u32x2 v;
                v.x = half_of(r[0], j) | (half_of(r[1], j) << 16);
                v.y = half_of(r[2], j) | (half_of(r[3], j) << 16);
                reinterpret_cast<u32x2 *>(s)[n * (2 * ROW_UNITS) + g] = v;
            }
        }
    }
}

// TA: A is M-contiguous (stride_am == 1), else K-contiguous.
// TB: B is K-contiguous (stride_bk == 1), else N-contiguous.
template <int IN, int OUT, int BM, int BN, bool RAGGED, bool TA, bool TB>
__global__ __launch_bounds__(256) void gemm_mfma16_kernel(GemmArgs p, int64_t grid_m,
                                                          int64_t grid_n)
{
    constexpr int WM = BM / 2, WN = BN / 2;       // wave tile
    constexpr int MI = WM / 32, NI = WN / 32;     // 32x32 MFMA tiles per wave
    constexpr int A_UNITS = BM * ROW_UNITS;
    constexpr int STAGE_UNITS = (BM + BN) * ROW_UNITS;

    __shared__ u32x4 lds[2 * STAGE_UNITS];

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    int64_t pid_m, pid_n;
    grouped_tile(xcd_remap(blockIdx.x, grid_m * grid_n), grid_m, grid_n, GROUP_M, pid_m, pid_n);
    const int64_t m0 = pid_m * BM, n0 = pid_n * BN;

    const uint16_t *A = static_cast<const uint16_t *>(p.A);
    const uint16_t *B = static_cast<const uint16_t *>(p.B);

    u32x4 ra[BM / 32];
    u32x4 rb[BN / 32];

    auto load_tile = [&](int64_t k0) __attribute__((always_inline)) {
        load_operand<BM, !TA, RAGGED>(ra, A, m0, p.sam, p.sak, p.M, p.K, k0, t);
        load_operand<BN, TB, RAGGED>(rb, B, n0, p.sbn, p.sbk, p.N, p.K, k0, t);
    };
    auto store_tile = [&](int stage) __attribute__((always_inline)) {
        u32x4 *sa = lds + stage * STAGE_UNITS;
        store_operand<BM, !TA>(ra, sa, t);
        store_operand<BN, TB>(rb, sa + A_UNITS, t);
    };

    floatx16 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
            acc[i][j] = floatx16{0.0f};

    // LDS fragment addresses of this lane (stage 0, kk = 0).
    const int frag_row = lane & 31, frag_k = lane >> 5;
    const int sa_off = (wm * WM + frag_row) * ROW_UNITS + frag_k;
    const int sb_off = A_UNITS + (wn * WN + frag_row) * ROW_UNITS + frag_k;

    // The tile product of one LDS stage: BK/16 steps of MI x NI MFMAs, with
    // the fragments of step kk+1 read while step kk's MFMAs run.
    auto compute_stage = [&](int stage) __attribute__((always_inline)) {
        const u32x4 *sa = lds + stage * STAGE_UNITS + sa_off;
        const u32x4 *sb = lds + stage * STAGE_UNITS + sb_off;
        u32x4 fa[2][MI], fb[2][NI];
#pragma unroll
        for (int i = 0; i < MI; ++i)
            fa[0][i] = sa[i * 32 * ROW_UNITS];
#pragma unroll
        for (int j = 0; j < NI; ++j)
            fb[0][j] = sb[j * 32 * ROW_UNITS];
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int cur = kk & 1;
            if (kk + 1 < BK / 16) {
#pragma unroll
                for (int i = 0; i < MI; ++i)
                    fa[cur ^ 1][i] = sa[i * 32 * ROW_UNITS + 2 * (kk + 1)];
#pragma unroll
                for (int j = 0; j < NI; ++j)
                    fb[cur ^ 1][j] = sb[j * 32 * ROW_UNITS + 2 * (kk + 1)];
            }
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NI; ++j)
                    acc[i][j] = mfma<IN>(fa[cur][i], fb[cur][j], acc[i][j]);
        }
    };

    // Two LDS stages; the last K-chunk is peeled so the steady-state loop
    // carries no conditionals.
    const int64_t nk = cdiv(p.K, BK);
    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int64_t kt = 0; kt + 1 < nk; ++kt) {
        const int cur = static_cast<int>(kt & 1);
        debug_sync();
        load_tile((kt + 1) * BK);
        // keep the loads issued before the MFMAs so their latency is hidden
        __builtin_amdgcn_sched_barrier(0);
        compute_stage(cur);
        __builtin_amdgcn_sched_barrier(0);
        store_tile(cur ^ 1);
        __syncthreads();
    }
    compute_stage(static_cast<int>((nk - 1) & 1));

    // Epilogue: lane holds column (lane % 32) and rows 8*(v/4) + 4*(lane/32) + v%4
    // of each 32x32 tile.
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int64_t col = n0 + wn * WN + j * 32 + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = m0 + wm * WM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (!RAGGED || (row < p.M && col < p.N))
                    store_elem<OUT>(p.C, row * p.scm + col * p.scn, acc[i][j][v]);
            }
        }
    }
}

template <int IN, int OUT, int BM, int BN, bool TA, bool TB>
hipError_t launch_tile(const GemmArgs &a, bool ragged, hipStream_t s)
{
    const int64_t gm = cdiv(a.M, BM), gn = cdiv(a.N, BN);
    const int64_t tiles = gm * gn;
    if (tiles > 0x7fffffffLL)
        return hipErrorInvalidConfiguration;
    if (ragged)
        hipLaunchKernelGGL((gemm_mfma16_kernel<IN, OUT, BM, BN, true, TA, TB>),
                           dim3((unsigned)tiles), dim3(256), 0, s, a, gm, gn);
    else
        hipLaunchKernelGGL((gemm_mfma16_kernel<IN, OUT, BM, BN, false, TA, TB>),
                           dim3((unsigned)tiles), dim3(256), 0, s, a, gm, gn);
    return hipGetLastError();
}

template <int IN, int OUT, int BM, int BN>
hipError_t dispatch_layout(const GemmArgs &a, int layout, bool ragged, hipStream_t s)
{
    switch (layout) {
    case 0: return launch_tile<IN, OUT, BM, BN, false, false>(a, ragged, s);
    case DTM_LAYOUT_A_M_CONTIG: return launch_tile<IN, OUT, BM, BN, true, false>(a, ragged, s);
    case DTM_LAYOUT_B_K_CONTIG: return launch_tile<IN, OUT, BM, BN, false, true>(a, ragged, s);
    case DTM_LAYOUT_A_M_CONTIG | DTM_LAYOUT_B_K_CONTIG:
        return launch_tile<IN, OUT, BM, BN, true, true>(a, ragged, s);
    }
    return hipErrorInvalidValue;
}

template <int IN, int OUT>
hipError_t dispatch_tile(const GemmArgs &a, int bm, int bn, int layout, bool ragged,
                         hipStream_t s)
{
    if (bm == 256 && bn == 256)
        return dispatch_layout<IN, OUT, 256, 256>(a, layout, ragged, s);
    if (bm == 128 && bn == 128)
        return dispatch_layout<IN, OUT, 128, 128>(a, layout, ragged, s);
    return hipErrorInvalidConfiguration;
}

template <int IN>
hipError_t dispatch_out(const GemmArgs &a, int out, int bm, int bn, int layout, bool ragged,
                        hipStream_t s)
{
    switch (out) {
    case DTM_F32: return dispatch_tile<IN, DTM_F32>(a, bm, bn, layout, ragged, s);
    case DTM_F16: return dispatch_tile<IN, DTM_F16>(a, bm, bn, layout, ragged, s);
    case DTM_BF16: return dispatch_tile<IN, DTM_BF16>(a, bm, bn, layout, ragged, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool mfma16_has_config(int bm, int bn, int bk)
{
    return bk == BK && ((bm == 256 && bn == 256) || (bm == 128 && bn == 128));
}

hipError_t launch_mfma16(const GemmArgs &a, int in, int out, int bm, int bn, int bk, int layout,
                         bool ragged, hipStream_t s)
{
    if (bk != BK)
        return hipErrorInvalidConfiguration;
    switch (in) {
    case DTM_F16: return dispatch_out<DTM_F16>(a, out, bm, bn, layout, ragged, s);
    case DTM_BF16: return dispatch_out<DTM_BF16>(a, out, bm, bn, layout, ragged, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace dtm
