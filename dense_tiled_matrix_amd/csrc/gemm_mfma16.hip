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
//  * A (K-contiguous) and B (N-contiguous) tiles are read from global memory
//    with 16-byte loads, coalesced along each operand's contiguous axis.
//  * In LDS both tiles are stored "row x k" with k contiguous, so both
//    fragment reads are single ds_read_b128.  B arrives N-contiguous; each
//    thread loads a KB x 8 (k x n) block and transposes it in registers
//    before writing it.  Rows are padded by one 16-byte unit (stride 144 B),
//    which spreads 16 consecutive rows over distinct bank groups for the
//    fragment reads.
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
// are zero.  `valid` <= 0 gives all zeros without touching memory.
__device__ __forceinline__ u32x4 load8_masked(const uint16_t *p, int64_t valid)
{
    if (valid >= 8)
        return *reinterpret_cast<const u32x4 *>(p);
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

template <int IN, int OUT, int BM, int BN, bool RAGGED>
__global__ __launch_bounds__(256) void gemm_mfma16_kernel(GemmArgs p, int64_t grid_m,
                                                          int64_t grid_n)
{
    constexpr int WM = BM / 2, WN = BN / 2;       // wave tile
    constexpr int MI = WM / 32, NI = WN / 32;     // 32x32 MFMA tiles per wave
    constexpr int A_UNITS = BM * ROW_UNITS;
    constexpr int STAGE_UNITS = (BM + BN) * ROW_UNITS;
    constexpr int A_LOADS = BM * (BK / 8) / 256;  // 16-byte A chunks per thread
    constexpr int KB = BN / 32;                   // k-rows of the thread's B block
    constexpr int KG = BK / KB;                   // B k-groups
    static_assert(A_LOADS * 256 == BM * (BK / 8), "A tile must split evenly");
    static_assert(KB == 8 || KB == 4, "B block is 8x8 or 4x8");

    __shared__ u32x4 lds[2 * STAGE_UNITS];

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    int64_t pid_m, pid_n;
    grouped_tile(xcd_remap(blockIdx.x, grid_m * grid_n), grid_m, grid_n, GROUP_M, pid_m, pid_n);
    const int64_t m0 = pid_m * BM, n0 = pid_n * BN;

    const uint16_t *A = static_cast<const uint16_t *>(p.A);
    const uint16_t *B = static_cast<const uint16_t *>(p.B);

    // A: thread loads chunk (t % 8) of rows (t / 8) + 32 i.
    const int a_chunk = t & 7, a_row = t >> 3;
    const uint16_t *a_base = A + (m0 + a_row) * p.sam + 8 * a_chunk;
    // B: thread loads rows KB*g .. KB*g+KB-1, columns 8c .. 8c+7.
    const int b_g = t % KG, b_c = t / KG;
    const uint16_t *b_base = B + (int64_t)(KB * b_g) * p.sbk + n0 + 8 * b_c;

    u32x4 ra[A_LOADS];
    u32x4 rb[KB];

    // Global -> registers for the K-chunk starting at k0.
    auto load_tile = [&](int64_t k0) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < A_LOADS; ++i) {
            const uint16_t *src = a_base + (int64_t)(32 * i) * p.sam + k0;
            if constexpr (RAGGED) {
                const bool row_ok = (m0 + a_row + 32 * i) < p.M;
                ra[i] = load8_masked(src, row_ok ? p.K - (k0 + 8 * a_chunk) : 0);
            } else {
                ra[i] = *reinterpret_cast<const u32x4 *>(src);
            }
        }
#pragma unroll
        for (int i = 0; i < KB; ++i) {
            const uint16_t *src = b_base + (k0 + i) * p.sbk;
            if constexpr (RAGGED) {
                const bool k_ok = (k0 + KB * b_g + i) < p.K;
                rb[i] = load8_masked(src, k_ok ? p.N - (n0 + 8 * b_c) : 0);
            } else {
                rb[i] = *reinterpret_cast<const u32x4 *>(src);
            }
        }
    };

    // Registers -> LDS stage; B's KB x 8 block is transposed on the way so
    // that column j becomes a k-contiguous run in LDS row n = 8c + j.
    auto store_tile = [&](int stage) __attribute__((always_inline)) {
        u32x4 *sa = lds + stage * STAGE_UNITS;
        u32x4 *sb = sa + A_UNITS;
#pragma unroll
        for (int i = 0; i < A_LOADS; ++i)
            sa[(a_row + 32 * i) * ROW_UNITS + a_chunk] = ra[i];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int n = 8 * b_c + j;
            if constexpr (KB == 8) {
                u32x4 v;
                v.x = half_of(rb[0], j) | (half_of(rb[1], j) << 16);
                v.y = half_of(rb[2], j) | (half_of(rb[3], j) << 16);
                v.z = half_of(rb[4], j) | (half_of(rb[5], j) << 16);
                v.w = half_of(rb[6], j) | (half_of(rb[7], j) << 16);
                sb[n * ROW_UNITS + b_g] = v;
            } else {
                u32x2 v;
                v.x = half_of(rb[0], j) | (half_of(rb[1], j) << 16);
                v.y = half_of(rb[2], j) | (half_of(rb[3], j) << 16);
                reinterpret_cast<u32x2 *>(sb)[n * (2 * ROW_UNITS) + b_g] = v;
            }
        }
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

template <int IN, int OUT, int BM, int BN>
hipError_t launch_tile(const GemmArgs &a, bool ragged, hipStream_t s)
{
    const int64_t gm = cdiv(a.M, BM), gn = cdiv(a.N, BN);
    const int64_t tiles = gm * gn;
    if (tiles > 0x7fffffffLL)
        return hipErrorInvalidConfiguration;
    if (ragged)
        hipLaunchKernelGGL((gemm_mfma16_kernel<IN, OUT, BM, BN, true>), dim3((unsigned)tiles),
                           dim3(256), 0, s, a, gm, gn);
    else
        hipLaunchKernelGGL((gemm_mfma16_kernel<IN, OUT, BM, BN, false>), dim3((unsigned)tiles),
                           dim3(256), 0, s, a, gm, gn);
    return hipGetLastError();
}

template <int IN, int OUT>
hipError_t dispatch_tile(const GemmArgs &a, int bm, int bn, bool ragged, hipStream_t s)
{
    if (bm == 256 && bn == 256)
        return launch_tile<IN, OUT, 256, 256>(a, ragged, s);
    if (bm == 128 && bn == 128)
        return launch_tile<IN, OUT, 128, 128>(a, ragged, s);
    return hipErrorInvalidConfiguration;
}

template <int IN>
hipError_t dispatch_out(const GemmArgs &a, int out, int bm, int bn, bool ragged, hipStream_t s)
{
    switch (out) {
    case DTM_F32: return dispatch_tile<IN, DTM_F32>(a, bm, bn, ragged, s);
    case DTM_F16: return dispatch_tile<IN, DTM_F16>(a, bm, bn, ragged, s);
    case DTM_BF16: return dispatch_tile<IN, DTM_BF16>(a, bm, bn, ragged, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool mfma16_has_config(int bm, int bn, int bk)
{
    return bk == BK && ((bm == 256 && bn == 256) || (bm == 128 && bn == 128));
}

hipError_t launch_mfma16(const GemmArgs &a, int in, int out, int bm, int bn, int bk, bool ragged,
                         hipStream_t s)
{
    if (bk != BK)
        return hipErrorInvalidConfiguration;
    switch (in) {
    case DTM_F16: return dispatch_out<DTM_F16>(a, out, bm, bn, ragged, s);
    case DTM_BF16: return dispatch_out<DTM_BF16>(a, out, bm, bn, ragged, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace dtm
