// gemm_mfma32.hip -- fp32 GEMM on the gfx950 matrix cores.
//
// The blocked product of "Chapter 13: The Blocked Matmul Kernel" (section
// 13.1: one workgroup per output tile, a K-loop over chunks into an fp32
// accumulator zeroed once; section 13.2: exact zeros outside M, N, K) for
// fp32 operands, with full-precision fp32 products -- no reduced-precision
// input rounding of the kind "Triton matmul" warns about under "Precision"
// (gfx950 has no such fp32 matrix mode).
//
// gfx950 design:
//  * 256 threads = 4 wave64s in 2 x 2; each wave owns (BM/2) x (BN/2) of C
//    as 32 x 32 tiles of v_mfma_f32_32x32x2_f32 (one fp32 of A and one of B
//    per lane per instruction, 16 fp32 results per lane).  Tiles of 128 x 128
//    (64 x 64 per wave, three workgroups per CU), 192 x 192 (96 x 96 per
//    wave, one per CU: for grids the other two fill poorly, 3000^3 86 -> 114
//    TFLOP/s) or 256 x 256 (128 x 128 per wave in the accumulation
//    registers, one workgroup per CU, half the LDS reads per MFMA of the
//    128-wide tile: 4096^3 121 -> 134 TFLOP/s, 8192^3 126 -> 132).
//  * K-chunks 16 deep (32 deep at 192 x 192, and at 256 x 256 unless a plan
//    names 16: 144 KiB of LDS, one barrier and one refill round per 32 k;
//    4096^3 and 8192^3 gained about 1%), two LDS stages, loaded through registers one chunk
//    ahead.  A K-contiguous operand (A row-major, or B given as the
//    transpose of an N x K array) goes to LDS as it is; an M- or
//    N-contiguous one is loaded along its contiguous axis and each thread
//    transposes its 2 x 4 block on the way, so LDS holds both operands
//    k-contiguous, rows padded by 16 bytes (80 or 144 bytes: consecutive
//    rows start in different bank groups).
//  * Which k a lane feeds at each MFMA step is a fixed permutation shared by
//    A and B: lane half h at step s = 4t + e uses k = 8t + 4h + e, so one
//    16-byte LDS read serves four steps.  The sum over k is unchanged.
//  * The RAGGED instantiation zero-fills every slot outside the views.  Its
//    unaligned twin (AL = false) serves views whose base or leading
//    dimension is off a 16-byte boundary, with float-aligned 16-byte loads
//    and element loads at the edges: any fp32 view with a unit stride along
//    one axis runs on the matrix cores.
#include "launch.h"

namespace dtm {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int64_t GROUP_M = 4;

// A chunk is BK k deep (16, or 32 at 256 x 256); an LDS stage row holds BK
// floats of one row or column plus a 16-byte pad.
template <int BK> constexpr int row_floats() { return BK + 4; }

// 4 consecutive floats at p[0..3]; positions >= valid are zero, valid <= 0
// reads nothing.  All four valid: one 16-byte load (AL: p is 16-byte
// aligned; otherwise p is only float-aligned and the copy lets the compiler
// pick the load, which on gfx950 is still one dwordx4: unaligned views
// 4096^3 113 -> 138 TFLOP/s, 2048^3 77 -> 113 against four element loads).
// Fewer valid: element loads.
template <bool AL = true>
__device__ __forceinline__ f32x4 load4_masked(const float *p, int64_t valid)
{
    f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
    if (valid >= 4) {
        if constexpr (AL)
            return *reinterpret_cast<const f32x4 *>(p);
        __builtin_memcpy(&v, p, sizeof(v));
        return v;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (e < valid)
            v[e] = p[e];
    return v;
}

// Global -> registers for the R x BK tile of one operand starting at row
// (or column) mn0 and k0; X addresses element (mn, k) at mn*s_mn + k*s_k and
// the operand has ext rows.  Each of the 256 threads holds R*BK/1024 16-byte
// units (units<BK, R>()):
//  K-contiguous (KC): unit i is chunk t % (BK/4) (k 4c .. 4c+3) of row
//  t / (BK/4) + (1024/BK) i;
//  otherwise: units 2q and 2q+1 are k-rows kk and kk+1 of block b = t + 256 q,
//  kk = 2 (b % (BK/2)), at rows 4 (b / (BK/2)) .. +3 (k-pair fastest:
//  conflict-free LDS writes, and each load instruction reads 8 k-rows x 128
//  contiguous bytes).
// RAGGED: slots outside the view are exact zeros and are never read.  AL:
// every 4-float unit starts on a 16-byte boundary (else element loads; only
// with RAGGED).  load_unit fetches unit i.
template <int BK, int R> constexpr int units() { return R * BK / 1024; }

template <int BK, int R, bool KC, bool RAGGED, bool AL>
__device__ __forceinline__ void load_unit(f32x4 &r, int i, const float *X, int64_t mn0,
                                          int64_t s_mn, int64_t s_k, int64_t ext, int64_t K,
                                          int64_t k0, int t)
{
    if constexpr (KC) {
        const int c = t % (BK / 4), row = t / (BK / 4);
        const int64_t mn = mn0 + row + (1024 / BK) * i;
        const float *src = X + mn * s_mn + k0 + 4 * c;
        if constexpr (RAGGED)
            r = load4_masked<AL>(src, mn < ext ? K - (k0 + 4 * c) : 0);
        else
            r = *reinterpret_cast<const f32x4 *>(src);
    } else {
        const int b = t + 256 * (i >> 1), e = i & 1;
        const int kk = 2 * (b % (BK / 2)), cc = b / (BK / 2);
        const int64_t k = k0 + kk + e;
        const float *src = X + k * s_k + mn0 + 4 * cc;
        if constexpr (RAGGED)
            r = load4_masked<AL>(src, k < K ? ext - (mn0 + 4 * cc) : 0);
        else
            r = *reinterpret_cast<const f32x4 *>(src);
    }
}

// Registers -> the operand's part of an LDS stage (rows of BK + 4 floats, k
// contiguous), unit i; an M/N-contiguous operand's units go in pairs, as a
// transposed 2 x 4 block, at the even index.
template <int BK, int R, bool KC>
__device__ __forceinline__ void store_unit(const f32x4 (&r)[(units<BK, R>())], int i, float *s,
                                           int t)
{
    constexpr int ROW_F = row_floats<BK>();
    if constexpr (KC) {
        const int c = t % (BK / 4), row = t / (BK / 4);
        *reinterpret_cast<f32x4 *>(s + (row + (1024 / BK) * i) * ROW_F + 4 * c) = r[i];
    } else if ((i & 1) == 0) {
        const int b = t + 256 * (i >> 1);
        const int kk = 2 * (b % (BK / 2)), cc = b / (BK / 2);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *reinterpret_cast<f32x2 *>(s + (4 * cc + j) * ROW_F + kk) = f32x2{r[i][j], r[i + 1][j]};
    }
}

template <int BK, int R, bool KC, bool RAGGED, bool AL>
__device__ __forceinline__ void load_operand(f32x4 (&r)[(units<BK, R>())], const float *X,
                                             int64_t mn0, int64_t s_mn, int64_t s_k, int64_t ext,
                                             int64_t K, int64_t k0, int t)
{
#pragma unroll
    for (int i = 0; i < units<BK, R>(); ++i)
        load_unit<BK, R, KC, RAGGED, AL>(r[i], i, X, mn0, s_mn, s_k, ext, K, k0, t);
}

template <int BK, int R, bool KC>
__device__ __forceinline__ void store_operand(const f32x4 (&r)[(units<BK, R>())], float *s, int t)
{
#pragma unroll
    for (int i = 0; i < units<BK, R>(); ++i)
        store_unit<BK, R, KC>(r, i, s, t);
}

// TA: A is M-contiguous (stride_am == 1), else K-contiguous.
// TB: B is K-contiguous (stride_bk == 1), else N-contiguous.
template <int OUT, int BM, int BN, int BK, bool RAGGED, bool TA, bool TB, bool AL = true>
__global__ __launch_bounds__(256) void gemm_mfma32_kernel(GemmArgs p, int64_t grid_m,
                                                          int64_t grid_n)
{
    static_assert(AL || RAGGED, "unaligned operands take the range-checked form");
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int MI = WM / 32, NI = WN / 32;
    constexpr int ROW_F = row_floats<BK>();
    constexpr int A_F = BM * ROW_F;                 // floats of one A stage
    constexpr int STAGE_F = (BM + BN) * ROW_F;
    static_assert(BK == 16 || BK == 32, "chunks of 16 or 32 k");
    static_assert(BM % 64 == 0 && BN % 64 == 0 && units<BK, BM>() % 2 == 0 &&
                      units<BK, BN>() % 2 == 0 && BM * BK % 1024 == 0 && BN * BK % 1024 == 0,
                  "operand tiles split over 256 threads in pairs of 16-byte units");

    // The interior 128 x 128 form reserves 88 KiB of LDS so that it runs one
    // workgroup per CU: three of them per CU ran slower than one (4096^3 on
    // 128-wide tiles 104 against 135 TFLOP/s, 4608^3 109 against 113), while
    // the range-checked form gains from three (6000^3 121 against 101).
    constexpr int LDS_F = BM == 128 && !RAGGED ? 22528 : 2 * STAGE_F;
    static_assert(LDS_F >= 2 * STAGE_F, "two stages");
    __shared__ __attribute__((aligned(16))) float lds[LDS_F];

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    int64_t pid_m, pid_n;
    grouped_tile(xcd_remap(blockIdx.x, grid_m * grid_n), grid_m, grid_n, GROUP_M, pid_m, pid_n);
    const int64_t m0 = pid_m * BM, n0 = pid_n * BN;
    const float *A = static_cast<const float *>(p.A);
    const float *B = static_cast<const float *>(p.B);

    constexpr int UA = units<BK, BM>(), UB = units<BK, BN>(), NU = UA + UB;
    f32x4 ra[UA];
    f32x4 rb[UB];

    auto load_tile = [&](int64_t k0) __attribute__((always_inline)) {
        load_operand<BK, BM, !TA, RAGGED, AL>(ra, A, m0, p.sam, p.sak, p.M, p.K, k0, t);
        load_operand<BK, BN, TB, RAGGED, AL>(rb, B, n0, p.sbn, p.sbk, p.N, p.K, k0, t);
    };
    auto store_tile = [&](int stage) __attribute__((always_inline)) {
        float *sa = lds + stage * STAGE_F;
        store_operand<BK, BM, !TA>(ra, sa, t);
        store_operand<BK, BN, TB>(rb, sa + A_F, t);
    };

    floatx16 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
            acc[i][j] = floatx16{0.0f};

    // lane (row/col lane%32, half h = lane/32) reads 16-byte chunk 2u + h of
    // its row for u < BK/8: k = 8u + 4h + e feeds MFMA step 4u + e.
    const int fr = lane & 31, fh = lane >> 5;
    // One chunk's MFMAs from `stage`; with `pipe`, the next chunk (k0 = kn)
    // is loaded into registers, one 16-byte unit every LS MFMAs, during the
    // first quarter of them, and written to stage `nxt` the same way from
    // 5/8 of them on.  (Issued apart from the MFMAs, the loads and stores
    // took 780 of each chunk's 9565 shader cycles at 256 x 256; interleaved,
    // the chunk takes 9155.  Stores from 1/2 or 3/4 on: level.)
    constexpr int NM = (BK / 8) * 4 * MI * NI;  // MFMAs per chunk
    constexpr int LS = NM / 4 / NU > 0 ? NM / 4 / NU : 1;
    constexpr int SQ0 = NM * 5 / 8;
    auto hook = [&](int q, int64_t kn, int nxt) __attribute__((always_inline)) {
        if (q % LS == 0 && q / LS < NU) {
            const int x = q / LS;
            if (x < UA)
                load_unit<BK, BM, !TA, RAGGED, AL>(ra[x], x, A, m0, p.sam, p.sak, p.M, p.K, kn,
                                                   t);
            else
                load_unit<BK, BN, TB, RAGGED, AL>(rb[x - UA], x - UA, B, n0, p.sbn, p.sbk, p.N,
                                                  p.K, kn, t);
        }
        if (q >= SQ0 && (q - SQ0) % LS == 0 && (q - SQ0) / LS < NU) {
            const int x = (q - SQ0) / LS;
            float *sa = lds + nxt * STAGE_F;
            if (x < UA)
                store_unit<BK, BM, !TA>(ra, x, sa, t);
            else
                store_unit<BK, BN, TB>(rb, x - UA, sa + A_F, t);
        }
    };
    auto is_hook = [&](int q) __attribute__((always_inline)) {
        return (q % LS == 0 && q / LS < NU) ||
               (q >= SQ0 && (q - SQ0) % LS == 0 && (q - SQ0) / LS < NU);
    };
    constexpr int U = BK / 8;             // fragment groups per chunk (even)
    constexpr int QB = (U - 1) * 4 * MI * NI + 3 * MI * NI;  // the barrier's place
    static_assert(SQ0 + (NU - 1) * LS < QB, "every LDS write is issued before the barrier");
    auto read_frag = [&](int stage, int u, f32x4(&fa)[MI], f32x4(&fb)[NI])
                         __attribute__((always_inline)) {
        const float *sa = lds + stage * STAGE_F + (wm * WM + fr) * ROW_F;
        const float *sb = lds + stage * STAGE_F + A_F + (wn * WN + fr) * ROW_F;
#pragma unroll
        for (int i = 0; i < MI; ++i)
            fa[i] = *reinterpret_cast<const f32x4 *>(sa + i * 32 * ROW_F + 4 * (2 * u + fh));
#pragma unroll
        for (int j = 0; j < NI; ++j)
            fb[j] = *reinterpret_cast<const f32x4 *>(sb + j * 32 * ROW_F + 4 * (2 * u + fh));
    };
    auto mfmas = [&](const f32x4(&fa)[MI], const f32x4(&fb)[NI], int u, int e0, int e1, bool pipe,
                     int64_t kn, int nxt) __attribute__((always_inline)) {
#pragma unroll
        for (int e = e0; e < e1; ++e)
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NI; ++j) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i][e], fb[j][e], acc[i][j],
                                                                    0, 0, 0);
                    const int q = ((u * 4 + e) * MI + i) * NI + j;
                    if (pipe && is_hook(q)) {
                        // kept in place: left alone, the compiler sinks
                        // the loads behind the last MFMAs
                        __builtin_amdgcn_sched_barrier(0);
                        hook(q, kn, nxt);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
    };
    // Fragments of group u + 1 are read while group u's MFMAs run; the
    // next chunk's first group is read right after the end-of-chunk
    // barrier, under the chunk's last MI x NI MFMAs, so no chunk starts
    // by waiting on LDS (4096^3 and 8192^3 +1.3%: left to the compiler, the
    // loop began with eight reads and a wait for them).
    f32x4 fa[2][MI], fb[2][NI];

    const int64_t nk = cdiv(p.K, BK);
    load_tile(0);
    store_tile(0);
    __syncthreads();
    read_frag(0, 0, fa[0], fb[0]);
    for (int64_t kt = 0; kt + 1 < nk; ++kt) {
        const int cur = static_cast<int>(kt & 1);
        const int64_t kn = (kt + 1) * BK;
        debug_sync();
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = u & 1;
            if (u + 1 < U) {
                read_frag(cur, u + 1, fa[c ^ 1], fb[c ^ 1]);
                mfmas(fa[c], fb[c], u, 0, 4, true, kn, cur ^ 1);
            } else {
                mfmas(fa[c], fb[c], u, 0, 3, true, kn, cur ^ 1);
                __builtin_amdgcn_sched_barrier(0);
                __syncthreads();
                read_frag(cur ^ 1, 0, fa[c ^ 1], fb[c ^ 1]);
                __builtin_amdgcn_sched_barrier(0);
                mfmas(fa[c], fb[c], u, 3, 4, false, 0, 0);
            }
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = u & 1;
        if (u + 1 < U)
            read_frag(static_cast<int>((nk - 1) & 1), u + 1, fa[c ^ 1], fb[c ^ 1]);
        mfmas(fa[c], fb[c], u, 0, 4, false, 0, 0);
    }

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

template <int OUT, int T, int BK, bool TA, bool TB>
hipError_t launch_tile(const GemmArgs &a, bool ragged, bool aligned, hipStream_t s)
{
    const int64_t gm = cdiv(a.M, T), gn = cdiv(a.N, T);
    const int64_t tiles = gm * gn;
    if (tiles > 0x7fffffffLL)
        return hipErrorInvalidConfiguration;
    if (!aligned)
        hipLaunchKernelGGL((gemm_mfma32_kernel<OUT, T, T, BK, true, TA, TB, false>),
                           dim3((unsigned)tiles), dim3(256), 0, s, a, gm, gn);
    else if (ragged)
        hipLaunchKernelGGL((gemm_mfma32_kernel<OUT, T, T, BK, true, TA, TB>),
                           dim3((unsigned)tiles), dim3(256), 0, s, a, gm, gn);
    else
        hipLaunchKernelGGL((gemm_mfma32_kernel<OUT, T, T, BK, false, TA, TB>),
                           dim3((unsigned)tiles), dim3(256), 0, s, a, gm, gn);
    return hipGetLastError();
}

template <int OUT, int T, int BK>
hipError_t dispatch_layout(const GemmArgs &a, int layout, bool ragged, bool aligned,
                           hipStream_t s)
{
    switch (layout) {
    case 0: return launch_tile<OUT, T, BK, false, false>(a, ragged, aligned, s);
    case DTM_LAYOUT_A_M_CONTIG:
        return launch_tile<OUT, T, BK, true, false>(a, ragged, aligned, s);
    case DTM_LAYOUT_B_K_CONTIG:
        return launch_tile<OUT, T, BK, false, true>(a, ragged, aligned, s);
    case DTM_LAYOUT_A_M_CONTIG | DTM_LAYOUT_B_K_CONTIG:
        return launch_tile<OUT, T, BK, true, true>(a, ragged, aligned, s);
    }
    return hipErrorInvalidValue;
}

// (tile, chunk depth): (256, 32), (256, 16), (192, 32) or (128, 16).
template <int OUT>
hipError_t dispatch_tile(const GemmArgs &a, int tile, int bk, int layout, bool ragged,
                         bool aligned, hipStream_t s)
{
    if (tile == 256)
        return bk == 32 ? dispatch_layout<OUT, 256, 32>(a, layout, ragged, aligned, s)
                        : dispatch_layout<OUT, 256, 16>(a, layout, ragged, aligned, s);
    if (tile == 192)
        return dispatch_layout<OUT, 192, 32>(a, layout, ragged, aligned, s);
    return dispatch_layout<OUT, 128, 16>(a, layout, ragged, aligned, s);
}

}  // namespace

bool mfma32_has_config(int bm, int bn, int bk)
{
    return bm == bn && ((bm == 256 && (bk == 16 || bk == 32)) || (bm == 192 && bk == 32) ||
                        (bm == 128 && bk == 16));
}

hipError_t launch_mfma32(const GemmArgs &a, int out, int bm, int bn, int bk, int layout,
                         bool ragged, bool aligned, hipStream_t s)
{
    if (!mfma32_has_config(bm, bn, bk))
        return hipErrorInvalidConfiguration;
    switch (out) {
    case DTM_F32: return dispatch_tile<DTM_F32>(a, bm, bk, layout, ragged, aligned, s);
    case DTM_F16: return dispatch_tile<DTM_F16>(a, bm, bk, layout, ragged, aligned, s);
    case DTM_BF16: return dispatch_tile<DTM_BF16>(a, bm, bk, layout, ragged, aligned, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace dtm
