// gemm_generic.hip -- the strided/edge GEMM kernel for any layout and dtype.
//
// "Chapter 13: The Blocked Matmul Kernel", sections 13.1 and 13.2: one
// workgroup per BLOCK_M x BLOCK_N output tile; the K-loop stages a
// BLOCK_M x BLOCK_K tile of A and a BLOCK_K x BLOCK_N tile of B in LDS,
// reading element (r,k) at base + r*stride_r + k*stride_c and writing an
// exact zero wherever r >= M, k >= K or c >= N (a select, never a multiply by
// a mask, so NaN or Inf outside the views cannot leak in); each thread then
// adds its TM x TN share of the tile product into fp32 registers that were
// zeroed once before the loop.  The store is masked to i < M, j < N.
//
// This path serves every layout the MFMA kernels do not: transposed and
// broadcast views, leading dimensions that are not 16-byte multiples,
// unaligned bases, and the small forced tiles (4x4x4) of the worked examples.
//
// ACC16 instantiations (fp16 inputs only) reproduce the fp16-accumulator
// variant of section 13.3 as a negative control: each K-chunk's tile product
// is formed in fp32 as above, rounded to fp16, and added into an fp16
// accumulator with an fp16 addition (round to nearest even), so the rounding
// error grows with the number of chunks.
#include "launch.h"

namespace dtm {
namespace {

template <int IN, int OUT, int BM, int BN, int BK, int TM, int TN, bool ACC16>
__global__ __launch_bounds__((BM / TM) * (BN / TN)) void gemm_generic_kernel(GemmArgs p,
                                                                               int64_t grid_n)
{
    static_assert(!ACC16 || IN == DTM_F16, "the fp16 accumulator is for fp16 inputs");
    constexpr int THREADS = (BM / TM) * (BN / TN);
    // k-major tiles: thread (ty, tx) reads TM consecutive A values and TN
    // consecutive B values per k.
    __shared__ float As[BK][BM + 1];
    __shared__ float Bs[BK][BN + 1];

    const int t = threadIdx.x;
    const int64_t tile = blockIdx.x;
    const int64_t m0 = (tile / grid_n) * BM;
    const int64_t n0 = (tile % grid_n) * BN;
    const int tx = t % (BN / TN);
    const int ty = t / (BN / TN);

    // Walk the staged tiles along the operand's unit-stride axis when it has
    // one, so that neighbouring threads read neighbouring addresses.
    const bool a_k_fast = (p.sak == 1) || (p.sam != 1 && (p.sak < 0 ? -p.sak : p.sak) <=
                                                           (p.sam < 0 ? -p.sam : p.sam));
    const bool b_n_fast = (p.sbn == 1) || (p.sbk != 1 && (p.sbn < 0 ? -p.sbn : p.sbn) <=
                                                           (p.sbk < 0 ? -p.sbk : p.sbk));

    float acc[TM][TN];
    _Float16 acc16[TM][TN];  // ACC16 only
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            acc[i][j] = 0.0f;
            acc16[i][j] = static_cast<_Float16>(0.0f);
        }

    for (int64_t k0 = 0; k0 < p.K; k0 += BK) {
        debug_sync();
        for (int e = t; e < BM * BK; e += THREADS) {
            const int r = a_k_fast ? e / BK : e % BM;
            const int c = a_k_fast ? e % BK : e / BM;
            const int64_t gi = m0 + r, gk = k0 + c;
            float v = 0.0f;
            if (gi < p.M && gk < p.K)
                v = load_elem<IN>(p.A, gi * p.sam + gk * p.sak);
            As[c][r] = v;
        }
        for (int e = t; e < BK * BN; e += THREADS) {
            const int c = b_n_fast ? e % BN : e / BK;
            const int r = b_n_fast ? e / BN : e % BK;
            const int64_t gk = k0 + r, gj = n0 + c;
            float v = 0.0f;
            if (gk < p.K && gj < p.N)
                v = load_elem<IN>(p.B, gk * p.sbk + gj * p.sbn);
            Bs[r][c] = v;
        }
        __syncthreads();
#pragma unroll 4
        for (int kk = 0; kk < BK; ++kk) {
            float a[TM], b[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                a[i] = As[kk][ty * TM + i];
#pragma unroll
            for (int j = 0; j < TN; ++j)
                b[j] = Bs[kk][tx * TN + j];
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        }
        if constexpr (ACC16) {
            // the chunk's product, rounded to fp16, then an fp16 addition
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    acc16[i][j] = acc16[i][j] + static_cast<_Float16>(acc[i][j]);
                    acc[i][j] = 0.0f;
                }
        }
        __syncthreads();
    }
    if constexpr (ACC16) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = static_cast<float>(acc16[i][j]);  // exact
    }

#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t gi = m0 + ty * TM + i;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t gj = n0 + tx * TN + j;
            if (gi < p.M && gj < p.N)
                store_elem<OUT>(p.C, gi * p.scm + gj * p.scn, acc[i][j]);
        }
    }
}

template <int IN, int OUT, int BM, int BN, int BK, int TM, int TN, bool ACC16>
hipError_t launch_cfg(const GemmArgs &a, hipStream_t s)
{
    const int64_t gm = cdiv(a.M, BM), gn = cdiv(a.N, BN);
    const int64_t tiles = gm * gn;
    if (tiles > 0x7fffffffLL)
        return hipErrorInvalidConfiguration;
    constexpr int THREADS = (BM / TM) * (BN / TN);
    hipLaunchKernelGGL((gemm_generic_kernel<IN, OUT, BM, BN, BK, TM, TN, ACC16>), dim3((unsigned)tiles),
                       dim3(THREADS), 0, s, a, gn);
    return hipGetLastError();
}

struct Cfg {
    int bm, bn, bk, tm, tn;
};
// The tile shapes this kernel is built for.
constexpr Cfg kConfigs[] = {
    {4, 4, 4, 1, 1}, {16, 16, 16, 1, 1}, {32, 32, 16, 2, 2}, {64, 64, 16, 4, 4}, {128, 128, 8, 8, 8},
};

template <int IN, int OUT, bool ACC16>
hipError_t dispatch_tile(const GemmArgs &a, int bm, int bn, int bk, hipStream_t s)
{
    if (bm == 4 && bn == 4 && bk == 4)
        return launch_cfg<IN, OUT, 4, 4, 4, 1, 1, ACC16>(a, s);
    if (bm == 16 && bn == 16 && bk == 16)
        return launch_cfg<IN, OUT, 16, 16, 16, 1, 1, ACC16>(a, s);
    if (bm == 32 && bn == 32 && bk == 16)
        return launch_cfg<IN, OUT, 32, 32, 16, 2, 2, ACC16>(a, s);
    if (bm == 64 && bn == 64 && bk == 16)
        return launch_cfg<IN, OUT, 64, 64, 16, 4, 4, ACC16>(a, s);
    if (bm == 128 && bn == 128 && bk == 8)
        return launch_cfg<IN, OUT, 128, 128, 8, 8, 8, ACC16>(a, s);
    return hipErrorInvalidConfiguration;
}

template <int IN, bool ACC16>
hipError_t dispatch_out(const GemmArgs &a, int out, int bm, int bn, int bk, hipStream_t s)
{
    switch (out) {
    case DTM_F32: return dispatch_tile<IN, DTM_F32, ACC16>(a, bm, bn, bk, s);
    case DTM_F16: return dispatch_tile<IN, DTM_F16, ACC16>(a, bm, bn, bk, s);
    case DTM_BF16: return dispatch_tile<IN, DTM_BF16, ACC16>(a, bm, bn, bk, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool generic_has_config(int bm, int bn, int bk)
{
    for (const Cfg &c : kConfigs)
        if (c.bm == bm && c.bn == bn && c.bk == bk)
            return true;
    return false;
}

int generic_threads(int bm, int bn, int bk)
{
    for (const Cfg &c : kConfigs)
        if (c.bm == bm && c.bn == bn && c.bk == bk)
            return (c.bm / c.tm) * (c.bn / c.tn);
    return 0;
}

hipError_t launch_generic(const GemmArgs &a, int in, int out, int bm, int bn, int bk,
                          hipStream_t s)
{
    switch (in) {
    case DTM_F32: return dispatch_out<DTM_F32, false>(a, out, bm, bn, bk, s);
    case DTM_F16: return dispatch_out<DTM_F16, false>(a, out, bm, bn, bk, s);
    case DTM_BF16: return dispatch_out<DTM_BF16, false>(a, out, bm, bn, bk, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_generic_fp16acc(const GemmArgs &a, int out, int bm, int bn, int bk,
                                  hipStream_t s)
{
    return dispatch_out<DTM_F16, true>(a, out, bm, bn, bk, s);
}

// ---- K == 0: the empty sum -------------------------------------------------

namespace {
template <int OUT> __global__ __launch_bounds__(256) void zero_fill_kernel(GemmArgs p)
{
    const int64_t total = p.M * p.N;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * 256) {
        const int64_t i = e / p.N, j = e % p.N;
        store_elem<OUT>(p.C, i * p.scm + j * p.scn, 0.0f);
    }
}
}  // namespace

hipError_t launch_zero_fill(const GemmArgs &a, int out, hipStream_t s)
{
    const int64_t total = a.M * a.N;
    const int64_t want = cdiv(total, 256);
    const unsigned blocks = (unsigned)(want < 65536 ? (want > 0 ? want : 1) : 65536);
    switch (out) {
    case DTM_F32: hipLaunchKernelGGL(zero_fill_kernel<DTM_F32>, dim3(blocks), dim3(256), 0, s, a); break;
    case DTM_F16: hipLaunchKernelGGL(zero_fill_kernel<DTM_F16>, dim3(blocks), dim3(256), 0, s, a); break;
    case DTM_BF16: hipLaunchKernelGGL(zero_fill_kernel<DTM_BF16>, dim3(blocks), dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dtm
