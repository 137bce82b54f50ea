// gemm_splitk.hip -- second pass of split-K: C = sum of the fp32 partial
// tiles, in slice order, converted once to the output dtype.
//
// "Chapter 13: The Blocked Matmul Kernel", section 13.3 keeps the running
// sum in fp32 and converts only at the store.  With K split into S slices
// each slice has its own fp32 accumulator (zeroed once, section 13.1); this
// pass adds the S partial sums in fp32 in the fixed order s = 0, 1, ..., S-1
// (the result does not depend on scheduling) and converts once.
#include "launch.h"

namespace dtm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Each thread reduces 4 consecutive columns of one row (N % 4 == 0, so the
// 16-byte loads of every slice are aligned).
template <int OUT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs p, int64_t splits,
                                                            const float *__restrict__ ws)
{
    const int64_t MN = p.M * p.N;
    const int64_t groups_per_row = p.N / 4;
    const int64_t groups = p.M * groups_per_row;
    for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < groups;
         g += (int64_t)gridDim.x * 256) {
        const int64_t i = g / groups_per_row;
        const int64_t j = (g - i * groups_per_row) * 4;
        const int64_t e = i * p.N + j;
        const float *src = ws + e;
        f32x4 acc = *reinterpret_cast<const f32x4 *>(src);
        int64_t s = 1;
        // Loads of BATCH slices are issued together (memory-level
        // parallelism), then added one by one in slice order.
        constexpr int BATCH = 8;
        for (; s + BATCH <= splits; s += BATCH) {
            f32x4 v[BATCH];
#pragma unroll
            for (int q = 0; q < BATCH; ++q)
                v[q] = *reinterpret_cast<const f32x4 *>(src + (s + q) * MN);
#pragma unroll
            for (int q = 0; q < BATCH; ++q)
                acc += v[q];
        }
        for (; s < splits; ++s)
            acc += *reinterpret_cast<const f32x4 *>(src + s * MN);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            store_elem<OUT>(p.C, i * p.scm + (j + q) * p.scn, acc[q]);
    }
}

}  // namespace

hipError_t launch_splitk_reduce(const GemmArgs &a, int out, int64_t splits, const float *ws,
                                hipStream_t s)
{
    if (a.N % 4 != 0 || splits < 1)
        return hipErrorInvalidConfiguration;
    const int64_t groups = a.M * (a.N / 4);
    const int64_t want = cdiv(groups, 256);
    const unsigned blocks = (unsigned)(want < 4096 ? (want > 0 ? want : 1) : 4096);
    switch (out) {
    case DTM_F32:
        hipLaunchKernelGGL(splitk_reduce_kernel<DTM_F32>, dim3(blocks), dim3(256), 0, s, a, splits,
                           ws);
        break;
    case DTM_F16:
        hipLaunchKernelGGL(splitk_reduce_kernel<DTM_F16>, dim3(blocks), dim3(256), 0, s, a, splits,
                           ws);
        break;
    case DTM_BF16:
        hipLaunchKernelGGL(splitk_reduce_kernel<DTM_BF16>, dim3(blocks), dim3(256), 0, s, a, splits,
                           ws);
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dtm
