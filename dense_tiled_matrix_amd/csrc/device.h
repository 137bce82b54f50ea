// device.h -- element access and conversions shared by the gfx950 kernels.
//
// Inputs are decoded exactly to fp32 (fp16 and bf16 are subsets of fp32).
// The fp32 accumulator is converted to the output dtype once, at the store,
// rounding to nearest with ties to even ("Chapter 13: The Blocked Matmul
// Kernel", section 13.3: precision is lost only at the final cast).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dtm_gemm.h"

namespace dtm {

// A debug build (DTM_DEBUG_BARRIERS=1; `python -m dense_tiled_matrix_amd.build
// --debug-barriers` makes libdtm_gemm_debug.so) adds, at the top of every K
// iteration of the LDS-staged GEMM kernels, a wait for every outstanding
// global load and LDS access and then a workgroup barrier.  The arithmetic
// and its order are unchanged, so that build's results are bit-identical to
// the normal build's; a difference exposes a missing wait or barrier.
#ifndef DTM_DEBUG_BARRIERS
#define DTM_DEBUG_BARRIERS 0
#endif
__device__ __forceinline__ void debug_sync()
{
#if DTM_DEBUG_BARRIERS
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt, expcnt and lgkmcnt all 0
    __builtin_amdgcn_s_barrier();
#endif
}

// Problem description passed by value to every kernel.  Strides are in
// elements; pointers address element (0,0) of each view.
struct GemmArgs {
    int64_t M, N, K;
    const void *A;
    int64_t sam, sak;
    const void *B;
    int64_t sbk, sbn;
    void *C;
    int64_t scm, scn;
};

template <int D> struct Elem;
template <> struct Elem<DTM_F32> { using bits = uint32_t; };
template <> struct Elem<DTM_F16> { using bits = uint16_t; };
template <> struct Elem<DTM_BF16> { using bits = uint16_t; };

// Exact fp32 value of element `idx` of a dtype-D array.
template <int D> __device__ __forceinline__ float load_elem(const void *p, int64_t idx)
{
    if constexpr (D == DTM_F32) {
        return static_cast<const float *>(p)[idx];
    } else if constexpr (D == DTM_F16) {
        return static_cast<float>(static_cast<const _Float16 *>(p)[idx]);
    } else {
        const uint32_t b = static_cast<const uint16_t *>(p)[idx];
        return __uint_as_float(b << 16);
    }
}

// fp32 -> bf16 bits, nearest-even; NaN stays a (quiet) NaN, overflow carries
// into the exponent and gives infinity.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v)
{
    const uint32_t u = __float_as_uint(v);
    const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    const uint32_t quiet_nan = (u >> 16) | 0x0040u;
    // a select, not a branch: the epilogue converts many values per lane
    return static_cast<uint16_t>(((u & 0x7fffffffu) > 0x7f800000u) ? quiet_nan : rounded);
}

// fp32 -> fp16 bits, nearest-even (the hardware conversion in the default
// rounding mode), overflow to infinity.
__device__ __forceinline__ uint16_t f32_to_f16_rne(float v)
{
    _Float16 h = static_cast<_Float16>(v);
    return __builtin_bit_cast(uint16_t, h);
}

template <int D> __device__ __forceinline__ void store_elem(void *p, int64_t idx, float v)
{
    if constexpr (D == DTM_F32) {
        static_cast<float *>(p)[idx] = v;
    } else if constexpr (D == DTM_F16) {
        static_cast<uint16_t *>(p)[idx] = f32_to_f16_rne(v);
    } else {
        static_cast<uint16_t *>(p)[idx] = f32_to_bf16_rne(v);
    }
}

__host__ __device__ constexpr int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Map a linear workgroup id onto a tile index so that the workgroups the
// hardware sends to one XCD (ids congruent mod 8) get consecutive tile
// indices.  Bijective on [0, tiles).
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t tiles)
{
    constexpr int64_t XCDS = 8;
    const int64_t xcd = bid % XCDS, local = bid / XCDS;
    const int64_t base = tiles / XCDS, rem = tiles % XCDS;
    return xcd * base + (xcd < rem ? xcd : rem) + local;
}

// Tile index -> (pid_m, pid_n), walking GROUP_M tile-rows at a time so that
// consecutive tiles share rows of A and columns of B.
__device__ __forceinline__ void grouped_tile(int64_t t, int64_t grid_m, int64_t grid_n,
                                             int64_t group_m, int64_t &pid_m, int64_t &pid_n)
{
    const int64_t group_size = group_m * grid_n;
    const int64_t group = t / group_size;
    const int64_t first_m = group * group_m;
    const int64_t gm = (grid_m - first_m) < group_m ? (grid_m - first_m) : group_m;
    const int64_t in_group = t - group * group_size;
    pid_m = first_m + in_group % gm;
    pid_n = in_group / gm;
}

}  // namespace dtm
