// launch.h -- host-side launchers of the gfx950 kernels (internal).
#pragma once

#include <hip/hip_runtime.h>

#include "device.h"

namespace dtm {

// Generic strided kernel: any strides, any dtype pair, tiles from the fixed
// list below.  Returns false when (bm, bn, bk) is not one of them.
bool generic_has_config(int bm, int bn, int bk);
int generic_threads(int bm, int bn, int bk);
hipError_t launch_generic(const GemmArgs &a, int in_dtype, int out_dtype, int bm, int bn, int bk,
                          hipStream_t s);
// The same kernel with the fp16 accumulator of the negative control (fp16
// inputs): every K-chunk product rounded to fp16 and added in fp16.
hipError_t launch_generic_fp16acc(const GemmArgs &a, int out_dtype, int bm, int bn, int bk,
                                  hipStream_t s);

// Register-staged MFMA kernel for fp16/bf16 inputs in every operand layout
// (`layout`: dtm_layout bits); any M, N, K (edge tiles masked).
bool mfma16_has_config(int bm, int bn, int bk);
hipError_t launch_mfma16(const GemmArgs &a, int in_dtype, int out_dtype, int bm, int bn, int bk,
                         int layout, bool ragged, hipStream_t s);

// Deep-pipelined MFMA kernel (tile x tile x 32 tiles, tile 256, 192 or 128,
// global -> LDS DMA) when M and N are multiples of the tile and K of 32, for
// every operand layout: `layout` holds dtm_layout bits (A M-contiguous, B
// K-contiguous).  `waves` per workgroup: at tile 256, 8 (each owns 128 x 64
// of the tile, two waves per SIMD) or 4 (128 x 128 each, one wave per SIMD:
// a third fewer LDS reads per MFMA; the interior form only); at tile 192, 4
// (96 x 96 each; 96 KiB of LDS, one workgroup per CU); at tile 128, 4
// (64 x 64 each; 64 KiB of LDS, so two workgroups share a CU).
bool mfma16_dma_fits(int64_t M, int64_t N, int64_t K, int64_t splits, int tile);
bool mfma16_dma_waves_ok(int tile, int waves, bool ragged);
hipError_t launch_mfma16_dma(const GemmArgs &a, int in_dtype, int out_dtype, int layout, int tile,
                             int waves, hipStream_t s);
// The same kernel on ragged shapes (its range-checked form): any M and N,
// K % 8 == 0, an M-contiguous A needs M % 8 == 0 and an N-contiguous B
// N % 8 == 0; both views non-negatively strided and at most 2^31 bytes
// (a_bytes, b_bytes: the byte extents of the views).  With splits > 1 the
// slices hold cdiv(K, splits) rounded up to 32 (the last may be shorter,
// none empty) and N % 4 == 0 (the second pass reads 4 columns at a time).
bool mfma16_dma_ragged_fits(int64_t M, int64_t N, int64_t K, int layout, uint64_t a_bytes,
                            uint64_t b_bytes, int64_t splits, int tile);
hipError_t launch_mfma16_dma_ragged(const GemmArgs &a, int in_dtype, int out_dtype, int layout,
                                    uint64_t a_bytes, uint64_t b_bytes, int tile, int waves,
                                    hipStream_t s);
// Split-K on the same kernel (either form): fp32 partial tiles written
// densely to ws[splits][M][N] (a.C and its strides are not used).
hipError_t launch_mfma16_dma_partials(const GemmArgs &a, int in_dtype, int layout, int64_t splits,
                                      bool ragged, uint64_t a_bytes, uint64_t b_bytes, int tile,
                                      int waves, float *ws, hipStream_t s);
// 128 x 128 tiles whose 4 waves split the K loop (interior shapes only:
// M, N multiples of 128, K of 128 * splits; non-negative strides within the
// buffer-load span).  Direct: C in out_dtype; partials: fp32 ws[splits][M][N].
bool mfma16_wavek_fits(const GemmArgs &a, int layout, int64_t splits);
hipError_t launch_mfma16_wavek(const GemmArgs &a, int in_dtype, int out_dtype, int layout,
                               hipStream_t s);
hipError_t launch_mfma16_wavek_partials(const GemmArgs &a, int in_dtype, int layout,
                                        int64_t splits, float *ws, hipStream_t s);
// C = sum over s of ws[s] in order s = 0, 1, ..., converted once to out_dtype.
hipError_t launch_splitk_reduce(const GemmArgs &a, int out_dtype, int64_t splits, const float *ws,
                                hipStream_t s);

// MFMA kernel for fp32 inputs in every operand layout (128 x 128 x 16 tiles).
bool mfma32_has_config(int bm, int bn, int bk);
// aligned: both operands' bases and leading dimensions on 16-byte
// boundaries; otherwise the range-checked form with element loads.
hipError_t launch_mfma32(const GemmArgs &a, int out_dtype, int bm, int bn, int bk, int layout,
                         bool ragged, bool aligned, hipStream_t s);

// One MFMA of the pipelined kernels on a 16 x 32 A and a 32 x 16 B, through
// their LDS staging, fragment reads and epilogue lane map (layout: dtm_layout
// bits; pair: the paired-stage row layout).  C: 16 x 16 fp32, row-major.
hipError_t launch_mfma_probe(int in_dtype, int layout, bool pair, const void *A, const void *B,
                             float *C, hipStream_t s);

// Writes zeros to the M x N view of C (the K == 0 product).
hipError_t launch_zero_fill(const GemmArgs &a, int out_dtype, hipStream_t s);

}  // namespace dtm
