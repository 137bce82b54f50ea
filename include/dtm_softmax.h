/*
 * dtm_softmax.h -- C ABI of the row softmax on gfx950 (the second workload).
 *
 * Computes, for every row i < M of an M x N view X,
 *
 *     Y[i][j] = exp(X[i][j] - m_i) / sum over j' < N of exp(X[i][j'] - m_i),
 *     m_i     = max over j < N of X[i][j],
 *
 * the row softmax of "Triton from zero, Lesson 4: Block Pointers",
 * homework 4, where the columns a tile holds past N are masked to -inf so
 * that they neither win the max nor add to the sum.  Arithmetic is fp32 over
 * the exactly decoded inputs; Y is converted once to its dtype (round to
 * nearest, ties to even).  Special values follow the formula's arithmetic:
 * -inf elements give 0; a row of -inf, or one holding +inf or NaN, is NaN.
 *
 * Status codes and dtype codes are those of dtm_gemm.h.
 */
#ifndef DTM_SOFTMAX_H
#define DTM_SOFTMAX_H

#include <stdint.h>

#include "dtm_gemm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Launch forms a plan can name. */
typedef enum {
    DTM_SOFTMAX_NONE = 0,   /* nothing to launch (M == 0 or N == 0) */
    DTM_SOFTMAX_WAVE = 1,   /* one wave64 per row, 4 rows per workgroup, row in registers */
    DTM_SOFTMAX_BLOCK = 2,  /* one 1024-thread workgroup per row, row in registers */
    DTM_SOFTMAX_ONLINE = 3, /* one workgroup per row, running max/sum pass then a write pass */
    DTM_SOFTMAX_SPLIT = 4   /* few long rows: each row cut into `parts` workgroups; a pass
                               writing each part's max/sum to the stream's reserved
                               workspace, then a pass merging them in a fixed order and
                               writing */
} dtm_softmax_form;

/* What row_softmax() would launch.  Produced on the host only. */
typedef struct {
    int32_t form;           /* dtm_softmax_form */
    int32_t threads;        /* threads per workgroup */
    int32_t rows_per_block; /* rows one workgroup handles */
    int32_t chunks;         /* chunks each thread holds (WAVE, BLOCK) or per tile (ONLINE) */
    int32_t chunk_elems;    /* elements per chunk: 16 bytes of input when vectorized, else 1 */
    int32_t vectorized;     /* 1 when rows are unit-stride and 16-byte aligned (16-byte loads) */
    int64_t grid;           /* workgroups */
    int32_t passes;         /* reads of X per element: 1, or 2 for ONLINE and SPLIT */
    int32_t parts;          /* SPLIT: workgroups per row (else 1) */
} dtm_softmax_plan;

/*
 * row_softmax -- Y = softmax over the columns of each row of X.
 * M, N: rows and columns of the views.  X: element (i, j) at
 *   X + i*stride_xm + j*stride_xn (any strides, including 0 or negative).
 * Y: element (i, j) at Y + i*stride_ym + j*stride_yn; the caller owns it; its
 *   strides must not make two (i, j) share an element (DTM_ERR_STRIDE).
 * Y may be exactly X (same pointer, strides and element size: in place);
 *   any other overlap of their byte ranges is DTM_ERR_ALIAS.
 * in_dtype, out_dtype: dtm_dtype of X and Y.  stream: hipStream_t or NULL.
 * The SPLIT form keeps 8*M*parts bytes of statistics in the workspace
 * reserved for (current device, stream) by gemm_workspace_reserve (the one
 * split-K uses); it splits a row only into as many parts as fit there, and
 * with no room for two parts it runs an unsplit form.  Allocates nothing and
 * does not wait for the GPU.
 * With pointer checks on (gemm_set_pointer_checks), X's and Y's byte ranges
 *   must each lie in one device allocation of the current device, else
 *   DTM_ERR_POINTER.
 * Every check runs before any launch; on error nothing is launched.
 * Returns a dtm_status.
 */
int row_softmax(int64_t M, int64_t N, const void *X, int64_t stride_xm, int64_t stride_xn,
                void *Y, int64_t stride_ym, int64_t stride_yn, int in_dtype, int out_dtype,
                void *stream);

/*
 * row_softmax_plan -- validate the arguments of row_softmax() and report the
 * plan it would launch, on the host, without touching a GPU (the SPLIT form's
 * part count as with an unbounded workspace).  Writes *out.
 * Returns the status row_softmax() would return before launching.
 */
int row_softmax_plan(int64_t M, int64_t N, const void *X, int64_t stride_xm, int64_t stride_xn,
                     const void *Y, int64_t stride_ym, int64_t stride_yn, int in_dtype,
                     int out_dtype, dtm_softmax_plan *out);

#ifdef __cplusplus
}
#endif

#endif /* DTM_SOFTMAX_H */
