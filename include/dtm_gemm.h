/*
 * dtm_gemm.h -- C ABI of libdtm_gemm.so, a blocked GEMM C = A.B for AMD
 * MI355X (gfx950).
 *
 * The operation.  "Chapter 13: The Blocked Matmul Kernel" (Triton from first
 * principles), section 13.1: a 2-D grid of BLOCK_M x BLOCK_N output tiles;
 * each tile walks the shared dimension K in BLOCK_K chunks and adds every
 * chunk's tile product into one fp32 accumulator that is initialised once,
 * before the loop.  Section 13.2: rows >= M, columns >= N and k >= K are
 * masked so that they contribute exact zeros.  Section 13.3: the accumulator
 * stays fp32 whatever the input dtype and is converted to the output dtype
 * once, at the store.  Operands are strided row/column views as in the
 * section 13.1 kernel signature (stride_am, stride_ak, stride_bk, stride_bn,
 * stride_cm, stride_cn), with strides counted in elements, not bytes
 * ("Triton from zero, Lesson 4: Block Pointers", section 2).  The result is
 *
 *     C[i][j] = sum over k in [0, K) of A[i][k] * B[k][j],  0 <= i < M, 0 <= j < N,
 *
 * with fp32 products and sums and one round-to-nearest-even conversion of
 * the fp32 accumulator to out_dtype.
 *
 * Conventions shared by every entry point below.
 *   - Element (i,k) of A is at A + i*stride_am + k*stride_ak, element (k,j)
 *     of B at B + k*stride_bk + j*stride_bn, element (i,j) of C at
 *     C + i*stride_cm + j*stride_cn (all in elements of the operand's dtype).
 *   - A and B share in_dtype.  C has out_dtype.  The accumulator is fp32.
 *   - C is overwritten (no alpha/beta, no accumulate-into-C).  Nothing of C's
 *     allocation outside the M x N view is written.
 *   - All pointers are device memory on the current HIP device, owned by the
 *     caller.  The library keeps no pointer after a call returns.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream)
 *     and the call returns without waiting; the result is visible once the
 *     caller synchronises that stream.  gemm, gemm_ex and row_softmax never
 *     allocate or free device memory and never wait for the GPU: the only
 *     device memory they use beyond the caller's views is a workspace the
 *     caller passes (gemm_ex) or reserved beforehand for the stream with
 *     gemm_workspace_reserve.  (The HIP runtime itself loads a kernel's
 *     code object on that kernel's first launch in the process; code that
 *     must not see even that, such as a stream capture, runs each plan once
 *     beforehand.)  Calls are thread-safe: calls on one stream that use its
 *     reserved workspace queue their launches one call at a time.
 *   - Every argument check runs on the host before anything is launched; on
 *     a non-zero status nothing was launched and C is untouched.
 *   - A and B may have any strides, including zero (broadcast), negative and
 *     transposed views.  Layouts the MFMA kernels do not cover run on the
 *     generic strided kernel instead of being rejected.  The library cannot
 *     check that pointers and strides stay inside the caller's allocations.
 *   - M == 0 or N == 0 is a successful no-op.  K == 0 writes zeros (the empty
 *     sum) to the M x N view of C.
 *   - Sweeps: the environment variable DTM_GEMM_FORCE, read once when the
 *     library is loaded, gives a tile configuration to every call that passes
 *     none (gemm(); gemm_plan(), gemm_ex() and gemm_ex_noalloc() with
 *     force == NULL).  Comma-separated fields: "BMxBNxBK" for the tile, and
 *     kernel=<dtm_kernel number or gemm_kernel_name>, split=<S>,
 *     threads=<T>, dp_rows=<R>, with the meaning of dtm_tile_config's fields
 *     (e.g. DTM_GEMM_FORCE=128x128x32,split=4).  Unset or empty: off.  A value
 *     that does not parse makes those calls return DTM_ERR_CONFIG.
 */
#ifndef DTM_GEMM_H
#define DTM_GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. */
typedef enum {
    DTM_F32 = 0,  /* IEEE binary32 */
    DTM_F16 = 1,  /* IEEE binary16 */
    DTM_BF16 = 2  /* bfloat16: the upper 16 bits of a binary32 */
} dtm_dtype;

/* Status codes returned by every entry point. */
typedef enum {
    DTM_OK = 0,
    DTM_ERR_INVALID_DIM = 1,  /* M, N or K negative or above 2^31-1 */
    DTM_ERR_NULL_POINTER = 2, /* a needed pointer (A, B, C or an out-parameter) is NULL */
    DTM_ERR_DTYPE = 3,        /* in_dtype or out_dtype is not a dtm_dtype */
    DTM_ERR_STRIDE = 4,       /* C strides negative or making two (i,j) share an element,
                                 or a view whose address range overflows 64 bits */
    DTM_ERR_ALIAS = 5,        /* C's address range intersects A's or B's */
    DTM_ERR_CONFIG = 6,       /* a forced tile configuration that does not exist or
                                 cannot serve this problem */
    DTM_ERR_WORKSPACE = 7,    /* workspace smaller than a forced split needs, or
                                 gemm_workspace_reserve could not allocate */
    DTM_ERR_DEVICE = 8,       /* the current device is not gfx950 or cannot be queried */
    DTM_ERR_LAUNCH = 9,       /* the HIP runtime reported an error when launching */
    DTM_ERR_POINTER = 10,     /* pointer checks on (gemm_set_pointer_checks): a view's
                                 byte range is not inside one device-memory allocation of
                                 the current device */
    DTM_ERR_SCRATCH = 11      /* gemm_ex_noalloc: the plan needs more split-K scratch than
                                 its fixed array holds (gemm_noalloc_scratch_bytes) */
} dtm_status;

/* Kernels a plan can name. */
typedef enum {
    DTM_KERNEL_NONE = 0,      /* nothing to launch (M == 0 or N == 0) */
    DTM_KERNEL_ZERO_FILL = 1, /* K == 0: write zeros to C */
    DTM_KERNEL_GENERIC = 2,   /* any strides and dtypes; fp32 FMA on LDS tiles */
    DTM_KERNEL_MFMA_F16 = 3,  /* fp16/bf16 inputs on MFMA (layouts: dtm_layout) */
    DTM_KERNEL_MFMA_F32 = 4,  /* fp32 inputs on fp32 MFMA (one unit stride per operand) */
    DTM_KERNEL_GENERIC_FP16ACC = 5, /* negative control, only when forced through gemm_ex and
                                      gemm_plan: fp16 inputs, the generic kernel with the
                                      fp16 accumulator of "Chapter 13: The Blocked Matmul
                                      Kernel", section 13.3 -- each BLOCK_K chunk's tile
                                      product (fp32) is rounded to fp16 and added into an
                                      fp16 accumulator; not a correct GEMM, it shows the
                                      accumulation error the fp32 accumulator avoids */
    DTM_KERNEL_MFMA_F16_WAVEK = 6 /* fp16/bf16 inputs on MFMA, 128 x 128 x 32 tiles whose 4
                                     waves each accumulate the whole tile over every fourth
                                     32-deep chunk of the K loop ("Chapter 13", section
                                     13.1's K loop, split four ways inside the workgroup),
                                     summed in LDS in a fixed order; M and N multiples of
                                     128, K of 128 * split_k, no dp_rows */
} dtm_kernel;

/* Operand layouts the MFMA kernels read at full speed (bits of
 * dtm_plan.layout).  Each operand must have one unit stride; for the
 * pipelined fp16/bf16 kernels its other stride (the leading dimension) must
 * be a multiple of 16 bytes and its base 16-byte aligned; fp16/bf16 views
 * with an even leading dimension and a 4-byte-aligned base run on the
 * register-staged kernel's range-checked form, and fp32 views off those
 * boundaries on the fp32 kernel's range-checked form.  With neither bit set, A
 * is K-contiguous (stride_ak == 1) and B is N-contiguous (stride_bn == 1):
 * both row-major.  A transposed view sets a bit.  Any other layout runs on
 * the generic kernel. */
typedef enum {
    DTM_LAYOUT_A_M_CONTIG = 1, /* A has stride_am == 1 (e.g. the transpose of a K x M array) */
    DTM_LAYOUT_B_K_CONTIG = 2  /* B has stride_bk == 1 (e.g. the transpose of an N x K array) */
} dtm_layout;

/* A tile configuration.  Zero fields mean "the selector chooses". */
typedef struct {
    int32_t kernel;  /* dtm_kernel, or 0 */
    int32_t block_m; /* BLOCK_M x BLOCK_N output tile, BLOCK_K chunk of K */
    int32_t block_n;
    int32_t block_k;
    int32_t split_k; /* number of K slices summed by a second pass; 0 or 1 = none */
    int32_t threads; /* workgroup size of the pipelined MFMA kernel (block_k 32): at
                        256 x 256, 512 (8 waves) or 256 (4 waves, not on its range-checked
                        form); at 192 x 192 and 128 x 128, 256; must be 0 for any other
                        kernel or tile */
    int32_t dp_rows; /* with split_k > 1 on the pipelined kernel: the first dp_rows rows
                        of C (a multiple of block_m, below M) run unsplit and only the
                        rows below them in split_k slices; 0 = every row split */
    uint64_t workspace_limit; /* bytes of workspace the selector may plan for (it splits K
                                 only as far as the partials fit); 0 = no limit beyond the
                                 workspace the call has.  A forced split_k is not capped. */
} dtm_tile_config;

/* What gemm() would launch for a problem.  Produced on the host only. */
typedef struct {
    int32_t kernel;           /* dtm_kernel */
    int32_t block_m, block_n, block_k;
    int64_t grid_m;           /* cdiv(M, block_m) output tiles along M */
    int64_t grid_n;           /* cdiv(N, block_n) output tiles along N */
    int64_t k_iters;          /* K-loop trip count of one tile: cdiv(K_slice, block_k) */
    int32_t split_k;          /* K slices (1 = the whole K in one accumulator) */
    int32_t threads;          /* threads per workgroup */
    int32_t fast_path;        /* 1 when a matrix-core kernel's layout predicate holds:
                                 fp16/bf16 one unit stride per operand, the other
                                 stride even and the base 4-byte aligned (16-byte
                                 boundaries for the pipelined kernels; dtm_layout);
                                 fp32 one unit stride per operand, any alignment */
    int32_t ragged;           /* 1 when M, N or K is not a multiple of its block */
    int32_t layout;           /* dtm_layout bits of the operands (MFMA kernels; 0 otherwise) */
    uint64_t workspace_bytes; /* device scratch the plan needs (split-K partials) */
    int64_t dp_rows;          /* with split_k > 1: rows [0, dp_rows) run unsplit in full
                                 rounds of tiles, rows [dp_rows, M) in split_k slices
                                 (k_iters counts a slice); 0 = every row split */
} dtm_plan;

/*
 * gemm -- C = A.B (the computation stated at the top of this header), the
 * host wrapper of "Chapter 13: The Blocked Matmul Kernel", section 13.1: the
 * caller owns C, K is the logical shared dimension (independent of the
 * storage A and B are views into, as in section 13.2's sentinel example) and
 * the output dtype is the caller's choice (section 13.3).
 * in_dtype: dtype of A and B; out_dtype: dtype of C.  stream: hipStream_t or
 * NULL.
 * The library picks the kernel and tile with its selector.  A plan that
 * splits K keeps fp32 partials in the workspace reserved for (current
 * device, stream) by gemm_workspace_reserve; the selector splits only as far
 * as they fit there (with nothing reserved, it does not split).  Allocates
 * nothing, frees nothing and does not wait for the GPU.  A plan with
 * dtm_plan.dp_rows > 0 runs as launches in stream order on row ranges of the
 * same views: the unsplit top rows, then the split rows and their sum.
 * Returns a dtm_status.
 */
int gemm(int64_t M, int64_t N, int64_t K,
         const void *A, int64_t stride_am, int64_t stride_ak,
         const void *B, int64_t stride_bk, int64_t stride_bn,
         void *C, int64_t stride_cm, int64_t stride_cn,
         int in_dtype, int out_dtype, void *stream);

/*
 * gemm_plan -- validate the arguments of gemm() and report the plan it would
 * launch, on the host, without touching a GPU: the launch grid
 * (cdiv(M, BLOCK_M), cdiv(N, BLOCK_N)) and the K-loop trip count
 * cdiv(K, BLOCK_K) of "Chapter 13: The Blocked Matmul Kernel", section 13.1
 * (Worked Example 13.1.1: grid (2, 2) with 2 K-iterations for M = N = K = 8
 * on 4 x 4 x 4 tiles).  `force` may be NULL (the selector decides) or a
 * configuration as for gemm_ex().  The plan is the one gemm_ex() runs with a
 * caller's workspace of at least plan.workspace_bytes, and the one gemm()
 * runs when the stream's reserved workspace is at least that large; with a
 * smaller workspace the selector splits K less (force->workspace_limit shows
 * that plan).  Writes *out.  Returns the status gemm()/gemm_ex() would
 * return before launching.
 */
int gemm_plan(int64_t M, int64_t N, int64_t K,
              const void *A, int64_t stride_am, int64_t stride_ak,
              const void *B, int64_t stride_bk, int64_t stride_bn,
              const void *C, int64_t stride_cm, int64_t stride_cn,
              int in_dtype, int out_dtype,
              const dtm_tile_config *force, dtm_plan *out);

/*
 * gemm_ex -- gemm() with a forced tile configuration and an optional
 * caller-owned workspace.  The tile sizes are the BLOCK_M, BLOCK_N, BLOCK_K
 * meta-parameters of "Chapter 13: The Blocked Matmul Kernel", section 13.1,
 * which that chapter's worked examples set by hand (4 x 4 x 4 in Worked
 * Example 13.1.1).
 * force: NULL or a dtm_tile_config whose non-zero fields override the
 *   selector (for example {DTM_KERNEL_GENERIC, 4, 4, 4, 0, 0, 0, 0} runs 4x4x4
 *   tiles).  A configuration the library does not have, or an MFMA kernel
 *   for a layout it cannot serve, gives DTM_ERR_CONFIG.
 * workspace, workspace_bytes: device memory (16-byte aligned) the plan may
 *   use for split-K partials; the selector splits K only as far as they fit.
 *   NULL means the workspace reserved for the stream (gemm_workspace_reserve),
 *   as in gemm().  A forced split_k needing more than the workspace gives
 *   DTM_ERR_WORKSPACE.  A caller's workspace must not be in use by other
 *   work that can run concurrently on the device.
 * Allocates nothing and does not wait for the GPU.  Returns a dtm_status.
 */
int gemm_ex(int64_t M, int64_t N, int64_t K,
            const void *A, int64_t stride_am, int64_t stride_ak,
            const void *B, int64_t stride_bk, int64_t stride_bn,
            void *C, int64_t stride_cm, int64_t stride_cn,
            int in_dtype, int out_dtype,
            const dtm_tile_config *force, void *workspace, uint64_t workspace_bytes,
            void *stream);

/*
 * gemm_workspace_reserve -- make sure the library holds at least `bytes` of
 * device workspace for (current device, stream), for the split-K partials
 * of gemm()/gemm_ex() and the split-row statistics of row_softmax() on that
 * stream.  Unlike those calls it may allocate, and when it replaces a
 * smaller buffer it first waits for the stream's earlier work.  Call it
 * outside any code that must not allocate (for example before a graph
 * capture).  Never shrinks.  Returns DTM_OK, or DTM_ERR_WORKSPACE when the
 * allocation (or the wait) fails, leaving nothing reserved.
 * (The splitting it serves is not on the pages: "Chapter 13: The Blocked
 * Matmul Kernel", section 13.1 gives each tile one accumulator over the
 * whole K; split-K gives each K slice its own fp32 accumulator and sums
 * them in fp32, section 13.3's accumulation precision.)
 */
int gemm_workspace_reserve(uint64_t bytes, void *stream);

/* gemm_workspace_release -- wait for the stream, then free its reserved
 * workspace (later calls on it plan without one).  Returns DTM_OK or
 * DTM_ERR_WORKSPACE when the wait fails. */
int gemm_workspace_release(void *stream);

/* gemm_workspace_reserved -- bytes reserved for (current device, stream);
 * 0 when none. */
uint64_t gemm_workspace_reserved(void *stream);

/*
 * gemm_ex_noalloc -- gemm_ex() for callers that cannot allocate device
 * memory at all, not even once beforehand with gemm_workspace_reserve: code
 * recorded under stream capture, serving loops and hosts that forbid
 * allocation.  The same arguments as gemm_ex() without the workspace: a plan
 * that splits K keeps its fp32 partials in a fixed array of device memory
 * that is part of the library (gemm_noalloc_scratch_bytes() bytes, 32 MiB;
 * each GPU the library runs on holds its own copy until the process ends).
 * The selector splits only as far as the partials fit in it; a forced
 * split_k that needs more returns DTM_ERR_SCRATCH before anything is
 * launched.  The first call on a device looks up that device's copy of the
 * array (no allocation); no call allocates, frees or waits for the GPU.
 * Every call on a GPU uses that GPU's one array: calls that overlap on one
 * GPU (other streams, other threads) race on it and must be serialised by
 * the caller.  Results equal gemm_ex()'s with the same plan.  The HIP
 * runtime still takes device memory for a kernel's code on that kernel's
 * first launch in the process (as through any entry point): launch each
 * plan once beforehand where device memory must not move.  Returns a
 * dtm_status.
 */
int gemm_ex_noalloc(int64_t M, int64_t N, int64_t K,
                    const void *A, int64_t stride_am, int64_t stride_ak,
                    const void *B, int64_t stride_bk, int64_t stride_bn,
                    void *C, int64_t stride_cm, int64_t stride_cn,
                    int in_dtype, int out_dtype,
                    const dtm_tile_config *force, void *stream);

/* gemm_noalloc_scratch_bytes -- the size of gemm_ex_noalloc's fixed array. */
uint64_t gemm_noalloc_scratch_bytes(void);

/* gemm_status_string -- a static, NUL-terminated description of a status.
 * Every check runs before anything is launched, so a bad call fails on the
 * host with a message rather than on the GPU (the "Triton matmul" notes,
 * "Things that break": the failure to want is the one raised before the
 * GPU is reached). */
const char *gemm_status_string(int status);

/* gemm_kernel_name -- a static name for a dtm_kernel value. */
const char *gemm_kernel_name(int kernel);

/* gemm_set_pointer_checks -- debug checks of the caller's pointers, off by
 * default (the library cannot otherwise tell a wrong pointer or stride from
 * a right one: a view that runs past its memory gives wrong results or a
 * memory fault, not an error).  When on (on != 0), gemm, gemm_ex and
 * row_softmax first ask the HIP runtime, for every operand view they would
 * touch, for the allocation holding its lowest byte, and return
 * DTM_ERR_POINTER -- launching nothing -- unless the view's whole byte range
 * lies in that one allocation and the allocation is device memory of the
 * current device.  It costs a few runtime queries per call.  The initial
 * setting is on when the environment variable DTM_CHECK_POINTERS is set to
 * a value other than "0" when the library loads.  Process-wide and
 * thread-safe; returns the previous setting (0 or 1). */
int gemm_set_pointer_checks(int on);

/*
 * gemm_mfma_probe -- diagnostic: one 16 x 16 x 32 matrix-core product of the
 * fp16/bf16 kernels, C = A.B for a 16 x 32 A and a 32 x 16 B, with the
 * operands staged in LDS, their fragments read and the result stored exactly
 * as those kernels do (the layouts behind the tile product of "Chapter 13:
 * The Blocked Matmul Kernel", section 13.1, on this hardware).  On
 * integer-valued inputs the result is exact, so it pins the lane <-> element
 * maps of both operands and the result.
 * in_dtype: DTM_F16 or DTM_BF16.  layout: dtm_layout bits.  paired: 1 for
 * the 128-byte rows of the paired stages, 0 for the 64-byte rows.
 * A: 512 elements, element (i, k) at A[i*32 + k], or at A[k*16 + i] with
 * DTM_LAYOUT_A_M_CONTIG.  B: 512 elements, element (k, j) at B[k*16 + j], or
 * at B[j*32 + k] with DTM_LAYOUT_B_K_CONTIG.  C: 256 fp32, element (i, j) at
 * C[i*16 + j].  Device memory, 16-byte aligned, owned by the caller.
 * Enqueued on `stream`.  Returns a dtm_status.
 */
int gemm_mfma_probe(int in_dtype, int layout, int paired, const void *A, const void *B, void *C,
                    void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DTM_GEMM_H */
