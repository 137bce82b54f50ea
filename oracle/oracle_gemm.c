/*
 * oracle_gemm.c -- CPU oracle for the blocked GEMM C = A.B and for the row
 * softmax (the second workload, at the end of this file)
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or helper with the HIP library: its dtype codes, decoders and
 * rounding are its own.
 *
 * What it computes.  "Chapter 13: The Blocked Matmul Kernel" (Triton from
 * first principles), section 13.1, has each program own one output tile and
 * walk the shared dimension K in chunks, adding every chunk's tile product
 * into one accumulator that starts at zero; section 13.2 masks rows >= M,
 * columns >= N and k >= K so that out-of-range slots contribute exact zeros
 * (Lesson 4 "Block Pointers", section 3: zero padding is exact for a matmul).
 * The result is therefore the plain definition
 *
 *     C[i][j] = sum over k in [0, K) of A[i][k] * B[k][j],
 *
 * and the oracle is that definition: no tiles, no masks, k ascending, the
 * running sum held in fp64.  Every product of two fp32, fp16 or bf16 values
 * is exact in fp64 (at most 48 significand bits), so the fp64 result depends
 * only on the fixed summation order.  Comparing against an fp64 result of the
 * identical rounded inputs is section 13.3's method (Worked Example 13.3.1).
 *
 * Operands are read through element strides, as in the section 13.1 kernel
 * signature (stride_am, stride_ak, stride_bk, stride_bn); strides may be
 * zero or negative.  Outputs are dense row-major M x N arrays.
 *
 * The fp16-accumulator variant of section 13.3 (partial tile product cast to
 * fp16 each K-chunk, then added into an fp16 accumulator) is emulated by
 * oracle_gemm_fp16acc for the accumulation-error report.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* The oracle's own dtype codes. */
enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };

/* ---- decoding: bits -> exact double ------------------------------------ */

static double dec_f16(uint16_t h)
{
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);            /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25); /* (1 + m/2^10) * 2^(e-15) */
    return s ? -v : v;
}

static double dec_bf16(uint16_t b)
{
    int s = b >> 15, e = (b >> 7) & 255, m = b & 127;
    double v;
    if (e == 0)
        v = ldexp((double)m, -133);           /* m * 2^-133 */
    else if (e == 255)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + m), e - 134); /* (1 + m/2^7) * 2^(e-127) */
    return s ? -v : v;
}

static double dec_f32(uint32_t u)
{
    int s = u >> 31, e = (u >> 23) & 255;
    uint32_t m = u & 0x7FFFFFu;
    double v;
    if (e == 0)
        v = ldexp((double)m, -149);
    else if (e == 255)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(0x800000u + m), e - 150);
    return s ? -v : v;
}

static double dec(const void *base, int64_t idx, int dtype)
{
    if (dtype == OR_F32)
        return dec_f32(((const uint32_t *)base)[idx]);
    if (dtype == OR_F16)
        return dec_f16(((const uint16_t *)base)[idx]);
    return dec_bf16(((const uint16_t *)base)[idx]);
}

/* ---- rounding: double -> bits, round to nearest, ties to even ----------- */

/* Round x to a binary format with `mant` stored fraction bits and an
 * `ebits`-wide exponent field (IEEE layout, gradual underflow).  Ties go to
 * the even significand; magnitudes that round beyond the largest finite value
 * become infinity; NaN becomes the quiet NaN of the format. */
static uint32_t rne(double x, int mant, int ebits)
{
    const int bias = (1 << (ebits - 1)) - 1;
    const uint32_t emax_field = (1u << ebits) - 1;
    const uint32_t sign = signbit(x) ? (1u << (mant + ebits)) : 0u;
    if (isnan(x))
        return sign | (emax_field << mant) | (1u << (mant - 1));
    double ax = fabs(x);
    if (isinf(ax))
        return sign | (emax_field << mant);
    if (ax == 0.0)
        return sign;
    int e;
    (void)frexp(ax, &e);
    e -= 1;                        /* ax in [2^e, 2^(e+1)) */
    const int emin = 1 - bias;     /* exponent of the smallest normal */
    if (e < emin)
        e = emin;                  /* subnormal: quantum is 2^(emin-mant) */
    double q = ldexp(ax, mant - e); /* ax in units of the quantum (exact) */
    double r = nearbyint(q);        /* default mode: nearest, ties to even */
    uint64_t n = (uint64_t)r;
    if (n == (2ull << mant)) {     /* carried into the next binade */
        n >>= 1;
        e += 1;
    }
    if (n < (1ull << mant))        /* still subnormal (e == emin) */
        return sign | (uint32_t)n;
    if (e > bias)
        return sign | (emax_field << mant); /* overflow */
    return sign | ((uint32_t)(e + bias) << mant) | (uint32_t)(n - (1ull << mant));
}

static uint32_t enc(double x, int dtype)
{
    if (dtype == OR_F32)
        return rne(x, 23, 8);
    if (dtype == OR_F16)
        return rne(x, 10, 5);
    return rne(x, 7, 8);
}

static void store(void *base, int64_t idx, int dtype, double x)
{
    if (dtype == OR_F32)
        ((uint32_t *)base)[idx] = enc(x, dtype);
    else
        ((uint16_t *)base)[idx] = (uint16_t)enc(x, dtype);
}

static int valid_dtype(int d) { return d == OR_F32 || d == OR_F16 || d == OR_BF16; }

/* ---- exported codecs (for pinning the decoders and the rounding) -------- */

int oracle_decode_array(const void *bits, int64_t n, int dtype, double *out)
{
    if (!valid_dtype(dtype) || n < 0)
        return -1;
    for (int64_t i = 0; i < n; ++i)
        out[i] = dec(bits, i, dtype);
    return 0;
}

int oracle_encode_array(const double *x, int64_t n, int dtype, void *bits)
{
    if (!valid_dtype(dtype) || n < 0)
        return -1;
    for (int64_t i = 0; i < n; ++i)
        store(bits, i, dtype, x[i]);
    return 0;
}

/* ---- the product -------------------------------------------------------- */

/* Decode the rows x cols view at `base` (element strides sr, sc) into a dense
 * row-major array of doubles. */
static double *decode_view(const void *base, int64_t rows, int64_t cols, int64_t sr,
                           int64_t sc, int dtype)
{
    size_t n = (size_t)(rows > 0 ? rows : 1) * (size_t)(cols > 0 ? cols : 1);
    double *d = (double *)malloc(n * sizeof(double));
    if (!d)
        return NULL;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            d[r * cols + c] = dec(base, r * sr + c * sc, dtype);
    return d;
}

/*
 * C64[i*N + j] = sum_{k ascending} A[i,k] * B[k,j] in fp64, and
 * Cout[i*N + j] = that sum rounded once to out_dtype (nearest, ties to even).
 * Element (i,k) of A is at A + i*sam + k*sak (elements), (k,j) of B at
 * B + k*sbk + j*sbn.  C64 or Cout may be NULL.  K == 0 gives zeros.
 * nthreads <= 0 uses every core OpenMP sees.
 * Returns 0, or -1 on a bad argument, -2 when out of memory.
 */
int oracle_gemm(int64_t M, int64_t N, int64_t K,
                const void *A, int64_t sam, int64_t sak,
                const void *B, int64_t sbk, int64_t sbn,
                int in_dtype, int out_dtype,
                double *C64, void *Cout, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || !valid_dtype(in_dtype) || !valid_dtype(out_dtype))
        return -1;
    if (M == 0 || N == 0)
        return 0;
    if (K > 0 && (!A || !B))
        return -1;
    double *Ad = decode_view(A, M, K, sam, sak, in_dtype);
    double *Bd = decode_view(B, K, N, sbk, sbn, in_dtype);
    if (!Ad || !Bd) {
        free(Ad);
        free(Bd);
        return -2;
    }
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel reduction(| : failed)
    {
        /* one fp64 accumulator per output column of the current row */
        double *acc = (double *)malloc((size_t)N * sizeof(double));
        if (!acc) {
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = 0; i < M; ++i) {
                for (int64_t j = 0; j < N; ++j)
                    acc[j] = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    const double a = Ad[i * K + k];
                    const double *brow = Bd + k * N;
                    for (int64_t j = 0; j < N; ++j)
                        acc[j] += a * brow[j];
                }
                for (int64_t j = 0; j < N; ++j) {
                    if (C64)
                        C64[i * N + j] = acc[j];
                    if (Cout)
                        store(Cout, i * N + j, out_dtype, acc[j]);
                }
            }
            free(acc);
        }
    }
    free(Ad);
    free(Bd);
    return failed ? -2 : 0;
}

/*
 * Emulation of section 13.3's fp16-accumulator kernel: the accumulator is an
 * fp16 value that starts at zero; for each K-chunk [k0, k0+BK) the chunk's
 * tile product is formed (here exactly, in fp64), rounded to fp16, and added
 * into the accumulator with the sum rounded to fp16 again.  Writes fp16 bits,
 * dense row-major M x N.
 */
int oracle_gemm_fp16acc(int64_t M, int64_t N, int64_t K,
                        const void *A, int64_t sam, int64_t sak,
                        const void *B, int64_t sbk, int64_t sbn,
                        int in_dtype, int64_t BK, uint16_t *Cout16)
{
    if (M < 0 || N < 0 || K < 0 || BK <= 0 || !valid_dtype(in_dtype) || !Cout16)
        return -1;
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            double acc = 0.0; /* always holds an fp16 value */
            for (int64_t k0 = 0; k0 < K; k0 += BK) {
                const int64_t k1 = k0 + BK < K ? k0 + BK : K;
                double partial = 0.0;
                for (int64_t k = k0; k < k1; ++k)
                    partial += dec(A, i * sam + k * sak, in_dtype) *
                               dec(B, k * sbk + j * sbn, in_dtype);
                const double p16 = dec_f16((uint16_t)rne(partial, 10, 5));
                acc = dec_f16((uint16_t)rne(acc + p16, 10, 5));
            }
            Cout16[i * N + j] = (uint16_t)rne(acc, 10, 5);
        }
    }
    return 0;
}

/* ---- row softmax -------------------------------------------------------- */

/*
 * oracle_softmax -- the row softmax of "Triton from zero, Lesson 4: Block
 * Pointers", homework 4: for every row i of the M x N view X,
 *
 *     m_i    = max over j < N of X[i][j]
 *     Y[i][j] = exp(X[i][j] - m_i) / sum over j' < N of exp(X[i][j'] - m_i).
 *
 * The homework's kernel loads a row tile, replaces the columns at or beyond
 * N by -inf (so they can neither win the max nor add to the sum: exp(-inf)
 * is 0), takes the max, exponentiates the shifted values, sums them and
 * divides.  Here there is no tile, so no padding: the same three steps over
 * exactly the N columns, in fp64 over the exact decoded inputs (j
 * ascending for the sum), then one round-to-nearest-even conversion to the
 * output dtype.
 *
 * Special values follow the formula's own IEEE arithmetic: a NaN element
 * is ignored by the max but makes the sum, hence the whole row, NaN; a +inf
 * element makes the row NaN (inf - inf); a row whose elements are all -inf
 * has m = -inf and is NaN (-inf - -inf); -inf elements of any other row
 * give exact zeros.
 *
 * X is read through element strides (stride_xm, stride_xn), which may be
 * zero or negative.  Y64 (fp64) and Yout (out_dtype bits) are dense
 * row-major M x N arrays.
 */
int oracle_softmax(int64_t M, int64_t N, const void *X, int64_t sxm, int64_t sxn,
                   int in_dtype, int out_dtype, double *Y64, void *Yout, int nthreads)
{
    if (M < 0 || N < 0 || !valid_dtype(in_dtype) || !valid_dtype(out_dtype))
        return -1;
    if (M == 0 || N == 0)
        return 0;
    if (!X || !Y64 || !Yout)
        return -1;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#else
    (void)nthreads;
#endif
    for (int64_t i = 0; i < M; ++i) {
        double *y = Y64 + i * N;
        double m = -INFINITY;
        for (int64_t j = 0; j < N; ++j) {
            const double x = dec(X, i * sxm + j * sxn, in_dtype);
            y[j] = x;
            if (x > m) /* false for NaN: the max ignores it */
                m = x;
        }
        double sum = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            y[j] = exp(y[j] - m);
            sum += y[j];
        }
        for (int64_t j = 0; j < N; ++j) {
            y[j] = y[j] / sum;
            store(Yout, i * N + j, out_dtype, y[j]);
        }
    }
    return 0;
}
