// softmax.hip -- row softmax on gfx950, the second workload.
//
// "Triton from zero, Lesson 4: Block Pointers", homework 4: each row of an
// M x N view becomes exp(x - max) / sum(exp(x - max)); the columns a tile
// holds past N are given -inf before the max, so they can neither win it nor
// add to the sum (zero padding would be wrong for the max, section 3's
// gotcha).  Here such slots are simply never read and contribute exactly 0
// to the sum.  Arithmetic is fp32 (inputs are decoded exactly); exp(d) is
// computed as 2^(d log2 e) on the hardware base-2 exponential (v_exp_f32,
// about 1 ulp; results below 2^-126 flush to zero), the row sum's
// reciprocal is taken once (IEEE-rounded) and multiplies every term, and
// the result is converted once to the output dtype.  (The library's expf
// and a per-element IEEE division cost ~25 VALU instructions per element,
// which made the kernel arithmetic-bound on this part.)
//
// The operation reads and writes each element once: it is bound by HBM
// bandwidth, not by arithmetic, so there is no matrix-core work here.  What
// matters is that every row is read once, with 16-byte loads when the rows
// are unit-stride and aligned, and that the reductions stay on chip:
//  * WAVE form: one wave64 per row, four rows per workgroup; each lane holds
//    CH chunks of E elements in registers (16-bit inputs stay packed; with
//    up to 4 chunks the exponentials are kept for the write, with more they
//    are recomputed from the packed input); max and sum are reduced across
//    the wave with lane shuffles.  16-bit outputs are packed in pairs by the
//    hardware conversions.
//  * BLOCK form: one 1024-thread workgroup per row (rows too long for one
//    wave), up to 16 chunks per thread for fp32 rows (64 Ki elements) and 8
//    for 16-bit ones; wave results are combined through LDS.
//  * ONLINE form: rows too long for the workgroup's registers.  One pass
//    keeps, per thread, a running max m and a sum s of exp(x - m), rescaling
//    s by exp(m_old - m_new) when the max grows; the threads' (m, s) pairs
//    are combined the same way; a second pass reads the row again and
//    writes exp(x - m) / s.  Two reads and one write per element.
//  * SPLIT form: rows too long for one workgroup per row to fill the chip
//    (few rows): each row is cut into parts, one workgroup per (row, part);
//    a first kernel writes each part's (max, sum) pair to a small
//    workspace, a second merges the row's pairs in a fixed order and writes
//    its part.  Also two reads and one write per element.
// Special values follow the formula's own arithmetic: a NaN element does not
// change the max (fmaxf) but makes the sum NaN, a +inf element makes the row
// NaN, a row of -inf has max -inf and is NaN, other -inf elements give 0.
// In-place use (Y the same view as X) is safe: every thread finishes reading
// the row, or its element, before any thread writes it.
#include "softmax_launch.h"

namespace dtm {
namespace {

constexpr int WAVE = 64;
constexpr int BLOCK_THREADS = 1024;
constexpr int BLOCK_WAVES = BLOCK_THREADS / WAVE;

template <int D> struct Bytes;
template <> struct Bytes<DTM_F32> { static constexpr int value = 4; };
template <> struct Bytes<DTM_F16> { static constexpr int value = 2; };
template <> struct Bytes<DTM_BF16> { static constexpr int value = 2; };

// Elements per chunk: one 16-byte load when vectorised, else one element.
template <int IN, bool VEC> constexpr int chunk_elems() { return VEC ? 16 / Bytes<IN>::value : 1; }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// One chunk as loaded: E elements of the input dtype, packed.
template <int IN, int E> struct Packed {
    static constexpr int WORDS = (E * Bytes<IN>::value + 3) / 4;
    uint32_t w[WORDS];
    __device__ __forceinline__ float get(int e) const
    {
        if constexpr (IN == DTM_F32) {
            return __uint_as_float(w[e]);
        } else {
            const uint32_t h = (w[e >> 1] >> (16 * (e & 1))) & 0xffffu;
            if constexpr (IN == DTM_F16)
                return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
            else
                return __uint_as_float(h << 16);
        }
    }
};

// Loads the E elements of the chunk starting at column `col` of row `row`;
// columns >= N are not read (their slots are 0 and callers skip them).
template <int IN, bool VEC, int E>
__device__ __forceinline__ void load_chunk(const SoftmaxArgs &p, int64_t row, int64_t col,
                                           Packed<IN, E> &v)
{
    const int64_t base = row * p.sxm;
    if constexpr (VEC) {
        if (col + E <= p.N) {
            const u32x4 w = *reinterpret_cast<const u32x4 *>(
                static_cast<const char *>(p.X) + (base + col) * Bytes<IN>::value);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                v.w[i] = w[i];
            return;
        }
    }
#pragma unroll
    for (int i = 0; i < Packed<IN, E>::WORDS; ++i)
        v.w[i] = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        if (col + e < p.N) {
            const int64_t idx = base + (col + e) * p.sxn;
            if constexpr (IN == DTM_F32)
                v.w[e] = static_cast<const uint32_t *>(p.X)[idx];
            else
                v.w[e >> 1] |= static_cast<uint32_t>(static_cast<const uint16_t *>(p.X)[idx])
                               << (16 * (e & 1));
        }
    }
}

// Tells the compiler the packed words may have changed, so values decoded
// from them are decoded again after this point instead of being kept in
// registers (16-bit chunks stay packed: half the registers).  Emits nothing.
template <int IN, int E, int CH>
__device__ __forceinline__ void keep_packed(Packed<IN, E> (&x)[CH])
{
#pragma unroll
    for (int q = 0; q < CH; ++q)
#pragma unroll
        for (int i = 0; i < Packed<IN, E>::WORDS; ++i)
            asm volatile("" : "+v"(x[q].w[i]));
}

// exp(d) for d <= 0 (or NaN): 2^(d log2 e) on the hardware exponential.
__device__ __forceinline__ float exp_shifted(float d)
{
    constexpr float LOG2E = 1.4426950408889634f;
    return __builtin_amdgcn_exp2f(d * LOG2E);
}

template <int OUT, bool VEC, int E>
__device__ __forceinline__ void store_chunk(const SoftmaxArgs &p, int64_t row, int64_t col,
                                            const float (&y)[E])
{
    const int64_t base = row * p.sym;
    if constexpr (VEC) {
        if (col + E <= p.N) {
            char *dst = static_cast<char *>(p.Y) + (base + col) * Bytes<OUT>::value;
            if constexpr (OUT == DTM_F32) {
#pragma unroll
                for (int h = 0; h < E / 4; ++h)
                    *reinterpret_cast<u32x4 *>(dst + 16 * h) =
                        u32x4{__float_as_uint(y[4 * h]), __float_as_uint(y[4 * h + 1]),
                              __float_as_uint(y[4 * h + 2]), __float_as_uint(y[4 * h + 3])};
            } else {
                // pairs through the packed hardware conversions
                // (v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32: nearest-even, like
                // store_elem, one instruction per two elements)
                uint32_t w[E / 2];
#pragma unroll
                for (int h = 0; h < E / 2; ++h) {
                    const f32x2 pair{y[2 * h], y[2 * h + 1]};
                    if constexpr (OUT == DTM_F16)
                        w[h] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pair, f16x2));
                    else
                        w[h] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pair, bf16x2));
                }
                if constexpr (E == 8) {
                    *reinterpret_cast<u32x4 *>(dst) = u32x4{w[0], w[1], w[2], w[3]};
                } else {  // E == 4: 8 bytes
                    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                    *reinterpret_cast<u32x2 *>(dst) = u32x2{w[0], w[1]};
                }
            }
            return;
        }
    }
#pragma unroll
    for (int e = 0; e < E; ++e)
        if (col + e < p.N)
            store_elem<OUT>(p.Y, base + (col + e) * p.syn, y[e]);
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = WAVE / 2; o > 0; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o, WAVE));
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = WAVE / 2; o > 0; o >>= 1)
        v += __shfl_xor(v, o, WAVE);
    return v;
}

// Combines two (max, sum of exp(x - max)) pairs.  When both maxima are
// equal (including both -inf) no rescaling is applied.
__device__ __forceinline__ void merge_ms(float &m, float &s, float m2, float s2)
{
    const float mn = fmaxf(m, m2);
    const float a = (m == mn) ? s : s * exp_shifted(m - mn);
    const float b = (m2 == mn) ? s2 : s2 * exp_shifted(m2 - mn);
    m = mn;
    s = a + b;
}

// The exponential is the costliest step per element (v_exp_f32 issues at a
// quarter of the VALU rate).  With few chunks per lane the wave form keeps
// exp(x - m) in registers for the write; with more, the registers that
// would take cost more in occupancy than the second exponential costs
// (measured: 16-chunk fp32 and fp16 rows 12-13% slower when kept; 1-chunk
// bf16 rows 11% faster), so the write recomputes it from the packed input.
constexpr int KEEP_EXP_MAX_CH = 4;

// exp(x - m) of every element a thread holds, kept for the write, and their
// sum.  Slots past N get 0.  `col_of(q)`: first column of chunk q.
template <int IN, int E, int CH, typename ColOf>
__device__ __forceinline__ float exps_and_sum(const Packed<IN, E> (&x)[CH], float m, int64_t N,
                                              ColOf col_of, float (&ex)[CH][E])
{
    float s = 0.0f;
#pragma unroll
    for (int q = 0; q < CH; ++q) {
        const int64_t col = col_of(q);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            ex[q][e] = col + e < N ? exp_shifted(x[q].get(e) - m) : 0.0f;
            s += ex[q][e];
        }
    }
    return s;
}

// Sum of exp(x - m) over the elements a thread holds (columns < N).
template <int IN, int E, int CH, typename ColOf>
__device__ __forceinline__ float exp_sum(const Packed<IN, E> (&x)[CH], float m, int64_t N,
                                         ColOf col_of)
{
    float s = 0.0f;
#pragma unroll
    for (int q = 0; q < CH; ++q) {
        const int64_t col = col_of(q);
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (col + e < N)
                s += exp_shifted(x[q].get(e) - m);
    }
    return s;
}

// Writes exp(x - m) * r for chunk x (the exponential computed again).
template <int OUT, bool VEC, int IN, int E>
__device__ __forceinline__ void store_recomputed(const SoftmaxArgs &p, int64_t row, int64_t col,
                                                 const Packed<IN, E> &x, float m, float r)
{
    float y[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        y[e] = exp_shifted(x.get(e) - m) * r;
    store_chunk<OUT, VEC, E>(p, row, col, y);
}

// Writes chunk `ex` times r.
template <int OUT, bool VEC, int E>
__device__ __forceinline__ void store_scaled(const SoftmaxArgs &p, int64_t row, int64_t col,
                                             const float (&ex)[E], float r)
{
    float y[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        y[e] = ex[e] * r;
    store_chunk<OUT, VEC, E>(p, row, col, y);
}

// ---- WAVE form ---------------------------------------------------------------

template <int IN, int OUT, int CH, bool VEC>
__global__ __launch_bounds__(4 * WAVE) void softmax_wave_kernel(SoftmaxArgs p)
{
    constexpr int E = chunk_elems<IN, VEC>();
    const int lane = threadIdx.x & (WAVE - 1);
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (row >= p.M)
        return;  // a whole wave leaves together; no barrier follows

    Packed<IN, E> x[CH];
    float m = -INFINITY;
#pragma unroll
    for (int q = 0; q < CH; ++q) {
        const int64_t col = (static_cast<int64_t>(q) * WAVE + lane) * E;
        load_chunk<IN, VEC, E>(p, row, col, x[q]);
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (col + e < p.N)
                m = fmaxf(m, x[q].get(e));
    }
    m = wave_max(m);
    keep_packed(x);
    auto col_of = [&](int q) { return (static_cast<int64_t>(q) * WAVE + lane) * E; };
    if constexpr (CH <= KEEP_EXP_MAX_CH) {
        float ex[CH][E];
        const float r = 1.0f / wave_sum(exps_and_sum<IN, E, CH>(x, m, p.N, col_of, ex));
#pragma unroll
        for (int q = 0; q < CH; ++q)
            store_scaled<OUT, VEC, E>(p, row, col_of(q), ex[q], r);
    } else {
        const float r = 1.0f / wave_sum(exp_sum<IN, E, CH>(x, m, p.N, col_of));
        keep_packed(x);
#pragma unroll
        for (int q = 0; q < CH; ++q)
            store_recomputed<OUT, VEC, IN, E>(p, row, col_of(q), x[q], m, r);
    }
}

// ---- BLOCK and ONLINE forms ---------------------------------------------------

// Reduces one value per wave across the workgroup through LDS; every thread
// gets the result.  `red` holds BLOCK_WAVES floats; two barriers.
template <bool MAX>
__device__ __forceinline__ float block_reduce(float v, float *red)
{
    const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x >> 6;
    v = MAX ? wave_max(v) : wave_sum(v);
    if (lane == 0)
        red[wave] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int w = 1; w < BLOCK_WAVES; ++w)
        r = MAX ? fmaxf(r, red[w]) : r + red[w];
    __syncthreads();  // red may be reused
    return r;
}

template <int IN, int OUT, int CH, bool VEC>
__global__ __launch_bounds__(BLOCK_THREADS) void softmax_block_kernel(SoftmaxArgs p)
{
    constexpr int E = chunk_elems<IN, VEC>();
    __shared__ float red[BLOCK_WAVES];
    const int64_t row = blockIdx.x;
    const int t = threadIdx.x;

    Packed<IN, E> x[CH];
    float m = -INFINITY;
#pragma unroll
    for (int q = 0; q < CH; ++q) {
        const int64_t col = (static_cast<int64_t>(q) * BLOCK_THREADS + t) * E;
        load_chunk<IN, VEC, E>(p, row, col, x[q]);
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (col + e < p.N)
                m = fmaxf(m, x[q].get(e));
    }
    m = block_reduce<true>(m, red);
    keep_packed(x);
    auto col_of = [&](int q) { return (static_cast<int64_t>(q) * BLOCK_THREADS + t) * E; };
    const float r = 1.0f / block_reduce<false>(exp_sum<IN, E, CH>(x, m, p.N, col_of), red);
    keep_packed(x);
#pragma unroll
    for (int q = 0; q < CH; ++q)
        store_recomputed<OUT, VEC, IN, E>(p, row, col_of(q), x[q], m, r);
}

// ONLINE and SPLIT work in tiles of BLOCK_THREADS x ONLINE_CH chunks.
constexpr int ONLINE_CH = 2;  // chunks per thread per tile (loads in flight)
template <int IN, bool VEC> constexpr int64_t online_tile()
{
    return static_cast<int64_t>(BLOCK_THREADS) * ONLINE_CH * chunk_elems<IN, VEC>();
}

// The (max, sum of exp(x - max)) pair of columns [cb, ce) of `row`, for the
// whole workgroup: per thread a running pair over the tiles, rescaled when
// the max grows, then merged across the wave and across waves.  cb is a
// multiple of the tile and ce is N or a multiple of the tile, so no chunk
// straddles ce.  Every thread returns the workgroup's pair.
template <int IN, bool VEC>
__device__ __forceinline__ void range_stats(const SoftmaxArgs &p, int64_t row, int64_t cb,
                                            int64_t ce, float &m, float &s, float *red_m,
                                            float *red_s)
{
    constexpr int E = chunk_elems<IN, VEC>();
    constexpr int CH = ONLINE_CH;
    constexpr int64_t TILE = online_tile<IN, VEC>();
    const int t = threadIdx.x;
    const int lane = t & (WAVE - 1), wave = t >> 6;
    m = -INFINITY;
    s = 0.0f;
    for (int64_t c0 = cb; c0 < ce; c0 += TILE) {
        Packed<IN, E> x[CH];
        float tm = -INFINITY;
#pragma unroll
        for (int q = 0; q < CH; ++q) {
            const int64_t col = c0 + (static_cast<int64_t>(q) * BLOCK_THREADS + t) * E;
            load_chunk<IN, VEC, E>(p, row, col, x[q]);
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (col + e < p.N)
                    tm = fmaxf(tm, x[q].get(e));
        }
        float ts = 0.0f;
#pragma unroll
        for (int q = 0; q < CH; ++q) {
            const int64_t col = c0 + (static_cast<int64_t>(q) * BLOCK_THREADS + t) * E;
            // a -inf element adds exactly 0 (even when the tile's max is
            // -inf too); a row of -inf still ends NaN in the write pass,
            // where the row max is -inf
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float v = x[q].get(e);
                if (col + e < p.N && v != -INFINITY)
                    ts += exp_shifted(v - tm);
            }
        }
        merge_ms(m, s, tm, ts);
    }
#pragma unroll
    for (int o = WAVE / 2; o > 0; o >>= 1) {
        const float m2 = __shfl_xor(m, o, WAVE), s2 = __shfl_xor(s, o, WAVE);
        merge_ms(m, s, m2, s2);
    }
    if (lane == 0) {
        red_m[wave] = m;
        red_s[wave] = s;
    }
    __syncthreads();
    m = red_m[0];
    s = red_s[0];
#pragma unroll
    for (int w = 1; w < BLOCK_WAVES; ++w)
        merge_ms(m, s, red_m[w], red_s[w]);
}

// Writes exp(x - m) * r for columns [cb, ce) of `row` (r = 1 / row sum).
template <int IN, int OUT, bool VEC>
__device__ __forceinline__ void range_write(const SoftmaxArgs &p, int64_t row, int64_t cb,
                                            int64_t ce, float m, float r)
{
    constexpr int E = chunk_elems<IN, VEC>();
    constexpr int CH = ONLINE_CH;
    constexpr int64_t TILE = online_tile<IN, VEC>();
    const int t = threadIdx.x;
    for (int64_t c0 = cb; c0 < ce; c0 += TILE) {
        Packed<IN, E> x[CH];
#pragma unroll
        for (int q = 0; q < CH; ++q)
            load_chunk<IN, VEC, E>(p, row, c0 + (static_cast<int64_t>(q) * BLOCK_THREADS + t) * E,
                                   x[q]);
#pragma unroll
        for (int q = 0; q < CH; ++q) {
            const int64_t col = c0 + (static_cast<int64_t>(q) * BLOCK_THREADS + t) * E;
            float y[E];
#pragma unroll
            for (int e = 0; e < E; ++e)
                y[e] = exp_shifted(x[q].get(e) - m) * r;
            store_chunk<OUT, VEC, E>(p, row, col, y);
        }
    }
}

template <int IN, int OUT, bool VEC>
__global__ __launch_bounds__(BLOCK_THREADS) void softmax_online_kernel(SoftmaxArgs p)
{
    __shared__ float red_m[BLOCK_WAVES], red_s[BLOCK_WAVES];
    const int64_t row = blockIdx.x;
    float m, s;
    range_stats<IN, VEC>(p, row, 0, p.N, m, s, red_m, red_s);
    range_write<IN, OUT, VEC>(p, row, 0, p.N, m, 1.0f / s);
}

// ---- SPLIT form: each row cut into `parts` ranges of `part_len` columns ----
// (a multiple of the tile), one workgroup per (row, part).  The stats kernel
// writes each range's (max, sum) pair to ws[2 (row*parts + part) + {0, 1}];
// the write kernel merges the row's pairs in the fixed order part = 0, 1, ...
// (so every workgroup of a row gets the same row max and sum, and the result
// does not depend on scheduling) and writes its range.

template <int IN, bool VEC>
__global__ __launch_bounds__(BLOCK_THREADS) void softmax_split_stats_kernel(SoftmaxArgs p,
                                                                            int64_t parts,
                                                                            int64_t part_len,
                                                                            float *ws)
{
    __shared__ float red_m[BLOCK_WAVES], red_s[BLOCK_WAVES];
    const int64_t row = blockIdx.x / parts, part = blockIdx.x % parts;
    const int64_t cb = part * part_len;
    const int64_t ce = cb + part_len < p.N ? cb + part_len : p.N;
    float m, s;
    range_stats<IN, VEC>(p, row, cb, ce, m, s, red_m, red_s);
    if (threadIdx.x == 0) {
        ws[2 * blockIdx.x] = m;
        ws[2 * blockIdx.x + 1] = s;
    }
}

template <int IN, int OUT, bool VEC>
__global__ __launch_bounds__(BLOCK_THREADS) void softmax_split_write_kernel(SoftmaxArgs p,
                                                                            int64_t parts,
                                                                            int64_t part_len,
                                                                            const float *ws)
{
    const int64_t row = blockIdx.x / parts, part = blockIdx.x % parts;
    const int64_t cb = part * part_len;
    const int64_t ce = cb + part_len < p.N ? cb + part_len : p.N;
    const float *w = ws + 2 * row * parts;
    float m = w[0], s = w[1];
    for (int64_t q = 1; q < parts; ++q)
        merge_ms(m, s, w[2 * q], w[2 * q + 1]);
    range_write<IN, OUT, VEC>(p, row, cb, ce, m, 1.0f / s);
}

// ---- launchers ------------------------------------------------------------------

template <int IN, int OUT, bool VEC>
hipError_t launch_form(const SoftmaxArgs &a, int form, int ch, float *ws, hipStream_t s)
{
    if (form == SOFTMAX_WAVE) {
        const dim3 grid((unsigned)cdiv(a.M, 4)), block(4 * WAVE);
        switch (ch) {
        case 1: hipLaunchKernelGGL((softmax_wave_kernel<IN, OUT, 1, VEC>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((softmax_wave_kernel<IN, OUT, 2, VEC>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((softmax_wave_kernel<IN, OUT, 4, VEC>), grid, block, 0, s, a); break;
        case 8: hipLaunchKernelGGL((softmax_wave_kernel<IN, OUT, 8, VEC>), grid, block, 0, s, a); break;
        case 16: hipLaunchKernelGGL((softmax_wave_kernel<IN, OUT, 16, VEC>), grid, block, 0, s, a); break;
        default: return hipErrorInvalidConfiguration;
        }
    } else if (form == SOFTMAX_BLOCK) {
        const dim3 grid((unsigned)a.M), block(BLOCK_THREADS);
        switch (ch) {
        case 1: hipLaunchKernelGGL((softmax_block_kernel<IN, OUT, 1, VEC>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((softmax_block_kernel<IN, OUT, 2, VEC>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((softmax_block_kernel<IN, OUT, 4, VEC>), grid, block, 0, s, a); break;
        case 8: hipLaunchKernelGGL((softmax_block_kernel<IN, OUT, 8, VEC>), grid, block, 0, s, a); break;
        case 16:
            // 16 chunks per thread: fp32 rows only (16-bit rows of that many
            // chunks would not fit the 128 VGPRs a 1024-thread workgroup allows)
            if constexpr (IN == DTM_F32) {
                hipLaunchKernelGGL((softmax_block_kernel<IN, OUT, 16, VEC>), grid, block, 0, s, a);
                break;
            }
            return hipErrorInvalidConfiguration;
        default: return hipErrorInvalidConfiguration;
        }
    } else if (form == SOFTMAX_ONLINE) {
        hipLaunchKernelGGL((softmax_online_kernel<IN, OUT, VEC>), dim3((unsigned)a.M),
                           dim3(BLOCK_THREADS), 0, s, a);
    } else if (form == SOFTMAX_SPLIT) {
        const int64_t parts = ch, part_len = cdiv(cdiv(a.N, parts), online_tile<IN, VEC>()) *
                                             online_tile<IN, VEC>();
        if (!ws || (parts - 1) * part_len >= a.N)
            return hipErrorInvalidConfiguration;
        const dim3 grid((unsigned)(a.M * parts)), block(BLOCK_THREADS);
        hipLaunchKernelGGL((softmax_split_stats_kernel<IN, VEC>), grid, block, 0, s, a, parts,
                           part_len, ws);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        hipLaunchKernelGGL((softmax_split_write_kernel<IN, OUT, VEC>), grid, block, 0, s, a,
                           parts, part_len, static_cast<const float *>(ws));
    } else {
        return hipErrorInvalidConfiguration;
    }
    return hipGetLastError();
}

template <int IN, int OUT>
hipError_t dispatch_vec(const SoftmaxArgs &a, int form, int ch, bool vec, float *ws,
                        hipStream_t s)
{
    return vec ? launch_form<IN, OUT, true>(a, form, ch, ws, s)
               : launch_form<IN, OUT, false>(a, form, ch, ws, s);
}

template <int IN>
hipError_t dispatch_out(const SoftmaxArgs &a, int out, int form, int ch, bool vec, float *ws,
                        hipStream_t s)
{
    switch (out) {
    case DTM_F32: return dispatch_vec<IN, DTM_F32>(a, form, ch, vec, ws, s);
    case DTM_F16: return dispatch_vec<IN, DTM_F16>(a, form, ch, vec, ws, s);
    case DTM_BF16: return dispatch_vec<IN, DTM_BF16>(a, form, ch, vec, ws, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

int softmax_chunk_elems(int in_dtype, bool vec) { return vec ? (in_dtype == DTM_F32 ? 4 : 8) : 1; }
int softmax_form_threads(int form) { return form == SOFTMAX_WAVE ? 4 * WAVE : BLOCK_THREADS; }
int softmax_form_lanes(int form) { return form == SOFTMAX_WAVE ? WAVE : BLOCK_THREADS; }

int64_t softmax_tile(int in_dtype, bool vec)
{
    return static_cast<int64_t>(BLOCK_THREADS) * ONLINE_CH * softmax_chunk_elems(in_dtype, vec);
}

hipError_t launch_softmax(const SoftmaxArgs &a, int in, int out, int form, int ch, bool vec,
                          float *ws, hipStream_t s)
{
    if (a.M <= 0 || a.N <= 0 || a.M > 0x7fffffffLL)
        return hipErrorInvalidConfiguration;
    switch (in) {
    case DTM_F32: return dispatch_out<DTM_F32>(a, out, form, ch, vec, ws, s);
    case DTM_F16: return dispatch_out<DTM_F16>(a, out, form, ch, vec, ws, s);
    case DTM_BF16: return dispatch_out<DTM_BF16>(a, out, form, ch, vec, ws, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace dtm
