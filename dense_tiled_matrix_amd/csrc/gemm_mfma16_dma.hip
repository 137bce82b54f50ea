// gemm_mfma16_dma.hip -- deep-pipelined MFMA GEMM for fp16/bf16 inputs on
// gfx950, for problems whose M, N are multiples of 256 and K of 32.
//
// The computation is the blocked product of "Chapter 13: The Blocked Matmul
// Kernel" (section 13.1): one workgroup per 256 x 256 output tile, a K-loop
// over 32-deep chunks adding each chunk's tile product into an fp32
// accumulator zeroed once before the loop, and a single conversion to the
// output dtype at the store (section 13.3).  No edge masking is needed on
// this path ("Triton from zero, Lesson 4: Block Pointers", homework 3: pay
// only for the raggedness a problem has); ragged problems use the other MFMA
// kernel.
//
// gfx950 design:
//  * 4 wave64s (2 x 2), each owning 128 x 128 of C as 4 x 4 tiles of
//    v_mfma_f32_32x32x16_{f16,bf16}; 256 fp32 accumulators per lane in the
//    AccVGPR file.
//  * Operands move global -> LDS with global_load_lds_dwordx4 (each wave
//    instruction writes 1 KiB of LDS, lane i's 16 bytes at offset 16*i), so
//    no VGPRs stage them.  Four LDS stages of (16 + 16) KiB: a chunk is
//    loaded three to four chunks of MFMA time before it is read.  One
//    barrier per chunk, after a wait for exactly the loads of the chunk
//    about to be read; the loads are issued one after every second MFMA.
//  * A is stored row-major (64 bytes per row); the 16-byte chunk c of row r
//    sits at position c ^ f(r), f(r) = (r >> 2) & 3, so each group of 16
//    consecutive rows read by a fragment load (one chunk each) covers all 64
//    banks once.  (Measured on gfx950 with SQ_LDS_BANK_CONFLICT: zero
//    conflicts for this pattern; other XOR patterns cost 4-12 extra cycles
//    per ds_read_b128.)
//  * B stays N-contiguous (512 bytes per k-row); chunk c of k-row k sits at
//    c ^ g(k), g = {0, 6, 10, 12}[k % 4] (measured conflict-free for the
//    transposing reads below; no swizzle costs about 6 extra cycles each).  Fragments are read with
//    ds_read_b64_tr_b16, which hands lane i of each 16-lane group the
//    i-th column of a 4 x 16 block whose rows the lanes address, i.e. four
//    consecutive k of one column -- the MFMA B operand -- with no transpose
//    anywhere else.
//  * Workgroup ids are remapped so that each XCD owns a compact group of
//    tiles (shared A rows and B columns stay in its L2).
#include "launch.h"

namespace dtm {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T *)(p))

constexpr int BM = 256, BN = 256, BK = 32, STAGES = 4;
constexpr int A_STAGE_BYTES = BM * BK * 2;  // 16 KiB
constexpr int B_STAGE_BYTES = BK * BN * 2;  // 16 KiB
constexpr int STAGE_BYTES = A_STAGE_BYTES + B_STAGE_BYTES;
#ifndef DTM_DMA_GROUP_M
#define DTM_DMA_GROUP_M 4
#endif
constexpr int64_t GROUP_M = DTM_DMA_GROUP_M;  // tile-rows walked together per XCD

// s_waitcnt immediate (gfx9 layout): vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8],
// vmcnt[5:4] in bits [15:14].
constexpr int waitcnt_imm(int vm, int lgkm)
{
    return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | (((vm >> 4) & 3) << 14);
}

__device__ __forceinline__ int swz_a(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int swz_b(int k)
{
    // 0, 6, 10, 12 for k % 4 = 0..3
    return (0xCA60 >> (4 * (k & 3))) & 15;
}

// 16 bytes per lane from global memory straight into LDS at
// lds_addr + 16 * lane (global_load_lds_dwordx4; M0 holds the LDS address).
__device__ __forceinline__ void dma16(const void *gptr, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(gptr), "s"(lds_addr)
                 : "memory", "m0");
}

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

template <int IN, int OUT, int NWAVES>
__global__ __launch_bounds__(64 * NWAVES) void gemm_mfma16_dma_kernel(GemmArgs p, int64_t grid_m,
                                                                      int64_t grid_n,
                                                                      int64_t k_split,
                                                                      int64_t c_split_stride)
{
    // Split-K: workgroup ids beyond one grid of tiles take further slices of
    // K, k_split elements each, and write their fp32 partial tile to
    // C + slice * c_split_stride.  Without a split, k_split = K and the
    // stride is unused.
    // Waves form a 2 x (NWAVES/2) grid over the 256 x 256 tile; each owns
    // 128 rows and 256/(NWAVES/2) columns as MT x NT tiles of 32 x 32.
    constexpr int WAVES_N = NWAVES / 2;
    constexpr int WN_COLS = BN / WAVES_N;
    constexpr int MT = 4, NT = WN_COLS / 32;
    constexpr int NREAD = MT + 2 * NT;           // LDS reads per k-step
    constexpr int NMFMA = MT * NT;               // MFMAs per k-step
    constexpr int DPO = 16 / NWAVES;             // 1 KiB loads per operand per wave per chunk
    constexpr int DMA_GROUP = 2 * DPO;           // loads per wave per chunk
    static_assert(NREAD <= NMFMA && DMA_GROUP <= NMFMA / 2, "interleave slots");

    __shared__ __attribute__((aligned(1024))) char lds[STAGES * STAGE_BYTES];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    int64_t pid_m, pid_n;
    const int64_t tiles = grid_m * grid_n;
    const int64_t splits = p.K / k_split;
    // consecutive remapped ids (one XCD) share a K slice and differ in tile
    const int64_t t_id = xcd_remap(blockIdx.x, tiles * splits);
    const int64_t slice = t_id / tiles;
    grouped_tile(t_id - slice * tiles, grid_m, grid_n, GROUP_M, pid_m, pid_n);
    const int64_t m0 = pid_m * BM, n0 = pid_n * BN;
    const int64_t kb = slice * k_split;

    const uint16_t *A = static_cast<const uint16_t *>(p.A);
    const uint16_t *B = static_cast<const uint16_t *>(p.B);

    // ---- load source addresses of this lane ------------------------------
    // A load j of wave w fills LDS bytes 1024*(DPO*w + j) .. +1023 of the A
    // stage: rows 16*(DPO*w + j) + lane/4, physical chunk lane%4.
    const uint16_t *a_src[DPO];
#pragma unroll
    for (int j = 0; j < DPO; ++j) {
        const int r = 16 * (DPO * wave + j) + (lane >> 2);
        const int c = (lane & 3) ^ swz_a(r);
        a_src[j] = A + (m0 + r) * p.sam + kb + 8 * c;
    }
    // B load j of wave w fills k-rows 2*(DPO*w + j) + lane/32, physical
    // chunk lane%32.
    const uint16_t *b_src[DPO];
#pragma unroll
    for (int j = 0; j < DPO; ++j) {
        const int k = 2 * (DPO * wave + j) + (lane >> 5);
        const int c = (lane & 31) ^ swz_b(k);
        b_src[j] = B + (kb + k) * p.sbk + n0 + 8 * c;
    }
    const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(LDS_PTR(char, lds)));
    const uint32_t a_dst0 = lds_base + (DPO * wave) * 1024;
    const uint32_t b_dst0 = lds_base + A_STAGE_BYTES + (DPO * wave) * 1024;

    // Load d (0 .. DMA_GROUP-1) of chunk kt into LDS stage `stage`.  Inline
    // assembly, so the compiler neither reorders nor waits on these
    // asynchronous LDS writes; the loop waits for them explicitly (vmcnt)
    // before a barrier.
    auto dma_one = [&](int64_t kt, int stage, int d) __attribute__((always_inline)) {
        const int64_t k0 = kt * BK;
        const uint32_t so = static_cast<uint32_t>(stage) * STAGE_BYTES;
        if (d < DPO)
            dma16(a_src[d] + k0, a_dst0 + so + 1024 * d);
        else
            dma16(b_src[d - DPO] + k0 * p.sbk, b_dst0 + so + 1024 * (d - DPO));
    };

    // ---- fragment read offsets (bytes within a stage) ---------------------
    // A: lane reads row wm*128 + i*32 + lane%32, logical chunk 2*kk + lane/32.
    int a_off[MT][2];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int r = wm * 128 + i * 32 + (lane & 31);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
            a_off[i][kk] = r * 64 + (((2 * kk + (lane >> 5)) ^ swz_a(r)) * 16);
    }
    // B (transposing read): within 16-lane group G = lane/16, lane i = lane%16
    // addresses k-row kk*16 + 8*(G/2) + 4*e + i/4 at column
    // wn*WN_COLS + j*32 + 16*(G%2) + 4*(i%4).
    const int G = lane >> 4, li = lane & 15;
    int b_off[NT][2][2];
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int k = kk * 16 + 8 * (G >> 1) + 4 * e + (li >> 2);
                const int n = wn * WN_COLS + j * 32 + 16 * (G & 1) + 4 * (li & 3);
                b_off[j][kk][e] = A_STAGE_BYTES + k * 512 + (((n >> 3) ^ swz_b(k)) * 16) +
                                  ((n >> 2) & 1) * 8;
            }

    // Fragments of one 16-deep k-step.
    struct Frags {
        u32x4 a[MT], b[NT];
    };
    // Read q of a k-step's fragments: q < MT the A blocks, then the low and
    // high halves of the NT B blocks.
    auto read_one = [&](Frags &f, const char *st, int kk, int q) __attribute__((always_inline)) {
        if (q < MT) {
            f.a[q] = *LDS_PTR(const u32x4, st + a_off[q][kk]);
        } else {
            const int j = (q - MT) >> 1, e = (q - MT) & 1;
            const s16x4 v =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, st + b_off[j][kk][e]));
            const u32x2 w = __builtin_bit_cast(u32x2, v);
            if (e == 0) {
                f.b[j].x = w.x;
                f.b[j].y = w.y;
            } else {
                f.b[j].z = w.x;
                f.b[j].w = w.y;
            }
        }
    };
    auto read_frags = [&](Frags &f, int stage, int kk) __attribute__((always_inline)) {
        const char *st = lds + stage * STAGE_BYTES;
#pragma unroll
        for (int q = 0; q < NREAD; ++q)
            read_one(f, st, kk, q);
    };

    floatx16 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
            acc[i][j] = floatx16{0.0f};

    auto mfmas = [&](const Frags &f) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < NT; ++j)
                acc[i][j] = mfma<IN>(f.a[i], f.b[j], acc[i][j]);
    };

    // The MFMAs of one k-step with the reads of the next k-step's fragments
    // interleaved one after each MFMA, and (when `dma`) the loads of chunk
    // `dma_kt` one after every second MFMA.
    auto half_step = [&](const Frags &cur, Frags &next, const char *next_st, int next_kk,
                         bool dma, int64_t dma_kt, int dma_stage) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < NMFMA; ++q) {
            const int i = q / NT, j = q % NT;
            acc[i][j] = mfma<IN>(cur.a[i], cur.b[j], acc[i][j]);
            if (q < NREAD)
                read_one(next, next_st, next_kk, q);
            if (dma && (q & 1) && (q >> 1) < DMA_GROUP)
                dma_one(dma_kt, dma_stage, q >> 1);
            if (dma) {
                __builtin_amdgcn_sched_barrier(0);  // keep this group in place
            } else {
                __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);  // the MFMA
                if (q < NREAD)
                    __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);  // the read
            }
        }
    };

    // Pipeline.  Chunk kt lives in stage kt % 4.  Iteration kt: MFMAs of
    // k-step 0 while reading k-step 1's fragments; wait until this wave's
    // loads of chunk kt + 1 have landed and all its LDS reads have returned,
    // then barrier -- after it every wave is done with stage kt % 4, since
    // both k-steps of chunk kt were read before it; MFMAs of k-step 1 while
    // reading chunk kt + 1's first fragments and loading chunk kt + 4 into
    // stage kt % 4.  Chunks kt + 2 .. kt + 4 are in flight meanwhile.  Past
    // the end the loads re-read the last chunk into the freed stage, which
    // keeps the number of loads in flight the same every iteration.
    const int64_t nk = k_split / BK;
#pragma unroll
    for (int s = 0; s < STAGES; ++s)
#pragma unroll
        for (int d = 0; d < DMA_GROUP; ++d)
            dma_one(s < nk ? s : nk - 1, s, d);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(3 * DMA_GROUP, 0));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    Frags f0, f1;
    read_frags(f0, 0, 0);
    for (int64_t kt = 0; kt + 1 < nk; ++kt) {
        const int stage = static_cast<int>(kt % STAGES);
        const char *st = lds + stage * STAGE_BYTES;
        half_step(f0, f1, st, 1, false, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * DMA_GROUP, 0));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        const int64_t kl = kt + STAGES < nk ? kt + STAGES : nk - 1;
        half_step(f1, f0, lds + ((stage + 1) % STAGES) * STAGE_BYTES, 0, true, kl, stage);
        __builtin_amdgcn_sched_barrier(0);
    }
    // last chunk
    read_frags(f1, static_cast<int>((nk - 1) % STAGES), 1);
    mfmas(f0);
    mfmas(f1);
    // no load may still be writing LDS when the workgroup ends
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));

    // Epilogue: lane holds column lane%32 and rows 8*(v/4) + 4*(lane/32) + v%4
    // of each 32x32 tile.
    void *c_out = static_cast<char *>(p.C) + slice * c_split_stride * (OUT == DTM_F32 ? 4 : 2);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int64_t col = n0 + wn * WN_COLS + j * 32 + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = m0 + wm * 128 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                store_elem<OUT>(c_out, row * p.scm + col * p.scn, acc[i][j][v]);
            }
        }
    }
}

#ifndef DTM_DMA_WAVES
#define DTM_DMA_WAVES 8
#endif

template <int IN, int OUT>
hipError_t launch(const GemmArgs &a, int64_t splits, hipStream_t s)
{
    const int64_t gm = a.M / BM, gn = a.N / BN;
    hipLaunchKernelGGL((gemm_mfma16_dma_kernel<IN, OUT, DTM_DMA_WAVES>),
                       dim3((unsigned)(gm * gn * splits)), dim3(64 * DTM_DMA_WAVES), 0, s, a, gm, gn,
                       a.K / splits, a.M * a.N);
    return hipGetLastError();
}

template <int IN>
hipError_t dispatch_out(const GemmArgs &a, int out, int64_t splits, hipStream_t s)
{
    switch (out) {
    case DTM_F32: return launch<IN, DTM_F32>(a, splits, s);
    case DTM_F16: return launch<IN, DTM_F16>(a, splits, s);
    case DTM_BF16: return launch<IN, DTM_BF16>(a, splits, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool mfma16_dma_fits(int64_t M, int64_t N, int64_t K, int64_t splits)
{
    return M > 0 && N > 0 && K > 0 && splits > 0 && M % BM == 0 && N % BN == 0 &&
           K % (BK * splits) == 0 && (M / BM) * (N / BN) * splits <= 0x7fffffffLL;
}

hipError_t launch_mfma16_dma(const GemmArgs &a, int in, int out, hipStream_t s)
{
    if (!mfma16_dma_fits(a.M, a.N, a.K, 1))
        return hipErrorInvalidConfiguration;
    switch (in) {
    case DTM_F16: return dispatch_out<DTM_F16>(a, out, 1, s);
    case DTM_BF16: return dispatch_out<DTM_BF16>(a, out, 1, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_mfma16_dma_partials(const GemmArgs &a, int in, int64_t splits, float *ws,
                                      hipStream_t s)
{
    if (!mfma16_dma_fits(a.M, a.N, a.K, splits))
        return hipErrorInvalidConfiguration;
    GemmArgs w = a;
    w.C = ws;  // dense fp32 [splits][M][N]
    w.scm = a.N;
    w.scn = 1;
    switch (in) {
    case DTM_F16: return dispatch_out<DTM_F16>(w, DTM_F32, splits, s);
    case DTM_BF16: return dispatch_out<DTM_BF16>(w, DTM_F32, splits, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace dtm
