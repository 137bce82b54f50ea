// gemm_mfma16_wavek.hip -- the fp16/bf16 MFMA GEMM on 128 x 128 tiles whose
// K loop is split across the workgroup's 4 waves (DTM_KERNEL_MFMA_F16_WAVEK).
//
// The computation is the blocked product of "Chapter 13: The Blocked Matmul
// Kernel" (section 13.1): one workgroup per output tile (per K slice with
// split-K), fp32 accumulators zeroed once, one conversion at the store
// (section 13.3).  Inside the workgroup the K loop's 32-deep chunks are dealt
// to the waves in turn, and the four partial tiles are added in a fixed
// order before the store.  Interior shapes only: M and N multiples of 128,
// each K slice a multiple of 128.
#include <type_traits>

#include "mfma16_stage.h"

namespace dtm {
namespace {

// 128 x 128 tiles with the K loop split across the workgroup's 4 waves:
// every wave accumulates the whole tile (128 x 128, like a wave of the
// 256-wide tile) over every fourth 32-deep chunk, and the four partial tiles
// are summed in LDS at the end.  Against the 4 waves of 64 x 64 of
// gemm_mfma16_dma_kernel at tile 128, each MFMA needs half the LDS fragment
// reads and each barrier covers 64 MFMAs per wave instead of 16; the global
// bytes per tile are the same.  Meant for few output tiles and long K (the
// split-K plans), where the 256-wide tiles would need 4x the partials.
//
// LDS: a region is 4 consecutive chunks (128 k) of A's 128 rows and of B's
// 128 columns, each operand's part (32 KiB) laid out exactly as one operand
// of a region of the 256-wide paired stages whose "256 rows" are (k half h2,
// row r) with k = 64 * h2 + ..: chunk c of a region (k 32c ..) sits where the
// paired layout keeps rows/columns 128 * (c / 2) .. of half c % 2.  Wave w
// reads chunk w of each region with the paired form's fragment offsets.
// Region r's fragments sit in registers while regions r + 1 and r + 2 sit in
// four of five 32 KiB slots (all 160 KiB of LDS), so a load has more than a
// whole iteration before it is waited for (against one region ahead: long-K
// 512 x 512 x 65536 5% slower warm, 18% slower cold).  The fifth slot lets
// the refill start with the iteration: in its first half a wave reads region
// r + 1's B fragments and loads A's part of region r + 3 into the free slot;
// after a barrier it reads region r + 1's A fragments and loads B's part of
// region r + 3 into the B slot just read, whose A slot then becomes the free
// one.  Each half then issues 8 of a wave's 16 loads (a region's 64 KiB take
// the CU's address unit about as long as the iteration's MFMAs; with all 16
// in the 40 MFMAs after the reads the loop ran 1742 shader cycles an
// iteration against 1425 now, 1024 being the MFMAs alone).  K slices are
// whole regions (128 k).
//
// The sum of the four wave tiles goes through LDS in two passes of half the
// tile's rows each: every wave writes its blocks of that half, then the two
// waves that own a quarter of it read the four contributions back and add
// them as (w0 + w2) + (w1 + w3), the same order for every element whichever
// wave adds, and store their quarter.
template <int IN, int OUT, bool TA, bool TB>
__global__ __launch_bounds__(256) void gemm_mfma16_wavek_kernel(GemmArgs p, int64_t grid_m,
                                                                int64_t grid_n, int64_t splits,
                                                                int64_t k_split,
                                                                int64_t c_split_stride)
{
    constexpr int TILE = 128, VT = 256;    // tile; width of the paired layout reused
    constexpr int RK = 4 * BK;             // k per region
    constexpr int HALF = VT * BK * 2;      // 16 KiB
    constexpr int OPB = 2 * HALF;          // an operand's part of a region: 32 KiB
    constexpr int LPR = krow_chunks<VT>(); // 16-byte chunks per (virtual) k-row: 32
    constexpr int ROWB = VT * 2;
    constexpr bool A_KC = !TA, B_KC = TB;
    constexpr int MT = 8, NT = 8;
    constexpr int A_READS = MT * (A_KC ? 1 : 2);
    constexpr int B_READS = NT * (B_KC ? 1 : 2);
    constexpr int NMFMA = MT * NT;               // 64
    constexpr int SEGS = OPB / 1024 / 4;         // 1 KiB loads per operand per wave: 8
    constexpr int GROUP = 2 * SEGS;              // loads per wave per refill: 16
    static_assert(NMFMA % 2 == 0 && B_READS <= NMFMA / 2 && A_READS <= NMFMA / 2,
                  "wave-K schedule");

    __shared__ __attribute__((aligned(1024))) char lds[5 * OPB];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);

    int64_t pid_m, pid_n;
    const int64_t tiles = grid_m * grid_n;
    const int64_t t_id = xcd_remap(blockIdx.x, tiles * splits);
    const int64_t slice = t_id / tiles;
    grouped_tile(t_id - slice * tiles, grid_m, grid_n, GROUP_M, pid_m, pid_n);
    const int64_t m0 = pid_m * TILE, n0 = pid_n * TILE;
    const int64_t kb = slice * k_split;

    // This lane's element offset from the tile's origin for load `seg` of a
    // region.  K-contiguous: virtual row R = 8 seg + lane / 8 is row R % 128,
    // k 64 (R / 128) + 8 u; otherwise virtual k-row kp (0..63) and 16-byte
    // column chunk c (0..31) are k 64 (c / 16) + kp, columns 8 (c % 16) ...
    auto region_elem = [&](bool kc, int64_t s_mn, int64_t s_k, int seg)
                           __attribute__((always_inline)) {
        if (kc) {
            const int R = 8 * seg + (lane >> 3);
            const int u = (lane & 7) ^ swz_row128(R);
            return static_cast<int64_t>(R & (TILE - 1)) * s_mn + 64 * (R >> 7) + 8 * u;
        }
        const int g = 64 * seg + lane, kp = g / LPR;
        const int c = krow_logical<VT>(g % LPR, kp % BK);
        return static_cast<int64_t>(64 * (c >> 4) + kp) * s_k + 8 * (c & 15);
    };
    const uint16_t *a_org =
        static_cast<const uint16_t *>(p.A) + (A_KC ? m0 * p.sam + kb : kb * p.sak + m0);
    const uint16_t *b_org =
        static_cast<const uint16_t *>(p.B) + (B_KC ? n0 * p.sbn + kb : kb * p.sbk + n0);
    uint32_t a_voff[SEGS], b_voff[SEGS];
#pragma unroll
    for (int d = 0; d < SEGS; ++d) {
        a_voff[d] = static_cast<uint32_t>(2 * region_elem(A_KC, p.sam, p.sak, SEGS * wave + d));
        b_voff[d] = static_cast<uint32_t>(2 * region_elem(B_KC, p.sbn, p.sbk, SEGS * wave + d));
    }
    const int64_t a_reg = A_KC ? RK : RK * p.sak;
    const int64_t b_reg = B_KC ? RK : RK * p.sbk;
    const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(LDS_PTR(char, lds)));
    const uint32_t a_dst0 = lds_base + (SEGS * wave) * 1024;
    const uint32_t b_dst0 = lds_base + (SEGS * wave) * 1024;

    // This wave's chunk of a region: rows/columns 128 (wave / 2) .. of the
    // virtual layout, half wave % 2.
    const int vbase = 128 * (wave >> 1), hh = wave & 1;
    int a_off[MT], b_off[NT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int o = frag_off_pair<A_KC, VT>(vbase + i * 16, lane);
        a_off[i] = A_KC ? (o ^ (64 * hh)) : o + hh * HALF;
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int o = frag_off_pair<B_KC, VT>(vbase + j * 16, lane);
        b_off[j] = B_KC ? (o ^ (64 * hh)) : o + hh * HALF;
    }

    u32x4 fa0[MT], fa1[MT], fb0[NT], fb1[NT];
    auto read_a = [&](u32x4 (&fa)[MT], const char *rg, int i) __attribute__((always_inline)) {
        if constexpr (A_KC) {
            fa[i] = *LDS_PTR(const u32x4, rg + a_off[i]);
        } else {
            read_tr_half(fa[i], 0, rg + a_off[i]);
            read_tr_half(fa[i], 1, rg + a_off[i] + 4 * ROWB);
        }
    };
    auto read_b = [&](u32x4 (&fb)[NT], const char *rg, int q) __attribute__((always_inline)) {
        if constexpr (B_KC)
            fb[q] = *LDS_PTR(const u32x4, rg + b_off[q]);
        else
            read_tr_half(fb[q >> 1], q & 1, rg + b_off[q >> 1] + 4 * ROWB * (q & 1));
    };
    constexpr int A_PER = A_KC ? 1 : 2;

    floatx4 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
            acc[i][j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

    // Pipeline: region r in registers, regions r + 1 and r + 2 in four of
    // the five slots (slots of operand parts, tracked in sa1/sb1, sa2/sb2,
    // sf below).  Iteration r: wait for region r + 1's loads (region
    // r + 2's may be in flight) and for this wave's reads of the last
    // iteration, and barrier; during MFMAs 0 .. H - 1 of region r read region
    // r + 1's B fragments and load A's part of region r + 3 into the free
    // slot; wait for the reads and barrier (every wave is done with region
    // r + 1's B slot); during MFMAs H .. 63 read region r + 1's A fragments
    // and load B's part of region r + 3 into that B slot.  Region r + 1's A
    // slot is the next free one: the next iteration's wait and barrier cover
    // every wave's reads of it.  Loads past the slice's end read a zero-sized
    // buffer: no memory traffic, and they only fill a slot that is not read
    // again.  (H = 24 and 40 measured level with 32.)
    constexpr int H = NMFMA / 2;
    constexpr int P2 = NMFMA - H;
    // load d of A's (dma_a) or B's (dma_b) part of region j into `slot`
    // (offsets below PAIR_SPAN_MAX: wavek_span_ok); a region past the slice's
    // end (!live) reads a zero-sized buffer
    auto dma_a = [&](int64_t j, bool live, int slot, int d) __attribute__((always_inline)) {
        dma16_buf(buffer_rsrc(a_org + j * a_reg, live ? PAIR_SPAN_MAX : 0u), a_voff[d],
                  a_dst0 + static_cast<uint32_t>(slot) * OPB + 1024 * d);
    };
    auto dma_b = [&](int64_t j, bool live, int slot, int d) __attribute__((always_inline)) {
        dma16_buf(buffer_rsrc(b_org + j * b_reg, live ? PAIR_SPAN_MAX : 0u), b_voff[d],
                  b_dst0 + static_cast<uint32_t>(slot) * OPB + 1024 * d);
    };
    auto step = [&](const u32x4 (&fa)[MT], u32x4 (&fan)[MT], const u32x4 (&fb)[NT],
                    u32x4 (&fbn)[NT], const char *nra, const char *nrb, bool full, int64_t dma_j,
                    bool live, int slot_a, int slot_b) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < NMFMA; ++q) {
            const int i = q / NT, j = q % NT;
            acc[i][j] = mfma<IN>(fa[i], fb[j], acc[i][j]);
            if (full) {
                if (q < H) {
                    const int r0 = q * B_READS / H, r1 = (q + 1) * B_READS / H;
#pragma unroll
                    for (int r = r0; r < r1; ++r)
                        read_b(fbn, nrb, r);
                    const int d0 = q * SEGS / H, d1 = (q + 1) * SEGS / H;
#pragma unroll
                    for (int d = d0; d < d1; ++d)
                        dma_a(dma_j, live, slot_a, d);
                }
                if (q == H - 1) {
                    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
                    __builtin_amdgcn_s_barrier();
                    asm volatile("" ::: "memory");
                }
                if (q >= H) {
                    const int r0 = (q - H) * A_READS / P2, r1 = (q + 1 - H) * A_READS / P2;
#pragma unroll
                    for (int r = r0; r < r1; ++r)
                        if (r % A_PER == 0)
                            read_a(fan, nra, r / A_PER);
                    const int d0 = (q - H) * SEGS / P2, d1 = (q + 1 - H) * SEGS / P2;
#pragma unroll
                    for (int d = d0; d < d1; ++d)
                        dma_b(dma_j, live, slot_b, d);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    const int64_t nr = k_split / RK;  // regions in this slice, >= 1
    // region 0 in slots (0, 1), region 1 in (2, 3); after region 0 is in
    // registers, region 2 goes to (4, 1) and slot 0 is free
#pragma unroll
    for (int d = 0; d < SEGS; ++d)
        dma_a(0, true, 0, d);
#pragma unroll
    for (int d = 0; d < SEGS; ++d)
        dma_b(0, true, 1, d);
#pragma unroll
    for (int d = 0; d < SEGS; ++d)
        dma_a(1, nr > 1, 2, d);
#pragma unroll
    for (int d = 0; d < SEGS; ++d)
        dma_b(1, nr > 1, 3, d);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(GROUP, 0));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < MT; ++i)
        read_a(fa0, lds, i);
#pragma unroll
    for (int q = 0; q < B_READS; ++q)
        read_b(fb0, lds + OPB, q);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int d = 0; d < SEGS; ++d)
        dma_a(2, nr > 2, 4, d);
#pragma unroll
    for (int d = 0; d < SEGS; ++d)
        dma_b(2, nr > 2, 1, d);
    // slots of region r + 1 (sa1, sb1) and r + 2 (sa2, sb2), and the free one
    int sa1 = 2, sb1 = 3, sa2 = 4, sb2 = 1, sf = 0;

    auto iter = [&](const u32x4 (&fa)[MT], u32x4 (&fan)[MT], const u32x4 (&fb)[NT],
                    u32x4 (&fbn)[NT], int64_t r) __attribute__((always_inline)) {
        // region r + 1 loaded; every wave's reads of the last iteration done
        // (the free slot was region r's A part)
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(GROUP, 0));
        __builtin_amdgcn_s_barrier();
        debug_sync();
        asm volatile("" ::: "memory");
        step(fa, fan, fb, fbn, lds + sa1 * OPB, lds + sb1 * OPB, true, r + 3, r + 3 < nr, sf,
             sb1);
        __builtin_amdgcn_sched_barrier(0);
        // region r + 3 took (sf, sb1); region r + 1's A slot is free once
        // every wave's reads of it are done (the next iteration's wait)
        const int f = sa1, ob1 = sb1;
        sa1 = sa2;
        sb1 = sb2;
        sa2 = sf;
        sb2 = ob1;
        sf = f;
    };
    int64_t r = 0;
    if ((nr & 1) == 0) {
        iter(fa0, fa1, fb0, fb1, 0);
#pragma unroll
        for (int i = 0; i < MT; ++i)
            fa0[i] = fa1[i];
#pragma unroll
        for (int j = 0; j < NT; ++j)
            fb0[j] = fb1[j];
        r = 1;
    }
    for (; r + 2 < nr; r += 2) {
        iter(fa0, fa1, fb0, fb1, r);
        iter(fa1, fa0, fb1, fb0, r + 1);
    }
    step(fa0, fa1, fb0, fb1, lds, lds, false, 0, false, 0, 0);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));

    // The sum of the four wave tiles, through LDS (1 KiB per 16 x 16 block
    // of one wave: lane l's 4 values at 16 l), in two passes of half the
    // tile's rows: every wave writes its blocks of half h, then the two
    // waves whose quarters lie in that half (wave w owns blocks i = 2 w,
    // 2 w + 1) read the four contributions back, add them as (w0 + w2) +
    // (w1 + w3) and store.  Written per wave so that every block index is
    // known at compile time; the accumulators go to LDS straight from the
    // accumulation registers.
    __builtin_amdgcn_s_barrier();
    void *c_out = static_cast<char *>(p.C) + slice * c_split_stride * (OUT == DTM_F32 ? 4 : 2);
    auto finish = [&](auto w_tag) __attribute__((always_inline)) {
        constexpr int W = decltype(w_tag)::value, H = W >> 1;
        constexpr int WB = 32 * 1024;  // one wave's half: 4 x 8 blocks
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int i = 4 * h; i < 4 * h + 4; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    lds_write_acc(lds_base + W * WB + ((i & 3) * NT + j) * 1024 + lane * 16,
                                  acc[i][j]);
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
            __builtin_amdgcn_s_barrier();
            if (h == H) {
#pragma unroll
                for (int i = 2 * W; i < 2 * W + 2; ++i) {
#pragma unroll
                    for (int j = 0; j < NT; ++j) {
                        const int o = ((i & 3) * NT + j) * 1024 + lane * 16;
                        floatx4 c[4];
#pragma unroll
                        for (int w = 0; w < 4; ++w)
                            c[w] = *LDS_PTR(const floatx4, lds + w * WB + o);
                        const floatx4 v = (c[0] + c[2]) + (c[1] + c[3]);
                        const int64_t col = n0 + j * 16 + (lane & 15);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int64_t row = m0 + i * 16 + 4 * (lane >> 4) + e;
                            store_elem<OUT>(c_out, row * p.scm + col * p.scn, v[e]);
                        }
                    }
                }
            }
            if (h == 0) {
                __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
                __builtin_amdgcn_s_barrier();
            }
        }
    };
    switch (wave) {
    case 0: finish(std::integral_constant<int, 0>{}); break;
    case 1: finish(std::integral_constant<int, 1>{}); break;
    case 2: finish(std::integral_constant<int, 2>{}); break;
    default: finish(std::integral_constant<int, 3>{}); break;
    }
}

// ---- wave-K launches -------------------------------------------------------

// Every wave-K load offset, from its tile's origin, stays below
// PAIR_SPAN_MAX bytes: a K-contiguous operand spans 128 rows of its leading
// dimension (plus 128 k), an M/N-contiguous one 128 k-rows (plus 128
// columns).
bool wavek_span_ok(const GemmArgs &a, bool ta, bool tb)
{
    const uint64_t lim = PAIR_SPAN_MAX;
    const uint64_t a_span = 2 * (128ull * (uint64_t)(!ta ? a.sam : a.sak) + 128);
    const uint64_t b_span = 2 * (128ull * (uint64_t)(tb ? a.sbn : a.sbk) + 128);
    return a.sam >= 0 && a.sak >= 0 && a.sbk >= 0 && a.sbn >= 0 && a_span < lim && b_span < lim;
}

template <int IN, int OUT, bool TA, bool TB>
hipError_t wavek_launch(const GemmArgs &a, int64_t splits, hipStream_t s)
{
    const int64_t gm = a.M / 128, gn = a.N / 128;
    hipLaunchKernelGGL((gemm_mfma16_wavek_kernel<IN, OUT, TA, TB>), dim3((unsigned)(gm * gn * splits)),
                       dim3(256), 0, s, a, gm, gn, splits, a.K / splits, a.M * a.N);
    return hipGetLastError();
}

template <int IN, int OUT>
hipError_t wavek_layout(const GemmArgs &a, int layout, int64_t splits, hipStream_t s)
{
    switch (layout) {
    case 0: return wavek_launch<IN, OUT, false, false>(a, splits, s);
    case DTM_LAYOUT_A_M_CONTIG: return wavek_launch<IN, OUT, true, false>(a, splits, s);
    case DTM_LAYOUT_B_K_CONTIG: return wavek_launch<IN, OUT, false, true>(a, splits, s);
    case DTM_LAYOUT_A_M_CONTIG | DTM_LAYOUT_B_K_CONTIG:
        return wavek_launch<IN, OUT, true, true>(a, splits, s);
    }
    return hipErrorInvalidValue;
}

template <int IN>
hipError_t wavek_out(const GemmArgs &a, int layout, int out, int64_t splits, hipStream_t s)
{
    switch (out) {
    case DTM_F32: return wavek_layout<IN, DTM_F32>(a, layout, splits, s);
    case DTM_F16: return wavek_layout<IN, DTM_F16>(a, layout, splits, s);
    case DTM_BF16: return wavek_layout<IN, DTM_BF16>(a, layout, splits, s);
    }
    return hipErrorInvalidValue;
}

hipError_t wavek_in(const GemmArgs &a, int in, int layout, int out, int64_t splits, hipStream_t s)
{
    if (!mfma16_wavek_fits(a, layout, splits))
        return hipErrorInvalidConfiguration;
    switch (in) {
    case DTM_F16: return wavek_out<DTM_F16>(a, layout, out, splits, s);
    case DTM_BF16: return wavek_out<DTM_BF16>(a, layout, out, splits, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool mfma16_wavek_fits(const GemmArgs &a, int layout, int64_t splits)
{
    const bool ta = layout & DTM_LAYOUT_A_M_CONTIG, tb = layout & DTM_LAYOUT_B_K_CONTIG;
    return a.M > 0 && a.N > 0 && a.K > 0 && splits > 0 && a.M % 128 == 0 && a.N % 128 == 0 &&
           a.K % (128 * splits) == 0 && (a.M / 128) * (a.N / 128) * splits <= 0x7fffffffLL &&
           wavek_span_ok(a, ta, tb);
}

hipError_t launch_mfma16_wavek(const GemmArgs &a, int in, int out, int layout, hipStream_t s)
{
    return wavek_in(a, in, layout, out, 1, s);
}

hipError_t launch_mfma16_wavek_partials(const GemmArgs &a, int in, int layout, int64_t splits,
                                        float *ws, hipStream_t s)
{
    GemmArgs w = a;
    w.C = ws;  // dense fp32 [splits][M][N]
    w.scm = a.N;
    w.scn = 1;
    return wavek_in(w, in, layout, DTM_F32, splits, s);
}

}  // namespace dtm
