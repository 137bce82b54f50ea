// mfma16_stage.h -- what the fp16/bf16 MFMA kernels with global -> LDS
// staging share (gemm_mfma16_dma.hip, gemm_mfma16_wavek.hip): vector types,
// the LDS DMA loads, the swizzled staging layouts and their fragment reads,
// and the 16 x 16 x 32 MFMA.  The layouts are described where they are
// first used, in gemm_mfma16_dma.hip's file comment.
#pragma once

#include <cstdint>

#include "launch.h"

namespace dtm {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T *)(p))

constexpr int BK = 32, STAGES = 4;
// A TILE x TILE output tile stages TILE x BK of each operand per chunk:
// 16 KiB each at TILE = 256, 12 KiB at 192, 8 KiB at 128.
template <int TILE> constexpr int operand_stage_bytes() { return TILE * BK * 2; }
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

// Swizzles of the two staging forms (see the file comment).
__device__ __forceinline__ int swz_row(int r) { return (r >> 1) & 3; }
__device__ __forceinline__ int swz_krow(int k)
{
    // 0, 6, 10, 12 for k % 4 = 0..3, XOR 2 when k % 16 >= 8: a fragment read
    // has 16-lane groups on k-rows 8 apart, which then land on other banks
    return ((0xCA60 >> (4 * (k & 3))) & 15) ^ ((k & 8) >> 2);
}

// 16 bytes per lane from global memory straight into LDS at
// lds_addr + 16 * lane (global_load_lds_dwordx4; M0 holds the LDS address).
//
// These loads are written in inline asm, each block setting M0 itself, and
// the kernels wait for them with explicit s_waitcnt.  The compiler's builtins
// for the same instructions (global_load_lds, raw_ptr_buffer_load_lds) make
// it treat every load in flight as a possible writer of any later LDS read
// of the same array, so it puts s_waitcnt vmcnt(0) before the fragment reads
// (checked in the wave-K kernel's assembly: 30 vmcnt waits against 5), which
// would serialize the pipelines.  The compiler warns that M0, a register it
// reserves, is in the clobber list; in these kernels it never uses M0 itself
// (every M0 reference in their assembly is one of these blocks' writes,
// each followed by its load), so nothing of its own is overwritten.
__device__ __forceinline__ void dma16(const void *gptr, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(gptr), "s"(lds_addr)
                 : "memory", "m0");
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource (gfx9 layout) over `bytes` bytes at `base`: loads at
// byte offsets >= bytes return zeros.
__device__ __forceinline__ i32x4 buffer_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r.x = __builtin_amdgcn_readfirstlane(static_cast<int>(a & 0xffffffffu));
    r.y = __builtin_amdgcn_readfirstlane(static_cast<int>((a >> 32) & 0xffffu));  // stride 0
    r.z = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
    r.w = 0x00020000;  // 32-bit data format, untyped access
    return r;
}

// As dma16, from byte offset `voff` of a buffer resource.
__device__ __forceinline__ void dma16_buf(const i32x4 &rsrc, uint32_t voff, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(lds_addr)
                 : "memory", "m0");
}

// Offset past every buffer this kernel builds (they are at most 2^31 bytes).
constexpr uint32_t OUTSIDE = 0x80000000u;

// An M/N-contiguous operand is staged as BK k-rows of TILE elements, TILE / 8
// 16-byte chunks per k-row, filled in order by the 1 KiB load segments.
template <int TILE> constexpr int krow_chunks() { return TILE / 8; }

// Physical chunk, within k-row k of such a stage, of logical chunk c, and
// back.  TILE 256 and 128 XOR the chunk index with swz_krow(k).  A 192-wide
// k-row (24 chunks, 384 bytes) already puts odd k-rows 32 banks on, so
// there the chunk index is rotated by 2 * ((k >> 1) & 1) + 4 * ((k >> 3) & 1):
// the eight k-rows a 32-lane half of a fragment read touches (k0..k0+3 and
// k0+8..k0+11) then cover the 64 banks once (checked on every fragment of
// the tile against a model of 32 lanes served per cycle).  Both keep k and
// k + 4 (the two halves of a fragment, k % 8 < 4) on the same permutation.
template <int TILE> __device__ __forceinline__ int krow_phys(int c, int k)
{
    if constexpr (TILE == 192) {
        const int p = c + (k & 2) + ((k & 8) >> 1);
        return p >= 24 ? p - 24 : p;
    } else {
        return c ^ swz_krow(k);
    }
}
template <int TILE> __device__ __forceinline__ int krow_logical(int p, int k)
{
    if constexpr (TILE == 192) {
        const int c = p - (k & 2) - ((k & 8) >> 1);
        return c < 0 ? c + 24 : c;
    } else {
        return p ^ swz_krow(k);
    }
}

// Global source of this lane for 1 KiB segment `seg` of an operand's stage.
// X points at element (0, 0) of the operand viewed as [mn][k]; mn0 and kb
// are the tile's first row/column and the slice's first k.
//  K-contiguous (KC): rows 16*seg + lane/4, physical chunk lane % 4; the
//    logical chunk is the physical one XOR the row's swizzle.
//  otherwise: g = 64*seg + lane, k-row g / LPR, physical chunk g % LPR (the
//    logical one from krow_logical).  Chunk kt of
// the K loop is kt * BK elements further along K.
template <bool KC, int TILE>
__device__ __forceinline__ const uint16_t *stage_src(const uint16_t *X, int64_t mn0, int64_t s_mn,
                                                     int64_t s_k, int64_t kb, int seg, int lane)
{
    if constexpr (KC) {
        const int r = 16 * seg + (lane >> 2);
        const int c = (lane & 3) ^ swz_row(r);
        return X + (mn0 + r) * s_mn + kb + 8 * c;
    } else {
        constexpr int LPR = krow_chunks<TILE>();
        const int g = 64 * seg + lane, k = g / LPR;
        const int c = krow_logical<TILE>(g % LPR, k);
        return X + (kb + k) * s_k + mn0 + 8 * c;
    }
}

// RAGGED form of stage_src: the byte offset of chunk 0 from the operand's
// origin, and a limit such that chunk kt exists in the view iff
// kt * BK < klim (klim = 0 when the lane's row or columns lie outside the
// view).  K is a multiple of 8 and, for an M/N-contiguous operand, so is its
// extent, so each 16-byte chunk is either wholly inside or wholly outside.
template <bool KC, int TILE>
__device__ __forceinline__ void stage_off(int64_t mn0, int64_t s_mn, int64_t s_k, int64_t ext,
                                          int64_t K, int64_t kb, int seg, int lane,
                                          uint32_t &off, int &klim)
{
    int64_t mn, kf, e;
    bool ok;
    if constexpr (KC) {
        const int r = 16 * seg + (lane >> 2);
        const int c = (lane & 3) ^ swz_row(r);
        mn = mn0 + r;
        kf = kb + 8 * c;
        e = mn * s_mn + kf;
        ok = mn < ext;
    } else {
        constexpr int LPR = krow_chunks<TILE>();
        const int g = 64 * seg + lane, k = g / LPR;
        const int c = krow_logical<TILE>(g % LPR, k);
        mn = mn0 + 8 * c;
        kf = kb + k;
        e = kf * s_k + mn;
        ok = mn < ext;
    }
    ok = ok && kf < K;
    off = ok ? static_cast<uint32_t>(2 * e) : 0u;
    klim = ok ? static_cast<int>(K - kf) : 0;
}

// Half (e = 0: k 0..3, e = 1: k 4..7) of a fragment by a transposing read.
__device__ __forceinline__ void read_tr_half(u32x4 &f, int e, const char *p)
{
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, p));
    const u32x2 w = __builtin_bit_cast(u32x2, v);
    if (e == 0) {
        f.x = w.x;
        f.y = w.y;
    } else {
        f.z = w.x;
        f.w = w.y;
    }
}

template <int IN>
__device__ __forceinline__ floatx4 mfma(const u32x4 &a, const u32x4 &b, const floatx4 &c)
{
    if constexpr (IN == DTM_F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                      __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0,
                                                       0);
}

// Byte offset, within an operand's stage, of this lane's fragment read for
// the 16 rows/columns starting at `base` (one whole 32-deep chunk: lane l
// holds 8 consecutive k, k-group l/16, of row/column l%16).
//  K-contiguous: row base + l%16, logical chunk l/16 (one b128 read).
//  otherwise: within 16-lane group G = l/16, lane i = l%16 addresses k-row
//    8*G + i/4 at column base + 4*(i%4); the second read (k + 4) is 4
//    k-rows on.
template <bool KC, int TILE> __device__ __forceinline__ int frag_off(int base, int lane)
{
    const int G = lane >> 4, li = lane & 15;
    if constexpr (KC) {
        const int r = base + li;
        return r * 64 + ((G ^ swz_row(r)) * 16);
    } else {
        const int k = 8 * G + (li >> 2);
        const int n = base + 4 * (li & 3);
        return k * (TILE * 2) + krow_phys<TILE>(n >> 3, k) * 16 + ((n >> 2) & 1) * 8;
    }
}

// Byte extent of the raw buffer each paired-stage load addresses: one chunk
// pair of one operand's tile, from the tile's origin (TILE rows of a
// K-contiguous operand, 64 k-rows of an M/N-contiguous one).
constexpr uint32_t PAIR_SPAN_MAX = 0x80000000u;

// Swizzle of the 128-byte rows of the paired stages: 16-byte unit u of row r
// sits at u ^ ((r >> 1) & 7).  Measured with an in-bounds probe of the
// fragment read order (lane l: row l % 16, unit 4h + l / 16 for either 32-k
// half h): no SQ_LDS_BANK_CONFLICT, against 1/6 to 3/8 of the LDS-active
// cycles for (r >> 1) & 3, (r >> 1) & 6 or no swizzle.
__device__ __forceinline__ int swz_row128(int r) { return (r >> 1) & 7; }

// Byte offset, within a paired-stage region's operand part, of this lane's
// fragment read for the 16 rows/columns starting at `base`, first 32-k half.
// K-contiguous: row base + l % 16 of 128 bytes, unit l / 16 (swizzled);
// otherwise the one-chunk layout of frag_off.
template <bool KC, int TILE> __device__ __forceinline__ int frag_off_pair(int base, int lane)
{
    if constexpr (KC) {
        const int G = lane >> 4, r = base + (lane & 15);
        return r * 128 + ((G ^ swz_row128(r)) * 16);
    } else {
        return frag_off<false, TILE>(base, lane);
    }
}

// 16 bytes of accumulation registers to LDS (ds_write_b128 takes AGPR data
// on this architecture), so that the compiler does not copy a whole
// accumulator array into VGPRs first.  The caller waits (lgkmcnt) for it.
__device__ __forceinline__ void lds_write_acc(uint32_t lds_addr, const floatx4 &v)
{
    asm volatile("ds_write_b128 %0, %1" : : "v"(lds_addr), "a"(v) : "memory");
}

}  // namespace
}  // namespace dtm
