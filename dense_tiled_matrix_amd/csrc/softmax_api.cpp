// softmax_api.cpp -- the C ABI of the row softmax: validation, plan, launch.
//
// The operation is the row softmax of "Triton from zero, Lesson 4: Block
// Pointers", homework 4 (see include/dtm_softmax.h).  Every check runs on
// the host before any launch; a non-zero status means nothing was launched.
#include <cstring>

#include "dtm_softmax.h"
#include "host_util.h"
#include "softmax_launch.h"

namespace {

#ifndef DTM_SOFTMAX_WAVE_MIN_ROWS
#define DTM_SOFTMAX_WAVE_MIN_ROWS 2048
#endif
#ifndef DTM_SOFTMAX_BLOCK_MAX_CH
#define DTM_SOFTMAX_BLOCK_MAX_CH 16
#endif
#ifndef DTM_SOFTMAX_SPLIT_MAX_ROWS
#define DTM_SOFTMAX_SPLIT_MAX_ROWS 128
#endif
#ifndef DTM_SOFTMAX_SPLIT_WGS
#define DTM_SOFTMAX_SPLIT_WGS 256
#endif
constexpr int64_t BLOCK_MAX_CH = DTM_SOFTMAX_BLOCK_MAX_CH;      // chunks per thread, fp32 rows
constexpr int64_t SPLIT_MAX_ROWS = DTM_SOFTMAX_SPLIT_MAX_ROWS;  // rows below which rows split
constexpr int64_t SPLIT_WGS = DTM_SOFTMAX_SPLIT_WGS;            // workgroups a split aims for

struct SCall {
    int64_t M, N;
    const void *X;
    int64_t sxm, sxn;
    const void *Y;
    int64_t sym, syn;
    int in, out;
};

int validate(const SCall &c)
{
    constexpr int64_t kMaxDim = 0x7fffffffLL;
    if (c.M < 0 || c.N < 0 || c.M > kMaxDim || c.N > kMaxDim)
        return DTM_ERR_INVALID_DIM;
    if (!dtm::valid_dtype(c.in) || !dtm::valid_dtype(c.out))
        return DTM_ERR_DTYPE;
    if (c.M == 0 || c.N == 0)
        return DTM_OK;
    if (!c.X || !c.Y)
        return DTM_ERR_NULL_POINTER;
    if (!dtm::c_strides_ok(c.M, c.N, c.sym, c.syn))
        return DTM_ERR_STRIDE;
    uintptr_t xlo, xhi, ylo, yhi;
    if (!dtm::view_range(c.X, c.M, c.N, c.sxm, c.sxn, dtm::item_size(c.in), xlo, xhi) ||
        !dtm::view_range(c.Y, c.M, c.N, c.sym, c.syn, dtm::item_size(c.out), ylo, yhi))
        return DTM_ERR_STRIDE;
    const bool in_place = c.X == c.Y && c.sxm == c.sym && c.sxn == c.syn &&
                          dtm::item_size(c.in) == dtm::item_size(c.out);
    if (!in_place && ylo < xhi && xlo < yhi)
        return DTM_ERR_ALIAS;
    return DTM_OK;
}

// 16-byte loads along the rows: unit column strides, 16-byte aligned rows of
// X, and rows of Y aligned to the size of one chunk's output (at most 16).
bool vectorizable(const SCall &c)
{
    if (c.sxn != 1 || c.syn != 1)
        return false;
    const int64_t in_sz = dtm::item_size(c.in), out_sz = dtm::item_size(c.out);
    const int64_t e = 16 / in_sz;
    const int64_t yal = e * out_sz < 16 ? e * out_sz : 16;
    const uintptr_t x = reinterpret_cast<uintptr_t>(c.X), y = reinterpret_cast<uintptr_t>(c.Y);
    if (x % 16 || y % yal)
        return false;
    if (c.M > 1 && ((c.sxm * in_sz) % 16 || (c.sym * out_sz) % yal))
        return false;
    return true;
}

// Past 4 chunks per thread the BLOCK form's workgroup fills a CU's
// registers; it then pays against the ONLINE form (which reads each row
// twice) only when the row fills at least 3/4 of the chunks it is given
// (measured: rows of 40000 fp32, 61% of 16 chunks, 4-8% slower than ONLINE;
// rows that fill 76-100% of 8 or 16 chunks 2-27% faster).
bool block_fill_pays(int64_t N, int64_t chunk_row)
{
    if (N <= chunk_row * 4)
        return true;
    int64_t ch = 1;
    while (chunk_row * ch < N)
        ch *= 2;
    return 4 * N >= 3 * chunk_row * ch;
}

// ws_budget: bytes of workspace the call can use (UINT64_MAX: no limit);
// the SPLIT form keeps 8 bytes per row and part in it, so its part count is
// capped to what fits, and without room for two parts the row is not split.
int make_plan(const SCall &c, uint64_t ws_budget, dtm_softmax_plan *out)
{
    if (!out)
        return DTM_ERR_NULL_POINTER;
    std::memset(out, 0, sizeof(*out));
    const int st = validate(c);
    if (st != DTM_OK)
        return st;
    dtm_softmax_plan p;
    std::memset(&p, 0, sizeof(p));
    if (c.M == 0 || c.N == 0) {
        p.form = DTM_SOFTMAX_NONE;
        *out = p;
        return DTM_OK;
    }
    const bool vec = vectorizable(c);
    const int64_t e = dtm::softmax_chunk_elems(c.in, vec);
    const int64_t wave_lanes = dtm::softmax_form_lanes(dtm::SOFTMAX_WAVE);
    const int64_t block_lanes = dtm::softmax_form_lanes(dtm::SOFTMAX_BLOCK);
    // A wave per row while a row fits in a wave's registers (16 chunks per
    // lane) and there are enough rows to fill the chip; a workgroup per row
    // while it fits in the workgroup's registers (16 chunks per thread for
    // fp32, 8 for 16-bit inputs, whose 16 would not fit the 128 VGPRs of a
    // 1024-thread workgroup); beyond that the two-pass online form.
    const bool many_rows = c.M >= DTM_SOFTMAX_WAVE_MIN_ROWS;
    const int64_t block_max_ch = c.in == DTM_F32 ? BLOCK_MAX_CH : (BLOCK_MAX_CH < 8 ? BLOCK_MAX_CH : 8);
    int form, ch = 0;
    if (c.N <= wave_lanes * e * 16 && (many_rows || c.N <= wave_lanes * e * 2)) {
        form = dtm::SOFTMAX_WAVE;
        for (ch = 1; wave_lanes * e * ch < c.N; ch *= 2) {
        }
    } else if (c.N <= block_lanes * e * block_max_ch && block_fill_pays(c.N, block_lanes * e)) {
        form = dtm::SOFTMAX_BLOCK;
        for (ch = 1; block_lanes * e * ch < c.N; ch *= 2) {
        }
    } else {
        form = dtm::SOFTMAX_ONLINE;
        ch = 2;
    }
    // Few rows that are long: split each row over several workgroups so the
    // chip fills (about SPLIT_WGS workgroups, parts of at least one tile).
    int64_t parts = 1;
    if (form != dtm::SOFTMAX_WAVE && c.M < SPLIT_MAX_ROWS) {
        const int64_t tile = dtm::softmax_tile(c.in, vec);
        const int64_t want = dtm::cdiv(SPLIT_WGS, c.M), tiles = dtm::cdiv(c.N, tile);
        parts = want < tiles ? want : tiles;
        const uint64_t fit = ws_budget / (8u * static_cast<uint64_t>(c.M));
        if (static_cast<uint64_t>(parts) > fit)
            parts = static_cast<int64_t>(fit);
        if (parts >= 2) {
            // no empty part: part length rounded up to whole tiles
            const int64_t len = dtm::cdiv(dtm::cdiv(c.N, parts), tile) * tile;
            parts = dtm::cdiv(c.N, len);
        }
        if (parts >= 2) {
            form = dtm::SOFTMAX_SPLIT;
            ch = 2;
        } else {
            parts = 1;
        }
    }
    p.form = form;
    p.threads = dtm::softmax_form_threads(form);
    p.rows_per_block = form == dtm::SOFTMAX_WAVE ? p.threads / static_cast<int>(wave_lanes) : 1;
    p.chunks = ch;
    p.chunk_elems = static_cast<int32_t>(e);
    p.vectorized = vec ? 1 : 0;
    p.grid = dtm::cdiv(c.M, p.rows_per_block) * parts;
    p.passes = form == dtm::SOFTMAX_ONLINE || form == dtm::SOFTMAX_SPLIT ? 2 : 1;
    p.parts = static_cast<int32_t>(parts);
    *out = p;
    return DTM_OK;
}

SCall make_call(int64_t M, int64_t N, const void *X, int64_t sxm, int64_t sxn, const void *Y,
                int64_t sym, int64_t syn, int in, int out)
{
    return SCall{M, N, X, sxm, sxn, Y, sym, syn, in, out};
}

}  // namespace

extern "C" {

int row_softmax(int64_t M, int64_t N, const void *X, int64_t stride_xm, int64_t stride_xn,
                void *Y, int64_t stride_ym, int64_t stride_yn, int in_dtype, int out_dtype,
                void *stream)
{
    const SCall c = make_call(M, N, X, stride_xm, stride_xn, Y, stride_ym, stride_yn, in_dtype,
                              out_dtype);
    // the split form's workspace: what is reserved for this stream, leased
    // until the launches are queued (no allocation here)
    const dtm::WorkspaceLease lease(stream);
    dtm_softmax_plan p;
    int st = make_plan(c, lease.bytes(), &p);
    if (st != DTM_OK)
        return st;
    if (p.form == DTM_SOFTMAX_NONE)
        return DTM_OK;
    st = dtm::check_device();
    if (st != DTM_OK)
        return st;
    if (dtm::pointer_checks_on()) {
        // X and Y inside device allocations of this device (validate has
        // already shown both ranges are representable)
        uintptr_t lo, hi;
        dtm::view_range(X, M, N, stride_xm, stride_xn, dtm::item_size(in_dtype), lo, hi);
        st = dtm::check_view_memory(lo, hi);
        if (st != DTM_OK)
            return st;
        dtm::view_range(Y, M, N, stride_ym, stride_yn, dtm::item_size(out_dtype), lo, hi);
        st = dtm::check_view_memory(lo, hi);
        if (st != DTM_OK)
            return st;
    }
    const dtm::SoftmaxArgs a{M, N, X, stride_xm, stride_xn, Y, stride_ym, stride_yn};
    float *ws = p.form == DTM_SOFTMAX_SPLIT ? static_cast<float *>(lease.ptr()) : nullptr;
    const hipError_t e = dtm::launch_softmax(
        a, in_dtype, out_dtype, p.form, p.form == DTM_SOFTMAX_SPLIT ? p.parts : p.chunks,
        p.vectorized != 0, ws, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? DTM_OK : DTM_ERR_LAUNCH;
}

int row_softmax_plan(int64_t M, int64_t N, const void *X, int64_t stride_xm, int64_t stride_xn,
                     const void *Y, int64_t stride_ym, int64_t stride_yn, int in_dtype,
                     int out_dtype, dtm_softmax_plan *out)
{
    return make_plan(make_call(M, N, X, stride_xm, stride_xn, Y, stride_ym, stride_yn, in_dtype,
                               out_dtype),
                     UINT64_MAX, out);
}

}  // extern "C"
