// host_util.h -- host-side argument checks shared by the C-ABI entry points
// (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "dtm_gemm.h"

namespace dtm {

inline bool valid_dtype(int d) { return d == DTM_F32 || d == DTM_F16 || d == DTM_BF16; }
inline int64_t item_size(int d) { return d == DTM_F32 ? 4 : 2; }

// Byte range [lo, hi) spanned by a rows x cols view; false on overflow.
inline bool view_range(const void *base, int64_t rows, int64_t cols, int64_t sr, int64_t sc,
                int64_t item, uintptr_t &lo, uintptr_t &hi)
{
    int64_t er, ec;
    if (__builtin_mul_overflow(rows - 1, sr, &er) || __builtin_mul_overflow(cols - 1, sc, &ec))
        return false;
    const int64_t mn = (er < 0 ? er : 0) + (ec < 0 ? ec : 0);
    const int64_t mx = (er > 0 ? er : 0) + (ec > 0 ? ec : 0);
    int64_t blo, bhi;
    if (__builtin_mul_overflow(mn, item, &blo) || __builtin_mul_overflow(mx + 1, item, &bhi))
        return false;
    const uintptr_t b = reinterpret_cast<uintptr_t>(base);
    lo = b + static_cast<uintptr_t>(blo);  // wraps correctly for negative offsets
    hi = b + static_cast<uintptr_t>(bhi);
    if (blo < 0 && static_cast<uintptr_t>(-blo) > b)
        return false;
    if (hi < b)
        return false;
    return true;
}

// Distinct (i, j) of an M x N view with these strides never share an element.
inline bool c_strides_ok(int64_t M, int64_t N, int64_t scm, int64_t scn)
{
    if (scm < 0 || scn < 0)
        return false;
    if (M > 1 && scm == 0)
        return false;
    if (N > 1 && scn == 0)
        return false;
    if (M <= 1 || N <= 1)
        return true;
    // the smaller stride's axis must fit entirely inside one step of the larger
    int64_t s_small = scm, n_small = M, s_big = scn;
    if (scn < scm) {
        s_small = scn;
        n_small = N;
        s_big = scm;
    }
    int64_t span;
    if (__builtin_mul_overflow(s_small, n_small, &span))
        return false;
    return s_big >= span;
}

// Whether the optional pointer checks are on (gemm_set_pointer_checks).
bool pointer_checks_on();

// DTM_OK when the byte range [lo, hi) lies inside one device-memory
// allocation of the current device (as the HIP runtime reports it), else
// DTM_ERR_POINTER.  Only called with pointer checks on.
int check_view_memory(uintptr_t lo, uintptr_t hi);

// DTM_OK when the current HIP device is a gfx950, else DTM_ERR_DEVICE
// (cached per device).
int check_device();

// The workspace reserved for (current device, stream) by
// gemm_workspace_reserve, leased for one call: the lease holds that
// workspace's lock until it is destroyed, so every launch of the call that
// uses it is queued before another call (or a reservation) can touch it.
// ptr() == nullptr and bytes() == 0 when nothing is reserved.  Never
// allocates and never waits for the GPU.
struct WorkspaceEntry;
class WorkspaceLease {
public:
    explicit WorkspaceLease(void *stream);
    void *ptr() const { return ptr_; }
    uint64_t bytes() const { return bytes_; }

private:
    std::unique_lock<std::mutex> lock_;
    void *ptr_ = nullptr;
    uint64_t bytes_ = 0;
};

// Grow the workspace of (current device, stream) to at least `bytes` (waits
// for the stream before freeing a smaller one); release frees it (after
// waiting for the stream).  DTM_OK or DTM_ERR_WORKSPACE.
int workspace_reserve(void *stream, uint64_t bytes);
int workspace_release(void *stream);
uint64_t workspace_reserved(void *stream);

// gemm_ex with `ws` (ws_bytes) as its workspace, memory the library owns
// (left out of the pointer checks).
int gemm_ex_library_ws(int64_t M, int64_t N, int64_t K, const void *A, int64_t sam, int64_t sak,
                       const void *B, int64_t sbk, int64_t sbn, void *C, int64_t scm, int64_t scn,
                       int in_dtype, int out_dtype, const dtm_tile_config *force, void *ws,
                       uint64_t ws_bytes, void *stream);

}  // namespace dtm
