// gemm_noalloc.hip -- gemm_ex_noalloc: gemm_ex for callers that cannot
// allocate device memory at all, not even once beforehand through
// gemm_workspace_reserve (code under stream capture, serving loops, hosts
// that forbid allocation).  The split-K partials go into `scratch`, a fixed
// array of device memory that is part of the library's code object: each
// GPU the library runs on holds its own copy until the process ends.
//
// Its device address is taken once per device, with that device current,
// on the entry point's first call there (hipGetSymbolAddress), and kept; the
// kernels get that address as their workspace argument.  The name `scratch`
// itself is a host-side stand-in and is never passed to a kernel.
//
// Every call on one GPU shares that GPU's array and it keeps whatever the
// last call left: the split-K pass writes every partial before the sum reads
// it, so nothing has to start at zero.  Calls that overlap on one GPU (two
// streams, or two threads) race on the array.
#include <mutex>

#include "dtm_gemm.h"
#include "host_util.h"

namespace {

constexpr uint64_t SCRATCH_BYTES = 32ull << 20;  // 32 MiB: the largest split-K workspace served
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];

// The device address of the current device's `scratch`, looked up on the
// first call on that device.
int scratch_address(void **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return DTM_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return DTM_ERR_DEVICE;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DTM_OK;
}

}  // namespace

extern "C" {

int gemm_ex_noalloc(int64_t M, int64_t N, int64_t K, const void *A, int64_t stride_am,
                    int64_t stride_ak, const void *B, int64_t stride_bk, int64_t stride_bn,
                    void *C, int64_t stride_cm, int64_t stride_cn, int in_dtype, int out_dtype,
                    const dtm_tile_config *force, void *stream)
{
    // the selector plans within the array; a forced split that needs more
    // is refused before anything else happens
    dtm_tile_config cfg{};
    if (force)
        cfg = *force;
    if (cfg.workspace_limit == 0 || cfg.workspace_limit > SCRATCH_BYTES)
        cfg.workspace_limit = SCRATCH_BYTES;
    dtm_plan plan;
    int st = gemm_plan(M, N, K, A, stride_am, stride_ak, B, stride_bk, stride_bn, C, stride_cm,
                       stride_cn, in_dtype, out_dtype, &cfg, &plan);
    if (st != DTM_OK)
        return st;
    if (plan.workspace_bytes > SCRATCH_BYTES)
        return DTM_ERR_SCRATCH;
    if (plan.kernel == DTM_KERNEL_NONE)
        return DTM_OK;
    st = dtm::check_device();
    if (st != DTM_OK)
        return st;
    void *ws = nullptr;
    st = scratch_address(&ws);
    if (st != DTM_OK)
        return st;
    return dtm::gemm_ex_library_ws(M, N, K, A, stride_am, stride_ak, B, stride_bk, stride_bn, C,
                                   stride_cm, stride_cn, in_dtype, out_dtype, &cfg, ws,
                                   SCRATCH_BYTES, stream);
}

uint64_t gemm_noalloc_scratch_bytes(void) { return SCRATCH_BYTES; }

}  // extern "C"
