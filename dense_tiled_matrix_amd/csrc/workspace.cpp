// workspace.cpp -- the device workspace the library keeps for split-K
// partials and the split-row softmax statistics, one per (device, stream).
//
// It is reserved only by gemm_workspace_reserve(), which may allocate and
// wait for the stream; gemm(), gemm_ex() and row_softmax() only lease what is
// already reserved (no allocation, no free, no wait) and plan within it.
// A lease holds the entry's lock from reading the pointer until the call has
// queued every launch that uses it, so the partial-product and reduction
// launches of two calls on one stream from two threads cannot interleave,
// and a reservation cannot free a buffer a call is about to launch on.
// Entries are never removed (release frees the memory, keeps the entry), so
// a pointer to one stays valid for the life of the process.
#include <map>
#include <memory>
#include <mutex>
#include <utility>

#include "dtm_gemm.h"
#include "host_util.h"

namespace dtm {

struct WorkspaceEntry {
    std::mutex m;
    void *ptr = nullptr;
    uint64_t bytes = 0;
};

namespace {
std::mutex g_map_mutex;
std::map<std::pair<int, void *>, std::unique_ptr<WorkspaceEntry>> g_entries;

WorkspaceEntry *find_entry(void *stream, bool create)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_map_mutex);
    const auto key = std::make_pair(dev, stream);
    auto it = g_entries.find(key);
    if (it != g_entries.end())
        return it->second.get();
    if (!create)
        return nullptr;
    auto e = std::make_unique<WorkspaceEntry>();
    WorkspaceEntry *raw = e.get();
    g_entries.emplace(key, std::move(e));
    return raw;
}
}  // namespace

WorkspaceLease::WorkspaceLease(void *stream)
{
    WorkspaceEntry *e = find_entry(stream, false);
    if (!e)
        return;
    lock_ = std::unique_lock<std::mutex>(e->m);
    ptr_ = e->ptr;
    bytes_ = e->ptr ? e->bytes : 0;
}

int workspace_reserve(void *stream, uint64_t bytes)
{
    WorkspaceEntry *e = find_entry(stream, true);
    if (!e)
        return DTM_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(e->m);
    if (e->ptr && e->bytes >= bytes)
        return DTM_OK;
    if (bytes == 0)
        return DTM_OK;
    if (e->ptr) {
        // earlier work on the stream may still read the old buffer
        if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess)
            return DTM_ERR_WORKSPACE;
        (void)hipFree(e->ptr);
        e->ptr = nullptr;
        e->bytes = 0;
    }
    void *p = nullptr;
    if (hipMalloc(&p, bytes) != hipSuccess) {
        (void)hipGetLastError();
        return DTM_ERR_WORKSPACE;
    }
    e->ptr = p;
    e->bytes = bytes;
    return DTM_OK;
}

int workspace_release(void *stream)
{
    WorkspaceEntry *e = find_entry(stream, false);
    if (!e)
        return DTM_OK;
    std::lock_guard<std::mutex> lock(e->m);
    if (!e->ptr)
        return DTM_OK;
    if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess)
        return DTM_ERR_WORKSPACE;
    (void)hipFree(e->ptr);
    e->ptr = nullptr;
    e->bytes = 0;
    return DTM_OK;
}

uint64_t workspace_reserved(void *stream)
{
    WorkspaceEntry *e = find_entry(stream, false);
    if (!e)
        return 0;
    std::lock_guard<std::mutex> lock(e->m);
    return e->ptr ? e->bytes : 0;
}

}  // namespace dtm

extern "C" {

int gemm_workspace_reserve(uint64_t bytes, void *stream)
{
    return dtm::workspace_reserve(stream, bytes);
}

int gemm_workspace_release(void *stream) { return dtm::workspace_release(stream); }

uint64_t gemm_workspace_reserved(void *stream) { return dtm::workspace_reserved(stream); }

}  // extern "C"
