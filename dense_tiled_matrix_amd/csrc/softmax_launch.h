// softmax_launch.h -- host-side launcher of the row-softmax kernels (internal).
#pragma once

#include <hip/hip_runtime.h>

#include "device.h"

namespace dtm {

// Row softmax problem passed by value to every kernel.  Strides are in
// elements; pointers address element (0, 0) of each view.
struct SoftmaxArgs {
    int64_t M, N;
    const void *X;
    int64_t sxm, sxn;
    void *Y;
    int64_t sym, syn;
};

// Launch forms (see softmax.hip).
enum { SOFTMAX_WAVE = 1, SOFTMAX_BLOCK = 2, SOFTMAX_ONLINE = 3, SOFTMAX_SPLIT = 4 };

// Elements one chunk holds: 16 bytes of input when vectorised, else 1.
int softmax_chunk_elems(int in_dtype, bool vec);
// Threads per workgroup and threads per row of a form.
int softmax_form_threads(int form);
int softmax_form_lanes(int form);
// Columns one ONLINE/SPLIT tile covers (a SPLIT part is a multiple of it).
int64_t softmax_tile(int in_dtype, bool vec);
// `ch` chunks per thread: WAVE 1, 2, 4, 8, 16; BLOCK 1, 2, 4; ONLINE ignores
// it; SPLIT: the number of parts per row, with `ws` holding 2 * M * parts
// floats (device memory).
hipError_t launch_softmax(const SoftmaxArgs &a, int in_dtype, int out_dtype, int form, int ch,
                          bool vec, float *ws, hipStream_t s);

}  // namespace dtm
