// api_internal.hpp -- what api.cpp lends to the other host-side entry points
// of the library (the no-allocation forward in noalloc.hip, the construction
// in build.hip).
#pragma once
#include <string>

#include "archead.h"

namespace archead {

// records msg as the calling thread's last error and returns s
archead_status api_fail(archead_status s, const std::string &msg);

// Test hook: with ARCHEAD_TEST_ALLOC_LIMIT=<bytes> in the environment, every
// device allocation of the library larger than that is refused (the caller
// reports ARCHEAD_ENOMEM, as for a failed hipMalloc) before any HIP call.
bool alloc_refused(size_t bytes);

// ARCHEAD_OK and the device the handle lives on, or ARCHEAD_EINVAL for a bad handle
archead_status handle_device(archead_t h, int *device);

// bytes of a workspace laid out for M rows, and the two ranges of it that
// must read as zero when a call starts: [0, zero_head) and [zero_tail, total)
size_t workspace_bytes(archead_t h, int64_t M, size_t *zero_head, size_t *zero_tail);

// archead_forward_argmax (automatic path) on a workspace the caller provides,
// laid out for ws_cap >= M rows; nothing is allocated
archead_status forward_in_workspace(archead_t h, int64_t M, const void *X, float *logits, int32_t *argmax,
                                    void *hip_stream, void *ws, int64_t ws_cap);

} // namespace archead
