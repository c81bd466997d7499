// kernels.hpp -- host-side launchers of the ARCHead forward kernels.
#pragma once
#include <hip/hip_runtime.h>

#include "layout.hpp"

namespace archead {

// a1: t = X (sB o B8)^T and s = X (sD o D8)^T as bf16 hi/lo pairs, and the
// per-(group, row) X sums the residual kernels need.
hipError_t launch_proj(const DevHead &h, const Work &w, const uint16_t *X, hipStream_t st);

// a2-S: register-dequantised MFMA over vocabulary tiles (any M; the packed
// fields are streamed once per 32 hidden states): a residual-stream kernel
// then a low-rank + epilogue kernel.  logits may be null, in which case
// scratch (M x V fp32) carries the residual term between the two.  argmax may
// be null; when set, the per-workgroup partials are left in w.part and
// launch_argmax must follow (*argmax_done reports whether it already ran).
hipError_t launch_vtile_skinny(const DevHead &h, const Work &w, const uint16_t *X, float *logits,
                               float *scratch, int32_t *argmax, hipStream_t st, bool *argmax_done);

// number of argmax partials per row the skinny path writes
int64_t skinny_n_part(const DevHead &h, int64_t M);

// a3: reduce the argmax partial keys of each row to an index.
hipError_t launch_argmax(const Work &w, int64_t n_part, int32_t *argmax, hipStream_t st);

} // namespace archead
