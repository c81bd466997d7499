// kernels.hpp -- host-side launchers of the ARCHead forward kernels.
#pragma once
#include <hip/hip_runtime.h>

#include "layout.hpp"

namespace archead {

// a1: t = X (sB o B8)^T and s = X (sD o D8)^T as bf16 hi/lo pairs, and the
// per-(group, row) X sums the residual kernels need.
hipError_t launch_proj(const DevHead &h, const Work &w, const uint16_t *X, hipStream_t st);

// a1 for large M on the matrix cores: fp32 t and s into w.tf32 / w.sf32 (no
// per-group X sums); it pairs with the large-M vocabulary-tile kernel.
hipError_t launch_proj_mfma(const DevHead &h, const Work &w, const uint16_t *X, hipStream_t st);

// a2-S: one streaming kernel over vocabulary tiles (any M; the packed codes
// are streamed once per 32 hidden states): per v-block the low-rank codes,
// then the SC4 residual, then the logits (if logits is not null) and, if
// argmax is not null, the per-workgroup top-1 partials in w.part (and, with
// w.want_lse, the log-sum-exp summaries in w.lsep), which launch_finish
// reduces.
hipError_t launch_vtile_skinny(const DevHead &h, const Work &w, const uint16_t *X, float *logits,
                               int32_t *argmax, hipStream_t st);

// number of argmax partials per row the skinny path writes for M rows, and
// the largest such number over every M (sizes the workspace)
int64_t skinny_n_part(const DevHead &h, int64_t M);
int64_t skinny_max_n_part(const Shape &s);

// a2-S for batched decode (2 <= M <= 32, g = 128): one persistent streaming
// kernel, one workgroup of 8 waves per compute unit, X staged in LDS slab by
// slab (vtile2.hip).  Needs launch_proj first; argmax partials as for the
// other a2-S kernel, one per workgroup.
bool stream2_ok(const DevHead &h, int64_t M);
int64_t stream2_n_part(const DevHead &h, int64_t M);
int64_t stream2_max_n_part(const Shape &s);
hipError_t launch_vtile_stream2(const DevHead &h, const Work &w, const uint16_t *X, float *logits,
                                int32_t *argmax, hipStream_t st);

// a2-L: LDS-staged fp16 MFMA over [128 hidden states x 512 vocabulary rows]
// tiles for large M.  Needs launch_proj_mfma then launch_prep_lds first.
// Every B operand is an integer code times its row-normalised scale, rounded
// once to fp16; the A operands are X, and the fp16 hi/lo parts of t and s,
// scaled by a per-row power of two.  Argmax partials as for a2-S.
hipError_t launch_prep_lds(const DevHead &h, const Work &w, const uint16_t *X, hipStream_t st);
hipError_t launch_vtile_lds(const DevHead &h, const Work &w, float *logits, int32_t *argmax,
                            hipStream_t st);
int64_t lds_n_part(const DevHead &h, int64_t M);
int64_t lds_max_n_part(const Shape &s);
// stages of the a2-L kernel (rows of its stage-fill table in the workspace)
int64_t lds_stages(const Shape &s);

// smallest M for which the automatic choice takes a2-L
constexpr int64_t kLdsMinM = 128;

// a1 + a2 + a3 in one launch for M <= kDecodeMaxM: the projection columns
// computed by the grid's first waves, the argmax resolved by the last
// workgroup.  mx = false: VALU bf16-pair dot products (a2-G); mx = true:
// the same stream with the products on the matrix cores (a2-S, g = 128,
// M = 1).
// With w.want_lse the last workgroup also merges every workgroup's
// log-sum-exp summary into lse (and nll, with w.targets).
// decode_ok tells whether a shape and M are supported.
bool decode_ok(const DevHead &h, int64_t M, bool mx);
// Top-k selection inside the same launch: the K largest logits of each hidden
// state (values and indices, M x K) and, with u, one draw per hidden state
// from them at the temperature whose log2(e) / tau is scale.
struct DecodeTopk {
    int K;
    float *values;
    int32_t *indices;
    const float *u;  // may be null (no draw)
    float scale;
    int32_t *samples;
};
bool decode_topk_ok(const DevHead &h, int64_t M, bool mx);
hipError_t launch_decode(const DevHead &h, const Work &w, const uint16_t *X, float *logits, int32_t *argmax,
                         float *lse, float *nll, bool mx, hipStream_t st, const DecodeTopk *tk = nullptr);
// keys the single-launch selection writes per hidden state (workspace sizing)
int64_t decode_topk_keys(const Shape &s);

// a3 (and the log-normaliser): reduce each row's argmax partial keys to an
// index (argmax not null) and its log-sum-exp summaries to lse and, with
// targets, nll = lse - the target's logit (lse not null).
hipError_t launch_finish(const Work &w, int64_t n_part, int64_t V, int32_t *argmax, float *lse, float *nll,
                         hipStream_t st);

// top-k: the K largest logits of each row (larger value first, equal values
// by lower index), 1 <= K <= min(kTopKMax, V), over logits already written:
// per-slice selection, then a per-row merge (topk.hip).
constexpr int kTopKMax = 16;
int64_t topk_slices(int64_t V);
hipError_t launch_topk(const Work &w, const float *logits, int64_t V, int K, float *values,
                       int32_t *indices, hipStream_t st);

// top-k sampling: per row, the index drawn from its K candidates (values in
// descending order) at temperature > 0 with the uniform number u[m] in [0, 1).
hipError_t launch_topk_sample(const float *values, const int32_t *indices, int64_t M, int K, float temperature,
                              const float *u, int32_t *samples, hipStream_t st);

} // namespace archead
