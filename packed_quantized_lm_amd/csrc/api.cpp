// api.cpp -- the C ABI declared in include/archead.h.
//
// Host side only: argument validation, the one-time relayout and upload of
// the packed fields (pack_load), the per-handle workspace, and dispatch of the
// forward kernels on the caller's stream.
#include "archead.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <set>
#include <string>
#include <thread>
#include <vector>

#include "api_internal.hpp"
#include "kernels.hpp"
#include "layout.hpp"

using namespace archead;

namespace {

constexpr uint64_t kMagic = 0x41524348454144ull; // "ARCHEAD"
constexpr int64_t kMaxM = int64_t(1) << 20;
constexpr size_t kAlign = 256;

thread_local std::string g_err;

std::mutex g_live_mu;
std::set<const void *> g_live;

archead_status fail(archead_status s, const std::string &msg)
{
    g_err = msg;
    return s;
}

#define HIP_TRY(expr)                                                                          \
    do {                                                                                       \
        hipError_t e_ = (expr);                                                                \
        if (e_ != hipSuccess)                                                                  \
            return fail(ARCHEAD_EHIP, std::string(#expr) + ": " + hipGetErrorString(e_));      \
    } while (0)

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

} // namespace

struct archead_head {
    uint64_t magic;
    Shape s;
    DevHead dev;
    void *block;        // one allocation holding every packed array
    size_t block_bytes;
    void *ws;           // workspace
    size_t ws_bytes;
    int64_t ws_M;       // largest M the workspace holds
    int device;
};

namespace {

bool live(archead_t h)
{
    std::lock_guard<std::mutex> g(g_live_mu);
    return h && g_live.count(h) && h->magic == kMagic;
}

struct WsLayout {
    size_t t16, s16, xsneg, tf32, sf32, xsw, tsw, ssw, xsc, lfill, part, lsep, tl, tkp, sync, keys, colflag, ppart, pcnt,
        total;
};

int64_t round_m(int64_t M) { return (M + 31) / 32 * 32; }
int64_t round_m128(int64_t M) { return (M + 127) / 128 * 128; }

// top-k keys the workspace holds: the slice kernel's M x slices x K, or the
// single launch's per-workgroup lists
int64_t tkp_keys(const Shape &s, int64_t Mmax)
{
    return std::max<int64_t>(std::max<int64_t>(Mmax, 1) * topk_slices(s.V) * kTopKMax, decode_topk_keys(s));
}

int64_t max_n_part(const Shape &s)
{
    return std::max<int64_t>(std::max({skinny_max_n_part(s), lds_max_n_part(s), stream2_max_n_part(s)}), 1);
}

WsLayout ws_layout(const Shape &s, int64_t Mmax)
{
    const int64_t Mp = round_m(std::max<int64_t>(Mmax, 1));
    WsLayout L;
    size_t off = 0;
    L.t16 = off;
    off = align_up(off + size_t(2) * Mp * s.kpad() * 2);
    L.s16 = off;
    off = align_up(off + size_t(2) * Mp * s.rpad() * 2);
    L.xsneg = off;
    off = align_up(off + size_t(s.G()) * Mp * 4);
    const int64_t Mq = round_m128(std::max<int64_t>(Mmax, 1));
    L.tf32 = off;
    off = align_up(off + size_t(Mp) * s.kpad() * 4);
    L.sf32 = off;
    off = align_up(off + size_t(Mp) * s.rpad() * 4);
    L.xsw = off;
    off = align_up(off + size_t(Mq) * s.d * 2);
    L.tsw = off;
    off = align_up(off + size_t(2) * Mq * s.kpad() * 2);
    L.ssw = off;
    off = align_up(off + size_t(2) * Mq * s.rpad() * 2);
    L.xsc = off;
    off = align_up(off + size_t(Mq) * 2 * 4);
    L.lfill = off;
    off = align_up(off + size_t(lds_stages(s)) * 16 * 4);
    L.part = off;
    off = align_up(off + size_t(std::max<int64_t>(Mmax, 1)) * max_n_part(s) * 8);
    L.lsep = off;
    off = align_up(off + size_t(std::max<int64_t>(Mmax, 1)) * max_n_part(s) * 8);
    L.tl = off;
    off = align_up(off + size_t(std::max<int64_t>(Mmax, 1)) * 4);
    L.tkp = off;
    off = align_up(off + size_t(tkp_keys(s, Mmax)) * 8);
    L.sync = off;
    off = align_up(off + kSyncWords * 4);
    L.keys = off;
    off = align_up(off + kKeyWords * 8);
    L.colflag = off;
    off = align_up(off + size_t(std::max<int64_t>(s.k + s.r, 1)) * 4);
    const int64_t ptiles = std::max<int64_t>((s.k + s.r + 15) / 16, 1);
    L.ppart = off;
    off = align_up(off + size_t(ptiles) * kProjKS * 2 * 64 * 4 * 4);
    L.pcnt = off;
    off = align_up(off + size_t(ptiles) * 4);
    L.total = off;
    return L;
}

// Grows the workspace in stream order: the new buffer is allocated and zeroed
// on st, and the old one is released on st behind the work already enqueued
// there (which may still be reading it).  Nothing waits for the device.  A
// stream that is being captured into a graph cannot grow it (the allocation
// and the zero fill would become graph nodes that outlive this call's
// bookkeeping): that is an error telling the caller to reserve first.
archead_status grow_workspace(archead_t h, int64_t M, hipStream_t st)
{
    if (M <= h->ws_M && h->ws)
        return ARCHEAD_OK;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    HIP_TRY(hipStreamIsCapturing(st, &cap));
    if (cap != hipStreamCaptureStatusNone)
        return fail(ARCHEAD_EINVAL, "the workspace holds M <= " + std::to_string(h->ws_M) + " and M = " +
                                        std::to_string(M) + " would grow it while the stream is "
                                        "capturing: call archead_reserve before the capture");
    WsLayout L = ws_layout(h->s, M);
    if (archead::alloc_refused(L.total))
        return fail(ARCHEAD_ENOMEM, "workspace of " + std::to_string(L.total) + " bytes refused (ARCHEAD_TEST_ALLOC_LIMIT)");
    void *p = nullptr;
    hipError_t e = hipMallocAsync(&p, L.total, st);
    if (e != hipSuccess)
        return fail(ARCHEAD_ENOMEM, std::string("workspace hipMallocAsync: ") + hipGetErrorString(e));
    e = hipMemsetAsync(p, 0, L.total, st);
    if (e != hipSuccess) {
        (void)hipFreeAsync(p, st);
        return fail(ARCHEAD_EHIP, std::string("workspace zero fill: ") + hipGetErrorString(e));
    }
    if (h->ws)
        HIP_TRY(hipFreeAsync(h->ws, st));
    h->ws = p;
    h->ws_bytes = L.total;
    h->ws_M = M;
    return ARCHEAD_OK;
}

// The per-call view of a workspace at base laid out for up to cap rows.
Work make_work_in(const Shape &s, void *base, int64_t cap, int64_t M)
{
    WsLayout L = ws_layout(s, cap);
    char *b = (char *)base;
    Work w;
    w.M = M;
    w.Mp = round_m(cap);
    w.t16 = (uint16_t *)(b + L.t16);
    w.s16 = (uint16_t *)(b + L.s16);
    w.xsneg = (float *)(b + L.xsneg);
    w.tf32 = (float *)(b + L.tf32);
    w.sf32 = (float *)(b + L.sf32);
    w.xsw = (uint16_t *)(b + L.xsw);
    w.tsw = (uint16_t *)(b + L.tsw);
    w.ssw = (uint16_t *)(b + L.ssw);
    w.xsc = (float *)(b + L.xsc);
    w.lfill = (int32_t *)(b + L.lfill);
    w.Mq = round_m128(std::max<int64_t>(cap, 1));
    w.part = (uint64_t *)(b + L.part);
    w.n_part = 0;
    w.part_cap = std::max<int64_t>(cap, 1) * max_n_part(s);
    w.lsep = (uint64_t *)(b + L.lsep);
    w.tl = (float *)(b + L.tl);
    w.tkp = (uint64_t *)(b + L.tkp);
    w.tkp_cap = tkp_keys(s, cap);
    w.want_lse = 0;
    w.targets = nullptr;
    w.sync = (uint32_t *)(b + L.sync);
    w.keys = (uint64_t *)(b + L.keys);
    w.colflag = (uint32_t *)(b + L.colflag);
    w.ppart = (float *)(b + L.ppart);
    w.pcnt = (uint32_t *)(b + L.pcnt);
    return w;
}

Work make_work(archead_t h, int64_t M) { return make_work_in(h->s, h->ws, h->ws_M, M); }

archead_status validate_shape(int64_t V, int64_t d, int64_t k, int64_t r, int64_t g)
{
    if (V < 1 || V >= (int64_t(1) << 31))
        return fail(ARCHEAD_ESHAPE, "V must satisfy 1 <= V < 2^31");
    if (d < kKChunk || d % kKChunk || d > (int64_t(1) << 20))
        return fail(ARCHEAD_ESHAPE, "d must be a multiple of 128 in [128, 2^20]");
    if (g < kKStep || g % kKStep || d % g)
        return fail(ARCHEAD_ESHAPE, "g must be a multiple of 32 that divides d");
    if (k < 0 || k > 4096 || r < 0 || r > 4096)
        return fail(ARCHEAD_ESHAPE, "k and r must lie in [0, 4096]");
    if ((V + kVB - 1) / kVB * (d / 2) * kVB > (int64_t(1) << 40))
        return fail(ARCHEAD_ESHAPE, "head too large");
    return ARCHEAD_OK;
}

} // namespace

namespace archead {

archead_status api_fail(archead_status s, const std::string &msg) { return fail(s, msg); }

bool alloc_refused(size_t bytes)
{
    const char *v = std::getenv("ARCHEAD_TEST_ALLOC_LIMIT");
    if (!v || !*v)
        return false;
    char *end = nullptr;
    const unsigned long long lim = std::strtoull(v, &end, 10);
    return end != v && bytes > lim;
}

archead_status handle_device(archead_t h, int *device)
{
    g_err.clear();
    if (!live(h))
        return fail(ARCHEAD_EINVAL, "invalid or freed handle");
    *device = h->device;
    return ARCHEAD_OK;
}

size_t workspace_bytes(archead_t h, int64_t M, size_t *zero_head, size_t *zero_tail)
{
    const WsLayout L = ws_layout(h->s, std::max<int64_t>(M, 1));
    *zero_head = L.xsneg; // t16, s16: their padding columns must read as zero
    *zero_tail = L.sync;  // sync, keys, colflag: counters that start at zero
    return L.total;
}

} // namespace archead

extern "C" {

const char *archead_status_string(archead_status s)
{
    switch (s) {
    case ARCHEAD_OK: return "ARCHEAD_OK";
    case ARCHEAD_EINVAL: return "ARCHEAD_EINVAL: invalid argument";
    case ARCHEAD_ESHAPE: return "ARCHEAD_ESHAPE: unsupported shape";
    case ARCHEAD_ERANGE: return "ARCHEAD_ERANGE: field value out of range";
    case ARCHEAD_ENOMEM: return "ARCHEAD_ENOMEM: allocation failed";
    case ARCHEAD_EHIP: return "ARCHEAD_EHIP: HIP runtime error";
    }
    return "ARCHEAD: unknown status";
}

const char *archead_last_error(void) { return g_err.c_str(); }

archead_status archead_pack_load(int64_t V, int64_t d, int64_t k, int64_t r, int64_t g,
                                 const int8_t *A5, const uint16_t *sA, const int8_t *B8,
                                 const uint16_t *sB, const uint8_t *R4, const uint16_t *sR,
                                 const int8_t *C8, const uint16_t *sC, const int8_t *D8,
                                 const uint16_t *sD, void *hip_stream, archead_t *out)
{
    g_err.clear();
    if (!out)
        return fail(ARCHEAD_EINVAL, "out is NULL");
    *out = nullptr;
    archead_status st = validate_shape(V, d, k, r, g);
    if (st != ARCHEAD_OK)
        return st;
    if (!R4 || !sR)
        return fail(ARCHEAD_EINVAL, "R4 and sR are required");
    if (k > 0 && (!A5 || !sA || !B8 || !sB))
        return fail(ARCHEAD_EINVAL, "A5, sA, B8, sB are required when k > 0");
    if (r > 0 && (!C8 || !sC || !D8 || !sD))
        return fail(ARCHEAD_EINVAL, "C8, sC, D8, sD are required when r > 0");
    for (int64_t i = 0; i < V * k; ++i)
        if (A5[i] < -16 || A5[i] > 15)
            return fail(ARCHEAD_ERANGE, "A5 value outside [-16, 15] at flat index " + std::to_string(i));

    Shape s{V, d, k, r, g};
    // device block layout
    size_t off = 0;
    auto place = [&](size_t bytes) {
        size_t o = off;
        off = align_up(off + std::max<size_t>(bytes, 1));
        return o;
    };
    const size_t o_r4 = place(s.n_r4() * 4), o_sr = place(s.n_sr() * 2);
    const size_t o_srp = place(s.n_sr() * 2), o_rsc = place(s.n_rows() * 4);
    const size_t o_lr = place(s.n_lr_words() * 4);
    const size_t o_sa = place(s.n_rows() * 2);
    const size_t o_sc = place(s.n_rows() * 2), o_b8 = place(size_t(k) * d);
    const size_t o_sb = place(size_t(k) * 4), o_d8 = place(size_t(r) * d);
    const size_t o_sd = place(size_t(r) * s.G() * 4);
    const size_t total = off;

    if (archead::alloc_refused(total))
        return fail(ARCHEAD_ENOMEM, "packed head of " + std::to_string(total) + " bytes refused (ARCHEAD_TEST_ALLOC_LIMIT)");
    std::vector<char> host;
    try {
        host.assign(total, 0);
    } catch (...) {
        return fail(ARCHEAD_ENOMEM, "host staging allocation failed");
    }
    char *hb = host.data();
    HostDevImage img{(uint32_t *)(hb + o_r4), (uint16_t *)(hb + o_sr), (uint32_t *)(hb + o_lr),
                     (uint16_t *)(hb + o_srp),
                     (float *)(hb + o_rsc), (uint16_t *)(hb + o_sa),
                     (uint16_t *)(hb + o_sc), (float *)(hb + o_sb), (float *)(hb + o_sd)};
    relayout(s, A5, sA, sB, R4, sR, C8, sC, sD, img,
             (int)std::min(16u, std::max(1u, std::thread::hardware_concurrency())));
    if (k > 0)
        std::memcpy(hb + o_b8, B8, size_t(k) * d);
    if (r > 0)
        std::memcpy(hb + o_d8, D8, size_t(r) * d);

    hipStream_t stream = (hipStream_t)hip_stream;
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    int n_cu = 0;
    HIP_TRY(hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev));
    void *block = nullptr;
    hipError_t e = hipMalloc(&block, total);
    if (e != hipSuccess)
        return fail(ARCHEAD_ENOMEM, std::string("hipMalloc of the packed head: ") + hipGetErrorString(e));
    e = hipMemcpyAsync(block, hb, total, hipMemcpyHostToDevice, stream);
    if (e == hipSuccess)
        e = hipStreamSynchronize(stream);
    if (e != hipSuccess) {
        (void)hipFree(block);
        return fail(ARCHEAD_EHIP, std::string("upload of the packed head: ") + hipGetErrorString(e));
    }

    archead_head *h = new (std::nothrow) archead_head();
    if (!h) {
        (void)hipFree(block);
        return fail(ARCHEAD_ENOMEM, "handle allocation failed");
    }
    char *db = (char *)block;
    h->magic = kMagic;
    h->s = s;
    h->dev.s = s;
    h->dev.r4 = (const uint32_t *)(db + o_r4);
    h->dev.sr = (const uint16_t *)(db + o_sr);
    h->dev.lr = (const uint32_t *)(db + o_lr);
    h->dev.n_cu = n_cu > 0 ? n_cu : 1;
    h->dev.srp = (const uint16_t *)(db + o_srp);
    h->dev.rsc = (const float *)(db + o_rsc);
    h->dev.sa = (const uint16_t *)(db + o_sa);
    h->dev.sc = (const uint16_t *)(db + o_sc);
    h->dev.b8 = (const int8_t *)(db + o_b8);
    h->dev.sb = (const float *)(db + o_sb);
    h->dev.d8 = (const int8_t *)(db + o_d8);
    h->dev.sd = (const float *)(db + o_sd);
    h->block = block;
    h->block_bytes = total;
    h->ws = nullptr;
    h->ws_bytes = 0;
    h->ws_M = 0;
    h->device = dev;
    st = grow_workspace(h, 1, stream);
    if (st == ARCHEAD_OK && hipStreamSynchronize(stream) != hipSuccess)
        st = fail(ARCHEAD_EHIP, "workspace set-up did not complete");
    if (st != ARCHEAD_OK) {
        (void)hipFree(block);
        delete h;
        return st;
    }
    {
        std::lock_guard<std::mutex> gl(g_live_mu);
        g_live.insert(h);
    }
    *out = h;
    return ARCHEAD_OK;
}

archead_status archead_reserve(archead_t h, int64_t M_max, void *hip_stream)
{
    g_err.clear();
    if (!live(h))
        return fail(ARCHEAD_EINVAL, "invalid or freed handle");
    if (M_max < 0)
        return fail(ARCHEAD_EINVAL, "M_max < 0");
    if (M_max > kMaxM)
        return fail(ARCHEAD_ESHAPE, "M_max above 2^20");
    HIP_TRY(hipSetDevice(h->device));
    archead_status st = grow_workspace(h, std::max<int64_t>(M_max, 1), (hipStream_t)hip_stream);
    if (st != ARCHEAD_OK)
        return st;
    // a reservation is made ahead of the hot path: wait for it, so that the
    // workspace is ready for calls on any stream
    HIP_TRY(hipStreamSynchronize((hipStream_t)hip_stream));
    return ARCHEAD_OK;
}

// ws_ext: a caller-provided workspace laid out for ws_cap rows (nothing is
// allocated then); otherwise the handle's own, grown as needed.
static archead_status forward_impl(archead_t h, int64_t M, const void *X, float *logits,
                                   int32_t *argmax, int path, void *hip_stream, hipEvent_t ev0,
                                   hipEvent_t ev1, const int32_t *targets = nullptr,
                                   float *lse = nullptr, float *nll = nullptr, void *ws_ext = nullptr,
                                   int64_t ws_cap = 0, const DecodeTopk *tk = nullptr, bool *tk_done = nullptr)
{
    if (tk_done)
        *tk_done = false;
    g_err.clear();
    if (!live(h))
        return fail(ARCHEAD_EINVAL, "invalid or freed handle");
    if (M < 0)
        return fail(ARCHEAD_EINVAL, "M < 0");
    if (M > kMaxM)
        return fail(ARCHEAD_ESHAPE, "M above 2^20");
    if (path < ARCHEAD_PATH_AUTO || path > ARCHEAD_PATH_LDS)
        return fail(ARCHEAD_EINVAL, "unknown path");
    if (M == 0)
        return ARCHEAD_OK;
    if (!logits && !argmax && !lse)
        return fail(ARCHEAD_EINVAL, "logits, argmax and lse are all NULL");
    if ((targets != nullptr) != (nll != nullptr))
        return fail(ARCHEAD_EINVAL, "targets and nll must be given together");
    if (nll && !lse)
        return fail(ARCHEAD_EINVAL, "nll needs lse");
    if (!X)
        return fail(ARCHEAD_EINVAL, "X is NULL");
    if (((uintptr_t)X) % 16)
        return fail(ARCHEAD_EINVAL, "X must be 16-byte aligned");
    hipStream_t st = (hipStream_t)hip_stream;
    HIP_TRY(hipSetDevice(h->device));
    if (!ws_ext) {
        archead_status s = grow_workspace(h, M, st);
        if (s != ARCHEAD_OK)
            return s;
    } else if (ws_cap < M) {
        return fail(ARCHEAD_EINVAL, "workspace too small");
    }

    int chosen = path;
    if (chosen == ARCHEAD_PATH_AUTO) {
        chosen = M >= kLdsMinM ? ARCHEAD_PATH_LDS : ARCHEAD_PATH_SKINNY;
        // one hidden state on a head the matrix-core single launch does not
        // take (g != 128): the VALU single launch outruns the streaming kernel
        if (M == 1 && !decode_ok(h->dev, 1, true) && decode_ok(h->dev, 1, false))
            chosen = ARCHEAD_PATH_GEMV;
    }
    if (chosen == ARCHEAD_PATH_GEMV && !decode_ok(h->dev, M, false))
        return fail(ARCHEAD_ESHAPE, "the GEMV path takes M <= " + std::to_string(kDecodeMaxM) +
                                        ", d a multiple of 512 and a head whose staging fits in LDS");
    // the skinny path runs as one launch where the shape allows
    const bool one_launch = chosen == ARCHEAD_PATH_GEMV ||
                            (chosen == ARCHEAD_PATH_SKINNY && decode_ok(h->dev, M, true));

    Work w = ws_ext ? make_work_in(h->s, ws_ext, ws_cap, M) : make_work(h, M);
    w.want_lse = lse ? 1 : 0;
    w.targets = targets;
    const uint16_t *Xb = (const uint16_t *)X;
    if (one_launch) { // projection, tiles and argmax (and the top-k selection where it fits)
        const bool fused_tk = tk && decode_topk_ok(h->dev, M, chosen == ARCHEAD_PATH_SKINNY);
        if (ev0)
            HIP_TRY(hipEventRecord(ev0, st));
        HIP_TRY(launch_decode(h->dev, w, Xb, logits, argmax, lse, nll, chosen == ARCHEAD_PATH_SKINNY, st,
                              fused_tk ? tk : nullptr));
        if (tk_done)
            *tk_done = fused_tk;
        if (ev1)
            HIP_TRY(hipEventRecord(ev1, st));
        return ARCHEAD_OK;
    }
    if (chosen == ARCHEAD_PATH_LDS) {
        HIP_TRY(launch_proj_mfma(h->dev, w, Xb, st));
        HIP_TRY(launch_prep_lds(h->dev, w, Xb, st));
    } else {
        HIP_TRY(launch_proj(h->dev, w, Xb, st));
    }
    // batched decode on the persistent slab-staged kernel where it applies
    const bool s2 = chosen == ARCHEAD_PATH_SKINNY && stream2_ok(h->dev, M);
    if (ev0)
        HIP_TRY(hipEventRecord(ev0, st));
    if (chosen == ARCHEAD_PATH_LDS)
        HIP_TRY(launch_vtile_lds(h->dev, w, logits, argmax, st));
    else if (s2)
        HIP_TRY(launch_vtile_stream2(h->dev, w, Xb, logits, argmax, st));
    else
        HIP_TRY(launch_vtile_skinny(h->dev, w, Xb, logits, argmax, st));
    if (ev1)
        HIP_TRY(hipEventRecord(ev1, st));
    if (argmax || lse) {
        const int64_t n_part = chosen == ARCHEAD_PATH_LDS ? lds_n_part(h->dev, M)
                               : s2                       ? stream2_n_part(h->dev, M)
                                                          : skinny_n_part(h->dev, M);
        HIP_TRY(launch_finish(w, n_part, h->s.V, argmax, lse, nll, st));
    }
    return ARCHEAD_OK;
}

archead_status archead_forward_path(archead_t h, int64_t M, const void *X, float *logits,
                                    int32_t *argmax, int path, void *hip_stream)
{
    return forward_impl(h, M, X, logits, argmax, path, hip_stream, nullptr, nullptr);
}

archead_status archead_forward_timed(archead_t h, int64_t M, const void *X, float *logits,
                                     int32_t *argmax, int path, void *hip_stream,
                                     void *ev_before, void *ev_after)
{
    if (!ev_before || !ev_after) {
        g_err = "ev_before and ev_after are required";
        return ARCHEAD_EINVAL;
    }
    return forward_impl(h, M, X, logits, argmax, path, hip_stream, (hipEvent_t)ev_before,
                        (hipEvent_t)ev_after);
}

archead_status archead_forward(archead_t h, int64_t M, const void *X, float *logits,
                               void *hip_stream)
{
    if (!logits) {
        g_err = "logits is NULL";
        return ARCHEAD_EINVAL;
    }
    return archead_forward_path(h, M, X, logits, nullptr, ARCHEAD_PATH_AUTO, hip_stream);
}

archead_status archead_forward_argmax(archead_t h, int64_t M, const void *X, float *logits,
                                      int32_t *argmax, void *hip_stream)
{
    if (!argmax) {
        g_err = "argmax is NULL";
        return ARCHEAD_EINVAL;
    }
    return archead_forward_path(h, M, X, logits, argmax, ARCHEAD_PATH_AUTO, hip_stream);
}

archead_status archead_forward_ce_path(archead_t h, int64_t M, const void *X, const int32_t *targets,
                                      float *logits, int32_t *argmax, float *lse, float *nll, int path,
                                      void *hip_stream)
{
    if (!lse) {
        g_err = "lse is NULL";
        return ARCHEAD_EINVAL;
    }
    return forward_impl(h, M, X, logits, argmax, path, hip_stream, nullptr, nullptr, targets, lse, nll);
}

// the forward plus the K largest logits per hidden state (and, with u, one
// draw from them): inside the single launch where it runs, otherwise the
// slice and merge kernels over the written logits (and the draw kernel)
static archead_status topk_impl(archead_t h, int64_t M, const void *X, int32_t K, float *logits, float *values,
                                int32_t *indices, int path, void *hip_stream, const float *u, float temperature,
                                int32_t *samples)
{
    // the same scale the separate draw kernel takes (launch_topk_sample)
    const float scale = u ? 1.44269504088896340736f / temperature : 0.f;
    DecodeTopk tk{K, values, indices, u, scale, samples};
    bool done = false;
    archead_status st = forward_impl(h, M, X, logits, nullptr, path, hip_stream, nullptr, nullptr, nullptr, nullptr,
                                     nullptr, nullptr, 0, &tk, &done);
    if (st != ARCHEAD_OK || M == 0 || done)
        return st;
    Work w = make_work(h, M);
    HIP_TRY(launch_topk(w, logits, h->s.V, K, values, indices, (hipStream_t)hip_stream));
    if (u)
        HIP_TRY(launch_topk_sample(values, indices, M, K, temperature, u, samples, (hipStream_t)hip_stream));
    return ARCHEAD_OK;
}

archead_status archead_forward_topk_path(archead_t h, int64_t M, const void *X, int32_t K, float *logits,
                                        float *values, int32_t *indices, int path, void *hip_stream)
{
    g_err.clear();
    if (!logits || !values || !indices)
        return fail(ARCHEAD_EINVAL, "logits, values and indices are required");
    if (!live(h))
        return fail(ARCHEAD_EINVAL, "invalid or freed handle");
    if (K < 1 || K > kTopKMax || int64_t(K) > h->s.V)
        return fail(ARCHEAD_EINVAL, "K must satisfy 1 <= K <= min(" + std::to_string(kTopKMax) + ", V)");
    return topk_impl(h, M, X, K, logits, values, indices, path, hip_stream, nullptr, 0.f, nullptr);
}

archead_status archead_forward_sample(archead_t h, int64_t M, const void *X, int32_t K, float temperature,
                                      const float *u, float *logits, float *values, int32_t *indices,
                                      int32_t *samples, void *hip_stream)
{
    g_err.clear();
    // the weights are 2^((v_j - v_0) log2(e) / tau): the factor log2(e) / tau
    // must be finite too, which rules out subnormal temperatures
    if (!(temperature > 0.f) || !std::isfinite(temperature) ||
        !std::isfinite(1.4426950408889634f / temperature))
        return fail(ARCHEAD_EINVAL, "temperature must be positive and finite, with log2(e) / temperature finite");
    if (!u || !samples)
        return fail(ARCHEAD_EINVAL, "u and samples are required");
    if (!logits || !values || !indices)
        return fail(ARCHEAD_EINVAL, "logits, values and indices are required");
    if (!live(h))
        return fail(ARCHEAD_EINVAL, "invalid or freed handle");
    if (K < 1 || K > kTopKMax || int64_t(K) > h->s.V)
        return fail(ARCHEAD_EINVAL, "K must satisfy 1 <= K <= min(" + std::to_string(kTopKMax) + ", V)");
    return topk_impl(h, M, X, K, logits, values, indices, ARCHEAD_PATH_AUTO, hip_stream, u, temperature, samples);
}

archead_status archead_forward_topk(archead_t h, int64_t M, const void *X, int32_t K, float *logits,
                                    float *values, int32_t *indices, void *hip_stream)
{
    return archead_forward_topk_path(h, M, X, K, logits, values, indices, ARCHEAD_PATH_AUTO, hip_stream);
}

archead_status archead_forward_ce(archead_t h, int64_t M, const void *X, const int32_t *targets,
                                  float *logits, int32_t *argmax, float *lse, float *nll, void *hip_stream)
{
    return archead_forward_ce_path(h, M, X, targets, logits, argmax, lse, nll, ARCHEAD_PATH_AUTO, hip_stream);
}

archead_status archead_packed_bytes(archead_t h, uint64_t *bytes)
{
    g_err.clear();
    if (!live(h) || !bytes)
        return fail(ARCHEAD_EINVAL, "invalid handle or NULL output");
    const Shape &s = h->s;
    auto B = [](uint64_t numel, uint64_t bits) { return (numel * bits + 7) / 8; };
    const uint64_t G = s.G();
    // a head without a core (k = 0) or without a correction (r = 0) holds no
    // row scales for it
    *bytes = B(s.V * s.d, 4) + B(s.V * G, 16) + B(s.V * s.k, 5) + B(s.k > 0 ? s.V : 0, 16) +
             B(s.k * s.d, 8) + B(s.k, 16) + B(s.V * s.r, 8) + B(s.r > 0 ? s.V : 0, 16) +
             B(s.r * s.d, 8) + B(s.r * G, 16);
    return ARCHEAD_OK;
}

archead_status archead_device_bytes(archead_t h, uint64_t *bytes)
{
    g_err.clear();
    if (!live(h) || !bytes)
        return fail(ARCHEAD_EINVAL, "invalid handle or NULL output");
    *bytes = h->block_bytes + h->ws_bytes;
    return ARCHEAD_OK;
}

archead_status archead_free(archead_t h)
{
    g_err.clear();
    if (!h)
        return ARCHEAD_OK;
    {
        std::lock_guard<std::mutex> gl(g_live_mu);
        if (!g_live.count(h))
            return fail(ARCHEAD_EINVAL, "invalid or already freed handle");
        g_live.erase(h);
    }
    (void)hipSetDevice(h->device);
    hipError_t e = hipDeviceSynchronize();
    if (h->ws)
        (void)hipFree(h->ws);
    if (h->block)
        (void)hipFree(h->block);
    h->magic = 0;
    delete h;
    if (e != hipSuccess)
        return fail(ARCHEAD_EHIP, std::string("hipDeviceSynchronize: ") + hipGetErrorString(e));
    return ARCHEAD_OK;
}

} // extern "C"

namespace archead {

archead_status forward_in_workspace(archead_t h, int64_t M, const void *X, float *logits, int32_t *argmax,
                                    void *hip_stream, void *ws, int64_t ws_cap)
{
    return forward_impl(h, M, X, logits, argmax, ARCHEAD_PATH_AUTO, hip_stream, nullptr, nullptr, nullptr,
                        nullptr, nullptr, ws, ws_cap);
}

} // namespace archead
