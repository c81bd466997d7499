// decode.hip -- the whole packed ARCHead forward for M <= 2 in one launch,
// with VALU dot products (bf16 pairs into fp32) or, at M = 1, matrix-core
// products.
//
// ARCHead paper, section 3.2, eq 7 with W_d from eq 3 and the INT8 factors
// of the text after eq 7:
//   t = X (sB o B8)^T,  s = X (sD o D8)^T                          (a1)
//   logits[m,v] = sum_grp sR[v,grp] sum_{j in grp} X[m,j] R4[v,j]
//               + sA[v] sum_i A5[v,i] t[m,i] + sC[v] sum_i C8[v,i] s[m,i]   (a2)
//   argmax[m] = lowest index of the row maximum                     (a3)
//
// One workgroup = 4 waves x NV v-blocks of 16 vocabulary rows.  A wave
// streams, for its v-blocks, every SC4 residual chunk and then every
// low-rank chunk (the chunk stream of layout.hpp), two chunks per prefetch
// buffer and two buffers in flight.  Lane l works on row l % 16 of each
// v-block and on the 8 columns 8(l/16) .. +7 of each K-step, exactly the
// lanes' share of the packed chunk: its codes become bf16 integer pairs by
// exponent splicing and enter v_dot2_f32_bf16 against pairs of X (residual)
// or of the bf16 hi/lo parts of t and s (low-rank).  The four lanes that
// share a row meet by two shuffles at the end.
//
// a1 runs inside the same launch: wave w of the grid computes columns w,
// w + nw, ... of t and s (nw waves) and publishes them through device-scope
// stores followed by an increment of a counter.  The residual needs none of
// it; three quarters through its residual a wave reads the count once, and if
// every column is published it copies t and s to LDS, and otherwise computes
// them itself.  No wave ever waits for another wave.
//
// a3 runs inside it too: each workgroup folds its top-1 keys into 64-bit
// atomic maxima, and the last workgroup to finish turns the keys into
// indices and zeroes the keys and the counters for the next call.  Counters
// and keys that many workgroups update are split over 16 addresses
// (layout.hpp), since atomics on one address serialise.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace archead {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// c + the dot product of 8 bf16 pairs held as two u32x4
__device__ __forceinline__ float dot8(u32x4 a, u32x4 b, float c)
{
    c = dot2(a.x, b.x, c);
    c = dot2(a.y, b.y, c);
    c = dot2(a.z, b.z, c);
    return dot2(a.w, b.w, c);
}

__device__ __forceinline__ float dot8c(u32x4 a, uint32_t k, float c)
{
    c = dot2(a.x, k, c);
    c = dot2(a.y, k, c);
    c = dot2(a.z, k, c);
    return dot2(a.w, k, c);
}

// Cross-workgroup hand-offs use device-scope (sc1) stores and loads, which
// are coherent across the XCDs' L2 caches, plus a wait for completion;
// agent-scope release fences would write back whole L2 caches instead.
__device__ __forceinline__ void store_device(uint16_t *p, uint16_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Keeps one K-step's loads and arithmetic together: no memory access moves
// across it in the optimiser (empty asm with a memory clobber) or in the
// machine scheduler.
__device__ __forceinline__ void step_fence()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Marks an accumulator as read and written here (no instruction): the
// arithmetic that feeds it cannot be sunk past this point, which would keep
// the operands of several K-steps live at once.
__device__ __forceinline__ void pin(float &x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin4(f32x4 &x) { asm volatile("" : "+v"(x)); }

constexpr uint32_t kBf16One = 0x3F803F80u; // bf16 pair (1, 1)

struct DecodeArgs {
    DevHead h;
    Work w;
    const uint16_t *X;
    float *logits;   // M x V, may be null
    int32_t *argmax; // M, may be null
    float *lse, *nll; // M each, may be null (lse with a.w.want_lse; nll with targets)
    int64_t nvb, nkc, G, na, nlr;
    int gsteps;
    int ntask;       // k + r projection columns
    int ntwg;        // projection-only workgroups, first in the grid (0: the
                     // streaming waves compute the columns themselves)
    int nwg;         // streaming workgroups, after them
    unsigned lds_sa, lds_x, lds_ts, lds_xs; // byte offsets of the sA/sC, X, t/s and group-sum regions (sr at 0)
    // top-k selection in the same launch (tk_K > 0): each streaming wave
    // writes the largest argmax key of its rows to tkw[m][wave] (and the
    // logits); the last workgroup selects the K largest logits of each
    // hidden state into tk_vals / tk_idx [MF][K] and, with tk_u, draws one of
    // them per hidden state at the temperature whose log2(e) / tau is
    // tk_scale into tk_samples
    int tk_K, tk_L;  // K, and wave keys per thread of the final selection (<= kTkKeys)
    uint64_t *tkw;
    float *tk_vals;
    int32_t *tk_idx;
    const float *tk_u;
    float tk_scale;
    int32_t *tk_samples;
    unsigned lds_tk; // byte offset of the selection's LDS region
};

// The final selection reads every wave's key, kTkKeys per thread of the
// last workgroup (all loads in flight at once), so it covers up to
// 64 kTkKeys workgroups.
constexpr int kTkKeys = 12;
// selection LDS: [0, 256) selected keys, per-wave bounds, counters; [256,
// 512) partial-rank counters; then the
// threads' maxima [256]; then the wave keys at or above the bound, at most
// 4 K Q (Q = wave keys per thread; at most K threads of a wave hold a
// maximum at or above that wave's bound), and the candidate rows, at most
// K NV 16, each with kTkSpare slots past its capacity (read, never used, by
// the ranking's eight-key steps)
constexpr unsigned kTkSpare = 8;
constexpr unsigned kTkMiscBytes = 512;

// log-sum-exp summaries each lane of the last workgroup loads at once, and
// the bits of the empty summary (-inf, 0)
constexpr int kLseBatch = 16;
constexpr uint64_t kLseEmpty = 0xFF800000u;

// v-blocks per wave: five at M = 1, four at M = 2 (whose accumulators need
// the registers), with two prefetch pairs at two waves per SIMD
constexpr int decode_nv(int MF) { return MF == 1 ? 5 : 4; }

template <int NV>
struct DChunk {
    u32x4 q[NV];
};

template <int NV>
struct DPair {
    DChunk<NV> h0, h1;
};

// LDS of one workgroup:
//   sr  [4*NV][G][16]        fp16  residual scales of its v-blocks
//   sa  [2][4*NV][16]        fp16  sA, then sC, of its rows
//   x   [MF][d]              bf16  the hidden states
//   ts  [4 waves] x { t hi [MF][kpad], t lo [MF][kpad], s hi [MF][rpad], s lo [MF][rpad] }  bf16
//   xs  [4 waves][MF][G]     fp32  -136 (sum of X over group grp), a
//                                  quarter of it in the VALU variant
//
// A wave's chunk stream: the first three quarters of the residual K-chunks,
// then the low-rank chunks, then the remaining residual K-chunks.  Placing the low-rank chunks
// in the middle lets the projection finish long before they are needed and
// keeps the waves from all reaching the low-rank work at once at the end.
template <int MF, int GS, bool MX>
__global__ __launch_bounds__(256, 2) void gemv_decode_kernel(DecodeArgs a)
{
    static_assert(!MX || GS == 4, "the matrix-core variant folds one g = 128 group per chunk");
    constexpr int NV = decode_nv(MF);
    extern __shared__ __attribute__((aligned(16))) char smem[];
    __shared__ uint64_t red[4][MF];
    __shared__ LsePart lred[4][MF];
    __shared__ int s_last; // this workgroup is the last one counted (top-k selection)
    const uint16_t *s_sr = (const uint16_t *)smem;
    const uint16_t *s_x = (const uint16_t *)(smem + a.lds_x);

    const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nvb = a.nvb, nkc = a.nkc, G = a.G, na = a.na, nlr = a.nlr;
    const int64_t d = a.h.s.d, V = a.h.s.V, k = a.h.s.k;
    const int64_t kst = a.h.s.kst(), rst = a.h.s.rst(), kpad = a.h.s.kpad(), rpad = a.h.s.rpad();
    const int gsteps = GS ? GS : a.gsteps;
    const int ntask = a.ntask;
    const bool proj_wg = (int)blockIdx.x < a.ntwg;
    __builtin_amdgcn_s_setprio(3); // lowered by the streaming waves as they go (pace below)
    const int64_t bid = (int64_t)blockIdx.x - a.ntwg; // streaming workgroup index
    const int64_t wg_vb0 = (proj_wg ? 0 : bid) * 4 * NV;
    const int64_t vb0 = wg_vb0 + wv * NV;
    uint16_t *s_ts = (uint16_t *)(smem + a.lds_ts) + wv * (2 * MF * (kpad + rpad));
    uint32_t *const sync = a.w.sync;
    // the call's tag: column flags equal to it were written by this call
    const uint32_t epoch = __hip_atomic_load(sync + sync_epoch(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    int64_t vb[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v)
        vb[v] = vb0 + v < nvb ? vb0 + v : nvb - 1;
    // cross-entropy targets (uniform: scalar loads, complete long before use)
    int32_t tgt[MF];
#pragma unroll
    for (int m = 0; m < MF; ++m)
        tgt[m] = (a.w.want_lse && a.w.targets) ? a.w.targets[m] : -1;

    // ---- a1: column i of t (i < k) or s (i >= k) for every row m, as a
    // bf16 hi/lo pair in lane m ----
    auto column = [&](int i, uint16_t (&hi)[MF], uint16_t (&lo)[MF]) __attribute__((always_inline)) {
        const bool isd = i >= k;
        const int64_t c = isd ? i - k : i;
        const int8_t *row = isd ? a.h.d8 + c * d : a.h.b8 + c * d;
        float acc[MF];
#pragma unroll
        for (int m = 0; m < MF; ++m)
            acc[m] = 0.f;
        const u32x4 z = {0u, 0u, 0u, 0u};
        for (int64_t j00 = 0; j00 < d; j00 += 4096) {
            u32x4 wq[4];
            float sc[4];
            // every load of the pass is issued before the first multiply
            // (addresses clamped in range, results selected afterwards)
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int64_t j0 = j00 + 1024 * it + 16 * lane;
                const int64_t jc = j0 < d ? j0 : 0;
                wq[it] = *(const u32x4 *)(row + jc);
                sc[it] = isd ? a.h.sd[c * G + jc / a.h.s.g] : 1.0f;
            }
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const bool ok = j00 + 1024 * it + 16 * lane < d;
                wq[it] = ok ? wq[it] : z;
            }
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int64_t j0 = j00 + 1024 * it + 16 * lane;
                const bool ok = j0 < d;
#pragma unroll
                for (int m = 0; m < MF; ++m) {
                    const u32x4 *xp = (const u32x4 *)(s_x + m * d + (ok ? j0 : 0));
                    const u32x4 x0 = ok ? xp[0] : z, x1 = ok ? xp[1] : z;
                    acc[m] = __builtin_fmaf(sc[it], dot16(wq[it], x0, x1), acc[m]);
                }
            }
        }
#pragma unroll
        for (int m = 0; m < MF; ++m) {
            for (int off = 32; off >= 1; off >>= 1)
                acc[m] += __shfl_xor(acc[m], off);
            const float t = isd ? acc[m] : acc[m] * a.h.sb[c];
            hi[m] = f32_to_bf16_rne(t);
            lo[m] = f32_to_bf16_rne(t - __uint_as_float((uint32_t)hi[m] << 16));
        }
    };
    // publish column i to the workspace: device-scope stores, completed
    // before the column's flag is set to the call's tag (no cache write-back
    // needed: they went to the device's coherence point)
    auto publish = [&](int i) __attribute__((always_inline)) {
        uint16_t hi[MF], lo[MF];
        column(i, hi, lo);
        const bool isd = i >= k;
        const int64_t c = isd ? i - k : i;
        const int64_t Mp = a.w.Mp;
#pragma unroll
        for (int m = 0; m < MF; ++m)
            if (lane == m) {
                store_device(isd ? a.w.s16 + m * rpad + c : a.w.t16 + m * kpad + c, hi[m]);
                store_device(isd ? a.w.s16 + (Mp + m) * rpad + c : a.w.t16 + (Mp + m) * kpad + c, lo[m]);
            }
        wait_vm_all();
        if (lane == 0) {
            __hip_atomic_store(a.w.colflag + i, __builtin_amdgcn_readfirstlane(epoch) + 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_add(sync + sync_published(), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    };

    // wave-level copy of n16 16-byte pieces from the workspace to LDS, read
    // at device scope (the data were written by other workgroups of this
    // launch)
    auto wave_dma16 = [&](const void *src, void *dst, int64_t n16) __attribute__((always_inline)) {
        for (int64_t i0 = 0; i0 < n16; i0 += 64) {
            const int64_t i = i0 + lane;
            if (i < n16)
                lds_dma16<true>((const u32x4 *)src + i, (u32x4 *)dst + i0);
        }
    };
    // t and s of the MF rows into this wave's LDS region, copied from the
    // workspace once every column is published (nothing in this kernel ever
    // waits for another wave)
    auto stage_ts = [&]() __attribute__((always_inline)) {
        const int64_t Mp = a.w.Mp;
        wave_dma16(a.w.t16, s_ts, MF * kpad / 8);
        wave_dma16(a.w.t16 + Mp * kpad, s_ts + MF * kpad, MF * kpad / 8);
        wave_dma16(a.w.s16, s_ts + 2 * MF * kpad, MF * rpad / 8);
        wave_dma16(a.w.s16 + Mp * rpad, s_ts + 2 * MF * kpad + MF * rpad, MF * rpad / 8);
    };
    // Fallback when the count fell short: build t and s in LDS column by
    // column.  A column whose flag carries this call's tag is read from the
    // workspace after the flag (its values were complete before the flag
    // was set); every other column the wave computes itself.
    auto build_ts = [&]() __attribute__((always_inline)) {
        uint32_t *r = (uint32_t *)s_ts; // padding columns must read as 0
        const int64_t nw32 = MF * (kpad + rpad); // 2 * MF * (kpad + rpad) bf16
        for (int64_t i = lane; i < nw32; i += 64)
            r[i] = 0u;
        const uint32_t tag = __builtin_amdgcn_readfirstlane(epoch) + 1u;
        const int64_t Mp = a.w.Mp;
        for (int q = 0; q * 64 < ntask; ++q) {
            const int i = q * 64 + lane;
            const bool valid = i < ntask;
            const uint32_t f =
                __hip_atomic_load(a.w.colflag + (valid ? i : ntask - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const bool pub = valid && f == tag;
            if (pub) {
                const bool isd = i >= k;
                const int64_t c = isd ? i - k : i;
#pragma unroll
                for (int m = 0; m < MF; ++m) {
                    const uint16_t hi = __hip_atomic_load(isd ? a.w.s16 + m * rpad + c : a.w.t16 + m * kpad + c,
                                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    const uint16_t lo =
                        __hip_atomic_load(isd ? a.w.s16 + (Mp + m) * rpad + c : a.w.t16 + (Mp + m) * kpad + c,
                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (isd) {
                        s_ts[2 * MF * kpad + m * rpad + c] = hi;
                        s_ts[2 * MF * kpad + (MF + m) * rpad + c] = lo;
                    } else {
                        s_ts[m * kpad + c] = hi;
                        s_ts[(MF + m) * kpad + c] = lo;
                    }
                }
            }
            uint64_t miss = __ballot(valid && !pub);
            while (miss) {
                const int j = q * 64 + __builtin_ctzll(miss);
                miss &= miss - 1;
                uint16_t hi[MF], lo[MF];
                column(j, hi, lo);
                const bool isd = j >= k;
                const int64_t c = isd ? j - k : j;
#pragma unroll
                for (int m = 0; m < MF; ++m)
                    if (lane == m) {
                        if (isd) {
                            s_ts[2 * MF * kpad + m * rpad + c] = hi[m];
                            s_ts[2 * MF * kpad + (MF + m) * rpad + c] = lo[m];
                        } else {
                            s_ts[m * kpad + c] = hi[m];
                            s_ts[(MF + m) * kpad + c] = lo[m];
                        }
                    }
            }
        }
    };

    // ---- the chunk stream, in pairs of chunks ----
    const int64_t nrp = nkc / 2, nlp = nlr / 2;                  // both even
    // residual pairs before the low-rank ones (even; with no low-rank
    // chunks, all but the last two)
    const int64_t nrp1 = nlr > 0 ? ((3 * nrp / 4) & ~int64_t(1)) : nrp - 2;
    const int64_t c1 = 2 * nrp1, c2 = c1 + nlr, npairs = nrp + nlp;
    const u32x4 *lrp = (const u32x4 *)a.h.lr;
    const u32x4 *r4p = (const u32x4 *)a.h.r4;
    auto load_chunk = [&](DChunk<NV> &c, int64_t ci) __attribute__((always_inline)) {
        const u32x4 *base = ci < c1   ? r4p + ci * nvb * 64
                            : ci < c2 ? lrp + (ci - c1) * nvb * 64
                                      : r4p + (ci - nlr) * nvb * 64;
#pragma unroll
        for (int v = 0; v < NV; ++v)
            c.q[v] = __builtin_nontemporal_load(&base[vb[v] * 64 + lane]);
    };
    auto load_pair = [&](DPair<NV> &p, int64_t pi) __attribute__((always_inline)) { // pi < npairs
        load_chunk(p.h0, 2 * pi);
        load_chunk(p.h1, 2 * pi + 1);
    };

    // Completion count, run by wave 0 of every workgroup once the workgroup
    // is done: projection-only workgroups are counted too (with no keys or
    // summaries of their own), so the last workgroup counted -- which
    // resolves the argmax and the log-normaliser and bumps the call counter
    // -- comes after every workgroup of the grid, and the bump after every
    // workgroup's read of the counter at its start.
    // (wave 0) count this workgroup; true for the last workgroup of the grid
    auto count_wg = [&](bool with_keys) __attribute__((always_inline)) -> bool {
        const int nall = a.ntwg + a.nwg;
        const int nslot = nall < kSyncGroups ? nall : kSyncGroups;
        const int slot = (int)(blockIdx.x % nslot);
        const uint32_t slot_size = (uint32_t)((nall - 1 - slot) / nslot + 1);
        if (with_keys && a.argmax && lane < MF) {
            const uint64_t kk = umax64(umax64(red[0][lane], red[1][lane]), umax64(red[2][lane], red[3][lane]));
            __hip_atomic_fetch_max(a.w.keys + slot * 32 + lane, kk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (with_keys && a.w.want_lse && lane < MF) {
            const LsePart p = lse_merge(lse_merge(lred[0][lane], lred[1][lane]), lse_merge(lred[2][lane], lred[3][lane]));
            __hip_atomic_store(a.w.lsep + (int64_t)lane * a.nwg + bid, lse_bits(p), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
        wait_vm_all();
        uint32_t prev = 0;
        if (lane == 0)
            prev = __hip_atomic_fetch_add(sync + sync_slot_done(slot), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((uint32_t)__builtin_amdgcn_readfirstlane(prev) == slot_size - 1) {
            uint32_t prev2 = 0;
            if (lane == 0) {
                __hip_atomic_store(sync + sync_slot_done(slot), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                prev2 = __hip_atomic_fetch_add(sync + sync_top_done(), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            return (uint32_t)__builtin_amdgcn_readfirstlane(prev2) == (uint32_t)(nslot - 1);
        }
        return false;
    };
    // (wave 0 of the last workgroup) the argmax and the log-normaliser from
    // every workgroup's keys and summaries; counters back to zero for the
    // next call, which the call counter then tags
    auto resolve_final = [&]() __attribute__((always_inline)) {
        const int nall = a.ntwg + a.nwg;
        const int nslot = nall < kSyncGroups ? nall : kSyncGroups;
        {
            {
                if (a.argmax) {
                    // lane s * MF + m takes (and clears) key m of slot s
                    const int s = lane / MF, m = lane % MF;
                    uint64_t kk = 0;
                    if (s < nslot)
                        kk = __hip_atomic_exchange(a.w.keys + s * 32 + m, (uint64_t)0, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
    #pragma unroll
                    for (int off = MF; off < kSyncGroups * MF; off <<= 1)
                        kk = umax64(kk, shfl_xor_u64(kk, off));
                    if (lane < MF)
                        a.argmax[lane] = (int32_t)(0xFFFFFFFFu - (uint32_t)kk);
                }
                if (a.w.want_lse) {
                    // every workgroup's summary is final once every slot is counted
    #pragma unroll
                    for (int m = 0; m < MF; ++m) {
                        // the first 64 kLseBatch summaries with all their loads in
                        // flight at once (one round trip), any further ones after
                        const uint64_t *src = a.w.lsep + (int64_t)m * a.nwg;
                        uint64_t bits[kLseBatch];
    #pragma unroll
                        for (int j = 0; j < kLseBatch; ++j) {
                            const int i = lane + 64 * j;
                            bits[j] = i < a.nwg ? __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                                : kLseEmpty;
                        }
                        LsePart p{-__builtin_inff(), 0.f};
    #pragma unroll
                        for (int j = 0; j < kLseBatch; ++j)
                            p = lse_merge(p, lse_unbits(bits[j]));
                        for (int i = lane + 64 * kLseBatch; i < a.nwg; i += 64)
                            p = lse_merge(p, lse_unbits(__hip_atomic_load(src + i, __ATOMIC_RELAXED,
                                                                          __HIP_MEMORY_SCOPE_AGENT)));
                        p = lse_merge64(p);
                        if (lane == 0) {
                            const float L = p.mx + logf(p.s);
                            a.lse[m] = L;
                            if (a.nll) {
                                const int32_t t = a.w.targets[m];
                                a.nll[m] = (t >= 0 && (int64_t)t < V)
                                               ? L - __hip_atomic_load(a.w.tl + m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                               : __builtin_nanf("");
                            }
                        }
                    }
                }
                if (lane == 0) {
                    __hip_atomic_store(sync + sync_top_done(), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_fetch_add(sync + sync_epoch(), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
    };
    auto count_and_finish = [&](bool with_keys) __attribute__((always_inline)) {
        if (count_wg(with_keys))
            resolve_final();
    };

    // ---- top-k selection (tk_K > 0) ----
    // Every streaming wave leaves the largest key of its rows in tkw (one key
    // per wave and hidden state) and its logits in memory.  Let T be the K-th
    // largest of those wave keys: K distinct logit keys reach T, so each of
    // the K largest logit keys is at least T, and a wave whose largest key is
    // below T holds none of them.  The last workgroup therefore
    //   1. loads the wave keys, thread t keys t, t + 256, ... (tk_L of them,
    //      all in flight at once);
    //   2. takes in each wave the K-th largest of its threads' maxima: the
    //      largest of the four, B, is at most T (K distinct wave keys reach it);
    //   3. gathers the wave keys at or above B into LDS (at most K threads per
    //      wave hold one, so at most 4 K tk_L keys) and ranks them: the K
    //      largest name the source waves, the K-th of them is T;
    //   4. loads the logits of the source waves (K NV 16 rows at most) and
    //      gathers the keys at or above T;
    //   5. ranks those: the K largest, in order.
    // With fewer than K nonzero wave keys (tiny heads) T is 0 and every row
    // of every wave is a candidate.
    //
    // Appends the keys whose predicate holds to s[] (capacity cap; counter
    // *cnt): one LDS atomic per wave reserves the wave's block, and each lane
    // writes at the block's start plus the number of earlier items of the
    // wave (lower item index, then lower lane).
    auto wave_append = [&](const auto &pr, const auto &key, uint32_t *cnt, uint64_t *s,
                           uint32_t cap) __attribute__((always_inline)) {
        constexpr int N = sizeof(pr) / sizeof(pr[0]);
        uint32_t off[N], run = 0;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const uint64_t bal = __ballot(pr[i]);
            off[i] = run + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
            run += (uint32_t)__popcll(bal);
        }
        if (run == 0)
            return;
        uint32_t base = 0;
        if (lane == 0)
            base = atomicAdd(cnt, run);
        base = (uint32_t)__builtin_amdgcn_readfirstlane(base);
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (pr[i] && base + off[i] < cap)
                s[base + off[i]] = key[i];
    };
    // The K largest of n unique nonzero keys in LDS, to out[0, K) in
    // descending order (zeros past n), by all 256 threads.  A key's rank is
    // the number of keys above it.  With n <= 64 the comparisons are split
    // over the four waves (lane c ranks key c against keys j = wave mod 4)
    // and the partial ranks meet in LDS counters; with n <= 256 each thread
    // ranks one key against all n; beyond that wave 0 takes K rounds of a
    // wave maximum below the previous winner.  s_rank[64] is zero on entry
    // and on exit.
    auto select_k = [&](const uint64_t *s, uint32_t n, uint64_t *out, uint32_t *s_rank)
                        __attribute__((always_inline)) {
        const int K = a.tk_K;
        const uint32_t t = threadIdx.x;
        if (n <= 64) {
            if ((uint32_t)lane < n) {
                const uint64_t c = s[lane];
                uint32_t part = 0;
#pragma unroll
                for (uint32_t j0 = 0; j0 < 64; j0 += 16) {
                    if (j0 >= n)
                        break;
                    uint64_t q[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t j = j0 + 4 * i + wv;
                        q[i] = s[j < n ? j : n - 1];
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        part += (j0 + 4 * i + wv < n && q[i] > c) ? 1u : 0u;
                }
                if (part)
                    atomicAdd(s_rank + lane, part);
            }
            __syncthreads();
            if (t < n) {
                const uint32_t rank = s_rank[t];
                s_rank[t] = 0;
                if (rank < (uint32_t)K)
                    out[rank] = s[t];
            } else if (t < (uint32_t)K) {
                out[t] = 0;
            }
        } else if (n <= 256) {
            if (t < n) {
                const uint64_t c = s[t];
                uint32_t rank = 0;
                // eight keys per step, read together (the arrays keep kTkSpare
                // slots past their capacity, so the reads stay inside them)
                for (uint32_t j = 0; j < n; j += 8) {
                    uint64_t q[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        q[i] = s[j + i];
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        rank += (j + i < n && q[i] > c) ? 1u : 0u;
                }
                if (rank < (uint32_t)K)
                    out[rank] = c;
            } else if (t < (uint32_t)K) {
                out[t] = 0;
            }
        } else if (wv == 0) {
            uint64_t win = 0;
            for (int r = 0; r < K; ++r) {
                uint64_t best = 0;
                for (uint32_t q = lane; q < n; q += 64) {
                    const uint64_t k = s[q];
                    best = ((r == 0 || k < win) && k > best) ? k : best;
                }
                win = wave_max_u64(best);
                if (lane == 0)
                    out[r] = win;
            }
        }
        __syncthreads();
    };
    auto topk_resolve = [&]() __attribute__((always_inline)) {
        constexpr int SI = (kTopKMax * NV * kVB + 255) / 256; // rows of the source waves per thread
        const int K = a.tk_K, Q = a.tk_L;
        const int64_t nw = (int64_t)a.nwg * 4;
        uint64_t *const s_win = (uint64_t *)(smem + a.lds_tk);            // [16] selected keys
        uint64_t *const s_bnd = s_win + 16;                               // [4] per-wave bounds
        uint32_t *const s_cnt = (uint32_t *)(s_win + 20);                 // [2] gather counters
        uint32_t *const s_rank = (uint32_t *)(smem + a.lds_tk + 256);     // [64] partial ranks
        uint64_t *const s_tm = (uint64_t *)(smem + a.lds_tk + kTkMiscBytes); // [256] thread maxima
        uint64_t *const s_wk = s_tm + 256;                                // [4 K Q + spare] wave keys >= B
        const uint32_t cap1 = 4u * (uint32_t)K * (uint32_t)Q;
        uint64_t *const s_cand = s_wk + cap1 + kTkSpare;                  // [K NV 16 + spare] candidates
        const uint32_t cap2 = (uint32_t)K * NV * kVB;
        const int t = threadIdx.x;
        if (t < 64)
            s_rank[t] = 0; // ordered before its first use by the barriers below
        for (int m = 0; m < MF; ++m) {
            if (t < 2)
                s_cnt[t] = 0;
            if (lane == 0)
                s_bnd[wv] = 0;
            // 1.
            uint64_t kk[kTkKeys];
            uint64_t tmax = 0;
#pragma unroll
            for (int i = 0; i < kTkKeys; ++i) {
                const int64_t g = t + 256 * i;
                const bool ok = i < Q && g < nw;
                kk[i] = __hip_atomic_load(a.tkw + (ok ? m * nw + g : 0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            // the draw's uniform number, read beside the wave keys (one round
            // trip for both; an atomic load stays where it is written)
            const float um = a.tk_u ? __hip_atomic_load(a.tk_u + m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.f;
#pragma unroll
            for (int i = 0; i < kTkKeys; ++i) {
                const bool ok = i < Q && (int64_t)(t + 256 * i) < nw;
                kk[i] = ok ? kk[i] : 0;
                tmax = umax64(tmax, kk[i]);
            }
            s_tm[t] = tmax;
            __syncthreads();
            // 2.
            {
                const uint64_t *w = s_tm + wv * 64;
                uint32_t rank = 0;
                for (int j = 0; j < 64; j += 2) {
                    const uint64_t s0 = w[j], s1 = w[j + 1];
                    rank += (s0 > tmax ? 1u : 0u) + (s1 > tmax ? 1u : 0u);
                }
                if (tmax != 0 && rank == (uint32_t)(K - 1))
                    s_bnd[wv] = tmax;
            }
            __syncthreads();
            // 3.
            const uint64_t B = umax64(umax64(s_bnd[0], s_bnd[1]), umax64(s_bnd[2], s_bnd[3]));
            {
                bool pr[kTkKeys];
#pragma unroll
                for (int i = 0; i < kTkKeys; ++i)
                    pr[i] = kk[i] != 0 && kk[i] >= B;
                wave_append(pr, kk, s_cnt, s_wk, cap1);
            }
            __syncthreads();
            select_k(s_wk, s_cnt[0] < cap1 ? s_cnt[0] : cap1, s_win, s_rank);
            // 4.
            const uint64_t T = s_win[K - 1];
            float y[SI];
            int64_t row[SI];
#pragma unroll
            for (int i = 0; i < SI; ++i) {
                const int it = t + 256 * i;
                const int src = it / (NV * kVB);
                const uint64_t wk = src < K ? s_win[src] : 0;
                const int64_t gws = (int64_t)((0xFFFFFFFFu - (uint32_t)wk) / kVB) / NV;
                row[i] = wk != 0 ? gws * NV * kVB + (it - src * NV * kVB) : V;
                y[i] = __hip_atomic_load(a.logits + m * V + (row[i] < V ? row[i] : 0), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
            }
            {
                bool pr[SI];
                uint64_t key[SI];
#pragma unroll
                for (int i = 0; i < SI; ++i) {
                    key[i] = argmax_key(y[i], (uint32_t)(row[i] < V ? row[i] : 0));
                    pr[i] = row[i] < V && key[i] >= T;
                }
                wave_append(pr, key, s_cnt + 1, s_cand, cap2);
            }
            __syncthreads();
            // 5.
            select_k(s_cand, s_cnt[1] < cap2 ? s_cnt[1] : cap2, s_win, s_rank);
            if (wv == 0) {
                if (lane < K) {
                    const uint64_t k = s_win[lane];
                    a.tk_idx[m * K + lane] = (int32_t)(0xFFFFFFFFu - (uint32_t)k);
                    a.tk_vals[m * K + lane] = key_value(k);
                }
                if (a.tk_u && lane == 0) {
                    // candidate j weighs 2^((v_j - v_0) log2(e) / tau); the draw
                    // is the first j whose running sum exceeds u times the total
                    float v[16], cum[16], c = 0.f;
#pragma unroll
                    for (int j = 0; j < 16; ++j)
                        v[j] = key_value(s_win[j < K ? j : K - 1]);
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        c += j < K ? __builtin_amdgcn_exp2f((v[j] - v[0]) * a.tk_scale) : 0.f;
                        cum[j] = c;
                    }
                    const float tu = um * c;
                    int pick = K - 1;
#pragma unroll
                    for (int j = 15; j >= 0; --j)
                        pick = (j < K && cum[j] > tu) ? j : pick;
                    a.tk_samples[m] = (int32_t)(0xFFFFFFFFu - (uint32_t)s_win[pick]);
                }
            }
            __syncthreads(); // the next hidden state reuses the LDS
        }
    };

    // Projection columns.  With projection-only workgroups, their wave pw
    // publishes columns pw, pw + 4 ntwg, ...; they start at once, stream
    // nothing and leave.  Without them, streaming wave gw publishes columns
    // gw, gw + nw, ... (nw streaming waves) before its residual.
    if (proj_wg) {
        const int64_t nx = MF * d / 8;
        for (int64_t i0 = 0; i0 < nx; i0 += 256) {
            const int64_t i = i0 + threadIdx.x;
            if (i < nx)
                __builtin_amdgcn_global_load_lds((const void *)((const u32x4 *)a.X + i),
                                                 (__attribute__((address_space(3))) void *)((u32x4 *)(smem + a.lds_x) + i0 + wv * 64), 16, 0, 0);
        }
        __syncthreads();
        // up to PB columns per batch, all their loads issued together, one
        // wait for all their stores: under the full memory load of the
        // streaming workgroups every round trip is long
        constexpr int PB = MF == 1 ? 4 : 2;
        const int64_t stride = (int64_t)a.ntwg * 4;
        const uint32_t tag = __builtin_amdgcn_readfirstlane(epoch) + 1u;
        const int64_t Mp = a.w.Mp;
        const u32x4 z = {0u, 0u, 0u, 0u};
        for (int64_t i0 = (int64_t)blockIdx.x * 4 + wv; i0 < ntask; i0 += PB * stride) {
            int ci[PB];
#pragma unroll
            for (int b = 0; b < PB; ++b) {
                const int64_t i = i0 + b * stride;
                ci[b] = (int)(i < ntask ? i : ntask - 1); // past the end: repeat the last column
            }
            float acc[PB][MF];
#pragma unroll
            for (int b = 0; b < PB; ++b)
#pragma unroll
                for (int m = 0; m < MF; ++m)
                    acc[b][m] = 0.f;
            for (int64_t j00 = 0; j00 < d; j00 += 4096) {
                u32x4 wq[PB][4];
                float sc[PB][4];
#pragma unroll
                for (int b = 0; b < PB; ++b) {
                    const bool isd = ci[b] >= k;
                    const int64_t c = isd ? ci[b] - k : ci[b];
                    const int8_t *row = isd ? a.h.d8 + c * d : a.h.b8 + c * d;
#pragma unroll
                    for (int it = 0; it < 4; ++it) {
                        const int64_t j0 = j00 + 1024 * it + 16 * lane;
                        const int64_t jc = j0 < d ? j0 : 0;
                        wq[b][it] = *(const u32x4 *)(row + jc);
                        sc[b][it] = isd ? a.h.sd[c * G + jc / a.h.s.g] : 1.0f;
                    }
                }
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const int64_t j0 = j00 + 1024 * it + 16 * lane;
                    const bool ok = j0 < d;
#pragma unroll
                    for (int m = 0; m < MF; ++m) {
                        const u32x4 *xp = (const u32x4 *)(s_x + m * d + (ok ? j0 : 0));
                        const u32x4 x0 = ok ? xp[0] : z, x1 = ok ? xp[1] : z;
#pragma unroll
                        for (int b = 0; b < PB; ++b)
                            acc[b][m] = __builtin_fmaf(sc[b][it], dot16(ok ? wq[b][it] : z, x0, x1), acc[b][m]);
                    }
                }
            }
#pragma unroll
            for (int b = 0; b < PB; ++b) {
                const bool isd = ci[b] >= k;
                const int64_t c = isd ? ci[b] - k : ci[b];
#pragma unroll
                for (int m = 0; m < MF; ++m) {
                    float v = acc[b][m];
                    for (int off = 32; off >= 1; off >>= 1)
                        v += __shfl_xor(v, off);
                    const float t = isd ? v : v * a.h.sb[c];
                    const uint16_t hi = f32_to_bf16_rne(t);
                    const uint16_t lo = f32_to_bf16_rne(t - __uint_as_float((uint32_t)hi << 16));
                    if (lane == m && i0 + b * stride < ntask) {
                        store_device(isd ? a.w.s16 + m * rpad + c : a.w.t16 + m * kpad + c, hi);
                        store_device(isd ? a.w.s16 + (Mp + m) * rpad + c : a.w.t16 + (Mp + m) * kpad + c, lo);
                    }
                }
            }
            wait_vm_all();
            if (lane < PB && i0 + lane * stride < ntask) {
                __hip_atomic_store(a.w.colflag + i0 + lane * stride, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_fetch_add(sync + sync_published(), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        __syncthreads(); // every column of this workgroup is published
        if (a.tk_K) { // the last workgroup counted runs the selection with all its waves
            if (wv == 0) {
                const bool last = count_wg(false);
                if (lane == 0)
                    s_last = last ? 1 : 0;
            }
            __syncthreads();
            if (s_last) {
                topk_resolve();
                if (wv == 0)
                    resolve_final();
            }
            return;
        }
        if (wv == 0)
            count_and_finish(false);
        return;
    }
    const int64_t gw = bid * 4 + wv, nw = (int64_t)a.nwg * 4;

    {   // residual scales, row scales of the low-rank terms and X into LDS,
        // issued before the first prefetches so that the wait for them
        // leaves the prefetches in flight
        const int64_t nvb_wg = (nvb - wg_vb0) < 4 * NV ? (nvb - wg_vb0) : 4 * NV;
        const int64_t nsr = nvb_wg * G * kVB / 8, nsa = nvb_wg * kVB / 8, nx = MF * d / 8;
        for (int64_t i0 = 0; i0 < nsr; i0 += 256) {
            const int64_t i = i0 + threadIdx.x;
            if (i < nsr)
                lds_dma16<false>((const u32x4 *)(a.h.sr + wg_vb0 * G * kVB) + i, (u32x4 *)smem + i0 + wv * 64);
        }
        if (threadIdx.x < 64) {
            for (int64_t i0 = 0; i0 < nsa; i0 += 64)
                if (i0 + lane < nsa) {
                    lds_dma16<false>((const u32x4 *)(a.h.sa + wg_vb0 * kVB) + i0 + lane, (u32x4 *)(smem + a.lds_sa) + i0);
                    lds_dma16<false>((const u32x4 *)(a.h.sc + wg_vb0 * kVB) + i0 + lane,
                                     (u32x4 *)(smem + a.lds_sa) + 4 * NV * kVB / 8 + i0);
                }
        }
        for (int64_t i0 = 0; i0 < nx; i0 += 256) {
            const int64_t i = i0 + threadIdx.x;
            if (i < nx)
                lds_dma16<false>((const u32x4 *)a.X + i, (u32x4 *)(smem + a.lds_x) + i0 + wv * 64);
        }
    }
    DPair<NV> P0, P1;
    load_pair(P0, 0);
    load_pair(P1, 1);
    // this wave's copies have landed once at most its 4 NV prefetches are
    // outstanding; after the barrier, every wave's have
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(4 * NV));
    __syncthreads();
    if (a.ntwg == 0)
        for (int64_t i = gw; i < ntask; i += nw)
            publish((int)i);

    // The offset of the residual codes, -136 sum_{j in grp} X[m,j], for
    // every group, once per wave: in the VALU variant each of the four lanes
    // of a row adds a quarter.  A lane sums one group, starting at a piece
    // that depends on the lane, so that lanes reading groups a multiple of
    // the LDS banks apart do not all meet in one bank.
    float *const s_xs = (float *)(smem + a.lds_xs) + wv * MF * G;
    {
        const uint32_t one = vgpr_const(kBf16One);
        const int pg = (int)(a.h.s.g / 8), nG = (int)G;
        for (int i = lane; i < MF * nG; i += 64) {
            const uint16_t *xp = s_x + (i / nG) * d + (int64_t)(i % nG) * a.h.s.g;
            float sum = 0.f;
            int pp = lane % pg;
            for (int p = 0; p < pg; ++p) {
                sum = dot8c(*(const u32x4 *)(xp + 8 * pp), one, sum);
                pp = pp + 1 == pg ? 0 : pp + 1;
            }
            s_xs[i] = (MX ? -136.f : -34.f) * sum;
        }
    }

    // VALU variant: per-lane partial sums over the lane's columns
    float tot[NV][MF], g[NV][MF];
#pragma unroll
    for (int m = 0; m < MF; ++m)
#pragma unroll
        for (int v = 0; v < NV; ++v)
            tot[v][m] = g[v][m] = 0.f;
    // matrix-core variant: [16 rows of X (row m in lanes 16(m/4)..) x 16
    // vocabulary rows] tiles; lane l holds rows 4(l/16) + i of column l % 16.
    // Chunk kc accumulates into gq[kc & 1] and is folded one chunk later
    // (reading an accumulator right after its MFMAs would stall the wave).
    // Only rows m < MF of the tiles are kept in the running totals (lanes
    // 0..15 hold them, MF <= 4).
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 gq[2][NV];
    float acc[NV][MF];
    bool pend = false; // chunk kc - 1 still to fold
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int m = 0; m < MF; ++m)
            acc[v][m] = 0.f;
    const int64_t xrow = lr < MF ? lr : MF - 1; // A-operand rows past M repeat the last row
    const uint32_t kMagic = vgpr_const(kBf16Magic);

    auto fold_mx = [&](int sel, int64_t kc) __attribute__((always_inline)) {
        float xo[MF];
#pragma unroll
        for (int m = 0; m < MF; ++m)
            xo[m] = s_xs[m * G + kc];
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const float scl = h2f(s_sr[((wv * NV + v) * G + kc) * kVB + lr]);
#pragma unroll
            for (int m = 0; m < MF; ++m)
                acc[v][m] = __builtin_fmaf(scl, gq[sel][v][m] + xo[m], acc[v][m]);
        }
    };
    auto flush_mx = [&](int64_t kc_last) __attribute__((always_inline)) {
        // (constant accumulator indices only: a run-time index would put the
        // accumulators in scratch memory)
        if (MX && pend) {
            if (kc_last & 1)
                fold_mx(1, kc_last);
            else
                fold_mx(0, kc_last);
        }
        pend = false;
    };

    // residual K-chunk kc: 4 K-steps; each g-group is folded with its scale
    // when it ends: tot += sR (sum x (q + 136) - 136 sum x)
    auto res_chunk = [&](const DChunk<NV> &c, int64_t kc, int sel) __attribute__((always_inline)) {
        if constexpr (MX) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int64_t ks = kc * 4 + s;
                const u32x4 xa = *(const u32x4 *)(s_x + xrow * d + ks * kKStep + 8 * lq);
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    const uint32_t wd = s == 0 ? c.q[v].x : s == 1 ? c.q[v].y : s == 2 ? c.q[v].z : c.q[v].w;
                    gq[sel][v] = mfma_bf16(xa, r4_bf16(wd, kMagic), s == 0 ? zero4 : gq[sel][v]);
                }
#pragma unroll
                for (int v = 0; v < NV; ++v)
                    pin4(gq[sel][v]);
                step_fence();
            }
            if (pend)
                fold_mx(sel ^ 1, kc - 1);
            pend = true;
            step_fence();
            return;
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int64_t ks = kc * 4 + s;
            u32x4 x[MF];
#pragma unroll
            for (int m = 0; m < MF; ++m) {
                x[m] = *(const u32x4 *)(s_x + m * d + ks * kKStep + 8 * lq);
            }
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const uint32_t wd = s == 0 ? c.q[v].x : s == 1 ? c.q[v].y : s == 2 ? c.q[v].z : c.q[v].w;
                const u32x4 b = r4_bf16(wd, kMagic);
#pragma unroll
                for (int m = 0; m < MF; ++m)
                    g[v][m] = dot8(x[m], b, g[v][m]);
            }
            const bool gend = GS == 4 ? s == 3 : (ks % gsteps) == gsteps - 1;
            if (gend) {
                const int64_t grp = GS == 4 ? kc : ks / gsteps;
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    const float scl = h2f(s_sr[((wv * NV + v) * G + grp) * kVB + lr]);
#pragma unroll
                    for (int m = 0; m < MF; ++m) {
                        tot[v][m] = __builtin_fmaf(scl, g[v][m] + s_xs[m * G + grp], tot[v][m]);
                        g[v][m] = 0.f;
                    }
                }
            }
            // one K-step at a time: the hidden-state fragments and
            // dequantised codes of later K-steps are not hoisted into
            // registers early, nor this step's arithmetic sunk late
#pragma unroll
            for (int m = 0; m < MF; ++m)
#pragma unroll
                for (int v = 0; v < NV; ++v)
                    pin(g[v][m]);
            step_fence();
        }
    };
    // low-rank chunk j: three core K-steps (A5 + 16 against t) or two
    // correction K-steps (C8 against s); K-steps beyond the rank are skipped
    float ga[NV][MF], gc[NV][MF];
    f32x4 gam[NV], gcm[NV];
    const uint16_t *s_t = s_ts, *s_s = s_ts + 2 * MF * kpad;
    auto lr_chunk = [&](const DChunk<NV> &c, int64_t j) __attribute__((always_inline)) {
        if constexpr (MX) {
            if (j < na) {
#pragma unroll
                for (int q = 0; q < 3; ++q) {
                    const int64_t ks = 3 * j + q;
                    if (ks >= kst)
                        break;
                    const u32x4 th = *(const u32x4 *)(s_t + xrow * kpad + ks * kKStep + 8 * lq);
                    const u32x4 tl = *(const u32x4 *)(s_t + (MF + xrow) * kpad + ks * kKStep + 8 * lq);
#pragma unroll
                    for (int v = 0; v < NV; ++v) {
                        const uint32_t wn = q == 0 ? c.q[v].x : q == 1 ? c.q[v].y : c.q[v].z;
                        const u32x4 b = a5_bf16_q(wn, c.q[v].w, q);
                        gam[v] = mfma_bf16(tl, b, mfma_bf16(th, b, gam[v]));
                    }
#pragma unroll
                    for (int v = 0; v < NV; ++v)
                        pin4(gam[v]);
                    step_fence();
                }
            } else {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int64_t ks = 2 * (j - na) + hh;
                    if (ks >= rst)
                        break;
                    const u32x4 sh = *(const u32x4 *)(s_s + xrow * rpad + ks * kKStep + 8 * lq);
                    const u32x4 sl = *(const u32x4 *)(s_s + (MF + xrow) * rpad + ks * kKStep + 8 * lq);
#pragma unroll
                    for (int v = 0; v < NV; ++v) {
                        u32x2 w;
                        w.x = hh == 0 ? c.q[v].x : c.q[v].z;
                        w.y = hh == 0 ? c.q[v].y : c.q[v].w;
                        const u32x4 b = c8_bf16(w);
                        gcm[v] = mfma_bf16(sl, b, mfma_bf16(sh, b, gcm[v]));
                    }
#pragma unroll
                    for (int v = 0; v < NV; ++v)
                        pin4(gcm[v]);
                    step_fence();
                }
            }
            return;
        }
        if (j < na) {
#pragma unroll
            for (int q = 0; q < 3; ++q) {
                const int64_t ks = 3 * j + q;
                if (ks >= kst)
                    break;
                u32x4 th[MF], tl[MF];
#pragma unroll
                for (int m = 0; m < MF; ++m) {
                    th[m] = *(const u32x4 *)(s_t + m * kpad + ks * kKStep + 8 * lq);
                    tl[m] = *(const u32x4 *)(s_t + (MF + m) * kpad + ks * kKStep + 8 * lq);
                }
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    const uint32_t wn = q == 0 ? c.q[v].x : q == 1 ? c.q[v].y : c.q[v].z;
                    const u32x4 b = a5_bf16_q(wn, c.q[v].w, q);
#pragma unroll
                    for (int m = 0; m < MF; ++m)
                        ga[v][m] = dot8(tl[m], b, dot8(th[m], b, ga[v][m]));
                }
#pragma unroll
                for (int m = 0; m < MF; ++m)
#pragma unroll
                    for (int v = 0; v < NV; ++v)
                        pin(ga[v][m]);
                step_fence();
            }
        } else {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int64_t ks = 2 * (j - na) + hh;
                if (ks >= rst)
                    break;
                u32x4 sh[MF], sl[MF];
#pragma unroll
                for (int m = 0; m < MF; ++m) {
                    sh[m] = *(const u32x4 *)(s_s + m * rpad + ks * kKStep + 8 * lq);
                    sl[m] = *(const u32x4 *)(s_s + (MF + m) * rpad + ks * kKStep + 8 * lq);
                }
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    u32x2 w;
                    w.x = hh == 0 ? c.q[v].x : c.q[v].z;
                    w.y = hh == 0 ? c.q[v].y : c.q[v].w;
                    const u32x4 b = c8_bf16(w);
#pragma unroll
                    for (int m = 0; m < MF; ++m)
                        gc[v][m] = dot8(sl[m], b, dot8(sh[m], b, gc[v][m]));
                }
#pragma unroll
                for (int m = 0; m < MF; ++m)
#pragma unroll
                    for (int v = 0; v < NV; ++v)
                        pin(gc[v][m]);
                step_fence();
            }
        }
    };

    // two pairs per iteration: residual pairs pi, pi + 1 (K-chunks kc0 ..
    // kc0 + 3) or low-rank pairs pi, pi + 1; the last iteration issues no
    // loads (no load sits under a branch, which would make the compiler copy
    // the prefetch buffers)
    // Pacing.  The two workgroups that share a compute unit put a wave on
    // every SIMD each, and the instruction arbiter favours the older wave:
    // left alone, the first workgroup on each unit finishes long before the
    // second, which then streams its last quarter with half the unit's loads
    // in flight.  Each wave starts at the highest priority and drops a level
    // as it enters each further quarter of its chunk pairs, so that the wave
    // behind is issued first and the two stay within about a quarter.
    int pace_lvl = 0;
    auto pace = [&](int64_t pi) __attribute__((always_inline)) {
        const int lvl = (int)((4 * pi) / npairs);
        if (lvl != pace_lvl) {
            pace_lvl = lvl;
            if (lvl == 1)
                __builtin_amdgcn_s_setprio(2);
            else if (lvl == 2)
                __builtin_amdgcn_s_setprio(1);
            else
                __builtin_amdgcn_s_setprio(0);
        }
    };
    auto res_iter = [&](int64_t pi, int64_t kc0, bool load) __attribute__((always_inline)) { // kc0 % 4 == 0
        pace(pi);
        // each chunk's registers are refilled as soon as the chunk is used,
        // so that close to four chunks stay in flight
        res_chunk(P0.h0, kc0, 0);
        if (load)
            load_chunk(P0.h0, 2 * pi + 4);
        __builtin_amdgcn_sched_barrier(0);
        res_chunk(P0.h1, kc0 + 1, 1);
        if (load)
            load_chunk(P0.h1, 2 * pi + 5);
        __builtin_amdgcn_sched_barrier(0);
        res_chunk(P1.h0, kc0 + 2, 0);
        if (load)
            load_chunk(P1.h0, 2 * pi + 6);
        __builtin_amdgcn_sched_barrier(0);
        res_chunk(P1.h1, kc0 + 3, 1);
        if (load)
            load_chunk(P1.h1, 2 * pi + 7);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto lr_iter = [&](int64_t pi) __attribute__((always_inline)) {
        pace(pi);
        lr_chunk(P0.h0, 2 * pi - c1);
        load_chunk(P0.h0, 2 * pi + 4);
        __builtin_amdgcn_sched_barrier(0);
        lr_chunk(P0.h1, 2 * pi + 1 - c1);
        load_chunk(P0.h1, 2 * pi + 5);
        __builtin_amdgcn_sched_barrier(0);
        lr_chunk(P1.h0, 2 * pi + 2 - c1);
        load_chunk(P1.h0, 2 * pi + 6);
        __builtin_amdgcn_sched_barrier(0);
        lr_chunk(P1.h1, 2 * pi + 3 - c1);
        load_chunk(P1.h1, 2 * pi + 7);
        __builtin_amdgcn_sched_barrier(0);
    };

    // One control path for every shape (separate paths for the cases made
    // the register allocator spill the prefetch buffers).  The second-last
    // iteration before the low-rank pairs reads the count of published
    // columns, issued ahead of the iteration's prefetch so that waiting for
    // it costs nothing (loads complete in order).  The count grows by k + r
    // per call and is never reset, so it equals (k + r)(calls before + 1)
    // exactly when this call has published every column.  t and s are then
    // copied to LDS at the start of the last iteration and waited for at its
    // end, where only that iteration's prefetches may still be in flight; if
    // the count fell short, the column flags tell which columns the wave
    // must compute itself.
    int64_t pi = 0;
    for (; pi + 4 < nrp1; pi += 2)
        res_iter(pi, 2 * pi, true);
    uint32_t seen = 0;
    if (nrp1 >= 4) {
        seen = __hip_atomic_load(sync + sync_published(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        res_iter(pi, 2 * pi, true);
        pi += 2;
    }
    const bool ready = nlr > 0 && nrp1 >= 4 &&
                       (uint32_t)__builtin_amdgcn_readfirstlane(seen) ==
                           (uint32_t)ntask * ((uint32_t)__builtin_amdgcn_readfirstlane(epoch) + 1u);
    if (ready)
        stage_ts();
    if (nrp1 >= 2) {
        res_iter(pi, 2 * pi, true);
        pi += 2;
    }
    flush_mx(2 * pi - 1);
    if (nlr > 0) {
        if (ready) {
            // the copy has landed once at most the 4 NV prefetches issued
            // after it are outstanding
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(4 * NV));
            asm volatile("" ::: "memory");
        } else {
            build_ts();
            wait_vm_all();
        }
    }
    // the offset of the core codes, -144 sum_i t[m,i] (hi and lo parts),
    // once per wave (in the VALU variant a quarter per lane of a row)
    float nto[MF];
#pragma unroll
    for (int m = 0; m < MF; ++m) {
        const uint32_t one = vgpr_const(kBf16One);
        float sum = 0.f;
        for (int64_t i = lane; i < kpad / 8; i += 64) {
            sum = dot8c(*(const u32x4 *)(s_t + m * kpad + 8 * i), one, sum);
            sum = dot8c(*(const u32x4 *)(s_t + (MF + m) * kpad + 8 * i), one, sum);
        }
        for (int off = 32; off >= 1; off >>= 1)
            sum += __shfl_xor(sum, off);
        nto[m] = (MX ? -144.f : -36.f) * sum;
    }
#pragma unroll
    for (int m = 0; m < MF; ++m)
#pragma unroll
        for (int v = 0; v < NV; ++v)
            ga[v][m] = gc[v][m] = 0.f;
#pragma unroll
    for (int v = 0; v < NV; ++v)
        gam[v] = gcm[v] = zero4;
    // at least two residual pairs follow, so every iteration prefetches
    for (; pi < nrp1 + nlp; pi += 2)
        lr_iter(pi);
    // tot += sA (A5 t - 144 sum t) + sC (C8 s)
    const uint16_t *s_sa = (const uint16_t *)(smem + a.lds_sa) + wv * NV * kVB;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const float sa = h2f(s_sa[v * kVB + lr]), sc = h2f(s_sa[4 * NV * kVB + v * kVB + lr]);
        if constexpr (MX) {
#pragma unroll
            for (int m = 0; m < MF; ++m)
                acc[v][m] = __builtin_fmaf(sa, gam[v][m] + nto[m], __builtin_fmaf(sc, gcm[v][m], acc[v][m]));
        } else {
#pragma unroll
            for (int m = 0; m < MF; ++m)
                tot[v][m] = __builtin_fmaf(sa, ga[v][m] + nto[m], __builtin_fmaf(sc, gc[v][m], tot[v][m]));
        }
    }
    for (; pi + 2 < npairs; pi += 2)
        res_iter(pi, 2 * pi - nlr, true);
    res_iter(pi, 2 * pi - nlr, false);
    flush_mx(nkc - 1);

    // ---- logits: the four lanes of a row add their partial sums ----
    uint64_t key[MF];
    float yv[NV][MF];
#pragma unroll
    for (int m = 0; m < MF; ++m)
        key[m] = 0;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int64_t row = vb0 + v < nvb ? (vb0 + v) * kVB + lr : V;
#pragma unroll
        for (int m = 0; m < MF; ++m) {
            float y;
            if constexpr (MX) {
                y = acc[v][m]; // row m of lanes 0..15 (MF <= 4)
            } else {
                y = tot[v][m];
                y += __shfl_xor(y, 16);
                y += __shfl_xor(y, 32);
            }
            yv[v][m] = y + 0.0f; // -0 stored as +0, as the keys order it
            if (row < V)
                key[m] = umax64(key[m], argmax_key(y, (uint32_t)row));
        }
    }
    auto store_logits = [&]() __attribute__((always_inline)) {
        if (!a.logits)
            return;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int64_t row = vb0 + v < nvb ? (vb0 + v) * kVB + lr : V;
#pragma unroll
            for (int m = 0; m < MF; ++m)
                if (row < V && lq == 0)
                    a.logits[m * V + row] = yv[v][m];
        }
    };

    // ---- a3: workgroup maximum per row; then per slot of workgroups (the
    // workgroups b with b % nslot == s) an atomic max and a count; the last
    // workgroup of each slot counts the slot as done, and the last slot
    // reads every slot's keys, resolves them and resets every counter ----
    if (a.argmax) {
#pragma unroll
        for (int m = 0; m < MF; ++m) {
            uint64_t kk = key[m];
            kk = umax16_u64(kk);
            if (lane == 0)
                red[wv][m] = kk;
        }
    }
    // the wave's (max, sum exp) per hidden state over its live rows (lanes
    // 0..15 hold rows lr of the wave's v-blocks), and the target's logit from
    // the lane that holds it, complete before the workgroup is counted
    if (a.w.want_lse) {
#pragma unroll
        for (int m = 0; m < MF; ++m) {
            float mx = -__builtin_inff();
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int64_t row = vb0 + v < nvb ? (vb0 + v) * kVB + lr : V;
                if (row < V) {
                    mx = fmaxf(mx, yv[v][m]);
                    if (row == tgt[m] && lane < 16)
                        __hip_atomic_store(a.w.tl + m, yv[v][m], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            mx = max16(mx);
            float sx = 0.f;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int64_t row = vb0 + v < nvb ? (vb0 + v) * kVB + lr : V;
                if (row < V)
                    sx += exp_le0(yv[v][m] - mx);
            }
            sx = sum16(sx);
            if (lane == 0)
                lred[wv][m] = LsePart{mx, sx};
        }
        wait_vm_all();
    }
    // top-k: the wave's largest key of each hidden state (rows in lanes
    // 0..15) and its logits, with device-scope stores complete before the
    // workgroup is counted (the last workgroup reads both)
    if (a.tk_K) {
        const int64_t nw = (int64_t)a.nwg * 4;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int64_t row = vb0 + v < nvb ? (vb0 + v) * kVB + lr : V;
#pragma unroll
            for (int m = 0; m < MF; ++m)
                if (row < V && lq == 0)
                    __hip_atomic_store(a.logits + m * V + row, yv[v][m], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int m = 0; m < MF; ++m) {
            const uint64_t kk = umax16_u64(key[m]);
            if (lane == 0)
                __hip_atomic_store(a.tkw + m * nw + bid * 4 + wv, kk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        wait_vm_all();
    }
    // every wave of the workgroup is past its last use of the counters (and
    // its top-k stores are complete)
    __syncthreads();
    if (a.tk_K) {
        if (wv == 0) {
            const bool last = count_wg(true);
            if (lane == 0)
                s_last = last ? 1 : 0;
        }
        __syncthreads();
        if (s_last) {
            topk_resolve();
            if (wv == 0)
                resolve_final();
        }
        return;
    }
    if (wv != 0) {
        store_logits();
        return;
    }
    // wave 0.  Device-scope atomics are performed at the device's coherence
    // point; each is complete before the count that follows it, so a slot's
    // keys are final once its count is full, and every key is final once
    // every slot is counted.
    count_and_finish(true);
    store_logits();
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
static size_t dal16(size_t x) { return (x + 15) / 16 * 16; }

struct DecodeLds {
    unsigned sa, x, ts, xs, tk;
    size_t total;
};

// streaming workgroups of the single launch for M hidden states
static int64_t decode_nwg(const Shape &s, int64_t M) { return (s.nvb() + 4 * decode_nv((int)M) - 1) / (4 * decode_nv((int)M)); }

// wave keys per thread of the last workgroup's top-k selection
static int decode_tk_keys(const Shape &s, int64_t M) { return (int)((decode_nwg(s, M) + 63) / 64); }

static DecodeLds decode_lds(const Shape &s, int64_t M, int K = 0)
{
    DecodeLds L;
    L.sa = (unsigned)dal16(size_t(4) * decode_nv((int)M) * s.G() * kVB * 2);
    L.x = (unsigned)(L.sa + size_t(2) * 4 * decode_nv((int)M) * kVB * 2);
    L.ts = (unsigned)(L.x + dal16(size_t(M) * s.d * 2));
    L.xs = (unsigned)dal16(L.ts + size_t(4) * 2 * M * (s.kpad() + s.rpad()) * 2);
    L.total = L.xs + size_t(4) * M * s.G() * 4;
    L.tk = (unsigned)dal16(L.total);
    if (K > 0)
        L.total = L.tk + kTkMiscBytes + 256 * 8 + (size_t(4) * K * decode_tk_keys(s, M) + kTkSpare) * 8 +
                  (size_t(K) * decode_nv((int)M) * kVB + kTkSpare) * 8;
    return L;
}

typedef void (*DecodeKernel)(DecodeArgs);

template <DecodeKernel K>
static bool scratch_free() // asked once per instance
{
    static const bool ok = [] {
        hipFuncAttributes fa;
        return hipFuncGetAttributes(&fa, (const void *)K) == hipSuccess && fa.localSizeBytes == 0;
    }();
    return ok;
}

// The kernel instance for (M, g, mx), or null when the shape is outside the
// single-launch path.  Instances are used only where they were compiled
// without scratch (private) memory: their timing assumes no spill traffic
// on the vector-memory counter, and the larger-M instances that would need
// it are not offered.
static DecodeKernel decode_kernel(const DevHead &h, int64_t M, bool mx)
{
    // residual pairs and low-rank pairs each come in even counts (n_lr is a
    // multiple of 4 by construction); the matrix-core variant folds one
    // g = 128 group per K-chunk
    if (M < 1 || M > kDecodeMaxM || h.s.nkc() % 4 != 0 || decode_lds(h.s, M).total > 159 * 1024)
        return nullptr;
    const bool g128 = h.s.g == 4 * kKStep;
    if (mx) {
        if (g128 && M == 1 && scratch_free<gemv_decode_kernel<1, 4, true>>())
            return gemv_decode_kernel<1, 4, true>;
        return nullptr;
    }
    if (M == 1) {
        if (g128)
            return scratch_free<gemv_decode_kernel<1, 4, false>>() ? gemv_decode_kernel<1, 4, false> : nullptr;
        return scratch_free<gemv_decode_kernel<1, 0, false>>() ? gemv_decode_kernel<1, 0, false> : nullptr;
    }
    // M = 2 only with g = 128 (the general-g instance needs scratch memory)
    if (g128)
        return scratch_free<gemv_decode_kernel<2, 4, false>>() ? gemv_decode_kernel<2, 4, false> : nullptr;
    return nullptr;
}

bool decode_ok(const DevHead &h, int64_t M, bool mx) { return decode_kernel(h, M, mx) != nullptr; }

bool decode_topk_ok(const DevHead &h, int64_t M, bool mx)
{
    return decode_ok(h, M, mx) && decode_tk_keys(h.s, M) <= kTkKeys &&
           decode_lds(h.s, M, 16).total <= 72 * 1024; // two workgroups per compute unit
}

int64_t decode_topk_keys(const Shape &s) { return int64_t(kDecodeMaxM) * ((s.nvb() + 15) / 16) * 16; }

hipError_t launch_decode(const DevHead &h, const Work &w, const uint16_t *X, float *logits, int32_t *argmax,
                         float *lse, float *nll, bool mx, hipStream_t st, const DecodeTopk *tk)
{
    const DecodeKernel kern = decode_kernel(h, w.M, mx);
    if (!kern)
        return hipErrorInvalidValue;
    const int K = tk ? tk->K : 0;
    if (tk && (K < 1 || K > kTopKMax || !decode_topk_ok(h, w.M, mx)))
        return hipErrorInvalidValue;
    const DecodeLds L = decode_lds(h.s, w.M, K);
    DecodeArgs a;
    a.h = h;
    a.w = w;
    a.X = X;
    a.logits = logits;
    a.argmax = argmax;
    a.lse = lse;
    a.nll = nll;
    a.nvb = h.s.nvb();
    a.nkc = h.s.nkc();
    a.G = h.s.G();
    a.na = h.s.lr_na();
    a.nlr = (h.s.k + h.s.r) > 0 ? h.s.n_lr() : 0;
    a.gsteps = (int)(h.s.g / kKStep);
    a.ntask = (int)(h.s.k + h.s.r);
    const int nv = decode_nv((int)w.M);
    a.nwg = (int)((a.nvb + 4 * nv - 1) / (4 * nv));
    // projection-only workgroups take the slots the streaming ones leave
    // free (two workgroups per CU), at least one column per wave
    const int64_t spare = int64_t(2) * h.n_cu - a.nwg;
    a.ntwg = spare > 0 ? (int)std::min<int64_t>(spare, (a.ntask + 3) / 4) : 0;
    if (w.want_lse && (!lse || int64_t(a.nwg) * w.M > w.part_cap))
        return hipErrorInvalidValue; // the summaries do not fit the workspace
    a.lds_sa = L.sa;
    a.lds_x = L.x;
    a.lds_ts = L.ts;
    a.lds_xs = L.xs;
    a.lds_tk = L.tk;
    a.tk_K = K;
    a.tk_L = K ? decode_tk_keys(h.s, w.M) : 0;
    a.tkw = w.tkp;
    a.tk_vals = tk ? tk->values : nullptr;
    a.tk_idx = tk ? tk->indices : nullptr;
    a.tk_u = tk ? tk->u : nullptr;
    a.tk_scale = tk ? tk->scale : 0.f;
    a.tk_samples = tk ? tk->samples : nullptr;
    if (K && w.M * int64_t(a.nwg) * 4 > w.tkp_cap)
        return hipErrorInvalidValue; // the waves' keys do not fit the workspace
    if (L.total > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)L.total);
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)(a.ntwg + a.nwg)), dim3(256), L.total, st, a);
    return hipGetLastError();
}

} // namespace archead
