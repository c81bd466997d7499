// decode.hip -- the whole packed ARCHead forward for M <= 4 in one launch,
// with VALU dot products (bf16 pairs into fp32).
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
// a1 runs inside the same launch: the first k + r waves of the grid each
// take one column of t or s (claimed through a counter) and publish it with
// a release increment of a second counter; a wave reads t and s only after
// that counter reaches k + r, which it first helps along by claiming any
// column still unclaimed, so no wave ever waits on a wave that has not
// started.  The residual needs none of it, so the projection has long
// finished when the first low-rank chunk arrives.
//
// a3 runs inside it too: each workgroup folds its top-1 keys into one 64-bit
// atomic max per row, and the workgroup that finishes last turns the keys
// into indices and zeroes the keys and the counters for the next call.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "kernels.hpp"

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

// s_waitcnt vmcnt(0): every vector memory access of the wave, stores and
// atomics included, has completed
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

constexpr int kDmaDevice = 16; // cache-policy operand of global_load_lds: sc1, device scope

constexpr uint32_t kBf16Neg136 = 0xC308C308u; // bf16 pair (-136, -136)
constexpr uint32_t kBf16Neg144 = 0xC310C310u; // bf16 pair (-144, -144)

struct DecodeArgs {
    DevHead h;
    Work w;
    const uint16_t *X;
    float *logits;   // M x V, may be null
    int32_t *argmax; // M, may be null
    int64_t nvb, nkc, G, na, nlr;
    int gsteps;
    int ntask;       // k + r projection columns
    int nwg;         // workgroups in the grid
    unsigned lds_x, lds_ts; // byte offsets of the X and t/s regions (sr at 0)
};

// v-blocks per wave: five while the accumulators of MF rows leave room for
// two prefetch pairs at two waves per SIMD, fewer above
constexpr int decode_nv(int MF) { return MF <= 2 ? 5 : 3; }

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
//   x   [MF][d]              bf16  the hidden states
//   ts  [4 waves] x { t hi [MF][kpad], t lo [MF][kpad], s hi [MF][rpad], s lo [MF][rpad] }  bf16
template <int MF, int GS>
__global__ __launch_bounds__(256, 2) void gemv_decode_kernel(DecodeArgs a)
{
    constexpr int NV = decode_nv(MF);
    extern __shared__ __attribute__((aligned(16))) char smem[];
    __shared__ uint64_t red[4][MF];
    __shared__ int s_last;
    const uint16_t *s_sr = (const uint16_t *)smem;
    const uint16_t *s_x = (const uint16_t *)(smem + a.lds_x);

    const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nvb = a.nvb, nkc = a.nkc, G = a.G, na = a.na, nlr = a.nlr;
    const int64_t d = a.h.s.d, V = a.h.s.V, k = a.h.s.k;
    const int64_t kst = a.h.s.kst(), rst = a.h.s.rst(), kpad = a.h.s.kpad(), rpad = a.h.s.rpad();
    const int gsteps = GS ? GS : a.gsteps;
    const int64_t wg_vb0 = (int64_t)blockIdx.x * 4 * NV;
    const int64_t vb0 = wg_vb0 + wv * NV;
    uint16_t *s_ts = (uint16_t *)(smem + a.lds_ts) + wv * (2 * MF * (kpad + rpad));
    uint32_t *claimed = a.w.sync, *finished = a.w.sync + 1, *wg_done = a.w.sync + 2;

    int64_t vb[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v)
        vb[v] = vb0 + v < nvb ? vb0 + v : nvb - 1;

    // ---- a1: one column of t or s per task, for every row m ----
    auto claim = [&]() __attribute__((always_inline)) -> int {
        uint32_t t = 0;
        if (lane == 0)
            t = __hip_atomic_fetch_add(claimed, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return (int)__builtin_amdgcn_readfirstlane(t);
    };
    auto run_task = [&](int i) __attribute__((always_inline)) {
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
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int64_t j0 = j00 + 1024 * it + 16 * lane;
                const bool ok = j0 < d;
                wq[it] = ok ? *(const u32x4 *)(row + j0) : z;
                sc[it] = (ok && isd) ? a.h.sd[c * G + j0 / a.h.s.g] : 1.0f;
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
        for (int m = 0; m < MF; ++m)
            for (int off = 32; off >= 1; off >>= 1)
                acc[m] += __shfl_xor(acc[m], off);
        const int64_t Mp = a.w.Mp;
#pragma unroll
        for (int m = 0; m < MF; ++m)
            if (lane == m) {
                const float t = isd ? acc[m] : acc[m] * a.h.sb[c];
                const uint16_t hi = f32_to_bf16_rne(t);
                const uint16_t lo = f32_to_bf16_rne(t - __uint_as_float((uint32_t)hi << 16));
                uint16_t *ph = isd ? a.w.s16 + m * rpad + c : a.w.t16 + m * kpad + c;
                uint16_t *pl = isd ? a.w.s16 + (Mp + m) * rpad + c : a.w.t16 + (Mp + m) * kpad + c;
                store_device(ph, hi);
                store_device(pl, lo);
            }
        // publish: the device-scope stores have completed before the count
        // goes up (no cache write-back needed: they went to the device's
        // coherence point)
        wait_vm_all();
        if (lane == 0)
            __hip_atomic_fetch_add(finished, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };

    // wave-level direct-to-LDS copy of n16 16-byte pieces, read at device
    // scope (the data were written by other workgroups of this launch)
    auto wave_dma16 = [&](const void *src, void *dst, int64_t n16) __attribute__((always_inline)) {
        for (int64_t i0 = 0; i0 < n16; i0 += 64) {
            const int64_t i = i0 + lane;
            if (i < n16)
                __builtin_amdgcn_global_load_lds((const void *)((const u32x4 *)src + i),
                                                 (__attribute__((address_space(3))) void *)((u32x4 *)dst + i0), 16, 0,
                                                 kDmaDevice);
        }
    };
    // t and s of the MF rows into this wave's LDS region, once every column
    // is published.  Every column was claimed at the start by a running wave
    // that computes it before it waits for anything, so the wait ends.
    // The wait is bounded all the same (about 2^20 x 128 clocks, far beyond
    // any projection), so that a launch always ends: if the counters were
    // ever left inconsistent, the logits come out wrong instead.
    auto wait_and_stage_ts = [&]() __attribute__((always_inline)) {
        const uint32_t need = (uint32_t)a.ntask;
        for (int spin = 0; spin < (1 << 20); ++spin) {
            if (__hip_atomic_load(finished, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= need)
                break;
            __builtin_amdgcn_s_sleep(2);
        }
        const int64_t Mp = a.w.Mp;
        wave_dma16(a.w.t16, s_ts, MF * kpad / 8);
        wave_dma16(a.w.t16 + Mp * kpad, s_ts + MF * kpad, MF * kpad / 8);
        wave_dma16(a.w.s16, s_ts + 2 * MF * kpad, MF * rpad / 8);
        wave_dma16(a.w.s16 + Mp * rpad, s_ts + 2 * MF * kpad + MF * rpad, MF * rpad / 8);
        // the copies must land before the first LDS read of t and s; the
        // compiler's own tracking of direct-to-LDS copies does not cover
        // every read of the region, so wait here explicitly
        wait_vm_all();
    };

    // ---- chunk stream: residual chunks 0 .. nkc-1, then the low-rank chunks ----
    const int64_t ntot = nkc + nlr, npairs = (ntot + 1) / 2;
    const u32x4 *lrp = (const u32x4 *)a.h.lr;
    const u32x4 *r4p = (const u32x4 *)a.h.r4;
    auto load_chunk = [&](DChunk<NV> &c, int64_t ci) __attribute__((always_inline)) {
        const u32x4 *base = ci < nkc ? r4p + ci * nvb * 64 : lrp + (ci - nkc) * nvb * 64;
#pragma unroll
        for (int v = 0; v < NV; ++v)
            c.q[v] = __builtin_nontemporal_load(&base[vb[v] * 64 + lane]);
    };
    auto load_pair = [&](DPair<NV> &p, int64_t pi) __attribute__((always_inline)) { // pi < npairs
        load_chunk(p.h0, 2 * pi);
        load_chunk(p.h1, 2 * pi + 1);
    };

    // projection columns: wave gw takes one claim for each of the indices
    // gw, gw + nw, gw + 2 nw, ... below k + r (nw waves in the grid), so the
    // grid makes exactly k + r claims, all at its start, and every column is
    // claimed by a wave that is running
    const int64_t gw = (int64_t)blockIdx.x * 4 + wv, nw = (int64_t)a.nwg * 4;
    const int ntask_here = gw < a.ntask ? (int)((a.ntask - 1 - gw) / nw + 1) : 0;
    int task = ntask_here > 0 ? claim() : a.ntask;

    DPair<NV> P0, P1;
    load_pair(P0, 0);
    load_pair(P1, 1);
    {   // residual scales and X into LDS
        const int64_t nvb_wg = (nvb - wg_vb0) < 4 * NV ? (nvb - wg_vb0) : 4 * NV;
        const int64_t nsr = nvb_wg * G * kVB / 8, nx = MF * d / 8;
        for (int64_t i0 = 0; i0 < nsr; i0 += 256) {
            const int64_t i = i0 + threadIdx.x;
            if (i < nsr)
                __builtin_amdgcn_global_load_lds((const void *)((const u32x4 *)(a.h.sr + wg_vb0 * G * kVB) + i),
                                                 (__attribute__((address_space(3))) void *)((u32x4 *)smem + i0 + wv * 64), 16, 0, 0);
        }
        for (int64_t i0 = 0; i0 < nx; i0 += 256) {
            const int64_t i = i0 + threadIdx.x;
            if (i < nx)
                __builtin_amdgcn_global_load_lds((const void *)((const u32x4 *)a.X + i),
                                                 (__attribute__((address_space(3))) void *)((u32x4 *)(smem + a.lds_x) + i0 + wv * 64), 16, 0, 0);
        }
    }
    __syncthreads();
    for (int j = 0; j < ntask_here; ++j) {
        if (j > 0)
            task = claim();
        if (task < a.ntask) // always true while the counters start at zero
            run_task(task);
    }

    // per-lane partial sums over the lane's columns
    float tot[NV][MF], g[NV][MF], xn[MF], ga[NV][MF], gc[NV][MF], nt[MF];
#pragma unroll
    for (int m = 0; m < MF; ++m) {
        xn[m] = nt[m] = 0.f;
#pragma unroll
        for (int v = 0; v < NV; ++v)
            tot[v][m] = g[v][m] = ga[v][m] = gc[v][m] = 0.f;
    }
    const uint32_t kMagic = vgpr_const(kBf16Magic);
    const uint32_t c136 = vgpr_const(kBf16Neg136), c144 = vgpr_const(kBf16Neg144);

    // residual chunk kc: 4 K-steps; each g-group is folded with its scale
    // when it ends: tot += sR (sum x (q + 136) - 136 sum x)
    auto res_chunk = [&](const DChunk<NV> &c, int64_t kc) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int64_t ks = kc * 4 + s;
            u32x4 x[MF];
#pragma unroll
            for (int m = 0; m < MF; ++m) {
                x[m] = *(const u32x4 *)(s_x + m * d + ks * kKStep + 8 * lq);
                xn[m] = dot8c(x[m], c136, xn[m]);
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
                        tot[v][m] = __builtin_fmaf(scl, g[v][m] + xn[m], tot[v][m]);
                        g[v][m] = 0.f;
                    }
                }
#pragma unroll
                for (int m = 0; m < MF; ++m)
                    xn[m] = 0.f;
            }
            // one K-step at a time: the dequantised codes of later K-steps
            // are not hoisted into registers early
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // low-rank chunk j: three core K-steps (A5 + 16 against t) or two
    // correction K-steps (C8 against s); K-steps beyond the rank are skipped
    const uint16_t *s_t = s_ts, *s_s = s_ts + 2 * MF * kpad;
    auto lr_chunk = [&](const DChunk<NV> &c, int64_t j) __attribute__((always_inline)) {
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
                    nt[m] = dot8c(tl[m], c144, dot8c(th[m], c144, nt[m]));
                }
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    const uint32_t wn = q == 0 ? c.q[v].x : q == 1 ? c.q[v].y : c.q[v].z;
                    const u32x4 b = a5_bf16_q(wn, c.q[v].w, q);
#pragma unroll
                    for (int m = 0; m < MF; ++m)
                        ga[v][m] = dot8(tl[m], b, dot8(th[m], b, ga[v][m]));
                }
                __builtin_amdgcn_sched_barrier(0);
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
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    // residual pairs (nkc / 2 of them, an even count), then the low-rank
    // pairs (nlr / 2, also even); the loads of the last residual pairs
    // already fetch the first low-rank chunks.  The last iteration issues no
    // loads (no load sits under a branch, which would make the compiler copy
    // the prefetch buffers).
    const int64_t nrp = nkc / 2;
    auto res_iter = [&](int64_t pi, bool load) __attribute__((always_inline)) {
        res_chunk(P0.h0, 2 * pi);
        res_chunk(P0.h1, 2 * pi + 1);
        if (load)
            load_pair(P0, pi + 2);
        __builtin_amdgcn_sched_barrier(0);
        res_chunk(P1.h0, 2 * pi + 2);
        res_chunk(P1.h1, 2 * pi + 3);
        if (load)
            load_pair(P1, pi + 3);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto lr_iter = [&](int64_t pi, bool load) __attribute__((always_inline)) {
        lr_chunk(P0.h0, 2 * pi - nkc);
        lr_chunk(P0.h1, 2 * pi + 1 - nkc);
        if (load)
            load_pair(P0, pi + 2);
        __builtin_amdgcn_sched_barrier(0);
        lr_chunk(P1.h0, 2 * pi + 2 - nkc);
        lr_chunk(P1.h1, 2 * pi + 3 - nkc);
        if (load)
            load_pair(P1, pi + 3);
        __builtin_amdgcn_sched_barrier(0);
    };
    int64_t pi = 0;
    for (; pi + 2 < npairs; pi += 2) {
        if (pi >= nrp)
            break;
        res_iter(pi, true);
    }
    if (nlr == 0) {
        res_iter(pi, false);
    } else {
        wait_and_stage_ts();
        for (; pi + 2 < npairs; pi += 2)
            lr_iter(pi, true);
        lr_iter(pi, false);
    }

    // ---- logits: the four lanes of a row add their partial sums ----
    float sa[NV], sc[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        sa[v] = h2f(a.h.sa[vb[v] * kVB + lr]);
        sc[v] = h2f(a.h.sc[vb[v] * kVB + lr]);
    }
    uint64_t key[MF];
#pragma unroll
    for (int m = 0; m < MF; ++m)
        key[m] = 0;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int64_t row = vb0 + v < nvb ? (vb0 + v) * kVB + lr : V;
#pragma unroll
        for (int m = 0; m < MF; ++m) {
            float y = __builtin_fmaf(sa[v], ga[v][m] + nt[m], __builtin_fmaf(sc[v], gc[v][m], tot[v][m]));
            y += __shfl_xor(y, 16);
            y += __shfl_xor(y, 32);
            if (row < V) {
                if (a.logits && lq == 0)
                    a.logits[m * V + row] = y;
                key[m] = umax64(key[m], argmax_key(y, (uint32_t)row));
            }
        }
    }

    // ---- a3: workgroup maximum per row, then one atomic max per row ----
    if (a.argmax) {
#pragma unroll
        for (int m = 0; m < MF; ++m) {
            uint64_t kk = key[m];
            kk = umax64(kk, shfl_xor_u64(kk, 1));
            kk = umax64(kk, shfl_xor_u64(kk, 2));
            kk = umax64(kk, shfl_xor_u64(kk, 4));
            kk = umax64(kk, shfl_xor_u64(kk, 8));
            if (lane == 0)
                red[wv][m] = kk;
        }
        __syncthreads();
        if (threadIdx.x < MF) {
            const int m = threadIdx.x;
            const uint64_t kk = umax64(umax64(red[0][m], red[1][m]), umax64(red[2][m], red[3][m]));
            __hip_atomic_fetch_max(a.w.keys + m, kk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    // the last workgroup to finish resolves the keys and resets the counters;
    // the barrier waits for the key updates (device-scope atomics) to complete
    // before the workgroup counts itself done
    __syncthreads();
    if (threadIdx.x == 0)
        s_last = __hip_atomic_fetch_add(wg_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 (uint32_t)(a.nwg - 1);
    __syncthreads();
    if (s_last) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        if (a.argmax && threadIdx.x < MF) {
            const uint64_t kk = __hip_atomic_exchange(a.w.keys + threadIdx.x, (uint64_t)0, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
            a.argmax[threadIdx.x] = (int32_t)(0xFFFFFFFFu - (uint32_t)kk);
        }
        if (threadIdx.x == 0) {
            __hip_atomic_store(claimed, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(finished, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(wg_done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
static size_t dal16(size_t x) { return (x + 15) / 16 * 16; }

struct DecodeLds {
    unsigned x, ts;
    size_t total;
};

static DecodeLds decode_lds(const Shape &s, int64_t M)
{
    DecodeLds L;
    L.x = (unsigned)dal16(size_t(4) * decode_nv((int)M) * s.G() * kVB * 2);
    L.ts = (unsigned)(L.x + dal16(size_t(M) * s.d * 2));
    L.total = L.ts + size_t(4) * 2 * M * (s.kpad() + s.rpad()) * 2;
    return L;
}

bool gemv_decode_ok(const DevHead &h, int64_t M)
{
    // residual pairs and low-rank pairs each come in even counts (n_lr is a
    // multiple of 4 by construction)
    return M >= 1 && M <= kDecodeMaxM && h.s.nkc() % 4 == 0 && decode_lds(h.s, M).total <= 159 * 1024;
}

template <int MF>
static hipError_t launch_mf(const DecodeArgs &a, size_t lds, hipStream_t st)
{
    auto kern = a.gsteps == 4 ? gemv_decode_kernel<MF, 4> : gemv_decode_kernel<MF, 0>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)a.nwg), dim3(256), lds, st, a);
    return hipGetLastError();
}

hipError_t launch_gemv_decode(const DevHead &h, const Work &w, const uint16_t *X, float *logits,
                              int32_t *argmax, hipStream_t st)
{
    if (!gemv_decode_ok(h, w.M))
        return hipErrorInvalidValue;
    const DecodeLds L = decode_lds(h.s, w.M);
    DecodeArgs a;
    a.h = h;
    a.w = w;
    a.X = X;
    a.logits = logits;
    a.argmax = argmax;
    a.nvb = h.s.nvb();
    a.nkc = h.s.nkc();
    a.G = h.s.G();
    a.na = h.s.lr_na();
    a.nlr = (h.s.k + h.s.r) > 0 ? h.s.n_lr() : 0;
    a.gsteps = (int)(h.s.g / kKStep);
    a.ntask = (int)(h.s.k + h.s.r);
    const int nv = decode_nv((int)w.M);
    a.nwg = (int)((a.nvb + 4 * nv - 1) / (4 * nv));
    a.lds_x = L.x;
    a.lds_ts = L.ts;
    switch (w.M) {
    case 1: return launch_mf<1>(a, L.total, st);
    case 2: return launch_mf<2>(a, L.total, st);
    case 3: return launch_mf<3>(a, L.total, st);
    default: return launch_mf<4>(a, L.total, st);
    }
}

} // namespace archead
