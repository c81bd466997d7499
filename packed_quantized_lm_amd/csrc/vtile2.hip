// vtile2.hip -- the vocabulary-tile step for batched decode (2 <= M <= 32,
// g = 128): a persistent streaming kernel with the hidden states staged in
// LDS, all at once where they fit, else slab by slab.
//
// ARCHead paper, section 3.2, eq 7 with W_d from eq 3 and the INT8 factors
// of the text after eq 7.  Per vocabulary row v and hidden state m:
//   logits[m,v] = sA[v] sum_i A5[v,i] t[m,i] + sC[v] sum_i C8[v,i] s[m,i]
//               + sum_grp sR[v,grp] sum_{j in grp} X[m,j] R4[v,j]
// with t = X (sB o B8)^T and s = X (sD o D8)^T from the projection kernel.
//
// One workgroup of 8 waves per compute unit; the grid's waves split the
// v-blocks (16 vocabulary rows each) into equal contiguous ranges, which a
// wave streams in groups of NV v-blocks: per group the low-rank chunks, then
// the residual K-chunks (the chunk stream of layout.hpp), with NB = 4 chunks
// in flight and the stream running on from one group into the next.
//
// The products are v_mfma_f32_16x16x32_bf16 with 16 hidden states as the A
// operand and a v-block's 16 rows as the B operand (codes spliced into exact
// bf16 integers, device.hpp).  The A operands -- X, and the bf16 hi/lo parts
// of t and s -- are read from LDS, where they sit in MFMA fragment order (one
// 1 KiB block per 16 rows x 32 columns: lane l's 16 bytes at 16 l), so the
// reads are free of bank conflicts.  t and s, and the workgroup's residual
// and row scales, are staged once.  Where all of
// X fits beside them (one m-tile and d up to about 2560), X is staged once
// too and the stream has no barrier; otherwise X is staged in slabs of four
// K-chunks (512 columns), two slab buffers, the next slab's copy issued by
// the eight waves together after their first chunk of the current slab and
// checked at the slab boundary by one wait (three chunks' loads were issued
// after it) and one barrier.  The only other vector-memory loads of the loop
// are the packed codes.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "kernels.hpp"

namespace archead {

namespace {

constexpr int kS2Waves = 8;  // waves per workgroup, one workgroup per compute unit
constexpr int kS2Slab = 4;   // residual K-chunks per X slab
constexpr int kS2NB = 4;     // chunks in flight per wave
constexpr int kS2MaxM = 32;
// dynamic LDS of a workgroup: 160 KiB less the kernel's static arrays (at
// most 4.3 KiB at two m-tiles) and a margin
constexpr size_t kS2Lds = 154 * 1024;

struct Stream2Args {
    DevHead h;
    Work w;
    const uint16_t *X;
    float *logits; // M x V, may be null
    int want_argmax;
    int64_t nvb, nkc, G, na, nlr, kst, rst, kpad, rpad;
    int64_t nlr_used; // low-rank chunks that carry K-steps (>= 1 when nlr > 0)
    int ngroups;   // groups of NV v-blocks per wave
    int n_slab;    // X slabs per group (nkc / kS2Slab)
    unsigned lds_x, lds_ts, lds_xs, lds_sr, lds_sa; // byte offsets of the LDS regions
};

// v-block range [lo, hi) of wave gw of W
__device__ __forceinline__ int64_t wave_lo(int64_t gw, int64_t W, int64_t nvb) { return gw * nvb / W; }

// XF: all of X staged once (when it fits in LDS next to the rest), so the
// stream needs no barrier; otherwise slab by slab in two buffers.
template <int MT, int NV, bool XF>
__global__ __launch_bounds__(kS2Waves * 64, 1) void vtile_stream2_kernel(Stream2Args a)
{
    extern __shared__ __attribute__((aligned(16))) char smem[];
    __shared__ uint64_t red[kS2Waves][MT * 16];
    __shared__ LsePart lred[kS2Waves][MT * 16];
    __shared__ int32_t s_tgt[64];
    uint16_t *const s_x = (uint16_t *)(smem + a.lds_x);   // [2][MT][16][64][8] bf16 (XF: [MT][d / 32][64][8])
    uint16_t *const s_ts = (uint16_t *)(smem + a.lds_ts); // t [MT][kst][2][64][8], then s [MT][rst][2][64][8]
    float *const s_xs = (float *)(smem + a.lds_xs);       // [G][MT*16]  -136 sum of X over the group
    uint16_t *const s_sr = (uint16_t *)(smem + a.lds_sr); // [v-blocks of the workgroup][G][16] fp16
    uint16_t *const s_sa = (uint16_t *)(smem + a.lds_sa); // [v-blocks of the workgroup][16] sA, then the same for sC

    const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nvb = a.nvb, nkc = a.nkc, G = a.G, na = a.na, nlr = a.nlr;
    const int64_t kst = a.kst, rst = a.rst, kpad = a.kpad, rpad = a.rpad;
    const int64_t M = a.w.M, Mp = a.w.Mp, d = a.h.s.d, V = a.h.s.V;
    const int ngroups = a.ngroups, n_slab = a.n_slab;
    const int64_t W = (int64_t)gridDim.x * kS2Waves;
    const int64_t gw = (int64_t)blockIdx.x * kS2Waves + wv;
    const int64_t lo = wave_lo(gw, W, nvb), hi = wave_lo(gw + 1, W, nvb);
    const int64_t wg_lo = wave_lo((int64_t)blockIdx.x * kS2Waves, W, nvb);
    const int64_t wg_hi = wave_lo((int64_t)blockIdx.x * kS2Waves + kS2Waves, W, nvb);
    // a slot past the wave's range streams the range's last v-block again
    // (or, for an empty range, a v-block of the workgroup) and stores nothing
    const int64_t vlast = hi > lo ? hi - 1 : (wg_hi > wg_lo ? wg_hi - 1 : (lo < nvb ? lo : nvb - 1));
    auto vblock = [&](int64_t j, int v) -> int64_t {
        const int64_t b = lo + j * NV + v;
        return b < hi ? b : vlast;
    };

    // ---- staging: issued before the first prefetches, checked once ----
    {
        // residual scales of the workgroup's v-blocks (contiguous)
        const int64_t nsr = (wg_hi > wg_lo ? wg_hi - wg_lo : 0) * G * kVB / 8;
        const u32x4 *src = (const u32x4 *)(a.h.sr + wg_lo * G * kVB);
        for (int64_t i0 = wv * 64; i0 < nsr; i0 += kS2Waves * 64)
            if (i0 + lane < nsr)
                lds_dma16<false>(src + i0 + lane, (u32x4 *)s_sr + i0);
        // the rows' sA and sC, read at each group's start: from LDS, a read
        // there waits for no chunk load in flight
        const int64_t nsa = (wg_hi - wg_lo) * kVB / 8; // 16-byte pieces of each
        const u32x4 *sa_src = (const u32x4 *)(a.h.sa + wg_lo * kVB);
        const u32x4 *sc_src = (const u32x4 *)(a.h.sc + wg_lo * kVB);
        for (int64_t i0 = wv * 64; i0 < 2 * nsa; i0 += kS2Waves * 64) {
            const int64_t i = i0 + lane;
            if (i < 2 * nsa)
                lds_dma16<false>(i < nsa ? sa_src + i : sc_src + (i - nsa), (u32x4 *)s_sa + i0);
        }
        // -136 sum of X per group: xs[grp][j] = xsneg[grp][j]
        const int64_t nxs = G * MT * 16;
        for (int64_t i0 = wv * 64; i0 < nxs; i0 += kS2Waves * 64) {
            const int64_t i = i0 + lane < nxs ? i0 + lane : nxs - 1;
            lds_dma4(a.w.xsneg + (i / (MT * 16)) * Mp + i % (MT * 16), s_xs + i0);
        }
        if (a.w.want_lse && a.w.targets && wv == 0) // rows past M repeat the last target
            lds_dma4(a.w.targets + (lane < M ? lane : M - 1), s_tgt);
        // t and s in fragment order: block (mt, ks, half) takes rows
        // 16 mt + l % 16 (clamped below M) and columns 32 ks + 8 (l / 16) ..
        const int64_t ntb = MT * kst * 2, nsb = MT * rst * 2;
        for (int64_t b = wv; b < ntb + nsb; b += kS2Waves) {
            const bool ist = b < ntb;
            const int64_t bb = ist ? b : b - ntb, ksn = ist ? kst : rst, pitch = ist ? kpad : rpad;
            const int64_t mt = bb / (ksn * 2), ks = (bb / 2) % ksn, h = bb % 2;
            const int64_t r = mt * 16 + lr < M ? mt * 16 + lr : M - 1;
            const uint16_t *base = ist ? a.w.t16 : a.w.s16;
            lds_dma16<false>(base + (h * Mp + r) * pitch + ks * kKStep + 8 * lq, s_ts + b * 512);
        }
    }
    // X slab S (of every group's slabs in turn) into buffer S % 2: block
    // (mt, kl) of K-step 16 (S mod n_slab) + kl
    auto copy_slab = [&](int64_t S) __attribute__((always_inline)) {
        const int64_t sl = S % n_slab;
        uint16_t *dst = s_x + (S & 1) * (MT * 16 * 512);
#pragma unroll
        for (int q = 0; q < MT * 16 / kS2Waves; ++q) {
            const int b = wv + kS2Waves * q, mt = b / 16, kl = b % 16;
            const int64_t r = mt * 16 + lr < M ? mt * 16 + lr : M - 1;
            lds_dma16<false>(a.X + r * d + (sl * 16 + kl) * kKStep + 8 * lq, dst + b * 512);
        }
    };
    const int64_t nks = d / kKStep;
    if constexpr (XF) {
        // every K-step block of every m-tile, once: block b = mt nks + ks
        for (int64_t b = wv; b < MT * nks; b += kS2Waves) {
            const int64_t mt = b / nks, ks = b - (b / nks) * nks;
            const int64_t r = mt * 16 + lr < M ? mt * 16 + lr : M - 1;
            lds_dma16<false>(a.X + r * d + ks * kKStep + 8 * lq, s_x + b * 512);
        }
    } else {
        copy_slab(0);
    }

    // ---- the chunk stream: item it = (group it / per, chunk it % per) ----
    const int64_t per = nlr + nkc; // a multiple of kS2NB
    const u32x4 *lrp = (const u32x4 *)a.h.lr;
    const u32x4 *r4p = (const u32x4 *)a.h.r4;
    u32x4 buf[kS2NB][NV];
    // the low-rank chunks that carry K-steps; those past them pad the stream
    // to a multiple of kS2NB and are never used: their slot reads the last
    // used low-rank chunk again (same v-blocks, just read: a cache hit), so
    // that every item still issues NV loads
    const int64_t nlr_used = a.nlr_used;
    auto load_item = [&](u32x4(&q)[NV], int64_t j, int64_t c) __attribute__((always_inline)) {
        if (j >= ngroups) { // past the end: the last item again (never used)
            j = ngroups - 1;
            c = per - 1;
        }
        const int64_t cl = c < nlr_used ? c : nlr_used - 1;
        const u32x4 *base = c < nlr ? lrp + cl * nvb * 64 : r4p + (c - nlr) * nvb * 64;
#pragma unroll
        for (int v = 0; v < NV; ++v)
            q[v] = __builtin_nontemporal_load(&base[vblock(j, v) * 64 + lane]);
    };
#pragma unroll
    for (int b = 0; b < kS2NB; ++b)
        load_item(buf[b], b / per, b % per);
    // this wave's staging copies have landed once at most its prefetches
    // are outstanding; after the barrier, every wave's have
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(kS2NB * NV));
    __syncthreads();

    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const uint32_t kMagic = vgpr_const(kBf16Magic);
    const u32x4 neg144 = {0xC310C310u, 0xC310C310u, 0xC310C310u, 0xC310C310u}; // bf16 -144
    auto tfrag = [&](int mt, int64_t ks, int h) -> u32x4 {
        return *(const u32x4 *)(s_ts + (((mt * kst + ks) * 2 + h) * 64 + lane) * 8);
    };
    auto sfrag = [&](int mt, int64_t ks, int h) -> u32x4 {
        return *(const u32x4 *)(s_ts + MT * kst * 1024 + (((mt * rst + ks) * 2 + h) * 64 + lane) * 8);
    };
    // this wave's running top-1 key and (max, sum exp) per hidden state, in
    // LDS (the wave's own entries: no barrier), merged group by group
    for (int i = lane; i < MT * 16; i += 64) {
        red[wv][i] = 0;
        lred[wv][i] = LsePart{-__builtin_inff(), 0.f};
    }

    f32x4 acc[NV][MT];
    int64_t jn = kS2NB / per, cn = kS2NB % per; // the next item to load
    auto advance = [&]() __attribute__((always_inline)) {
        if (++cn == per) {
            cn = 0;
            ++jn;
        }
    };

    for (int64_t j = 0; j < ngroups; ++j) {
        int64_t vb[NV];
        float sa[NV], sc[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            vb[v] = vblock(j, v);
            sa[v] = h2f(s_sa[(vb[v] - wg_lo) * kVB + lr]);
            sc[v] = h2f(s_sa[(wg_hi - wg_lo + vb[v] - wg_lo) * kVB + lr]);
        }

        // low-rank chunks: three core K-steps (A5 against t) or two
        // correction K-steps (C8 against s); K-steps beyond the rank are
        // skipped.  Each chunk's sums are folded into acc with the row's
        // scale (sA or sC) at the chunk's end, in passes of NH v-blocks: one
        // chunk's sums and acc are all the low-rank phase holds besides the
        // chunk buffers.
        constexpr int NH = (MT == 2 && NV > 4) ? 3 : NV;
        {
            // acc starts at sA (-144 sum_i t[m, i]): the core codes are a + 144
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                f32x4 nt = zero;
                for (int64_t ks = 0; ks < kst; ++ks) {
                    nt = mfma_bf16(tfrag(mt, ks, 0), neg144, nt);
                    nt = mfma_bf16(tfrag(mt, ks, 1), neg144, nt);
                }
#pragma unroll
                for (int v = 0; v < NV; ++v)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[v][mt][i] = sa[v] * nt[i];
            }
            auto lr_chunk = [&](const u32x4(&q)[NV], int64_t c) __attribute__((always_inline)) {
                const bool core = c < na;
                // a correction chunk past the rank (the stream's padding) has no K-step
                if (!core && 2 * (c - na) >= rst)
                    return;
#pragma unroll
                for (int v0 = 0; v0 < NV; v0 += NH) {
                    const int vn = v0 + NH < NV ? v0 + NH : NV;
                    f32x4 g[NH][MT];
                    if (core) {
#pragma unroll
                        for (int qq = 0; qq < 3; ++qq) {
                            const int64_t ks = 3 * c + qq;
                            if (ks >= kst)
                                break;
                            u32x4 th[MT], tl[MT];
#pragma unroll
                            for (int mt = 0; mt < MT; ++mt) {
                                th[mt] = tfrag(mt, ks, 0);
                                tl[mt] = tfrag(mt, ks, 1);
                            }
#pragma unroll
                            for (int v = v0; v < vn; ++v) {
                                const uint32_t wn = qq == 0 ? q[v].x : qq == 1 ? q[v].y : q[v].z;
                                const u32x4 b = a5_bf16_q(wn, q[v].w, qq);
#pragma unroll
                                for (int mt = 0; mt < MT; ++mt)
                                    g[v - v0][mt] = mfma_bf16(tl[mt], b, mfma_bf16(th[mt], b, qq == 0 ? zero : g[v - v0][mt]));
                            }
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    } else {
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh) {
                            const int64_t ks = 2 * (c - na) + hh;
                            if (ks >= rst)
                                break;
                            u32x4 sh[MT], sl[MT];
#pragma unroll
                            for (int mt = 0; mt < MT; ++mt) {
                                sh[mt] = sfrag(mt, ks, 0);
                                sl[mt] = sfrag(mt, ks, 1);
                            }
#pragma unroll
                            for (int v = v0; v < vn; ++v) {
                                u32x2 w;
                                w.x = hh == 0 ? q[v].x : q[v].z;
                                w.y = hh == 0 ? q[v].y : q[v].w;
                                const u32x4 b = c8_bf16(w);
#pragma unroll
                                for (int mt = 0; mt < MT; ++mt)
                                    g[v - v0][mt] = mfma_bf16(sl[mt], b, mfma_bf16(sh[mt], b, hh == 0 ? zero : g[v - v0][mt]));
                            }
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
#pragma unroll
                    for (int v = v0; v < vn; ++v) {
                        const float scl = core ? sa[v] : sc[v];
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                acc[v][mt][i] = __builtin_fmaf(scl, g[v - v0][mt][i], acc[v][mt][i]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
            for (int64_t c = 0; c < nlr; c += kS2NB) {
#pragma unroll
                for (int b = 0; b < kS2NB; ++b) {
                    lr_chunk(buf[b], c + b);
                    load_item(buf[b], jn, cn);
                    advance();
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }

        // residual K-chunks, slab by slab; each chunk is one g = 128 group,
        // folded with its scale: acc += sR (sum x (q + 136) - 136 sum x),
        // the group's sum starting from -136 sum x (the first product's C)
        // no load older than the chunk stream's is outstanding: said here,
        // so that no wait for one is placed in the loop
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(kS2NB * NV));
        for (int64_t s = 0; s < n_slab; ++s) {
            const int64_t S = j * n_slab + s;
            const uint16_t *xs_base;
            if constexpr (XF) {
                xs_base = s_x + s * 16 * 512; // K-step 16 s of m-tile 0 (m-tile mt: + mt nks blocks)
            } else {
                // the copy of slab S went out right after the first chunk
                // reload of the slab before it (at the start, for slab 0):
                // at least (kS2NB - 1) NV chunk loads were issued after it, so
                // with at most that many outstanding the copy has landed
                __builtin_amdgcn_s_waitcnt(waitcnt_vm((kS2NB - 1) * NV));
                __syncthreads(); // every wave's part of slab S is in; slab S - 1 is done with
                xs_base = s_x + (S & 1) * (MT * 16 * 512);
            }
#pragma unroll
            for (int b = 0; b < kS2NB; ++b) {
                const int64_t kc = s * kS2Slab + b;
                if constexpr (!XF) { // the waves behind in the slab go first
                    if (b == 0)
                        __builtin_amdgcn_s_setprio(3);
                    else if (b == 1)
                        __builtin_amdgcn_s_setprio(2);
                    else if (b == 2)
                        __builtin_amdgcn_s_setprio(1);
                    else
                        __builtin_amdgcn_s_setprio(0);
                }
                // the chunk's v-blocks in passes of NH, each with its own group sums
#pragma unroll
                for (int v0 = 0; v0 < NV; v0 += NH) {
                    const int vn = v0 + NH < NV ? v0 + NH : NV;
                    f32x4 xs[MT];
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        xs[mt] = *(const f32x4 *)(s_xs + kc * (MT * 16) + mt * 16 + 4 * lq);
                    f32x4 g[NH][MT];
#pragma unroll
                    for (int st = 0; st < 4; ++st) {
                        u32x4 xf[MT];
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt)
                            xf[mt] = *(const u32x4 *)(xs_base + (((XF ? mt * nks : mt * 16) + b * 4 + st) * 64 + lane) * 8);
#pragma unroll
                        for (int v = v0; v < vn; ++v) {
                            const uint32_t wd = st == 0 ? buf[b][v].x : st == 1 ? buf[b][v].y
                                                : st == 2 ? buf[b][v].z : buf[b][v].w;
                            const u32x4 bb = r4_bf16(wd, kMagic);
#pragma unroll
                            for (int mt = 0; mt < MT; ++mt)
                                g[v - v0][mt] = mfma_bf16(xf[mt], bb, st == 0 ? xs[mt] : g[v - v0][mt]);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    if (vn == NV) { // the chunk's codes are used up: its slot takes the next item
                        load_item(buf[b], jn, cn);
                        advance();
                        if constexpr (!XF)
                            if (b == 0 && S + 1 < (int64_t)ngroups * n_slab)
                                copy_slab(S + 1);
                    }
#pragma unroll
                    for (int v = v0; v < vn; ++v) {
                        const int64_t vrow = vb[v] - wg_lo;
                        const float scl = h2f(s_sr[(vrow * G + kc) * kVB + lr]);
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                acc[v][mt][i] = __builtin_fmaf(scl, g[v - v0][mt][i], acc[v][mt][i]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }

        // this group's logits, and its top-1 keys and (max, sum exp)
        // summaries merged into the wave's running ones.  The lane index is
        // made opaque here, so that the epilogue's per-lane addresses are
        // formed here and not kept live across the stream.
        int elane = lane;
        asm volatile("" : "+v"(elane));
        const int elr = elane & 15, elq = elane >> 4;
        float *const lgp = a.logits ? a.logits + (int64_t)(4 * elq) * V + elr : nullptr;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int idx = mt * 16 + 4 * elq + i;
                const int64_t m = idx;
                const int32_t tgt = (a.w.want_lse && a.w.targets) ? s_tgt[idx] : -1;
                uint64_t k = 0;
                float gmx = -__builtin_inff();
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    const bool live = lo + j * NV + v < hi;
                    const int64_t row = vb[v] * kVB + elr;
                    if (live && row < V && m < M) {
                        const float y = acc[v][mt][i];
                        if (lgp)
                            lgp[(int64_t)(mt * 16 + i) * V + vb[v] * kVB] = y;
                        k = umax64(k, argmax_key(y, (uint32_t)row));
                        gmx = fmaxf(gmx, y);
                        if (row == tgt)
                            a.w.tl[m] = y;
                    }
                }
                if (a.want_argmax) {
                    k = umax16_u64(k);
                    if (elr == 0)
                        red[wv][idx] = umax64(red[wv][idx], k);
                }
                if (a.w.want_lse) {
                    const float mx = max16(gmx);
                    float sx = 0.f;
                    if (mx != -__builtin_inff()) {
#pragma unroll
                        for (int v = 0; v < NV; ++v) {
                            const bool live = lo + j * NV + v < hi;
                            const int64_t row = vb[v] * kVB + elr;
                            if (live && row < V && m < M)
                                sx += exp_le0(acc[v][mt][i] - mx);
                        }
                    }
                    sx = sum16(sx);
                    if (elr == 0)
                        lred[wv][idx] = lse_merge(lred[wv][idx], LsePart{mx, sx});
                }
            }
    }

    // ---- the workgroup's top-1 partial keys and summaries ----
    if (!a.want_argmax && !a.w.want_lse)
        return; // uniform across the grid
    __syncthreads();
    if (threadIdx.x < MT * 16) {
        const int64_t m = threadIdx.x;
        if (m < M && a.want_argmax) {
            uint64_t k = red[0][threadIdx.x];
#pragma unroll
            for (int w2 = 1; w2 < kS2Waves; ++w2)
                k = umax64(k, red[w2][threadIdx.x]);
            a.w.part[m * a.w.n_part + blockIdx.x] = k;
        }
        if (m < M && a.w.want_lse) {
            LsePart p = lred[0][threadIdx.x];
#pragma unroll
            for (int w2 = 1; w2 < kS2Waves; ++w2)
                p = lse_merge(p, lred[w2][threadIdx.x]);
            a.w.lsep[m * a.w.n_part + blockIdx.x] = lse_bits(p);
        }
    }
}

struct Stream2Plan {
    bool ok, xfull;
    int MT, NV, nwg, ngroups;
    unsigned lds_x, lds_ts, lds_xs, lds_sr, lds_sa;
    size_t lds;
};

size_t al256(size_t x) { return (x + 255) / 256 * 256; }

Stream2Plan stream2_plan(const DevHead &h, int64_t M)
{
    Stream2Plan p{};
    const Shape &s = h.s;
    const int64_t nlr = (s.k + s.r) > 0 ? s.n_lr() : 0;
    p.ok = M >= 2 && M <= kS2MaxM && s.g == 4 * kKStep && s.nkc() % kS2Slab == 0 &&
           (nlr + s.nkc()) % kS2NB == 0;
    if (!p.ok)
        return p;
    p.MT = M <= 16 ? 1 : 2;
    const int64_t nvb = s.nvb();
    // one workgroup per compute unit; v-blocks per wave, in groups of NV
    p.nwg = (int)std::min<int64_t>(h.n_cu, (nvb + kS2Waves - 1) / kS2Waves);
    const int64_t W = int64_t(p.nwg) * kS2Waves;
    const int64_t per_wave = (nvb + W - 1) / W;
    // NV = 5 covers the Qwen head's 4.6 v-blocks per wave in one group; a
    // range of 8 takes two groups of 4; one m-tile leaves room for more
    p.NV = p.MT == 2 ? (per_wave <= 5 ? 5 : 4) : (per_wave <= 5 ? 5 : 4);
    p.ngroups = (int)((per_wave + p.NV - 1) / p.NV);
    const size_t ts_bytes = size_t(p.MT) * (s.kst() + s.rst()) * 2 * 1024;
    const size_t xs_bytes = size_t(s.G()) * p.MT * 16 * 4;
    // the workgroup's v-block range holds at most 8 per_wave v-blocks
    const size_t sr_bytes = size_t(kS2Waves) * per_wave * s.G() * kVB * 2;
    // and sA, sC of those rows
    const size_t sa_bytes = size_t(2) * kS2Waves * per_wave * kVB * 2;
    const size_t rest = al256(ts_bytes) + al256(xs_bytes) + al256(sr_bytes) + al256(sa_bytes);
    // all of X in LDS where it fits (no barrier in the stream), else two slabs
    const size_t x_full = size_t(p.MT) * (s.d / kKStep) * 1024, x_slabs = size_t(2) * p.MT * 16 * 1024;
    p.xfull = al256(x_full) + rest <= kS2Lds;
    const size_t x_bytes = p.xfull ? x_full : x_slabs;
    p.lds_x = 0;
    p.lds_ts = (unsigned)al256(x_bytes);
    p.lds_xs = (unsigned)(p.lds_ts + al256(ts_bytes));
    p.lds_sr = (unsigned)(p.lds_xs + al256(xs_bytes));
    p.lds_sa = (unsigned)(p.lds_sr + al256(sr_bytes));
    p.lds = p.lds_sa + al256(sa_bytes);
    if (p.lds > kS2Lds)
        p.ok = false;
    return p;
}

template <int MT, int NV, bool XF>
hipError_t launch2(const Stream2Args &a, const Stream2Plan &p, hipStream_t st)
{
    auto kern = vtile_stream2_kernel<MT, NV, XF>;
    hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)p.nwg), dim3(kS2Waves * 64), p.lds, st, a);
    return hipGetLastError();
}

} // namespace

bool stream2_ok(const DevHead &h, int64_t M) { return stream2_plan(h, M).ok; }

int64_t stream2_max_n_part(const Shape &s) { return (s.nvb() + kS2Waves - 1) / kS2Waves; }

int64_t stream2_n_part(const DevHead &h, int64_t M) { return stream2_plan(h, M).nwg; }

hipError_t launch_vtile_stream2(const DevHead &h, const Work &w, const uint16_t *X, float *logits,
                                int32_t *argmax, hipStream_t st)
{
    const Stream2Plan p = stream2_plan(h, w.M);
    if (!p.ok)
        return hipErrorInvalidValue;
    Stream2Args a;
    a.h = h;
    a.w = w;
    a.w.n_part = p.nwg;
    if (w.M * a.w.n_part > w.part_cap)
        return hipErrorInvalidValue; // argmax partials would not fit the workspace
    a.X = X;
    a.logits = logits;
    a.want_argmax = argmax ? 1 : 0;
    a.nvb = h.s.nvb();
    a.nkc = h.s.nkc();
    a.G = h.s.G();
    a.na = h.s.lr_na();
    a.nlr = (h.s.k + h.s.r) > 0 ? h.s.n_lr() : 0;
    a.nlr_used = a.nlr > 0 ? h.s.lr_na() + h.s.lr_nc() : 0;
    a.kst = h.s.kst();
    a.rst = h.s.rst();
    a.kpad = h.s.kpad();
    a.rpad = h.s.rpad();
    a.ngroups = p.ngroups;
    a.n_slab = (int)(h.s.nkc() / kS2Slab);
    a.lds_x = p.lds_x;
    a.lds_ts = p.lds_ts;
    a.lds_xs = p.lds_xs;
    a.lds_sr = p.lds_sr;
    a.lds_sa = p.lds_sa;
    if (p.MT == 1 && p.xfull)
        return p.NV == 5 ? launch2<1, 5, true>(a, p, st) : launch2<1, 4, true>(a, p, st);
    if (p.MT == 1)
        return p.NV == 5 ? launch2<1, 5, false>(a, p, st) : launch2<1, 4, false>(a, p, st);
    if (p.xfull)
        return p.NV == 5 ? launch2<2, 5, true>(a, p, st) : launch2<2, 4, true>(a, p, st);
    return p.NV == 5 ? launch2<2, 5, false>(a, p, st) : launch2<2, 4, false>(a, p, st);
}

} // namespace archead
