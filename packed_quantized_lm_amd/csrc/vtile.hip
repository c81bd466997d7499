// vtile.hip -- the vocabulary-tile step of the packed ARCHead forward for
// small and moderate M (decode and batched decode): one streaming kernel.
//
// ARCHead paper, section 3.2, eq 7: logits = X W_d^T + (X B_w^T) A_w^T with
// W_d = Q5(A_c) Q8(B_c) + Q_SC4(...) (eq 3).  Per vocabulary row v:
//   logits[m,v] = sA[v] sum_i A5[v,i] t[m,i] + sC[v] sum_i C8[v,i] s[m,i]
//               + sum_grp sR[v,grp] sum_{j in grp} X[m,j] R4[v,j]
// with t = X (sB o B8)^T and s = X (sD o D8)^T from the projection kernel.
//
// Each wave owns NV v-blocks (16 vocabulary rows each) and streams, per
// v-block, first the low-rank chunks (5-bit core and INT8 correction codes)
// and then the SC4 residual chunks, all in the same 1 KiB-per-v-block chunk
// format and through the same two-buffer prefetch, so the wave never waits
// on a short dependent reduction; it then writes the logits and the
// workgroup's top-1 partial keys.
//
// MFMA: v_mfma_f32_16x16x32_bf16 with the hidden states (or t, s) as the A
// operand and 16 vocabulary rows as the B operand, so a wave's output tile is
// [16 hidden states x 16 rows]; lane l holds rows m = 4(l/16) + i, i = 0..3,
// of column v = l % 16.  Integer codes become exact bf16 integers by exponent
// splicing (device.hpp); each g-group of the residual is accumulated on its
// own and folded in with its scale; t and s enter as bf16 hi/lo pairs.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "kernels.hpp"

namespace archead {

struct StreamArgs {
    DevHead h;
    Work w;
    const uint16_t *X;
    float *logits; // M x V, may be null
    int want_argmax;
    int64_t nvb, nkc, G, na, nlr;
    int gsteps;
    int64_t tl_rows; // most rows of t and s an m-tile stages in LDS per hi/lo half
    int n_mt;        // m-tiles; with a 1-D grid, workgroup b takes v-range b / n_mt and
                     // m-tile b % n_mt, so the m-tiles of a v-range run side by side
                     // (their second read of the codes is served by the memory-side cache)
    unsigned lds_xs, lds_x, lds_t, lds_s; // byte offsets of the LDS regions (sr at 0)
};

template <int NV, int MT, bool XL>
struct Chunk {
    u32x4 q[NV];
    u32x4 xf[XL ? 1 : MT][4]; // hidden-state fragments (global-memory variant)
};

// LDS staging of one workgroup (4 waves x NV v-blocks):
//   sr  [4*NV][G][16]    fp16  residual scales of the workgroup's v-blocks
//   xs  [G][MT*16]       fp32  -136 x per-group sums of X for the m-tile
//   x   [M][d]           bf16  the hidden states (XL: small M*d only)
//   t   [2][rows][kpad]  bf16 hi/lo of t for the m-tile's live rows (TL)
//   s   [2][rows][rpad]  bf16 hi/lo of s (TL)
// so that the only vector-memory loads of the streaming loop are the packed
// codes themselves (plus X fragments when X does not fit).  A wave whose
// v-blocks lie beyond the head streams the last v-block again and stores
// nothing, so every wave reaches the final barrier.
//
// WIDE (decode: X in LDS, one group per chunk, chunk counts that are
// multiples of 4): each prefetch buffer holds two K-chunks, so twice the
// bytes are in flight per v-block, at two waves per SIMD.
template <int NV, int MT, int GS, bool XL, bool TL, bool WIDE>
__global__ __launch_bounds__(256, WIDE ? 2 : (XL ? 3 : (MT == 1 ? 2 : 1))) void vtile_stream_kernel(StreamArgs a)
{
    extern __shared__ __attribute__((aligned(16))) char smem[];
    __shared__ uint64_t red[4][MT * 16];
    __shared__ LsePart lred[4][MT * 16];
    __shared__ int32_t s_tgt[64]; // targets of the m-tile's rows (cross-entropy)
    uint16_t *s_sr = (uint16_t *)smem;
    float *s_xs = (float *)(smem + a.lds_xs);
    uint16_t *s_x = (uint16_t *)(smem + a.lds_x);
    uint16_t *s_t = (uint16_t *)(smem + a.lds_t);
    uint16_t *s_s = (uint16_t *)(smem + a.lds_s);

    const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
    const int wv = threadIdx.x >> 6;
    const int64_t nvb = a.nvb, nkc = a.nkc, G = a.G, na = a.na, nlr = a.nlr;
    const int64_t kst = a.h.s.kst(), rst = a.h.s.rst(), kpad = a.h.s.kpad(), rpad = a.h.s.rpad();
    const int64_t vrange = (int64_t)blockIdx.x / a.n_mt, mtile = (int64_t)blockIdx.x % a.n_mt;
    const int64_t wg_vb0 = vrange * 4 * NV;
    const int64_t vb0 = wg_vb0 + wv * NV;
    const int64_t M = a.w.M, Mp = a.w.Mp, d = a.h.s.d, V = a.h.s.V;
    const int64_t mbase = mtile * (MT * 16);
    const int64_t rows_live = (M - mbase) < MT * 16 ? (M - mbase) : MT * 16;
    const int gsteps = GS ? GS : a.gsteps;

    int64_t vb[NV];
    for (int v = 0; v < NV; ++v)
        vb[v] = vb0 + v < nvb ? vb0 + v : nvb - 1;

    // LDS staging by direct-to-LDS copies (global_load_lds): every copy of
    // the workgroup is in flight at once, and the barrier before the
    // streaming loop waits for all of them (one memory latency in total).
    // A copy instruction writes its 64 lanes' pieces to consecutive LDS
    // addresses from a wave-uniform base.
    auto stage16 = [&](const void *src, void *dst, int64_t n16) { // n16 pieces of 16 bytes
        for (int64_t i0 = 0; i0 < n16; i0 += 256) {
            const int64_t i = i0 + threadIdx.x;
            uint32_t *d0 = (uint32_t *)dst + (i0 + wv * 64) * 4;
            if (i < n16)
                __builtin_amdgcn_global_load_lds((const void *)((const u32x4 *)src + i),
                                                 (__attribute__((address_space(3))) void *)d0, 16, 0, 0);
        }
    };
    auto stage_all = [&]() {
        const int64_t nvb_wg = (nvb - wg_vb0) < 4 * NV ? (nvb - wg_vb0) : 4 * NV;
        stage16(a.h.sr + wg_vb0 * G * kVB, s_sr, nvb_wg * G * kVB / 8);
        // xs[grp][j] = xsneg[grp][mbase + j]: 4-byte pieces, 4 groups per copy
        for (int64_t i0 = 0; i0 < G * MT * 16; i0 += 256) {
            const int64_t i = i0 + threadIdx.x;
            const int64_t grp = i / (MT * 16), j = i % (MT * 16);
            float *d0 = s_xs + i0 + wv * 64;
            if (i < G * MT * 16)
                __builtin_amdgcn_global_load_lds((const void *)(a.w.xsneg + grp * Mp + mbase + j),
                                                 (__attribute__((address_space(3))) void *)d0, 4, 0, 0);
        }
        if (a.w.want_lse && a.w.targets && wv == 0) { // rows past M repeat the last target
            const int64_t m = mbase + lane < M ? mbase + lane : M - 1;
            __builtin_amdgcn_global_load_lds((const void *)(a.w.targets + m),
                                             (__attribute__((address_space(3))) void *)s_tgt, 4, 0, 0);
        }
        if (XL)
            stage16(a.X, s_x, M * d / 8);
        if (TL) { // rows mbase .. mbase+rows_live-1 of both halves, hi half first
            const int64_t nt8 = kpad / 8, ns8 = rpad / 8; // 16-byte pieces per row
            for (int h = 0; h < 2; ++h) {
                stage16(a.w.t16 + (h * Mp + mbase) * kpad, s_t + h * rows_live * kpad, rows_live * nt8);
                stage16(a.w.s16 + (h * Mp + mbase) * rpad, s_s + h * rows_live * rpad, rows_live * ns8);
            }
        }
    };

    // Rows m >= M of the A operand only feed output rows that are never
    // stored, so they read the last live row instead of branching around the
    // load (a load under a divergent branch would make the compiler wait for
    // every outstanding load, prefetches included, at the join).
    const uint16_t *xp[MT];
    for (int mt = 0; mt < MT; ++mt) {
        const int64_t m = mbase + mt * 16 + lr;
        xp[mt] = a.X + (m < M ? m : M - 1) * d + 8 * lq;
    }
    const uint16_t *xl = s_x + (lr < M ? lr : M - 1) * d + 8 * lq; // XL: MT == 1, mbase == 0
    const uint16_t *tb = TL ? s_t : a.w.t16 + mbase * kpad;
    const uint16_t *sb = TL ? s_s : a.w.s16 + mbase * rpad;
    const int64_t hst = TL ? rows_live : Mp; // rows between the hi and lo halves
    int64_t trow[MT];
    for (int mt = 0; mt < MT; ++mt)
        trow[mt] = (mt * 16 + lr) < rows_live ? (mt * 16 + lr) : rows_live - 1;

    float sa[NV], sc[NV];
    for (int v = 0; v < NV; ++v) {
        sa[v] = h2f(a.h.sa[vb[v] * kVB + lr]);
        sc[v] = h2f(a.h.sc[vb[v] * kVB + lr]);
    }

    const int64_t ntot = nlr + nkc;
    const u32x4 *lrp = (const u32x4 *)a.h.lr;
    const u32x4 *r4p = (const u32x4 *)a.h.r4;
    // chunk ci of the wave's stream: low-rank chunks 0 .. nlr-1, then the
    // residual K-chunks; indices past the end re-read the last chunk
    auto load_chunk = [&](Chunk<NV, MT, XL> &c, int64_t ci) {
        ci = ci < ntot ? ci : ntot - 1;
        const u32x4 *base = ci < nlr ? lrp + ci * nvb * 64 : r4p + (ci - nlr) * nvb * 64;
        for (int v = 0; v < NV; ++v)
            c.q[v] = __builtin_nontemporal_load(&base[vb[v] * 64 + lane]);
        if (!XL) {
            const int64_t kc = ci < nlr ? 0 : ci - nlr;
#pragma unroll
            for (int s = 0; s < 4; ++s)
                for (int mt = 0; mt < MT; ++mt)
                    c.xf[mt][s] = *(const u32x4 *)(xp[mt] + (kc * 4 + s) * kKStep);
        }
    };

    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const uint32_t kMagic = vgpr_const(kBf16Magic);
    const u32x4 neg144 = {0xC310C310u, 0xC310C310u, 0xC310C310u, 0xC310C310u}; // bf16 -144
    f32x4 acc[NV][MT], ga[NV][MT], gc[NV][MT], nt[MT];
    for (int mt = 0; mt < MT; ++mt) {
        nt[mt] = zero;
        for (int v = 0; v < NV; ++v)
            ga[v][mt] = gc[v][mt] = zero;
    }

    // low-rank chunk j: three core K-steps (A5 against t) or two correction
    // K-steps (C8 against s); K-steps beyond the rank are skipped
    auto lr_chunk = [&](const Chunk<NV, MT, XL> &c, int64_t j) {
        if (j < na) {
#pragma unroll
            for (int q = 0; q < 3; ++q) {
                const int64_t ks = 3 * j + q;
                if (ks >= kst)
                    break;
                u32x4 th[MT], tl[MT];
                for (int mt = 0; mt < MT; ++mt) {
                    th[mt] = *(const u32x4 *)(tb + trow[mt] * kpad + ks * kKStep + 8 * lq);
                    tl[mt] = *(const u32x4 *)(tb + (hst + trow[mt]) * kpad + ks * kKStep + 8 * lq);
                    nt[mt] = mfma_bf16(th[mt], neg144, nt[mt]);
                    nt[mt] = mfma_bf16(tl[mt], neg144, nt[mt]);
                }
                for (int v = 0; v < NV; ++v) {
                    const uint32_t wn = q == 0 ? c.q[v].x : q == 1 ? c.q[v].y : c.q[v].z;
                    const u32x4 b = a5_bf16_q(wn, c.q[v].w, q);
                    for (int mt = 0; mt < MT; ++mt) {
                        ga[v][mt] = mfma_bf16(th[mt], b, ga[v][mt]);
                        ga[v][mt] = mfma_bf16(tl[mt], b, ga[v][mt]);
                    }
                }
            }
        } else {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int64_t ks = 2 * (j - na) + hh;
                if (ks >= rst)
                    break;
                u32x4 sh[MT], sl[MT];
                for (int mt = 0; mt < MT; ++mt) {
                    sh[mt] = *(const u32x4 *)(sb + trow[mt] * rpad + ks * kKStep + 8 * lq);
                    sl[mt] = *(const u32x4 *)(sb + (hst + trow[mt]) * rpad + ks * kKStep + 8 * lq);
                }
                for (int v = 0; v < NV; ++v) {
                    u32x2 w;
                    w.x = hh == 0 ? c.q[v].x : c.q[v].z;
                    w.y = hh == 0 ? c.q[v].y : c.q[v].w;
                    const u32x4 b = c8_bf16(w);
                    for (int mt = 0; mt < MT; ++mt) {
                        gc[v][mt] = mfma_bf16(sh[mt], b, gc[v][mt]);
                        gc[v][mt] = mfma_bf16(sl[mt], b, gc[v][mt]);
                    }
                }
            }
        }
    };
    // acc = sA (A5 t - 144 sum t) + sC (C8 s)
    auto fold_lr = [&]() {
        for (int v = 0; v < NV; ++v)
            for (int mt = 0; mt < MT; ++mt)
                for (int i = 0; i < 4; ++i)
                    acc[v][mt][i] = __builtin_fmaf(sa[v], ga[v][mt][i] + nt[mt][i], sc[v] * gc[v][mt][i]);
    };

    auto x_frags = [&](const Chunk<NV, MT, XL> &c, int64_t kc, u32x4(&xf)[MT][4]) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
            for (int mt = 0; mt < MT; ++mt)
                xf[mt][s] = XL ? *(const u32x4 *)(xl + (kc * 4 + s) * kKStep) : c.xf[XL ? 0 : mt][s];
    };
    // one residual K-step: dequantise NV dwords and issue their MFMAs
    auto kstep = [&](const Chunk<NV, MT, XL> &c, int s, const u32x4(&xf)[MT][4], f32x4(&g)[NV][MT], bool fresh) {
        for (int v = 0; v < NV; ++v) {
            const uint32_t wd = s == 0 ? c.q[v].x : s == 1 ? c.q[v].y : s == 2 ? c.q[v].z : c.q[v].w;
            const u32x4 b = r4_bf16(wd, kMagic);
            for (int mt = 0; mt < MT; ++mt)
                g[v][mt] = mfma_bf16(xf[mt][s], b, fresh ? zero : g[v][mt]);
        }
    };
    // fold one finished residual group: acc += sR (g - 136 sum X)
    auto fold = [&](const f32x4(&g)[NV][MT], int64_t grp) {
        f32x4 xs[MT];
        for (int mt = 0; mt < MT; ++mt)
            xs[mt] = *(const f32x4 *)(s_xs + grp * (MT * 16) + mt * 16 + 4 * lq);
        for (int v = 0; v < NV; ++v) {
            const float scl = h2f(s_sr[((wv * NV + v) * G + grp) * kVB + lr]);
            for (int mt = 0; mt < MT; ++mt)
                for (int i = 0; i < 4; ++i)
                    acc[v][mt][i] = __builtin_fmaf(scl, g[v][mt][i] + xs[mt][i], acc[v][mt][i]);
        }
    };

    if constexpr (WIDE) {
        static_assert(XL && GS == 4, "the wide pipeline is for decode shapes");
        struct Wide {
            Chunk<NV, MT, XL> h0, h1;
        };
        auto load2 = [&](Wide &w, int64_t i) { // stream chunks 2i, 2i + 1
            load_chunk(w.h0, 2 * i);
            load_chunk(w.h1, 2 * i + 1);
        };
        f32x4 gA[NV][MT], gB[NV][MT];
        auto mfma_chunk = [&](const Chunk<NV, MT, XL> &c, int64_t kc, f32x4(&g)[NV][MT]) {
            u32x4 xf[MT][4];
            x_frags(c, kc, xf);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                kstep(c, s, xf, g, s == 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        Wide wA, wB;
        load2(wA, 0);
        load2(wB, 1);
        stage_all();
        __syncthreads(); // LDS staging complete
        const int64_t nl2 = nlr / 2; // double chunks of low-rank codes (even)
        for (int64_t i = 0; i < nl2; i += 2) {
            lr_chunk(wA.h0, 2 * i);
            lr_chunk(wA.h1, 2 * i + 1);
            load2(wA, i + 2);
            __builtin_amdgcn_sched_barrier(0);
            lr_chunk(wB.h0, 2 * i + 2);
            lr_chunk(wB.h1, 2 * i + 3);
            load2(wB, i + 3);
            __builtin_amdgcn_sched_barrier(0);
        }
        fold_lr();
        // residual chunk kc: buffer (kc / 2) % 2, half kc % 2, group
        // accumulator kc % 2, folded one chunk later
        for (int64_t t = 0; t < nkc / 4; ++t) {
            const int64_t kc = 4 * t;
            mfma_chunk(wA.h0, kc, gA);
            if (t > 0)
                fold(gB, kc - 1);
            mfma_chunk(wA.h1, kc + 1, gB);
            fold(gA, kc);
            load2(wA, nl2 + 2 * t + 2);
            __builtin_amdgcn_sched_barrier(0);
            mfma_chunk(wB.h0, kc + 2, gA);
            fold(gB, kc + 1);
            mfma_chunk(wB.h1, kc + 3, gB);
            fold(gA, kc + 2);
            load2(wB, nl2 + 2 * t + 3);
            __builtin_amdgcn_sched_barrier(0);
        }
        fold(gB, nkc - 1);
    } else {
    Chunk<NV, MT, XL> bufA, bufB;
    load_chunk(bufA, 0);
    load_chunk(bufB, 1);
    stage_all();
    __syncthreads(); // LDS staging complete

    // low-rank chunks (nlr is even): bufA holds chunk c, bufB chunk c + 1
    for (int64_t c = 0; c < nlr; c += 2) {
        lr_chunk(bufA, c);
        load_chunk(bufA, c + 2);
        __builtin_amdgcn_sched_barrier(0);
        lr_chunk(bufB, c + 1);
        load_chunk(bufB, c + 3);
        __builtin_amdgcn_sched_barrier(0);
    }
    // folded at once (one drain of the matrix pipeline per wave) so that the
    // low-rank accumulators are dead before the residual ones go live
    fold_lr();
    // residual K-chunk kc now sits in buffer kc % 2; loads name stream
    // indices nlr + kc
    if (GS == 4) {
        // One g-group per chunk.  Chunk c goes to buffer c % 2 and group
        // accumulator c % 2, and is folded in one chunk later, after the next
        // chunk's MFMAs are issued: reading an accumulator right after its
        // MFMAs would stall the wave until the matrix pipeline drains.
        f32x4 gA[NV][MT], gB[NV][MT];
        auto mfma_chunk = [&](const Chunk<NV, MT, XL> &c, int64_t kc, f32x4(&g)[NV][MT]) {
            u32x4 xf[MT][4];
            x_frags(c, kc, xf);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                kstep(c, s, xf, g, s == 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        int64_t c = 0;
        if (nkc > 3) {
            mfma_chunk(bufA, 0, gA);
            load_chunk(bufA, nlr + 2);
            __builtin_amdgcn_sched_barrier(0);
            mfma_chunk(bufB, 1, gB);
            fold(gA, 0);
            load_chunk(bufB, nlr + 3);
            __builtin_amdgcn_sched_barrier(0);
            for (c = 2; c + 3 < nkc; c += 2) {
                mfma_chunk(bufA, c, gA);
                fold(gB, c - 1);
                load_chunk(bufA, nlr + c + 2);
                __builtin_amdgcn_sched_barrier(0);
                mfma_chunk(bufB, c + 1, gB);
                fold(gA, c);
                load_chunk(bufB, nlr + c + 3);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // tail: chunks c .. nkc-1 (at most three); A holds c, B holds c+1
        for (; c < nkc; c += 2) {
            mfma_chunk(bufA, c, gA);
            if (c > 0)
                fold(gB, c - 1);
            if (c + 2 < nkc)
                load_chunk(bufA, nlr + c + 2);
            if (c + 1 < nkc) {
                mfma_chunk(bufB, c + 1, gB);
                fold(gA, c);
                if (c + 3 < nkc)
                    load_chunk(bufB, nlr + c + 3);
            } else {
                fold(gA, c);
            }
        }
        if ((nkc & 1) == 0)
            fold(gB, nkc - 1);
    } else {
        // any other group size: fold each group as soon as it ends
        f32x4 g[NV][MT];
        for (int v = 0; v < NV; ++v)
            for (int mt = 0; mt < MT; ++mt)
                g[v][mt] = zero;
        auto do_chunk = [&](const Chunk<NV, MT, XL> &cb, int64_t kc) {
            u32x4 xf[MT][4];
            x_frags(cb, kc, xf);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int64_t ks = kc * 4 + s;
                const bool start = (ks % gsteps) == 0, end = (ks % gsteps) == gsteps - 1;
                kstep(cb, s, xf, g, start);
                if (end)
                    fold(g, ks / gsteps);
            }
        };
        int64_t c = 0;
        for (; c + 3 < nkc; c += 2) {
            do_chunk(bufA, c);
            load_chunk(bufA, nlr + c + 2);
            __builtin_amdgcn_sched_barrier(0);
            do_chunk(bufB, c + 1);
            load_chunk(bufB, nlr + c + 3);
            __builtin_amdgcn_sched_barrier(0);
        }
        for (; c < nkc; c += 2) {
            do_chunk(bufA, c);
            if (c + 2 < nkc)
                load_chunk(bufA, nlr + c + 2);
            if (c + 1 < nkc)
                do_chunk(bufB, c + 1);
        }
    }

    } // !WIDE

    // logits and the workgroup's top-1 partial keys
    uint64_t key[MT][4];
    for (int mt = 0; mt < MT; ++mt)
        for (int i = 0; i < 4; ++i) {
            const int64_t m = mbase + mt * 16 + 4 * lq + i;
            uint64_t k = 0;
            for (int v = 0; v < NV; ++v) {
                const int64_t row = vb0 + v < nvb ? (vb0 + v) * kVB + lr : V;
                if (row < V && m < M) {
                    if (a.logits)
                        a.logits[m * V + row] = acc[v][mt][i];
                    k = umax64(k, argmax_key(acc[v][mt][i], (uint32_t)row));
                }
            }
            key[mt][i] = k;
        }
    if (!a.want_argmax && !a.w.want_lse)
        return; // uniform across the grid
    if (a.want_argmax)
        for (int mt = 0; mt < MT; ++mt)
            for (int i = 0; i < 4; ++i) {
                uint64_t k = key[mt][i];
                k = umax16_u64(k);
                if (lr == 0)
                    red[wv][mt * 16 + 4 * lq + i] = k;
            }
    if (a.w.want_lse) {
        // the wave's (max, sum exp) per hidden state over its live rows, and
        // the logit of the target row where this lane holds it
        for (int mt = 0; mt < MT; ++mt)
            for (int i = 0; i < 4; ++i) {
                const int64_t m = mbase + mt * 16 + 4 * lq + i;
                const int32_t tgt = (a.w.targets && m < M) ? s_tgt[mt * 16 + 4 * lq + i] : -1;
                float mx = -__builtin_inff();
                for (int v = 0; v < NV; ++v) {
                    const int64_t row = vb0 + v < nvb ? (vb0 + v) * kVB + lr : V;
                    if (row < V && m < M) {
                        mx = fmaxf(mx, acc[v][mt][i]);
                        if (row == tgt)
                            a.w.tl[m] = acc[v][mt][i];
                    }
                }
                mx = max16(mx);
                float sx = 0.f;
                for (int v = 0; v < NV; ++v) {
                    const int64_t row = vb0 + v < nvb ? (vb0 + v) * kVB + lr : V;
                    if (row < V && m < M)
                        sx += exp_le0(acc[v][mt][i] - mx);
                }
                sx = sum16(sx);
                if (lr == 0)
                    lred[wv][mt * 16 + 4 * lq + i] = LsePart{mx, sx};
            }
    }
    __syncthreads();
    if (threadIdx.x < MT * 16) {
        const int64_t m = mbase + threadIdx.x;
        if (m < M && a.want_argmax) {
            const uint64_t k = umax64(umax64(red[0][threadIdx.x], red[1][threadIdx.x]),
                                      umax64(red[2][threadIdx.x], red[3][threadIdx.x]));
            a.w.part[m * a.w.n_part + vrange] = k;
        }
        if (m < M && a.w.want_lse) {
            const LsePart p = lse_merge(lse_merge(lred[0][threadIdx.x], lred[1][threadIdx.x]),
                                        lse_merge(lred[2][threadIdx.x], lred[3][threadIdx.x]));
            a.w.lsep[m * a.w.n_part + vrange] = lse_bits(p);
        }
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
constexpr int kNV = 4;   // v-blocks per wave
constexpr int kNV2 = 5;  // v-blocks per wave with two m-tiles (one workgroup per CU): 475
                         // workgroups at V = 151936 make two full rounds of the CUs
constexpr int kNVW = 5;  // v-blocks per wave, wide pipeline (two waves per SIMD)
constexpr int64_t kXLdsMaxBytes = 48 * 1024;  // X staged in LDS when M*d*2 fits
constexpr int64_t kTLdsMaxBytes = 64 * 1024;  // t and s staged in LDS when they fit

struct SkinnyPlan {
    int MT, nv;
    bool xl, wide;
};

static SkinnyPlan skinny_plan(const DevHead &h, int64_t M)
{
    SkinnyPlan p;
    p.MT = M <= 16 ? 1 : 2;
    p.xl = p.MT == 1 && M * h.s.d * 2 <= kXLdsMaxBytes;
    // the wide pipeline runs two waves per SIMD; it is taken only when all
    // of its waves are resident at once (a second, partial round of waves
    // would cost a whole round of time)
    const int64_t wide_waves = (h.s.nvb() + kNVW - 1) / kNVW;
    p.wide = p.xl && h.s.g == 4 * kKStep && h.s.nkc() % 4 == 0 && h.s.n_lr() % 4 == 0 &&
             wide_waves <= int64_t(h.n_cu) * 4 * 2;
    p.nv = p.wide ? kNVW : (p.MT == 2 ? kNV2 : kNV);
    return p;
}

int64_t skinny_n_part(const DevHead &h, int64_t M)
{
    const SkinnyPlan p = skinny_plan(h, M);
    return (h.s.nvb() + 4 * p.nv - 1) / (4 * p.nv);
}

int64_t skinny_max_n_part(const Shape &s)
{
    const int nv = kNV < kNVW ? kNV : kNVW;
    return (s.nvb() + 4 * nv - 1) / (4 * nv);
}

static size_t al16(size_t x) { return (x + 15) / 16 * 16; }

template <typename K, typename A>
static hipError_t launch(K kern, dim3 grid, size_t lds, hipStream_t st, const A &args)
{
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL(kern, grid, dim3(256), lds, st, args);
    return hipGetLastError();
}

template <int MT, bool XL, bool TL>
static hipError_t launch_gs(const StreamArgs &a, dim3 grid, size_t lds, hipStream_t st)
{
    constexpr int nv = MT == 2 ? kNV2 : kNV;
    switch (a.gsteps) {
    case 4: return launch(vtile_stream_kernel<nv, MT, 4, XL, TL, false>, grid, lds, st, a);
    default: return launch(vtile_stream_kernel<nv, MT, 0, XL, TL, false>, grid, lds, st, a);
    }
}

hipError_t launch_vtile_skinny(const DevHead &h, const Work &w, const uint16_t *X, float *logits,
                               int32_t *argmax, hipStream_t st)
{
    const SkinnyPlan p = skinny_plan(h, w.M);
    const int MT = p.MT;
    const unsigned gy = (unsigned)((w.M + 16 * MT - 1) / (16 * MT));

    StreamArgs a;
    a.h = h;
    a.w = w;
    a.w.n_part = skinny_n_part(h, w.M);
    if (w.M * a.w.n_part > w.part_cap)
        return hipErrorInvalidValue; // argmax partials would not fit the workspace
    a.X = X;
    a.logits = logits;
    a.want_argmax = argmax ? 1 : 0;
    a.nvb = h.s.nvb();
    a.nkc = h.s.nkc();
    a.G = h.s.G();
    a.na = h.s.lr_na();
    a.nlr = h.s.n_lr();
    a.gsteps = (int)(h.s.g / kKStep);
    a.tl_rows = w.M < 16 * MT ? w.M : 16 * MT;
    const bool XL = p.xl;
    const size_t t_bytes = al16(size_t(2) * a.tl_rows * h.s.kpad() * 2);
    const size_t s_bytes = al16(size_t(2) * a.tl_rows * h.s.rpad() * 2);
    const bool TL = t_bytes + s_bytes <= (size_t)kTLdsMaxBytes;
    a.lds_xs = (unsigned)al16(size_t(4) * p.nv * a.G * kVB * 2);
    a.lds_x = (unsigned)(a.lds_xs + al16(size_t(a.G) * MT * 16 * 4));
    a.lds_t = (unsigned)(a.lds_x + (XL ? al16(size_t(w.M) * h.s.d * 2) : 0));
    a.lds_s = (unsigned)(a.lds_t + (TL ? t_bytes : 0));
    const size_t lds = a.lds_s + (TL ? s_bytes : 0);
    a.n_mt = (int)gy;
    const dim3 grid((unsigned)(a.w.n_part * gy));
    if (p.wide)
        return TL ? launch(vtile_stream_kernel<kNVW, 1, 4, true, true, true>, grid, lds, st, a)
                  : launch(vtile_stream_kernel<kNVW, 1, 4, true, false, true>, grid, lds, st, a);
    if (MT == 1) {
        if (XL)
            return TL ? launch_gs<1, true, true>(a, grid, lds, st) : launch_gs<1, true, false>(a, grid, lds, st);
        return TL ? launch_gs<1, false, true>(a, grid, lds, st) : launch_gs<1, false, false>(a, grid, lds, st);
    }
    return TL ? launch_gs<2, false, true>(a, grid, lds, st) : launch_gs<2, false, false>(a, grid, lds, st);
}

} // namespace archead
