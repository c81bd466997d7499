// vtile.hip -- the vocabulary-tile step of the packed ARCHead forward for
// small and moderate M (decode and batched decode), as two streaming kernels.
//
// ARCHead paper, section 3.2, eq 7: logits = X W_d^T + (X B_w^T) A_w^T with
// W_d = Q5(A_c) Q8(B_c) + Q_SC4(...) (eq 3).  Per vocabulary row v:
//   logits[m,v] = sum_grp sR[v,grp] sum_{j in grp} X[m,j] R4[v,j]      (residual)
//               + sA[v] sum_i A5[v,i] t[m,i] + sC[v] sum_i C8[v,i] s[m,i]
// with t = X (sB o B8)^T and s = X (sD o D8)^T from the projection kernel.
//
// vtile_r4_kernel streams the SC4 residual (87 % of the packed bytes) and
// writes the residual term; vtile_lowrank_kernel then streams the 5-bit and
// INT8 factors, adds the two low-rank terms and produces the per-workgroup
// top-1 partials.  Keeping the short low-rank reduction out of the residual
// stream keeps that stream free of latency-bound tail work and register
// pressure; the price is one extra pass over M x V fp32 logits (0.6 MB at
// M = 1).
//
// Both kernels use v_mfma_f32_16x16x32_bf16 with the hidden states (or t, s)
// as the A operand and 16 vocabulary rows as the B operand, so a wave's
// output tile is [16 hidden states x 16 rows]; lane l holds rows
// m = 4(l/16) + i, i = 0..3, of column v = l % 16.  Integer codes are turned
// into exact bf16 integers by exponent splicing (see device.hpp); each
// g-group is accumulated on its own and folded in with its fp32 scale.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "kernels.hpp"

namespace archead {

// ---------------------------------------------------------------------------
// Residual stream.
// ---------------------------------------------------------------------------
struct R4Args {
    DevHead h;
    Work w;
    const uint16_t *X;
    float *dst; // M x V partial logits (the residual term)
    int64_t nvb, nkc, G;
    int gsteps;
    unsigned lds_xs, lds_x; // byte offsets of the LDS regions (sr at 0)
};

template <int NV, int MT, bool XL>
struct R4Chunk {
    u32x4 r4[NV];
    u32x4 xf[XL ? 1 : MT][4]; // hidden-state fragments (global-memory variant)
};

// LDS staging of one workgroup (4 waves x NV v-blocks):
//   sr  [4*NV][G][16] fp16  residual scales of the workgroup's v-blocks
//   xs  [G][MT*16]    fp32  -136 x per-group sums of X for the m-tile
//   x   [M][d]        bf16  the hidden states (XL: small M*d only)
// so that the only vector-memory loads of the streaming loop are the residual
// nibbles themselves (plus X fragments when X does not fit).
template <int NV, int MT, int GS, bool XL>
__global__ __launch_bounds__(256, XL ? 3 : (MT == 1 ? 2 : 1)) void vtile_r4_kernel(R4Args a)
{
    extern __shared__ __attribute__((aligned(16))) char smem[];
    uint16_t *s_sr = (uint16_t *)smem;
    float *s_xs = (float *)(smem + a.lds_xs);
    uint16_t *s_x = (uint16_t *)(smem + a.lds_x);

    const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
    const int wv = threadIdx.x >> 6;
    const int64_t nvb = a.nvb, nkc = a.nkc, G = a.G;
    const int64_t wg_vb0 = (int64_t)blockIdx.x * 4 * NV;
    const int64_t vb0 = wg_vb0 + wv * NV;
    const bool active = vb0 < nvb;
    const int64_t M = a.w.M, Mp = a.w.Mp, d = a.h.s.d, V = a.h.s.V;
    const int64_t mbase = (int64_t)blockIdx.y * (MT * 16);
    const int gsteps = GS ? GS : a.gsteps;

    int64_t vb[NV];
    for (int v = 0; v < NV; ++v)
        vb[v] = vb0 + v < nvb ? vb0 + v : nvb - 1;

    {
        const int64_t nvb_wg = (nvb - wg_vb0) < 4 * NV ? (nvb - wg_vb0) : 4 * NV;
        const int64_t n16 = nvb_wg * G * kVB / 8;
        const u32x4 *src = (const u32x4 *)(a.h.sr + wg_vb0 * G * kVB);
        for (int64_t i = threadIdx.x; i < n16; i += 256)
            ((u32x4 *)s_sr)[i] = src[i];
        for (int64_t i = threadIdx.x; i < G * MT * 16; i += 256) {
            const int64_t grp = i / (MT * 16), j = i % (MT * 16);
            s_xs[i] = a.w.xsneg[grp * Mp + mbase + j];
        }
        if (XL) {
            const int64_t n16x = M * d / 8;
            for (int64_t i = threadIdx.x; i < n16x; i += 256)
                ((u32x4 *)s_x)[i] = ((const u32x4 *)a.X)[i];
        }
    }
    __syncthreads();
    if (!active)
        return;

    // Rows m >= M of the A operand only feed output rows that are never
    // stored, so they read row M-1 instead of branching around the load (a
    // load under a divergent branch would make the compiler wait for every
    // outstanding load, prefetches included, at the join).
    const uint16_t *xp[MT];
    for (int mt = 0; mt < MT; ++mt) {
        const int64_t m = mbase + mt * 16 + lr;
        xp[mt] = a.X + (m < M ? m : M - 1) * d + 8 * lq;
    }
    const uint16_t *xl = s_x + (lr < M ? lr : M - 1) * d + 8 * lq; // XL: MT == 1, mbase == 0

    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const uint32_t kMagic = vgpr_const(kBf16Magic);
    f32x4 acc[NV][MT];
    for (int v = 0; v < NV; ++v)
        for (int mt = 0; mt < MT; ++mt)
            acc[v][mt] = zero;

    const u32x4 *r4 = (const u32x4 *)a.h.r4;
    auto load_chunk = [&](R4Chunk<NV, MT, XL> &c, int64_t kc) {
        for (int v = 0; v < NV; ++v)
            c.r4[v] = __builtin_nontemporal_load(&r4[(kc * nvb + vb[v]) * 64 + lane]);
        if (!XL) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
                for (int mt = 0; mt < MT; ++mt)
                    c.xf[mt][s] = *(const u32x4 *)(xp[mt] + (kc * 4 + s) * kKStep);
        }
    };
    auto x_frags = [&](const R4Chunk<NV, MT, XL> &c, int64_t kc, u32x4(&xf)[MT][4]) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
            for (int mt = 0; mt < MT; ++mt)
                xf[mt][s] = XL ? *(const u32x4 *)(xl + (kc * 4 + s) * kKStep) : c.xf[XL ? 0 : mt][s];
    };
    // one K-step: dequantise NV residual dwords and issue their MFMAs
    auto kstep = [&](const R4Chunk<NV, MT, XL> &c, int s, const u32x4(&xf)[MT][4], f32x4(&g)[NV][MT], bool fresh) {
        for (int v = 0; v < NV; ++v) {
            const uint32_t wd = s == 0 ? c.r4[v].x : s == 1 ? c.r4[v].y : s == 2 ? c.r4[v].z : c.r4[v].w;
            const u32x4 b = r4_bf16(wd, kMagic);
            for (int mt = 0; mt < MT; ++mt)
                g[v][mt] = mfma_bf16(xf[mt][s], b, fresh ? zero : g[v][mt]);
        }
    };
    // fold one finished group into the logits: acc += sR (g - 136 sum X)
    auto fold = [&](const f32x4(&g)[NV][MT], int64_t grp) {
        f32x4 xs[MT];
        for (int mt = 0; mt < MT; ++mt)
            xs[mt] = *(const f32x4 *)(s_xs + grp * (MT * 16) + mt * 16 + 4 * lq);
        for (int v = 0; v < NV; ++v) {
            const float sc = h2f(s_sr[((wv * NV + v) * G + grp) * kVB + lr]);
            for (int mt = 0; mt < MT; ++mt)
                for (int i = 0; i < 4; ++i)
                    acc[v][mt][i] = __builtin_fmaf(sc, g[v][mt][i] + xs[mt][i], acc[v][mt][i]);
        }
    };

    R4Chunk<NV, MT, XL> bufA, bufB;
    load_chunk(bufA, 0);
    load_chunk(bufB, nkc > 1 ? 1 : 0);

    if (GS == 4) {
        // One g-group per chunk.  Chunk c goes to buffer c % 2 and group
        // accumulator c % 2, and is folded in one chunk later, after the next
        // chunk's MFMAs are issued: reading an accumulator right after its
        // MFMAs would stall the wave until the matrix pipeline drains.
        f32x4 gA[NV][MT], gB[NV][MT];
        auto mfma_chunk = [&](const R4Chunk<NV, MT, XL> &c, int64_t kc, f32x4(&g)[NV][MT]) {
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
            load_chunk(bufA, 2);
            __builtin_amdgcn_sched_barrier(0);
            mfma_chunk(bufB, 1, gB);
            fold(gA, 0);
            load_chunk(bufB, 3);
            __builtin_amdgcn_sched_barrier(0);
            for (c = 2; c + 3 < nkc; c += 2) {
                mfma_chunk(bufA, c, gA);
                fold(gB, c - 1);
                load_chunk(bufA, c + 2);
                __builtin_amdgcn_sched_barrier(0);
                mfma_chunk(bufB, c + 1, gB);
                fold(gA, c);
                load_chunk(bufB, c + 3);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // tail: chunks c .. nkc-1 (at most three); A holds c, B holds c+1
        for (; c < nkc; c += 2) {
            mfma_chunk(bufA, c, gA);
            if (c > 0)
                fold(gB, c - 1);
            if (c + 2 < nkc)
                load_chunk(bufA, c + 2);
            if (c + 1 < nkc) {
                mfma_chunk(bufB, c + 1, gB);
                fold(gA, c);
                if (c + 3 < nkc)
                    load_chunk(bufB, c + 3);
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
        auto do_chunk = [&](const R4Chunk<NV, MT, XL> &cb, int64_t kc) {
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
            load_chunk(bufA, c + 2);
            __builtin_amdgcn_sched_barrier(0);
            do_chunk(bufB, c + 1);
            load_chunk(bufB, c + 3);
            __builtin_amdgcn_sched_barrier(0);
        }
        for (; c < nkc; c += 2) {
            do_chunk(bufA, c);
            if (c + 2 < nkc)
                load_chunk(bufA, c + 2);
            if (c + 1 < nkc)
                do_chunk(bufB, c + 1);
        }
    }

    for (int mt = 0; mt < MT; ++mt)
        for (int i = 0; i < 4; ++i) {
            const int64_t m = mbase + mt * 16 + 4 * lq + i;
            for (int v = 0; v < NV; ++v) {
                const int64_t row = vb0 + v < nvb ? (vb0 + v) * kVB + lr : V;
                if (row < V && m < M)
                    a.dst[m * V + row] = acc[v][mt][i];
            }
        }
}

// ---------------------------------------------------------------------------
// Low-rank terms, logits epilogue and top-1 partials.
// ---------------------------------------------------------------------------
struct LRArgs {
    DevHead h;
    Work w;
    const float *partial; // M x V residual term
    float *logits;        // may be null
    int want_argmax;
    int64_t nvb;
    unsigned lds_s; // byte offset of s16 in LDS (t16 at 0)
};

constexpr int kLRKB = 8; // core-factor K-steps whose codes one batch loads at once
constexpr int kLRRB = 4; // correction K-steps per batch

// TL: the bf16 hi/lo of t and s for the m-tile's live rows are staged in LDS
// (t16 [2][16MT][kpad], s16 [2][16MT][rpad]); otherwise (large ranks) they
// are read from the workspace directly.  Rows at or beyond M read row M-1.
// Every global load of a batch is issued before the first MFMA, so a wave
// costs about one memory latency per batch (one in total for ranks <= 256).
template <int NV, int MT, bool TL>
__global__ __launch_bounds__(256) void vtile_lowrank_kernel(LRArgs a)
{
    extern __shared__ __attribute__((aligned(16))) char smem[];
    uint16_t *s_t = (uint16_t *)smem;
    uint16_t *s_s = (uint16_t *)(smem + a.lds_s);

    const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
    const int wv = threadIdx.x >> 6;
    const int64_t nvb = a.nvb;
    const int64_t vb0 = ((int64_t)blockIdx.x * 4 + wv) * NV;
    const bool active = vb0 < nvb;
    const int64_t M = a.w.M, Mp = a.w.Mp, V = a.h.s.V;
    const int64_t mbase = (int64_t)blockIdx.y * (MT * 16);
    const int64_t kpad = a.h.s.kpad(), rpad = a.h.s.rpad();
    const int64_t kst = a.h.s.kst(), rst = a.h.s.rst(), ahg = a.h.s.a5h_groups();
    const int64_t rows_live = (M - mbase) < MT * 16 ? (M - mbase) : MT * 16;

    int64_t vb[NV];
    for (int v = 0; v < NV; ++v)
        vb[v] = vb0 + v < nvb ? vb0 + v : nvb - 1;

    // first batch of global loads: residual term of the wave's outputs, the
    // correction codes and the first core-factor codes
    f32x4 y[NV][MT];
    for (int v = 0; v < NV; ++v)
        for (int mt = 0; mt < MT; ++mt)
            for (int i = 0; i < 4; ++i) {
                const int64_t m = mbase + mt * 16 + 4 * lq + i;
                const int64_t row = vb[v] * kVB + lr;
                y[v][mt][i] = a.partial[(m < M ? m : M - 1) * V + (row < V ? row : V - 1)];
            }
    u32x2 c8r[NV][kLRRB];
    uint32_t wn[NV][kLRKB], wh[NV][kLRKB / 4];
    auto load_c8 = [&](int64_t ks0) {
        for (int q = 0; q < kLRRB; ++q) {
            const int64_t ks = ks0 + q < rst ? ks0 + q : rst - 1;
            for (int v = 0; v < NV; ++v)
                c8r[v][q] = *(const u32x2 *)(a.h.c8 + ((vb[v] * rst + ks) * 64 + lane) * 2);
        }
    };
    auto load_a5 = [&](int64_t ks0) {
        for (int q = 0; q < kLRKB; ++q) {
            const int64_t ks = ks0 + q < kst ? ks0 + q : kst - 1;
            for (int v = 0; v < NV; ++v)
                wn[v][q] = a.h.a5n[(vb[v] * kst + ks) * 64 + lane];
        }
        for (int q = 0; q < kLRKB / 4; ++q) {
            const int64_t g4 = ks0 / 4 + q < ahg ? ks0 / 4 + q : ahg - 1;
            for (int v = 0; v < NV; ++v)
                wh[v][q] = a.h.a5h[(vb[v] * ahg + g4) * 64 + lane];
        }
    };
    if (active && rst > 0)
        load_c8(0);
    if (active && kst > 0)
        load_a5(0);

    if (TL) {
        const int64_t nt8 = kpad / 8, ns8 = rpad / 8; // 16-byte pieces per row
        for (int64_t i = threadIdx.x; i < 2 * rows_live * nt8; i += 256) {
            const int64_t h = i / (rows_live * nt8), rem = i % (rows_live * nt8), rr = rem / nt8, c = rem % nt8;
            ((u32x4 *)s_t)[(h * MT * 16 + rr) * nt8 + c] = *(const u32x4 *)(a.w.t16 + (h * Mp + mbase + rr) * kpad + c * 8);
        }
        for (int64_t i = threadIdx.x; i < 2 * rows_live * ns8; i += 256) {
            const int64_t h = i / (rows_live * ns8), rem = i % (rows_live * ns8), rr = rem / ns8, c = rem % ns8;
            ((u32x4 *)s_s)[(h * MT * 16 + rr) * ns8 + c] = *(const u32x4 *)(a.w.s16 + (h * Mp + mbase + rr) * rpad + c * 8);
        }
    }
    __syncthreads();
    // tile rows r of the hi (h = 0) and lo (h = 1) halves
    const uint16_t *tb = TL ? s_t : a.w.t16 + mbase * kpad;
    const uint16_t *sb = TL ? s_s : a.w.s16 + mbase * rpad;
    const int64_t th_stride = TL ? MT * 16 : Mp; // rows between the hi and lo halves
    int64_t trow[MT];
    for (int mt = 0; mt < MT; ++mt)
        trow[mt] = (mt * 16 + lr) < rows_live ? (mt * 16 + lr) : rows_live - 1;

    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    if (active && rst > 0) {
        f32x4 g[NV][MT];
        for (int v = 0; v < NV; ++v)
            for (int mt = 0; mt < MT; ++mt)
                g[v][mt] = zero;
        for (int64_t ks0 = 0; ks0 < rst; ks0 += kLRRB) {
            if (ks0 > 0)
                load_c8(ks0);
#pragma unroll
            for (int q = 0; q < kLRRB; ++q) {
                const int64_t ks = ks0 + q;
                if (ks >= rst)
                    break;
                u32x4 sh[MT], sl[MT];
                for (int mt = 0; mt < MT; ++mt) {
                    sh[mt] = *(const u32x4 *)(sb + trow[mt] * rpad + ks * kKStep + 8 * lq);
                    sl[mt] = *(const u32x4 *)(sb + (th_stride + trow[mt]) * rpad + ks * kKStep + 8 * lq);
                }
                for (int v = 0; v < NV; ++v) {
                    const u32x4 b = c8_bf16(c8r[v][q]);
                    for (int mt = 0; mt < MT; ++mt) {
                        g[v][mt] = mfma_bf16(sh[mt], b, g[v][mt]);
                        g[v][mt] = mfma_bf16(sl[mt], b, g[v][mt]);
                    }
                }
            }
        }
        for (int v = 0; v < NV; ++v) {
            const float sc = h2f(a.h.sc[vb[v] * kVB + lr]);
            for (int mt = 0; mt < MT; ++mt)
                for (int i = 0; i < 4; ++i)
                    y[v][mt][i] = __builtin_fmaf(sc, g[v][mt][i], y[v][mt][i]);
        }
    }

    if (active && kst > 0) {
        const u32x4 neg144 = {0xC310C310u, 0xC310C310u, 0xC310C310u, 0xC310C310u};
        f32x4 g[NV][MT], nt[MT];
        for (int mt = 0; mt < MT; ++mt)
            nt[mt] = zero;
        for (int v = 0; v < NV; ++v)
            for (int mt = 0; mt < MT; ++mt)
                g[v][mt] = zero;
        for (int64_t ks0 = 0; ks0 < kst; ks0 += kLRKB) {
            if (ks0 > 0)
                load_a5(ks0);
#pragma unroll
            for (int q = 0; q < kLRKB; ++q) {
                const int64_t ks = ks0 + q;
                if (ks >= kst)
                    break;
                u32x4 th[MT], tl[MT];
                for (int mt = 0; mt < MT; ++mt) {
                    th[mt] = *(const u32x4 *)(tb + trow[mt] * kpad + ks * kKStep + 8 * lq);
                    tl[mt] = *(const u32x4 *)(tb + (th_stride + trow[mt]) * kpad + ks * kKStep + 8 * lq);
                    nt[mt] = mfma_bf16(th[mt], neg144, nt[mt]);
                    nt[mt] = mfma_bf16(tl[mt], neg144, nt[mt]);
                }
                for (int v = 0; v < NV; ++v) {
                    const u32x4 b = a5_bf16_q(wn[v][q], wh[v][q / 4], q % 4);
                    for (int mt = 0; mt < MT; ++mt) {
                        g[v][mt] = mfma_bf16(th[mt], b, g[v][mt]);
                        g[v][mt] = mfma_bf16(tl[mt], b, g[v][mt]);
                    }
                }
            }
        }
        for (int v = 0; v < NV; ++v) {
            const float sc = h2f(a.h.sa[vb[v] * kVB + lr]);
            for (int mt = 0; mt < MT; ++mt)
                for (int i = 0; i < 4; ++i)
                    y[v][mt][i] = __builtin_fmaf(sc, g[v][mt][i] + nt[mt][i], y[v][mt][i]);
        }
    }

    uint64_t key[MT][4];
    for (int mt = 0; mt < MT; ++mt)
        for (int i = 0; i < 4; ++i) {
            const int64_t m = mbase + mt * 16 + 4 * lq + i;
            uint64_t k = 0;
            if (active) {
                for (int v = 0; v < NV; ++v) {
                    const int64_t row = vb0 + v < nvb ? (vb0 + v) * kVB + lr : V;
                    if (row < V && m < M) {
                        if (a.logits)
                            a.logits[m * V + row] = y[v][mt][i];
                        k = umax64(k, argmax_key(y[v][mt][i], (uint32_t)row));
                    }
                }
            }
            key[mt][i] = k;
        }
    if (!a.want_argmax)
        return; // uniform across the grid
    __shared__ uint64_t red[4][MT * 16];
    for (int mt = 0; mt < MT; ++mt)
        for (int i = 0; i < 4; ++i) {
            uint64_t k = key[mt][i];
            k = umax64(k, shfl_xor_u64(k, 1));
            k = umax64(k, shfl_xor_u64(k, 2));
            k = umax64(k, shfl_xor_u64(k, 4));
            k = umax64(k, shfl_xor_u64(k, 8));
            if (lr == 0)
                red[wv][mt * 16 + 4 * lq + i] = k;
        }
    __syncthreads();
    if (threadIdx.x < MT * 16) {
        const int64_t m = mbase + threadIdx.x;
        const uint64_t k = umax64(umax64(red[0][threadIdx.x], red[1][threadIdx.x]),
                                  umax64(red[2][threadIdx.x], red[3][threadIdx.x]));
        if (m < M)
            a.w.part[m * a.w.n_part + blockIdx.x] = k;
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
constexpr int kR4NV = 4;
constexpr int kLRNV = 2;
constexpr int64_t kXLdsMaxBytes = 48 * 1024; // X staged in LDS when M*d*2 fits

int64_t skinny_n_part(const DevHead &h, int64_t M)
{
    (void)M;
    return (h.s.nvb() + 4 * kLRNV - 1) / (4 * kLRNV);
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

template <int MT, bool XL>
static hipError_t launch_r4(const R4Args &a, dim3 grid, size_t lds, hipStream_t st)
{
    switch (a.gsteps) {
    case 4: return launch(vtile_r4_kernel<kR4NV, MT, 4, XL>, grid, lds, st, a);
    default: return launch(vtile_r4_kernel<kR4NV, MT, 0, XL>, grid, lds, st, a);
    }
}

hipError_t launch_vtile_skinny(const DevHead &h, const Work &w, const uint16_t *X, float *logits,
                               float *scratch, int32_t *argmax, hipStream_t st, bool *argmax_done)
{
    const int MT = w.M <= 16 ? 1 : 2;
    const unsigned gy = (unsigned)((w.M + 16 * MT - 1) / (16 * MT));
    float *dst = logits ? logits : scratch;

    R4Args r;
    r.h = h;
    r.w = w;
    r.X = X;
    r.dst = dst;
    r.nvb = h.s.nvb();
    r.nkc = h.s.nkc();
    r.G = h.s.G();
    r.gsteps = (int)(h.s.g / kKStep);
    const bool XL = MT == 1 && w.M * h.s.d * 2 <= kXLdsMaxBytes;
    r.lds_xs = (unsigned)al16(size_t(4) * kR4NV * r.G * kVB * 2);
    r.lds_x = (unsigned)(r.lds_xs + al16(size_t(r.G) * MT * 16 * 4));
    const size_t lds_r = r.lds_x + (XL ? al16(size_t(w.M) * h.s.d * 2) : 0);
    const unsigned gx_r = (unsigned)((r.nvb + 4 * kR4NV - 1) / (4 * kR4NV));
    hipError_t e;
    if (MT == 1)
        e = XL ? launch_r4<1, true>(r, dim3(gx_r, gy), lds_r, st) : launch_r4<1, false>(r, dim3(gx_r, gy), lds_r, st);
    else
        e = launch_r4<2, false>(r, dim3(gx_r, gy), lds_r, st);
    if (e != hipSuccess)
        return e;

    LRArgs l;
    l.h = h;
    l.w = w;
    l.partial = dst;
    l.logits = logits;
    l.want_argmax = argmax ? 1 : 0;
    l.nvb = h.s.nvb();
    l.w.n_part = skinny_n_part(h, w.M);
    l.lds_s = (unsigned)al16(size_t(2) * MT * 16 * h.s.kpad() * 2);
    size_t lds_l = l.lds_s + al16(size_t(2) * MT * 16 * h.s.rpad() * 2) + 16;
    const bool TL = lds_l <= 64 * 1024;
    if (!TL)
        lds_l = 16;
    const unsigned gx_l = (unsigned)l.w.n_part;
    if (MT == 1)
        e = TL ? launch(vtile_lowrank_kernel<kLRNV, 1, true>, dim3(gx_l, gy), lds_l, st, l)
               : launch(vtile_lowrank_kernel<kLRNV, 1, false>, dim3(gx_l, gy), lds_l, st, l);
    else
        e = TL ? launch(vtile_lowrank_kernel<kLRNV, 2, true>, dim3(gx_l, gy), lds_l, st, l)
               : launch(vtile_lowrank_kernel<kLRNV, 2, false>, dim3(gx_l, gy), lds_l, st, l);
    *argmax_done = false;
    return e;
}

} // namespace archead
