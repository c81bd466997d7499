// forward.hip -- projection, skinny vocabulary-tile and argmax kernels of the
// packed ARCHead head forward on gfx950.
//
// ARCHead paper, section 3.2, eq 7: logits = X W_d^T + (X B_w^T) A_w^T, with
// W_d = Q5(A_c) Q8(B_c) + Q_SC4(...) (eq 3) and A_w, B_w stored as row/group
// INT8 (text after eq 7).  The forward is factored exactly as eq 7 factors
// it -- the narrow products X B^T are formed first (a1, proj_kernel), then
// every vocabulary row streams its residual nibbles once and adds its two
// low-rank terms (a2), then a per-token top-1 reduction runs across the
// vocabulary tiles (a3).
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "kernels.hpp"

namespace archead {

// ---------------------------------------------------------------------------
// a1: projection.  t[m,i] = sB[i] sum_j X[m,j] B8[i,j]; s[m,i] = sum over
// groups of sD[i,grp] sum_{j in grp} X[m,j] D8[i,j]; both split into bf16
// hi + lo (16 significant bits) for the MFMA K-extension of a2.  The extra
// last column block writes xsneg[grp][m] = -136 sum_{j in grp} X[m,j], the
// constant the offset-binary residual codes add to each group's dot product.
// ---------------------------------------------------------------------------
constexpr int kProjNI = 2; // output columns per wave
constexpr int kProjMB = 4; // hidden states per workgroup

struct ProjArgs {
    const uint16_t *X;
    int64_t M, Mp, d, k, r, g, G, kpad, rpad;
    const int8_t *b8;
    const float *sb;
    const int8_t *d8;
    const float *sd;
    uint16_t *t16, *s16;
    float *xsneg;
    int ncolblk;
};

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float i8(uint32_t w, int b) { return (float)(int8_t)(w >> (8 * b)); }

// 16 int8 weights x 16 bf16 activations, fp32 accumulation
__device__ __forceinline__ float dot16(u32x4 q, u32x4 x0, u32x4 x1)
{
    float s = 0.f;
    const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
    const uint32_t xw[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    for (int e = 0; e < 4; ++e) {
        s = __builtin_fmaf(bf_lo(xw[2 * e]), i8(qw[e], 0), s);
        s = __builtin_fmaf(bf_hi(xw[2 * e]), i8(qw[e], 1), s);
        s = __builtin_fmaf(bf_lo(xw[2 * e + 1]), i8(qw[e], 2), s);
        s = __builtin_fmaf(bf_hi(xw[2 * e + 1]), i8(qw[e], 3), s);
    }
    return s;
}

__global__ __launch_bounds__(256) void proj_kernel(ProjArgs a)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t m0 = (int64_t)blockIdx.y * kProjMB;

    if ((int)blockIdx.x == a.ncolblk) { // per-group sums of X
        for (int mi = wv; mi < kProjMB; mi += 4) {
            const int64_t m = m0 + mi;
            if (m >= a.M)
                break;
            const uint16_t *xr = a.X + m * a.d;
            for (int64_t c = lane; c < a.G; c += 64) {
                float s = 0.f;
                for (int64_t j = c * a.g; j < (c + 1) * a.g; j += 8) {
                    u32x4 v = *(const u32x4 *)(xr + j);
                    s += bf_lo(v.x) + bf_hi(v.x) + bf_lo(v.y) + bf_hi(v.y) +
                         bf_lo(v.z) + bf_hi(v.z) + bf_lo(v.w) + bf_hi(v.w);
                }
                a.xsneg[c * a.Mp + m] = -kR4Bias * s;
            }
        }
        return;
    }

    const int64_t ncol = a.k + a.r;
    const int64_t c0 = ((int64_t)blockIdx.x * 4 + wv) * kProjNI;
    if (c0 >= ncol)
        return;
    const int8_t *wrow[kProjNI];
    bool isd[kProjNI];
    int64_t colc[kProjNI];
    for (int ci = 0; ci < kProjNI; ++ci) {
        colc[ci] = c0 + ci < ncol ? c0 + ci : ncol - 1;
        isd[ci] = colc[ci] >= a.k;
        wrow[ci] = isd[ci] ? a.d8 + (colc[ci] - a.k) * a.d : a.b8 + colc[ci] * a.d;
    }
    float acc[kProjNI][kProjMB];
    for (int ci = 0; ci < kProjNI; ++ci)
        for (int mi = 0; mi < kProjMB; ++mi)
            acc[ci][mi] = 0.f;

    const u32x4 z = {0u, 0u, 0u, 0u};
    // four 1024-column slabs per pass: every load of a pass is issued before
    // the first multiply, so a pass costs one memory latency
    for (int64_t j00 = 0; j00 < a.d; j00 += 4096) {
        u32x4 wq[kProjNI][4];
        float sc[kProjNI][4];
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int64_t j0 = j00 + 1024 * it + 16 * lane;
            const bool ok = j0 < a.d;
            for (int ci = 0; ci < kProjNI; ++ci) {
                wq[ci][it] = ok ? *(const u32x4 *)(wrow[ci] + j0) : z;
                sc[ci][it] = (ok && isd[ci]) ? a.sd[(colc[ci] - a.k) * a.G + j0 / a.g] : 1.0f;
            }
        }
        for (int mi = 0; mi < kProjMB; ++mi) {
            const int64_t m = m0 + mi;
            if (m >= a.M)
                break;
            u32x4 x0[4], x1[4];
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int64_t j0 = j00 + 1024 * it + 16 * lane;
                const bool ok = j0 < a.d;
                const u32x4 *xp = (const u32x4 *)(a.X + m * a.d + (ok ? j0 : 0));
                x0[it] = ok ? xp[0] : z;
                x1[it] = ok ? xp[1] : z;
            }
#pragma unroll
            for (int it = 0; it < 4; ++it)
                for (int ci = 0; ci < kProjNI; ++ci)
                    acc[ci][mi] = __builtin_fmaf(sc[ci][it], dot16(wq[ci][it], x0[it], x1[it]), acc[ci][mi]);
        }
    }
    for (int ci = 0; ci < kProjNI; ++ci)
        for (int mi = 0; mi < kProjMB; ++mi) {
            float v = acc[ci][mi];
            for (int off = 32; off >= 1; off >>= 1)
                v += __shfl_xor(v, off);
            acc[ci][mi] = v;
        }
    for (int ci = 0; ci < kProjNI; ++ci) {
        const int64_t col = c0 + ci;
        if (col >= ncol)
            break;
        for (int mi = 0; mi < kProjMB; ++mi) {
            const int64_t m = m0 + mi;
            if (m >= a.M || lane != ci * kProjMB + mi)
                continue;
            float t = isd[ci] ? acc[ci][mi] : acc[ci][mi] * a.sb[col];
            uint16_t hi = f32_to_bf16_rne(t);
            uint16_t lo = f32_to_bf16_rne(t - __uint_as_float((uint32_t)hi << 16));
            if (isd[ci]) {
                const int64_t i = col - a.k;
                a.s16[m * a.rpad + i] = hi;
                a.s16[(a.Mp + m) * a.rpad + i] = lo;
            } else {
                a.t16[m * a.kpad + col] = hi;
                a.t16[(a.Mp + m) * a.kpad + col] = lo;
            }
        }
    }
}

hipError_t launch_proj(const DevHead &h, const Work &w, const uint16_t *X, hipStream_t st)
{
    ProjArgs a;
    a.X = X;
    a.M = w.M;
    a.Mp = w.Mp;
    a.d = h.s.d;
    a.k = h.s.k;
    a.r = h.s.r;
    a.g = h.s.g;
    a.G = h.s.G();
    a.kpad = h.s.kpad();
    a.rpad = h.s.rpad();
    a.b8 = h.b8;
    a.sb = h.sb;
    a.d8 = h.d8;
    a.sd = h.sd;
    a.t16 = w.t16;
    a.s16 = w.s16;
    a.xsneg = w.xsneg;
    const int64_t ncol = h.s.k + h.s.r;
    a.ncolblk = (int)((ncol + 4 * kProjNI - 1) / (4 * kProjNI));
    dim3 grid(a.ncolblk + 1, (unsigned)((w.M + kProjMB - 1) / kProjMB));
    hipLaunchKernelGGL(proj_kernel, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// a2-S: skinny vocabulary-tile kernel.
//
// One wave owns NV v-blocks (16 vocabulary rows each) and MT 16-row tiles of
// hidden states.  For every K-step of 32 columns it turns one residual dword
// per lane into 8 exact bf16 integers (q + 136) and issues
// v_mfma_f32_16x16x32_bf16 with the hidden states as the A operand, so the
// MFMA output tile is [16 hidden states x 16 vocabulary rows].  Each g-group
// is accumulated on its own, then folded into the running logits with its
// fp32 scale sR[v, grp] after adding the group's offset correction
// (-136 sum X).  The low-rank terms are a K-extension done first, while the
// first residual chunks are in flight: bf16 hi/lo of t and s against exact
// bf16 codes of A5 (a + 144, the offset removed by an MFMA against the
// constant -144) and C8, folded in with sA[v] and sC[v].
//
// Everything one residual chunk (128 columns) needs -- the residual dwords,
// the hidden-state fragments, the group scales and offsets -- is loaded one
// chunk ahead into a register buffer, so the MFMA loop never waits on a load
// issued in the same iteration.
// ---------------------------------------------------------------------------
struct VtArgs {
    DevHead h;
    Work w;
    const uint16_t *X;
    float *logits;
    int32_t *argmax;
    int64_t nvb, nkc, G;
    int gsteps;
    int want_argmax;
    unsigned lds_sr, lds_xs, lds_x; // byte offsets of the LDS regions
};

template <int NV, int MT, bool XL>
struct SkChunk {
    u32x4 r4[NV];
    u32x4 xf[XL ? 1 : MT][4]; // hidden-state fragments (global-memory variant only)
};

// LDS staging of one workgroup (4 waves x NV v-blocks):
//   sr  [4*NV][G][16] fp16  residual scales of the workgroup's v-blocks
//   xs  [G][MT*16]    fp32  -136 x per-group sums of X for the m-tile
//   x   [M][d]        bf16  the hidden states (XL only, small M*d)
// so that the only vector-memory loads in the streaming loop are the
// residual nibbles themselves.
// Decode instantiations (X in LDS) are held to three waves per SIMD so that a
// whole grid of 4-v-block waves is resident at once.
template <int NV, int MT, int GS, bool XL>
__global__ __launch_bounds__(256, XL ? 3 : 1) void vtile_skinny_kernel(VtArgs a)
{
    extern __shared__ __attribute__((aligned(16))) char smem[];
    uint16_t *s_sr = (uint16_t *)(smem + a.lds_sr);
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

    // ---- stage scales, group offsets and (small) X in LDS ----
    {
        const int64_t nvb_wg = (nvb - wg_vb0) < 4 * NV ? (nvb - wg_vb0) : 4 * NV;
        const int64_t n16 = nvb_wg * G * kVB / 8; // 16-byte pieces of sr
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

    const uint16_t *xp[MT];
    for (int mt = 0; mt < MT; ++mt) {
        const int64_t m = mbase + mt * 16 + lr;
        xp[mt] = a.X + (m < M ? m : M - 1) * d + 8 * lq;
    }
    const uint16_t *xl = s_x + (lr < M ? lr : M - 1) * d + 8 * lq; // XL: MT == 1, mbase == 0

    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 acc[NV][MT], accg[NV][MT];
    for (int v = 0; v < NV; ++v)
        for (int mt = 0; mt < MT; ++mt)
            acc[v][mt] = zero, accg[v][mt] = zero;

    auto group_start = [&](int64_t ks) {
        if (GS == 1) return true;
        if (GS == 2 || GS == 4) return (ks % (GS ? GS : 1)) == 0;
        return (ks % gsteps) == 0;
    };
    auto group_end = [&](int64_t ks) {
        if (GS == 1) return true;
        if (GS == 2 || GS == 4) return (ks % (GS ? GS : 1)) == (GS ? GS : 1) - 1;
        return (ks % gsteps) == gsteps - 1;
    };

    const u32x4 *r4 = (const u32x4 *)a.h.r4;
    auto load_chunk = [&](SkChunk<NV, MT, XL> &c, int64_t kc) {
        for (int v = 0; v < NV; ++v)
            c.r4[v] = __builtin_nontemporal_load(&r4[(kc * nvb + vb[v]) * 64 + lane]);
        if (!XL) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
                for (int mt = 0; mt < MT; ++mt)
                    c.xf[mt][s] = *(const u32x4 *)(xp[mt] + (kc * 4 + s) * kKStep);
        }
    };

    const uint32_t kMagic = vgpr_const(kBf16Magic);
    f32x4 xs_cur[MT];
    for (int mt = 0; mt < MT; ++mt)
        xs_cur[mt] = zero;
    auto do_chunk = [&](const SkChunk<NV, MT, XL> &c, int64_t kc) {
        u32x4 xf[MT][4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
            for (int mt = 0; mt < MT; ++mt)
                xf[mt][s] = XL ? *(const u32x4 *)(xl + (kc * 4 + s) * kKStep) : c.xf[XL ? 0 : mt][s];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int64_t ks = kc * 4 + s;
            const int64_t grp = ks / gsteps;
            if (group_start(ks)) {
                for (int mt = 0; mt < MT; ++mt)
                    xs_cur[mt] = *(const f32x4 *)(s_xs + grp * (MT * 16) + mt * 16 + 4 * lq);
                for (int v = 0; v < NV; ++v)
                    for (int mt = 0; mt < MT; ++mt)
                        accg[v][mt] = zero;
            }
            for (int v = 0; v < NV; ++v) {
                const uint32_t wd = s == 0 ? c.r4[v].x : s == 1 ? c.r4[v].y : s == 2 ? c.r4[v].z : c.r4[v].w;
                const u32x4 b = r4_bf16(wd, kMagic);
                for (int mt = 0; mt < MT; ++mt)
                    accg[v][mt] = mfma_bf16(xf[mt][s], b, accg[v][mt]);
            }
            if (group_end(ks)) {
                for (int v = 0; v < NV; ++v) {
                    const float sc = h2f(s_sr[((wv * NV + v) * G + grp) * kVB + lr]);
                    for (int mt = 0; mt < MT; ++mt)
                        for (int i = 0; i < 4; ++i)
                            acc[v][mt][i] = __builtin_fmaf(sc, accg[v][mt][i] + xs_cur[mt][i], acc[v][mt][i]);
                }
            }
        }
    };

    // three residual chunks in flight from the start
    SkChunk<NV, MT, XL> bufA, bufB, bufC;
    if (active) {
        load_chunk(bufA, 0);
        load_chunk(bufB, nkc > 1 ? 1 : 0);
        load_chunk(bufC, nkc > 2 ? 2 : 0);
    }

    const int64_t kpad = a.h.s.kpad(), rpad = a.h.s.rpad();
    const int64_t kst = a.h.s.kst(), rst = a.h.s.rst(), ahg = a.h.s.a5h_groups();

    // residual stream: the steady-state loops keep three chunks in flight and
    // have no branch around a load; the scheduling barriers stop the compiler
    // from sinking the prefetches to the end of the loop body
    if (active && GS == 4) {
        // One g-group per chunk.  Each chunk buffer has its own group
        // accumulator, and a group is folded in with its scale one chunk
        // later, after the next chunk's MFMAs are issued: reading an
        // accumulator right after its MFMAs would stall the wave until the
        // matrix pipeline drains, once per chunk.
        f32x4 gA[NV][MT], gB[NV][MT], gC[NV][MT];
        auto mfma_chunk = [&](const SkChunk<NV, MT, XL> &c, int64_t kc, f32x4(&g)[NV][MT]) {
            u32x4 xf[MT][4];
#pragma unroll
            for (int s = 0; s < 4; ++s)
                for (int mt = 0; mt < MT; ++mt)
                    xf[mt][s] = XL ? *(const u32x4 *)(xl + (kc * 4 + s) * kKStep) : c.xf[XL ? 0 : mt][s];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                for (int v = 0; v < NV; ++v) {
                    const uint32_t wd = s == 0 ? c.r4[v].x : s == 1 ? c.r4[v].y : s == 2 ? c.r4[v].z : c.r4[v].w;
                    const u32x4 b = r4_bf16(wd, kMagic);
                    for (int mt = 0; mt < MT; ++mt)
                        g[v][mt] = mfma_bf16(xf[mt][s], b, s == 0 ? zero : g[v][mt]);
                }
                // one K-step at a time: hoisting every dequantised operand of
                // the chunk ahead of the MFMAs costs occupancy for no gain
                __builtin_amdgcn_sched_barrier(0);
            }
        };
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
        int64_t kc = 0;
        if (nkc > 5) {
            mfma_chunk(bufA, 0, gA);
            load_chunk(bufA, 3);
            __builtin_amdgcn_sched_barrier(0);
            mfma_chunk(bufB, 1, gB);
            fold(gA, 0);
            load_chunk(bufB, 4);
            __builtin_amdgcn_sched_barrier(0);
            mfma_chunk(bufC, 2, gC);
            fold(gB, 1);
            load_chunk(bufC, 5);
            __builtin_amdgcn_sched_barrier(0);
            for (kc = 3; kc + 5 < nkc; kc += 3) {
                mfma_chunk(bufA, kc, gA);
                fold(gC, kc - 1);
                load_chunk(bufA, kc + 3);
                __builtin_amdgcn_sched_barrier(0);
                mfma_chunk(bufB, kc + 1, gB);
                fold(gA, kc);
                load_chunk(bufB, kc + 4);
                __builtin_amdgcn_sched_barrier(0);
                mfma_chunk(bufC, kc + 2, gC);
                fold(gB, kc + 1);
                load_chunk(bufC, kc + 5);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // tail: chunks kc .. nkc-1 (at most five) in buffers A, B, C, A, B;
        // gC holds chunk kc-1's group when kc > 0
        mfma_chunk(bufA, kc, gA);
        if (kc > 0)
            fold(gC, kc - 1);
        if (kc + 3 < nkc)
            load_chunk(bufA, kc + 3);
        if (kc + 1 < nkc) {
            mfma_chunk(bufB, kc + 1, gB);
            if (kc + 4 < nkc)
                load_chunk(bufB, kc + 4);
        }
        fold(gA, kc);
        if (kc + 2 < nkc)
            mfma_chunk(bufC, kc + 2, gC);
        if (kc + 1 < nkc)
            fold(gB, kc + 1);
        if (kc + 3 < nkc)
            mfma_chunk(bufA, kc + 3, gA);
        if (kc + 2 < nkc)
            fold(gC, kc + 2);
        if (kc + 4 < nkc)
            mfma_chunk(bufB, kc + 4, gB);
        if (kc + 3 < nkc)
            fold(gA, kc + 3);
        if (kc + 4 < nkc)
            fold(gB, kc + 4);
    } else if (active) {
        int64_t kc = 0;
        for (; kc + 5 < nkc; kc += 3) {
            do_chunk(bufA, kc);
            load_chunk(bufA, kc + 3);
            __builtin_amdgcn_sched_barrier(0);
            do_chunk(bufB, kc + 1);
            load_chunk(bufB, kc + 4);
            __builtin_amdgcn_sched_barrier(0);
            do_chunk(bufC, kc + 2);
            load_chunk(bufC, kc + 5);
            __builtin_amdgcn_sched_barrier(0);
        }
        // tail: chunks kc .. nkc-1 (at most five), A/B/C hold kc, kc+1, kc+2
        do_chunk(bufA, kc);
        if (kc + 3 < nkc)
            load_chunk(bufA, kc + 3);
        if (kc + 1 < nkc) {
            do_chunk(bufB, kc + 1);
            if (kc + 4 < nkc)
                load_chunk(bufB, kc + 4);
        }
        if (kc + 2 < nkc)
            do_chunk(bufC, kc + 2);
        if (kc + 3 < nkc)
            do_chunk(bufA, kc + 3);
        if (kc + 4 < nkc)
            do_chunk(bufB, kc + 4);
    }

    // Low-rank terms after the residual stream, so that their registers are
    // not live next to the three prefetch buffers.
    // correction term: (X B_w^T) A_w^T with C8 codes, scale sC[v]
    if (active && rst > 0) {
        for (int v = 0; v < NV; ++v)
            for (int mt = 0; mt < MT; ++mt)
                accg[v][mt] = zero;
        for (int64_t ks = 0; ks < rst; ++ks) {
            u32x4 sh[MT], sl[MT];
            u32x2 c[NV];
            for (int mt = 0; mt < MT; ++mt) {
                const int64_t m = mbase + mt * 16 + lr;
                sh[mt] = *(const u32x4 *)(a.w.s16 + m * rpad + ks * kKStep + 8 * lq);
                sl[mt] = *(const u32x4 *)(a.w.s16 + (Mp + m) * rpad + ks * kKStep + 8 * lq);
            }
            for (int v = 0; v < NV; ++v)
                c[v] = *(const u32x2 *)(a.h.c8 + ((vb[v] * rst + ks) * 64 + lane) * 2);
            for (int v = 0; v < NV; ++v) {
                const u32x4 b = c8_bf16(c[v]);
                for (int mt = 0; mt < MT; ++mt) {
                    accg[v][mt] = mfma_bf16(sh[mt], b, accg[v][mt]);
                    accg[v][mt] = mfma_bf16(sl[mt], b, accg[v][mt]);
                }
            }
        }
        for (int v = 0; v < NV; ++v) {
            const float sc = h2f(a.h.sc[vb[v] * kVB + lr]);
            for (int mt = 0; mt < MT; ++mt)
                for (int i = 0; i < 4; ++i)
                    acc[v][mt][i] = __builtin_fmaf(sc, accg[v][mt][i], acc[v][mt][i]);
        }
    }

    // core term: (X (sB o B8)^T)(sA o A5)^T with 5-bit codes a + 144
    if (active && kst > 0) {
        const u32x4 neg144 = {0xC310C310u, 0xC310C310u, 0xC310C310u, 0xC310C310u};
        f32x4 nt[MT];
        for (int mt = 0; mt < MT; ++mt)
            nt[mt] = zero;
        for (int v = 0; v < NV; ++v)
            for (int mt = 0; mt < MT; ++mt)
                accg[v][mt] = zero;
        for (int64_t g4 = 0; g4 < ahg; ++g4) {
            uint32_t wh[NV], wn[NV][4];
            u32x4 th[MT][4], tl[MT][4];
            const int nq = (int)(kst - g4 * 4 < 4 ? kst - g4 * 4 : 4);
            for (int v = 0; v < NV; ++v)
                wh[v] = a.h.a5h[(vb[v] * ahg + g4) * 64 + lane];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (q >= nq)
                    break;
                const int64_t ks = g4 * 4 + q;
                for (int v = 0; v < NV; ++v)
                    wn[v][q] = a.h.a5n[(vb[v] * kst + ks) * 64 + lane];
                for (int mt = 0; mt < MT; ++mt) {
                    const int64_t m = mbase + mt * 16 + lr;
                    th[mt][q] = *(const u32x4 *)(a.w.t16 + m * kpad + ks * kKStep + 8 * lq);
                    tl[mt][q] = *(const u32x4 *)(a.w.t16 + (Mp + m) * kpad + ks * kKStep + 8 * lq);
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (q >= nq)
                    break;
                for (int mt = 0; mt < MT; ++mt) {
                    nt[mt] = mfma_bf16(th[mt][q], neg144, nt[mt]);
                    nt[mt] = mfma_bf16(tl[mt][q], neg144, nt[mt]);
                }
                for (int v = 0; v < NV; ++v) {
                    const u32x4 b = a5_bf16_q(wn[v][q], wh[v], q);
                    for (int mt = 0; mt < MT; ++mt) {
                        accg[v][mt] = mfma_bf16(th[mt][q], b, accg[v][mt]);
                        accg[v][mt] = mfma_bf16(tl[mt][q], b, accg[v][mt]);
                    }
                }
            }
        }
        for (int v = 0; v < NV; ++v) {
            const float sc = h2f(a.h.sa[vb[v] * kVB + lr]);
            for (int mt = 0; mt < MT; ++mt)
                for (int i = 0; i < 4; ++i)
                    acc[v][mt][i] = __builtin_fmaf(sc, accg[v][mt][i] + nt[mt][i], acc[v][mt][i]);
        }
    }

    // epilogue: logits, then the per-workgroup argmax partial of every hidden state
    uint64_t key[MT][4];
    for (int mt = 0; mt < MT; ++mt) {
        for (int i = 0; i < 4; ++i) {
            const int64_t m = mbase + mt * 16 + 4 * lq + i;
            uint64_t k = 0;
            if (active) {
                for (int v = 0; v < NV; ++v) {
                    const int64_t row = vb0 + v < nvb ? (vb0 + v) * kVB + lr : V;
                    const bool ok = row < V && m < M;
                    const float y = acc[v][mt][i];
                    if (ok && a.logits)
                        a.logits[m * V + row] = y;
                    if (ok)
                        k = umax64(k, argmax_key(y, (uint32_t)row));
                }
            }
            key[mt][i] = k;
        }
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
    const int64_t n_part = a.w.n_part;
    if (threadIdx.x < MT * 16) {
        const int64_t m = mbase + threadIdx.x;
        const uint64_t k = umax64(umax64(red[0][threadIdx.x], red[1][threadIdx.x]),
                                  umax64(red[2][threadIdx.x], red[3][threadIdx.x]));
        if (m < M)
            a.w.part[m * n_part + blockIdx.x] = k;
    }
}

constexpr int kSkinnyNV = 4;
constexpr int64_t kXLdsMaxBytes = 48 * 1024; // X staged in LDS when M*d*2 fits

int64_t skinny_n_part(const DevHead &h, int64_t M)
{
    (void)M;
    return (h.s.nvb() + 4 * kSkinnyNV - 1) / (4 * kSkinnyNV);
}

template <int MT, int GS, bool XL>
static hipError_t launch_sk(const VtArgs &a, dim3 grid, size_t lds, hipStream_t st)
{
    auto k = vtile_skinny_kernel<kSkinnyNV, MT, GS, XL>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL(k, grid, dim3(256), lds, st, a);
    return hipGetLastError();
}

template <int MT, bool XL>
static hipError_t launch_sk_gs(const VtArgs &a, dim3 grid, size_t lds, hipStream_t st)
{
    switch (a.gsteps) {
    case 1: return launch_sk<MT, 1, XL>(a, grid, lds, st);
    case 2: return launch_sk<MT, 2, XL>(a, grid, lds, st);
    case 4: return launch_sk<MT, 4, XL>(a, grid, lds, st);
    default: return launch_sk<MT, 0, XL>(a, grid, lds, st);
    }
}

hipError_t launch_vtile_skinny(const DevHead &h, const Work &w, const uint16_t *X, float *logits,
                               int32_t *argmax, hipStream_t st, bool *argmax_done)
{
    VtArgs a;
    a.h = h;
    a.w = w;
    a.X = X;
    a.logits = logits;
    a.argmax = argmax;
    a.nvb = h.s.nvb();
    a.nkc = h.s.nkc();
    a.G = h.s.G();
    a.gsteps = (int)(h.s.g / kKStep);
    a.want_argmax = argmax ? 1 : 0;
    a.w.n_part = skinny_n_part(h, w.M);
    const unsigned gx = (unsigned)a.w.n_part;
    const int MT = w.M <= 16 ? 1 : 2;
    const unsigned gy = (unsigned)((w.M + 16 * MT - 1) / (16 * MT));
    // The top-1 reduction across workgroups runs as its own kernel: finishing
    // it inside this one (last workgroup reduces) needs a device-scope fence
    // per workgroup, which writes back the L2 of a multi-XCD part and costs
    // more than a kernel launch.
    *argmax_done = false;
    const bool XL = MT == 1 && w.M * h.s.d * 2 <= kXLdsMaxBytes;
    auto al = [](size_t x) { return (x + 15) / 16 * 16; };
    a.lds_sr = 0;
    a.lds_xs = (unsigned)al(size_t(4) * kSkinnyNV * a.G * kVB * 2);
    a.lds_x = (unsigned)(a.lds_xs + al(size_t(a.G) * MT * 16 * 4));
    const size_t lds = a.lds_x + (XL ? al(size_t(w.M) * h.s.d * 2) : 0);
    if (MT == 1)
        return XL ? launch_sk_gs<1, true>(a, dim3(gx, gy), lds, st)
                  : launch_sk_gs<1, false>(a, dim3(gx, gy), lds, st);
    return launch_sk_gs<2, false>(a, dim3(gx, gy), lds, st);
}

// ---------------------------------------------------------------------------
// a3: top-1 reduction across vocabulary tiles.  Keys order by value, then by
// lower index, so the maximum key is the first index of the maximum logit.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void argmax_kernel(const uint64_t *part, int64_t n_part,
                                                     int32_t *out, int64_t M)
{
    __shared__ uint64_t red[4];
    const int64_t m = blockIdx.x;
    if (m >= M)
        return;
    uint64_t key = 0;
    for (int64_t i = threadIdx.x; i < n_part; i += 256)
        key = umax64(key, part[m * n_part + i]);
    for (int off = 32; off >= 1; off >>= 1)
        key = umax64(key, shfl_xor_u64(key, off));
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = key;
    __syncthreads();
    if (threadIdx.x == 0) {
        key = umax64(umax64(red[0], red[1]), umax64(red[2], red[3]));
        out[m] = (int32_t)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFu));
    }
}

hipError_t launch_argmax(const Work &w, int64_t n_part, int32_t *argmax, hipStream_t st)
{
    hipLaunchKernelGGL(argmax_kernel, dim3((unsigned)w.M), dim3(256), 0, st, w.part, n_part,
                       argmax, w.M);
    return hipGetLastError();
}

} // namespace archead
