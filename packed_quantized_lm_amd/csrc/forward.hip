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
constexpr int kProjNI = 4; // output columns per wave
constexpr int kProjMB = 8; // hidden states per workgroup

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
    for (int ci = 0; ci < kProjNI; ++ci) {
        int64_t col = c0 + ci < ncol ? c0 + ci : ncol - 1;
        isd[ci] = col >= a.k;
        wrow[ci] = isd[ci] ? a.d8 + (col - a.k) * a.d : a.b8 + col * a.d;
    }
    float acc[kProjNI][kProjMB];
    for (int ci = 0; ci < kProjNI; ++ci)
        for (int mi = 0; mi < kProjMB; ++mi)
            acc[ci][mi] = 0.f;

    for (int64_t j0 = 16 * lane; j0 < a.d; j0 += 1024) {
        float w[kProjNI][16];
        float sc[kProjNI];
        for (int ci = 0; ci < kProjNI; ++ci) {
            u32x4 q = *(const u32x4 *)(wrow[ci] + j0);
            for (int b = 0; b < 4; ++b) {
                w[ci][b] = i8(q.x, b);
                w[ci][4 + b] = i8(q.y, b);
                w[ci][8 + b] = i8(q.z, b);
                w[ci][12 + b] = i8(q.w, b);
            }
            int64_t col = c0 + ci < ncol ? c0 + ci : ncol - 1;
            sc[ci] = isd[ci] ? a.sd[(col - a.k) * a.G + j0 / a.g] : 1.0f;
        }
        for (int mi = 0; mi < kProjMB; ++mi) {
            const int64_t m = m0 + mi;
            if (m >= a.M)
                break;
            const u32x4 *xp = (const u32x4 *)(a.X + m * a.d + j0);
            u32x4 x0 = xp[0], x1 = xp[1];
            float x[16] = {bf_lo(x0.x), bf_hi(x0.x), bf_lo(x0.y), bf_hi(x0.y),
                           bf_lo(x0.z), bf_hi(x0.z), bf_lo(x0.w), bf_hi(x0.w),
                           bf_lo(x1.x), bf_hi(x1.x), bf_lo(x1.y), bf_hi(x1.y),
                           bf_lo(x1.z), bf_hi(x1.z), bf_lo(x1.w), bf_hi(x1.w)};
            for (int ci = 0; ci < kProjNI; ++ci) {
                float dsum = 0.f;
                for (int e = 0; e < 16; ++e)
                    dsum = __builtin_fmaf(x[e], w[ci][e], dsum);
                acc[ci][mi] = __builtin_fmaf(sc[ci], dsum, acc[ci][mi]);
            }
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
// (-136 sum X).  The low-rank terms follow as a K-extension: bf16 hi/lo of t
// and s against exact bf16 codes of A5 (a + 144, offset removed by an MFMA
// against the constant -144) and C8, folded in with sA[v] and sC[v].
// ---------------------------------------------------------------------------
struct VtArgs {
    DevHead h;
    Work w;
    const uint16_t *X;
    float *logits;
    int64_t nvb, nkc, G;
    int gsteps;
    int want_argmax;
};

template <int NV, int MT, int GS>
__global__ __launch_bounds__(256) void vtile_skinny_kernel(VtArgs a)
{
    const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nvb = a.nvb, nkc = a.nkc, G = a.G;
    const int64_t vb0 = wave * NV;
    if (vb0 >= nvb)
        return;
    const int64_t M = a.w.M, Mp = a.w.Mp, d = a.h.s.d, V = a.h.s.V;
    const int64_t mbase = (int64_t)blockIdx.y * (MT * 16);
    const int gsteps = GS ? GS : a.gsteps;

    int64_t vb[NV];
    for (int v = 0; v < NV; ++v)
        vb[v] = vb0 + v < nvb ? vb0 + v : nvb - 1;

    const uint16_t *xp[MT];
    bool xok[MT];
    for (int mt = 0; mt < MT; ++mt) {
        const int64_t m = mbase + mt * 16 + lr;
        xok[mt] = m < M;
        xp[mt] = a.X + (xok[mt] ? m : 0) * d + 8 * lq;
    }

    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 acc[NV][MT], accg[NV][MT];
    for (int v = 0; v < NV; ++v)
        for (int mt = 0; mt < MT; ++mt)
            acc[v][mt] = zero, accg[v][mt] = zero;
    f32x4 xs[MT];
    for (int mt = 0; mt < MT; ++mt)
        xs[mt] = zero;
    uint16_t srv[NV];
    for (int v = 0; v < NV; ++v)
        srv[v] = 0;

    const u32x4 *r4 = (const u32x4 *)a.h.r4;
    auto load_chunk = [&](u32x4(&wb)[NV], int64_t kc) {
        for (int v = 0; v < NV; ++v)
            wb[v] = __builtin_nontemporal_load(&r4[(vb[v] * nkc + kc) * 64 + lane]);
    };

    auto do_chunk = [&](const u32x4(&wb)[NV], int64_t kc) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int64_t ks = kc * 4 + s;
            bool first, last;
            if (GS == 1) {
                first = last = true;
            } else if (GS == 2 || GS == 4) {
                constexpr int gs = GS ? GS : 1;
                first = (s % gs) == 0;
                last = (s % gs) == gs - 1;
            } else {
                first = (ks % gsteps) == 0;
                last = (ks % gsteps) == gsteps - 1;
            }
            const int64_t grp = ks / gsteps;
            if (first) {
                for (int mt = 0; mt < MT; ++mt)
                    xs[mt] = *(const f32x4 *)(a.w.xsneg + grp * Mp + mbase + mt * 16 + 4 * lq);
                for (int v = 0; v < NV; ++v) {
                    srv[v] = a.h.sr[(vb[v] * G + grp) * kVB + lr];
                    for (int mt = 0; mt < MT; ++mt)
                        accg[v][mt] = zero;
                }
            }
            u32x4 xf[MT];
            for (int mt = 0; mt < MT; ++mt) {
                u32x4 z = {0u, 0u, 0u, 0u};
                xf[mt] = xok[mt] ? *(const u32x4 *)(xp[mt] + ks * kKStep) : z;
            }
            for (int v = 0; v < NV; ++v) {
                const uint32_t wd = s == 0 ? wb[v].x : s == 1 ? wb[v].y : s == 2 ? wb[v].z : wb[v].w;
                const u32x4 b = r4_bf16(wd);
                for (int mt = 0; mt < MT; ++mt)
                    accg[v][mt] = mfma_bf16(xf[mt], b, accg[v][mt]);
            }
            if (last) {
                for (int v = 0; v < NV; ++v) {
                    const float sc = h2f(srv[v]);
                    for (int mt = 0; mt < MT; ++mt)
                        for (int i = 0; i < 4; ++i)
                            acc[v][mt][i] = __builtin_fmaf(sc, accg[v][mt][i] + xs[mt][i], acc[v][mt][i]);
                }
            }
        }
    };

    // residual stream, double buffered
    u32x4 bufA[NV], bufB[NV];
    load_chunk(bufA, 0);
    if (nkc > 1)
        load_chunk(bufB, 1);
    for (int64_t kc = 0; kc < nkc; kc += 2) {
        do_chunk(bufA, kc);
        if (kc + 2 < nkc)
            load_chunk(bufA, kc + 2);
        if (kc + 1 < nkc) {
            do_chunk(bufB, kc + 1);
            if (kc + 3 < nkc)
                load_chunk(bufB, kc + 3);
        }
    }

    const int64_t kpad = a.h.s.kpad(), rpad = a.h.s.rpad();
    const int64_t kst = a.h.s.kst(), rst = a.h.s.rst(), ahg = a.h.s.a5h_groups();

    // correction term: (X B_w^T) A_w^T with C8 codes, scale sC[v]
    if (rst > 0) {
        for (int v = 0; v < NV; ++v)
            for (int mt = 0; mt < MT; ++mt)
                accg[v][mt] = zero;
        for (int64_t ks = 0; ks < rst; ++ks) {
            u32x4 sh[MT], sl[MT];
            for (int mt = 0; mt < MT; ++mt) {
                const int64_t m = mbase + mt * 16 + lr;
                sh[mt] = *(const u32x4 *)(a.w.s16 + m * rpad + ks * kKStep + 8 * lq);
                sl[mt] = *(const u32x4 *)(a.w.s16 + (Mp + m) * rpad + ks * kKStep + 8 * lq);
            }
            for (int v = 0; v < NV; ++v) {
                const u32x2 c = *(const u32x2 *)(a.h.c8 + ((vb[v] * rst + ks) * 64 + lane) * 2);
                const u32x4 b = c8_bf16(c);
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
    if (kst > 0) {
        const u32x4 neg144 = {0xC310C310u, 0xC310C310u, 0xC310C310u, 0xC310C310u};
        f32x4 nt[MT];
        for (int mt = 0; mt < MT; ++mt)
            nt[mt] = zero;
        for (int v = 0; v < NV; ++v)
            for (int mt = 0; mt < MT; ++mt)
                accg[v][mt] = zero;
        for (int64_t g4 = 0; g4 < ahg; ++g4) {
            uint32_t wh[NV];
            for (int v = 0; v < NV; ++v)
                wh[v] = a.h.a5h[(vb[v] * ahg + g4) * 64 + lane];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t ks = g4 * 4 + q;
                if (ks >= kst)
                    break;
                u32x4 th[MT], tl[MT];
                for (int mt = 0; mt < MT; ++mt) {
                    const int64_t m = mbase + mt * 16 + lr;
                    th[mt] = *(const u32x4 *)(a.w.t16 + m * kpad + ks * kKStep + 8 * lq);
                    tl[mt] = *(const u32x4 *)(a.w.t16 + (Mp + m) * kpad + ks * kKStep + 8 * lq);
                    nt[mt] = mfma_bf16(th[mt], neg144, nt[mt]);
                    nt[mt] = mfma_bf16(tl[mt], neg144, nt[mt]);
                }
                for (int v = 0; v < NV; ++v) {
                    const uint32_t wn = a.h.a5n[(vb[v] * kst + ks) * 64 + lane];
                    const u32x4 b = a5_bf16_q(wn, wh[v], q);
                    for (int mt = 0; mt < MT; ++mt) {
                        accg[v][mt] = mfma_bf16(th[mt], b, accg[v][mt]);
                        accg[v][mt] = mfma_bf16(tl[mt], b, accg[v][mt]);
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

    // epilogue: logits and the per-wave argmax partial of every hidden state
    for (int mt = 0; mt < MT; ++mt) {
        for (int i = 0; i < 4; ++i) {
            const int64_t m = mbase + mt * 16 + 4 * lq + i;
            uint64_t key = 0;
            for (int v = 0; v < NV; ++v) {
                const int64_t row = vb0 + v < nvb ? (vb0 + v) * kVB + lr : V;
                const bool ok = row < V && m < M;
                const float y = acc[v][mt][i];
                if (ok && a.logits)
                    a.logits[m * V + row] = y;
                if (ok)
                    key = umax64(key, argmax_key(y, (uint32_t)row));
            }
            if (a.want_argmax) {
                key = umax64(key, shfl_xor_u64(key, 1));
                key = umax64(key, shfl_xor_u64(key, 2));
                key = umax64(key, shfl_xor_u64(key, 4));
                key = umax64(key, shfl_xor_u64(key, 8));
                if (lr == 0 && m < M)
                    a.w.part[m * a.w.n_part + wave] = key;
            }
        }
    }
}

constexpr int kSkinnyNV = 4;

int64_t skinny_n_part(const DevHead &h, int64_t M)
{
    (void)M;
    return (h.s.nvb() + kSkinnyNV - 1) / kSkinnyNV;
}

template <int MT, int GS>
static void launch_sk(const VtArgs &a, dim3 grid, hipStream_t st)
{
    hipLaunchKernelGGL((vtile_skinny_kernel<kSkinnyNV, MT, GS>), grid, dim3(256), 0, st, a);
}

template <int MT>
static void launch_sk_gs(const VtArgs &a, dim3 grid, hipStream_t st)
{
    switch (a.gsteps) {
    case 1: launch_sk<MT, 1>(a, grid, st); break;
    case 2: launch_sk<MT, 2>(a, grid, st); break;
    case 4: launch_sk<MT, 4>(a, grid, st); break;
    default: launch_sk<MT, 0>(a, grid, st); break;
    }
}

hipError_t launch_vtile_skinny(const DevHead &h, const Work &w, const uint16_t *X, float *logits,
                               bool want_argmax, hipStream_t st, int64_t *n_part_out)
{
    VtArgs a;
    a.h = h;
    a.w = w;
    a.X = X;
    a.logits = logits;
    a.nvb = h.s.nvb();
    a.nkc = h.s.nkc();
    a.G = h.s.G();
    a.gsteps = (int)(h.s.g / kKStep);
    a.want_argmax = want_argmax ? 1 : 0;
    const int64_t waves = (a.nvb + kSkinnyNV - 1) / kSkinnyNV;
    *n_part_out = waves;
    a.w.n_part = waves;
    if (w.M <= 16) {
        dim3 grid((unsigned)((waves + 3) / 4), 1);
        launch_sk_gs<1>(a, grid, st);
    } else {
        dim3 grid((unsigned)((waves + 3) / 4), (unsigned)((w.M + 31) / 32));
        launch_sk_gs<2>(a, grid, st);
    }
    return hipGetLastError();
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
