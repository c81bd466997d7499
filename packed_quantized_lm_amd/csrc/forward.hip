// forward.hip -- projection, skinny vocabulary-tile and argmax kernels of the
// packed ARCHead head forward on gfx950.
//
// ARCHead paper, section 3.2, eq 7: logits = X W_d^T + (X B_w^T) A_w^T, with
// W_d = Q5(A_c) Q8(B_c) + Q_SC4(...) (eq 3) and A_w, B_w stored as row/group
// INT8 (text after eq 7).  The forward is factored exactly as eq 7 factors
// it -- the narrow products X B^T are formed first (a1, proj_kernel), then
// every vocabulary row streams its residual nibbles once and adds its two
// low-rank terms (a2, vtile.hip), then a per-token top-1 reduction runs
// across the vocabulary tiles (a3).
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
    float *tf32, *sf32; // fp32 t and s (large-M projection)
    float *xsneg;
    int ncolblk;
    float *ppart;   // matrix-core projection for 5 <= M <= 32: slice partial sums
    uint32_t *pcnt; // and per-tile slice counts (zero between calls)
};

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

constexpr int kPSmallM = 4; // largest M of the one-workgroup-per-column projection
__global__ void proj_small_kernel(ProjArgs a);
template <int MT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1))) void proj_skinny_mfma_kernel(ProjArgs a);

static ProjArgs proj_args(const DevHead &h, const Work &w, const uint16_t *X)
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
    a.tf32 = w.tf32;
    a.sf32 = w.sf32;
    a.xsneg = w.xsneg;
    a.ppart = w.ppart;
    a.pcnt = w.pcnt;
    return a;
}

hipError_t launch_proj(const DevHead &h, const Work &w, const uint16_t *X, hipStream_t st)
{
    ProjArgs a = proj_args(h, w, X);
    const int64_t ncol = h.s.k + h.s.r;
    // the X-sum workgroup walks d in windows of 4096 columns, so each
    // g-group must fall inside one window
    if (w.M <= kPSmallM && (h.s.d <= 4096 || 4096 % h.s.g == 0)) {
        hipLaunchKernelGGL(proj_small_kernel, dim3((unsigned)(ncol + 1)), dim3(256), 0, st, a);
        return hipGetLastError();
    }
    if (w.M <= 32 && h.s.d <= 16384) { // matrix cores: a wave per (16 columns, K-slice), then a wave per X row
        const unsigned grid = (unsigned)((ncol + 15) / 16 * kProjKS + w.M);
        if (w.M <= 16)
            hipLaunchKernelGGL(proj_skinny_mfma_kernel<1>, dim3(grid), dim3(64), 0, st, a);
        else
            hipLaunchKernelGGL(proj_skinny_mfma_kernel<2>, dim3(grid), dim3(64), 0, st, a);
        return hipGetLastError();
    }
    a.ncolblk = (int)((ncol + 4 * kProjNI - 1) / (4 * kProjNI));
    dim3 grid(a.ncolblk + 1, (unsigned)((w.M + kProjMB - 1) / kProjMB));
    hipLaunchKernelGGL(proj_kernel, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// a1 for M <= 4 (decode): one workgroup per output column, whose 256 threads
// cover d in slices of 16 (a single round of loads spread over the chip at
// d <= 4096), plus one workgroup for the per-group X sums.  Each slice lies
// inside one g-group, so a D8 row's slice is scaled by its group scale before
// the workgroup reduction.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void proj_small_kernel(ProjArgs a)
{
    __shared__ float red[4][kPSmallM];
    __shared__ float part[256][kPSmallM];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t ncol = a.k + a.r;
    const int64_t col = blockIdx.x;
    const int64_t M = a.M;

    if (col == ncol) { // xsneg[grp][m] = -136 sum_{j in grp} X[m, j]
        const int64_t per = a.g / 16; // slices per group
        for (int64_t j00 = 0; j00 < a.d; j00 += 256 * 16) {
            const int64_t j0 = j00 + 16 * threadIdx.x;
            for (int m = 0; m < kPSmallM; ++m) {
                float sum = 0.f;
                if (j0 < a.d && m < M) {
                    const u32x4 x0 = *(const u32x4 *)(a.X + m * a.d + j0);
                    const u32x4 x1 = *(const u32x4 *)(a.X + m * a.d + j0 + 8);
                    const uint32_t xw[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
                    for (int e = 0; e < 8; ++e)
                        sum += bf_lo(xw[e]) + bf_hi(xw[e]);
                }
                part[threadIdx.x][m] = sum;
            }
            __syncthreads();
            // groups starting in this 4096-column window
            const int64_t ngrp = (a.d - j00 < 256 * 16 ? a.d - j00 : 256 * 16) / a.g;
            if (threadIdx.x < ngrp) {
                for (int m = 0; m < M; ++m) {
                    float sum = 0.f;
                    for (int64_t q = 0; q < per; ++q)
                        sum += part[threadIdx.x * per + q][m];
                    a.xsneg[(j00 / a.g + threadIdx.x) * a.Mp + m] = -kR4Bias * sum;
                }
            }
            __syncthreads();
        }
        return;
    }

    const bool isd = col >= a.k;
    const int8_t *wrow = isd ? a.d8 + (col - a.k) * a.d : a.b8 + col * a.d;
    float acc[kPSmallM] = {0.f, 0.f, 0.f, 0.f};
    for (int64_t j0 = 16 * threadIdx.x; j0 < a.d; j0 += 256 * 16) {
        const u32x4 w = *(const u32x4 *)(wrow + j0);
        const float sc = isd ? a.sd[(col - a.k) * a.G + j0 / a.g] : 1.f;
        for (int m = 0; m < kPSmallM; ++m) {
            if (m >= M)
                break;
            const u32x4 x0 = *(const u32x4 *)(a.X + m * a.d + j0);
            const u32x4 x1 = *(const u32x4 *)(a.X + m * a.d + j0 + 8);
            acc[m] = __builtin_fmaf(sc, dot16(w, x0, x1), acc[m]);
        }
    }
    for (int m = 0; m < kPSmallM; ++m) {
        float v = acc[m];
        for (int off = 32; off >= 1; off >>= 1)
            v += __shfl_xor(v, off);
        if (lane == 0)
            red[wv][m] = v;
    }
    __syncthreads();
    if (threadIdx.x < M) {
        const int m = threadIdx.x;
        const float v = red[0][m] + red[1][m] + red[2][m] + red[3][m];
        const float t = isd ? v : v * a.sb[col];
        const uint16_t hi = f32_to_bf16_rne(t);
        const uint16_t lo = f32_to_bf16_rne(t - __uint_as_float((uint32_t)hi << 16));
        if (isd) {
            a.s16[m * a.rpad + (col - a.k)] = hi;
            a.s16[(a.Mp + m) * a.rpad + (col - a.k)] = lo;
        } else {
            a.t16[m * a.kpad + col] = hi;
            a.t16[(a.Mp + m) * a.kpad + col] = lo;
        }
    }
}

// ---------------------------------------------------------------------------
// a1 for large M: the same products on the matrix cores, written as fp32 t
// and s for the large-M vocabulary-tile path.  A workgroup owns 16 output
// columns x 64 hidden states; its 4 waves split d into quarters and their
// partial sums meet in LDS.  Integer weights enter the MFMA as exact
// bf16 integers; each g-group of a D8 row is accumulated on its own and
// folded in with its scale (a group split between two waves is folded by
// both, which is the same sum).  No per-group X sums: the large-M
// vocabulary-tile kernel does not use them.
// ---------------------------------------------------------------------------
constexpr int kPMB = 4; // 16-row m-blocks per workgroup
constexpr int kPNB = 4; // K-steps per load batch

// 8 signed int8 values -> 8 exact bf16 integers
__device__ __forceinline__ u32x4 i8_bf16(u32x2 w)
{
    float f[8];
    for (int e = 0; e < 4; ++e) {
        f[e] = (float)(int8_t)(w.x >> (8 * e));
        f[4 + e] = (float)(int8_t)(w.y >> (8 * e));
    }
    return u32x4{pack_hi_halves(f[0], f[1]), pack_hi_halves(f[2], f[3]), pack_hi_halves(f[4], f[5]),
                 pack_hi_halves(f[6], f[7])};
}

__global__ __launch_bounds__(256) void proj_mfma_kernel(ProjArgs a)
{
    __shared__ f32x4 red[4][kPMB][64];
    const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t ncol = a.k + a.r;
    const int64_t c0 = (int64_t)blockIdx.x * 16;
    const int64_t c = c0 + lr < ncol ? c0 + lr : ncol - 1;
    const bool isd = c >= a.k;
    const int8_t *wrow = (isd ? a.d8 + (c - a.k) * a.d : a.b8 + c * a.d) + 8 * lq;
    const float *sdrow = a.sd + (isd ? (c - a.k) * a.G : 0);
    const int64_t mbase = (int64_t)blockIdx.y * (kPMB * 16);
    const uint16_t *xr[kPMB];
#pragma unroll
    for (int mb = 0; mb < kPMB; ++mb) {
        const int64_t m = mbase + 16 * mb + lr;
        xr[mb] = a.X + (m < a.M ? m : a.M - 1) * a.d + 8 * lq;
    }
    const int64_t nks = a.d / kKStep, gsteps = a.g / kKStep;
    const int64_t ks0 = wv * (nks / 4), ks1 = ks0 + nks / 4; // d is a multiple of 128

    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 acc[kPMB], gacc[kPMB];
#pragma unroll
    for (int mb = 0; mb < kPMB; ++mb)
        acc[mb] = gacc[mb] = zero;

    struct Batch {
        u32x4 x[kPNB][kPMB];
        u32x2 w[kPNB];
    };
    auto load = [&](Batch &b, int64_t ks) {
#pragma unroll
        for (int q = 0; q < kPNB; ++q) {
            const int64_t k = ks + q < ks1 ? ks + q : ks1 - 1;
#pragma unroll
            for (int mb = 0; mb < kPMB; ++mb)
                b.x[q][mb] = *(const u32x4 *)(xr[mb] + k * kKStep);
            b.w[q] = *(const u32x2 *)(wrow + k * kKStep);
        }
    };
    auto run = [&](const Batch &b, int64_t ks) {
#pragma unroll
        for (int q = 0; q < kPNB; ++q) {
            const int64_t k = ks + q;
            if (k >= ks1)
                break;
            const u32x4 bw = i8_bf16(b.w[q]);
#pragma unroll
            for (int mb = 0; mb < kPMB; ++mb)
                gacc[mb] = mfma_bf16(b.x[q][mb], bw, gacc[mb]);
            if ((k + 1) % gsteps == 0 || k + 1 == ks1) {
                const float sc = isd ? sdrow[k / gsteps] : 1.f;
#pragma unroll
                for (int mb = 0; mb < kPMB; ++mb) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[mb][i] = __builtin_fmaf(sc, gacc[mb][i], acc[mb][i]);
                    gacc[mb] = zero;
                }
            }
        }
    };
    Batch bA, bB;
    load(bA, ks0);
    for (int64_t ks = ks0; ks < ks1; ks += 2 * kPNB) {
        load(bB, ks + kPNB);
        run(bA, ks);
        load(bA, ks + 2 * kPNB);
        run(bB, ks + kPNB);
    }

#pragma unroll
    for (int mb = 0; mb < kPMB; ++mb)
        red[wv][mb][lane] = acc[mb];
    __syncthreads();
    if (wv != 0)
        return;
    const float sb = isd ? 1.f : a.sb[c];
#pragma unroll
    for (int mb = 0; mb < kPMB; ++mb) {
        const f32x4 v = red[0][mb][lane] + red[1][mb][lane] + red[2][mb][lane] + red[3][mb][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t m = mbase + 16 * mb + 4 * lq + i;
            if (m >= a.M || c0 + lr >= ncol)
                continue;
            if (isd)
                a.sf32[m * a.rpad + (c - a.k)] = v[i];
            else
                a.tf32[m * a.kpad + c] = v[i] * sb;
        }
    }
}

hipError_t launch_proj_mfma(const DevHead &h, const Work &w, const uint16_t *X, hipStream_t st)
{
    ProjArgs a = proj_args(h, w, X);
    const int64_t ncol = h.s.k + h.s.r;
    if (ncol == 0)
        return hipSuccess;
    dim3 grid((unsigned)((ncol + 15) / 16), (unsigned)((w.M + kPMB * 16 - 1) / (kPMB * 16)));
    hipLaunchKernelGGL(proj_mfma_kernel, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// a1 for 5 <= M <= 32 (batched decode): the products on the matrix cores,
// written as the bf16 hi/lo pairs of the small-M paths.  One wave per (16
// output columns, K-slice): kProjKS slices of d, so that the grid's loads
// (whose MFMA fragments touch 16 rows per instruction) spread over about
// kProjKS times as many compute units as tiles.  Each wave issues its loads
// up to sixteen K-steps at a time, stores its partial sums with device-scope
// stores and counts its tile; the last wave of a tile adds the slices in a
// fixed order and writes t, s.  Integer weights enter as exact bf16
// integers; each g-group of a D8 row is accumulated on its own and folded in
// with its scale (a group split between two slices is folded by both, the
// same sum).  Waves past the tiles write the per-group X sums, one row each,
// from coalesced loads.
// ---------------------------------------------------------------------------
constexpr int kPSKB = 16;       // K-steps per load batch
constexpr int kPSMaxD = 16384;  // widest d of the X-sum waves (their LDS row)

template <int MT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1))) void proj_skinny_mfma_kernel(ProjArgs a)
{
    const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
    const int64_t ncol = a.k + a.r;
    const int64_t ntile = (ncol + 15) / 16;
    const int64_t bid = blockIdx.x;

    if (bid >= ntile * kProjKS) { // per-group sums of X for row m
        __shared__ float s_c[kPSMaxD / 8];
        const int64_t m = bid - ntile * kProjKS;
        if (m >= a.M)
            return;
        const uint16_t *xr = a.X + m * a.d;
        const int64_t nch = a.d / 8; // 16-byte chunks of the row
        for (int64_t p0 = 0; p0 < nch; p0 += 64 * 8) {
            u32x4 v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int64_t p = p0 + 64 * q + lane;
                v[q] = p < nch ? *(const u32x4 *)(xr + 8 * p) : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int64_t p = p0 + 64 * q + lane;
                if (p < nch)
                    s_c[p] = bf_lo(v[q].x) + bf_hi(v[q].x) + bf_lo(v[q].y) + bf_hi(v[q].y) + bf_lo(v[q].z) +
                             bf_hi(v[q].z) + bf_lo(v[q].w) + bf_hi(v[q].w);
            }
        }
        __syncthreads();
        const int64_t cpg = a.g / 8;
        for (int64_t grp = lane; grp < a.G; grp += 64) {
            float sx = 0.f;
            for (int64_t p = grp * cpg; p < (grp + 1) * cpg; ++p)
                sx += s_c[p];
            a.xsneg[grp * a.Mp + m] = -kR4Bias * sx;
        }
        return;
    }

    const int64_t tile = bid / kProjKS, ks = bid - (bid / kProjKS) * kProjKS;
    const int64_t c0 = tile * 16;
    const int64_t c = c0 + lr < ncol ? c0 + lr : ncol - 1;
    const bool isd = c >= a.k;
    const int8_t *wrow = (isd ? a.d8 + (c - a.k) * a.d : a.b8 + c * a.d) + 8 * lq;
    const float *sdrow = a.sd + (isd ? (c - a.k) * a.G : 0);
    const uint16_t *xr[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int64_t m = 16 * mt + lr;
        xr[mt] = a.X + (m < a.M ? m : a.M - 1) * a.d + 8 * lq;
    }
    const int64_t nks = a.d / kKStep, gsteps = a.g / kKStep;
    const int64_t ks0 = ks * nks / kProjKS, ks1 = (ks + 1) * nks / kProjKS;

    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 acc[MT], gacc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        acc[mt] = gacc[mt] = zero;
    for (int64_t kb = ks0; kb < ks1; kb += kPSKB) {
        // every load of the batch -- operands and group scales -- before
        // its first product
        u32x4 x[kPSKB][MT];
        u32x2 w[kPSKB];
        float gs[kPSKB];
#pragma unroll
        for (int q = 0; q < kPSKB; ++q) {
            const int64_t k = kb + q < ks1 ? kb + q : ks1 - 1;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                x[q][mt] = *(const u32x4 *)(xr[mt] + k * kKStep);
            w[q] = *(const u32x2 *)(wrow + k * kKStep);
            gs[q] = isd ? sdrow[k / gsteps] : 1.f;
        }
#pragma unroll
        for (int q = 0; q < kPSKB; ++q) {
            const int64_t k = kb + q;
            if (k >= ks1)
                break;
            const u32x4 bw = i8_bf16(w[q]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                gacc[mt] = mfma_bf16(x[q][mt], bw, gacc[mt]);
            if ((k + 1) % gsteps == 0 || k + 1 == ks1) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[mt][i] = __builtin_fmaf(gs[q], gacc[mt][i], acc[mt][i]);
                    gacc[mt] = zero;
                }
            }
        }
    }
    // this slice's partial sums (pairs of floats as 64-bit device-scope
    // stores), complete before the tile's count
    uint64_t *pp = (uint64_t *)(a.ppart + ((tile * kProjKS + ks) * 2) * 256 + lane * 4);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 2; ++e)
            __hip_atomic_store(pp + mt * 128 + e,
                               (uint64_t)__float_as_uint(acc[mt][2 * e]) |
                                   ((uint64_t)__float_as_uint(acc[mt][2 * e + 1]) << 32),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    uint32_t prev = 0;
    if (lane == 0)
        prev = __hip_atomic_fetch_add(a.pcnt + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)__builtin_amdgcn_readfirstlane(prev) != (uint32_t)(kProjKS - 1))
        return;
    // the last slice of the tile: every slice's partials, in slice order
    if (lane == 0)
        __hip_atomic_store(a.pcnt + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // (pairs of floats as 64-bit device-scope loads, all in flight at once)
    const uint64_t *tp = (const uint64_t *)(a.ppart + (tile * kProjKS * 2) * 256 + lane * 4);
    float v[MT][4];
    uint64_t part[kProjKS][MT][2];
#pragma unroll
    for (int q = 0; q < kProjKS; ++q)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 2; ++e)
                part[q][mt][e] = __hip_atomic_load(tp + (q * 2 + mt) * 128 + e, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int q = 0; q < kProjKS; ++q)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint64_t pr = part[q][mt][i >> 1];
                const float x = __uint_as_float((uint32_t)(i & 1 ? pr >> 32 : pr));
                v[mt][i] = q == 0 ? x : v[mt][i] + x;
            }
    if (c0 + lr >= ncol)
        return;
    const float sb = isd ? 1.f : a.sb[c];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t m = 16 * mt + 4 * lq + i;
            if (m >= a.M)
                continue;
            const float t = v[mt][i] * sb;
            const uint16_t hi = f32_to_bf16_rne(t);
            const uint16_t lo = f32_to_bf16_rne(t - __uint_as_float((uint32_t)hi << 16));
            if (isd) {
                a.s16[m * a.rpad + (c - a.k)] = hi;
                a.s16[(a.Mp + m) * a.rpad + (c - a.k)] = lo;
            } else {
                a.t16[m * a.kpad + c] = hi;
                a.t16[(a.Mp + m) * a.kpad + c] = lo;
            }
        }
}

// ---------------------------------------------------------------------------
// a3: top-1 reduction across vocabulary tiles.  Keys order by value, then by
// lower index, so the maximum key is the first index of the maximum logit.
// ---------------------------------------------------------------------------
struct FinishArgs {
    const uint64_t *part; // [M][n_part] argmax keys
    const uint64_t *lsep; // [M][n_part] log-sum-exp summaries
    int64_t n_part, M, V;
    int32_t *argmax;        // may be null
    float *lse, *nll;       // may be null (nll needs targets)
    const int32_t *targets; // [M]
    const float *tl;        // [M] target logits
};

// One workgroup per row m: the first index of the largest logit, and
// lse = mx + log s over the merged summaries; nll = lse - the target's
// logit, NaN for a target outside [0, V).
__global__ __launch_bounds__(256) void finish_kernel(FinishArgs a)
{
    __shared__ uint64_t red[4];
    __shared__ LsePart lred[4];
    const int64_t m = blockIdx.x;
    if (m >= a.M)
        return;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    if (a.argmax) { // uniform
        uint64_t key = 0;
        for (int64_t i = threadIdx.x; i < a.n_part; i += 256)
            key = umax64(key, a.part[m * a.n_part + i]);
        for (int off = 32; off >= 1; off >>= 1)
            key = umax64(key, shfl_xor_u64(key, off));
        if (lane == 0)
            red[wv] = key;
    }
    if (a.lse) { // uniform
        LsePart p{-__builtin_inff(), 0.f};
        for (int64_t i = threadIdx.x; i < a.n_part; i += 256)
            p = lse_merge(p, lse_unbits(a.lsep[m * a.n_part + i]));
        p = lse_merge64(p);
        if (lane == 0)
            lred[wv] = p;
    }
    __syncthreads();
    if (threadIdx.x != 0)
        return;
    if (a.argmax) {
        const uint64_t key = umax64(umax64(red[0], red[1]), umax64(red[2], red[3]));
        a.argmax[m] = (int32_t)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFu));
    }
    if (a.lse) {
        const LsePart p = lse_merge(lse_merge(lred[0], lred[1]), lse_merge(lred[2], lred[3]));
        const float L = p.mx + logf(p.s);
        a.lse[m] = L;
        if (a.nll) {
            const int32_t t = a.targets[m];
            a.nll[m] = (t >= 0 && (int64_t)t < a.V) ? L - a.tl[m] : __builtin_nanf("");
        }
    }
}

hipError_t launch_finish(const Work &w, int64_t n_part, int64_t V, int32_t *argmax, float *lse, float *nll,
                         hipStream_t st)
{
    FinishArgs a;
    a.part = w.part;
    a.lsep = w.lsep;
    a.n_part = n_part;
    a.M = w.M;
    a.V = V;
    a.argmax = argmax;
    a.lse = lse;
    a.nll = nll;
    a.targets = w.targets;
    a.tl = w.tl;
    hipLaunchKernelGGL(finish_kernel, dim3((unsigned)w.M), dim3(256), 0, st, a);
    return hipGetLastError();
}

} // namespace archead
