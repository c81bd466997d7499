// vtile_lds.hip -- the vocabulary-tile step of the packed ARCHead forward for
// large M (prefill): LDS-staged MFMA over [128 hidden states x 512 rows].
//
// ARCHead paper, section 3.2, eq 7, with W_d of eq 3 and the INT8 correction
// factors stored after eq 7:
//   logits[m,v] = sC[v] C8[v,:].s[m,:] + sA[v] A5[v,:].t[m,:]
//               + sum_grp sR[v,grp] R4[v,grp].X[m,grp]
// At large M the step is bound by the matrix cores, not by HBM.  A workgroup
// of 8 waves owns 128 hidden states x 32 v-blocks; each wave keeps a
// [128 x 64] fp32 accumulator tile.  Everything a stage needs -- the A
// operand (X, t or s for the 128 rows), the code chunks of the 32 v-blocks
// and their residual scales -- is copied straight from global memory into
// LDS (global_load_lds), double-buffered with one barrier per stage.
//
// Precision (one accumulator per output, three phases):
//   1. correction: exact integer C8 codes (bf16) against s = s_hi + s_lo;
//   2. rescale by sC/sA, then the core: exact integer A5 codes against
//      t = t_hi + t_lo; rows whose sA or sC is zero have those codes masked;
//   3. rescale by sA 2^e_v 2^f_m, then the residual in fp16 MFMA: the code q
//      times the row-normalised scale sR 2^e_v, rounded once to fp16
//      (relative error <= 2^-12), against X 2^f_m converted to fp16 (exact
//      for every element within 2^29 of the row maximum);
// then the powers of two are removed.  Every other step is exact or fp32.
//
// Tiles are assigned so that the workgroups one XCD runs share v-ranges: the
// 16 m-tiles of a v-range run on the same XCD at about the same time, so its
// codes come from HBM once and then from that XCD's L2.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "kernels.hpp"

namespace archead {

constexpr int kLW = 8;             // waves per workgroup (two per SIMD)
constexpr int kLVB = 4;            // v-blocks per wave
constexpr int kLMB = 8;            // 16-row m-blocks per tile
constexpr int kLVR = kLW * kLVB;   // v-blocks per workgroup (512 rows)
constexpr int kLS = 32 / kLW;      // operand blocks each wave fills per stage
constexpr int kLRows = kLMB * 16;  // hidden states per tile
// one stage buffer, in 1 KiB blocks (uint32 offsets below)
constexpr int kLOpBlk = 32;                    // A operand: 32 blocks in lane order
constexpr int kLCodeOff = kLOpBlk * 256;       // code chunks of the 32 v-blocks
constexpr int kLScOff = kLCodeOff + kLVR * 256; // residual scales [4 K-steps][32 v-blocks][16] fp16
constexpr int kLStageWords = kLScOff + 4 * 256;

// ---------------------------------------------------------------------------
// X -> fp16 with a per-row power-of-two scale (max |X[m,:]| 2^f in
// [2^14, 2^15)); bf16 values convert exactly unless 2^29 below the maximum.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prep_x16_kernel(const uint16_t *X, int64_t d, uint16_t *x16,
                                                       float *xsc)
{
    __shared__ float red[4];
    const int64_t m = blockIdx.x;
    const uint16_t *xr = X + m * d;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    float mx = 0.f;
    for (int64_t j = threadIdx.x * 8; j < d; j += 256 * 8) {
        const u32x4 v = *(const u32x4 *)(xr + j);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        for (int q = 0; q < 4; ++q) {
            mx = fmaxf(mx, fabsf(__uint_as_float(w[q] << 16)));
            mx = fmaxf(mx, fabsf(__uint_as_float(w[q] & 0xFFFF0000u)));
        }
    }
    for (int off = 32; off >= 1; off >>= 1)
        mx = fmaxf(mx, __shfl_xor(mx, off));
    if (lane == 0)
        red[wv] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    int f = 0;
    if (mx > 0.f && mx <= 3.4028235e38f) {
        f = 14 - ilogbf(mx);
        f = f < -126 ? -126 : (f > 126 ? 126 : f);
    }
    for (int64_t j = threadIdx.x * 8; j < d; j += 256 * 8) {
        const u32x4 v = *(const u32x4 *)(xr + j);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t o[4];
        for (int q = 0; q < 4; ++q) {
            const _Float16 lo = (_Float16)ldexpf(__uint_as_float(w[q] << 16), f);
            const _Float16 hi = (_Float16)ldexpf(__uint_as_float(w[q] & 0xFFFF0000u), f);
            o[q] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
        *(u32x4 *)(x16 + m * d + j) = u32x4{o[0], o[1], o[2], o[3]};
    }
    if (threadIdx.x == 0) {
        xsc[2 * m] = ldexpf(1.f, -f);
        xsc[2 * m + 1] = ldexpf(1.f, f);
    }
}

// bf16 pair of exact integers (a + 144) -> bf16 pair a
__device__ __forceinline__ uint32_t unbias144(uint32_t p)
{
    const float lo = __uint_as_float(p << 16) - kA5Bias;
    const float hi = __uint_as_float(p & 0xFFFF0000u) - kA5Bias;
    return pack_hi_halves(lo, hi);
}

// residual dword -> 8 fp16 values q * s (q = nibble - 8), s2 = (s, s)
__device__ __forceinline__ u32x4 r4_f16_scaled(uint32_t w, uint32_t magic, f16x2 s2)
{
    const f16x2 bias = {(_Float16)1032.0f, (_Float16)1032.0f};
    const uint32_t m = 0x000F000Fu;
    const uint32_t x[4] = {(w & m) | magic, ((w >> 4) & m) | magic, ((w >> 8) & m) | magic,
                           ((w >> 12) & m) | magic};
    uint32_t o[4];
    for (int p = 0; p < 4; ++p) {
        f16x2 h = __builtin_bit_cast(f16x2, x[p]) - bias; // exact: q
        h = h * s2;                                       // rounded once
        o[p] = __builtin_bit_cast(uint32_t, h);
    }
    return u32x4{o[0], o[1], o[2], o[3]};
}

__device__ __forceinline__ u32x4 and4(u32x4 v, uint32_t m) { return u32x4{v.x & m, v.y & m, v.z & m, v.w & m}; }

struct LdsArgs {
    DevHead h;
    Work w;
    float *logits; // may be null
    int want_argmax;
    int gsteps;
    int64_t nvb, nkc, G, na, nc, kst, rst, kpad, rpad;
    int64_t p1, p2, nst; // first core stage, first residual stage, stage count (phases padded to even)
    int64_t n_vr, n_mt, n_tiles, per_xcd;
};

__device__ __forceinline__ void lds_dma16(const void *src, uint32_t *dst)
{
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
}

// Stages, in order: correction stages (two K-steps of s_hi/s_lo each), core
// stages (one K-step of t_hi/t_lo), residual stages (four K-steps of X), each
// phase padded to an even count; a pad stage contributes zero.
template <int GS>
__global__ __launch_bounds__(kLW * 64, 1) void vtile_lds_kernel(LdsArgs a)
{
    // two stage buffers as separate objects, so that the compiler can tell
    // the asynchronous fill of one from the reads of the other
    __shared__ __attribute__((aligned(16))) uint32_t s_buf0[kLStageWords];
    __shared__ __attribute__((aligned(16))) uint32_t s_buf1[kLStageWords];
    __shared__ __attribute__((aligned(16))) float s_fm[2 * kLRows]; // 2^f_m, then 2^-f_m
    __shared__ uint64_t s_red[kLW * kLRows];

    const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
    // wave index as a uniform value, so that everything derived from it
    // lives in scalar registers
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t bid = blockIdx.x;
    const int64_t L = (bid & 7) * a.per_xcd + (bid >> 3);
    if (L >= a.n_tiles)
        return; // the whole workgroup
    const int64_t vr = L / a.n_mt, mt = L % a.n_mt;
    const int64_t M = a.w.M, Mp = a.w.Mp, d = a.h.s.d, V = a.h.s.V;
    const int64_t nvb = a.nvb, G = a.G, nc = a.nc, kst = a.kst, rst = a.rst, nkc = a.nkc;
    const int64_t kpad = a.kpad, rpad = a.rpad, nst = a.nst, p1 = a.p1, p2 = a.p2;
    const int64_t mbase = mt * kLRows;
    const int64_t rows_live = (M - mbase) < kLRows ? (M - mbase) : kLRows;
    const int64_t wg_vb0 = vr * kLVR;
    const int64_t vb0 = wg_vb0 + wv * kLVB;
    const int gsteps = GS ? GS : a.gsteps;

    // bit v: sA of the lane's row in v-block v is nonzero; bit kLVB + v: sC
    uint32_t nz = 0;
#pragma unroll
    for (int v = 0; v < kLVB; ++v) {
        const int64_t vb = vb0 + v < nvb ? vb0 + v : nvb - 1;
        nz |= h2f(a.h.sa[vb * kVB + lr]) != 0.f ? 1u << v : 0u;
        nz |= h2f(a.h.sc[vb * kVB + lr]) != 0.f ? 1u << (kLVB + v) : 0u;
    }
    if (threadIdx.x < kLRows) {
        const int64_t m0 = mbase + threadIdx.x, m = m0 < M ? m0 : M - 1;
        s_fm[threadIdx.x] = a.w.xsc[2 * m + 1];       // 2^f_m
        s_fm[kLRows + threadIdx.x] = a.w.xsc[2 * m];  // 2^-f_m
    }

    // ---- stage fill --------------------------------------------------------
    // Operand block slot = kLS wv + i (i < kLS), m-block slot % 8:
    //   residual: K-step slot / 8 of the chunk (X rows)
    //   core:     half (slot / 8) % 2 of t (slots 16..31 repeat 0..15)
    //   correction: K-step slot / 16 of the pair, half (slot / 8) % 2 of s
    // Code block j = kLVB wv + i holds the chunk of v-block j of the workgroup.
    // Scale block st (residual stages): lane l covers v-block l / 2, rows
    // 8 (l % 2) .. +7, for the group of K-step st (one block when a group
    // spans the whole chunk).
    const uint16_t *x16t = a.w.x16 + mbase * d;
    const int64_t hsel = ((wv * kLS) >> 3) & 1; // (slot / 8) % 2 for this wave's slots
    const uint16_t *t16t = a.w.t16 + (hsel * Mp + mbase) * kpad;
    const uint16_t *s16t = a.w.s16 + (hsel * Mp + mbase) * rpad;
    const u32x4 *lrp = (const u32x4 *)a.h.lr;
    const u32x4 *r4p = (const u32x4 *)a.h.r4;
    const int mb0 = (wv * kLS) & 7; // m-block of slot i is mb0 + i
    uint32_t rowl[kLS];
#pragma unroll
    for (int i = 0; i < kLS; ++i) {
        const int64_t r = 16 * (mb0 + i) + lr;
        rowl[i] = (uint32_t)(r < rows_live ? r : rows_live - 1);
    }
    // scale rows this lane copies: v-block (lane / 2) of the workgroup
    const int64_t svb = wg_vb0 + (lane >> 1) < nvb ? wg_vb0 + (lane >> 1) : nvb - 1;
    const uint32_t soff = (uint32_t)(svb * G * kVB + 8 * (lane & 1)); // + grp * 16

    auto stage_fill = [&](int64_t s, uint32_t *buf) {
        const uint16_t *base;
        uint32_t stride;
        const u32x4 *cbase;
        int64_t kc = 0;
        if (s < p1) {
            const int64_t ks0 = 2 * s + ((wv * kLS) >> 4), ks = ks0 < rst ? ks0 : rst - 1;
            base = s16t + ks * kKStep;
            stride = (uint32_t)rpad;
            cbase = lrp + (a.na + (s < nc ? s : nc - 1)) * nvb * 64;
        } else if (s < p2) {
            const int64_t ks = s - p1 < kst ? s - p1 : kst - 1;
            base = t16t + ks * kKStep;
            stride = (uint32_t)kpad;
            cbase = lrp + (ks / 3) * nvb * 64;
        } else {
            kc = s - p2 < nkc ? s - p2 : nkc - 1;
            base = x16t + (kc * 4 + ((wv * kLS) >> 3)) * kKStep;
            stride = (uint32_t)d;
            cbase = r4p + kc * nvb * 64;
        }
#pragma unroll
        for (int i = 0; i < kLS; ++i)
            lds_dma16(base + (rowl[i] * stride + 8 * lq), buf + (wv * kLS + i) * 256);
#pragma unroll
        for (int i = 0; i < kLVB; ++i) {
            const int64_t vb = vb0 + i < nvb ? vb0 + i : nvb - 1;
            lds_dma16(cbase + vb * 64 + lane, buf + kLCodeOff + (wv * kLVB + i) * 256);
        }
        if (s >= p2 && (GS == 4 ? wv == 0 : wv < 4)) { // kLW >= 4
            const int64_t grp = GS == 4 ? kc : (kc * 4 + wv) / gsteps;
            lds_dma16(a.h.srp + (soff + grp * kVB), buf + kLScOff + (GS == 4 ? 0 : wv) * 256);
        }
    };

    // ---- compute -----------------------------------------------------------
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 T[kLMB][kLVB];
#pragma unroll
    for (int mb = 0; mb < kLMB; ++mb)
#pragma unroll
        for (int v = 0; v < kLVB; ++v)
            T[mb][v] = zero;
    const uint32_t magic16 = vgpr_const(kF16Magic);
    auto afrag = [&](const uint32_t *buf, int blk) { return *(const u32x4 *)(buf + blk * 256 + lane * 4); };
    auto codes = [&](const uint32_t *buf, u32x4(&c)[kLVB]) {
#pragma unroll
        for (int v = 0; v < kLVB; ++v)
            c[v] = *(const u32x4 *)(buf + kLCodeOff + (wv * kLVB + v) * 256 + lane * 4);
    };

    // No branch surrounds an MFMA (the accumulator tile would be copied at
    // every join): pad stages run with their codes masked to zero.
    auto compute_c8 = [&](int64_t s, const uint32_t *buf) {
        u32x4 c[kLVB];
        codes(buf, c);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const uint32_t live = (s < nc && 2 * s + hh < rst) ? 0xFFFFFFFFu : 0u;
            u32x4 bq[kLVB];
#pragma unroll
            for (int v = 0; v < kLVB; ++v) {
                u32x2 w2;
                w2.x = hh == 0 ? c[v].x : c[v].z;
                w2.y = hh == 0 ? c[v].y : c[v].w;
                bq[v] = and4(c8_bf16(w2), ((nz >> (kLVB + v)) & 1u ? 0xFFFFFFFFu : 0u) & live);
            }
#pragma unroll
            for (int mb = 0; mb < kLMB; ++mb) {
                const u32x4 ah = afrag(buf, (2 * hh) * 8 + mb);
                const u32x4 al = afrag(buf, (2 * hh + 1) * 8 + mb);
#pragma unroll
                for (int v = 0; v < kLVB; ++v) {
                    T[mb][v] = mfma_bf16(ah, bq[v], T[mb][v]);
                    T[mb][v] = mfma_bf16(al, bq[v], T[mb][v]);
                }
            }
        }
    };
    auto compute_a5 = [&](int64_t s, const uint32_t *buf) {
        u32x4 c[kLVB];
        codes(buf, c);
        const int64_t ks = s - p1;
        const uint32_t live = ks < kst ? 0xFFFFFFFFu : 0u;
        const int q = (int)(ks % 3);
        u32x4 bq[kLVB];
#pragma unroll
        for (int v = 0; v < kLVB; ++v) {
            const uint32_t wn = q == 0 ? c[v].x : q == 1 ? c[v].y : c[v].z;
            const u32x4 b = a5_bf16_q(wn, c[v].w, q);
            const uint32_t mk = ((nz >> v) & 1u ? 0xFFFFFFFFu : 0u) & live;
            bq[v] = u32x4{unbias144(b.x) & mk, unbias144(b.y) & mk, unbias144(b.z) & mk, unbias144(b.w) & mk};
        }
#pragma unroll
        for (int mb = 0; mb < kLMB; ++mb) {
            const u32x4 ah = afrag(buf, mb);
            const u32x4 al = afrag(buf, 8 + mb);
#pragma unroll
            for (int v = 0; v < kLVB; ++v) {
                T[mb][v] = mfma_bf16(ah, bq[v], T[mb][v]);
                T[mb][v] = mfma_bf16(al, bq[v], T[mb][v]);
            }
        }
    };
    auto compute_r4 = [&](int64_t s, const uint32_t *buf) {
        u32x4 c[kLVB];
        codes(buf, c);
        const uint32_t live = s - p2 < nkc ? 0xFFFFFFFFu : 0u;
        const uint16_t *scb = (const uint16_t *)(buf + kLScOff);
        uint32_t sc[kLVB][GS == 4 ? 1 : 4];
#pragma unroll
        for (int v = 0; v < kLVB; ++v)
#pragma unroll
            for (int st = 0; st < (GS == 4 ? 1 : 4); ++st)
                sc[v][st] = ((uint32_t)scb[(st * kLVR + wv * kLVB + v) * kVB + lr] * 0x10001u) & live;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            u32x4 bq[kLVB];
#pragma unroll
            for (int v = 0; v < kLVB; ++v) {
                const uint32_t wd = st == 0 ? c[v].x : st == 1 ? c[v].y : st == 2 ? c[v].z : c[v].w;
                bq[v] = r4_f16_scaled(wd, magic16, __builtin_bit_cast(f16x2, sc[v][GS == 4 ? 0 : st]));
            }
#pragma unroll
            for (int mb = 0; mb < kLMB; ++mb) {
                const u32x4 ax = afrag(buf, st * 8 + mb);
#pragma unroll
                for (int v = 0; v < kLVB; ++v)
                    T[mb][v] = mfma_f16(ax, bq[v], T[mb][v]);
            }
        }
    };

    stage_fill(0, s_buf0);
    __syncthreads(); // every wave's fill of stage 0 and the s_fm stores

    // Stage s (even) computes from s_buf0 while stage s+1 fills s_buf1; the
    // barrier after it also waits for that fill.  No fill is left in flight
    // past the last stage.
#define ARCHEAD_LDS_PHASE(S0, S1, COMPUTE)                                          \
    for (int64_t s = (S0); s < (S1); s += 2) {                                     \
        stage_fill(s + 1, s_buf1);                                                 \
        COMPUTE(s, s_buf0);                                                        \
        __syncthreads();                                                           \
        if (s + 2 < nst)                                                           \
            stage_fill(s + 2, s_buf0);                                             \
        COMPUTE(s + 1, s_buf1);                                                    \
        __syncthreads();                                                           \
    }

    // phase 1: correction (T = C8 . s)
    ARCHEAD_LDS_PHASE(0, p1, compute_c8)
    // T in units of sA (or of 1 where sA = 0)
#pragma unroll
    for (int v = 0; v < kLVB; ++v) {
        const int64_t vb = vb0 + v < nvb ? vb0 + v : nvb - 1;
        const float sa = h2f(a.h.sa[vb * kVB + lr]), sc = h2f(a.h.sc[vb * kVB + lr]);
        const float ratio = sc / (sa != 0.f ? sa : 1.f);
#pragma unroll
        for (int mb = 0; mb < kLMB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                T[mb][v][i] *= ratio;
    }
    // phase 2: core (T += A5 . t)
    ARCHEAD_LDS_PHASE(p1, p2, compute_a5)
    // T in units of 2^-(e_v + f_m)
    {
        f32x4 fm[kLMB];
#pragma unroll
        for (int mb = 0; mb < kLMB; ++mb)
            fm[mb] = *(const f32x4 *)(s_fm + mb * 16 + 4 * lq);
#pragma unroll
        for (int v = 0; v < kLVB; ++v) {
            const int64_t vb = vb0 + v < nvb ? vb0 + v : nvb - 1;
            const float sa = h2f(a.h.sa[vb * kVB + lr]);
            const float conv = (sa != 0.f ? sa : 1.f) / a.h.rsc[vb * kVB + lr];
#pragma unroll
            for (int mb = 0; mb < kLMB; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    T[mb][v][i] *= conv * fm[mb][i];
        }
    }
    // phase 3: residual (T += X' . (sR' o R4))
    ARCHEAD_LDS_PHASE(p2, nst, compute_r4)
#undef ARCHEAD_LDS_PHASE

    // back to logits units; write logits and the workgroup's top-1 keys
#pragma unroll
    for (int mb = 0; mb < kLMB; ++mb) {
        const f32x4 fi = *(const f32x4 *)(s_fm + kLRows + mb * 16 + 4 * lq);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t m = mbase + mb * 16 + 4 * lq + i;
            uint64_t k = 0;
#pragma unroll
            for (int v = 0; v < kLVB; ++v) {
                const int64_t vb = vb0 + v < nvb ? vb0 + v : nvb - 1;
                const int64_t row = (vb0 + v) * kVB + lr;
                const float y = T[mb][v][i] * a.h.rsc[vb * kVB + lr] * fi[i];
                if (m < M && vb0 + v < nvb && row < V) {
                    if (a.logits)
                        a.logits[m * V + row] = y;
                    k = umax64(k, argmax_key(y, (uint32_t)row));
                }
            }
            if (a.want_argmax) { // uniform across the grid
                k = umax64(k, shfl_xor_u64(k, 1));
                k = umax64(k, shfl_xor_u64(k, 2));
                k = umax64(k, shfl_xor_u64(k, 4));
                k = umax64(k, shfl_xor_u64(k, 8));
                if (lr == 0)
                    s_red[wv * kLRows + mb * 16 + 4 * lq + i] = k;
            }
        }
    }
    if (!a.want_argmax)
        return;
    __syncthreads();
    if (threadIdx.x < kLRows) {
        uint64_t k = 0;
#pragma unroll
        for (int w = 0; w < kLW; ++w)
            k = umax64(k, s_red[w * kLRows + threadIdx.x]);
        const int64_t m = mbase + threadIdx.x;
        if (m < M)
            a.w.part[m * a.w.n_part + vr] = k;
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
int64_t lds_n_part(const DevHead &h, int64_t M)
{
    (void)M;
    return lds_max_n_part(h.s);
}

int64_t lds_max_n_part(const Shape &s) { return (s.nvb() + kLVR - 1) / kLVR; }

hipError_t launch_prep_x16(const DevHead &h, const Work &w, const uint16_t *X, hipStream_t st)
{
    hipLaunchKernelGGL(prep_x16_kernel, dim3((unsigned)w.M), dim3(256), 0, st, X, h.s.d, w.x16, w.xsc);
    return hipGetLastError();
}

hipError_t launch_vtile_lds(const DevHead &h, const Work &w, float *logits, int32_t *argmax,
                            hipStream_t st)
{
    LdsArgs a;
    a.h = h;
    a.w = w;
    a.w.n_part = lds_n_part(h, w.M);
    if (w.M * a.w.n_part > w.part_cap)
        return hipErrorInvalidValue; // argmax partials would not fit the workspace
    a.logits = logits;
    a.want_argmax = argmax ? 1 : 0;
    a.gsteps = (int)(h.s.g / kKStep);
    a.nvb = h.s.nvb();
    a.nkc = h.s.nkc();
    a.G = h.s.G();
    a.na = h.s.lr_na();
    a.nc = h.s.lr_nc();
    a.kst = h.s.kst();
    a.rst = h.s.rst();
    a.kpad = h.s.kpad();
    a.rpad = h.s.rpad();
    a.p1 = (a.nc + 1) / 2 * 2;
    a.p2 = a.p1 + (a.kst + 1) / 2 * 2;
    a.nst = a.p2 + (a.nkc + 1) / 2 * 2;
    a.n_vr = a.w.n_part;
    a.n_mt = (w.M + kLRows - 1) / kLRows;
    a.n_tiles = a.n_vr * a.n_mt;
    const int64_t grid = (a.n_tiles + 7) / 8 * 8;
    a.per_xcd = grid / 8;
    if (a.gsteps == 4)
        hipLaunchKernelGGL(vtile_lds_kernel<4>, dim3((unsigned)grid), dim3(kLW * 64), 0, st, a);
    else
        hipLaunchKernelGGL(vtile_lds_kernel<0>, dim3((unsigned)grid), dim3(kLW * 64), 0, st, a);
    return hipGetLastError();
}

} // namespace archead
