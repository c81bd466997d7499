// vtile_lds.hip -- the vocabulary-tile step of the packed ARCHead forward for
// large M (prefill): LDS-staged fp16 MFMA over [128 hidden states x 512 rows].
//
// ARCHead paper, section 3.2, eq 7, with W_d of eq 3 and the INT8 correction
// factors stored after eq 7:
//   logits[m,v] = sC[v] C8[v,:].s[m,:] + sA[v] A5[v,:].t[m,:]
//               + sum_grp sR[v,grp] R4[v,grp].X[m,grp]
// At large M the step is bound by the matrix cores, not by HBM.  A workgroup
// of 8 waves owns 128 hidden states x 32 v-blocks; each wave keeps a
// [128 x 64] fp32 accumulator tile.  Everything a stage needs -- the A
// operand blocks for the 128 rows, the code words of the 32 v-blocks and
// their residual scales -- is copied straight from global memory into LDS
// (global_load_lds), double-buffered with one barrier per stage.
//
// One accumulator and one MFMA type (v_mfma_f32_16x16x32_f16) for all three
// terms, in three phases.  With e_r the exponent that puts the row's largest
// residual scale into [2^14, 2^15) (layout.hpp) and f_m a per-hidden-state
// power of two (prep_lds_kernel):
//   1. residual: B = q x (sR 2^(e_r - 10)), rounded once to fp16 (relative error at
//      most 2^-12 of this, the smallest, term; q and the power-of-two rescale
//      are exact), A = X 2^f_m in fp16 (exact for every element within 2^29
//      of the row's largest operand);
//   2. rescale the accumulator (fp32) to units of sA[v] 2^-f_m; core:
//      B = the exact integer codes A5, A = the fp16 hi + lo parts of
//      t 2^f_m (22 significant bits);
//   3. rescale to units of sC[v] 2^-f_m; correction: B = the exact integer
//      codes C8, A = hi + lo of s 2^f_m;
// and the epilogue multiplies by sC[v] 2^-f_m.  Rows whose sA (sC) is zero
// have their A5 (C8) codes masked and keep a unit divisor.  The correction
// phase goes last because its stage count (one stage per two K-steps of s)
// is often odd: the last phase needs no pad stage.
//
// Tiles are assigned to the XCDs (workgroup b runs on XCD b mod 8) so that
// operands are shared in an XCD's L2.  When the m-tile count is a multiple
// of 8, XCD x owns m-tiles x, x + 8, ... and all XCDs sweep the v-ranges in
// step: the A operands of an XCD's m-tiles (2.4 MB at M = 2048) stay in its
// L2, and each v-range's codes come from HBM about once and are then shared
// through the memory-side cache.  Otherwise an XCD runs all m-tiles of a
// v-range at about the same time, so that its codes come from HBM once and
// then from that XCD's L2.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "kernels.hpp"

namespace archead {

constexpr int kLW = 8;             // waves per workgroup (two per SIMD)
constexpr int kLVB = 4;            // v-blocks per wave
constexpr int kLMB = 8;            // 16-row m-blocks per tile
constexpr int kLVR = kLW * kLVB;   // v-blocks per workgroup (512 rows)
constexpr int kLS = 32 / kLW;      // operand blocks each wave copies per stage
constexpr int kLRows = kLMB * 16;  // hidden states per tile
// one stage buffer (uint32 offsets)
constexpr int kLCodeOff = 32 * 256;                  // 32 operand blocks of 1 KiB
constexpr int kLScOff = kLCodeOff + kLVR * 256;      // code words, 1 KiB per v-block
constexpr int kLStageWords = kLScOff + 4 * kLVR * 8; // residual scales [4 K-steps][32][16] fp16

// ---------------------------------------------------------------------------
// Operand preparation: per hidden state m, f_m puts the largest of |X[m,:]|,
// |t[m,:]|, |s[m,:]| into [2^14, 2^15); X 2^f_m (fp16) and the fp16 hi/lo
// parts of t 2^f_m and s 2^f_m are written in MFMA A-operand blocks of
// [16 rows x 32 columns] (lane l: row l % 16, columns 8 (l / 16) .. +7), so
// that each block is one contiguous 1 KiB copy.  Rows M .. (tile end) are
// zeros.
// ---------------------------------------------------------------------------
// Stages of the tile kernel, in order: nsr residual stages (one K-chunk
// each), nsa core stages, nsc correction stages.  The residual and core
// counts are padded to even (a stage pair shares the two LDS buffers); the
// correction phase comes last and is not padded.
struct LdsStages {
    int nst, p1, p2; // stage count; the core and correction phases start at p1, p2
    int nkc, nc, na, kst, rst, gsteps, nks;
};

static LdsStages lds_stage_info(const Shape &s)
{
    LdsStages t;
    t.nkc = (int)s.nkc();
    t.nc = (int)s.lr_nc();
    t.na = (int)s.lr_na();
    t.kst = (int)s.kst();
    t.rst = (int)s.rst();
    t.gsteps = (int)(s.g / kKStep);
    t.nks = (int)(s.d / kKStep);
    const int nsr = (t.nkc + 1) / 2 * 2, nsa = ((t.kst + 1) / 2 + 1) / 2 * 2, nsc = t.nc;
    t.p1 = nsr;
    t.p2 = nsr + nsa;
    t.nst = nsr + nsa + nsc;
    return t;
}

// Row s of the stage-fill table: what stage s copies, as small integers.
//   [0] A operand array (0: X, 1: s, 2: t)   [1] its KiB per 16-row m-block
//   [2 + fq] KiB offset of the A blocks of slot fq at m-block 0
//   [6] code stream (0: residual, 1: low-rank)   [7], [8] chunks of words 0-1, 2-3
//   [9] words taken from those chunks, a byte each   [10 + w] residual scale group of wave w
// The tile adds its own m-block and v-block offsets.
__device__ void lds_fill_entry(int s, const LdsStages &t, int32_t *e)
{
    const bool isr = s < t.p1, isc = s >= t.p2; // else core
    const int kc = s < t.nkc ? s : t.nkc - 1;
    // stage index within the correction (j1) and core (j2) phases
    const int j1 = s - t.p2 > 0 ? s - t.p2 : 0, j2 = s - t.p1 > 0 ? s - t.p1 : 0;
    const int rl = t.rst > 0 ? t.rst - 1 : 0, kl = t.kst > 0 ? t.kst - 1 : 0;
    e[0] = isr ? 0 : isc ? 1 : 2;
    e[1] = isr ? t.nks : isc ? 2 * t.rst : 2 * t.kst;
    for (int fq = 0; fq < 4; ++fq) {
        const int hh = fq >> 1, half = fq & 1;
        const int ksc = 2 * j1 + hh < rl ? 2 * j1 + hh : rl, ksa = 2 * j2 + hh < kl ? 2 * j2 + hh : kl;
        e[2 + fq] = isr ? 4 * kc + fq : isc ? 2 * ksc + half : 2 * ksa + half;
    }
    const int k0 = 2 * j2 < kl ? 2 * j2 : kl, k1 = 2 * j2 + 1 < kl ? 2 * j2 + 1 : kl;
    const int jc = j1 < t.nc - 1 ? j1 : (t.nc > 0 ? t.nc - 1 : 0);
    e[6] = isr ? 0 : 1;
    e[7] = isr ? kc : isc ? t.na + jc : k0 / 3;
    e[8] = isr ? kc : isc ? t.na + jc : k1 / 3;
    e[9] = isr || isc ? (0 | 1 << 8 | 2 << 16 | 3 << 24) : ((k0 % 3) | 3 << 8 | (k1 % 3) << 16 | 3 << 24);
    for (int w = 0; w < 4; ++w)
        e[10 + w] = t.gsteps == 4 ? kc : (kc * 4 + w) / t.gsteps;
    e[14] = e[15] = 0;
}

struct PrepArgs {
    const uint16_t *X;
    const float *tf32, *sf32;
    int64_t M, d, k, r, kst, rst, kpad, rpad;
    uint16_t *xsw, *tsw, *ssw;
    float *xsc;
    LdsStages st;
    int32_t *lfill;
};

__device__ __forceinline__ uint16_t f16_bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

__global__ __launch_bounds__(256) void prep_lds_kernel(PrepArgs a)
{
    __shared__ float red[4];
    if (blockIdx.x == 0)
        for (int s = threadIdx.x; s < a.st.nst; s += blockDim.x)
            lds_fill_entry(s, a.st, a.lfill + s * 16);
    const int64_t m = blockIdx.x;
    const bool live = m < a.M;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    float mx = 0.f;
    if (live) {
        const uint16_t *xr = a.X + m * a.d;
        for (int64_t j = threadIdx.x * 8; j < a.d; j += 256 * 8) {
            const u32x4 v = *(const u32x4 *)(xr + j);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
            for (int q = 0; q < 4; ++q) {
                mx = fmaxf(mx, fabsf(__uint_as_float(w[q] << 16)));
                mx = fmaxf(mx, fabsf(__uint_as_float(w[q] & 0xFFFF0000u)));
            }
        }
        for (int64_t c = threadIdx.x; c < a.k; c += 256)
            mx = fmaxf(mx, fabsf(a.tf32[m * a.kpad + c]));
        for (int64_t c = threadIdx.x; c < a.r; c += 256)
            mx = fmaxf(mx, fabsf(a.sf32[m * a.rpad + c]));
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
    if (threadIdx.x == 0) {
        a.xsc[2 * m] = ldexpf(1.f, -f);
        a.xsc[2 * m + 1] = ldexpf(1.f, f);
    }
    const int64_t mb16 = m >> 4, lrow = m & 15, nks = a.d / kKStep;
    // X: piece p = (K-step p / 4, quarter p % 4)
    for (int64_t p = threadIdx.x; p < a.d / 8; p += 256) {
        const int64_t ks = p >> 2, qq = p & 3;
        uint32_t o[4] = {0u, 0u, 0u, 0u};
        if (live) {
            const u32x4 v = *(const u32x4 *)(a.X + m * a.d + 8 * p);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
            for (int q = 0; q < 4; ++q)
                o[q] = (uint32_t)f16_bits(ldexpf(__uint_as_float(w[q] << 16), f)) |
                       ((uint32_t)f16_bits(ldexpf(__uint_as_float(w[q] & 0xFFFF0000u), f)) << 16);
        }
        *(u32x4 *)(a.xsw + ((mb16 * nks + ks) * 64 + lrow + 16 * qq) * 8) = u32x4{o[0], o[1], o[2], o[3]};
    }
    // t and s: hi and lo parts in consecutive blocks
    auto hilo = [&](const float *src, int64_t ncol, int64_t pitch, int64_t nst, uint16_t *dst) {
        for (int64_t p = threadIdx.x; p < nst * 4; p += 256) {
            const int64_t ks = p >> 2, qq = p & 3;
            uint16_t hi[8], lo[8];
            for (int e = 0; e < 8; ++e) {
                const int64_t c = 8 * p + e;
                const float v = (live && c < ncol) ? ldexpf(src[m * pitch + c], f) : 0.f;
                const _Float16 h = (_Float16)v;
                hi[e] = __builtin_bit_cast(uint16_t, h);
                lo[e] = f16_bits(v - (float)h);
            }
            uint32_t oh[4], ol[4];
            for (int q = 0; q < 4; ++q) {
                oh[q] = (uint32_t)hi[2 * q] | ((uint32_t)hi[2 * q + 1] << 16);
                ol[q] = (uint32_t)lo[2 * q] | ((uint32_t)lo[2 * q + 1] << 16);
            }
            const int64_t blk = (mb16 * nst + ks) * 2;
            *(u32x4 *)(dst + ((blk + 0) * 64 + lrow + 16 * qq) * 8) = u32x4{oh[0], oh[1], oh[2], oh[3]};
            *(u32x4 *)(dst + ((blk + 1) * 64 + lrow + 16 * qq) * 8) = u32x4{ol[0], ol[1], ol[2], ol[3]};
        }
    };
    hilo(a.tf32, a.k, a.kpad, a.kst, a.tsw);
    hilo(a.sf32, a.r, a.rpad, a.rst, a.ssw);
}

// ---------------------------------------------------------------------------
// B-operand dequantisation.
//
// Residual: a nibble u = q + 8 masked into bits 0-3 (4-7) of an fp16 half is
// the subnormal u 2^-24 (u 2^-20).  With S = srp = sR 2^(e_r + 14) (a
// normal fp16 below 2^15), one fused multiply-add per column pair,
//   u 2^-24 (S) + (-S 2^-21) = (u - 8) S 2^-24 = q sR 2^(e_r - 10),
//   u 2^-20 (S 2^-4) + (-S 2^-21) = the same,
// gives the product rounded once: the product of the two operands is exact
// inside the fma, and -S 2^-21 = -8 S 2^-24 is an exact normal fp16.  The
// kernel runs with fp16 denormals kept (the default mode).
// ---------------------------------------------------------------------------
struct R4Scale {
    f16x2 m0, m1, c; // S, S 2^-4, -S 2^-21 in both halves
};

__device__ __forceinline__ R4Scale r4_scale(uint32_t srp_bits)
{
    R4Scale r;
    r.m0 = __builtin_bit_cast(f16x2, srp_bits * 0x10001u);
    r.m1 = r.m0 * f16x2{(_Float16)0.0625f, (_Float16)0.0625f};
    r.c = r.m0 * f16x2{(_Float16)-4.76837158203125e-07f, (_Float16)-4.76837158203125e-07f}; // -2^-21
    return r;
}

__device__ __forceinline__ uint32_t f16x2_fma(uint32_t a, f16x2 b, f16x2 c)
{
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(f16x2, a), b, c));
}

// residual dword (8 offset-binary nibbles, slot order of layout.hpp): column
// pairs (0,1), (2,3), (4,5), (6,7) are the nibble pairs at bits (0,16),
// (4,20), (8,24), (12,28)
__device__ __forceinline__ u32x4 r4_f16(uint32_t w, const R4Scale &sc)
{
    const uint32_t w8 = w >> 8;
    return u32x4{f16x2_fma(w & 0x000F000Fu, sc.m0, sc.c), f16x2_fma(w & 0x00F000F0u, sc.m1, sc.c),
                 f16x2_fma(w8 & 0x000F000Fu, sc.m0, sc.c), f16x2_fma(w8 & 0x00F000F0u, sc.m1, sc.c)};
}

// exact fp16 integers from spliced codes: (1024 + u) - bias
__device__ __forceinline__ uint32_t f16x2_code(uint32_t spliced, float bias)
{
    const f16x2 b = {(_Float16)bias, (_Float16)bias};
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, spliced) - b);
}

// 5-bit core codes of one K-step as exact fp16 integers: nibble dword +
// high-bit dword (the K-step is number qq of its chunk)
__device__ __forceinline__ u32x4 a5_f16(uint32_t wn, uint32_t wh, int qq, uint32_t magic)
{
    const uint32_t m = 0x000F000Fu, hb = 0x00100010u;
    uint32_t o[4];
    for (int p = 0; p < 4; ++p) {
        const uint32_t u = ((wn >> (4 * p)) & m) | (rotr(wh, 4 * qq + p) & hb) | magic;
        o[p] = f16x2_code(u, 1040.f); // (1024 + a + 16) - 1040 = a
    }
    return u32x4{o[0], o[1], o[2], o[3]};
}

// correction codes of one K-step (two dwords of offset-binary bytes c ^ 0x80)
// as exact fp16 integers
__device__ __forceinline__ u32x4 c8_f16(uint32_t w0, uint32_t w1, uint32_t magic)
{
    // bytes 2p, 2p+1 of a dword into the low bytes of its two 16-bit halves
    // (v_perm_b32: selector 0x0c gives a zero byte)
    const uint32_t p0 = __builtin_amdgcn_perm(0u, w0, 0x0c010c00u), p1 = __builtin_amdgcn_perm(0u, w0, 0x0c030c02u);
    const uint32_t p2 = __builtin_amdgcn_perm(0u, w1, 0x0c010c00u), p3 = __builtin_amdgcn_perm(0u, w1, 0x0c030c02u);
    return u32x4{f16x2_code(p0 | magic, 1152.f), f16x2_code(p1 | magic, 1152.f), f16x2_code(p2 | magic, 1152.f),
                 f16x2_code(p3 | magic, 1152.f)}; // (1024 + c + 128) - 1152 = c
}

__device__ __forceinline__ u32x4 and4(u32x4 v, uint32_t m) { return u32x4{v.x & m, v.y & m, v.z & m, v.w & m}; }

struct LdsArgs {
    DevHead h;
    Work w;
    float *logits; // may be null
    int want_argmax;
    int gsteps;
    int64_t nvb, nkc, G, na, nc, kst, rst;
    int64_t nsr, nsc, nsa; // residual / correction / core stages (residual and core padded to even)
    int64_t n_vr, n_mt, n_tiles, per_xcd;
    int mt_major; // XCD x owns m-tiles x, x + 8, ... (n_mt % 8 == 0)
};

// direct copies into LDS: lane l's piece lands at dst + l pieces
__device__ __forceinline__ void lds_dma16(const void *src, uint32_t *dst)
{
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
}
__device__ __forceinline__ void lds_dma4(const void *src, uint32_t *dst)
{
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)dst, 4, 0, 0);
}

// Stages, in order: nsr residual stages (the four K-steps of K-chunk kc of
// X; a pad stage when nkc is odd), nsa core stages (K-steps 2j, 2j+1 of t;
// padded to even) and nc correction stages (K-steps 2j, 2j+1 of s).  Each
// stage has four operand slots q, each with 8 A blocks (one per m-block)
// and one B operand per v-block: core and correction slot q = 2 hh + half
// takes the hi or lo part of K-step 2j + hh; residual slot q is K-step q.
// Every stage runs the same 128 MFMAs per wave; slots past the end of a
// phase, and pad stages, have their B operands masked to zero.
template <int GS>
__global__ __launch_bounds__(kLW * 64, 1) void vtile_lds_kernel(LdsArgs a)
{
    // two stage buffers as separate objects, so that the compiler can tell
    // the asynchronous fill of one from the reads of the other
    __shared__ __attribute__((aligned(16))) uint32_t s_buf0[kLStageWords];
    __shared__ __attribute__((aligned(16))) uint32_t s_buf1[kLStageWords];
    __shared__ __attribute__((aligned(16))) float s_fm[2 * kLRows]; // 2^f_m, then 2^-f_m
    __shared__ uint64_t s_red[kLW * kLRows];
    __shared__ int32_t s_tgt[kLRows]; // targets of the tile's rows (cross-entropy)

    const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
    // wave index as a uniform value, so that everything derived from it
    // lives in scalar registers
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t bid = blockIdx.x;
    int64_t vr, mt;
    if (a.mt_major) {
        const int64_t x = bid & 7, j = bid >> 3, mpx = a.n_mt >> 3; // j-th tile of XCD x
        mt = x + 8 * (j % mpx);
        vr = j / mpx;
    } else {
        const int64_t L = (bid & 7) * a.per_xcd + (bid >> 3);
        if (L >= a.n_tiles)
            return; // the whole workgroup
        vr = L / a.n_mt;
        mt = L % a.n_mt;
    }
    const int64_t M = a.w.M, d = a.h.s.d, V = a.h.s.V;
    const int64_t nvb = a.nvb, G = a.G, nkc = a.nkc, kst = a.kst, rst = a.rst;
    // stage ranges: residual [0, p1), core [p1, p2), correction [p2, nst)
    const int64_t p1 = a.nsr, p2 = a.nsr + a.nsa, nst = a.nsr + a.nsa + a.nsc;
    const int64_t mbase = mt * kLRows, mb16_0 = mt * kLMB;
    const int64_t wg_vb0 = vr * kLVR;
    const int64_t vb0 = wg_vb0 + wv * kLVB;
    const int64_t nks = d / kKStep;
    const int gsteps = GS ? GS : a.gsteps;

    int64_t vb[kLVB];
    // bit v: sA of the lane's row in v-block v is nonzero; bit kLVB + v: sC
    uint32_t nz = 0;
#pragma unroll
    for (int v = 0; v < kLVB; ++v) {
        vb[v] = vb0 + v < nvb ? vb0 + v : nvb - 1;
        nz |= h2f(a.h.sa[vb[v] * kVB + lr]) != 0.f ? 1u << v : 0u;
        nz |= h2f(a.h.sc[vb[v] * kVB + lr]) != 0.f ? 1u << (kLVB + v) : 0u;
    }
    // unit divisors: sA (sC) of the lane's row, or 1 where it is zero
    auto pa = [&](int v) __attribute__((always_inline)) { const float x = h2f(a.h.sa[vb[v] * kVB + lr]); return x != 0.f ? x : 1.f; };
    auto pc = [&](int v) __attribute__((always_inline)) { const float x = h2f(a.h.sc[vb[v] * kVB + lr]); return x != 0.f ? x : 1.f; };
    if (threadIdx.x < kLRows) {
        const int64_t m = mbase + threadIdx.x; // below the prepared row count
        s_fm[threadIdx.x] = a.w.xsc[2 * m + 1];      // 2^f_m
        s_fm[kLRows + threadIdx.x] = a.w.xsc[2 * m]; // 2^-f_m
        if (a.w.want_lse && a.w.targets)
            s_tgt[threadIdx.x] = m < a.w.M ? a.w.targets[m] : -1;
    }

    // ---- stage fill --------------------------------------------------------
    // Operand block b = kLS wv + i holds slot q = b / 8, m-block b % 8; so
    // this wave copies slot fq, m-blocks fmb0 .. fmb0 + kLS - 1.
    const int fq = (wv * kLS) >> 3, fmb0 = (wv * kLS) & 7;
    const char *const lrb = (const char *)a.h.lr, *const r4b = (const char *)a.h.r4;
    const int64_t chunk_bytes = nvb * 1024; // one K-chunk of one stream
    // every copy reads a wave-uniform base plus one of two per-lane byte
    // offsets (no per-lane 64-bit address stays live across the stages)
    const uint32_t lane16 = (uint32_t)lane * 16u;
    // residual-scale rows this lane copies: v-block lane / 2 of the workgroup
    const int64_t svb = wg_vb0 + (lane >> 1) < nvb ? wg_vb0 + (lane >> 1) : nvb - 1;
    const uint32_t soffb = (uint32_t)(svb * G * kVB + 8 * (lane & 1)) * 2u; // + grp * 32

    // Stage s's copies, from row s of the stage-fill table (written by the
    // operand preparation; read through scalar loads): a few adds per copy
    // instead of recomputing the stage's indices in every wave.
    const char *const abases[3] = {(const char *)a.w.xsw, (const char *)a.w.ssw, (const char *)a.w.tsw};
    auto stage_fill = [&](int64_t s, uint32_t *buf) __attribute__((always_inline)) {
        typedef __attribute__((address_space(4))) const int32_t cint32;
        const cint32 *e = (cint32 *)a.w.lfill + s * 16;
        const int arr = e[0];
        const int64_t mstride = (int64_t)e[1] * 1024;
        const char *abase = (arr == 0 ? abases[0] : arr == 1 ? abases[1] : abases[2]) + mb16_0 * mstride +
                            (int64_t)e[2 + fq] * 1024;
        const char *cs = e[6] ? lrb : r4b;
        const char *c0 = cs + e[7] * chunk_bytes, *c1 = cs + e[8] * chunk_bytes;
        const uint32_t wsel = (uint32_t)e[9];
#pragma unroll
        for (int i = 0; i < kLS; ++i)
            lds_dma16(abase + (fmb0 + i) * mstride + lane16, buf + (wv * kLS + i) * 256);
        if (s < p1 || s >= p2) { // residual, correction: one whole chunk per v-block, 16-byte copies
#pragma unroll
            for (int v = 0; v < kLVB; ++v)
                lds_dma16(c0 + vb[v] * 1024 + lane16, buf + kLCodeOff + (wv * kLVB + v) * 256);
        } else { // words from up to two chunks: [4 words][lane], 4-byte copies
#pragma unroll
            for (int v = 0; v < kLVB; ++v)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    lds_dma4((q < 2 ? c0 : c1) + vb[v] * 1024 + ((wsel >> (8 * q)) & 0xFF) * 4 + lane16,
                             buf + kLCodeOff + (wv * kLVB + v) * 256 + q * 64);
        }
        if (s < p1 && (GS == 4 ? wv == 0 : wv < 4)) // kLW >= 4
            lds_dma16((const char *)a.h.srp + (int64_t)e[10 + wv] * (kVB * 2) + soffb,
                      buf + kLScOff + (GS == 4 ? 0 : wv) * (kLVR * 8));
    };

    // ---- compute -----------------------------------------------------------
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 T[kLMB][kLVB];
#pragma unroll
    for (int mb = 0; mb < kLMB; ++mb)
#pragma unroll
        for (int v = 0; v < kLVB; ++v)
            T[mb][v] = zero;
    const uint32_t magic = vgpr_const(kF16Magic);
    // code words: residual and correction stages hold [lane][4 words] per
    // v-block (read whole), core stages [4 words][lane]
    auto chunk = [&](const uint32_t *buf, int v) __attribute__((always_inline)) { return *(const u32x4 *)(buf + kLCodeOff + (wv * kLVB + v) * 256 + lane * 4); };
    auto code = [&](const uint32_t *buf, int v, int q) __attribute__((always_inline)) { return buf[kLCodeOff + (wv * kLVB + v) * 256 + q * 64 + lane]; };

    // the three stage kinds; no branch surrounds an MFMA (the accumulator
    // tile would be copied at every join): slots past the end of a phase, and
    // pad stages, have their B operands masked to zero
    auto mfma_slot = [&](const uint32_t *buf, int q, const u32x4(&bq)[kLVB]) __attribute__((always_inline)) {
#pragma unroll
        for (int mb = 0; mb < kLMB; ++mb) {
            const u32x4 ax = *(const u32x4 *)(buf + (q * 8 + mb) * 256 + lane * 4);
#pragma unroll
            for (int v = 0; v < kLVB; ++v)
                T[mb][v] = mfma_f16(ax, bq[v], T[mb][v]);
        }
    };
    auto compute_r4 = [&](int64_t s, const uint32_t *buf) __attribute__((always_inline)) {
        // pad stages: zero scales make every B operand zero
        const uint32_t live = s < nkc ? 0xFFFFu : 0u;
        const uint16_t *scb = (const uint16_t *)(buf + kLScOff);
        u32x4 c[kLVB];
#pragma unroll
        for (int v = 0; v < kLVB; ++v)
            c[v] = chunk(buf, v);
        R4Scale sc[kLVB];
        if constexpr (GS == 4)
#pragma unroll
            for (int v = 0; v < kLVB; ++v)
                sc[v] = r4_scale((uint32_t)scb[(wv * kLVB + v) * kVB + lr] & live);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            u32x4 bq[kLVB];
#pragma unroll
            for (int v = 0; v < kLVB; ++v) {
                if constexpr (GS != 4)
                    sc[v] = r4_scale((uint32_t)scb[(q * kLVR + wv * kLVB + v) * kVB + lr] & live);
                const uint32_t wd = q == 0 ? c[v].x : q == 1 ? c[v].y : q == 2 ? c[v].z : c[v].w;
                bq[v] = r4_f16(wd, sc[v]);
            }
            mfma_slot(buf, q, bq);
        }
    };
    auto compute_c8 = [&](int64_t s, const uint32_t *buf) __attribute__((always_inline)) {
        const int64_t j = s - p2;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const uint32_t live = (j < a.nc && 2 * j + hh < rst) ? 0xFFFFFFFFu : 0u;
            u32x4 bq[kLVB];
#pragma unroll
            for (int v = 0; v < kLVB; ++v) {
                const u32x4 c = chunk(buf, v);
                bq[v] = and4(c8_f16(hh == 0 ? c.x : c.z, hh == 0 ? c.y : c.w, magic),
                             ((nz >> (kLVB + v)) & 1u ? 0xFFFFFFFFu : 0u) & live);
            }
            mfma_slot(buf, 2 * hh, bq);     // hi part of s
            mfma_slot(buf, 2 * hh + 1, bq); // lo part of s
        }
    };
    auto compute_a5 = [&](int64_t s, const uint32_t *buf) __attribute__((always_inline)) {
        const int64_t j = s - p1;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int64_t ks = 2 * j + hh;
            const uint32_t live = ks < kst ? 0xFFFFFFFFu : 0u;
            const int qq = (int)(ks % 3);
            u32x4 bq[kLVB];
#pragma unroll
            for (int v = 0; v < kLVB; ++v)
                bq[v] = and4(a5_f16(code(buf, v, 2 * hh), code(buf, v, 2 * hh + 1), qq, magic),
                             ((nz >> v) & 1u ? 0xFFFFFFFFu : 0u) & live);
            mfma_slot(buf, 2 * hh, bq);
            mfma_slot(buf, 2 * hh + 1, bq);
        }
    };

    stage_fill(0, s_buf0);
    __syncthreads(); // every wave's fill of stage 0 and the s_fm stores

    // Stage s (even) computes from s_buf0 while stage s+1 fills s_buf1; the
    // barrier after it also waits for that fill.  No fill is left in flight
    // past the last stage.  Every phase starts on an even stage; only the
    // last one may end on an odd count, whose final stage (in s_buf0, filled
    // by the pair before it) runs alone.
#define ARCHEAD_LDS_PHASE(S0, S1, COMPUTE)                                          \
    for (int64_t s = (S0); s + 1 < (S1); s += 2) {                                 \
        stage_fill(s + 1, s_buf1);                                                 \
        COMPUTE(s, s_buf0);                                                        \
        __syncthreads();                                                           \
        if (s + 2 < nst)                                                           \
            stage_fill(s + 2, s_buf0);                                             \
        COMPUTE(s + 1, s_buf1);                                                    \
        __syncthreads();                                                           \
    }                                                                              \
    if (((S1) - (S0)) & 1) {                                                       \
        COMPUTE((S1) - 1, s_buf0);                                                 \
        __syncthreads();                                                           \
    }

    // phase 1: residual, in units of sR 2^(e_r - 10) 2^-f_m
    ARCHEAD_LDS_PHASE(0, p1, compute_r4)
    // to units of sA 2^-f_m
#pragma unroll
    for (int v = 0; v < kLVB; ++v) {
        const float f = a.h.rsc[vb[v] * kVB + lr] / pa(v);
#pragma unroll
        for (int mb = 0; mb < kLMB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                T[mb][v][i] *= f;
    }
    // phase 2: core
    ARCHEAD_LDS_PHASE(p1, p2, compute_a5)
    // to units of sC 2^-f_m
#pragma unroll
    for (int v = 0; v < kLVB; ++v) {
        const float f = pa(v) / pc(v);
#pragma unroll
        for (int mb = 0; mb < kLMB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                T[mb][v][i] *= f;
    }
    // phase 3: correction (the only phase that may end on an odd stage)
    ARCHEAD_LDS_PHASE(p2, nst, compute_c8)
#undef ARCHEAD_LDS_PHASE

    // back to logits units; write logits, the workgroup's top-1 keys and
    // its (max, sum exp) summaries.  The summaries go to the first stage
    // buffer: every stage has been consumed and no fill is in flight.
    LsePart *const s_lred = (LsePart *)s_buf0; // [kLW][kLRows]
    const bool want_lse = a.w.want_lse != 0;   // uniform across the grid
#pragma unroll
    for (int mb = 0; mb < kLMB; ++mb) {
        const f32x4 fi = *(const f32x4 *)(s_fm + kLRows + mb * 16 + 4 * lq);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t m = mbase + mb * 16 + 4 * lq + i;
            const int32_t tgt = (want_lse && a.w.targets && m < M) ? s_tgt[mb * 16 + 4 * lq + i] : -1;
            uint64_t k = 0;
            float y[kLVB], mx = -__builtin_inff();
#pragma unroll
            for (int v = 0; v < kLVB; ++v) {
                const int64_t row = (vb0 + v) * kVB + lr;
                y[v] = T[mb][v][i] * pc(v) * fi[i];
                if (m < M && vb0 + v < nvb && row < V) {
                    if (a.logits)
                        a.logits[m * V + row] = y[v];
                    k = umax64(k, argmax_key(y[v], (uint32_t)row));
                    mx = fmaxf(mx, y[v]);
                    if (row == tgt)
                        a.w.tl[m] = y[v];
                }
            }
            if (a.want_argmax) { // uniform across the grid
                k = umax16_u64(k);
                if (lr == 0)
                    s_red[wv * kLRows + mb * 16 + 4 * lq + i] = k;
            }
            if (want_lse) {
                mx = max16(mx);
                float sx = 0.f;
#pragma unroll
                for (int v = 0; v < kLVB; ++v) {
                    const int64_t row = (vb0 + v) * kVB + lr;
                    if (m < M && vb0 + v < nvb && row < V)
                        sx += exp_le0(y[v] - mx);
                }
                sx = sum16(sx);
                if (lr == 0)
                    s_lred[wv * kLRows + mb * 16 + 4 * lq + i] = LsePart{mx, sx};
            }
        }
    }
    if (!a.want_argmax && !want_lse)
        return;
    __syncthreads();
    if (threadIdx.x < kLRows) {
        const int64_t m = mbase + threadIdx.x;
        if (m < M && a.want_argmax) {
            uint64_t k = 0;
#pragma unroll
            for (int w = 0; w < kLW; ++w)
                k = umax64(k, s_red[w * kLRows + threadIdx.x]);
            a.w.part[m * a.w.n_part + vr] = k;
        }
        if (m < M && want_lse) {
            LsePart p = s_lred[threadIdx.x];
#pragma unroll
            for (int w = 1; w < kLW; ++w)
                p = lse_merge(p, s_lred[w * kLRows + threadIdx.x]);
            a.w.lsep[m * a.w.n_part + vr] = lse_bits(p);
        }
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
int64_t lds_max_n_part(const Shape &s) { return (s.nvb() + kLVR - 1) / kLVR; }

int64_t lds_stages(const Shape &s) { return lds_stage_info(s).nst; }

int64_t lds_n_part(const DevHead &h, int64_t M)
{
    (void)M;
    return lds_max_n_part(h.s);
}

hipError_t launch_prep_lds(const DevHead &h, const Work &w, const uint16_t *X, hipStream_t st)
{
    PrepArgs a;
    a.X = X;
    a.tf32 = w.tf32;
    a.sf32 = w.sf32;
    a.M = w.M;
    a.d = h.s.d;
    a.k = h.s.k;
    a.r = h.s.r;
    a.kst = h.s.kst();
    a.rst = h.s.rst();
    a.kpad = h.s.kpad();
    a.rpad = h.s.rpad();
    a.xsw = w.xsw;
    a.tsw = w.tsw;
    a.ssw = w.ssw;
    a.xsc = w.xsc;
    a.st = lds_stage_info(h.s);
    a.lfill = w.lfill;
    const int64_t rows = (w.M + kLRows - 1) / kLRows * kLRows; // the tiles' rows, <= Mq
    if (rows > w.Mq)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(prep_lds_kernel, dim3((unsigned)rows), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_vtile_lds(const DevHead &h, const Work &w, float *logits, int32_t *argmax,
                            hipStream_t st)
{
    LdsArgs a;
    a.h = h;
    a.w = w;
    a.w.n_part = lds_n_part(h, w.M);
    if (w.M * a.w.n_part > w.part_cap || (w.M + kLRows - 1) / kLRows * kLRows > w.Mq)
        return hipErrorInvalidValue; // the workspace does not hold this call
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
    const LdsStages t = lds_stage_info(h.s);
    a.nsr = t.p1;                  // one K-chunk per stage
    a.nsa = t.p2 - t.p1;           // two core K-steps per stage
    a.nsc = t.nst - t.p2;          // two correction K-steps per stage
    a.n_vr = a.w.n_part;
    a.n_mt = (w.M + kLRows - 1) / kLRows;
    a.n_tiles = a.n_vr * a.n_mt;
    a.mt_major = a.n_mt % 8 == 0;
    const int64_t grid = (a.n_tiles + 7) / 8 * 8;
    a.per_xcd = grid / 8;
    if (a.gsteps == 4)
        hipLaunchKernelGGL(vtile_lds_kernel<4>, dim3((unsigned)grid), dim3(kLW * 64), 0, st, a);
    else
        hipLaunchKernelGGL(vtile_lds_kernel<0>, dim3((unsigned)grid), dim3(kLW * 64), 0, st, a);
    return hipGetLastError();
}

} // namespace archead
