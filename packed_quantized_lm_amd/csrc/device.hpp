// device.hpp -- gfx950 device helpers shared by the ARCHead kernels.
//
// Exact-integer dequantisation by exponent splicing: OR-ing an unsigned
// integer u < 128 into the mantissa of bf16 128.0 (0x4300) gives the bf16
// value 128 + u exactly (the ulp at 128 is 1).  Likewise fp16 1024.0
// (0x6400) takes u < 1024 and gives 1024 + u.  Offset-binary storage
// (u = q + bias) therefore turns into exact small integers with one mask-or
// per column pair; the constant offset is removed inside the fp32 MFMA
// accumulator (bf16 paths) or by one packed fp16 add (fp16 paths).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.hpp"

namespace archead {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr uint32_t kBf16Magic = 0x43004300u;  // bf16 pair (128, 128)
constexpr uint32_t kF16Magic = 0x64006400u;   // fp16 pair (1024, 1024)
constexpr float kR4Bias = 136.0f;             // 128 + 8: bf16 value of residual q is q + 136
constexpr float kA5Bias = 144.0f;             // 128 + 16: bf16 value of core code a is a + 144

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

__device__ __forceinline__ uint32_t rotr(uint32_t x, uint32_t n)
{
    return __builtin_amdgcn_alignbit(x, x, n);
}

// A uniform constant held in a VGPR.  With the magic exponent in a VGPR and
// the mask in an SGPR the compiler emits one v_and_or_b32 per column pair
// (VOP3 takes no literal); given two literals it emits v_and + v_or.  Only
// this move is opaque: every instruction that feeds an MFMA is still the
// compiler's own, so its hazard tracking stays intact.
__device__ __forceinline__ uint32_t vgpr_const(uint32_t c)
{
    uint32_t r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "s"(c));
    return r;
}

// Residual dword (8 offset-binary nibbles, slot order of layout.hpp) ->
// 8 bf16 values q + 136, columns in natural order.  c must be
// vgpr_const(kBf16Magic).
__device__ __forceinline__ u32x4 r4_bf16(uint32_t w, uint32_t c)
{
    const uint32_t m = 0x000F000Fu;
    u32x4 o;
    o.x = (w & m) | c;
    o.y = ((w >> 4) & m) | c;
    o.z = ((w >> 8) & m) | c;
    o.w = ((w >> 12) & m) | c;
    return o;
}

__device__ __forceinline__ u32x4 r4_bf16(uint32_t w)
{
    u32x4 o;
    o.x = (w & 0x000F000Fu) | kBf16Magic;
    o.y = ((w >> 4) & 0x000F000Fu) | kBf16Magic;
    o.z = ((w >> 8) & 0x000F000Fu) | kBf16Magic;
    o.w = ((w >> 12) & 0x000F000Fu) | kBf16Magic;
    return o;
}

// Same nibbles -> 8 fp16 values q + 1032 (1024 + 8).
__device__ __forceinline__ u32x4 r4_f16_biased(uint32_t w)
{
    u32x4 o;
    o.x = (w & 0x000F000Fu) | kF16Magic;
    o.y = ((w >> 4) & 0x000F000Fu) | kF16Magic;
    o.z = ((w >> 8) & 0x000F000Fu) | kF16Magic;
    o.w = ((w >> 12) & 0x000F000Fu) | kF16Magic;
    return o;
}

// 5-bit core code of K-step q (0..3 within its high-bit dword): nibble plane
// dword wn + high-bit dword wh -> 8 bf16 values a + 144.
template <int Q>
__device__ __forceinline__ u32x4 a5_bf16(uint32_t wn, uint32_t wh)
{
    u32x4 o;
    o.x = ((wn & 0x000F000Fu) | kBf16Magic) | (rotr(wh, 4 * Q + 0) & 0x00100010u);
    o.y = (((wn >> 4) & 0x000F000Fu) | kBf16Magic) | (rotr(wh, 4 * Q + 1) & 0x00100010u);
    o.z = (((wn >> 8) & 0x000F000Fu) | kBf16Magic) | (rotr(wh, 4 * Q + 2) & 0x00100010u);
    o.w = (((wn >> 12) & 0x000F000Fu) | kBf16Magic) | (rotr(wh, 4 * Q + 3) & 0x00100010u);
    return o;
}

__device__ __forceinline__ u32x4 a5_bf16_q(uint32_t wn, uint32_t wh, int q)
{
    switch (q) {
    case 0: return a5_bf16<0>(wn, wh);
    case 1: return a5_bf16<1>(wn, wh);
    case 2: return a5_bf16<2>(wn, wh);
    default: return a5_bf16<3>(wn, wh);
    }
}

// Exact fp32 -> bf16 pair for values that bf16 represents exactly (the low
// 16 bits of both fp32 patterns are zero): take the two high halves.
__device__ __forceinline__ uint32_t pack_hi_halves(float lo, float hi)
{
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Correction factor bytes (offset binary c ^ 0x80, 8 columns in order) ->
// 8 exact bf16 integers c.
__device__ __forceinline__ u32x4 c8_bf16(u32x2 w)
{
    u32x4 o;
    float f0 = (float)((w.x >> 0) & 0xFFu) - 128.0f;
    float f1 = (float)((w.x >> 8) & 0xFFu) - 128.0f;
    float f2 = (float)((w.x >> 16) & 0xFFu) - 128.0f;
    float f3 = (float)((w.x >> 24) & 0xFFu) - 128.0f;
    float f4 = (float)((w.y >> 0) & 0xFFu) - 128.0f;
    float f5 = (float)((w.y >> 8) & 0xFFu) - 128.0f;
    float f6 = (float)((w.y >> 16) & 0xFFu) - 128.0f;
    float f7 = (float)((w.y >> 24) & 0xFFu) - 128.0f;
    o.x = pack_hi_halves(f0, f1);
    o.y = pack_hi_halves(f2, f3);
    o.z = pack_hi_halves(f4, f5);
    o.w = pack_hi_halves(f6, f7);
    return o;
}

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(a), as_f16x8(b), c, 0, 0, 0);
}

// bf16 halves of a packed pair as fp32 (exact)
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

__device__ __forceinline__ float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// Order-preserving map of fp32 to uint32 (for max over packed keys); -0 is
// folded onto +0 first so that equal values compare equal.
__device__ __forceinline__ uint32_t orderable(float f)
{
    uint32_t b = __float_as_uint(f + 0.0f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Argmax key: larger value wins, then the lower index (stored inverted).
__device__ __forceinline__ uint64_t argmax_key(float f, uint32_t idx)
{
    return ((uint64_t)orderable(f) << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m)
{
    uint32_t lo = __shfl_xor((uint32_t)v, m);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// ---- log-sum-exp partials ---------------------------------------------------
// A set of logits is summarised by (mx, s): its maximum and the sum of
// exp(y - mx) over it; the empty set is (-inf, 0).  Two summaries merge
// exactly in real arithmetic, so the tiles of a row can be reduced in any
// order.  exp(x) for x <= 0 is taken as 2^(x log2 e) on the hardware base-2
// exponential.
constexpr float kLog2e = 1.44269504088896340736f;
__device__ __forceinline__ float exp_le0(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

struct LsePart {
    float mx, s;
};

__device__ __forceinline__ LsePart lse_merge(LsePart a, LsePart b)
{
    const float mx = fmaxf(a.mx, b.mx);
    if (mx == -__builtin_inff())
        return {mx, 0.f};
    return {mx, a.s * exp_le0(a.mx - mx) + b.s * exp_le0(b.mx - mx)};
}

// a summary as one 64-bit word (for the single-launch path's atomic stores)
__device__ __forceinline__ uint64_t lse_bits(LsePart p)
{
    return ((uint64_t)__float_as_uint(p.s) << 32) | (uint64_t)__float_as_uint(p.mx);
}
__device__ __forceinline__ LsePart lse_unbits(uint64_t b)
{
    return {__uint_as_float((uint32_t)b), __uint_as_float((uint32_t)(b >> 32))};
}

// max / sum over each row of 16 lanes (one MFMA column group), every lane
// getting the result, with DPP lane moves instead of LDS permutes: swap
// neighbours (quad_perm 1,0,3,2), swap pairs (quad_perm 2,3,0,1), then -- all
// four lanes of a quad now equal -- mirror each half row (lane i <- 7 - i)
// and each row (lane i <- 15 - i), which meet quads and halves pairwise.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E, kDppRowMirror = 0x140, kDppHalfMirror = 0x141;
__device__ __forceinline__ float max16(float x)
{
    x = fmaxf(x, dpp_move<kDppQuadXor1>(x));
    x = fmaxf(x, dpp_move<kDppQuadXor2>(x));
    x = fmaxf(x, dpp_move<kDppHalfMirror>(x));
    return fmaxf(x, dpp_move<kDppRowMirror>(x));
}
__device__ __forceinline__ float sum16(float x)
{
    x += dpp_move<kDppQuadXor1>(x);
    x += dpp_move<kDppQuadXor2>(x);
    x += dpp_move<kDppHalfMirror>(x);
    return x + dpp_move<kDppRowMirror>(x);
}
// the same for the 64-bit argmax keys: the maximum key over each row of 16 lanes
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_move_u64(uint64_t v)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t umax16_u64(uint64_t k)
{
    k = umax64(k, dpp_move_u64<kDppQuadXor1>(k));
    k = umax64(k, dpp_move_u64<kDppQuadXor2>(k));
    k = umax64(k, dpp_move_u64<kDppHalfMirror>(k));
    return umax64(k, dpp_move_u64<kDppRowMirror>(k));
}

// lane src's 64-bit value, in every lane (src uniform)
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int src)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, src);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), src);
    return ((uint64_t)hi << 32) | lo;
}

// a DPP move applied to the rows in ROWMASK only; the other lanes keep v
template <int CTRL, int ROWMASK>
__device__ __forceinline__ uint64_t dpp_rows_u64(uint64_t v)
{
    const int lo = (int)(uint32_t)v, hi = (int)(uint32_t)(v >> 32);
    const uint32_t l = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROWMASK, 0xF, false);
    const uint32_t h = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROWMASK, 0xF, false);
    return ((uint64_t)h << 32) | l;
}
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

// the largest key of the wave, in every lane: the maximum within each row of
// 16 lanes, then lane 15 of rows 0 and 2 into rows 1 and 3, then lane 31
// into rows 2 and 3, so that lane 63 holds the wave's maximum
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k)
{
    k = umax16_u64(k);
    k = umax64(k, dpp_rows_u64<kDppRowBcast15, 0xA>(k));
    k = umax64(k, dpp_rows_u64<kDppRowBcast31, 0xC>(k));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)k, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(k >> 32), 63);
    return ((uint64_t)hi << 32) | lo;
}

// the logit an argmax key encodes (the inverse of orderable(); -0 comes back as +0)
__device__ __forceinline__ float key_value(uint64_t k)
{
    const uint32_t h = (uint32_t)(k >> 32);
    return __uint_as_float((h & 0x80000000u) ? (h & 0x7FFFFFFFu) : ~h);
}

// merge of the summaries held by all 64 lanes (every lane gets the result)
__device__ __forceinline__ LsePart lse_merge64(LsePart p)
{
#pragma unroll
    for (int off = 1; off < 64; off <<= 1)
        p = lse_merge(p, LsePart{__shfl_xor(p.mx, off), __shfl_xor(p.s, off)});
    return p;
}

// s_waitcnt vmcnt(0): every vector memory access of the wave, stores and
// atomics included, has completed
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// s_waitcnt operand for vmcnt(n) alone (n < 64; low four bits at 3:0, high
// two at 15:14; expcnt and lgkmcnt at their no-wait maxima)
constexpr unsigned waitcnt_vm(unsigned n) { return (n & 15u) | ((n >> 4) & 3u) << 14 | 0x7u << 4 | 0xFu << 8; }
static_assert(waitcnt_vm(0) == 0x0F70u, "vmcnt(0)");

// Direct copy of one 16-byte piece per lane from global memory (p, per
// lane) to LDS (dst + 16 lane; dst the same in every lane), sc1 (device
// scope) when DEVICE.  Written as inline assembly because its callers wait
// for the copy themselves with a partial vmcnt: the compiler, which cannot
// tell which LDS reads a copy may alias, would wait for every outstanding
// load (vmcnt(0)) before the next LDS read or barrier.  Hidden from the
// compiler's count of outstanding loads, the copy can only make its waits
// stricter than needed, never too weak.  M0 (the LDS base of the copy) is
// restored afterwards.
template <bool DEVICE>
__device__ __forceinline__ void lds_dma16(const void *p, void *dst)
{
    const uint32_t base =
        __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)dst);
    uint32_t m0;
    if constexpr (DEVICE)
        asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
                     "global_load_lds_dwordx4 %1, off sc1\n\ts_nop 0\n\ts_mov_b32 m0, %0"
                     : "=&s"(m0)
                     : "v"(p), "s"(base)
                     : "memory");
    else
        asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
                     "global_load_lds_dwordx4 %1, off\n\ts_nop 0\n\ts_mov_b32 m0, %0"
                     : "=&s"(m0)
                     : "v"(p), "s"(base)
                     : "memory");
}


// The same for one 4-byte piece per lane (LDS dst + 4 lane).
__device__ __forceinline__ void lds_dma4(const void *p, void *dst)
{
    const uint32_t base =
        __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)dst);
    uint32_t m0;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
                 "global_load_lds_dword %1, off\n\ts_nop 0\n\ts_mov_b32 m0, %0"
                 : "=&s"(m0)
                 : "v"(p), "s"(base)
                 : "memory");
}

} // namespace archead
