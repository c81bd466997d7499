// pack.cpp -- host relayout of the canonical packed fields into the device
// layout described in layout.hpp.  Runs once per archead_pack_load, on the
// host, split over threads by v-block ranges.
#include "layout.hpp"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

namespace archead {

float half_to_float(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

uint16_t float_to_half(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

namespace {

// nibble slot of column e (0..7) inside a lane's dword: pairs (2p, 2p+1)
// land in slots (p, p+4), i.e. the two 16-bit halves after a mask.
inline int slot(int e) { return (e >> 1) + 4 * (e & 1); }

inline int r4_value(const uint8_t *R4, int64_t row, int64_t col, int64_t d)
{
    uint8_t byte = R4[row * (d / 2) + col / 2];
    int n = (col & 1) ? (byte >> 4) : (byte & 0xF);
    return (n ^ 8) - 8; // 4-bit two's complement
}

void relayout_blocks(const Shape &s, const int8_t *A5, const uint16_t *sA, const uint8_t *R4,
                     const uint16_t *sR, const int8_t *C8, const uint16_t *sC,
                     const HostDevImage &o, int64_t vb0, int64_t vb1)
{
    const int64_t V = s.V, d = s.d, k = s.k, r = s.r, G = s.G();
    const int64_t nvb = s.nvb(), nkc = s.nkc();
    for (int64_t vb = vb0; vb < vb1; ++vb) {
        for (int lane = 0; lane < 64; ++lane) {
            const int64_t row = vb * kVB + (lane & 15);
            const bool live = row < V;
            const int quarter = lane >> 4;
            // SC4 residual, offset binary
            for (int64_t kc = 0; kc < nkc; ++kc) {
                for (int st = 0; st < 4; ++st) {
                    uint32_t w = 0;
                    for (int e = 0; e < 8; ++e) {
                        int64_t col = kc * kKChunk + st * kKStep + 8 * quarter + e;
                        int q = live ? r4_value(R4, row, col, d) : 0;
                        w |= (uint32_t)((q + 8) & 0xF) << (4 * slot(e));
                    }
                    o.r4[((kc * nvb + vb) * 64 + lane) * 4 + st] = w;
                }
            }
            // low-rank chunk stream: core K-steps in threes, then correction K-steps in twos
            {
                const int64_t na = s.lr_na(), nc = s.n_lr() - na;
                auto nib_word = [&](int64_t st, uint32_t *hbits, int q) {
                    uint32_t nw = 0;
                    for (int e = 0; e < 8; ++e) {
                        int64_t col = st * kKStep + 8 * quarter + e;
                        int a = (live && col < k) ? A5[row * k + col] : 0;
                        uint32_t u5 = (uint32_t)(a + 16);
                        nw |= (u5 & 0xF) << (4 * slot(e));
                        int bit = (4 + 4 * q + (e >> 1) + 16 * (e & 1)) & 31;
                        *hbits |= (u5 >> 4) << bit;
                    }
                    return nw;
                };
                for (int64_t j = 0; j < na; ++j) {
                    uint32_t hb = 0, w[4];
                    for (int q = 0; q < 3; ++q)
                        w[q] = nib_word(3 * j + q, &hb, q);
                    w[3] = hb;
                    for (int q = 0; q < 4; ++q)
                        o.lr[((j * nvb + vb) * 64 + lane) * 4 + q] = w[q];
                }
                for (int64_t j = 0; j < nc; ++j) {
                    uint32_t w[4] = {0, 0, 0, 0};
                    for (int h = 0; h < 2; ++h)
                        for (int e = 0; e < 8; ++e) {
                            int64_t col = (2 * j + h) * kKStep + 8 * quarter + e;
                            int c = (live && col < r) ? C8[row * r + col] : 0;
                            w[2 * h + (e >> 2)] |= (uint32_t)((uint8_t)c ^ 0x80u) << (8 * (e & 3));
                        }
                    for (int q = 0; q < 4; ++q)
                        o.lr[(((na + j) * nvb + vb) * 64 + lane) * 4 + q] = w[q];
                }
            }
        }
        for (int i = 0; i < kVB; ++i) {
            const int64_t row = vb * kVB + i;
            const bool live = row < V;
            for (int64_t c = 0; c < G; ++c)
                o.sr[(vb * G + c) * kVB + i] = live ? sR[row * G + c] : 0;
            // power-of-two rescale of the residual scales for the fp16 path:
            // the row's largest into [2^14, 2^15)
            float mr = 0.f;
            for (int64_t c = 0; live && c < G; ++c)
                mr = std::max(mr, std::fabs(half_to_float(sR[row * G + c])));
            const int er = (mr > 0.f && std::isfinite(mr)) ? -std::ilogb(mr) : 0;
            for (int64_t c = 0; c < G; ++c)
                o.srp[(vb * G + c) * kVB + i] =
                    live ? float_to_half(std::ldexp(half_to_float(sR[row * G + c]), er + 14)) : 0;
            o.rsc[row] = std::ldexp(1.0f, 10 - er);
            o.sa[row] = (live && k > 0) ? sA[row] : 0;
            o.sc[row] = (live && r > 0) ? sC[row] : 0;
        }
    }
}

} // namespace

void relayout(const Shape &s, const int8_t *A5, const uint16_t *sA, const uint16_t *sB,
              const uint8_t *R4, const uint16_t *sR, const int8_t *C8, const uint16_t *sC,
              const uint16_t *sD, const HostDevImage &o, int n_threads)
{
    const int64_t nvb = s.nvb(), G = s.G();
    for (int64_t i = 0; i < s.k; ++i)
        o.sb[i] = half_to_float(sB[i]);
    for (int64_t i = 0; i < s.r * G; ++i)
        o.sd[i] = half_to_float(sD[i]);
    n_threads = std::max(1, std::min<int>(n_threads, (int)std::min<int64_t>(nvb, 64)));
    std::vector<std::thread> pool;
    const int64_t per = (nvb + n_threads - 1) / n_threads;
    for (int t = 0; t < n_threads; ++t) {
        int64_t a = t * per, b = std::min(nvb, a + per);
        if (a >= b)
            break;
        pool.emplace_back(relayout_blocks, std::cref(s), A5, sA, R4, sR, C8, sC, std::cref(o), a, b);
    }
    for (auto &th : pool)
        th.join();
}

} // namespace archead
