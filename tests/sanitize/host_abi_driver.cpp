// host_abi_driver.cpp -- drives the library's host code (argument checks,
// the relayout of the packed fields into the device layout, workspace sizing)
// under AddressSanitizer and UndefinedBehaviorSanitizer.  TEST
// INFRASTRUCTURE: built and run by tests/test_sanitizers.py on a machine
// without a GPU, where archead_pack_load runs its whole host relayout and
// then fails at the first device call.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "archead.h"

namespace {

int failures = 0;

void expect(bool ok, const char *what)
{
    if (!ok) {
        std::fprintf(stderr, "FAILED: %s (last error: %s)\n", what, archead_last_error());
        ++failures;
    }
}

struct Fields {
    std::vector<int8_t> A5, B8, C8, D8;
    std::vector<uint8_t> R4;
    std::vector<uint16_t> sA, sB, sR, sC, sD;
};

// exact-size buffers (no slack), so that any read past an end is caught
Fields make(int64_t V, int64_t d, int64_t k, int64_t r, int64_t g, uint32_t seed)
{
    std::mt19937 rng(seed);
    auto u8 = [&] { return (uint8_t)(rng() & 0xFF); };
    auto half = [&] { return (uint16_t)(0x1C00 + (rng() % 0x0800)); }; // positive normal fp16
    Fields f;
    f.A5.resize(V * k);
    for (auto &x : f.A5)
        x = (int8_t)((int)(rng() % 32) - 16);
    f.B8.resize(k * d);
    for (auto &x : f.B8)
        x = (int8_t)u8();
    f.C8.resize(V * r);
    for (auto &x : f.C8)
        x = (int8_t)u8();
    f.D8.resize(r * d);
    for (auto &x : f.D8)
        x = (int8_t)u8();
    f.R4.resize(V * d / 2);
    for (auto &x : f.R4)
        x = u8();
    f.sA.resize(V);
    f.sC.resize(V);
    f.sB.resize(k);
    f.sR.resize(V * (d / g));
    f.sD.resize(r * (d / g));
    for (auto *v : {&f.sA, &f.sB, &f.sR, &f.sC, &f.sD})
        for (auto &x : *v)
            x = half();
    return f;
}

template <typename T>
const T *ptr(const std::vector<T> &v) { return v.empty() ? nullptr : v.data(); }

archead_status load(const Fields &f, int64_t V, int64_t d, int64_t k, int64_t r, int64_t g, archead_t *h)
{
    return archead_pack_load(V, d, k, r, g, ptr(f.A5), ptr(f.sA), ptr(f.B8), ptr(f.sB), ptr(f.R4), ptr(f.sR),
                             ptr(f.C8), ptr(f.sC), ptr(f.D8), ptr(f.sD), nullptr, h);
}

} // namespace

int main()
{
    const int64_t shapes[][5] = {
        // V, d, k, r, g
        {1, 128, 1, 1, 32},     {15, 128, 8, 4, 32},    {17, 256, 16, 4, 64},  {1000, 384, 33, 7, 96},
        {777, 512, 0, 16, 256}, {777, 512, 40, 0, 512}, {500, 512, 0, 0, 128}, {300, 1024, 256, 64, 128},
        {4099, 640, 64, 48, 128}, {33, 2560, 192, 48, 128}, {2, 128, 97, 65, 128}, {31, 1536, 96, 33, 96},
    };
    for (const auto &sh : shapes) {
        const int64_t V = sh[0], d = sh[1], k = sh[2], r = sh[3], g = sh[4];
        const Fields f = make(V, d, k, r, g, (uint32_t)(V * 131 + d + k * 7 + r));
        archead_t h = nullptr;
        const archead_status st = load(f, V, d, k, r, g, &h);
        // without a GPU the relayout completes and the upload fails
        expect(st == ARCHEAD_OK || st == ARCHEAD_EHIP || st == ARCHEAD_ENOMEM, "pack_load of a valid shape");
        if (st == ARCHEAD_OK)
            expect(archead_free(h) == ARCHEAD_OK, "free");
        else
            expect(h == nullptr, "no handle on failure");
    }
    // argument checks before anything touches the device
    {
        const Fields f = make(32, 128, 8, 4, 32, 1);
        archead_t h = nullptr;
        expect(load(f, 0, 128, 8, 4, 32, &h) == ARCHEAD_ESHAPE, "V = 0");
        expect(load(f, 32, 96, 8, 4, 32, &h) == ARCHEAD_ESHAPE, "d = 96");
        expect(load(f, 32, 128, 8, 4, 48, &h) == ARCHEAD_ESHAPE, "g = 48");
        expect(load(f, 32, 128, 5000, 4, 32, &h) == ARCHEAD_ESHAPE, "k = 5000");
        Fields bad = f;
        bad.A5[bad.A5.size() - 1] = 16;
        expect(load(bad, 32, 128, 8, 4, 32, &h) == ARCHEAD_ERANGE, "A5 out of range");
        expect(archead_pack_load(32, 128, 8, 4, 32, nullptr, nullptr, nullptr, nullptr, ptr(f.R4), ptr(f.sR),
                                 nullptr, nullptr, nullptr, nullptr, nullptr, &h) == ARCHEAD_EINVAL,
               "missing core fields");
        expect(archead_pack_load(32, 128, 8, 4, 32, ptr(f.A5), ptr(f.sA), ptr(f.B8), ptr(f.sB), ptr(f.R4),
                                 ptr(f.sR), ptr(f.C8), ptr(f.sC), ptr(f.D8), ptr(f.sD), nullptr,
                                 nullptr) == ARCHEAD_EINVAL,
               "NULL out");
    }
    // calls on a handle that was never made
    {
        archead_t bogus = reinterpret_cast<archead_t>(uintptr_t(0x1000));
        float y = 0.f;
        int32_t a = 0;
        uint64_t n = 0;
        expect(archead_forward(bogus, 1, &y, &y, nullptr) == ARCHEAD_EINVAL, "forward on a bogus handle");
        expect(archead_forward_argmax(bogus, 1, &y, &y, &a, nullptr) == ARCHEAD_EINVAL, "argmax on a bogus handle");
        expect(archead_forward_argmax_noalloc(bogus, 1, &y, &y, &a, nullptr) == ARCHEAD_EINVAL,
               "noalloc on a bogus handle");
        expect(archead_forward_topk(bogus, 1, &y, 4, &y, &y, &a, nullptr) == ARCHEAD_EINVAL, "topk on a bogus handle");
        expect(archead_reserve(bogus, 8, nullptr) == ARCHEAD_EINVAL, "reserve on a bogus handle");
        expect(archead_packed_bytes(bogus, &n) == ARCHEAD_EINVAL, "packed_bytes on a bogus handle");
        expect(archead_free(bogus) == ARCHEAD_EINVAL, "free of a bogus handle");
        expect(archead_free(nullptr) == ARCHEAD_OK, "free(NULL)");
        for (int s = 0; s <= 6; ++s)
            expect(archead_status_string((archead_status)s) != nullptr, "status string");
    }
    std::printf("host ABI driver: %d failure(s)\n", failures);
    return failures ? 1 : 0;
}
