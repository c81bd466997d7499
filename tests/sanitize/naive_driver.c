/* naive_driver.c -- runs the oracle's C triple loop (oracle/naive.c) on
 * random tiny heads with exact-size buffers, under AddressSanitizer and
 * UndefinedBehaviorSanitizer.  TEST INFRASTRUCTURE: built and run by
 * tests/test_sanitizers.py. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int naive_forward(int64_t V, int64_t d, int64_t k, int64_t r, int64_t g, int64_t M, const int8_t *A5,
                  const uint16_t *sA, const int8_t *B8, const uint16_t *sB, const uint8_t *R4,
                  const uint16_t *sR, const int8_t *C8, const uint16_t *sC, const int8_t *D8,
                  const uint16_t *sD, const uint16_t *X, double *out);

static uint32_t state = 12345u;
static uint32_t next(void)
{
    state ^= state << 13;
    state ^= state >> 17;
    state ^= state << 5;
    return state;
}

static void *fill(size_t n, size_t esz, int kind)
{
    unsigned char *p = (unsigned char *)malloc(n * esz ? n * esz : 1);
    for (size_t i = 0; i < n * esz; ++i)
        p[i] = (unsigned char)next();
    if (kind == 1) /* A5 in [-16, 15] */
        for (size_t i = 0; i < n; ++i)
            ((int8_t *)p)[i] = (int8_t)((int)(next() % 32) - 16);
    if (kind == 2) /* positive normal fp16 */
        for (size_t i = 0; i < n; ++i)
            ((uint16_t *)p)[i] = (uint16_t)(0x1C00 + next() % 0x0800);
    if (kind == 3) /* bf16 of moderate size */
        for (size_t i = 0; i < n; ++i)
            ((uint16_t *)p)[i] = (uint16_t)(0x3C00 + next() % 0x0600) | (uint16_t)((next() & 1) << 15);
    return p;
}

int main(void)
{
    const int64_t shapes[][6] = {{1, 128, 1, 1, 32, 1}, {15, 128, 8, 4, 32, 2}, {37, 128, 5, 3, 64, 3},
                                 {9, 256, 0, 0, 128, 1}, {20, 96, 7, 2, 32, 4}, {3, 64, 2, 0, 64, 2}};
    int bad = 0;
    for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s) {
        const int64_t V = shapes[s][0], d = shapes[s][1], k = shapes[s][2], r = shapes[s][3], g = shapes[s][4],
                      M = shapes[s][5];
        int8_t *A5 = fill(V * k, 1, 1), *B8 = fill(k * d, 1, 0), *C8 = fill(V * r, 1, 0), *D8 = fill(r * d, 1, 0);
        uint8_t *R4 = fill(V * d / 2, 1, 0);
        uint16_t *sA = fill(V, 2, 2), *sB = fill(k, 2, 2), *sR = fill(V * (d / g), 2, 2), *sC = fill(V, 2, 2),
                 *sD = fill(r * (d / g), 2, 2), *X = fill(M * d, 2, 3);
        double *out = (double *)malloc(sizeof(double) * M * V);
        if (naive_forward(V, d, k, r, g, M, A5, sA, B8, sB, R4, sR, C8, sC, D8, sD, X, out) != 0)
            ++bad;
        for (int64_t i = 0; i < M * V; ++i)
            if (!isfinite(out[i]))
                ++bad;
        free(A5), free(B8), free(C8), free(D8), free(R4), free(sA), free(sB), free(sR), free(sC), free(sD),
            free(X), free(out);
    }
    printf("naive driver: %d failure(s)\n", bad);
    return bad ? 1 : 0;
}
