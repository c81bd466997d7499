/*
 * naive.c -- independent triple-loop forward of the packed ARCHead head.
 * TEST INFRASTRUCTURE ONLY (part of the CPU oracle; never linked into the
 * product library).
 *
 * ARCHead paper, section 3.2, eqs 3, 6 and 7, with the INT8 correction
 * factors of the text after eq 7.  Every weight element is rebuilt from the
 * canonical bytes on the spot and multiplied into the logit in fp64:
 *
 *   W_hat[v][j] = sum_i sA[v] A5[v][i] sB[i] B8[i][j]
 *               + sR[v][j/g] R4[v][j]
 *               + sum_i sC[v] C8[v][i] sD[i][j/g] D8[i][j]
 *   out[m][v]   = sum_j X[m][j] W_hat[v][j]
 *
 * It decodes fp16, bf16 and the R4 nibbles with its own bit manipulation so
 * that it shares nothing with the numpy oracle it cross-checks.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static double half_to_double(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 10) & 0x1f;
    int man = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)man, -24);             /* subnormal: man * 2^-24 */
    else if (e == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(man | 0x400), e - 25); /* 1.man * 2^(e-15) */
    return sign ? -v : v;
}

static double bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static int r4_value(const uint8_t *R4, int64_t v, int64_t j, int64_t d)
{
    uint8_t byte = R4[v * (d / 2) + j / 2];
    int n = (j & 1) ? (byte >> 4) : (byte & 0x0f);
    return n >= 8 ? n - 16 : n;
}

/* All pointers are host memory in the canonical layout; out is M x V fp64. */
int naive_forward(int64_t V, int64_t d, int64_t k, int64_t r, int64_t g, int64_t M,
                  const int8_t *A5, const uint16_t *sA,
                  const int8_t *B8, const uint16_t *sB,
                  const uint8_t *R4, const uint16_t *sR,
                  const int8_t *C8, const uint16_t *sC,
                  const int8_t *D8, const uint16_t *sD,
                  const uint16_t *X, double *out)
{
    if (g <= 0 || d % g || d % 2)
        return 1;
    int64_t G = d / g;
    for (int64_t i = 0; i < M * V; ++i)
        out[i] = 0.0;
    for (int64_t v = 0; v < V; ++v) {
        for (int64_t j = 0; j < d; ++j) {
            double w = 0.0;
            for (int64_t i = 0; i < k; ++i)
                w += half_to_double(sA[v]) * (double)A5[v * k + i]
                   * half_to_double(sB[i]) * (double)B8[i * d + j];
            w += half_to_double(sR[v * G + j / g]) * (double)r4_value(R4, v, j, d);
            for (int64_t i = 0; i < r; ++i)
                w += half_to_double(sC[v]) * (double)C8[v * r + i]
                   * half_to_double(sD[i * G + j / g]) * (double)D8[i * d + j];
            for (int64_t m = 0; m < M; ++m)
                out[m * V + v] += bf16_to_double(X[m * d + j]) * w;
        }
    }
    return 0;
}
