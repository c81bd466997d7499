// build.hip -- construction of a packed ARCHead head on the GPU.
//
// ARCHead paper, section 3.4 (the construction algorithm; its listing is cut
// off after the inputs W, H, r_c, r_r, g, p, lambda in the extracted text),
// read through equations 2-5 and the INT8 text after eq 7:
//   1. damped metric (eq 2): C = H^T H / N, C_lambda = C + lambda mean(diag C) I,
//      T_p = C_lambda^p and its inverse;
//   2. rank-k core of W (text under eq 3): A_c = U_k S_k^(1/2),
//      B_c = S_k^(1/2) V_k^T;
//   3. eq 3: A5 = Q5(A_c) and B8 = Q8(B_c) with row scales, R4 = SC4 of
//      W - A_c B_c (the unquantised core) with (row, g-group) scales;
//   4. E = W - W_d, W_d = (sA o A5)(sB o B8) + sR o R4;
//   5. eqs 4-5: randomized rank-r SVD of E T_p = U S V^T,
//      A_w = U_r S_r, B_w = V_r^T T_p^-1;
//   6. C8 = Q8(A_w) with row scales, D8 = Q8(B_w) with (row, g-group) scales.
// Both SVDs are randomized (Gaussian test matrix, power iterations,
// oversampling), as the paper computes the correction's.  Every product is
// an fp64 GEMM on the matrix cores (v_mfma_f64_16x16x4_f64).  T_p for the
// dyadic powers p in {1/4, 1/2, 3/4, 1} comes from coupled Newton-Schulz
// iterations (GEMMs only); the small symmetric eigenproblems of the SVDs
// and of the orthonormalisations run as a parallel cyclic Jacobi method in
// one workgroup.  The quantisers take every rounding decision in fp64, as
// the symmetric quantiser reading of eq 3 states it: s = fp16(absmax / qmax)
// rounded to nearest even directly from fp64, q = rint(x / s) clamped.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <functional>
#include <utility>
#include <cmath>
#include <string>
#include <vector>

#include "archead.h"
#include "api_internal.hpp"
#include "device.hpp"

namespace archead {
namespace {

typedef __attribute__((ext_vector_type(4))) double f64x4;

// ---------------------------------------------------------------------------
// fp64 GEMM: C[m, n] = alpha sum_k A(m, k) B(k, n) + beta C[m, n], with
// A(m, k) = A[m lda + k] (or A[k lda + m] when ta), B(k, n) = B[k ldb + n]
// (or B[n ldb + k] when tb).  Workgroup tile 64 x 64, each wave 32 x 32 as
// 2 x 2 MFMA tiles of 16 x 16, K in steps of 4.  v_mfma_f64_16x16x4_f64:
// lane l holds A[l % 16][l / 16] and B[l / 16][l % 16]; its four results are
// D[l / 16 + 4 i][l % 16] (rows interleaved by four, unlike the fp32 forms'
// blocks of four consecutive rows).  Operands outside the matrices read as zero.
// ---------------------------------------------------------------------------
struct GemmArgs {
    const double *A, *B;
    double *C;
    int64_t M, N, K, lda, ldb, ldc;
    int ta, tb;
    double alpha, beta;
};

__global__ __launch_bounds__(256) void gemm_f64_kernel(GemmArgs g)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int li = lane & 15, lk = lane >> 4;
    const int64_t m0 = (int64_t)blockIdx.y * 64 + (wv >> 1) * 32;
    const int64_t n0 = (int64_t)blockIdx.x * 64 + (wv & 1) * 32;
    f64x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};
    for (int64_t k0 = 0; k0 < g.K; k0 += 4) {
        const int64_t k = k0 + lk;
        double av[2], bv[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int64_t m = m0 + 16 * i + li;
            const bool ok = m < g.M && k < g.K;
            const int64_t mc = ok ? m : 0, kc = ok ? k : 0;
            const double x = g.A[g.ta ? kc * g.lda + mc : mc * g.lda + kc];
            av[i] = ok ? x : 0.0;
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t n = n0 + 16 * j + li;
            const bool ok = n < g.N && k < g.K;
            const int64_t nc = ok ? n : 0, kc = ok ? k : 0;
            const double x = g.B[g.tb ? nc * g.ldb + kc : kc * g.ldb + nc];
            bv[j] = ok ? x : 0.0;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t m = m0 + 16 * i + lk + 4 * r, n = n0 + 16 * j + li;
                if (m < g.M && n < g.N) {
                    double *c = g.C + m * g.ldc + n;
                    *c = g.beta != 0.0 ? g.alpha * acc[i][j][r] + g.beta * *c : g.alpha * acc[i][j][r];
                }
            }
}

// ---------------------------------------------------------------------------
// small elementwise and reduction kernels
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void axpby_kernel(double *y, const double *x, int64_t n, double a, double b)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        y[i] = a * x[i] + b * y[i];
}

// A[i][i] += v for i < n (row pitch lda)
__global__ __launch_bounds__(256) void add_diag_kernel(double *A, int64_t n, int64_t lda, double v)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        A[i * lda + i] += v;
}

// out[0] = sum of x[i * stride] for i < n (one workgroup)
__global__ __launch_bounds__(256) void sum_kernel(const double *x, int64_t n, int64_t stride, int square,
                                                  double *out)
{
    __shared__ double red[256];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += 256) {
        const double v = x[i * stride];
        s += square ? v * v : v;
    }
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w)
            red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0)
        out[0] = red[0];
}

// columns scaled: Y[i][j] *= s[j] (rows x cols, pitch ld)
__global__ __launch_bounds__(256) void scale_cols_kernel(double *Y, int64_t rows, int64_t cols, int64_t ld,
                                                         const double *s)
{
    const int64_t n = rows * cols;
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < n; t += (int64_t)gridDim.x * 256) {
        const int64_t i = t / cols, j = t - (t / cols) * cols;
        Y[i * ld + j] *= s[j];
    }
}

// out (cols x rows) = in^T (in: rows x cols)
__global__ __launch_bounds__(256) void transpose_kernel(const double *in, int64_t rows, int64_t cols, double *out)
{
    const int64_t n = rows * cols;
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < n; t += (int64_t)gridDim.x * 256) {
        const int64_t i = t / cols, j = t - (t / cols) * cols;
        out[j * rows + i] = in[t];
    }
}

// rows scaled: Y[i][j] *= s[i]
__global__ __launch_bounds__(256) void scale_rows_kernel(double *Y, int64_t rows, int64_t cols, int64_t ld,
                                                         const double *s)
{
    const int64_t n = rows * cols;
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < n; t += (int64_t)gridDim.x * 256) {
        const int64_t i = t / cols, j = t - (t / cols) * cols;
        Y[i * ld + j] *= s[i];
    }
}

// ---------------------------------------------------------------------------
// Gaussian test matrix: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC 2011)
// counter (index, 0, 0, 0) under key (seed lo, seed hi), two of its four
// words into a Box-Muller pair, one normal deviate per element.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void philox_round(uint32_t (&c)[4], const uint32_t (&k)[2])
{
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0], p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0, hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    c[0] = hi1 ^ c[1] ^ k[0];
    c[1] = lo1;
    c[2] = hi0 ^ c[3] ^ k[1];
    c[3] = lo0;
}

__global__ __launch_bounds__(256) void gaussian_kernel(double *out, int64_t n, uint64_t seed)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        uint32_t c[4] = {(uint32_t)i, (uint32_t)((uint64_t)i >> 32), 0u, 0u};
        uint32_t k[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
        for (int r = 0; r < 10; ++r) {
            philox_round(c, k);
            k[0] += 0x9E3779B9u;
            k[1] += 0xBB67AE85u;
        }
        const double u1 = ((double)c[0] + 0.5) * 0x1p-32, u2 = ((double)c[1] + 0.5) * 0x1p-32;
        out[i] = sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
    }
}

// ---------------------------------------------------------------------------
// Symmetric eigenproblem of a small n x n matrix (n <= kJacMax) in one
// workgroup: parallel cyclic Jacobi.  Each round pairs the indices by the
// round-robin schedule (index n - 1 fixed, the others rotating; an odd n gets
// a dummy partner), computes every pair's rotation from the same matrix
// (Golub and Van Loan's symmetric Schur decomposition of the 2 x 2 block),
// then applies all row rotations, then all column rotations (pairs are
// disjoint, so each step is parallel), and the column rotations to the
// eigenvector matrix.  Sweeps stop when the off-diagonal norm is below
// 1e-14 of the matrix norm.  Results: evals (descending) and the matching
// eigenvectors as the columns of Vout (n x n, pitch n).  A is destroyed.
// ---------------------------------------------------------------------------
constexpr int kJacMax = 1024;

__global__ __launch_bounds__(256) void jacobi_kernel(double *A, double *Vw, int n, int max_sweeps, double *evals,
                                                     double *Vout)
{
    __shared__ int s_p[kJacMax / 2], s_q[kJacMax / 2];
    __shared__ double s_c[kJacMax / 2], s_s[kJacMax / 2];
    __shared__ double red[256];
    __shared__ int s_done;
    const int t = threadIdx.x;
    const int ne = n + (n & 1); // players, with a dummy when n is odd
    const int np = ne / 2;
    for (int64_t i = t; i < (int64_t)n * n; i += 256)
        Vw[i] = (i / n == i % n) ? 1.0 : 0.0;
    __syncthreads();
    for (int sweep = 0; sweep < max_sweeps; ++sweep) {
        // convergence: off-diagonal and total Frobenius norms
        double off = 0.0, tot = 0.0;
        for (int64_t i = t; i < (int64_t)n * n; i += 256) {
            const double v = A[i];
            tot += v * v;
            off += (i / n != i % n) ? v * v : 0.0;
        }
        red[t] = off;
        __syncthreads();
        for (int w = 128; w > 0; w >>= 1) {
            if (t < w)
                red[t] += red[t + w];
            __syncthreads();
        }
        const double off_all = red[0];
        __syncthreads();
        red[t] = tot;
        __syncthreads();
        for (int w = 128; w > 0; w >>= 1) {
            if (t < w)
                red[t] += red[t + w];
            __syncthreads();
        }
        if (t == 0)
            s_done = off_all <= 1e-28 * red[0] ? 1 : 0;
        __syncthreads();
        if (s_done)
            break;
        for (int round = 0; round < ne - 1; ++round) {
            // pair i: positions i and ne - 1 - i of the rotated schedule
            for (int i = t; i < np; i += 256) {
                auto player = [&](int pos) { return pos == ne - 1 ? ne - 1 : (pos + round) % (ne - 1); };
                int p = player(i), q = player(ne - 1 - i);
                if (p > q) {
                    const int x = p;
                    p = q;
                    q = x;
                }
                double c = 1.0, s = 0.0;
                if (q < n) {
                    const double apq = A[(int64_t)p * n + q];
                    if (apq != 0.0) {
                        const double tau = (A[(int64_t)q * n + q] - A[(int64_t)p * n + p]) / (2.0 * apq);
                        const double tt = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
                        c = 1.0 / sqrt(1.0 + tt * tt);
                        s = tt * c;
                    }
                }
                s_p[i] = p;
                s_q[i] = q;
                s_c[i] = c;
                s_s[i] = s;
            }
            __syncthreads();
            // rows p, q of A
            for (int64_t w = t; w < (int64_t)np * n; w += 256) {
                const int i = (int)(w / n), j = (int)(w - (w / n) * n);
                const int p = s_p[i], q = s_q[i];
                if (q < n && s_s[i] != 0.0) {
                    const double c = s_c[i], s = s_s[i];
                    const double ap = A[(int64_t)p * n + j], aq = A[(int64_t)q * n + j];
                    A[(int64_t)p * n + j] = c * ap - s * aq;
                    A[(int64_t)q * n + j] = s * ap + c * aq;
                }
            }
            __threadfence_block();
            __syncthreads();
            // columns p, q of A and of the eigenvectors
            for (int64_t w = t; w < (int64_t)np * n; w += 256) {
                const int i = (int)(w / n), r = (int)(w - (w / n) * n);
                const int p = s_p[i], q = s_q[i];
                if (q < n && s_s[i] != 0.0) {
                    const double c = s_c[i], s = s_s[i];
                    const double ap = A[(int64_t)r * n + p], aq = A[(int64_t)r * n + q];
                    A[(int64_t)r * n + p] = c * ap - s * aq;
                    A[(int64_t)r * n + q] = s * ap + c * aq;
                    const double vp = Vw[(int64_t)r * n + p], vq = Vw[(int64_t)r * n + q];
                    Vw[(int64_t)r * n + p] = c * vp - s * vq;
                    Vw[(int64_t)r * n + q] = s * vp + c * vq;
                }
            }
            __threadfence_block();
            __syncthreads();
        }
    }
    // descending order: the rank of eigenvalue i (ties by lower index first)
    for (int i = t; i < n; i += 256) {
        const double li = A[(int64_t)i * n + i];
        int rank = 0;
        for (int j = 0; j < n; ++j) {
            const double lj = A[(int64_t)j * n + j];
            rank += (lj > li || (lj == li && j < i)) ? 1 : 0;
        }
        evals[rank] = li;
        for (int r = 0; r < n; ++r)
            Vout[(int64_t)r * n + rank] = Vw[(int64_t)r * n + i];
    }
}

// ---------------------------------------------------------------------------
// quantisers (eq 3's Q_b and the INT8 factors after eq 7), every decision in fp64
// ---------------------------------------------------------------------------
// fp64 -> fp16 bit pattern, round to nearest even, directly (no fp32 step)
__device__ uint16_t f64_to_f16_rne(double x)
{
    const uint16_t sign = x < 0.0 ? 0x8000u : 0u;
    const double a = fabs(x);
    if (!(a == a))
        return 0x7E00u;
    if (a >= 65520.0) // at or past the midpoint above the largest finite half
        return sign | 0x7C00u;
    if (a < 0x1p-14) { // subnormal (or zero): a multiple of 2^-24, rounded
        const double q = rint(a * 0x1p24);
        return sign | (uint16_t)q; // q = 1024 is the smallest normal, encoded alike
    }
    const int e = ilogb(a);                  // a in [2^e, 2^(e+1)), -14 <= e <= 15
    double mq = rint(ldexp(a, 10 - e));      // in [1024, 2048]
    int ee = e;
    if (mq == 2048.0) {
        mq = 1024.0;
        ++ee;
    }
    if (ee > 15)
        return sign | 0x7C00u;
    return sign | (uint16_t)((ee + 15) << 10) | (uint16_t)((int)mq - 1024);
}

__device__ __forceinline__ double f16_bits_to_f64(uint16_t h) { return (double)__builtin_bit_cast(_Float16, h); }

struct QuantArgs {
    const double *x;  // rows x cols, pitch ld
    int64_t rows, cols, ld, group; // group: columns per scale (cols for row-wise)
    int bits;
    int8_t *q;        // rows x cols codes
    uint16_t *s;      // rows x (cols / group) fp16 scales
    double *deq;      // optional rows x cols: s q in fp64
};

// one thread per (row, group), grid-stride
__global__ __launch_bounds__(256) void quantize_kernel(QuantArgs a)
{
    const int64_t G = a.cols / a.group;
    const int qmax = (1 << (a.bits - 1)) - 1, qmin = -(1 << (a.bits - 1));
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < a.rows * G; t += (int64_t)gridDim.x * 256) {
        const int64_t row = t / G, grp = t - (t / G) * G;
        const double *x = a.x + row * a.ld + grp * a.group;
        double amax = 0.0;
        for (int64_t j = 0; j < a.group; ++j)
            amax = fmax(amax, fabs(x[j]));
        const uint16_t sb = f64_to_f16_rne(amax / (double)qmax);
        const double s = f16_bits_to_f64(sb);
        a.s[t] = sb;
        for (int64_t j = 0; j < a.group; ++j) {
            double q = 0.0;
            if (s > 0.0) {
                q = rint(x[j] / s);
                q = q < (double)qmin ? (double)qmin : (q > (double)qmax ? (double)qmax : q);
            }
            a.q[row * a.cols + grp * a.group + j] = (int8_t)q;
            if (a.deq)
                a.deq[row * a.cols + grp * a.group + j] = s * q;
        }
    }
}

// R4 codes (rows x d, int8 in [-8, 7]) -> canonical nibble bytes (rows x d/2):
// column 2c in the low nibble, 2c + 1 in the high one, two's complement
__global__ __launch_bounds__(256) void pack_r4_kernel(const int8_t *q, int64_t n_bytes, uint8_t *out)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n_bytes; i += (int64_t)gridDim.x * 256)
        out[i] = (uint8_t)(((uint8_t)q[2 * i] & 0xF) | (((uint8_t)q[2 * i + 1] & 0xF) << 4));
}

unsigned grid_for(int64_t n) { return (unsigned)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 4096)); }

#define BUILD_TRY(expr)                                                                        \
    do {                                                                                       \
        hipError_t e_ = (expr);                                                                \
        if (e_ != hipSuccess)                                                                  \
            throw std::string(#expr) + ": " + hipGetErrorString(e_);                           \
    } while (0)

// a device allocation of the construction that failed (or was refused by
// the ARCHEAD_TEST_ALLOC_LIMIT test hook)
struct BuildOom {
    size_t bytes;
};

// ---------------------------------------------------------------------------
// host orchestration (device memory from one arena the call allocates)
// ---------------------------------------------------------------------------
struct Builder {
    hipStream_t st;
    std::vector<void *> bufs;
    ~Builder()
    {
        for (void *p : bufs)
            (void)hipFree(p);
    }
    double *alloc(int64_t n)
    {
        const size_t bytes = (size_t)std::max<int64_t>(n, 1) * sizeof(double);
        void *p = nullptr;
        if (alloc_refused(bytes) || hipMalloc(&p, bytes) != hipSuccess)
            throw BuildOom{bytes};
        bufs.push_back(p);
        return (double *)p;
    }
    // C = alpha op(A) op(B) + beta C (row-major; op(X) is X^T when t)
    void gemm(int64_t M, int64_t N, int64_t K, double alpha, const double *A, int64_t lda, bool ta,
              const double *B, int64_t ldb, bool tb, double beta, double *C, int64_t ldc)
    {
        if (M == 0 || N == 0)
            return;
        GemmArgs g{A, B, C, M, N, K, lda, ldb, ldc, ta ? 1 : 0, tb ? 1 : 0, alpha, beta};
        hipLaunchKernelGGL(gemm_f64_kernel, dim3((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64)), dim3(256),
                           0, st, g);
        BUILD_TRY(hipGetLastError());
    }
    double scalar(const double *x, int64_t n, int64_t stride, bool square)
    {
        double *d = alloc(1);
        hipLaunchKernelGGL(sum_kernel, dim3(1), dim3(256), 0, st, x, n, stride, square ? 1 : 0, d);
        BUILD_TRY(hipGetLastError());
        double h = 0.0;
        BUILD_TRY(hipMemcpyAsync(&h, d, sizeof(double), hipMemcpyDeviceToHost, st));
        BUILD_TRY(hipStreamSynchronize(st));
        return h;
    }
    void axpby(double *y, const double *x, int64_t n, double a, double b)
    {
        hipLaunchKernelGGL(axpby_kernel, dim3(grid_for(n)), dim3(256), 0, st, y, x, n, a, b);
        BUILD_TRY(hipGetLastError());
    }
    void add_diag(double *A, int64_t n, double v)
    {
        hipLaunchKernelGGL(add_diag_kernel, dim3(grid_for(n)), dim3(256), 0, st, A, n, n, v);
        BUILD_TRY(hipGetLastError());
    }
    void identity(double *A, int64_t n)
    {
        BUILD_TRY(hipMemsetAsync(A, 0, (size_t)n * n * sizeof(double), st));
        add_diag(A, n, 1.0);
    }
    // eigenvalues (descending) and eigenvectors (columns of V) of the
    // symmetric n x n matrix S (destroyed)
    void eigh(double *S, int64_t n, double *evals, double *V)
    {
        if (n > kJacMax)
            throw std::string("small eigenproblem larger than the Jacobi kernel takes");
        double *work = alloc(n * n);
        hipLaunchKernelGGL(jacobi_kernel, dim3(1), dim3(256), 0, st, S, work, (int)n, 60, evals, V);
        BUILD_TRY(hipGetLastError());
    }
    // coupled Newton-Schulz: Y -> A^(1/2), Z -> A^(-1/2) for a symmetric
    // positive definite A (n x n), iterated on A / c with c = ||A||_F (so
    // that every eigenvalue lies in (0, 1]): T = 3 I - Z Y, Y <- Y T / 2,
    // Z <- T Z / 2, until ||I - Z Y||_F is at round-off
    std::pair<double *, double *> sqrt_pair(const double *A, int64_t n)
    {
        const double c = std::sqrt(scalar(A, n * n, 1, true));
        double *Y = alloc(n * n), *Z = alloc(n * n), *T = alloc(n * n), *Y2 = alloc(n * n), *Z2 = alloc(n * n);
        BUILD_TRY(hipMemcpyAsync(Y, A, (size_t)n * n * sizeof(double), hipMemcpyDeviceToDevice, st));
        axpby(Y, Y, n * n, 0.0, 1.0 / c);
        identity(Z, n);
        bool converged = false;
        for (int it = 0; it < 200 && !converged; ++it) {
            gemm(n, n, n, -1.0, Z, n, false, Y, n, false, 0.0, T, n);
            add_diag(T, n, 3.0);
            gemm(n, n, n, 0.5, Y, n, false, T, n, false, 0.0, Y2, n);
            gemm(n, n, n, 0.5, T, n, false, Z, n, false, 0.0, Z2, n);
            std::swap(Y, Y2);
            std::swap(Z, Z2);
            if (it % 4 == 3) {
                gemm(n, n, n, -1.0, Z, n, false, Y, n, false, 0.0, T, n);
                add_diag(T, n, 1.0);
                converged = std::sqrt(scalar(T, n * n, 1, true)) < 1e-12 * std::sqrt((double)n);
            }
        }
        if (!converged)
            throw std::string("the Newton-Schulz iteration for the metric did not converge");
        axpby(Y, Y, n * n, 0.0, std::sqrt(c));
        axpby(Z, Z, n * n, 0.0, 1.0 / std::sqrt(c));
        return {Y, Z};
    }

    // orthonormal columns of Y (rows x l) in place: G = Y^T Y = V L V^T,
    // Y <- Y V L^(-1/2), twice; directions with L below 1e-24 of the largest
    // are dropped (their columns become zero)
    void orth(double *Y, int64_t rows, int64_t l)
    {
        double *G = alloc(l * l), *V = alloc(l * l), *ev = alloc(l), *Y2 = alloc(rows * l);
        std::vector<double> hs(l);
        for (int pass = 0; pass < 2; ++pass) {
            gemm(l, l, rows, 1.0, Y, l, true, Y, l, false, 0.0, G, l);
            eigh(G, l, ev, V);
            BUILD_TRY(hipMemcpyAsync(hs.data(), ev, l * sizeof(double), hipMemcpyDeviceToHost, st));
            BUILD_TRY(hipStreamSynchronize(st));
            const double top = std::max(hs[0], 0.0);
            for (int64_t j = 0; j < l; ++j)
                hs[j] = hs[j] > 1e-24 * top && hs[j] > 0.0 ? 1.0 / std::sqrt(hs[j]) : 0.0;
            BUILD_TRY(hipMemcpyAsync(ev, hs.data(), l * sizeof(double), hipMemcpyHostToDevice, st));
            gemm(rows, l, l, 1.0, Y, l, false, V, l, false, 0.0, Y2, l);
            hipLaunchKernelGGL(scale_cols_kernel, dim3(grid_for(rows * l)), dim3(256), 0, st, Y2, rows, l, l, ev);
            BUILD_TRY(hipGetLastError());
            BUILD_TRY(hipMemcpyAsync(Y, Y2, (size_t)rows * l * sizeof(double), hipMemcpyDeviceToDevice, st));
        }
        BUILD_TRY(hipStreamSynchronize(st));
    }
};

// A linear operator X (m x n) given by its products with thin matrices:
// XB(B, n x l) -> m x l and XtB(B, m x l) -> n x l.
struct Operator {
    int64_t m, n;
    std::function<void(const double *, int64_t, double *)> XB, XtB;
};

// Randomized SVD of X to rank k (oversampling o, q power iterations):
// U (m x k), S (k), Vt (k x n), singular values descending.
void rsvd(Builder &b, const Operator &X, int64_t k, int64_t o, int q, uint64_t seed, double *U, double *S,
          double *Vt)
{
    const int64_t l = std::min<int64_t>(k + o, std::min(X.m, X.n));
    double *Om = b.alloc(X.n * l), *Y = b.alloc(X.m * l), *Z = b.alloc(X.n * l);
    hipLaunchKernelGGL(gaussian_kernel, dim3(grid_for(X.n * l)), dim3(256), 0, b.st, Om, X.n * l, seed);
    BUILD_TRY(hipGetLastError());
    X.XB(Om, l, Y);
    b.orth(Y, X.m, l);
    for (int it = 0; it < q; ++it) {
        X.XtB(Y, l, Z);
        b.orth(Z, X.n, l);
        X.XB(Z, l, Y);
        b.orth(Y, X.m, l);
    }
    // B = Y^T X (l x n) = (X^T Y)^T;  B B^T = W L W^T;  X ~ (Y W) L^(1/2) (L^(-1/2) W^T B)
    X.XtB(Y, l, Z); // Z = X^T Y (n x l), so B = Z^T
    double *BBt = b.alloc(l * l), *Wv = b.alloc(l * l), *ev = b.alloc(l);
    b.gemm(l, l, X.n, 1.0, Z, l, true, Z, l, false, 0.0, BBt, l);
    b.eigh(BBt, l, ev, Wv);
    std::vector<double> hs(l);
    BUILD_TRY(hipMemcpyAsync(hs.data(), ev, l * sizeof(double), hipMemcpyDeviceToHost, b.st));
    BUILD_TRY(hipStreamSynchronize(b.st));
    std::vector<double> sv(k), inv(k);
    for (int64_t j = 0; j < k; ++j) {
        sv[j] = j < l && hs[j] > 0.0 ? std::sqrt(hs[j]) : 0.0;
        inv[j] = sv[j] > 0.0 ? 1.0 / sv[j] : 0.0;
    }
    BUILD_TRY(hipMemcpyAsync(S, sv.data(), k * sizeof(double), hipMemcpyHostToDevice, b.st));
    double *dinv = b.alloc(k);
    BUILD_TRY(hipMemcpyAsync(dinv, inv.data(), k * sizeof(double), hipMemcpyHostToDevice, b.st));
    // U = Y W[:, :k]   (m x k)
    b.gemm(X.m, k, l, 1.0, Y, l, false, Wv, l, false, 0.0, U, k);
    // Vt = S^-1 W[:, :k]^T B = S^-1 (Z W[:, :k])^T: first T = Z W_k (n x k)
    double *T = b.alloc(X.n * k);
    b.gemm(X.n, k, l, 1.0, Z, l, false, Wv, l, false, 0.0, T, k);
    hipLaunchKernelGGL(scale_cols_kernel, dim3(grid_for(X.n * k)), dim3(256), 0, b.st, T, X.n, k, k, dinv);
    BUILD_TRY(hipGetLastError());
    // Vt = T^T (k x n)
    hipLaunchKernelGGL(transpose_kernel, dim3(grid_for(X.n * k)), dim3(256), 0, b.st, T, X.n, k, Vt);
    BUILD_TRY(hipGetLastError());
    BUILD_TRY(hipStreamSynchronize(b.st));
}

// T_p = C^p and T_p^-1 for the dyadic powers p in {1/4, 1/2, 3/4, 1}
void metric_power(Builder &b, const double *C, int64_t d, double p, double **T, double **Ti)
{
    auto half = b.sqrt_pair(C, d);
    if (p == 0.5) {
        *T = half.first;
        *Ti = half.second;
        return;
    }
    if (p == 1.0) {
        double *t = b.alloc(d * d), *ti = b.alloc(d * d);
        BUILD_TRY(hipMemcpyAsync(t, C, (size_t)d * d * sizeof(double), hipMemcpyDeviceToDevice, b.st));
        b.gemm(d, d, d, 1.0, half.second, d, false, half.second, d, false, 0.0, ti, d);
        *T = t;
        *Ti = ti;
        return;
    }
    auto quarter = b.sqrt_pair(half.first, d);
    if (p == 0.25) {
        *T = quarter.first;
        *Ti = quarter.second;
        return;
    }
    double *t = b.alloc(d * d), *ti = b.alloc(d * d); // p = 3/4: C^(1/2) C^(1/4)
    b.gemm(d, d, d, 1.0, half.first, d, false, quarter.first, d, false, 0.0, t, d);
    b.gemm(d, d, d, 1.0, half.second, d, false, quarter.second, d, false, 0.0, ti, d);
    *T = t;
    *Ti = ti;
}

void quantize(Builder &b, const double *x, int64_t rows, int64_t cols, int64_t ld, int bits, int64_t group,
              int8_t *q, uint16_t *s, double *deq)
{
    if (rows == 0 || cols == 0)
        return;
    QuantArgs a{x, rows, cols, ld, group, bits, q, s, deq};
    hipLaunchKernelGGL(quantize_kernel, dim3(grid_for(rows * (cols / group))), dim3(256), 0, b.st, a);
    BUILD_TRY(hipGetLastError());
}

} // namespace
} // namespace archead

using namespace archead;

namespace {

archead_status build_shape_ok(int64_t V, int64_t d, int64_t k, int64_t r, int64_t g, int64_t N)
{
    if (V < 1 || d < 128 || d % 128 || d > (int64_t(1) << 16) || g < 32 || g % 32 || d % g)
        return api_fail(ARCHEAD_ESHAPE, "construction needs V >= 1, d a multiple of 128 (at most 65536) and g a "
                                        "multiple of 32 dividing d");
    if (k < 0 || r < 0 || k + 16 > kJacMax || r + 16 > kJacMax || k > std::min(V, d) || r > std::min(V, d))
        return api_fail(ARCHEAD_ESHAPE, "construction needs 0 <= k, r <= min(V, d, 1008)");
    if (N < 1)
        return api_fail(ARCHEAD_ESHAPE, "construction needs at least one calibration row");
    return ARCHEAD_OK;
}

} // namespace

extern "C" archead_status archead_quantize(const double *x, int64_t rows, int64_t cols, int bits, int64_t group,
                                           int8_t *q, uint16_t *s, void *hip_stream)
{
    if (!x || !q || !s)
        return api_fail(ARCHEAD_EINVAL, "x, q and s are required");
    if (rows < 0 || cols < 1 || group < 1 || cols % group || bits < 2 || bits > 8)
        return api_fail(ARCHEAD_EINVAL, "rows >= 0, cols >= 1, a group size dividing cols, 2 <= bits <= 8");
    try {
        Builder b;
        b.st = (hipStream_t)hip_stream;
        quantize(b, x, rows, cols, cols, bits, group, q, s, nullptr);
    } catch (const std::string &e) {
        return api_fail(ARCHEAD_EHIP, e);
    } catch (const BuildOom &e) {
        return api_fail(ARCHEAD_ENOMEM, "device allocation of " + std::to_string(e.bytes) + " bytes failed");
    }
    return ARCHEAD_OK;
}

extern "C" archead_status archead_build(int64_t V, int64_t d, int64_t k, int64_t r, int64_t g, int64_t N,
                                        const double *W, const double *H, double p, double lambda,
                                        int power_iters, int oversample, uint64_t seed, int8_t *A5, uint16_t *sA,
                                        int8_t *B8, uint16_t *sB, uint8_t *R4, uint16_t *sR, int8_t *C8,
                                        uint16_t *sC, int8_t *D8, uint16_t *sD, void *hip_stream)
{
    archead_status st = build_shape_ok(V, d, k, r, g, N);
    if (st != ARCHEAD_OK)
        return st;
    if (!W || !H || !R4 || !sR || (k > 0 && (!A5 || !sA || !B8 || !sB)) || (r > 0 && (!C8 || !sC || !D8 || !sD)))
        return api_fail(ARCHEAD_EINVAL, "W, H and the output fields of the present terms are required");
    if (!(p == 0.25 || p == 0.5 || p == 0.75 || p == 1.0))
        return api_fail(ARCHEAD_EINVAL, "p must be one of 1/4, 1/2, 3/4, 1");
    if (!(lambda > 0.0) || !std::isfinite(lambda))
        return api_fail(ARCHEAD_EINVAL, "lambda must be positive and finite");
    if (power_iters < 0 || power_iters > 16 || oversample < 0 || oversample > 64)
        return api_fail(ARCHEAD_EINVAL, "0 <= power_iters <= 16 and 0 <= oversample <= 64");
    if (std::max(k, r) + oversample > kJacMax)
        return api_fail(ARCHEAD_EINVAL, "max(k, r) + oversample must not exceed " + std::to_string(kJacMax) +
                                            " (the sketch's eigenproblem runs in one workgroup)");
    try {
        Builder b;
        b.st = (hipStream_t)hip_stream;
        const int64_t G = d / g;
        // 1. damped metric (eq 2) and its p-th power
        double *C = b.alloc(d * d);
        b.gemm(d, d, N, 1.0 / (double)N, H, d, true, H, d, false, 0.0, C, d);
        const double cbar = b.scalar(C, d, d + 1, false) / (double)d;
        b.add_diag(C, d, lambda * cbar);
        double *T = nullptr, *Ti = nullptr;
        metric_power(b, C, d, p, &T, &Ti);
        // 2-3. core and SC4 residual
        double *R = b.alloc(V * d);
        BUILD_TRY(hipMemcpyAsync(R, W, (size_t)V * d * sizeof(double), hipMemcpyDeviceToDevice, b.st));
        double *E = b.alloc(V * d);
        BUILD_TRY(hipMemcpyAsync(E, W, (size_t)V * d * sizeof(double), hipMemcpyDeviceToDevice, b.st));
        if (k > 0) {
            Operator Wop{V, d,
                         [&](const double *B, int64_t l, double *out) { b.gemm(V, l, d, 1.0, W, d, false, B, l, false, 0.0, out, l); },
                         [&](const double *B, int64_t l, double *out) { b.gemm(d, l, V, 1.0, W, d, true, B, l, false, 0.0, out, l); }};
            double *U = b.alloc(V * k), *S = b.alloc(k), *Vt = b.alloc(k * d);
            rsvd(b, Wop, k, oversample, power_iters, seed, U, S, Vt);
            std::vector<double> hs(k);
            BUILD_TRY(hipMemcpyAsync(hs.data(), S, k * sizeof(double), hipMemcpyDeviceToHost, b.st));
            BUILD_TRY(hipStreamSynchronize(b.st));
            for (auto &x : hs)
                x = std::sqrt(x);
            double *rs = b.alloc(k);
            BUILD_TRY(hipMemcpyAsync(rs, hs.data(), k * sizeof(double), hipMemcpyHostToDevice, b.st));
            // A_c = U S^(1/2) (V x k); B_c = S^(1/2) Vt (k x d)
            hipLaunchKernelGGL(scale_cols_kernel, dim3(grid_for(V * k)), dim3(256), 0, b.st, U, V, k, k, rs);
            BUILD_TRY(hipGetLastError());
            double *Bc = Vt;
            hipLaunchKernelGGL(scale_rows_kernel, dim3(grid_for(k * d)), dim3(256), 0, b.st, Bc, k, d, d, rs);
            BUILD_TRY(hipGetLastError());
            double *dA = b.alloc(V * k), *dB = b.alloc(k * d);
            quantize(b, U, V, k, k, 5, k, A5, sA, dA);
            quantize(b, Bc, k, d, d, 8, d, B8, sB, dB);
            // R = W - A_c B_c (unquantised core, eq 3); E = W - dA dB (the quantised core)
            b.gemm(V, d, k, -1.0, U, k, false, Bc, d, false, 1.0, R, d);
            b.gemm(V, d, k, -1.0, dA, k, false, dB, d, false, 1.0, E, d);
        }
        int8_t *q4 = (int8_t *)b.alloc((V * d + 7) / 8);
        double *dR = b.alloc(V * d);
        quantize(b, R, V, d, d, 4, g, q4, sR, dR);
        hipLaunchKernelGGL(pack_r4_kernel, dim3(grid_for(V * d / 2)), dim3(256), 0, b.st, q4, V * d / 2, R4);
        BUILD_TRY(hipGetLastError());
        b.axpby(E, dR, V * d, -1.0, 1.0); // E = W - W_d
        // 5-6. correction: randomized SVD of E T_p, A_w = U_r S_r, B_w = V_r^T T_p^-1
        if (r > 0) {
            double *tmp_d = b.alloc(d * (r + oversample + 1)), *tmp_v = b.alloc(V * (r + oversample + 1));
            Operator Eop{V, d,
                         [&](const double *B, int64_t l, double *out) { // E (T B)
                             b.gemm(d, l, d, 1.0, T, d, false, B, l, false, 0.0, tmp_d, l);
                             b.gemm(V, l, d, 1.0, E, d, false, tmp_d, l, false, 0.0, out, l);
                         },
                         [&](const double *B, int64_t l, double *out) { // T (E^T B)
                             b.gemm(d, l, V, 1.0, E, d, true, B, l, false, 0.0, tmp_d, l);
                             b.gemm(d, l, d, 1.0, T, d, false, tmp_d, l, false, 0.0, out, l);
                         }};
            (void)tmp_v;
            double *Uw = b.alloc(V * r), *Sw = b.alloc(r), *Vwt = b.alloc(r * d);
            rsvd(b, Eop, r, oversample, power_iters, seed ^ 0x5DEECE66DULL, Uw, Sw, Vwt);
            hipLaunchKernelGGL(scale_cols_kernel, dim3(grid_for(V * r)), dim3(256), 0, b.st, Uw, V, r, r, Sw);
            BUILD_TRY(hipGetLastError());
            double *Bw = b.alloc(r * d);
            b.gemm(r, d, d, 1.0, Vwt, d, false, Ti, d, false, 0.0, Bw, d);
            quantize(b, Uw, V, r, r, 8, r, C8, sC, nullptr);
            quantize(b, Bw, r, d, d, 8, g, D8, sD, nullptr);
        }
        BUILD_TRY(hipStreamSynchronize(b.st));
        (void)G;
    } catch (const std::string &e) {
        return api_fail(ARCHEAD_EHIP, "construction: " + e);
    } catch (const BuildOom &e) {
        return api_fail(ARCHEAD_ENOMEM, "construction: device allocation of " + std::to_string(e.bytes) + " bytes failed");
    }
    return ARCHEAD_OK;
}
