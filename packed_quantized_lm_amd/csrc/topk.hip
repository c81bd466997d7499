// topk.hip -- the K largest logits of each hidden state (K <= kTopKMax), in
// order: larger value first, equal values by lower vocabulary index.
//
// The ARCHead pages measure how often the packed head keeps the dense head's
// top-1 token (section 1 and the results paragraphs); the same selection
// widened to K candidates is what a top-k sampling decode step needs.  It
// runs over the logits the forward has just written, in two levels:
//   1. each wave takes a slice of 1024 logits of one row and selects its K
//      largest keys in K rounds (wave maximum, then the lane that holds it
//      drops it);
//   2. one workgroup per row merges the slices' keys in K rounds: held in
//      registers (up to 4096 keys a row), the winner is dropped each round;
//      otherwise each round takes the largest key below the last one.
// Keys are the argmax keys (orderable value, inverted index), unique within
// a row, so "largest key below the previous" walks the order exactly.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "kernels.hpp"

namespace archead {

constexpr int kTkPer = 16;                // logits per lane in a slice
constexpr int64_t kTkSlice = 64 * kTkPer; // logits per slice (one wave)

int64_t topk_slices(int64_t V) { return (V + kTkSlice - 1) / kTkSlice; }

// the largest of N keys held by one lane, as a tree (short dependency chain)
template <int N>
__device__ __forceinline__ uint64_t lane_max(const uint64_t (&k)[N])
{
    uint64_t t[N];
#pragma unroll
    for (int c = 0; c < N; ++c)
        t[c] = k[c];
#pragma unroll
    for (int w = N / 2; w >= 1; w /= 2)
#pragma unroll
        for (int c = 0; c < w; ++c)
            t[c] = umax64(t[c], t[c + w]);
    return t[0];
}

struct TopkArgs {
    const float *logits; // [M][V]
    int64_t M, V, nslice;
    int K;
    uint64_t *part; // [M][nslice][K] keys, 0 = none
    float *values;  // [M][K]
    int32_t *indices;
    int keys_in_lds;
};

__global__ __launch_bounds__(256) void topk_slice_kernel(TopkArgs a)
{
    const int lane = threadIdx.x & 63;
    const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t m = gw / a.nslice, sl = gw % a.nslice;
    if (m >= a.M)
        return; // the whole wave
    const float *row = a.logits + m * a.V;
    uint64_t key[kTkPer];
    // every load issued before any is used: the index is clamped rather than
    // the load put under a branch (which would wait for each load in turn)
    float y[kTkPer];
#pragma unroll
    for (int c = 0; c < kTkPer; ++c) {
        const int64_t v = sl * kTkSlice + c * 64 + lane;
        y[c] = row[v < a.V ? v : a.V - 1];
    }
#pragma unroll
    for (int c = 0; c < kTkPer; ++c) {
        const int64_t v = sl * kTkSlice + c * 64 + lane;
        key[c] = v < a.V ? argmax_key(y[c], (uint32_t)v) : 0;
    }
    uint64_t mine = 0;
    for (int j = 0; j < a.K; ++j) {
        const uint64_t w = wave_max_u64(lane_max(key));
#pragma unroll
        for (int c = 0; c < kTkPer; ++c)
            key[c] = key[c] == w ? 0 : key[c];
        mine = lane == j ? w : mine;
    }
    if (lane < a.K)
        a.part[(m * a.nslice + sl) * a.K + lane] = mine;
}

constexpr int kTkReg = 16; // keys per thread of the merge when the row's keys fit registers

__global__ __launch_bounds__(256) void topk_merge_kernel(TopkArgs a)
{
    extern __shared__ uint64_t s_keys[]; // the row's keys (large rows only)
    __shared__ uint64_t red[4];
    __shared__ uint64_t s_win[kTopKMax]; // the rounds' winners
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t m = blockIdx.x;
    const int64_t n = a.nslice * a.K;
    const uint64_t *src = a.part + m * n;
    // the largest key of the workgroup; every thread gets it
    auto block_max = [&](uint64_t lm, int j) __attribute__((always_inline)) {
        lm = wave_max_u64(lm);
        if (lane == 0)
            red[wv] = lm;
        __syncthreads();
        const uint64_t w = umax64(umax64(red[0], red[1]), umax64(red[2], red[3]));
        if (threadIdx.x == 0)
            s_win[j] = w;
        __syncthreads(); // every wave has read red before the next round writes it
        return w;
    };
    if (n <= 256 * kTkReg) { // uniform: keys in registers, the winner dropped each round
        uint64_t key[kTkReg];
#pragma unroll
        for (int c = 0; c < kTkReg; ++c) { // clamped loads, all in flight at once
            const int64_t i = threadIdx.x + 256 * c;
            key[c] = src[i < n ? i : n - 1];
        }
#pragma unroll
        for (int c = 0; c < kTkReg; ++c)
            key[c] = threadIdx.x + 256 * c < n ? key[c] : 0;
        for (int j = 0; j < a.K; ++j) {
            const uint64_t w = block_max(lane_max(key), j);
#pragma unroll
            for (int c = 0; c < kTkReg; ++c)
                key[c] = key[c] == w ? 0 : key[c];
        }
    } else { // keys in LDS when they fit, else read again each round
        uint64_t prev = ~(uint64_t)0;
        if (a.keys_in_lds) {
            for (int64_t i = threadIdx.x; i < n; i += 256)
                s_keys[i] = src[i];
            __syncthreads();
            for (int j = 0; j < a.K; ++j) {
                uint64_t lm = 0;
                for (int64_t i = threadIdx.x; i < n; i += 256) {
                    const uint64_t k = s_keys[i];
                    lm = (k < prev && k > lm) ? k : lm;
                }
                prev = block_max(lm, j);
            }
        } else {
            for (int j = 0; j < a.K; ++j) {
                uint64_t lm = 0;
                for (int64_t i = threadIdx.x; i < n; i += 256) {
                    const uint64_t k = src[i];
                    lm = (k < prev && k > lm) ? k : lm;
                }
                prev = block_max(lm, j);
            }
        }
    }
    // the K outputs at once, after the rounds (no memory round trip inside them)
    if (threadIdx.x < a.K) {
        const uint32_t v = 0xFFFFFFFFu - (uint32_t)s_win[threadIdx.x]; // K <= V: a key exists
        a.indices[m * a.K + threadIdx.x] = (int32_t)v;
        a.values[m * a.K + threadIdx.x] = a.logits[m * a.V + v];
    }
}

// Top-k sampling, one thread per row: candidate j weighs
// exp((values[j] - values[0]) / tau) (computed as 2^(x log2 e / tau), x <= 0),
// and the draw is the first j whose running sum exceeds u times the total.
__global__ __launch_bounds__(256) void topk_sample_kernel(const float *values, const int32_t *indices, int64_t M,
                                                          int K, float scale, const float *u, int32_t *out)
{
    const int64_t m = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (m >= M)
        return;
    float v[kTopKMax];
#pragma unroll
    for (int j = 0; j < kTopKMax; ++j) // clamped loads, all in flight at once
        v[j] = values[m * K + (j < K ? j : K - 1)];
    float cum[kTopKMax], c = 0.f;
#pragma unroll
    for (int j = 0; j < kTopKMax; ++j) {
        c += j < K ? __builtin_amdgcn_exp2f((v[j] - v[0]) * scale) : 0.f;
        cum[j] = c;
    }
    const float t = u[m] * c;
    int pick = K - 1;
#pragma unroll
    for (int j = kTopKMax - 1; j >= 0; --j)
        pick = (j < K && cum[j] > t) ? j : pick;
    out[m] = indices[m * K + pick];
}

hipError_t launch_topk_sample(const float *values, const int32_t *indices, int64_t M, int K, float temperature,
                              const float *u, int32_t *samples, hipStream_t st)
{
    if (M == 0)
        return hipSuccess;
    const float scale = 1.44269504088896340736f / temperature;
    hipLaunchKernelGGL(topk_sample_kernel, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, st, values, indices, M,
                       K, scale, u, samples);
    return hipGetLastError();
}

hipError_t launch_topk(const Work &w, const float *logits, int64_t V, int K, float *values,
                       int32_t *indices, hipStream_t st)
{
    if (K < 1 || K > kTopKMax || K > V)
        return hipErrorInvalidValue;
    TopkArgs a;
    a.logits = logits;
    a.M = w.M;
    a.V = V;
    a.nslice = topk_slices(V);
    a.K = K;
    a.part = w.tkp;
    a.values = values;
    a.indices = indices;
    if (w.M * a.nslice * K > w.tkp_cap)
        return hipErrorInvalidValue; // the workspace does not hold this call
    const size_t lds = size_t(a.nslice) * K * 8;
    const bool regs = a.nslice * K <= 256 * kTkReg;
    a.keys_in_lds = !regs && lds <= 48 * 1024 ? 1 : 0;
    const int64_t waves = w.M * a.nslice;
    hipLaunchKernelGGL(topk_slice_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)w.M), dim3(256), a.keys_in_lds ? lds : 0, st, a);
    return hipGetLastError();
}

} // namespace archead
