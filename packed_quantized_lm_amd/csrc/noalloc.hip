// noalloc.hip -- archead_forward_argmax_noalloc: the forward with its top-1
// index, for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The kernels' workspace (projection outputs, argmax partial keys, work
// counters) lives in one file-scope device array of kScratchBytes per GPU,
// held until the process ends.  Host code never passes the array's name to a
// kernel: on first use on a device, with that device current, its address is
// looked up with hipGetSymbolAddress and kept per device.  Every call on a
// device shares that device's array, so calls that overlap on one GPU race;
// each call first clears the parts that must start at zero.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "api_internal.hpp"
#include "archead.h"
#include "layout.hpp"

namespace archead {
namespace {

constexpr size_t kScratchBytes = size_t(8) << 20;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::vector<void *> g_scratch_ptr; // per device id; null until looked up

// device address of this device's scratch array (the device is current)
archead_status scratch_address(int device, void **out)
{
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if ((int)g_scratch_ptr.size() <= device)
        g_scratch_ptr.resize(device + 1, nullptr);
    if (!g_scratch_ptr[device]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return api_fail(ARCHEAD_EHIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
        g_scratch_ptr[device] = p;
    }
    *out = g_scratch_ptr[device];
    return ARCHEAD_OK;
}

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// zero [0, n0) and [off1, off1 + n1) bytes of ws, 16 bytes per thread per
// step (every bound is a multiple of 16)
__global__ __launch_bounds__(256) void clear_kernel(char *ws, size_t n0, size_t off1, size_t n1)
{
    const u32x4 z = {0u, 0u, 0u, 0u};
    const size_t q0 = n0 / 16, q1 = n1 / 16;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < q0 + q1; i += (size_t)gridDim.x * 256) {
        const size_t off = i < q0 ? 16 * i : off1 + 16 * (i - q0);
        *(u32x4 *)(ws + off) = z;
    }
}

} // namespace
} // namespace archead

using namespace archead;

extern "C" archead_status archead_forward_argmax_noalloc(archead_t h, int64_t M, const void *X, float *logits,
                                                         int32_t *argmax, void *hip_stream)
{
    int device = 0;
    archead_status st = handle_device(h, &device);
    if (st != ARCHEAD_OK)
        return st;
    if (M < 0)
        return api_fail(ARCHEAD_EINVAL, "M < 0");
    if (M == 0)
        return ARCHEAD_OK;
    if (!argmax)
        return api_fail(ARCHEAD_EINVAL, "argmax is NULL");
    if (!X || ((uintptr_t)X) % 16)
        return api_fail(ARCHEAD_EINVAL, "X must be a 16-byte aligned device pointer");
    size_t zero_head = 0, zero_tail = 0;
    const size_t need = workspace_bytes(h, M, &zero_head, &zero_tail);
    if (need > kScratchBytes)
        return api_fail(ARCHEAD_ESHAPE, "M = " + std::to_string(M) + " needs a " + std::to_string(need) +
                                            "-byte workspace; the no-allocation forward holds at most " +
                                            std::to_string(kScratchBytes) + " bytes");
    hipError_t e = hipSetDevice(device);
    if (e != hipSuccess)
        return api_fail(ARCHEAD_EHIP, std::string("hipSetDevice: ") + hipGetErrorString(e));
    void *ws = nullptr;
    st = scratch_address(device, &ws);
    if (st != ARCHEAD_OK)
        return st;
    hipStream_t stream = (hipStream_t)hip_stream;
    const size_t n1 = need - zero_tail;
    const unsigned blocks = (unsigned)std::min<size_t>(64, (zero_head + n1) / (16 * 256) + 1);
    hipLaunchKernelGGL(clear_kernel, dim3(blocks), dim3(256), 0, stream, (char *)ws, zero_head, zero_tail, n1);
    e = hipGetLastError();
    if (e != hipSuccess)
        return api_fail(ARCHEAD_EHIP, std::string("clear_kernel: ") + hipGetErrorString(e));
    return forward_in_workspace(h, M, X, logits, argmax, hip_stream, ws, M);
}
