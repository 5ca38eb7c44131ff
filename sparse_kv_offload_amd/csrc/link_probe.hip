// Host-link read rate as the copy kernels see it: a streaming kernel reads a
// contiguous pinned, device-mapped host buffer with 16-byte loads (the same
// kind of access the miss copy makes, without its scatter), timed with HIP
// events.  It is the reference for the miss copy's link rate beside the
// bulk hipMemcpy rate (the copy engines), which kernels cannot reach.
#include <cstdio>
#include <cstring>

#include "sko.h"
#include "sko_internal.h"

namespace sko {
namespace {

// Every thread reads its 16-byte chunks i, i + stride, ... with four loads
// in flight; the values only feed a store that never happens for a zeroed
// buffer (the compiler cannot know), so every load is kept.
__global__ __launch_bounds__(256) void k_link_read(const uint4* __restrict__ src, int64_t n16,
                                                   uint32_t* __restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0u;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^ (d.x ^ d.y ^ d.z ^ d.w);
    }
    for (; i < n16; i += stride) {
        const uint4 a = src[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

int fail(int code, const char* what, hipError_t e) {
    char buf[256];
    snprintf(buf, sizeof buf, "sko_link_read_rate: %s%s%s", what, e != hipSuccess ? ": " : "",
             e != hipSuccess ? hipGetErrorString(e) : "");
    return set_error(code, buf);
}

}  // namespace
}  // namespace sko

extern "C" int sko_link_read_rate(int32_t device, int64_t bytes, int32_t reps, float* gbps) {
    using namespace sko;
    if (!gbps) return fail(SKO_E_INVAL, "NULL result pointer", hipSuccess);
    *gbps = 0.0f;
    if (device < 0 || bytes < (1 << 20) || bytes % 16 != 0 || reps < 1)
        return fail(SKO_E_INVAL, "needs device >= 0, bytes >= 1 MiB and a multiple of 16, reps >= 1", hipSuccess);
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    hipError_t e = hipSetDevice(device);
    if (e != hipSuccess) return fail(SKO_E_DEVICE, "hipSetDevice", e);
    void* host = nullptr;
    void* dev_view = nullptr;
    uint32_t* sink = nullptr;
    hipStream_t st = nullptr;
    hipEvent_t a = nullptr, b = nullptr;
    int rc = SKO_OK;
    float best_ms = 0.0f;
    if (hipHostMalloc(&host, (size_t)bytes, hipHostMallocMapped) != hipSuccess) {
        (void)hipGetLastError();
        host = nullptr;
        rc = fail(SKO_E_NOMEM, "pinned host buffer", hipSuccess);
    }
    if (rc == SKO_OK) {
        memset(host, 0, (size_t)bytes);
        e = hipHostGetDevicePointer(&dev_view, host, 0);
        if (e == hipSuccess) e = hipMalloc((void**)&sink, 4);
        if (e == hipSuccess) e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
        if (e == hipSuccess) e = hipEventCreate(&a);
        if (e == hipSuccess) e = hipEventCreate(&b);
        if (e != hipSuccess) rc = fail(SKO_E_DEVICE, "set-up", e);
    }
    // a few grid sizes (host reads in flight), best over the timed launches
    const int grids[] = {32, 64, 128, 256};
    for (int gi = 0; rc == SKO_OK && gi < 4; ++gi) {
        const dim3 grid(grids[gi]);
        for (int r = 0; rc == SKO_OK && r <= reps; ++r) {  // launch 0 warms up
            e = hipEventRecord(a, st);
            hipLaunchKernelGGL(k_link_read, grid, dim3(256), 0, st, static_cast<const uint4*>(dev_view), bytes / 16,
                               sink);
            if (e == hipSuccess) e = hipGetLastError();
            if (e == hipSuccess) e = hipEventRecord(b, st);
            if (e == hipSuccess) e = hipEventSynchronize(b);
            float ms = 0.0f;
            if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
            if (e != hipSuccess) rc = fail(SKO_E_DEVICE, "timed read", e);
            else if (r > 0 && ms > 0.0f && (best_ms == 0.0f || ms < best_ms)) best_ms = ms;
        }
    }
    if (st) (void)hipStreamSynchronize(st);
    if (a) (void)hipEventDestroy(a);
    if (b) (void)hipEventDestroy(b);
    if (st) (void)hipStreamDestroy(st);
    if (sink) (void)hipFree(sink);
    if (host) (void)hipHostFree(host);
    if (prev >= 0) (void)hipSetDevice(prev);
    if (rc == SKO_OK) *gbps = best_ms > 0.0f ? (float)((double)bytes / (best_ms * 1e-3) / 1e9) : 0.0f;
    return rc;
}
