// Host-link read rate as the copy kernels see it: a streaming kernel reads a
// contiguous pinned, device-mapped host buffer with 16-byte loads (the same
// kind of access the miss copy makes, without its scatter), timed with HIP
// events.  It is the reference for the miss copy's link rate beside the
// bulk hipMemcpy rate (the copy engines), which kernels cannot reach.
// Two device-memory probes sit beside it, the measured ceilings of the two
// HBM-bound kernels: random whole-row gathers as the attention makes them,
// and a plain streaming read as the indexer score pass makes it.
#include <algorithm>
#include <cstdio>
#include <cstring>
#include <vector>

#include "sko.h"
#include "sko_common.h"
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

int fail(int code, const char* what, hipError_t e, const char* fn = "sko_link_read_rate") {
    char buf[256];
    snprintf(buf, sizeof buf, "%s: %s%s%s", fn, what, e != hipSuccess ? ": " : "",
             e != hipSuccess ? hipGetErrorString(e) : "");
    return set_error(code, buf);
}

// Row gather as the attention makes it: block j reads `rows` rows of
// sequence j % nseq (rows of 72 x 16 B, at the slots listed for the block,
// each < slots) one 32-row tile at a time, thread t taking chunks t, t+256,
// ... of the tile, and folds them into one word that feeds a store that
// never happens for a zeroed buffer.
__global__ __launch_bounds__(256) void k_gather_rows(const uint4* __restrict__ rows_base,
                                                     const int32_t* __restrict__ slot_list, int slots, int nseq,
                                                     int rows, uint32_t* __restrict__ sink) {
    const uint4* __restrict__ hb = rows_base + (size_t)(blockIdx.x % nseq) * slots * kKvRowU4;
    const int32_t* __restrict__ sl = slot_list + (size_t)blockIdx.x * rows;
    uint32_t acc = 0u;
    for (int r0 = 0; r0 < rows; r0 += kAttnTileRows) {
        uint4 v[kAttnTileRows * kKvRowU4 / 256];
#pragma unroll
        for (int u = 0; u < kAttnTileRows * kKvRowU4 / 256; ++u) {
            const int idx = threadIdx.x + 256 * u;
            const int rr = idx / kKvRowU4;
            const int row = min(r0 + rr, rows - 1);
            v[u] = hb[(size_t)sl[row] * kKvRowU4 + (idx - rr * kKvRowU4)];
        }
#pragma unroll
        for (int u = 0; u < kAttnTileRows * kKvRowU4 / 256; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

// Streaming read of n 16-byte words: block j reads the contiguous part
// [j n / g, (j + 1) n / g) of the buffer, every thread kStreamUnroll
// nontemporal 16-byte loads at a time (a sweep of block size, blocks per CU
// and loads in flight per thread put this shape at the top).
constexpr int kStreamThreads = 512;
constexpr int kStreamUnroll = 4;
__global__ __launch_bounds__(kStreamThreads) void k_stream_read(const uint4* __restrict__ src, int64_t n,
                                                                uint32_t* __restrict__ sink) {
    const int64_t b0 = (int64_t)blockIdx.x * n / gridDim.x;
    const int64_t b1 = ((int64_t)blockIdx.x + 1) * n / gridDim.x;
    uint32_t acc = 0u;
    int64_t i = b0 + threadIdx.x;
    for (; i + (int64_t)(kStreamUnroll - 1) * kStreamThreads < b1; i += (int64_t)kStreamUnroll * kStreamThreads) {
        uint4 v[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) v[u] = load_nt_u4(src + i + (int64_t)u * kStreamThreads);
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < b1; i += kStreamThreads) {
        const uint4 v = load_nt_u4(src + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace
}  // namespace sko

extern "C" int sko_hbm_read_rate(int32_t device, int64_t bytes, int32_t reps, float* gbps) {
    using namespace sko;
    const char* fn = "sko_hbm_read_rate";
    if (!gbps) return fail(SKO_E_INVAL, "NULL result pointer", hipSuccess, fn);
    *gbps = 0.0f;
    constexpr int kRot = 4;  // buffers in rotation: each launch starts cold in the device-side caches
    if (device < 0 || bytes < (1 << 20) || bytes > ((int64_t)1 << 31) || bytes % 16 != 0 || reps < 1 || reps > 64)
        return fail(SKO_E_INVAL, "needs device >= 0, 1 MiB <= bytes <= 2 GiB and a multiple of 16, 1 <= reps <= 64",
                    hipSuccess, fn);
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    hipError_t e = hipSetDevice(device);
    if (e != hipSuccess) return fail(SKO_E_DEVICE, "hipSetDevice", e, fn);
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus < 1) cus = 256;
    const int64_t n = bytes / 16;
    uint4* buf = nullptr;
    uint32_t* sink = nullptr;
    hipStream_t st = nullptr;
    hipEvent_t a = nullptr, b = nullptr;
    int rc = SKO_OK;
    if (hipMalloc((void**)&buf, (size_t)kRot * bytes) != hipSuccess) {
        (void)hipGetLastError();
        rc = fail(SKO_E_NOMEM, "device buffers", hipSuccess, fn);
    }
    if (rc == SKO_OK) {
        e = hipMemset(buf, 0, (size_t)kRot * bytes);
        if (e == hipSuccess) e = hipMalloc((void**)&sink, 4);
        if (e == hipSuccess) e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
        if (e == hipSuccess) e = hipEventCreate(&a);
        if (e == hipSuccess) e = hipEventCreate(&b);
        if (e != hipSuccess) rc = fail(SKO_E_DEVICE, "set-up", e, fn);
    }
    // one warm-up launch per buffer, then reps * kRot launches, each timed
    // on its own (the median is reported)
    std::vector<float> times;
    for (int w = 0; rc == SKO_OK && w < kRot * (reps + 1); ++w) {
        const uint4* src = buf + (size_t)(w % kRot) * n;
        const bool timed = w >= kRot;
        if (timed) e = hipEventRecord(a, st);
        if (e == hipSuccess) {
            hipLaunchKernelGGL(k_stream_read, dim3(cus), dim3(kStreamThreads), 0, st, src, n, sink);
            e = hipGetLastError();
        }
        if (e == hipSuccess && timed) e = hipEventRecord(b, st);
        if (e == hipSuccess && timed) e = hipEventSynchronize(b);
        float ms = 0.0f;
        if (e == hipSuccess && timed) e = hipEventElapsedTime(&ms, a, b);
        if (e != hipSuccess) rc = fail(SKO_E_DEVICE, "timed read", e, fn);
        else if (timed) times.push_back(ms);
    }
    if (st) (void)hipStreamSynchronize(st);
    if (a) (void)hipEventDestroy(a);
    if (b) (void)hipEventDestroy(b);
    if (st) (void)hipStreamDestroy(st);
    if (sink) (void)hipFree(sink);
    if (buf) (void)hipFree(buf);
    if (prev >= 0) (void)hipSetDevice(prev);
    if (rc == SKO_OK && !times.empty()) {
        std::sort(times.begin(), times.end());
        const float ms = times[times.size() / 2];
        if (ms > 0.0f) *gbps = (float)((double)bytes / (ms * 1e-3) / 1e9);
    }
    return rc;
}

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

extern "C" int sko_hbm_gather_rate(int32_t device, int32_t seqs, int32_t slots, int32_t rows_per_seq,
                                   int32_t reps, float* gbps) {
    using namespace sko;
    const char* fn = "sko_hbm_gather_rate";
    if (!gbps) return fail(SKO_E_INVAL, "NULL result pointer", hipSuccess, fn);
    *gbps = 0.0f;
    constexpr int kRot = 8;        // buffers in rotation: consecutive launches read different memory
    constexpr int kBlockRows = 128;
    if (device < 0 || seqs < 1 || rows_per_seq < kBlockRows || rows_per_seq % kBlockRows != 0 ||
        slots < rows_per_seq || reps < 1 || (int64_t)seqs * slots > (1 << 22) || (int64_t)seqs * rows_per_seq > (1 << 22))
        return fail(SKO_E_INVAL,
                    "needs device >= 0, seqs >= 1, rows_per_seq a positive multiple of 128, slots >= rows_per_seq, "
                    "seqs*slots and seqs*rows_per_seq <= 2^22, reps >= 1",
                    hipSuccess, fn);
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    hipError_t e = hipSetDevice(device);
    if (e != hipSuccess) return fail(SKO_E_DEVICE, "hipSetDevice", e, fn);
    const int blocks = (int)((int64_t)seqs * rows_per_seq / kBlockRows);
    const size_t rot_rows = (size_t)seqs * slots;
    const size_t list_n = (size_t)blocks * kBlockRows;
    uint4* rows_dev = nullptr;
    int32_t* lists = nullptr;
    uint32_t* sink = nullptr;
    hipStream_t st = nullptr;
    hipEvent_t a = nullptr, b = nullptr;
    int rc = SKO_OK;
    if (hipMalloc((void**)&rows_dev, kRot * rot_rows * kKvRowBytes) != hipSuccess ||
        hipMalloc((void**)&lists, kRot * list_n * 4) != hipSuccess) {
        (void)hipGetLastError();
        rc = fail(SKO_E_NOMEM, "device buffers", hipSuccess, fn);
    }
    if (rc == SKO_OK) {
        // per rotation and block: rows distinct slots drawn by a partial
        // Fisher-Yates shuffle (a fixed 64-bit LCG), each < slots
        std::vector<int32_t> h(kRot * list_n);
        std::vector<int32_t> perm(slots);
        uint64_t x = 0x2545F4914F6CDD1DULL;
        for (int r = 0; r < kRot; ++r)
            for (int j = 0; j < blocks; ++j) {
                for (int i = 0; i < slots; ++i) perm[i] = i;
                for (int i = 0; i < kBlockRows; ++i) {
                    x = x * 6364136223846793005ULL + 1442695040888963407ULL;
                    const int k = i + (int)((x >> 33) % (uint64_t)(slots - i));
                    std::swap(perm[i], perm[k]);
                    h[((size_t)r * blocks + j) * kBlockRows + i] = perm[i];
                }
            }
        e = hipMemset(rows_dev, 0, kRot * rot_rows * kKvRowBytes);
        if (e == hipSuccess) e = hipMemcpy(lists, h.data(), h.size() * 4, hipMemcpyHostToDevice);
        if (e == hipSuccess) e = hipMalloc((void**)&sink, 4);
        if (e == hipSuccess) e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
        if (e == hipSuccess) e = hipEventCreate(&a);
        if (e == hipSuccess) e = hipEventCreate(&b);
        if (e != hipSuccess) rc = fail(SKO_E_DEVICE, "set-up", e, fn);
    }
    float ms = 0.0f;
    const int n = reps * kRot;
    for (int w = 0; rc == SKO_OK && w <= n; ++w) {  // launch 0 warms up, then n timed launches
        if (w == 1) e = hipEventRecord(a, st);
        const int r = w % kRot;
        hipLaunchKernelGGL(k_gather_rows, dim3(blocks), dim3(256), 0, st, rows_dev + (size_t)r * rot_rows * kKvRowU4,
                           lists + (size_t)r * list_n, slots, seqs, kBlockRows, sink);
        if (e == hipSuccess) e = hipGetLastError();
        if (e != hipSuccess) rc = fail(SKO_E_DEVICE, "timed gather", e, fn);
    }
    if (rc == SKO_OK) {
        e = hipEventRecord(b, st);
        if (e == hipSuccess) e = hipEventSynchronize(b);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
        if (e != hipSuccess) rc = fail(SKO_E_DEVICE, "timing", e, fn);
    }
    if (st) (void)hipStreamSynchronize(st);
    if (a) (void)hipEventDestroy(a);
    if (b) (void)hipEventDestroy(b);
    if (st) (void)hipStreamDestroy(st);
    if (sink) (void)hipFree(sink);
    if (lists) (void)hipFree(lists);
    if (rows_dev) (void)hipFree(rows_dev);
    if (prev >= 0) (void)hipSetDevice(prev);
    if (rc == SKO_OK && ms > 0.0f)
        *gbps = (float)((double)n * list_n * kKvRowBytes / (ms * 1e-3) / 1e9);
    return rc;
}
