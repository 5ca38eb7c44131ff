// Miss-only host -> device row copy.
//
// [LSO] section 4 "Decode step": only the miss rows are copied from host
// memory to the device, so transfer volume follows the top-k misses, not
// the sequence length ("Top-k miss rows" row of the transfer-granularity
// table).  The pool is pinned, device-mapped host memory; this kernel reads
// it directly over the host link (zero-copy) and writes the 1152-byte rows
// into their victim slots of the hot buffer.  The work list (source row,
// destination row) for all sequences of the layer comes from the LRU kernel,
// whose device-side counter gives the total, so no host sync is needed.
#include "sko_common.cuh"
#include "sko_internal.h"

namespace sko {

constexpr int kGatherUnroll = 4;
constexpr int kGatherThreads = 256;

// Sequence b's entries are glist[b * mstride + r] for r < counts[b][2].
// Each block first builds the prefix of the per-sequence miss counts in LDS;
// a flat 16-byte chunk index c then maps to entry e = c / 72 and, by binary
// search in the prefix, to (sequence, r).
__device__ __forceinline__ int find_seq(const int* pre, int B, int64_t e) {
    int lo = 0, hi = B;  // pre[lo] <= e < pre[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pre[mid] <= e) lo = mid; else hi = mid;
    }
    return lo;
}

__global__ __launch_bounds__(kGatherThreads) void k_gather_misses(const GatherEntry* __restrict__ glist,
                                                                  const int32_t* __restrict__ counts,
                                                                  const uint4* __restrict__ pool_layer,
                                                                  uint4* __restrict__ hot_layer, int B,
                                                                  int mstride) {
    extern __shared__ int pre[];  // B + 1
    __shared__ int scratch[kGatherThreads / 64 + 1];
    const int per = (B + kGatherThreads - 1) / kGatherThreads;
    const int b0 = threadIdx.x * per;
    int loc = 0;
    for (int b = b0; b < b0 + per && b < B; ++b) loc += std::min(std::max(counts[(size_t)b * 8 + 2], 0), mstride);
    int total;
    int run = block_exclusive_scan<kGatherThreads>(loc, &total, scratch);
    for (int b = b0; b < b0 + per && b < B; ++b) {
        pre[b] = run;
        run += std::min(std::max(counts[(size_t)b * 8 + 2], 0), mstride);
    }
    if (threadIdx.x == 0) pre[B] = total;
    __syncthreads();

    const int64_t chunks = (int64_t)total * kKvRowU4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    // several 16-byte host reads in flight per thread before the stores
    for (; c + (kGatherUnroll - 1) * stride < chunks; c += kGatherUnroll * stride) {
        uint4 v[kGatherUnroll];
        int64_t dst[kGatherUnroll];
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u) {
            const int64_t cc = c + u * stride;
            const int64_t e = cc / kKvRowU4;
            const int part = (int)(cc - e * kKvRowU4);
            const int b = find_seq(pre, B, e);
            const GatherEntry g = glist[(size_t)b * mstride + (e - pre[b])];
            v[u] = pool_layer[(int64_t)g.src_row * kKvRowU4 + part];
            dst[u] = (int64_t)g.dst_row * kKvRowU4 + part;
        }
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u) hot_layer[dst[u]] = v[u];
    }
    for (; c < chunks; c += stride) {
        const int64_t e = c / kKvRowU4;
        const int part = (int)(c - e * kKvRowU4);
        const int b = find_seq(pre, B, e);
        const GatherEntry g = glist[(size_t)b * mstride + (e - pre[b])];
        hot_layer[(int64_t)g.dst_row * kKvRowU4 + part] = pool_layer[(int64_t)g.src_row * kKvRowU4 + part];
    }
}

hipError_t launch_gather_misses(hipStream_t st, const GatherEntry* glist, const int32_t* counts,
                                const uint16_t* pool_layer, uint16_t* hot_layer, int B, int mstride,
                                int max_entries) {
    const int64_t max_chunks = (int64_t)max_entries * kKvRowU4;
    int grid = (int)std::min<int64_t>((max_chunks + kGatherThreads * kGatherUnroll - 1) /
                                          (kGatherThreads * kGatherUnroll), 2048);
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(k_gather_misses, dim3(grid), dim3(kGatherThreads), (size_t)(B + 1) * sizeof(int), st,
                       glist, counts, reinterpret_cast<const uint4*>(pool_layer),
                       reinterpret_cast<uint4*>(hot_layer), B, mstride);
    return hipGetLastError();
}

}  // namespace sko
