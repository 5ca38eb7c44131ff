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

__global__ __launch_bounds__(256) void k_gather_misses(const GatherEntry* __restrict__ glist,
                                                       const uint32_t* __restrict__ gather_total,
                                                       const uint4* __restrict__ pool_layer,
                                                       uint4* __restrict__ hot_layer,
                                                       uint32_t max_entries) {
    const int64_t chunks = (int64_t)std::min(*gather_total, max_entries) * kKvRowU4;
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
            const GatherEntry g = glist[e];
            v[u] = pool_layer[(int64_t)g.src_row * kKvRowU4 + part];
            dst[u] = (int64_t)g.dst_row * kKvRowU4 + part;
        }
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u) hot_layer[dst[u]] = v[u];
    }
    for (; c < chunks; c += stride) {
        const int64_t e = c / kKvRowU4;
        const int part = (int)(c - e * kKvRowU4);
        const GatherEntry g = glist[e];
        hot_layer[(int64_t)g.dst_row * kKvRowU4 + part] = pool_layer[(int64_t)g.src_row * kKvRowU4 + part];
    }
}

hipError_t launch_gather_misses(hipStream_t st, const GatherEntry* glist,
                                const uint32_t* gather_total, const uint16_t* pool_layer,
                                uint16_t* hot_layer, int max_entries) {
    const int64_t max_chunks = (int64_t)max_entries * kKvRowU4;
    int grid = (int)std::min<int64_t>((max_chunks + 256 * kGatherUnroll - 1) / (256 * kGatherUnroll), 2048);
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(k_gather_misses, dim3(grid), dim3(256), 0, st, glist, gather_total,
                       reinterpret_cast<const uint4*>(pool_layer), reinterpret_cast<uint4*>(hot_layer),
                       (uint32_t)max_entries);
    return hipGetLastError();
}

}  // namespace sko
