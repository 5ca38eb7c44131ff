// Miss-only host -> device row copy.
//
// [LSO] section 4 "Decode step": only the miss rows are copied from host
// memory to the device, so transfer volume follows the top-k misses, not
// the sequence length ("Top-k miss rows" row of the transfer-granularity
// table).  The pool is pinned, device-mapped host memory; this kernel reads
// it directly over the host link (zero-copy) and writes the 1152-byte rows
// into their victim slots of the hot buffer.  The work list (source row,
// destination row) of every sequence comes from the LRU kernel, with the
// per-sequence miss counts on the device, so no host sync is needed.
#include "sko_common.h"
#include "sko_internal.h"

namespace sko {

constexpr int kGatherThreads = 256;
constexpr int kRowsPerWave = 4;  // rows in flight per wave
constexpr int kGatherMaxBlocks = 512;  // bounds the host reads in flight

// Sequence b's entries are glist[b * mstride + r] for r < counts[b][2].
// Each block first builds the prefix of the per-sequence miss counts in LDS;
// a flat entry index e then maps to (sequence, r) by binary search.
__device__ __forceinline__ int find_seq(const int* pre, int B, int64_t e) {
    int lo = 0, hi = B;  // pre[lo] <= e < pre[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pre[mid] <= e) lo = mid; else hi = mid;
    }
    return lo;
}

// One wave copies whole rows: lanes 0..63 read chunks 0..63 of a 1152-byte
// row (one contiguous 1 KB read), lanes 0..7 the last 8 chunks; each wave
// keeps kRowsPerWave rows in flight before storing them.
__global__ __launch_bounds__(kGatherThreads) void k_gather_misses(const GatherEntry* __restrict__ glist,
                                                                  const int32_t* __restrict__ counts,
                                                                  const uint4* __restrict__ pool_layer,
                                                                  const uint4* __restrict__ recent_layer,
                                                                  const int32_t* __restrict__ ntok_layer,
                                                                  uint4* __restrict__ hot_layer, int B,
                                                                  int64_t cap, int mstride) {
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

    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    for (int64_t e0 = wave * kRowsPerWave; e0 < total; e0 += nwaves * kRowsPerWave) {
        uint4 a[kRowsPerWave], t8[kRowsPerWave];
        int64_t dst[kRowsPerWave];
#pragma unroll
        for (int r = 0; r < kRowsPerWave; ++r) {
            const int64_t e = std::min<int64_t>(e0 + r, total - 1);  // in range; duplicates are not stored
            const int b = find_seq(pre, B, e);
            const GatherEntry g = glist[(size_t)b * mstride + (e - pre[b])];
            // the newest token's row is read from its device copy
            const bool newest = g.src_row == (int64_t)b * cap + ntok_layer[b] - 1;
            const uint4* src = newest ? recent_layer + (int64_t)b * kKvRowU4 : pool_layer + (int64_t)g.src_row * kKvRowU4;
            a[r] = src[lane];
            t8[r] = make_uint4(0u, 0u, 0u, 0u);
            if (lane < kKvRowU4 - 64) t8[r] = src[64 + lane];
            dst[r] = (int64_t)g.dst_row * kKvRowU4;
        }
#pragma unroll
        for (int r = 0; r < kRowsPerWave; ++r) {
            if (e0 + r >= total) break;
            hot_layer[dst[r] + lane] = a[r];
            if (lane < kKvRowU4 - 64) hot_layer[dst[r] + 64 + lane] = t8[r];
        }
    }
}

hipError_t launch_gather_misses(hipStream_t st, const GatherEntry* glist, const int32_t* counts,
                                const uint16_t* pool_layer, const uint16_t* recent_layer,
                                const int32_t* ntok_layer, uint16_t* hot_layer, int B, int64_t cap, int mstride,
                                int max_entries) {
    const int rows_per_block = (kGatherThreads / 64) * kRowsPerWave;
    int grid = (int)std::min<int64_t>(((int64_t)max_entries + rows_per_block - 1) / rows_per_block,
                                      kGatherMaxBlocks);
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(k_gather_misses, dim3(grid), dim3(kGatherThreads), (size_t)(B + 1) * sizeof(int), st,
                       glist, counts, reinterpret_cast<const uint4*>(pool_layer),
                       reinterpret_cast<const uint4*>(recent_layer), ntok_layer,
                       reinterpret_cast<uint4*>(hot_layer), B, cap, mstride);
    return hipGetLastError();
}

}  // namespace sko
