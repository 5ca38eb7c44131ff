// Token append, indexer scoring and the packed top-k selection.
//
// Scoring and selection follow [LSO] section 4 "Decode step" (the indexer
// picks logical top-k positions) and the FlashOffloading explainer's decode
// paragraphs (every winner carries its token index and its residency in one
// int32, so the selection already says hit or miss).  The score of token i
// for query position p is the 64-d dot product q_p . K_i accumulated in
// binary32 by fused multiply-add in index order 0..63 from +0; winners are
// the min(k, L_t) largest (score, -index) pairs.
//
// Selection is a radix select over the monotone 32-bit key of the score:
//   1. k_score_hist: one pass over the indexer cache (the HBM stream) that
//      writes the keys and a 12-bit first-digit histogram per row;
//   2. k_topk_threshold: per row, the bucket holding the k-th largest key;
//   3. k_topk_filter: keys above that bucket are winners; keys in it are
//      staged (or taken whole when the bucket fits exactly);
//   4. k_topk_refine: exact selection inside the bucket on the composite
//      (low 20 key bits, inverted index), so ties go to smaller indices.
#include "sko_common.cuh"
#include "sko_internal.h"

namespace sko {

// ---------------------------------------------------------------- append

// Rows of the new tokens: 16-byte chunks 0..7 are the indexer row (to the
// device cache), chunks 8..79 the main-KV row (to the host pool through its
// device mapping).  Sets the sequence's token count to base + n.
__global__ __launch_bounds__(256) void k_append_rows(const uint4* __restrict__ idx_src,
                                                     const uint4* __restrict__ kv_src,
                                                     uint4* __restrict__ idx_layer,
                                                     uint4* __restrict__ pool_layer,
                                                     int32_t* __restrict__ ntok_layer, int seq0,
                                                     int64_t n, int64_t cap, int32_t base) {
    const int s = blockIdx.y;
    const int b = seq0 + s;
    const int64_t chunks = n * (kIdxRowU4 + kKvRowU4);
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks;
         c += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = c / (kIdxRowU4 + kKvRowU4);
        const int part = (int)(c - r * (kIdxRowU4 + kKvRowU4));
        const int64_t src_row = (int64_t)s * n + r;
        const int64_t dst_row = (int64_t)b * cap + base + r;
        if (part < kIdxRowU4)
            idx_layer[dst_row * kIdxRowU4 + part] = idx_src[src_row * kIdxRowU4 + part];
        else
            pool_layer[dst_row * kKvRowU4 + (part - kIdxRowU4)] =
                kv_src[src_row * kKvRowU4 + (part - kIdxRowU4)];
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) ntok_layer[b] = base + (int32_t)n;
}

hipError_t launch_append_rows(hipStream_t st, const uint16_t* idx_src, const uint16_t* kv_src,
                              uint16_t* idx_layer, uint16_t* pool_layer, int32_t* ntok_layer,
                              int seq0, int nseq, int64_t n, int64_t cap, int32_t base) {
    const int64_t chunks = n * (kIdxRowU4 + kKvRowU4);
    int gx = (int)std::min<int64_t>((chunks + 255) / 256, 4096);
    if (gx < 1) gx = 1;
    hipLaunchKernelGGL(k_append_rows, dim3(gx, nseq), dim3(256), 0, st,
                       reinterpret_cast<const uint4*>(idx_src), reinterpret_cast<const uint4*>(kv_src),
                       reinterpret_cast<uint4*>(idx_layer), reinterpret_cast<uint4*>(pool_layer),
                       ntok_layer, seq0, n, cap, base);
    return hipGetLastError();
}

__global__ void k_set_ntok(int32_t* ntok_layer, int seq0, int nseq, int32_t value) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < nseq) ntok_layer[seq0 + i] = value;
}

hipError_t launch_set_ntok(hipStream_t st, int32_t* ntok_layer, int seq0, int nseq, int32_t value) {
    hipLaunchKernelGGL(k_set_ntok, dim3((nseq + 255) / 256), dim3(256), 0, st, ntok_layer, seq0,
                       nseq, value);
    return hipGetLastError();
}

// ---------------------------------------------------------------- step init

// Clears the per-step counters with plain stores (no memset nodes, so the
// step stays safe to capture in a graph).
__global__ __launch_bounds__(256) void k_step_init(uint32_t* __restrict__ hist, RowMeta* __restrict__ meta,
                                                   uint32_t* __restrict__ gather_total, int rows) {
    const int64_t nh = (int64_t)rows * kHistBins;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nh;
         i += (int64_t)gridDim.x * blockDim.x)
        hist[i] = 0u;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < rows) meta[i] = RowMeta{-1, 0, 0, 0, 0, 0, {0, 0}};
    if (i == 0) *gather_total = 0u;
}

hipError_t launch_step_init(hipStream_t st, uint32_t* hist, RowMeta* meta, uint32_t* gather_total,
                            int rows) {
    int g = (int)std::min<int64_t>(((int64_t)rows * kHistBins + 255) / 256, 1024);
    g = std::max(g, (rows + 255) / 256);
    hipLaunchKernelGGL(k_step_init, dim3(g), dim3(256), 0, st, hist, meta, gather_total, rows);
    return hipGetLastError();
}

// ---------------------------------------------------------------- score

// One block scores `chunk` consecutive tokens of one sequence for NP query
// positions (p0 .. p0+NP-1).  Each thread owns whole tokens: the 128-byte
// row is loaded into registers and every position runs its 64-term FMA
// chain in index order.  The first-digit histogram is counted in LDS with
// two 16-bit counters per word (chunk < 65536) and flushed with one global
// atomic per non-empty bin.
template <int NP>
__global__ __launch_bounds__(256) void k_score_hist(const uint4* __restrict__ idx_layer,
                                                    const uint32_t* __restrict__ q_idx,
                                                    const int32_t* __restrict__ ntok_layer,
                                                    uint32_t* __restrict__ keys,
                                                    uint32_t* __restrict__ hist, int D, int p0,
                                                    int64_t cap, int chunk) {
    constexpr int HW = kHistBins / 2;  // packed words per position
    __shared__ uint32_t sh[NP * HW];
    const int b = blockIdx.y;
    const int64_t Lt = ntok_layer[b];
    const int64_t start = (int64_t)blockIdx.x * chunk;
    if (start >= Lt) return;
    const int64_t end = std::min<int64_t>(start + chunk, Lt);
    for (int i = threadIdx.x; i < NP * HW; i += blockDim.x) sh[i] = 0u;
    __syncthreads();

    const uint32_t* __restrict__ qb = q_idx + ((size_t)b * D + p0) * (kIdxDim / 2);
    const uint4* __restrict__ kb = idx_layer + (size_t)b * cap * kIdxRowU4;
    uint32_t* __restrict__ keyrow = keys + ((size_t)b * D + p0) * cap;

    for (int64_t i = start + threadIdx.x; i < end; i += blockDim.x) {
        uint32_t w[32];
#pragma unroll
        for (int c = 0; c < kIdxRowU4; ++c) {
            const uint4 v = kb[i * kIdxRowU4 + c];
            w[4 * c + 0] = v.x;
            w[4 * c + 1] = v.y;
            w[4 * c + 2] = v.z;
            w[4 * c + 3] = v.w;
        }
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                const uint32_t qw = qb[p * 32 + j];
                acc = __builtin_fmaf(bf16_lo(qw), bf16_lo(w[j]), acc);
                acc = __builtin_fmaf(bf16_hi(qw), bf16_hi(w[j]), acc);
            }
            if (acc == 0.0f) acc = 0.0f;  // store a zero as +0
            const uint32_t key = score_key(acc);
            keyrow[(size_t)p * cap + i] = key;
            const uint32_t bin = key >> (32 - kHistBits);
            atomicAdd(&sh[p * HW + (bin >> 1)], 1u << ((bin & 1u) << 4));
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < NP * HW; i += blockDim.x) {
        const uint32_t v = sh[i];
        if (v == 0u) continue;
        const int p = i / HW;
        const int bin = (i - p * HW) * 2;
        uint32_t* h = hist + ((size_t)b * D + p0 + p) * kHistBins;
        if (v & 0xFFFFu) atomicAdd(&h[bin], v & 0xFFFFu);
        if (v >> 16) atomicAdd(&h[bin + 1], v >> 16);
    }
}

static int score_chunk(int B, int64_t max_tokens_now) {
    // enough blocks to cover the chip several times, each block at least 512
    // tokens and below 65536 (16-bit LDS counters)
    int chunk = 512;
    while (chunk < 16384 && (int64_t)B * ((max_tokens_now + chunk * 2 - 1) / (chunk * 2)) >= 2048)
        chunk *= 2;
    return chunk;
}

hipError_t launch_score_hist(hipStream_t st, const uint16_t* idx_layer, const uint16_t* q_idx,
                             const int32_t* ntok_layer, uint32_t* keys, uint32_t* hist, int B,
                             int D, int64_t cap, int64_t max_tokens_now, int /*top_k*/) {
    if (max_tokens_now <= 0) return hipSuccess;
    const int chunk = score_chunk(B, max_tokens_now);
    const dim3 grid((unsigned)((max_tokens_now + chunk - 1) / chunk), (unsigned)B);
    const uint4* kb = reinterpret_cast<const uint4*>(idx_layer);
    const uint32_t* q = reinterpret_cast<const uint32_t*>(q_idx);
    for (int p0 = 0; p0 < D;) {
        const int np = std::min(4, D - p0);
        switch (np) {
            case 1: hipLaunchKernelGGL(k_score_hist<1>, grid, dim3(256), 0, st, kb, q, ntok_layer, keys, hist, D, p0, cap, chunk); break;
            case 2: hipLaunchKernelGGL(k_score_hist<2>, grid, dim3(256), 0, st, kb, q, ntok_layer, keys, hist, D, p0, cap, chunk); break;
            case 3: hipLaunchKernelGGL(k_score_hist<3>, grid, dim3(256), 0, st, kb, q, ntok_layer, keys, hist, D, p0, cap, chunk); break;
            default: hipLaunchKernelGGL(k_score_hist<4>, grid, dim3(256), 0, st, kb, q, ntok_layer, keys, hist, D, p0, cap, chunk); break;
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        p0 += np;
    }
    return hipSuccess;
}

// ---------------------------------------------------------------- threshold

// One block per (seq, position) row: walks the histogram from the top bucket
// down to the one that holds the k-th largest key.
__global__ __launch_bounds__(256) void k_topk_threshold(const uint32_t* __restrict__ hist,
                                                        RowMeta* __restrict__ meta,
                                                        const int32_t* __restrict__ ntok_layer,
                                                        int D, int top_k) {
    __shared__ int scratch[8];
    __shared__ RowMeta result;
    const int row = blockIdx.x;
    const int b = row / D;
    const int64_t Lt = ntok_layer[b];
    const int kk = (int)std::min<int64_t>(top_k, Lt);
    const uint32_t* h = hist + (size_t)row * kHistBins;
    // thread t owns the 16 bins 4095-16t .. 4080-16t (thread 0 the top ones)
    const int hi_bin = kHistBins - 1 - 16 * (int)threadIdx.x;
    uint32_t loc[16];
    int sum = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        loc[j] = h[hi_bin - j];
        sum += (int)loc[j];
    }
    if (threadIdx.x == 0) result = RowMeta{-1, 0, 0, 0, 0, 0, {0, 0}};
    int total;
    const int excl = block_exclusive_scan<256>(sum, &total, scratch);
    if (kk > 0 && excl < kk && excl + sum >= kk) {
        int c = excl;
        for (int j = 0; j < 16; ++j) {
            const int cnt = (int)loc[j];
            if (c + cnt >= kk) {
                result = RowMeta{hi_bin - j, c, kk - c, cnt, 0, 0, {0, 0}};
                break;
            }
            c += cnt;
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) meta[row] = result;
}

hipError_t launch_topk_threshold(hipStream_t st, const uint32_t* hist, RowMeta* meta,
                                 const int32_t* ntok_layer, int B, int D, int top_k) {
    hipLaunchKernelGGL(k_topk_threshold, dim3(B * D), dim3(256), 0, st, hist, meta, ntok_layer, D,
                       top_k);
    return hipGetLastError();
}

// ---------------------------------------------------------------- filter

__device__ __forceinline__ int32_t pack_winner(int64_t token, const int32_t* __restrict__ cs) {
    const bool miss = cs[token] == -1;
    return (int32_t)((uint32_t)token | (miss ? 0x80000000u : 0u));
}

__global__ __launch_bounds__(256) void k_topk_filter(const uint32_t* __restrict__ keys,
                                                     RowMeta* __restrict__ meta,
                                                     uint2* __restrict__ cand,
                                                     int32_t* __restrict__ topk,
                                                     const int32_t* __restrict__ cache_slots_layer,
                                                     const int32_t* __restrict__ ntok_layer, int D,
                                                     int64_t cap, int top_k, int chunk) {
    const int row = blockIdx.y;
    const int b = row / D;
    const int bucket = meta[row].bucket;
    if (bucket < 0) return;
    const int64_t Lt = ntok_layer[b];
    const int64_t start = (int64_t)blockIdx.x * chunk;
    if (start >= Lt) return;
    const int64_t end = std::min<int64_t>(start + chunk, Lt);
    const bool take_bucket = meta[row].need == meta[row].bucket_count;
    const uint32_t* __restrict__ krow = keys + (size_t)row * cap;
    const int32_t* __restrict__ cs = cache_slots_layer + (size_t)b * cap;
    int32_t* __restrict__ w = topk + (size_t)row * top_k;
    uint2* __restrict__ cr = cand + (size_t)row * cap;
    for (int64_t base = start; base < end; base += blockDim.x) {
        const int64_t i = base + threadIdx.x;
        const bool valid = i < end;
        const uint32_t key = valid ? krow[i] : 0u;
        const int bin = (int)(key >> (32 - kHistBits));
        const bool win = valid && (bin > bucket || (bin == bucket && take_bucket));
        const bool stage = valid && bin == bucket && !take_bucket;
        const int pw = wave_append(&meta[row].out_count, win);
        if (win && pw < top_k) w[pw] = pack_winner(i, cs);
        const int pc = wave_append(&meta[row].cand_count, stage);
        if (stage && pc < cap) cr[pc] = make_uint2(key, (uint32_t)i);
    }
}

hipError_t launch_topk_filter(hipStream_t st, const uint32_t* keys, RowMeta* meta, uint2* cand,
                              int32_t* topk, const int32_t* cache_slots_layer,
                              const int32_t* ntok_layer, int B, int D, int64_t cap, int top_k,
                              int64_t max_tokens_now) {
    if (max_tokens_now <= 0) return hipSuccess;
    int chunk = 1024;
    while (chunk < 65536 && (int64_t)B * D * ((max_tokens_now + chunk * 2 - 1) / (chunk * 2)) >= 2048)
        chunk *= 2;
    const dim3 grid((unsigned)((max_tokens_now + chunk - 1) / chunk), (unsigned)(B * D));
    hipLaunchKernelGGL(k_topk_filter, grid, dim3(256), 0, st, keys, meta, cand, topk,
                       cache_slots_layer, ntok_layer, D, cap, top_k, chunk);
    return hipGetLastError();
}

// ---------------------------------------------------------------- refine

// One block per row whose threshold bucket must be split.  Radix select,
// 8 bits per pass from the top, on the 52-bit composite
//     (low 20 bits of the key) << 32 | (0xFFFFFFFF - token)
// which is unique per candidate, so the selection is exact and equal scores
// go to the smaller token index.  Ends with the threshold composite T; the
// winners are the candidates with composite >= T.
__global__ __launch_bounds__(256) void k_topk_refine(const uint2* __restrict__ cand,
                                                     RowMeta* __restrict__ meta,
                                                     int32_t* __restrict__ topk,
                                                     const int32_t* __restrict__ cache_slots_layer,
                                                     int D, int64_t cap, int top_k) {
    __shared__ uint32_t h[256];
    __shared__ int scratch[8];
    __shared__ int s_digit, s_above;
    const int row = blockIdx.x;
    const int b = row / D;
    const RowMeta m = meta[row];
    if (m.bucket < 0 || m.need == 0 || m.need == m.bucket_count) return;
    const int c = (int)std::min<int64_t>(m.cand_count, cap);
    const uint2* __restrict__ cr = cand + (size_t)row * cap;
    auto composite = [](uint2 e) -> uint64_t {
        return ((uint64_t)(e.x & 0xFFFFFu) << 32) | (uint64_t)(0xFFFFFFFFu - e.y);
    };
    uint64_t prefix = 0;
    int rem = m.need;
    uint64_t T = 0;
    for (int shift = 48;; shift -= 8) {
        h[threadIdx.x] = 0u;
        __syncthreads();
        for (int i = threadIdx.x; i < c; i += blockDim.x) {
            const uint64_t comp = composite(cr[i]);
            if ((comp >> (shift + 8)) == prefix) atomicAdd(&h[(comp >> shift) & 255u], 1u);
        }
        __syncthreads();
        // thread t holds bin 255 - t; scan in descending bin order
        const int v = (int)h[255 - threadIdx.x];
        int total;
        const int excl = block_exclusive_scan<256>(v, &total, scratch);
        if (excl < rem && excl + v >= rem) {
            s_digit = 255 - (int)threadIdx.x;
            s_above = excl;
        }
        __syncthreads();
        const int d = s_digit;
        rem -= s_above;
        prefix = (prefix << 8) | (uint64_t)d;
        const bool done = ((int)h[d] == rem) || shift == 0;
        __syncthreads();
        if (done) {
            T = prefix << shift;
            break;
        }
    }
    const int32_t* __restrict__ cs = cache_slots_layer + (size_t)b * cap;
    int32_t* __restrict__ w = topk + (size_t)row * top_k;
    for (int base = 0; base < c; base += blockDim.x) {
        const int i = base + threadIdx.x;
        const bool valid = i < c;
        const uint2 e = valid ? cr[i] : make_uint2(0u, 0u);
        const bool win = valid && composite(e) >= T;
        const int pw = wave_append(&meta[row].out_count, win);
        if (win && pw < top_k) w[pw] = pack_winner(e.y, cs);
    }
}

hipError_t launch_topk_refine(hipStream_t st, const uint2* cand, RowMeta* meta, int32_t* topk,
                              const int32_t* cache_slots_layer, int B, int D, int64_t cap,
                              int top_k) {
    hipLaunchKernelGGL(k_topk_refine, dim3(B * D), dim3(256), 0, st, cand, meta, topk,
                       cache_slots_layer, D, cap, top_k);
    return hipGetLastError();
}

}  // namespace sko
