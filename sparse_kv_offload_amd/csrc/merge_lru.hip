// MTP merge/dedupe and the LRU residency update of the hot buffer.
//
// [LSO] section 4 "Decode step": a per-layer LRU residency table finds the
// hits, gives hot-buffer slots to the misses and picks the slots to evict.
// FlashOffloading explainer, decode paragraphs: hits need no host fetch,
// misses take the places of evicted tokens (the shelf size never changes),
// the D position lists are merged and deduplicated before loading, and the
// reverse index cache_slots maps a token to its slot or -1.
//
// Per (layer, seq) state: cache_slots[cap], slot_token[S], last_use[S]
// (step stamp, -1 = never used) and the recency order of the slots: every
// slot once, ascending by (last_use, slot).  At step t, for one sequence:
//   U = the tokens whose bit is set in the winner bitmap (the union of the
//       D position lists, already deduplicated and in token order);
//   hits are stamped t; misses M are listed in token order;
//   victims = the first |M| slots of the recency order that were not hit;
//   the r-th miss takes the r-th victim; a victim's previous owner (if any)
//   is evicted: cache_slots[old] = -1;
//   the new order keeps every untouched slot in place and appends the slots
//   stamped t (hits and victims) in slot order, so it stays sorted by
//   (last_use, slot) without any sort.
// The order lives in two buffers; the step reads one and writes the other.
//
// One 1024-thread block per sequence.  Before the merge it finishes the
// top-k of its D rows whose threshold bucket had to be split (exact radix
// select on the staged candidates); after it, it clears its rows' histograms
// and records for the next step.
#include "sko_common.cuh"
#include "sko_internal.h"

namespace sko {

constexpr int kLruThreads = 1024;

__device__ __forceinline__ bool is_touched(const uint32_t* touched, int32_t s) {
    return (touched[s >> 5] >> (s & 31)) & 1u;
}

__device__ __forceinline__ uint64_t refine_composite(uint2 e) {
    return ((uint64_t)(e.x & 0xFFFFFu) << 32) | (uint64_t)(0xFFFFFFFFu - e.y);
}

// Exact selection of `need` winners among the c staged bucket keys of one
// row.  Radix select, 8 bits per pass from the top, on the 52-bit composite
// (low 20 key bits) << 32 | (0xFFFFFFFF - token), which is unique per
// candidate (so equal scores go to the smaller token); ends with the
// threshold composite T and appends the candidates with composite >= T.
__device__ void refine_row(const uint2* __restrict__ cr, int c, int need, int32_t* __restrict__ out_count,
                           int32_t* __restrict__ w, const int32_t* __restrict__ cs,
                           uint32_t* __restrict__ wb, int top_k, uint32_t* h, int* scratch,
                           int* s_digit, int* s_above) {
    uint64_t prefix = 0;
    int rem = need;
    uint64_t T = 0;
    for (int shift = 48;; shift -= 8) {
        if (threadIdx.x < 256) h[threadIdx.x] = 0u;
        __syncthreads();
        for (int i = threadIdx.x; i < c; i += blockDim.x) {
            const uint64_t comp = refine_composite(cr[i]);
            if ((comp >> (shift + 8)) == prefix) atomicAdd(&h[(comp >> shift) & 255u], 1u);
        }
        __syncthreads();
        // thread t < 256 holds bin 255 - t; scan in descending bin order
        const int v = threadIdx.x < 256 ? (int)h[255 - threadIdx.x] : 0;
        int total;
        const int excl = block_exclusive_scan<kLruThreads>(v, &total, scratch);
        if (threadIdx.x < 256 && excl < rem && excl + v >= rem) {
            *s_digit = 255 - (int)threadIdx.x;
            *s_above = excl;
        }
        __syncthreads();
        const int d = *s_digit;
        rem -= *s_above;
        prefix = (prefix << 8) | (uint64_t)d;
        const bool done = ((int)h[d] == rem) || shift == 0;
        __syncthreads();
        if (done) {
            T = prefix << shift;
            break;
        }
    }
    for (int base = 0; base < c; base += blockDim.x) {
        const int i = base + threadIdx.x;
        const bool valid = i < c;
        const uint2 e = valid ? cr[i] : make_uint2(0u, 0u);
        const bool win = valid && refine_composite(e) >= T;
        const int pw = wave_append(out_count, win);
        if (win && pw < top_k) {
            const bool miss = cs[e.y] == -1;
            w[pw] = (int32_t)(e.y | (miss ? 0x80000000u : 0u));
            atomicOr(&wb[e.y >> 5], 1u << (e.y & 31u));
        }
    }
    __syncthreads();
}

__global__ __launch_bounds__(kLruThreads) void k_merge_lru(
    uint32_t* __restrict__ winners, uint32_t* __restrict__ hist, RowMeta* __restrict__ meta,
    const uint2* __restrict__ cand, int32_t* __restrict__ topk, const int32_t* __restrict__ ntok_layer,
    int32_t* __restrict__ cache_slots_layer, int32_t* __restrict__ slot_token_layer,
    int32_t* __restrict__ last_use_layer, const int32_t* __restrict__ order_cur,
    int32_t* __restrict__ order_next, int D, int top_k, int S, int64_t Sp, int64_t cap, int64_t wpr,
    int32_t t, int32_t* __restrict__ misses, int32_t* __restrict__ victims,
    int32_t* __restrict__ evict_old, int32_t* __restrict__ counts, GatherEntry* __restrict__ glist,
    unsigned long long* __restrict__ layer_stats) {
    __shared__ uint32_t touched[kMaxHotSlots / 32];
    __shared__ int32_t mlist[kMaxMerge];
    __shared__ int32_t vlist[kMaxMerge];
    __shared__ uint32_t h[256];
    __shared__ int scratch[kLruThreads / 64 + 1];
    __shared__ int s_digit, s_above;

    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t Lt = ntok_layer[b];
    const int kk = (int)std::min<int64_t>(top_k, Lt);
    int32_t* __restrict__ cs = cache_slots_layer + (size_t)b * cap;
    int32_t* __restrict__ st = slot_token_layer + (size_t)b * S;
    int32_t* __restrict__ lu = last_use_layer + (size_t)b * S;
    const int32_t* __restrict__ oc = order_cur + (size_t)b * Sp;
    int32_t* __restrict__ on = order_next + (size_t)b * Sp;
    uint32_t* __restrict__ wb = winners + (size_t)b * wpr;
    int32_t* __restrict__ cnt = counts + (size_t)b * 8;
    const int mstride = D * top_k;
    const int SW = (S + 31) / 32;

    // 0. finish the top-k of rows whose threshold bucket is split
    for (int p = 0; p < D; ++p) {
        const int row = b * D + p;
        const RowMeta m = meta[row];
        if (m.bucket < 0 || m.need == 0 || m.need == m.bucket_count) continue;
        const int c = (int)std::min<int64_t>(m.cand_count, cap);
        refine_row(cand + (size_t)row * cap, c, m.need, &meta[row].out_count, topk + (size_t)row * top_k, cs, wb,
                   top_k, h, scratch, &s_digit, &s_above);
    }

    for (int i = tid; i < SW; i += kLruThreads) touched[i] = 0u;
    if (tid == 0) cnt[7] = 0;
    __syncthreads();

    // 1. the union U in token order: count hits and misses per run of words
    const int64_t nwords = (Lt + 31) / 32;
    const int64_t wper = (nwords + kLruThreads - 1) / kLruThreads;
    const int64_t w0 = std::min<int64_t>(nwords, (int64_t)tid * wper);
    const int64_t w1 = std::min<int64_t>(nwords, w0 + wper);
    int nh_loc = 0, nm_loc = 0;
    for (int64_t w = w0; w < w1; ++w) {
        uint32_t bits = wb[w];
        while (bits) {
            const int e = __ffs((int)bits) - 1;
            bits &= bits - 1u;
            if (cs[w * 32 + e] < 0) ++nm_loc; else ++nh_loc;
        }
    }
    int nH, nM;
    (void)block_exclusive_scan<kLruThreads>(nh_loc, &nH, scratch);
    const int m_off = block_exclusive_scan<kLruThreads>(nm_loc, &nM, scratch);
    // misses listed in token order; hits stamped and marked; bitmap cleared
    {
        int o = m_off;
        for (int64_t w = w0; w < w1; ++w) {
            uint32_t bits = wb[w];
            if (!bits) continue;
            wb[w] = 0u;
            while (bits) {
                const int e = __ffs((int)bits) - 1;
                bits &= bits - 1u;
                const int32_t tok = (int32_t)(w * 32 + e);
                const int32_t slot = cs[tok];
                if (slot < 0) {
                    if (o < kMaxMerge) mlist[o] = tok;
                    ++o;
                } else if (slot < S) {
                    atomicOr(&touched[slot >> 5], 1u << (slot & 31));
                    lu[slot] = t;
                }
            }
        }
    }
    __syncthreads();

    int nEv = 0;
    const bool sane = nM <= kMaxMerge && nH + nM <= S;
    if (nM > 0 && sane) {
        // 2. victims: the first nM slots of the recency order not hit at t;
        //    they lie within its first nM + nH entries
        const int P = std::min(S, nM + nH);
        const int per = (P + kLruThreads - 1) / kLruThreads;
        const int p0 = std::min(P, tid * per), p1 = std::min(P, p0 + per);
        int c = 0;
        for (int i = p0; i < p1; ++i) c += !is_touched(touched, oc[i]);
        int avail;
        int vpos = block_exclusive_scan<kLruThreads>(c, &avail, scratch);
        for (int i = p0; i < p1 && vpos < nM; ++i) {
            const int32_t s = oc[i];
            if (!is_touched(touched, s)) vlist[vpos++] = s;
        }
        __syncthreads();
        for (int r = tid; r < nM; r += kLruThreads) {
            const int32_t s = vlist[r];
            if (s >= 0 && s < S) atomicOr(&touched[s >> 5], 1u << (s & 31));
        }
        __syncthreads();
        // 3. assignment: r-th miss -> r-th victim
        int ev_loc = 0;
        for (int r = tid; r < nM; r += kLruThreads) {
            const int32_t v = vlist[r];
            const int32_t m = mlist[r];
            if (avail < nM || v < 0 || v >= S || m < 0 || m >= cap) {
                cnt[7] = 1;  // invariant violated; reported in the counts record
                continue;
            }
            const int32_t old = st[v];
            if (old >= 0 && old < cap) {
                cs[old] = -1;
                ++ev_loc;
            }
            cs[m] = v;
            st[v] = m;
            lu[v] = t;
            misses[(size_t)b * mstride + r] = m;
            victims[(size_t)b * mstride + r] = v;
            evict_old[(size_t)b * mstride + r] = old;
            glist[(size_t)b * mstride + r] = GatherEntry{(uint32_t)((int64_t)b * cap + m), (uint32_t)((int64_t)b * S + v)};
        }
        int ev_total;
        (void)block_exclusive_scan<kLruThreads>(ev_loc, &ev_total, scratch);
        nEv = ev_total;
    } else if (nM > 0) {
        if (tid == 0) cnt[7] = 1;
    }
    __syncthreads();

    // 4. next recency order: untouched slots in their order, then the slots
    //    stamped t in slot order.  Runs are multiples of 4 entries (rows are
    //    padded to Sp, a multiple of 4) and read as 16-byte vectors.
    {
        const int per = ((S + kLruThreads - 1) / kLruThreads + 3) & ~3;
        const int s0 = std::min(S, tid * per), s1 = std::min(S, s0 + per);
        int keep = 0;
        for (int i = s0; i < s1; i += 4) {
            const int4 v = *reinterpret_cast<const int4*>(oc + i);
            keep += !is_touched(touched, v.x);
            if (i + 1 < s1) keep += !is_touched(touched, v.y);
            if (i + 2 < s1) keep += !is_touched(touched, v.z);
            if (i + 3 < s1) keep += !is_touched(touched, v.w);
        }
        int nkeep;
        int kpos = block_exclusive_scan<kLruThreads>(keep, &nkeep, scratch);
        for (int i = s0; i < s1; i += 4) {
            const int4 v = *reinterpret_cast<const int4*>(oc + i);
            const int32_t e4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (i + q < s1 && !is_touched(touched, e4[q]) && kpos < S) on[kpos++] = e4[q];
        }
        const int tw = (SW + kLruThreads - 1) / kLruThreads;
        const int q0 = std::min(SW, tid * tw), q1 = std::min(SW, q0 + tw);
        int ct = 0;
        for (int q = q0; q < q1; ++q) ct += __popc(touched[q]);
        int ntouched;
        int tpos = nkeep + block_exclusive_scan<kLruThreads>(ct, &ntouched, scratch);
        for (int q = q0; q < q1; ++q) {
            uint32_t bits = touched[q];
            while (bits) {
                const int e = __ffs((int)bits) - 1;
                bits &= bits - 1u;
                if (tpos < S) on[tpos++] = q * 32 + e;
            }
        }
    }

    // 5. counters; clear this sequence's selection scratch for the next step
    for (int i = tid; i < D * kHistBins; i += kLruThreads) hist[(size_t)b * D * kHistBins + i] = 0u;
    if (tid < D) meta[b * D + tid] = RowMeta{-1, 0, 0, 0, 0, 0, {0, 0}};
    if (tid == 0) {
        const int nU = nH + nM;
        cnt[0] = nU; cnt[1] = nH; cnt[2] = nM; cnt[3] = nEv;
        cnt[4] = kk; cnt[5] = (int32_t)Lt; cnt[6] = t;
        atomicAdd(&layer_stats[1], (unsigned long long)nU);
        atomicAdd(&layer_stats[2], (unsigned long long)nH);
        atomicAdd(&layer_stats[3], (unsigned long long)nM);
        atomicAdd(&layer_stats[4], (unsigned long long)nEv);
        if (b == 0) atomicAdd(&layer_stats[0], 1ull);
    }
}

hipError_t launch_merge_lru(hipStream_t st, uint32_t* winners, uint32_t* hist, RowMeta* meta,
                            const uint2* cand, int32_t* topk, const int32_t* ntok_layer,
                            int32_t* cache_slots_layer, int32_t* slot_token_layer,
                            int32_t* last_use_layer, const int32_t* order_cur, int32_t* order_next,
                            int B, int D, int top_k, int S, int64_t cap, int32_t t,
                            int32_t* misses, int32_t* victims, int32_t* evict_old, int32_t* counts,
                            GatherEntry* glist, unsigned long long* layer_stats) {
    const int64_t Sp = ((int64_t)S + 3) / 4 * 4;
    const int64_t wpr = (cap + 31) / 32;
    hipLaunchKernelGGL(k_merge_lru, dim3(B), dim3(kLruThreads), 0, st, winners, hist, meta, cand, topk,
                       ntok_layer, cache_slots_layer, slot_token_layer, last_use_layer, order_cur,
                       order_next, D, top_k, S, Sp, cap, wpr, t, misses, victims, evict_old, counts,
                       glist, layer_stats);
    return hipGetLastError();
}

__global__ void k_init_order(int32_t* __restrict__ order, int64_t n_seqs, int S, int64_t Sp) {
    const int64_t total = n_seqs * Sp;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t s = i % Sp;
        order[i] = s < S ? (int32_t)s : -1;
    }
}

hipError_t launch_init_order(hipStream_t st, int32_t* order, int64_t n_seqs, int S) {
    const int64_t Sp = ((int64_t)S + 3) / 4 * 4;
    const int64_t total = n_seqs * Sp;
    const int g = (int)std::min<int64_t>((total + 255) / 256, 4096);
    hipLaunchKernelGGL(k_init_order, dim3(std::max(g, 1)), dim3(256), 0, st, order, n_seqs, S, Sp);
    return hipGetLastError();
}

}  // namespace sko
