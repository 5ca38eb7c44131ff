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
// (step stamp, -1 = never used).  At step t, for one sequence:
//   U = sorted unique union of the D winner lists (token order);
//   hits (flag clear) are stamped t;
//   victims = slots not stamped t, ascending (last_use, slot);
//   the r-th ascending miss takes the r-th victim; a victim's previous
//   owner (if any) is evicted: cache_slots[old] = -1.
//
// One 1024-thread block per sequence:
//   1. bitonic sort of the D*kk packed winners by token (LDS);
//   2. unique + split into hits / misses with block scans; stamp hits;
//   3. radix select (11-bit digits) of the |M|-th smallest stamp over the
//      S slots, then an ordered collection of the victims;
//   4. bitonic sort of the victims by (stamp, slot);
//   5. assignment, eviction records, and a slot in the global gather list.
#include "sko_common.cuh"
#include "sko_internal.h"

namespace sko {

constexpr int kLruThreads = 1024;
constexpr int kLruDigit = 11;

template <typename T, typename KeyFn>
__device__ __forceinline__ void bitonic_sort_lds(T* a, int n2, KeyFn key) {
    // ascending sort of a[0..n2) (n2 a power of two) by key(a[i])
    for (int size = 2; size <= n2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = threadIdx.x; i < (n2 >> 1); i += blockDim.x) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const bool up = (lo & size) == 0;
                const T x = a[lo], y = a[hi];
                const bool swap = up ? (key(x) > key(y)) : (key(x) < key(y));
                if (swap) {
                    a[lo] = y;
                    a[hi] = x;
                }
            }
            __syncthreads();
        }
    }
}

__device__ __forceinline__ int next_pow2(int n) {
    int p = 1;
    while (p < n) p <<= 1;
    return p;
}

__global__ __launch_bounds__(kLruThreads) void k_merge_lru(
    const int32_t* __restrict__ topk, const int32_t* __restrict__ ntok_layer,
    int32_t* __restrict__ cache_slots_layer, int32_t* __restrict__ slot_token_layer,
    int32_t* __restrict__ last_use_layer, int D, int top_k, int S, int64_t cap, int32_t t,
    int32_t* __restrict__ misses, int32_t* __restrict__ victims, int32_t* __restrict__ evict_old,
    int32_t* __restrict__ counts, GatherEntry* __restrict__ glist,
    uint32_t* __restrict__ gather_total, unsigned long long* __restrict__ layer_stats) {
    __shared__ uint32_t wl[kMaxMerge];          // packed winners, then the miss list
    __shared__ unsigned long long vic[kMaxMerge];  // (stamp + 1) << 32 | slot
    __shared__ uint32_t hist[1 << kLruDigit];
    __shared__ int scratch[kLruThreads / 64 + 1];
    __shared__ int s_digit, s_below;
    __shared__ uint32_t s_kmin, s_kmax;
    __shared__ uint32_t s_gbase;

    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t Lt = ntok_layer[b];
    const int kk = (int)std::min<int64_t>(top_k, Lt);
    const int n = D * kk;
    int32_t* __restrict__ cs = cache_slots_layer + (size_t)b * cap;
    int32_t* __restrict__ st = slot_token_layer + (size_t)b * S;
    int32_t* __restrict__ lu = last_use_layer + (size_t)b * S;
    int32_t* __restrict__ cnt = counts + (size_t)b * 8;
    const int mstride = D * top_k;

    if (tid == 0) cnt[7] = 0;
    __syncthreads();
    if (n == 0) {
        if (tid == 0) {
            cnt[0] = 0; cnt[1] = 0; cnt[2] = 0; cnt[3] = 0;
            cnt[4] = 0; cnt[5] = (int32_t)Lt; cnt[6] = t; cnt[7] = 0;
        }
        return;
    }

    // 1. gather the D lists and sort by token
    const int n2 = next_pow2(n);
    for (int i = tid; i < n2; i += kLruThreads) {
        uint32_t v = 0x7FFFFFFFu;  // padding sorts last
        if (i < n) {
            const int p = i / kk, j = i - p * kk;
            v = (uint32_t)topk[((size_t)b * D + p) * top_k + j];
        }
        wl[i] = v;
    }
    __syncthreads();
    bitonic_sort_lds(wl, n2, [](uint32_t v) { return v & 0x7FFFFFFFu; });

    // 2. unique, split into hits and misses (each thread owns a contiguous run)
    const int per = (n2 + kLruThreads - 1) / kLruThreads;  // <= 8
    const int r0 = tid * per;
    uint32_t mine[8];
    uint32_t prev = (r0 > 0 && r0 - 1 < n) ? (wl[r0 - 1] & 0x7FFFFFFFu) : 0xFFFFFFFFu;
    int nu_loc = 0, nm_loc = 0;
    uint32_t newmask = 0, missmask = 0;
    for (int e = 0; e < per; ++e) {
        const int i = r0 + e;
        uint32_t v = (i < n) ? wl[i] : 0x7FFFFFFFu;
        mine[e] = v;
        if (i < n) {
            const uint32_t tok = v & 0x7FFFFFFFu;
            if (tok != prev) {
                newmask |= 1u << e;
                ++nu_loc;
                if (v >> 31) {
                    missmask |= 1u << e;
                    ++nm_loc;
                }
            }
            prev = tok;
        }
    }
    int nU, nM;
    const int u_off = block_exclusive_scan<kLruThreads>(nu_loc, &nU, scratch);
    (void)u_off;
    const int m_off = block_exclusive_scan<kLruThreads>(nm_loc, &nM, scratch);
    // misses into wl (in place: every thread's run was read above and the
    // scans contain barriers); hits stamped with t
    {
        int o = m_off;
        for (int e = 0; e < per; ++e) {
            if (!((newmask >> e) & 1u)) continue;
            const uint32_t tok = mine[e] & 0x7FFFFFFFu;
            if ((missmask >> e) & 1u) {
                wl[o++] = tok;
            } else if (tok < (uint32_t)cap) {
                const int32_t slot = cs[tok];
                if (slot >= 0 && slot < S) lu[slot] = t;
            }
        }
    }
    __syncthreads();

    int nEv = 0;
    if (nM > 0) {
        // 3. the nM least recently used slots among those not stamped t
        const int run = (S + kLruThreads - 1) / kLruThreads;
        const int s0 = std::min(S, tid * run), s1 = std::min(S, s0 + run);
        uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
        for (int s = s0; s < s1; ++s) {
            const int32_t u = lu[s];
            if (u < t) {
                const uint32_t key = (uint32_t)(u + 1);
                kmin = std::min(kmin, key);
                kmax = std::max(kmax, key);
            }
        }
        for (int o = 32; o > 0; o >>= 1) {
            kmin = std::min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
            kmax = std::max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
        }
        if (tid == 0) { s_kmin = 0xFFFFFFFFu; s_kmax = 0u; }
        __syncthreads();
        if ((tid & 63) == 0) {
            atomicMin(&s_kmin, kmin);
            atomicMax(&s_kmax, kmax);
        }
        __syncthreads();
        kmin = s_kmin;
        kmax = s_kmax;
        const uint32_t range = kmax - kmin;
        const int nb = range == 0 ? 0 : 32 - __clz((int)range);
        const int npass = std::max(1, (nb + kLruDigit - 1) / kLruDigit);
        uint64_t prefix = 0;
        int rem = nM;
        uint64_t lt_bound = 0;  // victims: key - kmin < lt_bound ...
        uint64_t eq_key = 0;    // ... plus the first r_eq slots with key - kmin == eq_key
        int r_eq = 0;
        for (int pass = npass - 1; pass >= 0; --pass) {
            const int shift = pass * kLruDigit;
            for (int i = tid; i < (1 << kLruDigit); i += kLruThreads) hist[i] = 0u;
            __syncthreads();
            for (int s = s0; s < s1; ++s) {
                const int32_t u = lu[s];
                if (u >= t) continue;
                const uint64_t kr = (uint64_t)((uint32_t)(u + 1) - kmin);
                if ((kr >> (shift + kLruDigit)) == prefix)
                    atomicAdd(&hist[(kr >> shift) & ((1u << kLruDigit) - 1)], 1u);
            }
            __syncthreads();
            // ascending scan: thread i holds bins 2i, 2i+1
            const int v0 = (int)hist[2 * tid], v1 = (int)hist[2 * tid + 1];
            int total;
            const int excl = block_exclusive_scan<kLruThreads>(v0 + v1, &total, scratch);
            if (excl < rem && excl + v0 >= rem) {
                s_digit = 2 * tid;
                s_below = excl;
            } else if (excl + v0 < rem && excl + v0 + v1 >= rem) {
                s_digit = 2 * tid + 1;
                s_below = excl + v0;
            }
            __syncthreads();
            const int d = s_digit;
            rem -= s_below;
            prefix = (prefix << kLruDigit) | (uint64_t)d;
            const int hd = (int)hist[d];
            __syncthreads();
            if (hd == rem) {  // the whole bucket goes: a strict bound suffices
                lt_bound = (prefix + 1) << shift;
                r_eq = 0;
                break;
            }
            if (pass == 0) {
                lt_bound = prefix;
                eq_key = prefix;
                r_eq = rem;
            }
        }
        // ordered collection (slot order) of exactly nM victims
        int c_lt = 0, c_eq = 0;
        for (int s = s0; s < s1; ++s) {
            const int32_t u = lu[s];
            if (u >= t) continue;
            const uint64_t kr = (uint64_t)((uint32_t)(u + 1) - kmin);
            if (kr < lt_bound) ++c_lt;
            else if (r_eq > 0 && kr == eq_key) ++c_eq;
        }
        int eq_total;
        const int eq_before = block_exclusive_scan<kLruThreads>(c_eq, &eq_total, scratch);
        const int take = std::max(0, std::min(c_eq, r_eq - eq_before));
        int sel_total;
        int pos = block_exclusive_scan<kLruThreads>(c_lt + take, &sel_total, scratch);
        int taken = 0;
        for (int s = s0; s < s1; ++s) {
            const int32_t u = lu[s];
            if (u >= t) continue;
            const uint32_t key = (uint32_t)(u + 1);
            const uint64_t kr = (uint64_t)(key - kmin);
            bool sel = kr < lt_bound;
            if (!sel && r_eq > 0 && kr == eq_key && taken < take) {
                sel = true;
                ++taken;
            }
            if (sel && pos < kMaxMerge) vic[pos++] = ((unsigned long long)key << 32) | (unsigned)s;
        }
        // 4. victims in (stamp, slot) order
        const int nv2 = next_pow2(nM);
        for (int i = nM + tid; i < nv2; i += kLruThreads) vic[i] = ~0ull;
        __syncthreads();
        if (range != 0) bitonic_sort_lds(vic, nv2, [](unsigned long long v) { return v; });
        if (tid == 0) s_gbase = atomicAdd(gather_total, (uint32_t)nM);
        __syncthreads();
        // 5. assignment
        const uint32_t gbase = s_gbase;
        int ev_loc = 0;
        // sel_total == nM always holds (S >= D*k); the guards keep a broken
        // invariant from turning into out-of-range stores
        for (int r = tid; r < nM; r += kLruThreads) {
            const uint32_t vu = (uint32_t)vic[r];
            const uint32_t mu = wl[r];
            if (sel_total != nM || vu >= (uint32_t)S || mu >= (uint32_t)cap) {
                cnt[7] = 1;  // invariant violated; reported in the counts record
                continue;
            }
            const int32_t v = (int32_t)vu;
            const int32_t m = (int32_t)mu;
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
            glist[gbase + r] = GatherEntry{(uint32_t)((int64_t)b * cap + m), (uint32_t)((int64_t)b * S + v)};
        }
        int ev_total;
        (void)block_exclusive_scan<kLruThreads>(ev_loc, &ev_total, scratch);
        nEv = ev_total;
    }
    if (tid == 0) {
        cnt[0] = nU; cnt[1] = nU - nM; cnt[2] = nM; cnt[3] = nEv;
        cnt[4] = kk; cnt[5] = (int32_t)Lt; cnt[6] = t;
        atomicAdd(&layer_stats[1], (unsigned long long)nU);
        atomicAdd(&layer_stats[2], (unsigned long long)(nU - nM));
        atomicAdd(&layer_stats[3], (unsigned long long)nM);
        atomicAdd(&layer_stats[4], (unsigned long long)nEv);
        if (b == 0) atomicAdd(&layer_stats[0], 1ull);
    }
}

hipError_t launch_merge_lru(hipStream_t st, const int32_t* topk, const int32_t* ntok_layer,
                            int32_t* cache_slots_layer, int32_t* slot_token_layer,
                            int32_t* last_use_layer, int B, int D, int top_k, int S,
                            int64_t cap, int32_t t, int32_t* misses, int32_t* victims,
                            int32_t* evict_old, int32_t* counts, GatherEntry* glist,
                            uint32_t* gather_total, unsigned long long* layer_stats) {
    hipLaunchKernelGGL(k_merge_lru, dim3(B), dim3(kLruThreads), 0, st, topk, ntok_layer,
                       cache_slots_layer, slot_token_layer, last_use_layer, D, top_k, S, cap, t,
                       misses, victims, evict_old, counts, glist, gather_total, layer_stats);
    return hipGetLastError();
}

}  // namespace sko
