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
// (step stamp, -1 = never used) and the recency list of the slots: every
// slot once, ascending by (last_use, slot), kept as a ring of slot ids.  At
// step t, for one sequence:
//   U = the tokens whose bit is set in the winner bitmap (the union of the
//       D position lists, already deduplicated and in token order);
//   hits are stamped t and their ring entries become tombstones (-1);
//   misses M are listed in token order;
//   victims = the first |M| live entries from the ring head (the least
//       recently used slots that were not hit); the head moves past them;
//   the r-th miss takes the r-th victim; a victim's previous owner (if any)
//   is evicted: cache_slots[old] = -1;
//   the slots stamped t (hits and victims) are appended at the tail in slot
//   order, so the live entries stay sorted by (last_use, slot) without any
//   sort, and a step touches O(|U| + S/32) entries instead of all S.
// When the ring would overflow, its live entries are compacted into the
// other ring buffer first (at most every ~S/|hits| steps).
//
// One 1024-thread block per sequence.  Before the merge it finishes the
// top-k of its D rows whose threshold bucket had to be split (exact radix
// select on the staged candidates); after it, it clears its rows' histograms
// and records for the next step.
#include "sko_common.h"
#include "sko_internal.h"

namespace sko {

constexpr int kLruThreads = 1024;

__device__ __forceinline__ bool is_touched(const uint32_t* touched, int32_t s) {
    return (touched[s >> 5] >> (s & 31)) & 1u;
}

// Staged bucket entries are (key, token | miss << 31): the low word is the
// packed winner value, the token is its low 31 bits.
__device__ __forceinline__ uint64_t refine_composite(uint2 e) {
    return ((uint64_t)(e.x & 0xFFFFFu) << 32) | (uint64_t)(0xFFFFFFFFu - (e.y & 0x7FFFFFFFu));
}

// Exact selection inside split threshold buckets.  For each row whose
// bucket must be split, `need` winners are chosen among its c staged bucket
// keys by radix select, from the top, on the 52-bit composite
// (low 20 key bits) << 32 | (0xFFFFFFFF - token), which is unique per
// candidate (so equal scores go to the smaller token); the result is the
// threshold composite T, and the candidates with composite >= T are
// appended to the row's winners.  Up to 4 rows run at once, one thread
// group each (the block's barriers are shared, every group has its own
// histogram and state; one wave per group scans the 256 bins).
struct RefineGroup {
    uint64_t prefix;
    uint64_t T;
    int rem;
    int done;
    int row;
    int c;
};

__device__ __forceinline__ void refine_rows(int b, int D, RowMeta* __restrict__ meta, const uint2* __restrict__ cand,
                                            int32_t* __restrict__ topk,
                                            uint32_t* __restrict__ wb, int top_k, int64_t cap, uint2* stage,
                                            int stage_cap, uint32_t (*hg)[256], RefineGroup* gs) {
    const int NG = D < 4 ? D : 4;
    const int gsize = (kLruThreads / NG) & ~63;  // whole waves per group
    const int tid = threadIdx.x;
    const int g = tid / gsize;  // < NG, except for leftover threads when NG = 3
    const int gt = tid - g * gsize;
    const int gl = gt & 63;
    const bool in_group = g < NG;
    const int gi = in_group ? g : 0;  // a valid index for threads outside any group
    const int stage_per = stage_cap / NG;
    for (int p0 = 0; p0 < D; p0 += NG) {
        if (in_group && gt == 0) {
            const int p = p0 + g;
            RefineGroup G{0, 0, 0, 1, -1, 0};
            if (p < D) {
                const int row = b * D + p;
                const RowMeta m = meta[row];
                G.row = row;
                if (m.bucket >= 0 && m.need > 0 && m.need != m.bucket_count) {
                    G.rem = m.need;
                    G.done = 0;
                    G.c = (int)std::min<int64_t>(m.cand_count, cap);
                }
            }
            gs[g] = G;
        }
        __syncthreads();
        const RefineGroup G = gs[gi];
        const bool active = in_group && !G.done;
        const uint2* __restrict__ cg = cand + (size_t)(active ? G.row : 0) * cap;
        const bool staged = active && G.c <= stage_per;
        uint2* sg = stage + (size_t)gi * stage_per;
        if (staged)
            for (int i = gt; i < G.c; i += gsize) sg[i] = cg[i];
        __syncthreads();
        int width = 8;
        for (int shift = 44;; shift -= width) {
            if (shift < 0) { width += shift; shift = 0; }
            if (active && gt < 256) hg[g][gt] = 0u;
            __syncthreads();
            const uint64_t gprefix = gs[gi].prefix;
            const int grem = gs[gi].rem;
            const bool gdone = !in_group || gs[gi].done;
            if (!gdone) {
                for (int i = gt; i < G.c; i += gsize) {
                    const uint64_t comp = refine_composite(staged ? sg[i] : cg[i]);
                    if ((comp >> (shift + width)) == gprefix)
                        atomicAdd(&hg[g][(comp >> shift) & ((1u << width) - 1u)], 1u);
                }
            }
            __syncthreads();
            if (gt < 64 && !gdone) {
                // lane gl holds bins 255-4gl .. 252-4gl (descending order)
                uint32_t v[4];
                int sum = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v[j] = hg[g][255 - 4 * gl - j];
                    sum += (int)v[j];
                }
                int incl = sum;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const int y = __shfl_up(incl, o);
                    if (gl >= o) incl += y;
                }
                const int excl = incl - sum;
                if (excl < grem && incl >= grem) {
                    int cacc = excl;
                    for (int j = 0; j < 4; ++j) {
                        const int cnt = (int)v[j];
                        if (cacc + cnt >= grem) {
                            const int d = 255 - 4 * gl - j;
                            const int rem = grem - cacc;
                            const uint64_t prefix = (gprefix << width) | (uint64_t)d;
                            gs[g].prefix = prefix;
                            gs[g].rem = rem;
                            if (cnt == rem || shift == 0) {
                                gs[g].done = 1;
                                gs[g].T = prefix << shift;
                            }
                            break;
                        }
                        cacc += cnt;
                    }
                }
            }
            __syncthreads();
            bool all_done = true;
            for (int q = 0; q < NG; ++q) all_done = all_done && gs[q].done;
            if (all_done || shift == 0) break;
        }
        // emit the bucket winners of each active row
        if (active) {
            const uint64_t T = gs[gi].T;
            for (int base = 0; base < G.c; base += gsize) {
                const int i = base + gt;
                const bool valid = i < G.c;
                const uint2 e = valid ? (staged ? sg[i] : cg[i]) : make_uint2(0u, 0u);
                const bool win = valid && refine_composite(e) >= T;
                const int pw = wave_append(&meta[G.row].out_count, win);
                if (win && pw < top_k) {
                    const uint32_t tok = e.y & 0x7FFFFFFFu;
                    topk[(size_t)G.row * top_k + pw] = (int32_t)e.y;
                    atomicOr(&wb[tok >> 5], 1u << (tok & 31u));
                }
            }
        }
        __syncthreads();
    }
}

constexpr int kBatch = 8;  // 16-byte loads in flight per thread per batch

// Per-thread contiguous run [r0, r1) of n items over the block, with the run
// length rounded up to a multiple of `align`.
__device__ __forceinline__ void thread_run(int64_t n, int align, int64_t* r0, int64_t* r1) {
    int64_t per = (n + kLruThreads - 1) / kLruThreads;
    per = (per + align - 1) / align * align;
    *r0 = std::min<int64_t>(n, (int64_t)threadIdx.x * per);
    *r1 = std::min<int64_t>(n, *r0 + per);
}

// Early miss copy inside the merge launch: blocks past the B merge blocks
// copy, from the pool into the sequence's spare hot rows, the rows of the
// misses marked in the miss bitmap (the union of the miss-flagged winners of
// a sequence is its miss set M; a winner's flag is its absence at step
// start), so the host-link transfer runs while the merge blocks update the
// LRU state.  Copy block j of sequence b takes bitmap words [W j, W j + W):
// it lists their tokens in LDS and copies each row into spare row r of the
// step's generation, where r is the token's rank among the sequence's
// misses in token order (the misses in the words before its own are counted
// first).  The merge blocks of the same launch compute the same ranks from
// their sorted miss list and give the r-th miss's victim slot that spare
// row, so no block waits for another.  The bitmap is left as it is for the
// other blocks' counts (the attention launch clears the words of the
// misses).
// The launch holds about kCopyBlocks copy blocks in all (each block a run
// of up to 1024 bitmap words, one per thread): on this link more blocks,
// i.e. more host reads in flight, lowered the transfer rate (2x the blocks:
// -15 %, 4x: -25 % at long context) and fewer left it idle (small).
constexpr int kCopyBlocks = 64;
// One row in flight per wave (about 1 000 rows over the launch, some 1.2 MB,
// several times the link's bandwidth-delay product).  Two rows per wave
// copied no faster and slowed everything else on the chip more: host reads
// in flight hold the memory system, so the LRU update beside them and any
// kernel on another stream wait longer (one box, layer-steps/s, two rows ->
// one: shelf_ctx8 2 724 -> 2 736, mtp3 1 225 -> 1 243, small 4 989 -> 5 045,
// long 4 335 -> 4 363; with eight waves of one row each the copy itself
// slowed, 270 -> 279 us at shelf_ctx8).
constexpr int kCopyRowsPerWave = 1;
// Kept off an XCD, the copy blocks of two handles' launches share the copy
// XCD; each copies with this many of its waves (one box, layer-steps/s, 16
// waves -> 8: shelf_ctx8 3 291 -> 3 311, small 5 284 -> 5 381; 4 waves lost
// 10 %).
constexpr int kSplitCopyWaves = 8;

__device__ __forceinline__ void copy_block(int cb, int nper, int copy_words, const uint32_t* __restrict__ miss_bits,
                                           const uint4* __restrict__ pool_layer, const uint4* __restrict__ recent_layer,
                                           uint4* __restrict__ hot_layer, const int32_t* __restrict__ spare_layer,
                                           int gen, int R, const int32_t* __restrict__ ntok_layer,
                                           int64_t cap, int64_t wpr, int mstride, int32_t* toks, int toks_cap,
                                           int copy_waves, int* scratch) {
    const int b = cb / nper;
    // this step's spare rows of the sequence (each < R)
    const int32_t* __restrict__ spare = spare_layer + ((size_t)b * 2 + gen) * mstride;
    const int part = cb - b * nper;
    const int64_t words_now = (ntok_layer[b] + 31) / 32;
    const int32_t newest = ntok_layer[b] - 1;  // its row is read from the device copy
    const uint32_t* __restrict__ mb = miss_bits + (size_t)b * wpr;
    // misses before this part (copy_words is a multiple of 4 and rows are
    // 16-byte aligned, so the count reads whole 16-byte words)
    const int64_t w_begin = (int64_t)part * copy_words;
    // no bit is set at or past the sequence's token count (a part may begin
    // there), and the bitmap row holds at least that many words rounded up
    // to 4
    const int64_t w_count = std::min(w_begin, words_now);
    int before = 0;
    for (int64_t q = threadIdx.x; 4 * q < w_count; q += kLruThreads) {
        const uint4 v = reinterpret_cast<const uint4*>(mb)[q];
        before += __popc(v.x) + __popc(v.y) + __popc(v.z) + __popc(v.w);
    }
    int base;
    (void)block_exclusive_scan<kLruThreads>(before, &base, scratch);
    const int64_t wi = w_begin + threadIdx.x;
    uint32_t bits = 0u;
    if ((int)threadIdx.x < copy_words && wi < words_now) bits = mb[wi];
    int total;
    int pos = block_exclusive_scan<kLruThreads>(__popc(bits), &total, scratch);
    if (total == 0) return;  // block-uniform
    // a sequence has at most D*k misses, which toks holds (a larger count
    // would be a broken invariant: the rows past it are not copied)
    total = std::min(total, toks_cap);
    while (bits) {
        const int e = __ffs((int)bits) - 1;
        bits &= bits - 1u;
        if (pos < toks_cap) toks[pos] = (int32_t)(wi * 32 + e);
        ++pos;
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int i0 = wave * kCopyRowsPerWave; wave < copy_waves && i0 < total; i0 += copy_waves * kCopyRowsPerWave) {
        uint4 a[kCopyRowsPerWave], t8[kCopyRowsPerWave];
#pragma unroll
        for (int r = 0; r < kCopyRowsPerWave; ++r) {
            const int i = min(i0 + r, total - 1);  // in range; duplicates are not stored
            const uint4* src = toks[i] == newest ? recent_layer + (int64_t)b * kKvRowU4
                                                 : pool_layer + ((int64_t)b * cap + toks[i]) * kKvRowU4;
            a[r] = src[lane];
            t8[r] = make_uint4(0u, 0u, 0u, 0u);
            if (lane < kKvRowU4 - 64) t8[r] = src[64 + lane];
        }
#pragma unroll
        for (int r = 0; r < kCopyRowsPerWave; ++r) {
            const int i = i0 + r;
            if (i >= total || base + i >= mstride) break;
            const int32_t row = spare[base + i];
            if (row < 0 || row >= R) continue;  // never with intact tables
            uint4* dst = hot_layer + ((int64_t)b * R + row) * kKvRowU4;
            dst[lane] = a[r];
            if (lane < kKvRowU4 - 64) dst[64 + lane] = t8[r];
        }
    }
}

__global__ __launch_bounds__(kLruThreads) void k_merge_lru(
    uint32_t* __restrict__ winners, uint32_t* __restrict__ hist, RowMeta* __restrict__ meta,
    const uint2* __restrict__ cand, int32_t* __restrict__ topk, const int32_t* __restrict__ ntok_layer,
    int32_t* __restrict__ cache_slots_layer, int32_t* __restrict__ slot_token_layer,
    int32_t* __restrict__ last_use_layer, int32_t* __restrict__ ring0_layer, int32_t* __restrict__ ring1_layer,
    int32_t* __restrict__ pos_layer, RingState* __restrict__ ring_state_layer, int D, int top_k, int S,
    int64_t C, int64_t cap, int64_t wpr,
    int32_t t, int32_t* __restrict__ misses, int32_t* __restrict__ victims,
    int32_t* __restrict__ evict_old, int32_t* __restrict__ counts, GatherEntry* __restrict__ glist,
    unsigned long long* __restrict__ layer_stats, int do_refine, int nseq, int copy_per_seq, int copy_words,
    uint32_t* __restrict__ miss_bits, const uint4* __restrict__ pool_layer, const uint4* __restrict__ recent_layer,
    uint4* __restrict__ hot_layer, int32_t* __restrict__ slot_row_layer, int32_t* __restrict__ spare_layer, int R,
    int32_t* __restrict__ wrow, int32_t* __restrict__ phys, int sort_winners,
    int test_violation, uint64_t* __restrict__ stamps, uint4* __restrict__ pool_newest, int ncopy, int xc,
    int tw, int mcap) {
    // instrumentation (stamps != nullptr): each block records when it
    // started and ended on the chip's constant-rate clock, so the host can
    // tell how long the copy blocks ran beside the LRU update
    const uint64_t t_start = stamps ? __builtin_amdgcn_s_memrealtime() : 0ull;
    // Sized for the handle (dynamic LDS, so that at small shelves and one
    // position a block leaves room on its CU for other kernels' blocks):
    //   touched [tw] words: the slots hit or taken at this step (tw >= S/32);
    //   lists [2 mcap] (mcap = D*k): [0, mcap) the misses, [mcap, 2 mcap) the
    //     union, later the victims; before the merge the whole area stages
    //     refine candidates (a copy block lists its part's misses there);
    //   marks [mcap]: per union entry, the positions holding it (sorting).
    extern __shared__ __align__(16) uint32_t lru_lds[];
    uint32_t* const touched = lru_lds;
    int32_t* const lists = reinterpret_cast<int32_t*>(lru_lds + tw);
    uint32_t* const marks = lru_lds + tw + 2 * mcap;
    __shared__ uint32_t hgrp[4][256];
    __shared__ RefineGroup rgrp[4];
    __shared__ int scratch[kLruThreads / 64 + 1];
    __shared__ int64_t s_newhead;
    int32_t* mlist = lists;
    int32_t* ulist = lists + mcap;
    int32_t* vlist = lists + mcap;
    uint2* cstage = reinterpret_cast<uint2*>(lists);

    // the block's part: merge block rb < nseq, or copy block rb - nseq.  Kept
    // off XCD xc (xc >= 0), the copy blocks are the launch's blocks on XCD
    // xc (copy block i / 8 for block i) and the merge blocks are work blocks
    // of the other XCDs, so the host reads never share a CU or an XCD with
    // other kernels' HBM accesses
    int rb = blockIdx.x;
    if (xc >= 0) {
        if (xcc_id() == xc) {
            rb = (int)(blockIdx.x >> 3) < ncopy ? nseq + (int)(blockIdx.x >> 3) : -1;
        } else {
            rb = split_block(blockIdx.x, xc);
            if (rb >= nseq) rb = -1;
        }
        if (rb < 0) return;  // block-uniform
    }
    if (rb >= nseq) {
        copy_block(rb - nseq, copy_per_seq, copy_words, miss_bits, pool_layer, recent_layer, hot_layer,
                   spare_layer, t & 1, R, ntok_layer, cap, wpr, D * top_k, lists, 2 * mcap,
                   xc >= 0 ? kSplitCopyWaves : kLruThreads / 64, scratch);
        if (stamps) {
            __syncthreads();
            if (threadIdx.x == 0) {
                stamps[2 * rb] = t_start;
                stamps[2 * rb + 1] = __builtin_amdgcn_s_memrealtime();
            }
        }
        return;
    }
    const int b = rb;
    const int tid = threadIdx.x;
    const int64_t Lt = ntok_layer[b];
    // the fused append: the newest token's row, which the score launch put in
    // its device copy, also goes to the host pool (no kernel of this step
    // reads it there: every copy takes the newest row from the device copy)
    if (pool_newest != nullptr && Lt > 0 && tid < kKvRowU4)
        pool_newest[((size_t)b * cap + (size_t)(Lt - 1)) * kKvRowU4 + tid] = recent_layer[(size_t)b * kKvRowU4 + tid];
    const int kk = (int)std::min<int64_t>(top_k, Lt);
    int32_t* __restrict__ cs = cache_slots_layer + (size_t)b * cap;
    int32_t* __restrict__ st = slot_token_layer + (size_t)b * S;
    int32_t* __restrict__ lu = last_use_layer + (size_t)b * S;
    int32_t* __restrict__ pos = pos_layer + (size_t)b * S;
    const RingState rs = ring_state_layer[b];
    int32_t* __restrict__ ring = (rs.cur ? ring1_layer : ring0_layer) + (size_t)b * C;
    int32_t* __restrict__ ring_other = (rs.cur ? ring0_layer : ring1_layer) + (size_t)b * C;
    uint32_t* __restrict__ wb = winners + (size_t)b * wpr;
    int32_t* __restrict__ cnt = counts + (size_t)b * 8;
    const int mstride = D * top_k;
    const int SW = (S + 31) / 32;
    // physical hot rows: slot s of the sequence lives in row P[s]; the
    // step's generation of spare rows (rows holding no slot) is Fc, the next
    // step's is Fn (both < R)
    int32_t* __restrict__ P = slot_row_layer + (size_t)b * S;
    const int32_t* __restrict__ Fc = spare_layer + ((size_t)b * 2 + (t & 1)) * mstride;
    int32_t* __restrict__ Fn = spare_layer + ((size_t)b * 2 + ((t & 1) ^ 1)) * mstride;

    // 0. finish the top-k of rows whose threshold bucket is split (unless
    //    k_topk_refine already did)
    if (do_refine) refine_rows(b, D, meta, cand, topk, wb, top_k, cap, cstage, mcap, hgrp, rgrp);

    for (int i = tid; i < SW; i += kLruThreads) touched[i] = 0u;
    if (tid == 0) cnt[7] = 0;
    __syncthreads();

    // 1. the union U in token order from the winner bitmap: each thread owns
    //    a contiguous run of words (16-byte loads, batched); one scan places
    //    every thread's tokens; the bitmap is cleared for the next step
    const int64_t nwords = (Lt + 31) / 32;
    int64_t w0, w1;
    thread_run(nwords, 4, &w0, &w1);
    int nu_loc = 0;
    for (int64_t w = w0; w < w1; w += 4 * kBatch) {
        uint4 v[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q)
            v[q] = (w + 4 * q < w1) ? *reinterpret_cast<const uint4*>(wb + w + 4 * q) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int q = 0; q < kBatch; ++q) nu_loc += __popc(v[q].x) + __popc(v[q].y) + __popc(v[q].z) + __popc(v[q].w);
    }
    int nU;
    int uo = block_exclusive_scan<kLruThreads>(nu_loc, &nU, scratch);
    if (nu_loc) {
        for (int64_t w = w0; w < w1; w += 4) {
            const uint4 v = *reinterpret_cast<const uint4*>(wb + w);
            if ((v.x | v.y | v.z | v.w) == 0u) continue;
            const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 4; ++q)
                for (uint32_t x = wv[q]; x; x &= x - 1u) {
                    if (uo < mcap) ulist[uo] = (int32_t)((w + q) * 32 + (__ffs((int)x) - 1));
                    ++uo;
                }
            *reinterpret_cast<uint4*>(wb + w) = make_uint4(0u, 0u, 0u, 0u);
        }
    }
    __syncthreads();
    nU = std::min(nU, mcap);

    // 1b. (sort_winners, at most 16 positions) each position's winners are
    //     rewritten in token order, so the attention's grouping of rows into
    //     chunks does not depend on the order in which the selection
    //     appended them: every entry finds its token in U (binary search)
    //     and marks it with its position (bit p, and bit 16 + p where the
    //     entry is a miss); a position's list is then U's entries marked p,
    //     placed by one scan.  A position whose marks do not add up to its
    //     count (which a well-formed list never gives) keeps its order.
    //     With one position U is the list itself: step 2 writes it back,
    //     with the residency bit that the selection packed (cs == -1 then
    //     as now, since only this launch changes cs).
    const bool sorted_lists = sort_winners && D <= 16;
    if (sorted_lists && D > 1) {
        for (int i = tid; i < nU; i += kLruThreads) marks[i] = 0u;
        __syncthreads();
        for (int e = tid; e < D * kk; e += kLruThreads) {
            const int p = e / kk;
            const int32_t packed = topk[((size_t)b * D + p) * top_k + (e - p * kk)];
            const int32_t tok = packed & 0x7FFFFFFF;
            int lo = 0, hi = nU;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (ulist[mid] < tok) lo = mid + 1;
                else hi = mid;
            }
            if (lo < nU && ulist[lo] == tok) atomicOr(&marks[lo], (1u << p) | (packed < 0 ? 1u << (16 + p) : 0u));
        }
        __syncthreads();
        int64_t r0, r1;
        thread_run(nU, 1, &r0, &r1);
        for (int p = 0; p < D; ++p) {
            int n_loc = 0;
            for (int64_t u = r0; u < r1; ++u) n_loc += (int)((marks[u] >> p) & 1u);
            int total;
            int o = block_exclusive_scan<kLruThreads>(n_loc, &total, scratch);
            if (total == kk) {
                int32_t* __restrict__ row = topk + ((size_t)b * D + p) * top_k;
                for (int64_t u = r0; u < r1; ++u) {
                    const uint32_t m = marks[u];
                    if ((m >> p) & 1u) row[o++] = ulist[u] | (int32_t)(((m >> (16 + p)) & 1u) << 31);
                }
            }
        }
        __syncthreads();
    }

    // 2. hits and misses: every thread looks up its contiguous run of U at
    //    once; misses listed in token order, hits stamped t and marked
    int64_t u0, u1;
    thread_run(nU, 1, &u0, &u1);
    constexpr int kMaxPer = kMaxMerge / kLruThreads;
    int32_t slot_of[kMaxPer];
    int nm_loc = 0;
#pragma unroll
    for (int q = 0; q < kMaxPer; ++q) {
        slot_of[q] = (u0 + q < u1) ? cs[ulist[u0 + q]] : 0;
    }
#pragma unroll
    for (int q = 0; q < kMaxPer; ++q) nm_loc += (u0 + q < u1 && slot_of[q] < 0) ? 1 : 0;
    if (sorted_lists && D == 1 && nU == kk) {
        int32_t* __restrict__ row = topk + (size_t)b * top_k;
#pragma unroll
        for (int q = 0; q < kMaxPer; ++q)
            if (u0 + q < u1) row[u0 + q] = ulist[u0 + q] | (slot_of[q] == -1 ? (int32_t)0x80000000u : 0);
    }
    int nM;
    int mo = block_exclusive_scan<kLruThreads>(nm_loc, &nM, scratch);
#pragma unroll
    for (int q = 0; q < kMaxPer; ++q) {
        if (u0 + q >= u1) continue;
        const int32_t slot = slot_of[q];
        if (slot < 0) {
            mlist[mo++] = ulist[u0 + q];
        } else if (slot < S) {
            atomicOr(&touched[slot >> 5], 1u << (slot & 31));
            lu[slot] = t;
            const int32_t rp = pos[slot];
            if (rp >= 0 && rp < C) ring[rp] = -1;  // the hit leaves its place in the list
        }
    }
    const int nH = nU - nM;
    __syncthreads();

    int nEv = 0;
    int avail = 0;
    const bool sane = nH + nM <= S;
    if (nM > 0 && sane) {
        // 3. victims: the first nM live ring entries from the head, scanned
        //    in windows of 8 consecutive entries per thread
        int found = 0;
        for (int64_t base = rs.head; found < nM && base < rs.tail; base += 8 * kLruThreads) {
            const int64_t e0 = base + 8 * (int64_t)tid;
            int32_t ent[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) ent[q] = (e0 + q < rs.tail) ? ring[(e0 + q) % C] : -1;
            int c = 0;
#pragma unroll
            for (int q = 0; q < 8; ++q) c += ent[q] >= 0 ? 1 : 0;
            int tot;
            int rank = found + block_exclusive_scan<kLruThreads>(c, &tot, scratch);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                if (ent[q] < 0) continue;
                if (rank < nM) vlist[rank] = ent[q];
                if (rank == nM - 1) s_newhead = e0 + q + 1;
                ++rank;
            }
            found += tot;
        }
        avail = found;
        __syncthreads();
        for (int r = tid; r < nM; r += kLruThreads) {
            const int32_t s = vlist[r];
            if (s >= 0 && s < S) atomicOr(&touched[s >> 5], 1u << (s & 31));
        }
        __syncthreads();
        // 4. assignment: r-th miss -> r-th victim.  The miss's row is spare
        //    row r of this step (where the copy puts it); the victim's old
        //    row becomes spare row r of the next step.
        int ev_loc = 0;
        for (int r = tid; r < nM; r += kLruThreads) {
            const int32_t v = vlist[r];
            const int32_t m = mlist[r];
            if (avail < nM || v < 0 || v >= S || m < 0 || m >= cap) {
                cnt[7] = 1;  // invariant violated; reported in the counts record
                Fn[r] = Fc[r];
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
            const int32_t row = Fc[r];
            Fn[r] = P[v];
            P[v] = row;
            misses[(size_t)b * mstride + r] = m;
            victims[(size_t)b * mstride + r] = v;
            evict_old[(size_t)b * mstride + r] = old;
            glist[(size_t)b * mstride + r] = GatherEntry{(uint32_t)((int64_t)b * cap + m), (uint32_t)((int64_t)b * R + row)};
        }
        int ev_total;
        (void)block_exclusive_scan<kLruThreads>(ev_loc, &ev_total, scratch);
        nEv = ev_total;
    } else if (nM > 0) {
        if (tid == 0) cnt[7] = 1;
    }
    {
        // spare rows no miss took stay spare
        const int taken = (nM > 0 && sane) ? std::min(nM, mstride) : 0;
        for (int r = taken + tid; r < mstride; r += kLruThreads) Fn[r] = Fc[r];
    }
    __syncthreads();

    // 5. ring maintenance: compact if the append would overflow, then append
    //    the slots stamped t (hits and victims) at the tail in slot order
    {
        const bool took = nM > 0 && sane && avail >= nM;
        const int nT = took ? nH + nM : nH;
        int64_t head = took ? s_newhead : rs.head;
        int64_t tail = rs.tail;
        int32_t cur = rs.cur;
        int32_t* rg = ring;
        if ((tail + nT) - head > C) {
            // live entries of [head, tail) -> ring_other[0 ..), in order
            const int64_t R = tail - head;
            int64_t i0, i1;
            thread_run(R, 1, &i0, &i1);
            int lc = 0;
            for (int64_t i = i0; i < i1; ++i) lc += ring[(head + i) % C] >= 0 ? 1 : 0;
            int nlive;
            int64_t lp = block_exclusive_scan<kLruThreads>(lc, &nlive, scratch);
            for (int64_t i = i0; i < i1; ++i) {
                const int32_t sl = ring[(head + i) % C];
                if (sl >= 0 && sl < S && lp < C) {
                    ring_other[lp] = sl;
                    pos[sl] = (int32_t)lp;
                    ++lp;
                }
            }
            head = 0;
            tail = nlive;
            cur ^= 1;
            rg = ring_other;
        }
        int64_t q0, q1;
        thread_run(SW, 1, &q0, &q1);
        int ct = 0;
        for (int64_t q = q0; q < q1; ++q) ct += __popc(touched[q]);
        int ntouched;
        int64_t tp = tail + block_exclusive_scan<kLruThreads>(ct, &ntouched, scratch);
        for (int64_t q = q0; q < q1; ++q) {
            uint32_t bits = touched[q];
            while (bits) {
                const int e = __ffs((int)bits) - 1;
                bits &= bits - 1u;
                const int32_t sl = (int32_t)(q * 32 + e);
                const int64_t ri = tp % C;
                rg[ri] = sl;
                pos[sl] = (int32_t)ri;
                ++tp;
            }
        }
        if (tid == 0) ring_state_layer[b] = RingState{head, tail + ntouched, cur, {0, 0, 0}};
    }

    // 7. the row the attention reads for each winner of this sequence, a
    //    hit's P[slot] or a miss's spare row (-1: none, only with a broken
    //    invariant), and the winner's slot in phys
    if (wrow != nullptr) {
        const bool assigned = nM > 0 && sane && avail >= nM;
        for (int e = tid; e < D * kk; e += kLruThreads) {
            const int p = e / kk;
            const size_t at = ((size_t)b * D + p) * top_k + (e - p * kk);
            const int32_t packed = topk[at];
            const int32_t tok = packed & 0x7FFFFFFF;
            int32_t rd = -1, slot = -1;
            if (packed >= 0) {
                slot = tok < cap ? cs[tok] : -1;
                if (slot >= S) slot = -1;
                rd = slot >= 0 ? P[slot] : -1;
            } else if (assigned) {
                int lo = 0, hi = nM;
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    if (mlist[mid] < tok) lo = mid + 1;
                    else hi = mid;
                }
                if (lo < nM && mlist[lo] == tok && lo < mstride && vlist[lo] >= 0 && vlist[lo] < S) {
                    slot = vlist[lo];
                    rd = Fc[lo];
                }
            }
            wrow[at] = (rd >= 0 && rd < R) ? rd : -1;
            phys[at] = slot;
        }
    }

    // 6. counters (rows that were rescanned); clear this sequence's selection
    // scratch for the next step
    __shared__ int s_rescans;
    if (tid == 0) s_rescans = 0;
    __syncthreads();
    if (tid < D && meta[b * D + tid].pre_count < kk) atomicAdd(&s_rescans, 1);
    __syncthreads();
    for (int i = tid; i < D * kHistBins; i += kLruThreads) hist[(size_t)b * D * kHistBins + i] = 0u;
    if (tid < D) meta[b * D + tid] = RowMeta{-1, 0, 0, 0, 0, 0, 0, 0};
    if (tid == 0) {
        if (s_rescans) atomicAdd(&layer_stats[5], (unsigned long long)s_rescans);
        // the newest token is never resident before its first step, so it
        // holds a slot now exactly when it was a miss; its row comes from
        // the device copy of the newest row, not over the host link
        if (Lt > 0 && cs[Lt - 1] >= 0) atomicAdd(&layer_stats[6], 1ull);
        cnt[0] = nU; cnt[1] = nH; cnt[2] = nM; cnt[3] = nEv;
        cnt[4] = kk; cnt[5] = (int32_t)Lt; cnt[6] = t;
        // a broken residency invariant (a miss without a victim, or a slot
        // or token out of range) is counted per layer, and the host refuses
        // further reads of the handle; the test switch raises the flag for
        // sequence 0 without changing any other work
        if (test_violation && b == 0) cnt[7] = 1;
        if (cnt[7]) atomicAdd(&layer_stats[7], 1ull);
        atomicAdd(&layer_stats[1], (unsigned long long)nU);
        atomicAdd(&layer_stats[2], (unsigned long long)nH);
        atomicAdd(&layer_stats[3], (unsigned long long)nM);
        atomicAdd(&layer_stats[4], (unsigned long long)nEv);
    }
    if (stamps) {
        __syncthreads();
        if (tid == 0) {
            stamps[2 * b] = t_start;
            stamps[2 * b + 1] = __builtin_amdgcn_s_memrealtime();
        }
    }
}

int merge_lru_touched_words(int S) { return ((S + 31) / 32 + 3) / 4 * 4; }

size_t merge_lru_lds_bytes(int S, int D, int top_k) {
    return 4 * ((size_t)merge_lru_touched_words(S) + 3 * (size_t)D * top_k);
}

hipError_t prepare_merge_lru(size_t lds_bytes) {
    // the attribute is the kernel's limit for every launch: it is set to the
    // largest size any handle can need (S and D*k at their limits), never
    // lowered
    const size_t most = merge_lru_lds_bytes(kMaxHotSlots, 1, kMaxMerge);
    if (lds_bytes > most) return hipErrorInvalidValue;
    return hipFuncSetAttribute(reinterpret_cast<const void*>(&k_merge_lru), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)most);
}

void copy_shape(int B, int64_t max_tokens_now, int* copy_per_seq, int* copy_words, int xcd_cus) {
    const int64_t words = std::max<int64_t>(1, (max_tokens_now + 31) / 32);
    if (xcd_cus > 0) {
        // the copy blocks of one XCD: about one per CU, each part at most
        // kLruThreads words and, unless that forces more, at least 32
        *copy_per_seq = (int)std::max<int64_t>(
            (words + kLruThreads - 1) / kLruThreads,
            std::min<int64_t>((xcd_cus + B - 1) / B, (words + 31) / 32));
    } else {
        const int64_t max_words =
            std::min<int64_t>(kLruThreads, std::max<int64_t>(32, (B * words + kCopyBlocks - 1) / kCopyBlocks));
        *copy_per_seq = (int)((words + max_words - 1) / max_words);
    }
    // equal parts (a remainder part would hold few tokens and leave its
    // block nearly idle while the others carry its share)
    *copy_words = (int)(((words + *copy_per_seq - 1) / *copy_per_seq + 3) / 4 * 4);
}

hipError_t launch_merge_lru(hipStream_t st, uint32_t* winners, uint32_t* hist, RowMeta* meta,
                            const uint2* cand, int32_t* topk, const int32_t* ntok_layer,
                            int32_t* cache_slots_layer, int32_t* slot_token_layer,
                            int32_t* last_use_layer, int32_t* ring0_layer, int32_t* ring1_layer,
                            int32_t* pos_layer, RingState* ring_state_layer,
                            int B, int D, int top_k, int S, int64_t cap, int32_t t,
                            int32_t* misses, int32_t* victims, int32_t* evict_old, int32_t* counts,
                            GatherEntry* glist, unsigned long long* layer_stats, bool do_refine,
                            uint32_t* miss_bits, const uint16_t* pool_layer, const uint16_t* recent_layer,
                            uint16_t* hot_layer, int32_t* slot_row_layer, int32_t* spare_layer, int R,
                            int32_t* wrow, int32_t* phys, bool sort_winners,
                            int64_t max_tokens_now, bool test_violation, uint64_t* stamps,
                            uint16_t* pool_newest, int xc, int xcd_cus) {
    const int64_t C = ring_capacity(S, D, top_k);
    const int64_t wpr = winner_words(cap);
    // B merge blocks, then (early copy) B * copy_per_seq copy blocks of
    // copy_words bitmap words each (a multiple of 4), about kCopyBlocks in all
    int copy_per_seq = 0, copy_words = 0;
    copy_shape(B, max_tokens_now, &copy_per_seq, &copy_words, xc >= 0 ? xcd_cus : 0);
    if (!miss_bits) copy_per_seq = 0;
    const int ncopy = B * copy_per_seq;
    const int tw = merge_lru_touched_words(S);
    const size_t lds = merge_lru_lds_bytes(S, D, top_k);
    // kept off XCD xc: the copy blocks are the blocks on it, one per group
    // of 8, and the merge blocks are work blocks of the other seven
    const unsigned grid = xc < 0 ? (unsigned)(B + ncopy)
                                 : (unsigned)(kXcds * std::max<int64_t>(ncopy, (B + kXcds - 2) / (kXcds - 1)));
    hipLaunchKernelGGL(k_merge_lru, dim3(grid), dim3(kLruThreads), lds, st, winners, hist, meta, cand, topk,
                       ntok_layer, cache_slots_layer, slot_token_layer, last_use_layer, ring0_layer,
                       ring1_layer, pos_layer, ring_state_layer, D, top_k, S, C, cap, wpr, t, misses, victims,
                       evict_old, counts, glist, layer_stats, do_refine ? 1 : 0, B, copy_per_seq, copy_words,
                       miss_bits,
                       reinterpret_cast<const uint4*>(pool_layer), reinterpret_cast<const uint4*>(recent_layer),
                       reinterpret_cast<uint4*>(hot_layer), slot_row_layer, spare_layer, R, wrow, phys,
                       sort_winners ? 1 : 0, test_violation ? 1 : 0, stamps, reinterpret_cast<uint4*>(pool_newest),
                       ncopy, xc, tw, D * top_k);
    return hipGetLastError();
}

// Exact selection inside the split threshold bucket of one row per block
// (256 threads), as refine_rows does inside the merge kernel: radix select
// from the top on the 52-bit composite, 8 bits per pass, over the staged
// bucket entries (in LDS when they fit); the entries with composite >= T
// are appended to the row's winners and marked in the winner bitmap, and
// in the miss bitmap when they are absent from the hot buffer.  The filter
// launch has completed, so the row's winner count is final: a staged row
// places its winners with one block scan (no global atomics), and its
// entries are loaded all at once, before the row's counts are known
// (clamped to the row, which holds cap entries).
constexpr int kRefineThreads = 256;
constexpr int kRefinePer = 16;
constexpr int kRefineStage = kRefineThreads * kRefinePer;

__global__ __launch_bounds__(kRefineThreads) void k_topk_refine(RowMeta* __restrict__ meta,
                                                                const uint2* __restrict__ cand,
                                                                int32_t* __restrict__ topk,
                                                                uint32_t* __restrict__ winners,
                                                                uint32_t* __restrict__ miss_bits, int D,
                                                                int top_k, int64_t cap, int64_t wpr, int nrows,
                                                                int xc) {
    __shared__ uint2 sg[kRefineStage];
    __shared__ uint32_t hg[256];
    __shared__ uint64_t s_prefix, s_T;
    __shared__ int s_rem, s_done;
    __shared__ int scratch[kRefineThreads / 64 + 1];
    const int row = split_block(blockIdx.x, xc);
    if (row < 0 || row >= nrows) return;  // block-uniform
    const int b = row / D;
    const int tid = threadIdx.x, lane = tid & 63;
    const uint2* __restrict__ cg = cand + (size_t)row * cap;
    uint2 pre[kRefinePer];
#pragma unroll
    for (int j = 0; j < kRefinePer; ++j) {
        const int64_t i = tid + (int64_t)kRefineThreads * j;
        pre[j] = cg[i < cap ? i : cap - 1];
    }
    const RowMeta m = meta[row];
    if (m.bucket < 0 || m.need <= 0 || m.need == m.bucket_count) return;  // block-uniform
    const int c = (int)std::min<int64_t>(m.cand_count, cap);
    const bool staged = c <= kRefineStage;
    if (staged) {
#pragma unroll
        for (int j = 0; j < kRefinePer; ++j) {
            const int i = tid + kRefineThreads * j;
            if (i < c) sg[i] = pre[j];
        }
    }
    if (tid == 0) {
        s_prefix = 0;
        s_T = 0;
        s_rem = m.need;
        s_done = 0;
    }
    __syncthreads();
    int width = 8;
    for (int shift = 44;; shift -= width) {
        if (shift < 0) {
            width += shift;
            shift = 0;
        }
        hg[tid] = 0u;
        __syncthreads();
        const uint64_t prefix = s_prefix;
        const int rem = s_rem;
        for (int i = tid; i < c; i += kRefineThreads) {
            const uint64_t comp = refine_composite(staged ? sg[i] : cg[i]);
            if ((comp >> (shift + width)) == prefix) atomicAdd(&hg[(comp >> shift) & ((1u << width) - 1u)], 1u);
        }
        __syncthreads();
        if (tid < 64) {
            // lane holds bins 255-4l .. 252-4l (descending order)
            uint32_t v[4];
            int sum = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[j] = hg[255 - 4 * lane - j];
                sum += (int)v[j];
            }
            int incl = sum;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(incl, o);
                if (lane >= o) incl += y;
            }
            const int excl = incl - sum;
            if (excl < rem && incl >= rem) {
                int cacc = excl;
                for (int j = 0; j < 4; ++j) {
                    const int cnt = (int)v[j];
                    if (cacc + cnt >= rem) {
                        const int d = 255 - 4 * lane - j;
                        const uint64_t np = (prefix << width) | (uint64_t)d;
                        s_prefix = np;
                        s_rem = rem - cacc;
                        if (cnt == rem - cacc || shift == 0) {
                            s_done = 1;
                            s_T = np << shift;
                        }
                        break;
                    }
                    cacc += cnt;
                }
            }
        }
        __syncthreads();
        if (s_done || shift == 0) break;
    }
    const uint64_t T = s_T;
    uint32_t* __restrict__ wb = winners + (size_t)b * wpr;
    uint32_t* __restrict__ mb = miss_bits ? miss_bits + (size_t)b * wpr : nullptr;
    auto take = [&](uint2 e, int pw) {
        const uint32_t tok = e.y & 0x7FFFFFFFu;
        if (pw < top_k) topk[(size_t)row * top_k + pw] = (int32_t)e.y;
        atomicOr(&wb[tok >> 5], 1u << (tok & 31u));
        if (mb && (e.y & 0x80000000u)) atomicOr(&mb[tok >> 5], 1u << (tok & 31u));
    };
    if (staged) {
        uint32_t wmask = 0u;
#pragma unroll
        for (int j = 0; j < kRefinePer; ++j) {
            const int i = tid + kRefineThreads * j;
            if (i < c && refine_composite(pre[j]) >= T) wmask |= 1u << j;
        }
        int total;
        int pw = m.out_count + block_exclusive_scan<kRefineThreads>(__popc(wmask), &total, scratch);
#pragma unroll
        for (int j = 0; j < kRefinePer; ++j)
            if ((wmask >> j) & 1u) take(pre[j], pw++);
        if (tid == 0) meta[row].out_count = m.out_count + total;
        return;
    }
    for (int base = 0; base < c; base += kRefineThreads) {
        const int i = base + tid;
        const bool valid = i < c;
        const uint2 e = valid ? cg[i] : make_uint2(0u, 0u);
        const bool win = valid && refine_composite(e) >= T;
        const int pw = wave_append(&meta[row].out_count, win);
        if (win) take(e, pw);
    }
}

hipError_t launch_topk_refine(hipStream_t st, RowMeta* meta, const uint2* cand, int32_t* topk, uint32_t* winners,
                              uint32_t* miss_bits, int B, int D, int top_k, int64_t cap, int xc) {
    hipLaunchKernelGGL(k_topk_refine, dim3(split_grid(B * D, xc)), dim3(kRefineThreads), 0, st, meta, cand, topk,
                       winners, miss_bits, D, top_k, cap, winner_words(cap), B * D, xc);
    return hipGetLastError();
}

__global__ void k_init_rings(int32_t* __restrict__ ring0, int32_t* __restrict__ pos,
                             RingState* __restrict__ state, int32_t* __restrict__ slot_row,
                             int32_t* __restrict__ spare, int64_t n_seqs, int S, int64_t C, int M) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (int64_t i = i0; i < n_seqs * C; i += stride) {
        const int64_t e = i % C;
        ring0[i] = e < S ? (int32_t)e : -1;
    }
    for (int64_t i = i0; i < n_seqs * S; i += stride) {
        pos[i] = (int32_t)(i % S);
        slot_row[i] = (int32_t)(i % S);  // slot s in row s
    }
    // both generations of spare rows: rows S .. S+M-1
    for (int64_t i = i0; i < n_seqs * 2 * M; i += stride) spare[i] = S + (int32_t)(i % M);
    for (int64_t i = i0; i < n_seqs; i += stride) state[i] = RingState{0, S, 0, {0, 0, 0}};
}

hipError_t launch_init_rings(hipStream_t st, int32_t* ring0, int32_t* pos, RingState* state, int32_t* slot_row,
                             int32_t* spare, int64_t n_seqs, int S, int64_t C, int M) {
    const int g = (int)std::min<int64_t>((n_seqs * C + 255) / 256, 4096);
    hipLaunchKernelGGL(k_init_rings, dim3(std::max(g, 1)), dim3(256), 0, st, ring0, pos, state, slot_row, spare,
                       n_seqs, S, C, M);
    return hipGetLastError();
}

}  // namespace sko
