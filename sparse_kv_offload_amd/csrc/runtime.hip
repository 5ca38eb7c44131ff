// Host runtime of libsko: the C ABI declared in include/sko.h.
//
// Owns the offload state of "Layerwise and Sparse KV Cache Offloading
// Design" section 4 ("Memory layout"): the full main-KV history in a pinned,
// device-mapped host pool; the indexer cache and the per-layer hot buffers
// in device memory; and the residency tables.  Every call validates all of
// its arguments before touching state (section 7 of the same page: a layout
// mismatch fails instead of leaving partial data); a HIP failure marks the
// handle FAILED so that later calls refuse instead of computing on corrupt
// state.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/sko.h"
#include "sko_common.h"
#include "sko_internal.h"

using namespace sko;

namespace {

constexpr int64_t kStagingRows = 65536;  // indexer rows per host-append piece
constexpr int kMaxCopySpans = 1 << 16;  // copy spans kept between two sko_set_timing calls
constexpr int kStampLaunches = 1024;     // timed LRU-update launches recorded between reads

thread_local std::string g_err;

int set_err(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int set_err(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

}  // namespace

namespace sko {
// The library's last error message (also for the prefill calls).
int set_error(int code, const char* msg) {
    g_err = msg;
    return code;
}
}  // namespace sko

namespace {

enum Stage {
    ST_APPEND = 0,
    ST_SCORE,
    ST_FILTER,
    ST_MERGE_LRU,
    ST_GATHER,
    ST_ATTN,
    ST_COMBINE,
    ST_REFINE,
    ST_ATTN_HITS,
    ST_COUNT
};
const char* const kStageNames[ST_COUNT] = {"append_rows",   "score_hist",   "topk_filter",  "merge_lru",
                                           "gather_misses", "attn_partial", "attn_combine", "topk_refine",
                                           "attn_hits"};

struct DeviceGuard {
    int prev = -1;
    bool ok = false;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) prev = -1;
        ok = hipSetDevice(dev) == hipSuccess;
    }
    ~DeviceGuard() {
        if (prev >= 0) (void)hipSetDevice(prev);
    }
};

}  // namespace

struct sko_handle {
    sko_config cfg{};
    hipStream_t stream = nullptr;
    bool failed = false;
    int L = 0, B = 0, k = 0, S = 0, D = 0, H = 0, HG = 0;
    int64_t cap = 0;
    int64_t ntiles = 0;  // indexer tiles of 64 tokens per sequence
    int64_t kcap = 0;    // key row stride (cap rounded up to 16)
    int64_t C = 0;       // recency ring capacity per sequence
    int64_t wpr = 0;     // winner-bitmap words per sequence

    // offload state
    uint16_t* pool_host = nullptr;  // pinned [L][B][cap][576]
    uint16_t* pool_dev = nullptr;   // device mapping of pool_host
    uint16_t* idx = nullptr;        // [L][B][ntiles][8][64] x 16 B (tiled); int8 indexer: [L][B][ntiles][4][64] x 16 B
    uint16_t* idx_scale = nullptr;  // int8 indexer: fp16 scales [L][B][ntiles * 64]
    uint32_t* qc8 = nullptr;        // int8 indexer: quantized queries [B][D][kQc8Words]
    bool c8 = false;                // the int8 indexer (SKO_FLAG_INDEXER_C8)
    // SKO_FLAG_HIT_OVERLAP: the attention over resident rows runs on `side`
    // (forked from the caller's stream after the selection, joined before
    // the combine) beside the copy launch
    bool hit_overlap = false;
    hipStream_t side = nullptr;
    hipEvent_t ev_fork = nullptr, ev_join = nullptr;
    hipEvent_t ev_switch = nullptr;  // orders the old stream's work before the new one's (sko_set_stream)
    uint16_t* staging = nullptr;    // device rows for host-source appends
    // hot rows: [L][B][R][576], R = S + D*k; slot s of (layer, seq) lives in
    // row slot_row[s], the other D*k rows are spare (two generations of the
    // spare list, the step's one chosen by the layer's step stamp)
    uint16_t* hot = nullptr;
    int R = 0;                      // physical rows per (layer, seq)
    int M = 0;                      // spare rows per (layer, seq) = D*k
    int32_t* slot_row = nullptr;    // [L][B][S]
    int32_t* spare_rows = nullptr;  // [L][B][2][M]
    uint16_t* recent = nullptr;     // [L][B][576] device copy of each sequence's newest main-KV row
    int32_t* cache_slots = nullptr; // [L][B][cap]
    int32_t* slot_token = nullptr;  // [L][B][S]
    int32_t* last_use = nullptr;    // [L][B][S]
    int32_t* ring[2] = {nullptr, nullptr};  // [L][B][C] recency rings (one live per sequence)
    int32_t* ring_pos = nullptr;            // [L][B][S] ring index of each slot
    RingState* ring_state = nullptr;        // [L][B]
    // [L][2][B] device token counts, two buffers per layer: ntok_sel[layer]
    // picks the current one.  The fused append and decode step reads the
    // current buffer in its score launch, which writes the counts after the
    // append into the other buffer; the step's later kernels read that one,
    // and the host then flips ntok_sel, so no kernel reads a count that
    // another kernel of the same launch writes.
    int32_t* ntok_dev = nullptr;
    std::vector<uint8_t> ntok_sel;  // [L]
    unsigned long long* stats = nullptr;  // [L][8]
    std::vector<int64_t> ntok;      // host mirror [L][B]
    std::vector<int32_t> step;      // [L]

    // per-step scratch (shared by all layers; steps are stream-ordered)
    uint32_t* keys = nullptr;       // [B][D][kcap], only with SKO_FLAG_KEEP_KEYS
    uint2* pre = nullptr;           // [B][D][cap] candidates at or above the floor
    // early miss copy: copy blocks of the merge launch copy the misses into
    // their spare hot rows while the merge blocks update the LRU state
    bool fused_copy = false;        // the attention launch copies the misses
    bool staged_copy = false;       // early copy (copy blocks in the LRU-update launch)
    uint32_t* miss_bits = nullptr;  // [B][wpr]
    int32_t* wrow = nullptr;        // [B][D][k]: per winner, the row the attention reads (not with the fused copy)
    int32_t* floor = nullptr;       // [L][B][D] candidate floor (first-digit bin)
    uint32_t* hist = nullptr;       // [B][D][4096]
    RowMeta* meta = nullptr;        // [B][D]
    uint2* cand = nullptr;          // [B][D][cap]
    uint32_t* winners = nullptr;    // [B][wpr] bitmap of this step's winners
    int32_t* topk = nullptr;        // [B][D][k]
    int32_t* phys = nullptr;        // [B][D][k]
    int32_t* misses = nullptr;      // [B][D*k]
    int32_t* victims = nullptr;     // [B][D*k]
    int32_t* evict_old = nullptr;   // [B][D*k]
    int32_t* counts = nullptr;      // [B][8]
    GatherEntry* glist = nullptr;   // [B*D*k]
    float* part_acc = nullptr;      // [B*D][HG][nchunk][16][512]
    float* part_ml = nullptr;       // [B*D][HG][nchunk][16][2]
    int rows_per_block = 32, nchunk = 1;
    int cu_count = 256;  // compute units of the device (launch sizing)
    // SKO_FLAG_XCD_SPLIT: the XCD of the copy blocks (every other block of
    // the step stays off it) and its CUs; -1 / 0 without the flag
    int xc = -1;
    int xcd_cus = 0;
    int last_layer = -1;

    // timing
    uint32_t timing_mask = 0;
    struct Pending {
        int stage;
        hipEvent_t a, b;
    };
    std::vector<Pending> pending;
    std::vector<hipEvent_t> spare;
    double total_ms[ST_COUNT] = {};
    int64_t launches[ST_COUNT] = {};
    // block start / end stamps of timed LRU-update launches (early copy):
    // [kStampLaunches][stamp_blocks][2] on the device clock
    uint64_t* stamps = nullptr;
    int stamp_blocks = 0;        // most blocks one LRU-update launch can hold
    int stamp_next = 0;
    struct StampLaunch {
        int slot, nmerge, nblocks;
    };
    std::vector<StampLaunch> stamp_pending;
    double clock_khz = 100000.0;  // device wall clock (s_memrealtime)
    double ovl_copy_ms = 0.0, ovl_merge_ms = 0.0, ovl_both_ms = 0.0;
    int64_t ovl_launches = 0;
    // the copy span (first copy block's start, last copy block's end) of each
    // recorded launch, on the device clock, in recording order
    std::vector<uint64_t> copy_spans;

    std::vector<void*> dev_allocs;

    size_t lb(int layer, int b) const { return (size_t)layer * B + b; }
    int32_t* ntok_buf(int layer, int which) const { return ntok_dev + ((size_t)layer * 2 + which) * B; }
    // indexer cache bytes of one (layer, seq): 128 B (bf16) or 64 B (int8) per token slot
    size_t idx_seq_bytes() const { return (size_t)ntiles * kIdxTile * (c8 ? kIdxDim : kIdxDim * 2); }
};

namespace {

int device_fail(sko_handle* h, hipError_t e, const char* what) {
    if (h) h->failed = true;
    return set_err(SKO_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool dev_alloc(sko_handle* h, void** p, size_t bytes) {
    *p = nullptr;
    if (bytes == 0) bytes = 16;
    if (hipMalloc(p, bytes) != hipSuccess) {
        *p = nullptr;
        (void)hipGetLastError();
        return false;
    }
    h->dev_allocs.push_back(*p);
    return true;
}

void free_all(sko_handle* h) {
    for (auto& p : h->pending) {
        (void)hipEventDestroy(p.a);
        (void)hipEventDestroy(p.b);
    }
    for (auto e : h->spare) (void)hipEventDestroy(e);
    if (h->ev_fork) (void)hipEventDestroy(h->ev_fork);
    if (h->ev_join) (void)hipEventDestroy(h->ev_join);
    if (h->ev_switch) (void)hipEventDestroy(h->ev_switch);
    h->ev_switch = nullptr;
    if (h->side) (void)hipStreamDestroy(h->side);
    h->ev_fork = h->ev_join = nullptr;
    h->side = nullptr;
    for (void* p : h->dev_allocs) (void)hipFree(p);
    if (h->pool_host) (void)hipHostFree(h->pool_host);
    h->dev_allocs.clear();
    h->pool_host = nullptr;
}

hipEvent_t take_event(sko_handle* h) {
    if (!h->spare.empty()) {
        hipEvent_t e = h->spare.back();
        h->spare.pop_back();
        return e;
    }
    // Timing-only events: the totals are read after a stream synchronize, so
    // the event needs no system-scope fence (which would write back and
    // invalidate caches between the kernels it brackets).
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    return e;
}

// Launch one stage on `st` (default: the handle's stream), bracketed by
// events when timing is on.
template <typename F>
int run_stage(sko_handle* h, int stage, F&& launch, hipStream_t st) {
    hipEvent_t a = nullptr, b = nullptr;
    const bool timed = (h->timing_mask >> stage) & 1u;
    if (timed) {
        a = take_event(h);
        b = take_event(h);
        if (a) (void)hipEventRecord(a, st);
    }
    hipError_t e = launch();
    if (e != hipSuccess) return device_fail(h, e, kStageNames[stage]);
    if (timed && a && b) {
        (void)hipEventRecord(b, st);
        h->pending.push_back({stage, a, b});
    }
    return SKO_OK;
}
template <typename F>
int run_stage(sko_handle* h, int stage, F&& launch) {
    return run_stage(h, stage, static_cast<F&&>(launch), h->stream);
}

int check_handle(sko_handle* h) {
    if (!h) return set_err(SKO_E_INVAL, "NULL handle");
    if (h->failed) return set_err(SKO_E_STATE, "handle is FAILED after an earlier device error or a broken invariant");
    return SKO_OK;
}

// After a stream synchronize: fold the recorded block stamps of timed
// LRU-update launches into the overlap totals.  Per launch, the copy span
// runs from the first copy block's start to the last one's end, the merge
// span likewise over the merge blocks, and the overlap is their
// intersection.
int collect_stamps(sko_handle* h) {
    if (h->stamp_pending.empty()) return SKO_OK;
    std::vector<uint64_t> v((size_t)h->stamp_blocks * 2);
    for (const auto& p : h->stamp_pending) {
        const hipError_t e = hipMemcpy(v.data(), h->stamps + (size_t)p.slot * h->stamp_blocks * 2,
                                       (size_t)p.nblocks * 2 * 8, hipMemcpyDeviceToHost);
        if (e != hipSuccess) return device_fail(h, e, "read block stamps");
        uint64_t m0 = ~0ull, m1 = 0, c0 = ~0ull, c1 = 0;
        for (int i = 0; i < p.nblocks; ++i) {
            const uint64_t a = v[2 * (size_t)i], b = v[2 * (size_t)i + 1];
            if (i < p.nmerge) {
                m0 = std::min(m0, a);
                m1 = std::max(m1, b);
            } else {
                c0 = std::min(c0, a);
                c1 = std::max(c1, b);
            }
        }
        if (p.nblocks <= p.nmerge || m1 < m0 || c1 < c0) continue;
        const double tick_ms = 1.0 / h->clock_khz;
        h->ovl_copy_ms += (double)(c1 - c0) * tick_ms;
        h->ovl_merge_ms += (double)(m1 - m0) * tick_ms;
        const uint64_t lo = std::max(m0, c0), hi = std::min(m1, c1);
        h->ovl_both_ms += hi > lo ? (double)(hi - lo) * tick_ms : 0.0;
        h->ovl_launches += 1;
        if (h->copy_spans.size() < 2 * (size_t)kMaxCopySpans) {
            h->copy_spans.push_back(c0);
            h->copy_spans.push_back(c1);
        }
    }
    h->stamp_pending.clear();
    return SKO_OK;
}

// After a stream synchronize: a merge launch that found a residency
// invariant broken (a miss without a victim, a slot or token out of range)
// counted it in its layer's statistics.  The results of that step are
// incomplete, so the handle is marked FAILED and the read is refused.
int check_invariants(sko_handle* h) {
    std::vector<unsigned long long> v((size_t)h->L * 8);
    const hipError_t e = hipMemcpy(v.data(), h->stats, v.size() * 8, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return device_fail(h, e, "read invariant flags");
    for (int l = 0; l < h->L; ++l)
        if (v[(size_t)l * 8 + 7] != 0) {
            h->failed = true;
            return set_err(SKO_E_STATE,
                           "layer %d: %llu sequence-steps broke a residency invariant (a miss without a "
                           "victim, or a slot or token out of range); the handle is FAILED",
                           l, v[(size_t)l * 8 + 7]);
        }
    return SKO_OK;
}

int validate_config(const sko_config* c) {
    if (!c) return set_err(SKO_E_INVAL, "NULL config");
    if (c->index_dim != SKO_INDEX_DIM || c->kv_dim != SKO_KV_DIM || c->v_dim != SKO_V_DIM)
        return set_err(SKO_E_INVAL, "row shapes must be index_dim=64, kv_dim=576, v_dim=512 (got %d/%d/%d)",
                       c->index_dim, c->kv_dim, c->v_dim);
    if (c->num_layers < 1 || c->batch < 1 || c->num_heads < 1 || c->top_k < 1 || c->mtp_positions < 1)
        return set_err(SKO_E_INVAL, "num_layers, batch, num_heads, top_k, mtp_positions must be >= 1");
    if (c->max_tokens < 1 || c->max_tokens >= 0x7FFFFFFFLL)
        return set_err(SKO_E_INVAL, "max_tokens must be in [1, 2^31-1)");
    if ((int64_t)c->hot_slots < (int64_t)c->mtp_positions * c->top_k)
        return set_err(SKO_E_INVAL, "hot_slots (%d) must be >= mtp_positions*top_k (%lld)", c->hot_slots,
                       (long long)c->mtp_positions * c->top_k);
    if (!(c->attn_scale > 0.0f) || !std::isfinite(c->attn_scale))
        return set_err(SKO_E_INVAL, "attn_scale must be finite and > 0");
    if ((c->flags & ~(SKO_FLAG_POOL_COHERENT | SKO_FLAG_POOL_NONCOHERENT | SKO_FLAG_KEEP_KEYS |
                      SKO_FLAG_SELECT_RESCAN | SKO_FLAG_FUSED_COPY | SKO_FLAG_LATE_COPY |
                      SKO_FLAG_EARLY_COPY | SKO_FLAG_INDEXER_C8 | SKO_FLAG_HIT_OVERLAP |
                      SKO_FLAG_TEST_VIOLATION | SKO_FLAG_XCD_SPLIT)) != 0 ||
        (c->flags & (SKO_FLAG_POOL_COHERENT | SKO_FLAG_POOL_NONCOHERENT)) ==
            (SKO_FLAG_POOL_COHERENT | SKO_FLAG_POOL_NONCOHERENT))
        return set_err(SKO_E_INVAL, "unknown or conflicting flags 0x%x", c->flags);
    {
        const uint32_t modes = c->flags & (SKO_FLAG_FUSED_COPY | SKO_FLAG_LATE_COPY | SKO_FLAG_EARLY_COPY);
        if (modes & (modes - 1))
            return set_err(SKO_E_INVAL, "at most one of SKO_FLAG_FUSED_COPY, _LATE_COPY, _EARLY_COPY");
        if ((modes & SKO_FLAG_FUSED_COPY) && (c->mtp_positions != 1 || c->num_heads > kAttnHeadGroup))
            return set_err(SKO_E_INVAL, "SKO_FLAG_FUSED_COPY needs mtp_positions == 1 and num_heads <= %d",
                           kAttnHeadGroup);
        if ((c->flags & SKO_FLAG_HIT_OVERLAP) && (modes & (SKO_FLAG_FUSED_COPY | SKO_FLAG_LATE_COPY)))
            return set_err(SKO_E_INVAL, "SKO_FLAG_HIT_OVERLAP needs the early copy");
        if ((c->flags & SKO_FLAG_XCD_SPLIT) &&
            ((modes & (SKO_FLAG_FUSED_COPY | SKO_FLAG_LATE_COPY)) || (c->flags & SKO_FLAG_HIT_OVERLAP)))
            return set_err(SKO_E_INVAL, "SKO_FLAG_XCD_SPLIT needs the early copy without SKO_FLAG_HIT_OVERLAP");
    }
    if (c->device < 0) return set_err(SKO_E_INVAL, "device must be >= 0");
    if (c->hot_slots > kMaxHotSlots)
        return set_err(SKO_E_UNSUPPORTED, "hot_slots above %d", kMaxHotSlots);
    if ((int64_t)c->mtp_positions * c->top_k > SKO_MAX_MERGE)
        return set_err(SKO_E_UNSUPPORTED, "mtp_positions*top_k above %d", SKO_MAX_MERGE);
    if ((int64_t)c->batch * c->max_tokens >= 0xFFFFFFFFLL || (int64_t)c->batch * c->hot_slots >= 0xFFFFFFFFLL)
        return set_err(SKO_E_UNSUPPORTED, "batch*max_tokens and batch*hot_slots must stay below 2^32");
    // the hot rows of every layer (S slot rows and D*k spare rows per
    // sequence) are addressed by int32 row numbers
    if ((int64_t)c->num_layers * c->batch * ((int64_t)c->hot_slots + (int64_t)c->mtp_positions * c->top_k) >=
        0x7FFFFFFFLL)
        return set_err(SKO_E_UNSUPPORTED, "num_layers*batch*(hot_slots + mtp_positions*top_k) must stay below 2^31");
    return SKO_OK;
}

int attn_rows_per_block(int k, int rows_total_pairs) {
    // Two 32-row tiles per block (a block overlaps one tile's load with the
    // other's compute, and the split-K partials, as large as 32 rows at 16
    // heads, are halved), doubled up to 256 rows while the launch would hold
    // more than one block per CU.  Tiny launches keep single tiles to have
    // more blocks.  Measured (layer-steps/s, one box): at most 512 blocks
    // against at most 256: shelf_ctx8 2 714 -> 2 727 (256 rows per block:
    // attention 22.6 -> 22.3 us, combine 5.8 -> 4.6 us); mtp3 with 512 rows
    // per block (256 blocks) lost (attention 28.9 -> 34.6 us), so blocks stay
    // at 256 rows; at most 1024 blocks lost everywhere (shelf_ctx8 2 642).
    auto blocks = [&](int64_t rpb) { return (int64_t)((k + rpb - 1) / rpb) * rows_total_pairs; };
    int rpb = 2 * kAttnTileRows;
    if (blocks(rpb) < 64) return kAttnTileRows;
    while (rpb < 8 * kAttnTileRows && blocks(rpb) > 256) rpb *= 2;
    return rpb;
}

}  // namespace

namespace {

// Per-step scratch of the decode step's kernels.  None of it carries state
// from one step to the next: the kernels leave the histograms, row records,
// winner and miss bitmaps cleared for the next step, and everything else is
// written before it is read within the step.
struct StepScratch {
    uint2* pre = nullptr;           // [B][D][cap] candidates at or above the floor
    uint2* cand = nullptr;          // [B][D][cap] staged bucket keys
    uint32_t* hist = nullptr;       // [B][D][4096]
    RowMeta* meta = nullptr;        // [B][D]
    uint32_t* winners = nullptr;    // [B][wpr]
    uint32_t* miss_bits = nullptr;  // [B][wpr] (early copy)
    int32_t* wrow = nullptr;        // [B][D][k] (early or late copy)
    GatherEntry* glist = nullptr;   // [B*D*k]
    float* part_acc = nullptr;      // [B*D][HG][nchunk][16][512]
    float* part_ml = nullptr;       // [B*D][HG][nchunk][16][2]
    uint32_t* qc8 = nullptr;        // [B][D][kQc8Words] (int8 indexer)
};

int validate_decode(sko_handle* h, int32_t layer, const void* q_idx, const void* q_attn, const float* out) {
    int rc = check_handle(h);
    if (rc != SKO_OK) return rc;
    if (layer < 0 || layer >= h->L) return set_err(SKO_E_INVAL, "layer %d out of range [0, %d)", layer, h->L);
    if (!q_idx || !q_attn || !out) return set_err(SKO_E_INVAL, "NULL query or output pointer");
    return SKO_OK;
}

// One decode step of `layer` (arguments already validated, device current),
// with the per-step scratch `sc`.  app_idx / app_kv non-null: the fused
// append, one new token per sequence (rows on the device, capacity already
// checked), appended inside the step.
int decode_step_impl(sko_handle* h, int32_t layer, const void* q_idx, const void* q_attn, float* out,
                     const StepScratch& sc, const void* app_idx = nullptr, const void* app_kv = nullptr) {
    int rc = SKO_OK;

    const int B = h->B, D = h->D, k = h->k, S = h->S, H = h->H;
    const int64_t cap = h->cap;
    const bool fused_append = app_idx != nullptr;
    if (fused_append)
        for (int b = 0; b < B; ++b) h->ntok[h->lb(layer, b)] += 1;
    int64_t max_now = 0;
    for (int b = 0; b < B; ++b) max_now = std::max(max_now, h->ntok[h->lb(layer, b)]);
    const int32_t t = h->step[layer];
    const size_t LBc = (size_t)layer * B * cap;
    const size_t LBs = (size_t)layer * B * S;
    const int R = h->R;
    const void* idx_layer = reinterpret_cast<const uint8_t*>(h->idx) + (size_t)layer * B * h->idx_seq_bytes();
    const uint16_t* scale_layer = h->c8 ? h->idx_scale + (size_t)layer * B * h->ntiles * kIdxTile : nullptr;
    const uint16_t* pool_layer = h->pool_dev + LBc * kKvDim;
    const uint16_t* recent_layer = h->recent + (size_t)layer * B * kKvDim;
    uint16_t* hot_layer = h->hot + (size_t)layer * B * R * kKvDim;
    int32_t* slot_row_layer = h->slot_row + LBs;
    int32_t* spare_layer = h->spare_rows + (size_t)layer * B * 2 * h->M;
    int32_t* cs = h->cache_slots + LBc;
    int32_t* st = h->slot_token + LBs;
    int32_t* lu = h->last_use + LBs;
    // the counts every kernel after the score launch reads: with the fused
    // append, the other buffer, which the score launch fills
    const int sel = h->ntok_sel[layer];
    const int32_t* ntok_in = h->ntok_buf(layer, sel);
    const int32_t* ntok = h->ntok_buf(layer, fused_append ? sel ^ 1 : sel);
    ScoreAppend app;
    if (fused_append) {
        app.idx = static_cast<const uint16_t*>(app_idx);
        app.kv = static_cast<const uint4*>(app_kv);
        app.idx_cache = reinterpret_cast<uint8_t*>(h->idx) + (size_t)layer * B * h->idx_seq_bytes();
        app.scales = h->c8 ? h->idx_scale + (size_t)layer * B * h->ntiles * kIdxTile : nullptr;
        app.recent = reinterpret_cast<uint4*>(h->recent + (size_t)layer * B * kKvDim);
        app.ntok_out = h->ntok_buf(layer, sel ^ 1);
    }
    const uint16_t* qi = static_cast<const uint16_t*>(q_idx);
    const uint16_t* qa = static_cast<const uint16_t*>(q_attn);

    int32_t* ring0 = h->ring[0] + (size_t)layer * B * h->C;
    int32_t* ring1 = h->ring[1] + (size_t)layer * B * h->C;
    int32_t* ring_pos = h->ring_pos + LBs;
    RingState* ring_state = h->ring_state + (size_t)layer * B;
    int32_t* floor_layer = h->floor + (size_t)layer * B * D;

    if ((rc = run_stage(h, ST_SCORE, [&] {
             return launch_score_hist(h->stream, idx_layer, qi, ntok_in, h->keys, sc.hist, floor_layer, sc.pre,
                                      sc.meta, cs, B, D, h->kcap, cap, h->ntiles, max_now, h->cu_count, scale_layer,
                                      sc.qc8, app, h->xc);
         })))
        return rc;
    const bool fused_copy = h->fused_copy;
    const bool staged = h->staged_copy;
    if ((rc = run_stage(h, ST_FILTER, [&] {
             return launch_topk_filter(h->stream, sc.hist, sc.meta, sc.pre, sc.cand, h->topk, cs, ntok, sc.winners,
                                       staged ? sc.miss_bits : nullptr, idx_layer, qi, floor_layer,
                                       (h->cfg.flags & SKO_FLAG_SELECT_RESCAN) != 0, B, D, cap, h->ntiles, k,
                                       max_now, scale_layer, h->c8 ? sc.qc8 : nullptr, h->xc);
         })))
        return rc;
    if (staged && (rc = run_stage(h, ST_REFINE, [&] {
                       // the split buckets first, so that the miss set is complete
                       // when the merge launch starts copying
                       return launch_topk_refine(h->stream, sc.meta, sc.cand, h->topk, sc.winners, sc.miss_bits, B,
                                                 D, k, cap, h->xc);
                   })))
        return rc;
    // split attention: the selection is complete, so the rows resident at
    // step start (whose slots and data the LRU update and the copy leave
    // alone) are attended on the side stream while the copy launch runs
    const bool split = staged && h->hit_overlap;
    if (split) {
        hipError_t e = hipEventRecord(h->ev_fork, h->stream);
        if (e == hipSuccess) e = hipStreamWaitEvent(h->side, h->ev_fork, 0);
        if (e != hipSuccess) return device_fail(h, e, "fork of the hit attention");
    }
    // timed early-copy launches also record their blocks' start and end
    uint64_t* stamps = nullptr;
    if (staged && h->stamps && ((h->timing_mask >> ST_MERGE_LRU) & 1u) &&
        (int)h->stamp_pending.size() < kStampLaunches) {
        int cps = 0, cw = 0;
        copy_shape(B, max_now, &cps, &cw, h->xcd_cus);
        // the record holds stamp_blocks blocks (the launch at full capacity);
        // a launch with more blocks is not recorded
        if (B + B * cps <= h->stamp_blocks) {
            const int slot = h->stamp_next++ % kStampLaunches;
            stamps = h->stamps + (size_t)slot * h->stamp_blocks * 2;
            h->stamp_pending.push_back({slot, B, B + B * cps});
        }
    }
    if ((rc = run_stage(h, ST_MERGE_LRU, [&] {
             return launch_merge_lru(h->stream, sc.winners, sc.hist, sc.meta, sc.cand, h->topk, ntok, cs, st, lu,
                                     ring0, ring1, ring_pos, ring_state, B, D, k, S, cap, t, h->misses, h->victims,
                                     h->evict_old, h->counts, sc.glist, h->stats + (size_t)layer * 8, !staged,
                                     staged ? sc.miss_bits : nullptr, pool_layer, recent_layer, hot_layer,
                                     slot_row_layer, spare_layer, R, fused_copy ? nullptr : sc.wrow, h->phys,
                                     /* the split attention reads the lists during this launch */ !h->hit_overlap,
                                     max_now, (h->cfg.flags & SKO_FLAG_TEST_VIOLATION) != 0, stamps,
                                     fused_append ? h->pool_dev + LBc * kKvDim : nullptr, h->xc, h->xcd_cus);
         })))
        return rc;
    // late copy: its own gather from the pool into the misses' rows; early:
    // the copy blocks of the LRU-update launch did it; fused: the attention
    // launch copies them itself
    if (!fused_copy && !staged && (rc = run_stage(h, ST_GATHER, [&] {
             return launch_gather_misses(h->stream, sc.glist, h->counts, pool_layer, recent_layer, ntok, hot_layer,
                                         B, cap, D * k, B * D * k);
         })))
        return rc;
    if (split) {
        if ((rc = run_stage(
                 h, ST_ATTN_HITS,
                 [&] {
                     return launch_attn_partial(h->side, h->topk, cs, slot_row_layer, hot_layer, R, qa, nullptr,
                                                recent_layer, ntok, sc.part_acc, sc.part_ml, h->phys, B, D, H, k,
                                                S, cap, h->rows_per_block, h->cfg.attn_scale, nullptr, nullptr, 1);
                 },
                 h->side)))
            return rc;
        const hipError_t e = hipEventRecord(h->ev_join, h->side);
        if (e != hipSuccess) return device_fail(h, e, "join of the hit attention");
    }
    if ((rc = run_stage(h, ST_ATTN, [&] {
             return launch_attn_partial(h->stream, h->topk, cs, slot_row_layer, hot_layer, R, qa,
                                        fused_copy ? pool_layer : nullptr, recent_layer, ntok, sc.part_acc,
                                        sc.part_ml, h->phys, B, D, H, k, S, cap, h->rows_per_block,
                                        h->cfg.attn_scale, fused_copy ? nullptr : sc.wrow,
                                        staged ? sc.miss_bits : nullptr, split ? 2 : 0, h->xc);
         })))
        return rc;
    if (split) {
        const hipError_t e = hipStreamWaitEvent(h->stream, h->ev_join, 0);
        if (e != hipSuccess) return device_fail(h, e, "join of the hit attention");
    }
    if ((rc = run_stage(h, ST_COMBINE, [&] {
             return launch_attn_combine(h->stream, sc.part_acc, sc.part_ml, out, B, D, H,
                                        h->nchunk * (split ? 2 : 1), h->xc);
         })))
        return rc;
    h->step[layer] += 1;
    h->last_layer = layer;
    if (fused_append) h->ntok_sel[layer] ^= 1;
    return SKO_OK;
}

// The step scratch the handle owns (sko_decode_step, sko_decode_step_append).
StepScratch handle_scratch(const sko_handle* h) {
    StepScratch sc;
    sc.pre = h->pre;
    sc.cand = h->cand;
    sc.hist = h->hist;
    sc.meta = h->meta;
    sc.winners = h->winners;
    sc.miss_bits = h->miss_bits;
    sc.wrow = h->wrow;
    sc.glist = h->glist;
    sc.part_acc = h->part_acc;
    sc.part_ml = h->part_ml;
    sc.qc8 = h->qc8;
    return sc;
}


// ---- the decode step without any allocation ---------------------------------
// For callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid it):
// sko_decode_step_static takes the per-step scratch from this file-scope
// array instead of the handle's own.  Each device that runs it holds one
// copy until the process ends.  In host code the name `scratch` is only a
// stand-in: its device address is looked up once per device at sko_create
// (hipGetSymbolAddress) and only that address is ever used.
constexpr size_t kStaticScratchBytes = (size_t)SKO_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};   // device address of `scratch` per device
int g_scratch_state[kMaxDevices] = {};    // 0: not looked up, 1: found, -1: lookup failed

// Called at sko_create with `device` current.
void resolve_static_scratch(int device) {
    if (device < 0 || device >= kMaxDevices) return;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_state[device] != 0) return;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
        (void)hipGetLastError();
        g_scratch_state[device] = -1;
        return;
    }
    g_scratch_addr[device] = ptr;
    g_scratch_state[device] = 1;
}

// Lays the step scratch of `h` out from `base` (256-byte aligned pieces);
// returns the bytes it needs (base may be null to only measure).
size_t layout_step_scratch(const sko_handle* h, unsigned char* base, StepScratch* sc, size_t* zero_bytes) {
    const size_t BD = (size_t)h->B * h->D;
    const size_t pchunks = (size_t)h->nchunk * (h->hit_overlap ? 2 : 1);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        unsigned char* p = base ? base + off : nullptr;
        off += (bytes + 255) / 256 * 256;
        return p;
    };
    // the parts that must start at zero come first, in one run
    sc->hist = reinterpret_cast<uint32_t*>(take(BD * kHistBins * 4));
    sc->meta = reinterpret_cast<RowMeta*>(take(BD * sizeof(RowMeta)));
    sc->winners = reinterpret_cast<uint32_t*>(take((size_t)h->B * h->wpr * 4));
    sc->miss_bits = h->staged_copy ? reinterpret_cast<uint32_t*>(take((size_t)h->B * h->wpr * 4)) : nullptr;
    *zero_bytes = off;
    sc->wrow = h->fused_copy ? nullptr : reinterpret_cast<int32_t*>(take(BD * h->k * 4));
    sc->pre = reinterpret_cast<uint2*>(take(BD * h->cap * sizeof(uint2)));
    sc->cand = reinterpret_cast<uint2*>(take(BD * h->cap * sizeof(uint2)));
    sc->glist = reinterpret_cast<GatherEntry*>(take(BD * h->k * sizeof(GatherEntry)));
    sc->part_acc = reinterpret_cast<float*>(take(BD * h->HG * pchunks * kAttnHeadGroup * kVDim * 4));
    sc->part_ml = reinterpret_cast<float*>(take(BD * h->HG * pchunks * kAttnHeadGroup * 2 * 4));
    sc->qc8 = h->c8 ? reinterpret_cast<uint32_t*>(take(BD * kQc8Words * 4)) : nullptr;
    return off;
}

// The XCD each block of a launch runs on (HW_REG_XCC_ID), for the check of
// SKO_FLAG_XCD_SPLIT at creation.
__global__ __launch_bounds__(64) void k_xcc_of_blocks(int32_t* __restrict__ out) {
    if (threadIdx.x == 0) out[blockIdx.x] = xcc_id();
}

// True when launches on `st` deal their blocks to the 8 XCDs in a fixed
// stripe: block i on XCD (i + o) mod 8 with one o per launch, every XCD
// taking part.  Launch sizes that are and are not multiples of 8.
bool xcd_stripe_holds(hipStream_t st) {
    const int sizes[] = {256, 61, 1000, 8};
    int total = 0;
    for (int n : sizes) total += n;
    int32_t* d = nullptr;
    if (hipMalloc((void**)&d, (size_t)total * 4) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    bool ok = true;
    int off = 0;
    for (int n : sizes) {
        hipLaunchKernelGGL(k_xcc_of_blocks, dim3(n), dim3(64), 0, st, d + off);
        if (hipGetLastError() != hipSuccess) ok = false;
        off += n;
    }
    std::vector<int32_t> x(total, -1);
    if (ok && hipMemcpyAsync(x.data(), d, (size_t)total * 4, hipMemcpyDeviceToHost, st) != hipSuccess) ok = false;
    if (ok && hipStreamSynchronize(st) != hipSuccess) ok = false;
    (void)hipFree(d);
    (void)hipGetLastError();
    off = 0;
    for (int n : sizes) {
        if (!ok) break;
        const int o = (x[off] % kXcds + kXcds) % kXcds;
        unsigned seen = 0;
        for (int i = 0; i < n; ++i) {
            const int v = x[off + i];
            if (v < 0 || v >= kXcds || ((v - i) % kXcds + kXcds) % kXcds != o) ok = false;
            else seen |= 1u << v;
        }
        if (n >= kXcds && seen != (1u << kXcds) - 1) ok = false;
        off += n;
    }
    return ok;
}

// Clears the first nz words of `z` and sets the first nf words of `f` to all
// ones (a kernel, not a memset, so the call can sit inside a captured graph).
__global__ __launch_bounds__(256) void k_clear_scratch(uint32_t* __restrict__ z, int64_t nz,
                                                       uint32_t* __restrict__ f, int64_t nf) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nz + nf; i += stride) {
        if (i < nz) z[i] = 0u;
        else f[i - nz] = 0xFFFFFFFFu;
    }
}

}  // namespace

extern "C" {

const char* sko_last_error(void) { return g_err.c_str(); }

const char* sko_version(void) { return "sko 0.1 (gfx950)"; }

int32_t sko_num_stages(void) { return ST_COUNT; }

const char* sko_stage_name(int32_t stage) {
    return (stage >= 0 && stage < ST_COUNT) ? kStageNames[stage] : "";
}

int sko_create(const sko_config* cfg, void* stream, sko_handle** out) {
    if (!out) return set_err(SKO_E_INVAL, "NULL out pointer");
    *out = nullptr;
    int rc = validate_config(cfg);
    if (rc != SKO_OK) return rc;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= cfg->device)
        return set_err(SKO_E_DEVICE, "HIP device %d not available", cfg->device);
    DeviceGuard guard(cfg->device);
    if (!guard.ok) return set_err(SKO_E_DEVICE, "hipSetDevice(%d) failed", cfg->device);

    sko_handle* h = new sko_handle();
    h->cfg = *cfg;
    h->stream = (hipStream_t)stream;
    h->L = cfg->num_layers;
    h->B = cfg->batch;
    h->k = cfg->top_k;
    h->S = cfg->hot_slots;
    h->D = cfg->mtp_positions;
    h->H = cfg->num_heads;
    h->HG = (h->H + kAttnHeadGroup - 1) / kAttnHeadGroup;
    h->cap = cfg->max_tokens;
    h->ntiles = (h->cap + kIdxTile - 1) / kIdxTile;
    h->kcap = (h->cap + 15) / 16 * 16;
    h->C = ring_capacity(h->S, h->D, h->k);
    h->M = h->D * h->k;
    h->R = h->S + h->M;
    h->wpr = winner_words(h->cap);
    h->ntok.assign((size_t)h->L * h->B, 0);
    h->ntok_sel.assign((size_t)h->L, 0);
    h->step.assign((size_t)h->L, 0);
    {
        int ncu = 0;
        if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, cfg->device) == hipSuccess && ncu > 0)
            h->cu_count = ncu;
    }
    // Early copy by default: extra blocks of the LRU-update launch copy the
    // misses into their spare hot rows while the update runs, so neither the
    // update nor the attention waits on the host link (measured against copying inside
    // the attention at one position: tiny +18 %, small +4.5 %, shelf even;
    // against the late copy: long +20 %, mtp3 +2 %).
    h->fused_copy = (cfg->flags & SKO_FLAG_FUSED_COPY) != 0;
    h->staged_copy = !h->fused_copy && !(cfg->flags & SKO_FLAG_LATE_COPY);
    h->c8 = (cfg->flags & SKO_FLAG_INDEXER_C8) != 0;
    h->hit_overlap = h->staged_copy && (cfg->flags & SKO_FLAG_HIT_OVERLAP) != 0;
    if (cfg->flags & SKO_FLAG_XCD_SPLIT) {
        if (h->cu_count % kXcds != 0 || !xcd_stripe_holds(h->stream)) {
            delete h;
            return set_err(SKO_E_UNSUPPORTED,
                           "SKO_FLAG_XCD_SPLIT: the device does not deal launch blocks to 8 XCDs in a fixed stripe");
        }
        h->xc = 0;
        h->xcd_cus = h->cu_count / kXcds;
    }
    // the LRU-update launch's LDS, sized for S and D*k
    if (prepare_merge_lru(merge_lru_lds_bytes(h->S, h->D, h->k)) != hipSuccess) {
        (void)hipGetLastError();
        delete h;
        return set_err(SKO_E_DEVICE, "the LRU-update kernel cannot take %zu bytes of LDS",
                       merge_lru_lds_bytes(h->S, h->D, h->k));
    }
    h->rows_per_block = attn_rows_per_block(h->k, h->B * h->D * h->HG);
    h->nchunk = (h->k + h->rows_per_block - 1) / h->rows_per_block;
    // the split attention writes the partials of both phases
    const size_t pchunks = (size_t)h->nchunk * (h->hit_overlap ? 2 : 1);

    const size_t LB = (size_t)h->L * h->B;
    const size_t BD = (size_t)h->B * h->D;
    const size_t pool_bytes = LB * (size_t)h->cap * kKvRowBytes;
    unsigned pool_flags = hipHostMallocMapped;
    if (cfg->flags & SKO_FLAG_POOL_COHERENT) pool_flags |= hipHostMallocCoherent;
    if (cfg->flags & SKO_FLAG_POOL_NONCOHERENT) pool_flags |= hipHostMallocNonCoherent;
    if (hipHostMalloc((void**)&h->pool_host, pool_bytes, pool_flags) != hipSuccess) {
        (void)hipGetLastError();
        h->pool_host = nullptr;
        free_all(h);
        delete h;
        return set_err(SKO_E_NOMEM, "pinned host pool of %zu bytes", pool_bytes);
    }
    if (hipHostGetDevicePointer((void**)&h->pool_dev, h->pool_host, 0) != hipSuccess) {
        (void)hipGetLastError();
        free_all(h);
        delete h;
        return set_err(SKO_E_DEVICE, "hipHostGetDevicePointer on the host pool failed");
    }
    bool ok = true;
    ok = ok && dev_alloc(h, (void**)&h->idx, LB * h->idx_seq_bytes());
    if (h->c8) {
        ok = ok && dev_alloc(h, (void**)&h->idx_scale, LB * h->ntiles * kIdxTile * 2);
        ok = ok && dev_alloc(h, (void**)&h->qc8, (size_t)h->B * h->D * kQc8Words * 4);
    }
    ok = ok && dev_alloc(h, (void**)&h->staging, (size_t)kStagingRows * kIdxDim * 2);
    // the hot rows of every (layer, seq): its S slots' rows and D*k spare
    // rows, which take the misses of a step
    ok = ok && dev_alloc(h, (void**)&h->hot, LB * h->R * (size_t)kKvRowBytes);
    ok = ok && dev_alloc(h, (void**)&h->slot_row, LB * h->S * 4);
    ok = ok && dev_alloc(h, (void**)&h->spare_rows, LB * 2 * h->M * 4);
    ok = ok && dev_alloc(h, (void**)&h->recent, LB * (size_t)kKvRowBytes);
    ok = ok && dev_alloc(h, (void**)&h->cache_slots, LB * h->cap * 4);
    ok = ok && dev_alloc(h, (void**)&h->slot_token, LB * h->S * 4);
    ok = ok && dev_alloc(h, (void**)&h->last_use, LB * h->S * 4);
    ok = ok && dev_alloc(h, (void**)&h->ring[0], LB * h->C * 4);
    ok = ok && dev_alloc(h, (void**)&h->ring[1], LB * h->C * 4);
    ok = ok && dev_alloc(h, (void**)&h->ring_pos, LB * h->S * 4);
    ok = ok && dev_alloc(h, (void**)&h->ring_state, LB * sizeof(RingState));
    ok = ok && dev_alloc(h, (void**)&h->ntok_dev, LB * 2 * 4);
    ok = ok && dev_alloc(h, (void**)&h->stats, (size_t)h->L * 8 * 8);
    if (cfg->flags & SKO_FLAG_KEEP_KEYS) ok = ok && dev_alloc(h, (void**)&h->keys, BD * h->kcap * 4);
    ok = ok && dev_alloc(h, (void**)&h->pre, BD * h->cap * sizeof(uint2));
    ok = ok && dev_alloc(h, (void**)&h->floor, LB * h->D * 4);
    if (h->staged_copy) ok = ok && dev_alloc(h, (void**)&h->miss_bits, (size_t)h->B * h->wpr * 4);
    if (!h->fused_copy) ok = ok && dev_alloc(h, (void**)&h->wrow, BD * h->k * 4);
    ok = ok && dev_alloc(h, (void**)&h->winners, (size_t)h->B * h->wpr * 4);
    ok = ok && dev_alloc(h, (void**)&h->hist, BD * kHistBins * 4);
    ok = ok && dev_alloc(h, (void**)&h->meta, BD * sizeof(RowMeta));
    ok = ok && dev_alloc(h, (void**)&h->cand, BD * h->cap * sizeof(uint2));
    ok = ok && dev_alloc(h, (void**)&h->topk, BD * h->k * 4);
    ok = ok && dev_alloc(h, (void**)&h->phys, BD * h->k * 4);
    ok = ok && dev_alloc(h, (void**)&h->misses, BD * h->k * 4);
    ok = ok && dev_alloc(h, (void**)&h->victims, BD * h->k * 4);
    ok = ok && dev_alloc(h, (void**)&h->evict_old, BD * h->k * 4);
    ok = ok && dev_alloc(h, (void**)&h->counts, (size_t)h->B * 8 * 4);
    ok = ok && dev_alloc(h, (void**)&h->glist, BD * h->k * sizeof(GatherEntry));
    ok = ok && dev_alloc(h, (void**)&h->part_acc, BD * h->HG * pchunks * kAttnHeadGroup * kVDim * 4);
    ok = ok && dev_alloc(h, (void**)&h->part_ml, BD * h->HG * pchunks * kAttnHeadGroup * 2 * 4);
    if (h->staged_copy) {
        int cps = 0, cw = 0;
        copy_shape(h->B, h->cap, &cps, &cw, h->xcd_cus);
        h->stamp_blocks = h->B + h->B * cps;
        ok = ok && dev_alloc(h, (void**)&h->stamps, (size_t)kStampLaunches * h->stamp_blocks * 2 * 8);
    }
    {
        int khz = 0;
        if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, cfg->device) == hipSuccess && khz > 0)
            h->clock_khz = khz;
    }
    if (!ok) {
        free_all(h);
        delete h;
        return set_err(SKO_E_NOMEM, "device allocation failed");
    }
    if (hipEventCreateWithFlags(&h->ev_switch, hipEventDisableTiming) != hipSuccess) {
        (void)hipGetLastError();
        h->ev_switch = nullptr;
        free_all(h);
        delete h;
        return set_err(SKO_E_DEVICE, "creating the stream-switch event failed");
    }
    if (h->hit_overlap &&
        (hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking) != hipSuccess ||
         hipEventCreateWithFlags(&h->ev_fork, hipEventDisableTiming) != hipSuccess ||
         hipEventCreateWithFlags(&h->ev_join, hipEventDisableTiming) != hipSuccess)) {
        (void)hipGetLastError();
        free_all(h);
        delete h;
        return set_err(SKO_E_DEVICE, "creating the side stream of the hit attention failed");
    }
    // initial state: empty shelf, empty reverse index, no tokens
    hipError_t e = hipSuccess;
    if (e == hipSuccess) e = hipMemsetAsync(h->cache_slots, 0xFF, LB * h->cap * 4, h->stream);
    if (e == hipSuccess) e = hipMemsetAsync(h->slot_token, 0xFF, LB * h->S * 4, h->stream);
    if (e == hipSuccess) e = hipMemsetAsync(h->last_use, 0xFF, LB * h->S * 4, h->stream);
    if (e == hipSuccess) e = hipMemsetAsync(h->ntok_dev, 0, LB * 2 * 4, h->stream);
    if (e == hipSuccess) e = hipMemsetAsync(h->hot, 0, LB * h->R * (size_t)kKvRowBytes, h->stream);
    if (e == hipSuccess) e = hipMemsetAsync(h->stats, 0, (size_t)h->L * 8 * 8, h->stream);
    if (e == hipSuccess) e = hipMemsetAsync(h->topk, 0, BD * h->k * 4, h->stream);
    if (e == hipSuccess) e = hipMemsetAsync(h->counts, 0, (size_t)h->B * 8 * 4, h->stream);
    if (e == hipSuccess) e = hipMemsetAsync(h->winners, 0, (size_t)h->B * h->wpr * 4, h->stream);
    // selection scratch starts cleared; every step's merge clears it again
    if (e == hipSuccess) e = hipMemsetAsync(h->hist, 0, BD * kHistBins * 4, h->stream);
    if (e == hipSuccess) e = hipMemsetAsync(h->meta, 0, BD * sizeof(RowMeta), h->stream);
    if (e == hipSuccess && h->staged_copy) e = hipMemsetAsync(h->miss_bits, 0, (size_t)h->B * h->wpr * 4, h->stream);
    if (e == hipSuccess && h->wrow) e = hipMemsetAsync(h->wrow, 0xFF, BD * h->k * 4, h->stream);
    if (e == hipSuccess) {
        // first step: every key is a candidate (or none, to force the rescan path)
        const std::vector<int32_t> fl(LB * h->D, (cfg->flags & SKO_FLAG_SELECT_RESCAN) ? kFloorRescanAll : 0);
        e = hipMemcpyAsync(h->floor, fl.data(), fl.size() * 4, hipMemcpyHostToDevice, h->stream);
        if (e == hipSuccess) e = hipStreamSynchronize(h->stream);
    }
    if (e == hipSuccess) e = hipMemsetAsync(h->idx, 0, LB * h->idx_seq_bytes(), h->stream);
    if (e == hipSuccess && h->c8) e = hipMemsetAsync(h->idx_scale, 0, LB * h->ntiles * kIdxTile * 2, h->stream);
    if (e == hipSuccess && h->c8) e = hipMemsetAsync(h->qc8, 0, (size_t)h->B * h->D * kQc8Words * 4, h->stream);
    if (e == hipSuccess) e = launch_init_rings(h->stream, h->ring[0], h->ring_pos, h->ring_state, h->slot_row, h->spare_rows,
                                                   (int64_t)LB, h->S, h->C, h->M);
    if (e == hipSuccess) e = hipStreamSynchronize(h->stream);
    if (e != hipSuccess) {
        set_err(SKO_E_DEVICE, "initialising state: %s", hipGetErrorString(e));
        free_all(h);
        delete h;
        return SKO_E_DEVICE;
    }
    // set-up of the no-allocation decode step on this device (once per device)
    resolve_static_scratch(cfg->device);
    *out = h;
    return SKO_OK;
}

int sko_set_stream(sko_handle* h, void* stream) {
    int rc = check_handle(h);
    if (rc != SKO_OK) return rc;
    const hipStream_t ns = (hipStream_t)stream;
    if (ns == h->stream) return SKO_OK;
    // Every step reads and writes the same handle state, so the new stream
    // waits for whatever is queued on the old one; later synchronizations
    // (reads, destroy) then cover both.
    DeviceGuard guard(h->cfg.device);
    if (!guard.ok) return device_fail(h, hipErrorInvalidDevice, "hipSetDevice");
    hipError_t e = hipEventRecord(h->ev_switch, h->stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(ns, h->ev_switch, 0);
    if (e != hipSuccess) return device_fail(h, e, "ordering the new stream after the old one");
    h->stream = ns;
    return SKO_OK;
}

int sko_append_token(sko_handle* h, int32_t layer, int32_t seq, const void* idx_rows,
                     const void* kv_rows, int64_t n, int32_t src_on_device) {
    int rc = check_handle(h);
    if (rc != SKO_OK) return rc;
    if (layer < 0 || layer >= h->L) return set_err(SKO_E_INVAL, "layer %d out of range [0, %d)", layer, h->L);
    if (seq != SKO_ALL_SEQS && (seq < 0 || seq >= h->B))
        return set_err(SKO_E_INVAL, "seq %d out of range", seq);
    if (n < 0) return set_err(SKO_E_INVAL, "n must be >= 0");
    if (n > 0 && (!idx_rows || !kv_rows)) return set_err(SKO_E_INVAL, "NULL row pointer");
    if (src_on_device != 0 && src_on_device != 1) return set_err(SKO_E_INVAL, "src_on_device must be 0 or 1");
    const int seq0 = seq == SKO_ALL_SEQS ? 0 : seq;
    const int nseq = seq == SKO_ALL_SEQS ? h->B : 1;
    for (int s = 0; s < nseq; ++s)
        if (h->ntok[h->lb(layer, seq0 + s)] + n > h->cap)
            return set_err(SKO_E_CAPACITY, "seq %d: %lld + %lld tokens exceed max_tokens %lld", seq0 + s,
                           (long long)h->ntok[h->lb(layer, seq0 + s)], (long long)n, (long long)h->cap);
    if (n == 0) return SKO_OK;
    DeviceGuard guard(h->cfg.device);
    if (!guard.ok) return device_fail(h, hipErrorInvalidDevice, "hipSetDevice");

    uint8_t* idx_layer = reinterpret_cast<uint8_t*>(h->idx) + (size_t)layer * h->B * h->idx_seq_bytes();
    uint16_t* scale_layer = h->c8 ? h->idx_scale + (size_t)layer * h->B * h->ntiles * kIdxTile : nullptr;
    uint16_t* pool_layer_dev = h->pool_dev + (size_t)layer * h->B * h->cap * kKvDim;
    uint16_t* recent_layer = h->recent + (size_t)layer * h->B * kKvDim;
    int32_t* ntok_layer = h->ntok_buf(layer, h->ntok_sel[layer]);
    // bf16 indexer rows are stored as they are, or rotated and quantized
    auto append_rows = [&](const uint16_t* is, const uint16_t* ks, uint16_t* pool, int b0, int nb, int64_t m,
                           int64_t base) {
        return h->c8 ? launch_append_rows_c8(h->stream, is, ks, idx_layer, scale_layer, pool, recent_layer,
                                             ntok_layer, b0, nb, m, h->cap, h->ntiles, (int32_t)base)
                     : launch_append_rows(h->stream, is, ks, reinterpret_cast<uint16_t*>(idx_layer), pool,
                                          recent_layer, ntok_layer, b0, nb, m, h->cap, h->ntiles, (int32_t)base);
    };
    const uint16_t* isrc = static_cast<const uint16_t*>(idx_rows);
    const uint16_t* ksrc = static_cast<const uint16_t*>(kv_rows);

    if (src_on_device) {
        // one launch per run of sequences that share a start position
        int s = 0;
        while (s < nseq) {
            const int64_t base = h->ntok[h->lb(layer, seq0 + s)];
            int e = s + 1;
            while (e < nseq && h->ntok[h->lb(layer, seq0 + e)] == base) ++e;
            rc = run_stage(h, ST_APPEND, [&] {
                return append_rows(isrc + (size_t)s * n * kIdxDim, ksrc + (size_t)s * n * kKvDim, pool_layer_dev,
                                   seq0 + s, e - s, n, base);
            });
            if (rc != SKO_OK) return rc;
            s = e;
        }
    } else {
        for (int s = 0; s < nseq; ++s) {
            const int b = seq0 + s;
            const int64_t base = h->ntok[h->lb(layer, b)];
            std::memcpy(h->pool_host + (h->lb(layer, b) * h->cap + base) * kKvDim, ksrc + (size_t)s * n * kKvDim,
                        (size_t)n * kKvRowBytes);
            // the newest row also to its device copy
            hipError_t er = hipMemcpyAsync(recent_layer + (size_t)b * kKvDim, ksrc + ((size_t)s * n + n - 1) * kKvDim,
                                           kKvRowBytes, hipMemcpyHostToDevice, h->stream);
            if (er != hipSuccess) return device_fail(h, er, "newest row host->device");
            // indexer rows: host -> staging rows -> tiled cache, in pieces
            for (int64_t r0 = 0; r0 < n; r0 += kStagingRows) {
                const int64_t m = std::min<int64_t>(kStagingRows, n - r0);
                hipError_t e = hipMemcpyAsync(h->staging, isrc + ((size_t)s * n + r0) * kIdxDim,
                                              (size_t)m * kIdxDim * 2, hipMemcpyHostToDevice, h->stream);
                if (e != hipSuccess) return device_fail(h, e, "indexer rows host->device");
                e = append_rows(h->staging, nullptr, nullptr, b, 1, m, base + r0);
                if (e != hipSuccess) return device_fail(h, e, "indexer rows to tiles");
            }
        }
        // the caller may reuse its host rows once the call returns
        hipError_t e = hipStreamSynchronize(h->stream);
        if (e != hipSuccess) return device_fail(h, e, "append sync");
    }
    for (int s = 0; s < nseq; ++s) h->ntok[h->lb(layer, seq0 + s)] += n;
    return SKO_OK;
}

int sko_decode_step(sko_handle* h, int32_t layer, const void* q_idx, const void* q_attn, float* out) {
    int rc = validate_decode(h, layer, q_idx, q_attn, out);
    if (rc != SKO_OK) return rc;
    DeviceGuard guard(h->cfg.device);
    if (!guard.ok) return device_fail(h, hipErrorInvalidDevice, "hipSetDevice");
    return decode_step_impl(h, layer, q_idx, q_attn, out, handle_scratch(h));
}

int sko_decode_step_append(sko_handle* h, int32_t layer, const void* idx_rows, const void* kv_rows,
                           const void* q_idx, const void* q_attn, float* out) {
    int rc = validate_decode(h, layer, q_idx, q_attn, out);
    if (rc != SKO_OK) return rc;
    if (!idx_rows || !kv_rows) return set_err(SKO_E_INVAL, "NULL row pointer");
    for (int b = 0; b < h->B; ++b)
        if (h->ntok[h->lb(layer, b)] + 1 > h->cap)
            return set_err(SKO_E_CAPACITY, "seq %d: %lld + 1 tokens exceed max_tokens %lld", b,
                           (long long)h->ntok[h->lb(layer, b)], (long long)h->cap);
    DeviceGuard guard(h->cfg.device);
    if (!guard.ok) return device_fail(h, hipErrorInvalidDevice, "hipSetDevice");
    return decode_step_impl(h, layer, q_idx, q_attn, out, handle_scratch(h), idx_rows, kv_rows);
}

int sko_decode_step_static(sko_handle* h, int32_t layer, const void* q_idx, const void* q_attn, float* out) {
    int rc = validate_decode(h, layer, q_idx, q_attn, out);
    if (rc != SKO_OK) return rc;
    const int dev = h->cfg.device;
    if (dev >= kMaxDevices || g_scratch_state[dev] != 1)
        return set_err(SKO_E_DEVICE, "the static scratch area of device %d is not available", dev);
    StepScratch sc;
    size_t zero_bytes = 0;
    const size_t need = layout_step_scratch(h, nullptr, &sc, &zero_bytes);
    if (need > kStaticScratchBytes)
        return set_err(SKO_E_UNSUPPORTED,
                       "sko_decode_step_static: this handle's step needs %zu bytes of scratch, the static area "
                       "holds %zu (use sko_decode_step)",
                       need, kStaticScratchBytes);
    DeviceGuard guard(dev);
    if (!guard.ok) return device_fail(h, hipErrorInvalidDevice, "hipSetDevice");
    unsigned char* base = static_cast<unsigned char*>(g_scratch_addr[dev]);
    (void)layout_step_scratch(h, base, &sc, &zero_bytes);
    // the area keeps the last call's contents (any handle's): clear what the
    // step expects to start cleared
    const int64_t nz = (int64_t)(zero_bytes / 4);
    const int64_t nf = sc.wrow ? (int64_t)((size_t)h->B * h->D * h->k) : 0;
    const int64_t blocks = std::min<int64_t>(1024, std::max<int64_t>(1, (nz + nf + 255) / 256));
    hipLaunchKernelGGL(k_clear_scratch, dim3((unsigned)blocks), dim3(256), 0, h->stream,
                       reinterpret_cast<uint32_t*>(base), nz, reinterpret_cast<uint32_t*>(sc.wrow), nf);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return device_fail(h, e, "clearing the static scratch");
    // no stage timing here: its events are created on demand
    const uint32_t mask = h->timing_mask;
    h->timing_mask = 0;
    rc = decode_step_impl(h, layer, q_idx, q_attn, out, sc);
    h->timing_mask = mask;
    return rc;
}

int sko_read_step(sko_handle* h, int32_t which, void* dst, int64_t bytes) {
    int rc = check_handle(h);
    if (rc != SKO_OK) return rc;
    if (!dst) return set_err(SKO_E_INVAL, "NULL destination");
    const size_t BD = (size_t)h->B * h->D;
    const void* src = nullptr;
    size_t size = 0;
    switch (which) {
        case SKO_BUF_TOPK: src = h->topk; size = BD * h->k * 4; break;
        case SKO_BUF_PHYS: src = h->phys; size = BD * h->k * 4; break;
        case SKO_BUF_COUNTS: src = h->counts; size = (size_t)h->B * sizeof(sko_seq_counts); break;
        case SKO_BUF_MISSES: src = h->misses; size = BD * h->k * 4; break;
        case SKO_BUF_VICTIMS: src = h->victims; size = BD * h->k * 4; break;
        case SKO_BUF_EVICT_OLD: src = h->evict_old; size = BD * h->k * 4; break;
        case SKO_BUF_KEYS:  // de-strided below
            if (!h->keys) return set_err(SKO_E_STATE, "score keys are kept only with SKO_FLAG_KEEP_KEYS");
            src = h->keys;
            size = BD * h->cap * 4;
            break;
        default: return set_err(SKO_E_INVAL, "unknown step buffer %d", which);
    }
    if ((size_t)bytes != size) return set_err(SKO_E_INVAL, "buffer %d holds %zu bytes, got %lld", which, size, (long long)bytes);
    DeviceGuard guard(h->cfg.device);
    hipError_t e = hipStreamSynchronize(h->stream);
    if (e != hipSuccess) return device_fail(h, e, "read step sync");
    if ((rc = check_invariants(h)) != SKO_OK) return rc;
    if (which == SKO_BUF_KEYS)
        e = hipMemcpy2D(dst, (size_t)h->cap * 4, src, (size_t)h->kcap * 4, (size_t)h->cap * 4, BD,
                        hipMemcpyDeviceToHost);
    else if (e == hipSuccess)
        e = hipMemcpy(dst, src, size, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return device_fail(h, e, "read step buffer");
    return SKO_OK;
}

int sko_read_table(sko_handle* h, int32_t layer, int32_t seq, int32_t which, void* dst, int64_t bytes) {
    int rc = check_handle(h);
    if (rc != SKO_OK) return rc;
    if (layer < 0 || layer >= h->L || seq < 0 || seq >= h->B) return set_err(SKO_E_INVAL, "layer/seq out of range");
    if (!dst) return set_err(SKO_E_INVAL, "NULL destination");
    const size_t lb = h->lb(layer, seq);
    const void* src = nullptr;
    size_t size = 0;
    bool host = false;
    switch (which) {
        case SKO_TAB_CACHE_SLOTS: src = h->cache_slots + lb * h->cap; size = (size_t)h->cap * 4; break;
        case SKO_TAB_SLOT_TOKEN: src = h->slot_token + lb * h->S; size = (size_t)h->S * 4; break;
        case SKO_TAB_LAST_USE: src = h->last_use + lb * h->S; size = (size_t)h->S * 4; break;
        case SKO_TAB_HOT: src = h->hot + lb * h->R * kKvDim; size = (size_t)h->S * kKvRowBytes; break;
        case SKO_TAB_INDEXER:
            src = reinterpret_cast<const uint8_t*>(h->idx) + lb * h->idx_seq_bytes();
            size = (size_t)h->cap * (h->c8 ? kIdxDim : kIdxDim * 2);
            break;
        case SKO_TAB_INDEXER_SCALE:
            if (!h->c8) return set_err(SKO_E_STATE, "SKO_TAB_INDEXER_SCALE needs SKO_FLAG_INDEXER_C8");
            src = h->idx_scale + lb * h->ntiles * kIdxTile;
            size = (size_t)h->cap * 2;
            break;
        case SKO_TAB_POOL: src = h->pool_host + lb * h->cap * kKvDim; size = (size_t)h->cap * kKvRowBytes; host = true; break;
        case SKO_TAB_NTOK: size = 8; break;
        case SKO_TAB_SLOT_ROW: src = h->slot_row + lb * h->S; size = (size_t)h->S * 4; break;
        case SKO_TAB_SPARE_ROWS:
            // the generation the layer's next step (stamp step[layer]) uses
            src = h->spare_rows + (lb * 2 + (h->step[layer] & 1)) * h->M;
            size = (size_t)h->M * 4;
            break;
        default: return set_err(SKO_E_INVAL, "unknown table %d", which);
    }
    if ((size_t)bytes != size) return set_err(SKO_E_INVAL, "table %d holds %zu bytes, got %lld", which, size, (long long)bytes);
    DeviceGuard guard(h->cfg.device);
    hipError_t e = hipStreamSynchronize(h->stream);
    if (e != hipSuccess) return device_fail(h, e, "read table sync");
    if ((rc = check_invariants(h)) != SKO_OK) return rc;
    if (which == SKO_TAB_NTOK) {
        int64_t v = h->ntok[lb];
        std::memcpy(dst, &v, 8);
    } else if (which == SKO_TAB_INDEXER) {
        // undo the 64-token tiling: [tile][chunk][token] x 16 B -> [token][chunk] x 16 B
        const int ru = h->c8 ? kIdxC8RowU4 : kIdxRowU4;
        std::vector<uint4> tiles((size_t)h->ntiles * ru * kIdxTile);
        e = hipMemcpy(tiles.data(), src, tiles.size() * sizeof(uint4), hipMemcpyDeviceToHost);
        if (e != hipSuccess) return device_fail(h, e, "read table");
        uint4* o = static_cast<uint4*>(dst);
        for (int64_t tok = 0; tok < h->cap; ++tok)
            for (int c = 0; c < ru; ++c)
                o[tok * ru + c] = tiles[h->c8 ? idx_c8_tile_u4(0, tok, c) : idx_tile_u4(0, tok, c)];
    } else if (which == SKO_TAB_HOT) {
        // the slots' rows in slot order (slot s lives in row slot_row[s])
        void* tmp = nullptr;
        e = hipMalloc(&tmp, size);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return set_err(SKO_E_NOMEM, "read table: %zu bytes of device memory", size);
        }
        e = launch_gather_slots(h->stream, static_cast<const uint16_t*>(src), h->slot_row + lb * h->S, h->S, h->R,
                                static_cast<uint16_t*>(tmp));
        if (e == hipSuccess) e = hipStreamSynchronize(h->stream);
        if (e == hipSuccess) e = hipMemcpy(dst, tmp, size, hipMemcpyDeviceToHost);
        (void)hipFree(tmp);
        if (e != hipSuccess) return device_fail(h, e, "read table");
    } else if (host) {
        std::memcpy(dst, src, size);
    } else {
        e = hipMemcpy(dst, src, size, hipMemcpyDeviceToHost);
        if (e != hipSuccess) return device_fail(h, e, "read table");
    }
    return SKO_OK;
}

int sko_get_stats(sko_handle* h, int32_t layer, sko_layer_stats* out) {
    int rc = check_handle(h);
    if (rc != SKO_OK) return rc;
    if (layer < 0 || layer >= h->L || !out) return set_err(SKO_E_INVAL, "bad layer or NULL output");
    DeviceGuard guard(h->cfg.device);
    unsigned long long v[8];
    hipError_t e = hipStreamSynchronize(h->stream);
    if (e != hipSuccess) return device_fail(h, e, "read stats sync");
    if ((rc = check_invariants(h)) != SKO_OK) return rc;
    e = hipMemcpy(v, h->stats + (size_t)layer * 8, sizeof(v), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return device_fail(h, e, "read stats");
    out->steps = h->step[layer];
    out->unique = (int64_t)v[1];
    out->hits = (int64_t)v[2];
    out->misses = (int64_t)v[3];
    out->evictions = (int64_t)v[4];
    out->direct_rows = (int64_t)v[6];
    out->h2d_bytes = ((int64_t)v[3] - (int64_t)v[6]) * kKvRowBytes;
    out->rescans = (int64_t)v[5];
    return SKO_OK;
}

int sko_set_timing(sko_handle* h, uint32_t stage_mask) {
    int rc = check_handle(h);
    if (rc != SKO_OK) return rc;
    DeviceGuard guard(h->cfg.device);
    (void)hipStreamSynchronize(h->stream);
    for (auto& p : h->pending) {
        h->spare.push_back(p.a);
        h->spare.push_back(p.b);
    }
    h->pending.clear();
    for (int i = 0; i < ST_COUNT; ++i) {
        h->total_ms[i] = 0.0;
        h->launches[i] = 0;
    }
    h->stamp_pending.clear();
    h->ovl_copy_ms = h->ovl_merge_ms = h->ovl_both_ms = 0.0;
    h->ovl_launches = 0;
    h->copy_spans.clear();
    h->timing_mask = stage_mask;
    return SKO_OK;
}

int sko_get_timing(sko_handle* h, double* total_ms, int64_t* launches, int32_t n) {
    int rc = check_handle(h);
    if (rc != SKO_OK) return rc;
    if (n < 0 || (n > 0 && (!total_ms || !launches))) return set_err(SKO_E_INVAL, "bad timing output");
    DeviceGuard guard(h->cfg.device);
    hipError_t e = hipStreamSynchronize(h->stream);
    if (e != hipSuccess) return device_fail(h, e, "timing sync");
    for (auto& p : h->pending) {
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) {
            h->total_ms[p.stage] += ms;
            h->launches[p.stage] += 1;
        }
        h->spare.push_back(p.a);
        h->spare.push_back(p.b);
    }
    h->pending.clear();
    if ((rc = collect_stamps(h)) != SKO_OK) return rc;
    for (int i = 0; i < n && i < ST_COUNT; ++i) {
        total_ms[i] = h->total_ms[i];
        launches[i] = h->launches[i];
    }
    return SKO_OK;
}

int sko_get_copy_overlap(sko_handle* h, double* copy_ms, double* merge_ms, double* overlap_ms,
                         int64_t* launches) {
    int rc = check_handle(h);
    if (rc != SKO_OK) return rc;
    if (!copy_ms || !merge_ms || !overlap_ms || !launches) return set_err(SKO_E_INVAL, "NULL output");
    DeviceGuard guard(h->cfg.device);
    const hipError_t e = hipStreamSynchronize(h->stream);
    if (e != hipSuccess) return device_fail(h, e, "overlap sync");
    if ((rc = collect_stamps(h)) != SKO_OK) return rc;
    *copy_ms = h->ovl_copy_ms;
    *merge_ms = h->ovl_merge_ms;
    *overlap_ms = h->ovl_both_ms;
    *launches = h->ovl_launches;
    return SKO_OK;
}

int sko_get_copy_spans(sko_handle* h, uint64_t* spans, int32_t max_spans, int32_t* n_spans, double* clock_khz) {
    int rc = check_handle(h);
    if (rc != SKO_OK) return rc;
    if (!n_spans || !clock_khz || max_spans < 0 || (max_spans > 0 && !spans))
        return set_err(SKO_E_INVAL, "bad copy-span output");
    DeviceGuard guard(h->cfg.device);
    const hipError_t e = hipStreamSynchronize(h->stream);
    if (e != hipSuccess) return device_fail(h, e, "copy-span sync");
    if ((rc = collect_stamps(h)) != SKO_OK) return rc;
    const int32_t n = (int32_t)(h->copy_spans.size() / 2);
    const int32_t m = std::min(n, max_spans);
    if (m > 0) std::memcpy(spans, h->copy_spans.data(), (size_t)m * 2 * sizeof(uint64_t));
    *n_spans = n;
    *clock_khz = h->clock_khz;
    return SKO_OK;
}

void sko_destroy(sko_handle* h) {
    if (!h) return;
    {
        DeviceGuard guard(h->cfg.device);
        (void)hipStreamSynchronize(h->stream);
        if (h->side) (void)hipStreamSynchronize(h->side);
        free_all(h);
    }
    delete h;
}

}  // extern "C"
