// Internal declarations of libsko: kernel launchers and device helpers.
// Used only by the library's own translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sko {

constexpr int kIdxDim = 64;
constexpr int kKvDim = 576;
constexpr int kVDim = 512;
constexpr int kIdxRowU4 = kIdxDim * 2 / 16;  // 8 x 16 B per indexer row
constexpr int kKvRowU4 = kKvDim * 2 / 16;    // 72 x 16 B per main-KV row
constexpr int kKvRowBytes = kKvDim * 2;      // 1152
constexpr int kHistBits = 12;                // first radix digit of the top-k
constexpr int kHistBins = 1 << kHistBits;
constexpr int kMaxMerge = 8192;              // D * k limit of the merge/LRU kernel
constexpr int kAttnHeadGroup = 16;           // heads per MFMA tile (M = 16)
constexpr int kAttnTileRows = 32;            // rows per attention tile

// Per (seq, position) row of the top-k selection.
struct RowMeta {
    int32_t bucket;        // first-digit bucket holding the k-th largest key (-1: none)
    int32_t above;         // keys in buckets above it
    int32_t need;          // winners still to take from the bucket
    int32_t bucket_count;  // keys in the bucket
    int32_t out_count;     // winners written so far
    int32_t cand_count;    // bucket keys staged for refinement
    int32_t pad[2];
};

struct GatherEntry {
    uint32_t src_row;  // b * cap + token  (within the layer's pool)
    uint32_t dst_row;  // b * S + slot     (within the layer's hot buffer)
};

// Launchers.  All enqueue on `st`; none synchronizes.
hipError_t launch_append_rows(hipStream_t st, const uint16_t* idx_src, const uint16_t* kv_src,
                              uint16_t* idx_layer, uint16_t* pool_layer, int32_t* ntok_layer,
                              int seq0, int nseq, int64_t n, int64_t cap, int32_t base);
hipError_t launch_set_ntok(hipStream_t st, int32_t* ntok_layer, int seq0, int nseq, int32_t value);

hipError_t launch_step_init(hipStream_t st, uint32_t* hist, RowMeta* meta, uint32_t* gather_total,
                            int rows);
hipError_t launch_score_hist(hipStream_t st, const uint16_t* idx_layer, const uint16_t* q_idx,
                             const int32_t* ntok_layer, uint32_t* keys, uint32_t* hist, int B,
                             int D, int64_t cap, int64_t max_tokens_now, int top_k);
hipError_t launch_topk_threshold(hipStream_t st, const uint32_t* hist, RowMeta* meta,
                                 const int32_t* ntok_layer, int B, int D, int top_k);
hipError_t launch_topk_filter(hipStream_t st, const uint32_t* keys, RowMeta* meta,
                              uint2* cand, int32_t* topk, const int32_t* cache_slots_layer,
                              const int32_t* ntok_layer, int B, int D, int64_t cap, int top_k,
                              int64_t max_tokens_now);
hipError_t launch_topk_refine(hipStream_t st, const uint2* cand, RowMeta* meta, int32_t* topk,
                              const int32_t* cache_slots_layer, int B, int D, int64_t cap,
                              int top_k);
hipError_t launch_merge_lru(hipStream_t st, const int32_t* topk, const int32_t* ntok_layer,
                            int32_t* cache_slots_layer, int32_t* slot_token_layer,
                            int32_t* last_use_layer, int B, int D, int top_k, int S,
                            int64_t cap, int32_t t, int32_t* misses, int32_t* victims,
                            int32_t* evict_old, int32_t* counts, GatherEntry* glist,
                            uint32_t* gather_total, unsigned long long* layer_stats);
hipError_t launch_gather_misses(hipStream_t st, const GatherEntry* glist,
                                const uint32_t* gather_total, const uint16_t* pool_layer,
                                uint16_t* hot_layer, int max_entries);
hipError_t launch_attn_partial(hipStream_t st, const int32_t* topk, const int32_t* cache_slots_layer,
                               const uint16_t* hot_layer, const uint16_t* q_attn,
                               const int32_t* ntok_layer, float* part_acc, float* part_ml,
                               int32_t* phys, int B, int D, int H, int top_k, int S, int64_t cap,
                               int rows_per_block, float scale);
hipError_t launch_attn_combine(hipStream_t st, const float* part_acc, const float* part_ml,
                               float* out, int B, int D, int H, int nchunk);

}  // namespace sko
