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
constexpr int kIdxTile = 64;                 // tokens per indexer tile (one wave)
constexpr int kHistBits = 12;                // first radix digit of the top-k
constexpr int kHistBins = 1 << kHistBits;
constexpr int kMaxMerge = 8192;              // D * k limit of the merge/LRU kernel
constexpr int kMaxHotSlots = 1 << 18;        // S limit (LDS bitmap of touched slots)
constexpr int kAttnHeadGroup = 16;           // heads per MFMA tile (M = 16)
constexpr int kAttnTileRows = 32;            // rows per attention tile
constexpr int kAttnMaxRowsPerBlock = 512;    // rows of one attention block (remap table)
constexpr int kFilterKeysPerThread = 16;
constexpr int kFilterSpan = 256 * kFilterKeysPerThread;  // keys per block pass
constexpr int kPreStage = 128;               // per-wave LDS staging of candidates
// The candidate floor of a row for the next step is one first-digit bin
// below the highest bin at which the row's count from the top reaches
// kFloorCover * k (so the floor admits well over k keys at the next step if
// the score distribution holds, and the next threshold has room to fall).
constexpr int kFloorCover = 2;
constexpr int kFloorRescanAll = kHistBins;   // a floor no key reaches


// Indexer cache layout in HBM (per layer): [B][ntiles][8 chunks][64 tokens]
// x 16 bytes, so that chunk c of 64 consecutive tokens is one contiguous
// 1 KB run: a wave reading one chunk for its 64 tokens is fully coalesced.
__host__ __device__ inline size_t idx_tile_u4(size_t seq_tiles_base, int64_t token, int chunk) {
    return ((seq_tiles_base + (size_t)(token / kIdxTile)) * kIdxRowU4 + chunk) * kIdxTile +
           (size_t)(token % kIdxTile);
}

// The int8 indexer (LIM C8): per token 64 int8 codes, as 4 chunks of 16
// bytes in the same tiled order ([B][ntiles][4 chunks][64 tokens] x 16 B),
// and one fp16 scale in a separate [B][ntiles * 64] array.  A quantized
// query row is kQc8Words words: 16 words of codes, then its fp16 scale bits.
constexpr int kIdxC8RowU4 = kIdxDim / 16;  // 4 x 16 B per int8 indexer row
constexpr int kQc8Words = kIdxDim / 4 + 1;
__host__ __device__ inline size_t idx_c8_tile_u4(size_t seq_tiles_base, int64_t token, int chunk) {
    return ((seq_tiles_base + (size_t)(token / kIdxTile)) * kIdxC8RowU4 + chunk) * kIdxTile +
           (size_t)(token % kIdxTile);
}

// Sets the message sko_last_error() returns; returns code.
int set_error(int code, const char* msg);

// Per (seq, position) row of the top-k selection.
struct RowMeta {
    int32_t bucket;        // first-digit bucket holding the k-th largest key (-1: none)
    int32_t above;         // keys in buckets above it
    int32_t need;          // winners still to take from the bucket
    int32_t bucket_count;  // keys in the bucket
    int32_t out_count;     // winners written so far
    int32_t cand_count;    // bucket keys staged for refinement
    int32_t pre_count;     // scored keys at or above the row's candidate floor
    int32_t pad;
};

// Words of the per-sequence winner bitmap (padded to 16 bytes).
__host__ __device__ inline int64_t winner_words(int64_t cap) { return ((cap + 31) / 32 + 3) / 4 * 4; }

// Recency list of one (layer, seq) hot buffer: a ring of slot ids (two
// buffers, `cur` selects the live one), -1 marking entries that moved.
// Live entries in [head, tail) are every slot once, ascending by
// (last_use, slot); pos[slot] is the ring index of its live entry.
struct RingState {
    int64_t head;
    int64_t tail;
    int32_t cur;
    int32_t pad[3];
};
__host__ __device__ inline int64_t ring_capacity(int S, int D, int k) {
    return ((2 * (int64_t)S + (int64_t)D * k) + 3) / 4 * 4;
}

struct GatherEntry {
    uint32_t src_row;  // b * cap + token  (within the layer's pool)
    uint32_t dst_row;  // b * S + slot     (within the layer's hot buffer)
};

// Launchers.  All enqueue on `st`; none synchronizes.
// recent_layer [B][576]: the device copy of each sequence's newest main-KV
// row (written with the last appended row when kv_src is given).
hipError_t launch_append_rows(hipStream_t st, const uint16_t* idx_src, const uint16_t* kv_src,
                              uint16_t* idx_layer, uint16_t* pool_layer, uint16_t* recent_layer,
                              int32_t* ntok_layer, int seq0, int nseq, int64_t n, int64_t cap, int64_t ntiles,
                              int32_t base);
// The same for the int8 indexer: each bf16 indexer row is rotated and
// quantized into its codes (idx_layer in the int8 layout) and fp16 scale.
hipError_t launch_append_rows_c8(hipStream_t st, const uint16_t* idx_src, const uint16_t* kv_src,
                                 uint8_t* idx_layer, uint16_t* scales_layer, uint16_t* pool_layer,
                                 uint16_t* recent_layer, int32_t* ntok_layer, int seq0, int nseq, int64_t n,
                                 int64_t cap, int64_t ntiles, int32_t base);
// The new token of every sequence, appended by the score launch itself
// (the fused append and decode step): its bf16 indexer row idx [B][64] and
// main-KV row kv [B][576], both on the device.  The launch scores the token
// from idx (its tile in the cache does not hold it yet); with `write` (the
// layer's first score launch) the block holding the token's tile also
// writes the indexer row to the cache (int8 indexer: its codes and scale),
// the main-KV row to recent, and ntok_out[b] = ntok_layer[b] + 1.  The host
// pool receives the main-KV row from the LRU-update launch.  idx null: no
// append.
struct ScoreAppend {
    const uint16_t* idx = nullptr;
    const uint4* kv = nullptr;
    void* idx_cache = nullptr;   // the layer's indexer cache (bf16 rows, or int8 codes)
    uint16_t* scales = nullptr;  // the layer's int8 indexer scales
    uint4* recent = nullptr;     // [B][72] the newest main-KV row of each sequence
    int32_t* ntok_out = nullptr;
    int write = 0;
};

// keys may be null (keys are then not stored); candidates (key, token |
// miss << 31) with first digit >= floor_layer[row] go to
// pre[row][0 .. meta[row].pre_count).  scales_layer non-null: the int8
// indexer (idx_layer in its layout); the queries are rotated and quantized
// in the launch and written to qc8 [B*D][kQc8Words] for the filter.
hipError_t launch_score_hist(hipStream_t st, const void* idx_layer, const uint16_t* q_idx,
                             const int32_t* ntok_layer, uint32_t* keys, uint32_t* hist,
                             const int32_t* floor_layer, uint2* pre, RowMeta* meta,
                             const int32_t* cache_slots_layer, int B, int D, int64_t kcap, int64_t cap,
                             int64_t ntiles, int64_t max_tokens_now, int cu_count,
                             const uint16_t* scales_layer, uint32_t* qc8, const ScoreAppend& app, int xc = -1);
// Also sets floor_layer for the next step (kFloorRescanAll when rescan_all).
// scales_layer / qc8 non-null: the int8 indexer (for the rescan path).
hipError_t launch_topk_filter(hipStream_t st, const uint32_t* hist, RowMeta* meta, const uint2* pre,
                              uint2* cand, int32_t* topk, const int32_t* cache_slots_layer,
                              const int32_t* ntok_layer, uint32_t* winners, uint32_t* miss_bits,
                              const void* idx_layer, const uint16_t* q_idx, int32_t* floor_layer,
                              bool rescan_all, int B, int D, int64_t cap, int64_t ntiles, int top_k,
                              int64_t max_tokens_now, const uint16_t* scales_layer, const uint32_t* qc8,
                              int xc = -1);
// Also finishes the top-k (split buckets) and clears the histograms and row
// records for the next step.  pool_newest non-null (the fused append): the
// merge block of each sequence also copies the newest token's main-KV row
// from recent_layer into pool_newest (the host pool of the layer, through
// its device mapping).
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
                            uint16_t* pool_newest, int xc = -1, int xcd_cus = 0);
// Dynamic LDS of the LRU-update launch for S slots and D*k winners (the
// touched-slot bitmap, the miss/union/victim lists and the sort marks), and
// the call that lets that kernel take it (before its first launch).
int merge_lru_touched_words(int S);
size_t merge_lru_lds_bytes(int S, int D, int top_k);
hipError_t prepare_merge_lru(size_t lds_bytes);
// Copy blocks of the early copy: copy_per_seq per sequence, each owning
// copy_words bitmap words (a multiple of 4, at most 1024).  xcd_cus > 0:
// the copy blocks run on one XCD of xcd_cus CUs (at least one block per CU).
void copy_shape(int B, int64_t max_tokens_now, int* copy_per_seq, int* copy_words, int xcd_cus = 0);
// Physical hot rows: each (layer, seq) has R = S + D*k rows; slot s lives
// in row slot_row[s], and the other D*k rows are spare, listed in
// spare [2][D*k] (two generations, the step's one chosen by t & 1).  The
// r-th miss of a step (in token order) is copied into spare row r of the
// step's generation, and the merge blocks give the r-th victim slot that
// row; the victim's old row becomes spare row r of the next generation.
// (miss_bits non-null: the launch also holds copy blocks that copy the rows
// marked in miss_bits [B][wpr] from the pool into those spare rows while the
// merge blocks update the LRU state; the bits stay set, the attention launch
// clears them.)  wrow non-null: the merge blocks write, per winner, the row
// the attention reads (-1: none) into wrow [B][D][k], and its slot into
// phys.  In every copy the newest token's row comes from recent_layer
// [B][576] instead of the pool.  With sort_winners (and at most 16
// positions) the merge blocks first rewrite each position's top-k list in
// token order, in every copy arrangement.
// Late copy from the pool into the misses' rows.  Work list: sequence b's
// entries are glist[b * D*k + r], r < counts[b][2] (destinations are row
// numbers from hot_layer).
hipError_t launch_gather_misses(hipStream_t st, const GatherEntry* glist, const int32_t* counts,
                                const uint16_t* pool_layer, const uint16_t* recent_layer,
                                const int32_t* ntok_layer, uint16_t* hot_layer, int B, int64_t cap, int mstride,
                                int max_entries);
// Resolves split threshold buckets, one row per block (for the early copy,
// so that the miss bitmap is complete before the merge launch).
hipError_t launch_topk_refine(hipStream_t st, RowMeta* meta, const uint2* cand, int32_t* topk, uint32_t* winners,
                              uint32_t* miss_bits, int B, int D, int top_k, int64_t cap, int xc = -1);
// The row each winner's attention reads: wrow non-null, the list the
// LRU-update launch wrote (the misses' words of miss_bits [B][wpr] are then
// cleared for the next step when miss_bits is non-null); otherwise
// slot_row[cache_slots[token]] (and with pool_layer non-null the launch
// also copies the rows that missed, packed topk entries < 0, from the pool
// into their rows; only valid when each row is read by one block: one
// position, at most 16 heads).  phase 1 attends only the rows resident at
// step start (tables), phase 2 only the misses (wrow).
hipError_t launch_attn_partial(hipStream_t st, const int32_t* topk, const int32_t* cache_slots_layer,
                               const int32_t* slot_row_layer, uint16_t* hot_layer, int R, const uint16_t* q_attn,
                               const uint16_t* pool_layer, const uint16_t* recent_layer, const int32_t* ntok_layer,
                               float* part_acc, float* part_ml, int32_t* phys, int B, int D, int H, int top_k, int S,
                               int64_t cap, int rows_per_block, float scale, const int32_t* wrow,
                               uint32_t* miss_bits, int phase, int xc = -1);
hipError_t launch_attn_combine(hipStream_t st, const float* part_acc, const float* part_ml,
                               float* out, int B, int D, int H, int nchunk, int xc = -1);
// Rings of n_seqs sequences: ring0 = 0..S-1, pos = identity, head 0, tail S;
// slot_row = identity, both spare generations S .. S+M-1.
hipError_t launch_init_rings(hipStream_t st, int32_t* ring0, int32_t* pos, RingState* state, int32_t* slot_row,
                             int32_t* spare, int64_t n_seqs, int S, int64_t C, int M);
// Rows slot_row[0 .. S) of one sequence's hot rows, in slot order, into dst
// [S][576] (device).
hipError_t launch_gather_slots(hipStream_t st, const uint16_t* hot_seq, const int32_t* slot_row_seq, int S, int R,
                               uint16_t* dst);

}  // namespace sko
