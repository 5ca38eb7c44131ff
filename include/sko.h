/*
 * sko.h — C ABI of the sparse decode offload step (libsko.so, gfx950).
 *
 * The operation is the per-layer decode step of "Layerwise and Sparse KV
 * Cache Offloading Design" (vLLM-Ascend design doc), section 4 "Sparse
 * Decode Offload": the full main-KV history lives in a pinned host pool; the
 * device holds the indexer cache and a fixed-size per-layer hot buffer; each
 * step appends the new token's rows, selects top-k tokens with the indexer,
 * updates an LRU residency table, copies only the missed rows host->device,
 * remaps the winners to hot-buffer slots and runs sparse attention over them.
 * The hot-shelf mechanics (hits need no fetch, misses take evicted slots,
 * fixed shelf size, a cache_slots reverse index that is -1 for absent
 * tokens, index and residency packed into one int32 per top-k winner, MTP
 * position lists merged and deduplicated before loading) follow the
 * decode paragraphs of the FlashOffloading explainer on learnaivisually.com.
 *
 * Data types: bf16 values are passed as raw 16-bit patterns (uint16_t).
 * Row shapes are fixed: indexer row = 64 bf16 (128 B); main-KV row = 576
 * bf16 (1152 B: 512 latent + 64 rope); attention K = all 576 columns,
 * V = the first 512.
 *
 * Conventions for every call:
 *  - Return 0 (SKO_OK) or a negative SKO_E_* code; sko_last_error() gives a
 *    message for the calling thread's last failure.
 *  - Arguments are validated completely before anything is changed or
 *    enqueued: a rejected call leaves the handle and all buffers untouched
 *    (the pages' design fails a transfer on a layout mismatch instead of
 *    leaving partial data; section 7 of the same page).
 *  - A HIP runtime failure after validation marks the handle FAILED; every
 *    later call except sko_destroy returns SKO_E_STATE (no silent
 *    corruption, no retry).  So does a broken residency invariant that a
 *    decode step found on the device (a miss with no victim slot left, a
 *    slot or token out of range: that step's rows are incomplete): the
 *    kernel counts it, and the next synchronizing read (sko_read_step,
 *    sko_read_table, sko_get_stats) marks the handle FAILED and returns
 *    SKO_E_STATE.
 *  - A handle is not thread-safe: drive it from one host thread.
 *  - All device work is enqueued on the stream given at create (or set by
 *    sko_set_stream), in call order (SKO_FLAG_HIT_OVERLAP also uses an
 *    internal stream, forked from and joined back into that stream within
 *    each decode step).  sko_link_read_rate, sko_hbm_gather_rate and
 *    sko_hbm_read_rate are independent of any handle.
 */
#ifndef SKO_H
#define SKO_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SKO_OK 0
#define SKO_E_INVAL (-1)       /* bad argument or configuration */
#define SKO_E_NOMEM (-2)       /* host pinned or device allocation failed */
#define SKO_E_DEVICE (-3)      /* HIP runtime error (handle is now FAILED) */
#define SKO_E_CAPACITY (-4)    /* append beyond max_tokens */
#define SKO_E_STATE (-5)       /* handle FAILED (device error or broken invariant), or state not kept */
#define SKO_E_UNSUPPORTED (-6) /* valid but outside what the kernels support */

#define SKO_ALL_SEQS (-1)

#define SKO_INDEX_DIM 64
#define SKO_KV_DIM 576
#define SKO_V_DIM 512
#define SKO_MAX_MERGE 8192 /* limit on mtp_positions * top_k */

/* sko_config.flags: host-pool allocation mode (at most one). Default: the
 * HIP runtime's default coherence for mapped pinned memory. */
#define SKO_FLAG_POOL_COHERENT 0x1u    /* fine-grained: device reads bypass its caches */
#define SKO_FLAG_POOL_NONCOHERENT 0x2u /* coarse-grained: device may cache pool lines */
/* Also store every score key of each step (readable with SKO_BUF_KEYS);
 * costs 4 bytes per token and position of HBM writes in the score pass. */
#define SKO_FLAG_KEEP_KEYS 0x4u
/* Testing: no candidate floor, so every step selects through the rescan
 * path (same results, slower). */
#define SKO_FLAG_SELECT_RESCAN 0x8u
/* How the rows that missed reach the device (at most one of these three;
 * all give the same results).  Each missed row is copied once, into the
 * device row its victim slot takes over (see the hot buffer at
 * sko_create).  Default (SKO_FLAG_EARLY_COPY): as soon as the selection is
 * known, extra blocks of the LRU-update launch copy the misses from the
 * pool, concurrently with the update.  SKO_FLAG_LATE_COPY: one kernel after
 * the LRU update copies them.  SKO_FLAG_FUSED_COPY: the attention launch
 * reads each missed row from the pool and stores it before attending (the
 * fused Copy-SFA operator of [LSO-zh] §4); only with one position and at
 * most 16 heads, where each row is read by one attention block
 * (SKO_E_INVAL otherwise). */
#define SKO_FLAG_FUSED_COPY 0x10u
#define SKO_FLAG_LATE_COPY 0x20u
#define SKO_FLAG_EARLY_COPY 0x40u
/* The int8 indexer (LIM C8 of [LSO-zh] §4: the indexer rotates query and
 * key by a Hadamard transform and quantizes both to int8, and the selection
 * takes the int8 query with fp16 dequantization scales).  Appended bf16
 * indexer rows are rotated, x' = (1/8) H x with H the 64 x 64 Sylvester
 * Hadamard matrix, each x'[i] a binary32 sum in index order from +0, and
 * quantized per row: s = max|x'| / 127, code = round-half-even(x' / s)
 * clamped to [-127, 127], scale stored as binary16 (a zero row: codes and
 * scale 0).  The query of each (seq, position) is treated the same way at
 * decode.  Score = (float(dot) * s_k) * s_q in binary32 with dot the exact
 * int32 sum of code products; the selection, residency, LRU and attention
 * are unchanged.  Halves the indexer bytes the score pass reads. */
#define SKO_FLAG_INDEXER_C8 0x80u
/* With the early copy: the attention is split by residency at step start.
 * The rows that were resident (hits) are attended on an internal stream,
 * forked from the caller's stream once the selection is known, while the
 * LRU-update launch copies the misses in (the overlap of the fused Copy-SFA
 * operator of [LSO-zh] §4: attention on resident rows while the missing
 * rows are in flight); the rows that missed are attended after that launch,
 * and the combine, after the join, merges both phases' partials.  A hit's
 * slot and row do not change during the step (victims are slots not hit at
 * this step), so both phases read what the unsplit attention reads; the
 * output differs only in fp32 summation order.  SKO_E_INVAL with
 * SKO_FLAG_FUSED_COPY or SKO_FLAG_LATE_COPY. */
#define SKO_FLAG_HIT_OVERLAP 0x100u
/* Testing only: the LRU-update launch reports a broken residency invariant
 * for sequence 0 at every step while doing its normal work, so that the
 * reporting path below can be exercised without a real fault. */
#define SKO_FLAG_TEST_VIOLATION 0x200u
/* Kept off one XCD (for two or more handles whose steps overlap, each on its
 * own stream, e.g. the two halves of a batch): the copy blocks of the
 * LRU-update launch run only on XCD 0, one block per CU, and every other
 * block of the decode step runs on the other seven XCDs.  A kernel's HBM
 * loads on a CU that also has host reads in flight wait behind them (the
 * kernel takes several times as long), so only with the host reads on CUs
 * of their own can one handle's selection and attention run while another
 * handle's misses cross the host link ([FO] decode paragraphs: miss loads
 * overlapped with the other work of the step).  Results are those of the
 * default early copy, bit for bit.  sko_create checks that the device deals
 * the blocks of a launch to 8 XCDs in a fixed stripe (block i on XCD
 * (i + o) mod 8) and fails with SKO_E_UNSUPPORTED otherwise; SKO_E_INVAL
 * with SKO_FLAG_FUSED_COPY, SKO_FLAG_LATE_COPY or SKO_FLAG_HIT_OVERLAP.
 * sko_append_token's own launch is not kept off XCD 0. */
#define SKO_FLAG_XCD_SPLIT 0x400u

typedef struct sko_handle sko_handle;

typedef struct sko_config {
    int32_t num_layers;    /* L >= 1 */
    int32_t batch;         /* B >= 1 sequences */
    int64_t max_tokens;    /* per-sequence capacity, 1 <= cap < 2^31 - 1 */
    int32_t index_dim;     /* must be 64 */
    int32_t kv_dim;        /* must be 576 */
    int32_t v_dim;         /* must be 512 */
    int32_t num_heads;     /* H >= 1 attention heads sharing the latent rows */
    int32_t top_k;         /* k >= 1 winners per query position */
    int32_t hot_slots;     /* S per (layer, seq); S >= mtp_positions * top_k */
    int32_t mtp_positions; /* D >= 1 query positions per step (MTP3 = 4) */
    float attn_scale;      /* finite, > 0; usually 1/sqrt(576) */
    int32_t device;        /* HIP device ordinal */
    uint32_t flags;        /* SKO_FLAG_* bits, 0 = defaults */
} sko_config;

/* Per-sequence counters of the most recent sko_decode_step on a layer. */
typedef struct sko_seq_counts {
    int32_t unique;    /* |U|: distinct winners over all positions */
    int32_t hits;      /* winners already resident */
    int32_t misses;    /* unique misses = rows copied host -> device */
    int32_t evictions; /* victims that held a token */
    int32_t selected;  /* min(top_k, tokens present) */
    int32_t tokens;    /* tokens present (L_t) */
    int32_t step;      /* the layer's step stamp t used */
    int32_t reserved;
} sko_seq_counts;

/* Cumulative counters of one layer since create. */
typedef struct sko_layer_stats {
    int64_t steps;
    int64_t unique;
    int64_t hits;
    int64_t misses;
    int64_t evictions;
    int64_t h2d_bytes; /* (misses - direct_rows) * 1152: rows read over the host link */
    int64_t rescans;   /* (seq, position) rows whose threshold fell below the
                          candidate floor, so the filter rescanned the row */
    int64_t direct_rows; /* misses that were the sequence's newest token: its
                            row is copied from the device copy kept by
                            sko_append_token, not read from the host pool */
} sko_layer_stats;

/*
 * sko_create — validate cfg, then allocate and own every buffer of the
 * offload state:
 *   host pool     pinned, device-mapped  [L][B][cap][576] bf16
 *   indexer cache device                 [L][B][cap][64]  bf16
 *   hot buffer    device                 [L][B][S+D*k][576] bf16 (zeroed):
 *                 S rows hold the S slots, the other D*k are spare; a
 *                 step copies its r-th miss (token order) into its r-th
 *                 spare row, the r-th victim slot takes that row over and
 *                 the victim's old row becomes spare.  Which row holds a
 *                 slot is internal: the slot contents ([LSO] §4, the
 *                 fixed-size hot buffer of S slots) are what
 *                 sko_read_table(SKO_TAB_HOT) returns.
 *   cache_slots   device                 [L][B][cap] int32 = -1
 *   slot_token    device                 [L][B][S]   int32 = -1
 *   last_use      device                 [L][B][S]   int32 = -1
 * plus per-step scratch.  `stream` is a hipStream_t (NULL = null stream)
 * owned by the caller.  On error *out = NULL and nothing leaks.
 * Errors: SKO_E_INVAL (NULL pointer, a dimension other than 64/576/512,
 * L/B/H/k/D < 1, S < D*k, cap out of range, bad scale, unknown or
 * conflicting flags),
 * SKO_E_UNSUPPORTED (D*k > SKO_MAX_MERGE, L*B*(S+D*k) hot rows or
 * B*max_tokens or B*S at or beyond the int32/uint32 row-number range),
 * SKO_E_NOMEM, SKO_E_DEVICE.
 */
int sko_create(const sko_config* cfg, void* stream, sko_handle** out);

/*
 * Replace the stream used for later calls (caller-owned hipStream_t).  The
 * new stream is made to wait (by an event) for everything already enqueued
 * on the old one, so no host synchronization is needed around a switch, and
 * later synchronizing calls (reads, sko_destroy) cover the work of both.
 * The old stream must stay valid until this call returns.
 * Errors: SKO_E_INVAL (NULL handle), SKO_E_STATE, SKO_E_DEVICE.
 */
int sko_set_stream(sko_handle* h, void* stream);

/*
 * sko_append_token — write n new tokens per sequence at the end of each
 * selected sequence: the main-KV rows go to their logical slots in the host
 * pool, the indexer rows to the device indexer cache ([LSO] §4 "Decode
 * step", first two items; the "Decode current KV to Decode host" row of the
 * transfer-granularity table: token rows).  A prefix load is one call with
 * n = context length.  The last main-KV row of each sequence is also kept
 * in a device copy: a new token is produced on the device, and when it is
 * selected at its first step (a miss, since it was never resident) its row
 * is moved into the hot buffer from that copy instead of over the host
 * link (counted in sko_layer_stats.direct_rows; results are unchanged).
 *   seq       0 <= seq < B, or SKO_ALL_SEQS (rows for sequence b start at
 *             row b*n of both inputs)
 *   idx_rows  [rows][64] bf16, kv_rows [rows][576] bf16, row-major,
 *             rows = n or B*n
 *   src_on_device  0: host memory (read before the call returns);
 *                  1: device memory, read in stream order (keep it live
 *                     until the stream passes this call)
 * Errors: SKO_E_INVAL, SKO_E_CAPACITY (any selected sequence would exceed
 * max_tokens; checked for all before any write), SKO_E_STATE.
 */
int sko_append_token(sko_handle* h, int32_t layer, int32_t seq, const void* idx_rows,
                     const void* kv_rows, int64_t n, int32_t src_on_device);

/*
 * sko_decode_step — one sparse decode step of `layer` for all B sequences
 * and D positions, enqueued on the stream (asynchronous; no host sync):
 * score -> packed top-k -> merge/dedupe -> LRU update -> miss-only gather
 * -> remap -> attention ([LSO] §4 "Decode step" items 3-7).  The gather
 * is done early (by extra blocks of the LRU-update launch), late, or inside
 * the attention launch, see SKO_FLAG_EARLY_COPY.  Everything runs on the
 * caller's stream (with SKO_FLAG_HIT_OVERLAP, part of the attention runs on
 * an internal stream that is forked from and joined back into it by events
 * within the call's stream order).
 *   q_idx   device [B][D][64] bf16 indexer queries
 *   q_attn  device [B][D][H][576] bf16 attention queries
 *   out     device [B][D][H][512] fp32 attention output
 * A sequence with no tokens selects nothing and gets a zero output.
 * The layer's step stamp advances by one per call.
 * Selection keeps, per (seq, position), the scored keys at or above a floor
 * set half an octave of score below the previous step's threshold; when
 * fewer than k keys reach it the row is rescanned from the indexer.  Both
 * paths give the same winners (the first step of a layer keeps every key).
 * Reproducible: the LRU-update launch puts each position's winners in token
 * order before the attention reads them, so the same inputs give the same
 * output bits on any stream and in any run (with at most 16 positions and
 * without SKO_FLAG_HIT_OVERLAP, whose hit attention reads the lists while
 * that launch runs; there the winners keep the order in which the selection
 * appended them and only the output's rounding varies).
 * Errors: SKO_E_INVAL (bad layer or NULL pointer), SKO_E_STATE, SKO_E_DEVICE.
 */
int sko_decode_step(sko_handle* h, int32_t layer, const void* q_idx, const void* q_attn,
                     float* out);

/*
 * sko_decode_step_append — sko_append_token of one new token for every
 * sequence (rows on the device) followed by sko_decode_step, in one call
 * with one launch fewer ([LSO] §4 "Decode step": the new token's rows are
 * written, then the step runs over every token including it).  The score
 * launch scores the new token from idx_rows and writes its indexer row to
 * the device cache and its main-KV row to the device copy of the newest
 * row; the LRU-update launch writes that row to the host pool.  Results,
 * tables and pool contents are those of the two calls.
 *   idx_rows  device [B][64] bf16, kv_rows device [B][576] bf16, read in
 *             stream order (keep them live until the stream passes this
 *             call)
 *   q_idx, q_attn, out  as for sko_decode_step
 * Errors: SKO_E_INVAL (bad layer or NULL pointer), SKO_E_CAPACITY (any
 * sequence at max_tokens; checked before any work), SKO_E_STATE,
 * SKO_E_DEVICE.
 */
int sko_decode_step_append(sko_handle* h, int32_t layer, const void* idx_rows, const void* kv_rows,
                           const void* q_idx, const void* q_attn, float* out);

/*
 * sko_decode_step_static — sko_decode_step for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same step, arguments and results,
 * but the kernels' per-step scratch (selection histograms and row records,
 * candidate lists, winner and miss bitmaps, the per-winner row pairs, the
 * gather list, the split-K attention partials, the int8 query codes) comes
 * from one static device array of the library, SKO_STATIC_SCRATCH_BYTES
 * (160 MiB), instead of the handle's own.  The call allocates nothing.
 * Each device the library runs on holds that array until the process ends;
 * its address is looked up at sko_create.  Every call on a device shares
 * the array, which keeps the last call's contents (the call clears what
 * must start cleared): calls that can overlap on one device (two handles,
 * or streams not ordered against each other) race.  No stage timing.
 * Errors: as sko_decode_step, plus SKO_E_UNSUPPORTED when the handle's step
 * needs more scratch than the array holds (about 16 B per token of
 * capacity per sequence and position, plus the attention partials), and
 * SKO_E_DEVICE when the array's address could not be found at create.
 */
#define SKO_STATIC_SCRATCH_BYTES (160ull << 20)
int sko_decode_step_static(sko_handle* h, int32_t layer, const void* q_idx, const void* q_attn,
                            float* out);

/* Buffers of the most recent sko_decode_step (any layer), for inspection. */
enum sko_step_buffer {
    SKO_BUF_TOPK = 1,      /* int32 [B][D][k]: packed winners (bit31 = miss), first `selected` valid, token order
                              (the selection's order with SKO_FLAG_HIT_OVERLAP or more than 16 positions) */
    SKO_BUF_PHYS = 2,      /* int32 [B][D][k]: hot slot of each TOPK entry, same order */
    SKO_BUF_COUNTS = 3,    /* sko_seq_counts [B] */
    SKO_BUF_MISSES = 4,    /* int32 [B][D*k]: miss tokens ascending, first `misses` valid */
    SKO_BUF_VICTIMS = 5,   /* int32 [B][D*k]: slot given to MISSES[r] */
    SKO_BUF_EVICT_OLD = 6, /* int32 [B][D*k]: previous owner of VICTIMS[r] or -1 */
    SKO_BUF_KEYS = 7       /* uint32 [B][D][cap]: ordered score keys, first `tokens` valid;
                              only with SKO_FLAG_KEEP_KEYS, else SKO_E_STATE */
};

/*
 * sko_read_step — synchronize the stream and copy one step buffer to host
 * memory `dst` of `bytes` (must equal the buffer's size).
 */
int sko_read_step(sko_handle* h, int32_t which, void* dst, int64_t bytes);

/* Per-(layer, seq) state tables, for inspection. */
enum sko_table {
    SKO_TAB_CACHE_SLOTS = 1, /* int32 [cap] */
    SKO_TAB_SLOT_TOKEN = 2,  /* int32 [S] */
    SKO_TAB_LAST_USE = 3,    /* int32 [S] */
    SKO_TAB_HOT = 4,         /* bf16 [S][576]: the row of each slot, in slot order */
    SKO_TAB_INDEXER = 5,     /* bf16 [cap][64]; with SKO_FLAG_INDEXER_C8 int8 codes [cap][64] */
    SKO_TAB_POOL = 6,        /* bf16 [cap][576] (host pool) */
    SKO_TAB_NTOK = 7,        /* int64 [1] tokens present */
    SKO_TAB_INDEXER_SCALE = 8, /* fp16 [cap] scales; only with SKO_FLAG_INDEXER_C8, else SKO_E_STATE */
    SKO_TAB_SLOT_ROW = 9,    /* int32 [S]: the device row holding each slot (0 <= row < S + D*k) */
    SKO_TAB_SPARE_ROWS = 10  /* int32 [D*k]: the spare rows the layer's next step copies its misses into;
                                with SKO_TAB_SLOT_ROW a permutation of 0 .. S + D*k - 1 */
};

/*
 * sko_read_table — synchronize the stream and copy one table of
 * (layer, seq) to host memory `dst` of `bytes` (must equal its size).
 */
int sko_read_table(sko_handle* h, int32_t layer, int32_t seq, int32_t which, void* dst,
                   int64_t bytes);

/* Cumulative counters of `layer` (synchronizes the stream). */
int sko_get_stats(sko_handle* h, int32_t layer, sko_layer_stats* out);

/*
 * Kernel timing: stages whose bit is set in `stage_mask` (bit i = stage i,
 * names from sko_stage_name) are bracketed by HIP events on the handle's
 * stream, and the elapsed times are accumulated per stage.  Each event pair
 * costs device time, so time only the stages of interest.  sko_set_timing
 * (any mask, 0 disables) synchronizes and clears the totals.
 * sko_get_timing synchronizes and returns the totals (ms) and launch counts
 * for up to `n` stages.
 */
int sko_set_timing(sko_handle* h, uint32_t stage_mask);
int sko_get_timing(sko_handle* h, double* total_ms, int64_t* launches, int32_t n);

/*
 * sko_get_copy_overlap — how long the early copy ran beside the LRU update
 * (the overlap of the miss transfer with other step work; the explainer's
 * decode paragraphs report 90-98 % of miss loads overlapped at batch >= 16).
 * While the stage "merge_lru" is timed (sko_set_timing) and the early copy
 * is in use, every block of the LRU-update launch records its start and end
 * on the device's constant-rate clock.  Per launch: the copy span (first copy
 * block's start to last copy block's end), the merge span (the same over the
 * LRU-update blocks) and their intersection.  Returns the sums (ms) and the
 * number of launches recorded since the last sko_set_timing; synchronizes.
 * At most 1024 launches are recorded between two reads (sko_get_timing also
 * reads); later ones are skipped.
 */
int sko_get_copy_overlap(sko_handle* h, double* copy_ms, double* merge_ms, double* overlap_ms,
                         int64_t* launches);

/*
 * sko_get_copy_spans — the copy span of every launch recorded as for
 * sko_get_copy_overlap (the first copy block's start and the last copy
 * block's end, in ticks of the device's constant-rate clock, which all
 * handles on the device share), in recording order: spans[2 i], spans[2 i +
 * 1] for launch i.  With two or more handles whose steps overlap (the two
 * micro-batches of SKO_FLAG_XCD_SPLIT), the union of all handles' spans is
 * the time during which any miss row is being copied over the host link.
 * Writes at most max_spans pairs; *n_spans receives the number recorded
 * (which may be larger; at most 65 536 are kept between two
 * sko_set_timing calls), *clock_khz the clock's rate.  Synchronizes.
 * SKO_E_INVAL for NULL outputs or max_spans < 0.
 */
int sko_get_copy_spans(sko_handle* h, uint64_t* spans, int32_t max_spans, int32_t* n_spans, double* clock_khz);
const char* sko_stage_name(int32_t stage);
int32_t sko_num_stages(void);

/*
 * sko_link_read_rate — the host-link read rate as kernels see it: a
 * streaming kernel reads `bytes` of pinned, device-mapped host memory
 * (contiguous 16-byte loads), timed by HIP events over `reps` launches at
 * each of a few grid sizes; *gbps receives the best rate (1e9 bytes/s).
 * The decode step moves only missed rows over that link ([LSO] §4 "Decode
 * step"; the early, late and fused copies all read the pool this way), so
 * this is their ceiling for contiguous data, beside the bulk hipMemcpy rate
 * of the copy engines.  Allocates, uses and frees its own buffer on
 * `device`; synchronous; independent of any handle.
 * Errors: SKO_E_INVAL (NULL gbps, device < 0, bytes < 1 MiB or not a
 * multiple of 16, reps < 1), SKO_E_NOMEM, SKO_E_DEVICE.
 */
int sko_link_read_rate(int32_t device, int64_t bytes, int32_t reps, float* gbps);

/*
 * sko_hbm_gather_rate — the HBM read rate of the attention's access pattern:
 * whole 1152-byte rows at random distinct slots of `seqs` sequences of
 * `slots` rows each, `rows_per_seq` rows per sequence, gathered by blocks of
 * 128 rows one 32-row tile at a time (the attention reads the selected rows
 * of the hot buffer this way, [LSO] §4 "Decode step" item 7).  Eight copies
 * of the rows are read in rotation, so a launch finds little of its rows in
 * the on-die caches; *gbps receives the average over reps x 8 timed
 * launches (1e9 bytes/s).  Allocates 8 x seqs x slots x 1152 bytes of device
 * memory, uses and frees it on `device`; synchronous; independent of any
 * handle.
 * Errors: SKO_E_INVAL (NULL gbps, device < 0, seqs < 1, rows_per_seq not a
 * positive multiple of 128, slots < rows_per_seq, seqs*slots or
 * seqs*rows_per_seq above 2^22, reps < 1), SKO_E_NOMEM, SKO_E_DEVICE.
 */
int sko_hbm_gather_rate(int32_t device, int32_t seqs, int32_t slots, int32_t rows_per_seq, int32_t reps,
                        float* gbps);

/*
 * sko_hbm_read_rate — the HBM rate of a plain streaming read, the access
 * pattern of the indexer score pass (every indexer row of the layer read
 * once per step, [LSO] §4 "Decode step" item 1): `bytes` bytes read with
 * 16-byte loads, one block per compute unit, each block a contiguous part.
 * Four buffers of `bytes` bytes are read in rotation, so a launch finds
 * little of its buffer in the on-die caches; *gbps receives the median of
 * reps x 4 launches each timed on its own (1e9 bytes/s).  Allocates 4 x
 * bytes of device memory, uses and frees it on `device`; synchronous;
 * independent of any handle.
 * Errors: SKO_E_INVAL (NULL gbps, device < 0, bytes below 1 MiB, above
 * 2 GiB or not a multiple of 16, reps outside 1..64), SKO_E_NOMEM,
 * SKO_E_DEVICE.
 */
int sko_hbm_read_rate(int32_t device, int64_t bytes, int32_t reps, float* gbps);

/* Destroy: synchronize the stream, free everything. NULL is a no-op. */
void sko_destroy(sko_handle* h);

/* Message for the calling thread's last failure ("" if none). */
const char* sko_last_error(void);

/* Library version string. */
const char* sko_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SKO_H */
