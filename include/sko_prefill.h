/*
 * sko_prefill.h — layerwise prefill offload on one MI355X (part of libsko).
 *
 * Follows "Layerwise and Sparse KV Cache Offloading Design" (vLLM-Ascend
 * design doc), section 3 "Layerwise Prefill Offload" (buffer planning,
 * execution pipeline, reuse invariant), and the FlashOffloading explainer's
 * prefill paragraphs (four layer-sized trays: B0 bound to layer 0, B1..B3
 * rotating; onload_layer_map sets how many layers ahead are loaded; the
 * exposed delay of a layer is the transfer time not covered by compute).
 *
 * The host pool holds every layer's KV (the single record); the device
 * holds a few layer-sized buffers.  For each layer of a prefill pass the
 * caller brackets its own compute with sko_prefill_begin_layer /
 * sko_prefill_end_layer on its compute stream; the library loads the
 * layer's cached prefix into the layer's buffer on a load stream (ahead of
 * time, as far as free buffers allow), makes the compute stream wait for
 * that load, and after the compute saves the rows the layer added back to
 * the host pool on a save stream.  A buffer is loaded again only after the
 * save of its previous occupant has completed (the reuse invariant, tracked
 * per physical buffer).  Loads and saves are hipMemcpyAsync between pinned
 * host memory and device memory (the copy engines), in the two directions
 * concurrently.  All calls are asynchronous unless stated.
 *
 * Error codes are those of sko.h (SKO_OK = 0, negative on error); on error
 * nothing is enqueued and sko_last_error() says why.
 */
#ifndef SKO_PREFILL_H
#define SKO_PREFILL_H

#include <stdint.h>

#include "sko.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * sko_prefill_plan — buffer planning (§3 "Buffer planning").  Host only.
 *   n_layers        N >= 1
 *   spec[N]         specification id per layer: layers with equal ids have
 *                   compatible main-KV layouts and may share a buffer
 *   independent[N]  1: the layer keeps a dedicated buffer; 0: reusable
 *   shared          B >= 0 shared buffers per group of compatible layers
 *   layer_bytes[N]  bytes of each layer's buffer (equal within one spec)
 *   buffer_of_layer[N]  out: physical buffer of each layer
 *   n_physical      out: number of physical buffers
 * Dedicated buffers are numbered first, in layer order; then, for each
 * group of compatible reusable layers (in order of first appearance) of R_g
 * layers, min(B, R_g) buffers taken in round-robin order by the group's
 * layers.  A uniform layout therefore needs I + min(B, R) buffers.
 * Errors: SKO_E_INVAL (N < 1, B < 0, a flag other than 0/1, a size <= 0,
 * two sizes for one spec, reusable layers with B = 0, NULL pointers).
 */
int sko_prefill_plan(int32_t n_layers, const int32_t* spec, const int32_t* independent, int32_t shared,
                     const int64_t* layer_bytes, int32_t* buffer_of_layer, int32_t* n_physical);

typedef struct sko_prefill_handle sko_prefill_handle;

typedef struct sko_prefill_config {
    int32_t num_layers;         /* N >= 1 */
    int32_t shared_buffers;     /* B >= 1 (all layers share one specification) */
    int32_t lookahead;          /* >= 1: while layer l computes, layers up to
                                   l + lookahead are loaded (the explainer's
                                   onload_layer_map), buffers permitting */
    int32_t row_bytes;          /* bytes of one token's KV row of one layer, > 0, multiple of 16 */
    int64_t capacity_tokens;    /* tokens one layer buffer holds (prefix + new rows), >= 1 */
    int32_t device;             /* HIP device ordinal */
    const int32_t* independent; /* [N] 1 = dedicated buffer (NULL: none); copied */
} sko_prefill_config;

/*
 * sko_prefill_create — plan the buffers (as sko_prefill_plan with one
 * spec), allocate them on the device, the pinned host pool
 * [N][capacity_tokens][row_bytes] (zeroed) and two copy streams.
 * compute_stream: the caller's stream (hipStream_t; NULL = default stream).
 * Errors: SKO_E_INVAL, SKO_E_NOMEM, SKO_E_DEVICE.
 */
int sko_prefill_create(const sko_prefill_config* cfg, void* compute_stream, sko_prefill_handle** out);

/* sko_prefill_destroy — synchronize the load, save and compute streams, then
 * free everything (NULL: no-op).  Device aliases of the layer buffers that
 * begin_layer handed out are invalid afterwards. */
int sko_prefill_destroy(sko_prefill_handle* h);

/*
 * sko_prefill_host_pool — the pinned host pool of `layer`: *rows points to
 * [capacity_tokens][row_bytes] bytes, the first *tokens of which are the
 * layer's KV.  The caller may write a cached prefix there between passes
 * (then sko_prefill_set_tokens), and read the saved rows after
 * sko_prefill_sync.
 */
int sko_prefill_host_pool(sko_prefill_handle* h, int32_t layer, void** rows, int64_t* tokens);

/* sko_prefill_set_tokens — tokens of `layer` already in its host pool (a
 * cached prefix written by the caller); only between passes.  Errors:
 * SKO_E_INVAL, SKO_E_CAPACITY, SKO_E_STATE (inside a pass). */
int sko_prefill_set_tokens(sko_prefill_handle* h, int32_t layer, int64_t tokens);

/*
 * sko_prefill_begin_layer — start layer `layer` of the current pass
 * (layers 0, 1, ..., N-1 in order; layer 0 starts a pass).  Issues the
 * prefix loads of layers up to layer + lookahead whose buffers are free,
 * and makes the compute stream wait for this layer's load.  *buffer: the
 * device address of the layer's buffer, whose first `tokens` rows (the
 * layer's KV so far) are valid in compute-stream order; the caller's
 * compute writes the layer's new rows right after them.
 * Errors: SKO_E_INVAL, SKO_E_STATE (out of order).
 */
int sko_prefill_begin_layer(sko_prefill_handle* h, int32_t layer, void** buffer);

/*
 * sko_prefill_end_layer — the layer's compute (enqueued on the compute
 * stream since begin) added `new_tokens` rows; save them to the host pool
 * after the compute, and issue the loads that waited for this buffer.
 * Errors: SKO_E_INVAL, SKO_E_CAPACITY (prefix + new > capacity),
 * SKO_E_STATE (not the layer begun last).
 */
int sko_prefill_end_layer(sko_prefill_handle* h, int32_t layer, int64_t new_tokens);

/* sko_prefill_sync — wait until every enqueued load, compute and save has
 * completed (host blocks). */
int sko_prefill_sync(sko_prefill_handle* h);

/*
 * sko_prefill_layer_timing — for `layer` in the last completed pass (after
 * sko_prefill_sync), in milliseconds: the load's duration (0 if the buffer
 * already held the layer), the time the compute stream waited for it (the
 * exposed delay: from the moment the compute stream was ready for the layer
 * to the end of the load, 0 if the load was done first), and the compute
 * time between begin and end.
 */
int sko_prefill_layer_timing(sko_prefill_handle* h, int32_t layer, float* load_ms, float* exposed_ms,
                             float* compute_ms);

/* Buffer assignment of a handle: buffer_of_layer[N], *n_physical. */
int sko_prefill_get_plan(sko_prefill_handle* h, int32_t* buffer_of_layer, int32_t* n_physical);

#ifdef __cplusplus
}
#endif

#endif /* SKO_PREFILL_H */
