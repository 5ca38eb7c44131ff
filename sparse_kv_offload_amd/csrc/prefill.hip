// Layerwise prefill offload: buffer planning and the load / compute / save
// pipeline over a few device buffers.
//
// "Layerwise and Sparse KV Cache Offloading Design" section 3: many logical
// layers map onto fewer physical buffers (dedicated ones, then shared ones
// in round-robin order, never across incompatible layouts); per layer the
// cached prefix is loaded, the buffer is used only once it is safe to
// overwrite, the layer computes and updates its KV, the update is saved to
// host memory, and later layers are prefetched meanwhile; a buffer is not
// reused before every consumer of its previous contents (its save) has
// finished, tracked per physical buffer.  The FlashOffloading explainer's
// prefill paragraphs give the four-tray instance (B0 bound to layer 0,
// B1..B3 rotating) and the lookahead of the loads (onload_layer_map).
//
// MI355X mapping: the buffers live in HBM, the host pool is pinned host
// memory, loads and saves are hipMemcpyAsync on two streams of their own
// (the copy engines move host-to-device and device-to-host concurrently),
// and every ordering is a HIP event: the compute stream waits for a layer's
// load, the save stream waits for the layer's compute, and the load stream
// waits for the save of the buffer's previous occupant.  No host thread
// waits inside a pass.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "sko_internal.h"
#include "sko_prefill.h"

using namespace sko;

namespace {

int perr(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int perr(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    return set_error(code, buf);
}

struct LayerEvents {
    hipEvent_t load_start = nullptr, load_end = nullptr;  // on the load stream
    hipEvent_t ready = nullptr, begun = nullptr, ended = nullptr;  // on the compute stream
    bool loaded = false;  // a load was issued for this layer in the current pass
};

}  // namespace

struct sko_prefill_handle {
    sko_prefill_config cfg{};
    int N = 0;
    std::vector<int32_t> dedicated;   // [N]
    std::vector<int32_t> buf_of;      // [N]
    int nbuf = 0;
    size_t buf_bytes = 0;             // capacity_tokens * row_bytes
    std::vector<uint8_t*> bufs;       // device buffers
    uint8_t* pool = nullptr;          // pinned host [N][capacity][row_bytes]
    std::vector<int64_t> tokens;      // [N] rows in the host pool
    hipStream_t compute = nullptr, load = nullptr, save = nullptr;
    std::vector<hipEvent_t> saved;    // [nbuf] save of the buffer's last occupant
    std::vector<int32_t> holder;      // [nbuf] layer whose KV the buffer holds (-1: none)
    std::vector<int32_t> pending_save;  // [nbuf] 1 while a save into the pool may still run
    std::vector<int32_t> busy;        // [nbuf] 1 from a layer's load (or reuse) until its end
    std::vector<LayerEvents> ev;      // [N]
    int next_layer = 0;               // next layer to begin
    int begun_layer = -1;             // layer begun and not yet ended
    int next_load = 0;                // next layer whose load is to be issued in this pass
    bool failed = false;
};

namespace {

int fail(sko_prefill_handle* h, hipError_t e, const char* what) {
    h->failed = true;
    return perr(SKO_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

struct Guard {
    int prev = -1;
    bool ok = false;
    explicit Guard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) prev = -1;
        ok = hipSetDevice(dev) == hipSuccess;
    }
    ~Guard() {
        if (prev >= 0) (void)hipSetDevice(prev);
    }
};

// Plan with validation; buffer_of_layer may alias nothing else.
int plan(int32_t n, const int32_t* spec, const int32_t* independent, int32_t shared, const int64_t* bytes,
         int32_t* buffer_of_layer, int32_t* n_physical) {
    if (n < 1 || shared < 0) return perr(SKO_E_INVAL, "n_layers must be >= 1 and shared >= 0");
    if (!spec || !independent || !bytes || !buffer_of_layer || !n_physical)
        return perr(SKO_E_INVAL, "NULL pointer");
    for (int l = 0; l < n; ++l) {
        if (independent[l] != 0 && independent[l] != 1) return perr(SKO_E_INVAL, "layer %d: flag must be 0 or 1", l);
        if (bytes[l] <= 0) return perr(SKO_E_INVAL, "layer %d: size must be > 0", l);
    }
    for (int l = 0; l < n; ++l)
        for (int m = 0; m < l; ++m)
            if (spec[l] == spec[m] && bytes[l] != bytes[m])
                return perr(SKO_E_INVAL, "layers %d and %d share a spec but not a size", m, l);
    std::vector<int32_t> out(n, -1);
    int next = 0;
    for (int l = 0; l < n; ++l)
        if (independent[l]) out[l] = next++;
    std::vector<int32_t> groups;
    for (int l = 0; l < n; ++l)
        if (!independent[l] && std::find(groups.begin(), groups.end(), spec[l]) == groups.end())
            groups.push_back(spec[l]);
    for (int32_t g : groups) {
        if (shared == 0) return perr(SKO_E_INVAL, "reusable layers need at least one shared buffer");
        int members = 0;
        for (int l = 0; l < n; ++l) members += (!independent[l] && spec[l] == g);
        const int nb = std::min(shared, members);
        int r = 0;
        for (int l = 0; l < n; ++l)
            if (!independent[l] && spec[l] == g) out[l] = next + (r++ % nb);
        next += nb;
    }
    std::copy(out.begin(), out.end(), buffer_of_layer);
    *n_physical = next;
    return SKO_OK;
}

void free_all(sko_prefill_handle* h) {
    for (uint8_t* b : h->bufs)
        if (b) (void)hipFree(b);
    if (h->pool) (void)hipHostFree(h->pool);
    for (hipEvent_t e : h->saved)
        if (e) (void)hipEventDestroy(e);
    for (LayerEvents& e : h->ev)
        for (hipEvent_t x : {e.load_start, e.load_end, e.ready, e.begun, e.ended})
            if (x) (void)hipEventDestroy(x);
    if (h->load) (void)hipStreamDestroy(h->load);
    if (h->save) (void)hipStreamDestroy(h->save);
}

int check(sko_prefill_handle* h) {
    if (!h) return perr(SKO_E_INVAL, "NULL handle");
    if (h->failed) return perr(SKO_E_STATE, "handle FAILED by an earlier device error");
    return SKO_OK;
}

uint8_t* pool_rows(sko_prefill_handle* h, int layer, int64_t row) {
    return h->pool + ((size_t)layer * h->cfg.capacity_tokens + row) * h->cfg.row_bytes;
}

// Issue the prefix loads of layers next_load .. limit whose buffers are
// free: no layer is using the buffer (its last occupant has ended, so that
// occupant's save is enqueued and the load stream can wait for it).  Loads
// stay in layer order.  Every save goes to one stream, so waiting for the
// buffer's last save also covers the earlier saves of the layer being
// loaded (its rows of the previous pass).
int issue_loads(sko_prefill_handle* h, int limit) {
    limit = std::min(limit, h->N - 1);
    while (h->next_load <= limit) {
        const int j = h->next_load;
        const int b = h->buf_of[j];
        LayerEvents& e = h->ev[j];
        if (h->busy[b]) break;
        if (h->holder[b] == j && h->dedicated[j]) {
            // a dedicated buffer still holding the layer: nothing to load
            e.loaded = false;
            h->busy[b] = 1;
            ++h->next_load;
            continue;
        }
        hipError_t r = hipSuccess;
        if (h->pending_save[b]) r = hipStreamWaitEvent(h->load, h->saved[b], 0);
        if (r == hipSuccess) r = hipEventRecord(e.load_start, h->load);
        const size_t bytes = (size_t)h->tokens[j] * h->cfg.row_bytes;
        if (r == hipSuccess && bytes)
            r = hipMemcpyAsync(h->bufs[b], pool_rows(h, j, 0), bytes, hipMemcpyHostToDevice, h->load);
        if (r == hipSuccess) r = hipEventRecord(e.load_end, h->load);
        if (r != hipSuccess) return fail(h, r, "prefix load");
        e.loaded = true;
        h->holder[b] = j;
        h->busy[b] = 1;
        ++h->next_load;
    }
    return SKO_OK;
}

}  // namespace

extern "C" {

int sko_prefill_plan(int32_t n_layers, const int32_t* spec, const int32_t* independent, int32_t shared,
                     const int64_t* layer_bytes, int32_t* buffer_of_layer, int32_t* n_physical) {
    return plan(n_layers, spec, independent, shared, layer_bytes, buffer_of_layer, n_physical);
}

int sko_prefill_create(const sko_prefill_config* cfg, void* compute_stream, sko_prefill_handle** out) {
    if (!cfg || !out) return perr(SKO_E_INVAL, "NULL config or output");
    *out = nullptr;
    const sko_prefill_config c = *cfg;
    if (c.num_layers < 1 || c.shared_buffers < 1 || c.lookahead < 1 || c.row_bytes <= 0 || c.row_bytes % 16 ||
        c.capacity_tokens < 1 || c.device < 0)
        return perr(SKO_E_INVAL, "num_layers, shared_buffers, lookahead, capacity_tokens >= 1; row_bytes a "
                                 "positive multiple of 16; device >= 0");
    const int N = c.num_layers;
    std::vector<int32_t> indep(N, 0), spec(N, 0), buf_of(N, -1);
    if (c.independent)
        for (int l = 0; l < N; ++l) indep[l] = c.independent[l];
    const int64_t bytes = c.capacity_tokens * (int64_t)c.row_bytes;
    std::vector<int64_t> sizes(N, bytes);
    int32_t nbuf = 0;
    int rc = plan(N, spec.data(), indep.data(), c.shared_buffers, sizes.data(), buf_of.data(), &nbuf);
    if (rc != SKO_OK) return rc;
    Guard g(c.device);
    if (!g.ok) return perr(SKO_E_DEVICE, "hipSetDevice(%d) failed", c.device);

    sko_prefill_handle* h = new sko_prefill_handle();
    h->cfg = c;
    h->cfg.independent = nullptr;
    h->N = N;
    h->dedicated = indep;
    h->buf_of = buf_of;
    h->nbuf = nbuf;
    h->buf_bytes = (size_t)bytes;
    h->compute = static_cast<hipStream_t>(compute_stream);
    h->tokens.assign(N, 0);
    h->holder.assign(nbuf, -1);
    h->pending_save.assign(nbuf, 0);
    h->busy.assign(nbuf, 0);
    h->bufs.assign(nbuf, nullptr);
    h->saved.assign(nbuf, nullptr);
    h->ev.resize(N);
    bool ok = true;
    for (int b = 0; b < nbuf && ok; ++b) ok = hipMalloc((void**)&h->bufs[b], h->buf_bytes) == hipSuccess;
    if (ok) ok = hipHostMalloc((void**)&h->pool, (size_t)N * h->buf_bytes, hipHostMallocDefault) == hipSuccess;
    if (!ok) {
        (void)hipGetLastError();
        free_all(h);
        delete h;
        return perr(SKO_E_NOMEM, "device buffers or pinned pool (%d x %zu bytes)", N, (size_t)bytes);
    }
    std::memset(h->pool, 0, (size_t)N * h->buf_bytes);
    hipError_t e = hipStreamCreateWithFlags(&h->load, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&h->save, hipStreamNonBlocking);
    for (int b = 0; b < nbuf && e == hipSuccess; ++b) e = hipEventCreateWithFlags(&h->saved[b], hipEventDisableTiming);
    for (int l = 0; l < N && e == hipSuccess; ++l) {
        LayerEvents& v = h->ev[l];
        for (hipEvent_t* x : {&v.load_start, &v.load_end, &v.ready, &v.begun, &v.ended})
            if (e == hipSuccess) e = hipEventCreate(x);
    }
    if (e != hipSuccess) {
        (void)hipGetLastError();
        free_all(h);
        delete h;
        return perr(SKO_E_DEVICE, "streams or events: %s", hipGetErrorString(e));
    }
    *out = h;
    return SKO_OK;
}

int sko_prefill_destroy(sko_prefill_handle* h) {
    if (!h) return SKO_OK;
    Guard g(h->cfg.device);
    // the caller's compute stream may still wait on the library's events or
    // write into its buffers: drain it too before anything is freed
    (void)hipStreamSynchronize(h->compute);
    if (h->load) (void)hipStreamSynchronize(h->load);
    if (h->save) (void)hipStreamSynchronize(h->save);
    free_all(h);
    delete h;
    return SKO_OK;
}

int sko_prefill_host_pool(sko_prefill_handle* h, int32_t layer, void** rows, int64_t* tokens) {
    if (!h) return perr(SKO_E_INVAL, "NULL handle");
    if (layer < 0 || layer >= h->N || !rows || !tokens) return perr(SKO_E_INVAL, "bad layer or NULL output");
    *rows = pool_rows(h, layer, 0);
    *tokens = h->tokens[layer];
    return SKO_OK;
}

int sko_prefill_set_tokens(sko_prefill_handle* h, int32_t layer, int64_t tokens) {
    int rc = check(h);
    if (rc != SKO_OK) return rc;
    if (layer < 0 || layer >= h->N || tokens < 0) return perr(SKO_E_INVAL, "bad layer or token count");
    if (tokens > h->cfg.capacity_tokens) return perr(SKO_E_CAPACITY, "%lld tokens exceed capacity %lld",
                                                     (long long)tokens, (long long)h->cfg.capacity_tokens);
    if (h->next_layer != 0 || h->begun_layer >= 0) return perr(SKO_E_STATE, "only between passes");
    h->tokens[layer] = tokens;
    // the host copy changed: a buffer holding this layer must load it again
    const int b = h->buf_of[layer];
    if (h->holder[b] == layer) h->holder[b] = -1;
    return SKO_OK;
}

int sko_prefill_begin_layer(sko_prefill_handle* h, int32_t layer, void** buffer) {
    int rc = check(h);
    if (rc != SKO_OK) return rc;
    if (!buffer) return perr(SKO_E_INVAL, "NULL output");
    if (layer != h->next_layer || h->begun_layer >= 0)
        return perr(SKO_E_STATE, "layer %d begun out of order (expected %d)", layer, h->next_layer);
    Guard g(h->cfg.device);
    if (layer == 0) h->next_load = 0;
    rc = issue_loads(h, layer + h->cfg.lookahead);
    if (rc != SKO_OK) return rc;
    LayerEvents& e = h->ev[layer];
    if (h->next_load <= layer) return perr(SKO_E_STATE, "layer %d could not be loaded", layer);
    hipError_t r = hipEventRecord(e.ready, h->compute);
    if (r == hipSuccess && e.loaded) r = hipStreamWaitEvent(h->compute, e.load_end, 0);
    if (r == hipSuccess) r = hipEventRecord(e.begun, h->compute);
    if (r != hipSuccess) return fail(h, r, "begin layer");
    h->begun_layer = layer;
    *buffer = h->bufs[h->buf_of[layer]];
    return SKO_OK;
}

int sko_prefill_end_layer(sko_prefill_handle* h, int32_t layer, int64_t new_tokens) {
    int rc = check(h);
    if (rc != SKO_OK) return rc;
    if (layer != h->begun_layer) return perr(SKO_E_STATE, "layer %d was not begun", layer);
    if (new_tokens < 0) return perr(SKO_E_INVAL, "new_tokens must be >= 0");
    if (h->tokens[layer] + new_tokens > h->cfg.capacity_tokens)
        return perr(SKO_E_CAPACITY, "layer %d: %lld + %lld tokens exceed capacity %lld", layer,
                    (long long)h->tokens[layer], (long long)new_tokens, (long long)h->cfg.capacity_tokens);
    Guard g(h->cfg.device);
    const int b = h->buf_of[layer];
    const size_t off = (size_t)h->tokens[layer] * h->cfg.row_bytes;
    hipError_t r = hipEventRecord(h->ev[layer].ended, h->compute);
    if (r == hipSuccess) r = hipStreamWaitEvent(h->save, h->ev[layer].ended, 0);
    if (r == hipSuccess && new_tokens)
        r = hipMemcpyAsync(pool_rows(h, layer, h->tokens[layer]), h->bufs[b] + off,
                           (size_t)new_tokens * h->cfg.row_bytes, hipMemcpyDeviceToHost, h->save);
    if (r == hipSuccess) r = hipEventRecord(h->saved[b], h->save);
    if (r != hipSuccess) return fail(h, r, "save");
    h->pending_save[b] = 1;
    h->busy[b] = 0;
    h->tokens[layer] += new_tokens;
    h->begun_layer = -1;
    h->next_layer = layer + 1 == h->N ? 0 : layer + 1;
    // loads that waited for this buffer (the next pass's start has none to issue)
    if (h->next_layer != 0) return issue_loads(h, h->next_layer + h->cfg.lookahead);
    return SKO_OK;
}

int sko_prefill_sync(sko_prefill_handle* h) {
    int rc = check(h);
    if (rc != SKO_OK) return rc;
    Guard g(h->cfg.device);
    hipError_t r = hipStreamSynchronize(h->load);
    if (r == hipSuccess) r = hipStreamSynchronize(h->compute);
    if (r == hipSuccess) r = hipStreamSynchronize(h->save);
    if (r != hipSuccess) return fail(h, r, "sync");
    std::fill(h->pending_save.begin(), h->pending_save.end(), 0);
    return SKO_OK;
}

int sko_prefill_layer_timing(sko_prefill_handle* h, int32_t layer, float* load_ms, float* exposed_ms,
                             float* compute_ms) {
    int rc = check(h);
    if (rc != SKO_OK) return rc;
    if (layer < 0 || layer >= h->N || !load_ms || !exposed_ms || !compute_ms)
        return perr(SKO_E_INVAL, "bad layer or NULL output");
    Guard g(h->cfg.device);
    const LayerEvents& e = h->ev[layer];
    float a = 0.0f, w = 0.0f, c = 0.0f;
    hipError_t r = hipSuccess;
    if (e.loaded) {
        r = hipEventElapsedTime(&a, e.load_start, e.load_end);
        if (r == hipSuccess) r = hipEventElapsedTime(&w, e.ready, e.load_end);
    }
    if (r == hipSuccess) r = hipEventElapsedTime(&c, e.begun, e.ended);
    if (r != hipSuccess) return fail(h, r, "layer timing (call sko_prefill_sync first)");
    *load_ms = a;
    *exposed_ms = w > 0.0f ? w : 0.0f;
    *compute_ms = c;
    return SKO_OK;
}

int sko_prefill_get_plan(sko_prefill_handle* h, int32_t* buffer_of_layer, int32_t* n_physical) {
    if (!h || !buffer_of_layer || !n_physical) return perr(SKO_E_INVAL, "NULL argument");
    std::copy(h->buf_of.begin(), h->buf_of.end(), buffer_of_layer);
    *n_physical = h->nbuf;
    return SKO_OK;
}

}  // extern "C"
