// C ABI of the gfx950 sparse KV row resolver: argument checking, context
// state and launch sequencing.  Every entry point returns a kvr_status and
// records a message for kvr_last_error(); no exception crosses the ABI.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>

#include "kvr_internal.h"

namespace kvr {
bool tile_magic_exact(int32_t row_bytes);

bool next_timing_events(const kvr_ctx *c, int32_t kind, hipStream_t s, hipEvent_t *start,
                        hipEvent_t *stop)
{
    LaunchLog *t = c ? c->timing : nullptr;
    if (!t || !t->on)
        return false;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
        return false;
    if (t->n >= t->limit) {
        ++t->missed;
        return false;
    }
    t->kind[t->n] = kind;
    *start = t->ev[2 * t->n];
    *stop = t->ev[2 * t->n + 1];
    ++t->n;
    return true;
}

namespace {

void free_timing(LaunchLog *t)
{
    if (!t)
        return;
    for (int32_t i = 0; i < 2 * t->cap; ++i)
        if (t->ev[i])
            (void)hipEventDestroy(t->ev[i]);
    delete[] t->ev;
    delete[] t->kind;
    delete t;
}

}  // namespace
}  // namespace kvr

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int hip_fail(hipError_t e, const char *what)
{
    return fail(KVR_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

int ok()
{
    g_err[0] = '\0';
    return KVR_OK;
}

int check_ctx(const kvr_ctx *c, bool need_meta = true)
{
    if (!c)
        return fail(KVR_E_ARG, "null context");
    if (need_meta && !c->meta_bound)
        return fail(KVR_E_ARG, "metadata not bound");
    return KVR_OK;
}

int check_layer(const kvr_ctx *c, int32_t layer)
{
    if (layer < 0 || layer >= c->cfg.n_layers)
        return fail(KVR_E_ARG, "layer %d outside [0, %d)", layer, c->cfg.n_layers);
    if (!c->layer_bound[layer])
        return fail(KVR_E_ARG, "layer %d not bound", layer);
    return KVR_OK;
}

int check_n(const kvr_ctx *c, int32_t n)
{
    if (n < 0 || n > c->cfg.n_req)
        return fail(KVR_E_ARG, "request count %d outside [0, %d]", n, c->cfg.n_req);
    return KVR_OK;
}

// The current device and the stream (the null stream: the current device's)
// must be the context's device.
int check_stream(const kvr_ctx *c, hipStream_t s)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    if (dev != c->device)
        return fail(KVR_E_ARG, "current device %d is not the context's device %d", dev, c->device);
    if (s) {
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice(s, &sdev);
        if (e != hipSuccess)
            return hip_fail(e, "hipStreamGetDevice");
        if (sdev != c->device)
            return fail(KVR_E_ARG, "the stream is on device %d, not the context's device %d",
                        (int)sdev, c->device);
    }
    return KVR_OK;
}

}  // namespace

namespace kvr {

int api_fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int api_ok()
{
    return ok();
}

}  // namespace kvr

extern "C" {

const char *kvr_last_error(void) { return g_err; }

int kvr_create(const kvr_config *cfg, kvr_ctx **out)
{
    if (!out)
        return fail(KVR_E_ARG, "null output pointer");
    *out = nullptr;
    if (!cfg)
        return fail(KVR_E_ARG, "null config");
    const kvr_config &c = *cfg;
    if (c.n_req < 1 || c.n_layers < 1)
        return fail(KVR_E_ARG, "n_req and n_layers must be >= 1");
    if (c.history_rows < 0 || c.max_new_rows < 0 ||
        (int64_t)c.history_rows + c.max_new_rows >= (int64_t)INT32_MAX)
        return fail(KVR_E_ARG, "history_rows + max_new_rows must be in [0, 2^31 - 1)");
    if (c.page_rows < 1)
        return fail(KVR_E_ARG, "page_rows must be >= 1");
    if (c.tail_rows < 0 || c.tail_rows >= (1 << 30))
        return fail(KVR_E_ARG, "tail_rows must be in [0, 2^30)");
    if (c.hot_slots < 1 || c.hot_slots > kvr::kMaxHotSlots)
        return fail(KVR_E_ARG, "hot_slots must be in [1, %d]", kvr::kMaxHotSlots);
    if (c.row_bytes < 16 || c.row_bytes % 16 != 0)
        return fail(KVR_E_ARG, "row_bytes must be a positive multiple of 16");
    if (c.sel_cap < 1 || c.sel_cap > kvr::kMaxSelCap)
        return fail(KVR_E_ARG, "sel_cap must be in [1, %d]", kvr::kMaxSelCap);
    if (c.reserved != 0)
        return fail(KVR_E_ARG, "reserved must be 0");
    if (c.pool_pages < 0 || c.pool_pages * (int64_t)c.page_rows >= ((int64_t)1 << 30))
        return fail(KVR_E_ARG, "pool_pages * page_rows must be in [0, 2^30)");
    if (!kvr::tile_magic_exact(c.row_bytes))
        return fail(KVR_E_ARG, "row_bytes %d too large for the copy tiles", c.row_bytes);

    kvr_ctx *ctx = new (std::nothrow) kvr_ctx();
    if (!ctx)
        return fail(KVR_E_ARG, "out of host memory");
    ctx->cfg = c;
    kvr::Shape &sh = ctx->shape;
    sh.n_req = c.n_req;
    sh.n_layers = c.n_layers;
    sh.H = c.history_rows;
    sh.max_new = c.max_new_rows;
    sh.P = c.page_rows;
    sh.T = c.tail_rows;
    sh.B = c.hot_slots;
    sh.R = c.row_bytes;
    sh.sel_cap = c.sel_cap;
    sh.n_pages = (c.history_rows + c.page_rows - 1) / c.page_rows;
    sh.full_rows = (c.history_rows / c.page_rows) * c.page_rows;
    sh.pool_rows = c.pool_pages * c.page_rows;
    sh.host_rows = (int64_t)c.history_rows + c.max_new_rows;
    ctx->resolve_lds = kvr::resolve_lds_bytes(sh);
    if (ctx->resolve_lds == 0) {
        delete ctx;
        return fail(KVR_E_ARG, "hot_slots %d with sel_cap %d does not fit one workgroup's LDS",
                    c.hot_slots, c.sel_cap);
    }

    hipError_t e = hipGetDevice(&ctx->device);
    if (e != hipSuccess) {
        delete ctx;
        return hip_fail(e, "hipGetDevice");
    }
    ctx->layers_h = new (std::nothrow) kvr::LayerPtrs[c.n_layers]();
    ctx->layer_bound = new (std::nothrow) bool[c.n_layers]();
    if (!ctx->layers_h || !ctx->layer_bound) {
        kvr_destroy(ctx);
        return fail(KVR_E_ARG, "out of host memory");
    }
    e = hipMalloc(&ctx->layers_d, sizeof(kvr::LayerPtrs) * c.n_layers);
    if (e != hipSuccess) {
        ctx->layers_d = nullptr;
        kvr_destroy(ctx);
        return hip_fail(e, "hipMalloc(layer table)");
    }
    e = hipMemset(ctx->layers_d, 0, sizeof(kvr::LayerPtrs) * c.n_layers);
    if (e == hipSuccess)
        e = kvr::prepare_resolve_kernel();
    if (e == hipSuccess)
        e = kvr::prepare_dedup_kernel();
    if (e == hipSuccess)
        e = kvr::prepare_step_kernel();
    if (e != hipSuccess) {
        kvr_destroy(ctx);
        return hip_fail(e, "kernel set-up");
    }
    *out = ctx;
    return ok();
}

int kvr_destroy(kvr_ctx *ctx)
{
    if (!ctx)
        return ok();
    if (ctx->layers_d)
        (void)hipFree(ctx->layers_d);
    delete[] ctx->layers_h;
    delete[] ctx->layer_bound;
    kvr::free_timing(ctx->timing);
    delete ctx;
    return ok();
}

int kvr_bind_metadata(kvr_ctx *ctx, int32_t *L, int32_t *page_map, uint8_t *host_valid,
                      int32_t *tag, uint32_t *stamp, uint32_t *clock)
{
    if (int rc = check_ctx(ctx, false))
        return rc;
    if (!L || !tag || !stamp || !clock)
        return fail(KVR_E_ARG, "L, tag, stamp and clock are required");
    if (ctx->shape.n_pages > 0 && (!page_map || !host_valid))
        return fail(KVR_E_ARG, "page_map and host_valid are required when H > 0");
    ctx->L = L;
    ctx->page_map = page_map;
    ctx->host_valid = host_valid;
    ctx->tag = tag;
    ctx->stamp = stamp;
    ctx->clock = clock;
    ctx->meta_bound = true;
    return ok();
}

int kvr_bind_layer(kvr_ctx *ctx, int32_t layer, void *tail, void *pool, void *hot, void *host)
{
    if (int rc = check_ctx(ctx, false))
        return rc;
    if (layer < 0 || layer >= ctx->cfg.n_layers)
        return fail(KVR_E_ARG, "layer %d outside [0, %d)", layer, ctx->cfg.n_layers);
    if (!hot || !host)
        return fail(KVR_E_ARG, "hot and host are required");
    if (ctx->shape.T > 0 && !tail)
        return fail(KVR_E_ARG, "tail is required when T > 0");
    if (ctx->shape.pool_rows > 0 && !pool)
        return fail(KVR_E_ARG, "pool is required when pool_pages > 0");
    void *host_dev = nullptr;
    hipError_t e = hipHostGetDevicePointer(&host_dev, host, 0);
    if (e != hipSuccess || !host_dev)
        return fail(KVR_E_ARG, "host store is not device-mapped pinned memory (%s)",
                    hipGetErrorString(e));
    kvr::LayerPtrs lp;
    lp.tail = static_cast<uint8_t *>(tail);
    lp.pool = static_cast<uint8_t *>(pool);
    lp.hot = static_cast<uint8_t *>(hot);
    lp.host = static_cast<uint8_t *>(host_dev);
    e = hipMemcpy(ctx->layers_d + layer, &lp, sizeof lp, hipMemcpyHostToDevice);
    if (e != hipSuccess)
        return hip_fail(e, "hipMemcpy(layer table)");
    ctx->layers_h[layer] = lp;
    ctx->layer_bound[layer] = true;
    return ok();
}

int kvr_init_state(kvr_ctx *ctx, void *stream)
{
    if (int rc = check_ctx(ctx))
        return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (int rc = check_stream(ctx, s))
        return rc;
    hipError_t e = kvr::launch_init_state(ctx, s);
    return e == hipSuccess ? ok() : hip_fail(e, "init_state launch");
}

int kvr_append_rows(kvr_ctx *ctx, int32_t n, const int32_t *req_ids, const void *new_rows,
                    int32_t *status, void *stream)
{
    if (int rc = check_ctx(ctx))
        return rc;
    if (int rc = check_n(ctx, n))
        return rc;
    for (int32_t l = 0; l < ctx->cfg.n_layers; ++l)
        if (int rc = check_layer(ctx, l))
            return rc;
    if (n > 0 && !new_rows)
        return fail(KVR_E_ARG, "new_rows is required");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (int rc = check_stream(ctx, s))
        return rc;
    if (n == 0)
        return ok();
    hipError_t e = kvr::launch_append(ctx, n, req_ids, static_cast<const uint8_t *>(new_rows),
                                      status, s);
    return e == hipSuccess ? ok() : hip_fail(e, "append launch");
}

static int check_resolve(kvr_ctx *ctx, int32_t n, const void *new_rows, int32_t *append_status,
                         const int32_t *sel, int32_t stride, uint32_t *loc, kvr_fill *fills,
                         int32_t *fill_count, int32_t fill_layer, int32_t *status)
{
    if (int rc = check_ctx(ctx))
        return rc;
    if (int rc = check_n(ctx, n))
        return rc;
    if (new_rows || append_status) {
        for (int32_t l = 0; l < ctx->cfg.n_layers; ++l)
            if (int rc = check_layer(ctx, l))
                return rc;
        if (n > 0 && !new_rows)
            return fail(KVR_E_ARG, "new_rows is required");
    }
    if (stride < 0 || stride > ctx->cfg.sel_cap)
        return fail(KVR_E_ARG, "stride %d outside [0, sel_cap=%d]", stride, ctx->cfg.sel_cap);
    if (n > 0 && ((stride > 0 && (!sel || !loc)) || !fills || !fill_count || !status))
        return fail(KVR_E_ARG, "sel, loc, fills, fill_count and status are required");
    if (fill_layer != -1)
        if (int rc = check_layer(ctx, fill_layer))
            return rc;
    return KVR_OK;
}

static int resolve_entry(kvr_ctx *ctx, int32_t n, const int32_t *req_ids, const void *new_rows,
                         int32_t *append_status, const int32_t *sel, const int32_t *sel_count,
                         int32_t stride, uint32_t *loc, kvr_fill *fills, int32_t *fill_count,
                         int32_t fill_layer, int32_t *status, kvr_stats *stats, void *stream,
                         int32_t *append_pos = nullptr)
{
    if (int rc = check_resolve(ctx, n, new_rows, append_status, sel, stride, loc, fills,
                               fill_count, fill_layer, status))
        return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (int rc = check_stream(ctx, s))
        return rc;
    if (n == 0)
        return ok();
    hipError_t e = kvr::launch_resolve(ctx, n, req_ids, sel, sel_count, stride, loc, fills,
                                       fill_count, status, stats, fill_layer >= 0 ? 1 : 0,
                                       static_cast<const uint8_t *>(new_rows), append_status,
                                       append_pos, s);
    if (e != hipSuccess)
        return hip_fail(e, "resolve launch");
    if (fill_layer >= 0) {
        e = kvr::launch_refill(ctx, &fill_layer, 1, n, req_ids, fills, fill_count, nullptr, s);
        if (e != hipSuccess)
            return hip_fail(e, "refill launch");
    }
    return ok();
}

int kvr_resolve_rows(kvr_ctx *ctx, int32_t n, const int32_t *req_ids, const int32_t *sel,
                     const int32_t *sel_count, int32_t stride, uint32_t *loc, kvr_fill *fills,
                     int32_t *fill_count, int32_t fill_layer, int32_t *status, kvr_stats *stats,
                     void *stream)
{
    return resolve_entry(ctx, n, req_ids, nullptr, nullptr, sel, sel_count, stride, loc, fills,
                         fill_count, fill_layer, status, stats, stream);
}

int kvr_append_resolve_rows(kvr_ctx *ctx, int32_t n, const int32_t *req_ids, const void *new_rows,
                            int32_t *append_status, const int32_t *sel, const int32_t *sel_count,
                            int32_t stride, uint32_t *loc, kvr_fill *fills, int32_t *fill_count,
                            int32_t fill_layer, int32_t *status, kvr_stats *stats, void *stream)
{
    if (n > 0 && !new_rows)
        return fail(KVR_E_ARG, "new_rows is required");
    return resolve_entry(ctx, n, req_ids, new_rows, append_status, sel, sel_count, stride, loc,
                         fills, fill_count, fill_layer, status, stats, stream);
}

int kvr_append_resolve_rows_deferred(kvr_ctx *ctx, int32_t n, const int32_t *req_ids,
                                     const void *new_rows, int32_t *append_status,
                                     int32_t *append_pos, const int32_t *sel,
                                     const int32_t *sel_count, int32_t stride, uint32_t *loc,
                                     kvr_fill *fills, int32_t *fill_count, int32_t fill_layer,
                                     int32_t *status, kvr_stats *stats, void *stream)
{
    if (n > 0 && (!new_rows || !append_pos))
        return fail(KVR_E_ARG, "new_rows and append_pos are required");
    return resolve_entry(ctx, n, req_ids, new_rows, append_status, sel, sel_count, stride, loc,
                         fills, fill_count, fill_layer, status, stats, stream, append_pos);
}

static int check_gather(kvr_ctx *ctx, int32_t n_layers, const int32_t *layers, int32_t n,
                        const uint32_t *loc, int32_t stride, void *const *out,
                        const void *new_rows, const int32_t *append_pos)
{
    if (int rc = check_ctx(ctx, false))
        return rc;
    if (int rc = check_n(ctx, n))
        return rc;
    if (n_layers < 0 || (n_layers > 0 && (!layers || !out)))
        return fail(KVR_E_ARG, "layers and out are required");
    if (stride < 0)
        return fail(KVR_E_ARG, "negative stride");
    if (n > 0 && stride > 0 && n_layers > 0 && !loc)
        return fail(KVR_E_ARG, "loc is required");
    for (int32_t t = 0; t < n_layers; ++t) {
        if (int rc = check_layer(ctx, layers[t]))
            return rc;
        if (!out[t] && n > 0 && stride > 0)
            return fail(KVR_E_ARG, "out[%d] is null", t);
    }
    if (append_pos) {
        // the appended rows go to the tail of every payload layer: the call
        // must name each layer of the context once
        if (!ctx->meta_bound)
            return fail(KVR_E_ARG, "metadata not bound");
        if (n > 0 && !new_rows)
            return fail(KVR_E_ARG, "new_rows is required");
        if (n_layers != ctx->cfg.n_layers)
            return fail(KVR_E_ARG, "deferred appends need all %d layers, got %d",
                        ctx->cfg.n_layers, n_layers);
        for (int32_t t = 1; t < n_layers; ++t)
            for (int32_t u = 0; u < t; ++u)
                if (layers[u] == layers[t])
                    return fail(KVR_E_ARG, "layer %d named twice", layers[t]);
    }
    return KVR_OK;
}

// The launches of a gather whose arguments are checked: one per group of up
// to kGatherLayersPerLaunch layers (with deferred appends a launch runs even
// for an empty selection: it still writes the appended rows).
static int gather_launch(kvr_ctx *ctx, int32_t mode, int32_t n_layers, const int32_t *layers,
                         int32_t n, const int32_t *req_ids, const uint32_t *loc,
                         const int32_t *sel, const int32_t *count, int32_t stride,
                         void *const *out, int32_t *status, hipStream_t s, const void *new_rows,
                         const int32_t *append_pos)
{
    const bool deferred = append_pos != nullptr;
    int rc = KVR_OK;
    kvr::GatherTarget targets[kvr::kGatherLayersPerLaunch];
    for (int32_t t0 = 0; rc == KVR_OK && n > 0 && (stride > 0 || deferred) && t0 < n_layers;
         t0 += kvr::kGatherLayersPerLaunch) {
        const int32_t nt = n_layers - t0 < kvr::kGatherLayersPerLaunch
                               ? n_layers - t0 : kvr::kGatherLayersPerLaunch;
        for (int32_t t = 0; t < nt; ++t) {
            targets[t].layer = layers[t0 + t];
            targets[t].out = static_cast<uint8_t *>(out[t0 + t]);
        }
        hipError_t e = kvr::launch_gather(ctx, mode, targets, nt, n, req_ids, loc, sel, count, stride,
                                          status, s, static_cast<const uint8_t *>(new_rows),
                                          append_pos);
        if (e != hipSuccess)
            rc = hip_fail(e, "gather launch");
    }
    return rc == KVR_OK ? ok() : rc;
}

static int gather_entry(kvr_ctx *ctx, int32_t mode, int32_t n_layers, const int32_t *layers,
                        int32_t n, const int32_t *req_ids, const uint32_t *loc, const int32_t *sel,
                        const int32_t *count, int32_t stride, void *const *out, int32_t *status,
                        void *stream, const void *new_rows = nullptr,
                        const int32_t *append_pos = nullptr)
{
    if (int rc = check_gather(ctx, n_layers, layers, n, loc, stride, out, new_rows, append_pos))
        return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (int rc = check_stream(ctx, s))
        return rc;
    return gather_launch(ctx, mode, n_layers, layers, n, req_ids, loc, sel, count, stride, out,
                         status, s, new_rows, append_pos);
}

int kvr_gather_rows(kvr_ctx *ctx, int32_t n_layers, const int32_t *layers, int32_t n,
                    const int32_t *req_ids, const uint32_t *loc, const int32_t *count,
                    int32_t stride, void *const *out, int32_t *status, void *stream)
{
    return gather_entry(ctx, kvr::kGatherAll, n_layers, layers, n, req_ids, loc, nullptr, count,
                        stride, out, status, stream);
}

int kvr_gather_resident_rows(kvr_ctx *ctx, int32_t n_layers, const int32_t *layers, int32_t n,
                             const int32_t *req_ids, const uint32_t *loc, const int32_t *count,
                             int32_t stride, void *const *out, int32_t *status, void *stream)
{
    return gather_entry(ctx, kvr::kGatherResident, n_layers, layers, n, req_ids, loc, nullptr,
                        count, stride, out, status, stream);
}

int kvr_fill_gather_rows(kvr_ctx *ctx, int32_t n_layers, const int32_t *layers, int32_t n,
                         const int32_t *req_ids, const uint32_t *loc, const int32_t *sel,
                         const int32_t *count, int32_t stride, void *const *out, int32_t *status,
                         void *stream)
{
    if (n > 0 && stride > 0 && n_layers > 0 && !sel)
        return fail(KVR_E_ARG, "sel is required");
    return gather_entry(ctx, kvr::kGatherFill, n_layers, layers, n, req_ids, loc, sel, count,
                        stride, out, status, stream);
}

int kvr_fused_gather_rows(kvr_ctx *ctx, int32_t n_layers, const int32_t *layers, int32_t n,
                          const int32_t *req_ids, const uint32_t *loc, const int32_t *sel,
                          const int32_t *count, int32_t stride, void *const *out, int32_t *status,
                          void *stream)
{
    if (n > 0 && stride > 0 && n_layers > 0 && !sel)
        return fail(KVR_E_ARG, "sel is required");
    return gather_entry(ctx, kvr::kGatherFused, n_layers, layers, n, req_ids, loc, sel, count,
                        stride, out, status, stream);
}

int kvr_fused_gather_append_rows(kvr_ctx *ctx, int32_t n_layers, const int32_t *layers, int32_t n,
                                 const int32_t *req_ids, const uint32_t *loc, const int32_t *sel,
                                 const int32_t *count, int32_t stride, void *const *out,
                                 int32_t *status, const void *new_rows, const int32_t *append_pos,
                                 void *stream)
{
    if (n > 0 && stride > 0 && n_layers > 0 && !sel)
        return fail(KVR_E_ARG, "sel is required");
    if (n > 0 && !append_pos)
        return fail(KVR_E_ARG, "append_pos is required");
    return gather_entry(ctx, kvr::kGatherFused, n_layers, layers, n, req_ids, loc, sel, count,
                        stride, out, status, stream, new_rows, append_pos);
}

int kvr_gather_resolve_rows(kvr_ctx *ctx, const kvr_gather_call *g, const kvr_resolve_call *r,
                            void *stream)
{
    if (!g && !r)
        return fail(KVR_E_ARG, "a gather or a resolve call is required");
    if (g && g->n > 0 && g->stride > 0 && g->n_layers > 0 && !g->sel)
        return fail(KVR_E_ARG, "gather: sel is required");
    if (g && g->n > 0 && !g->append_pos && g->new_rows)
        return fail(KVR_E_ARG, "gather: new_rows without append_pos");
    if (g) {
        if (int rc = check_gather(ctx, g->n_layers, g->layers, g->n, g->loc, g->stride, g->out,
                                  g->new_rows, g->append_pos))
            return rc;
    }
    if (r) {
        // an append beside a gather must leave the tail to a later gather
        if (r->n > 0 && r->new_rows && !r->append_pos)
            return fail(KVR_E_ARG, "resolve: an append needs append_pos (it is deferred)");
        if (int rc = check_resolve(ctx, r->n, r->new_rows, r->append_status, r->sel, r->stride,
                                   r->loc, r->fills, r->fill_count, -1, r->status))
            return rc;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (int rc = check_stream(ctx, s))
        return rc;
    const bool has_g = g && g->n > 0 && g->n_layers > 0 && (g->stride > 0 || g->append_pos);
    const bool has_r = r && r->n > 0;
    if (!has_g && !has_r)
        return ok();
    hipError_t e = hipSuccess;
    if (!has_g) {
        e = kvr::launch_resolve(ctx, r->n, r->req_ids, r->sel, r->sel_count, r->stride, r->loc,
                                r->fills, r->fill_count, r->status, r->stats, 0,
                                static_cast<const uint8_t *>(r->new_rows), r->append_status,
                                r->append_pos, s);
        return e == hipSuccess ? ok() : hip_fail(e, "resolve launch");
    }
    if (!has_r)
        return gather_entry(ctx, kvr::kGatherFused, g->n_layers, g->layers, g->n, g->req_ids,
                            g->loc, g->sel, g->count, g->stride, g->out, g->status, stream,
                            g->new_rows, g->append_pos);
    // the first (up to kGatherLayersPerLaunch) layers share the launch with
    // the resolve; more layers are gathered by launches of their own after it
    kvr::GatherTarget targets[kvr::kGatherLayersPerLaunch];
    const int32_t nt0 = g->n_layers < kvr::kGatherLayersPerLaunch ? g->n_layers
                                                                   : kvr::kGatherLayersPerLaunch;
    for (int32_t t = 0; t < nt0; ++t) {
        targets[t].layer = g->layers[t];
        targets[t].out = static_cast<uint8_t *>(g->out[t]);
    }
    e = kvr::launch_step(ctx, *g, targets, nt0, *r, s);
    if (e != hipSuccess)
        return hip_fail(e, "gather-resolve launch");
    // (the whole layer list was checked above: a deferred append names every
    // layer once, and these launches write the tails of the layers after nt0)
    if (g->n_layers > nt0)
        return gather_launch(ctx, kvr::kGatherFused, g->n_layers - nt0, g->layers + nt0, g->n,
                             g->req_ids, g->loc, g->sel, g->count, g->stride, g->out + nt0,
                             g->status, s, g->new_rows, g->append_pos);
    return ok();
}

int kvr_dedup_verify_selections(kvr_ctx *ctx, int32_t n, int32_t q, int32_t k, const int32_t *sel,
                                int32_t *union_rows, int32_t *union_count, int32_t *map,
                                void *stream)
{
    if (int rc = check_ctx(ctx, false))
        return rc;
    if (int rc = check_n(ctx, n))
        return rc;
    if (q < 1 || k < 0 || (int64_t)q * k > kvr::kMaxUnion)
        return fail(KVR_E_ARG, "need q >= 1, k >= 0 and q * k <= %d", kvr::kMaxUnion);
    if (n > 0 && (!union_count || (q * k > 0 && (!sel || !union_rows || !map))))
        return fail(KVR_E_ARG, "sel, union_rows, union_count and map are required");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (int rc = check_stream(ctx, s))
        return rc;
    if (n == 0)
        return ok();
    hipError_t e = kvr::launch_dedup(ctx, n, q, k, sel, union_rows, union_count, map, s);
    return e == hipSuccess ? ok() : hip_fail(e, "dedup launch");
}

int kvr_reuse_locations(kvr_ctx *ctx, int32_t mode, int32_t n_layers, const int32_t *dst_layers,
                        int32_t n, const int32_t *req_ids, const uint32_t *src_loc,
                        uint32_t *dst_loc, const int32_t *count, int32_t stride,
                        const kvr_fill *fills, const int32_t *fill_count, int32_t *status,
                        void *stream)
{
    if (int rc = check_ctx(ctx, false))
        return rc;
    if (int rc = check_n(ctx, n))
        return rc;
    if (mode != KVR_REUSE_SHARED_SOURCE && mode != KVR_REUSE_DISTINCT_PAYLOAD)
        return fail(KVR_E_ARG, "unknown reuse mode %d", mode);
    if (stride < 0)
        return fail(KVR_E_ARG, "negative stride");
    if (dst_loc && !src_loc && stride > 0 && n > 0)
        return fail(KVR_E_ARG, "src_loc is required to copy locations");
    if (mode == KVR_REUSE_DISTINCT_PAYLOAD) {
        if (n_layers < 0 || (n_layers > 0 && !dst_layers))
            return fail(KVR_E_ARG, "dst_layers is required to replay fills");
        for (int32_t t = 0; t < n_layers; ++t)
            if (int rc = check_layer(ctx, dst_layers[t]))
                return rc;
        if (n > 0 && n_layers > 0 && (!fills || !fill_count))
            return fail(KVR_E_ARG, "fills and fill_count are required to replay fills");
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (int rc = check_stream(ctx, s))
        return rc;
    if (n == 0)
        return ok();
    if (mode == KVR_REUSE_DISTINCT_PAYLOAD && n_layers > 0) {
        hipError_t e = kvr::launch_refill(ctx, dst_layers, n_layers, n, req_ids, fills, fill_count,
                                          status, s);
        if (e != hipSuccess)
            return hip_fail(e, "replay launch");
    }
    if (dst_loc && stride > 0 && dst_loc != src_loc) {
        hipError_t e = kvr::launch_copy_loc(ctx, n, src_loc, dst_loc, count, stride, s);
        if (e != hipSuccess)
            return hip_fail(e, "location copy launch");
    }
    return ok();
}

// Every payload layer is bound (page moves touch all of them).
static int check_all_layers(const kvr_ctx *ctx)
{
    for (int32_t l = 0; l < ctx->cfg.n_layers; ++l)
        if (!ctx->layer_bound[l])
            return fail(KVR_E_ARG, "layer %d not bound", l);
    return KVR_OK;
}

static const int32_t kMaxPageList = 65536;

static int check_page_list(const kvr_ctx *ctx, int32_t n, const void *a, const void *b,
                           const void *c)
{
    if (int rc = check_ctx(ctx))
        return rc;
    const int64_t most = (int64_t)ctx->cfg.n_req * ctx->shape.n_pages;
    if (n < 0 || n > most || n > kMaxPageList)
        return fail(KVR_E_ARG, "page count %d outside [0, min(%lld, %d)]", n, (long long)most,
                    kMaxPageList);
    if (n > 0 && (!a || !b || !c))
        return fail(KVR_E_ARG, "the page lists are required");
    return check_all_layers(ctx);
}

int kvr_reclaim_pages(kvr_ctx *ctx, int32_t n, const int32_t *req_ids, const int32_t *pages,
                      int32_t *freed_phys, int32_t *status, void *stream)
{
    if (int rc = check_page_list(ctx, n, req_ids, pages, freed_phys))
        return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (int rc = check_stream(ctx, s))
        return rc;
    if (n == 0)
        return ok();
    hipError_t e = kvr::launch_reclaim(ctx, n, req_ids, pages, freed_phys, status, s);
    return e == hipSuccess ? ok() : hip_fail(e, "reclaim launch");
}

int kvr_restore_pages(kvr_ctx *ctx, int32_t n, const int32_t *req_ids, const int32_t *pages,
                      const int32_t *phys, int32_t *status, void *stream)
{
    if (int rc = check_page_list(ctx, n, req_ids, pages, phys))
        return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (int rc = check_stream(ctx, s))
        return rc;
    if (n == 0)
        return ok();
    hipError_t e = kvr::launch_restore(ctx, n, req_ids, pages, phys, status, s);
    return e == hipSuccess ? ok() : hip_fail(e, "restore launch");
}

int kvr_status_summary(const int32_t *status, int32_t n, int32_t *first_bad)
{
    if ((!status && n > 0) || n < 0)
        return fail(KVR_E_ARG, "bad status array");
    int bad = 0;
    int first = -1;
    for (int32_t i = 0; i < n; ++i) {
        if (status[i] != KVR_OK) {
            if (first < 0)
                first = i;
            ++bad;
        }
    }
    if (first_bad)
        *first_bad = first;
    g_err[0] = '\0';
    return bad;
}

int kvr_host_alloc(size_t bytes, void **out)
{
    if (!out)
        return fail(KVR_E_ARG, "null output pointer");
    *out = nullptr;
    hipError_t e = hipHostMalloc(out, bytes ? bytes : 1, hipHostMallocDefault);
    if (e != hipSuccess) {
        *out = nullptr;
        return hip_fail(e, "hipHostMalloc");
    }
    return ok();
}

int kvr_host_free(void *ptr)
{
    if (!ptr)
        return ok();
    hipError_t e = hipHostFree(ptr);
    return e == hipSuccess ? ok() : hip_fail(e, "hipHostFree");
}

int kvr_timing_begin(kvr_ctx *ctx, int32_t capacity)
{
    if (int rc = check_ctx(ctx, false))
        return rc;
    if (capacity < 1 || capacity > (1 << 20))
        return fail(KVR_E_ARG, "timing capacity %d outside [1, 1048576]", capacity);
    if (int rc = check_stream(ctx, nullptr))
        return rc;
    kvr::LaunchLog *t = ctx->timing;
    if (!t || t->cap < capacity) {
        kvr::free_timing(t);
        ctx->timing = nullptr;
        t = new (std::nothrow) kvr::LaunchLog();
        if (!t)
            return fail(KVR_E_ARG, "out of host memory");
        t->ev = new (std::nothrow) hipEvent_t[2 * (size_t)capacity]();
        t->kind = new (std::nothrow) int32_t[capacity]();
        if (!t->ev || !t->kind) {
            kvr::free_timing(t);
            return fail(KVR_E_ARG, "out of host memory");
        }
        t->cap = capacity;
        for (int32_t i = 0; i < 2 * capacity; ++i) {
            hipError_t e = hipEventCreate(&t->ev[i]);
            if (e != hipSuccess) {
                t->ev[i] = nullptr;
                kvr::free_timing(t);
                return hip_fail(e, "hipEventCreate");
            }
        }
        ctx->timing = t;
    }
    t->limit = capacity;
    t->n = 0;
    t->missed = 0;
    t->on = true;
    return ok();
}

int kvr_timing_end(kvr_ctx *ctx, int32_t capacity, int32_t *kinds, float *ms, int32_t *n_recorded)
{
    if (int rc = check_ctx(ctx, false))
        return rc;
    kvr::LaunchLog *t = ctx->timing;
    if (!t || !t->on)
        return fail(KVR_E_ARG, "timing was not started");
    t->on = false;
    if (capacity < 0 || (capacity > 0 && (!kinds || !ms)))
        return fail(KVR_E_ARG, "kinds and ms must hold `capacity` entries");
    if (n_recorded)
        *n_recorded = t->n;
    const int32_t m = t->n < capacity ? t->n : capacity;
    for (int32_t i = 0; i < m; ++i) {
        hipError_t e = hipEventSynchronize(t->ev[2 * i + 1]);
        if (e == hipSuccess)
            e = hipEventElapsedTime(&ms[i], t->ev[2 * i], t->ev[2 * i + 1]);
        if (e != hipSuccess)
            return hip_fail(e, "reading launch events");
        kinds[i] = t->kind[i];
    }
    if (t->missed > 0)
        return fail(KVR_E_CAPACITY, "%d launches ran untimed past the capacity", t->missed);
    if (m < t->n)
        return fail(KVR_E_CAPACITY, "%d launches recorded, output holds %d", t->n, capacity);
    return ok();
}

}  // extern "C"
