// Internal declarations of the gfx950 sparse KV row resolver library.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>

#include "kvr.h"

namespace kvr {

constexpr int kMaxHotSlots = 8192;
constexpr int kMaxSelCap = 8192;
constexpr int kMaxUnion = 8192;        // q * k of one verification block
constexpr int kGatherLayersPerLaunch = 24;

// Location word layout (bits 31..30 place, 29..0 index; a hot-cache word
// carries the fresh flag in bit 29 and the slot in bits 28..0).
constexpr uint32_t kPlaceShift = 30;
constexpr uint32_t kIndexMask = 0x3FFFFFFFu;
constexpr uint32_t kFreshBit = KVR_LOC_FRESH;
constexpr uint32_t kSlotMask = kFreshBit - 1;

// Device-side pointers of one payload layer.
struct LayerPtrs {
    uint8_t *tail;        // [n_req][T][R]
    uint8_t *pool;        // [pool_pages][P][R]
    uint8_t *hot;         // [n_req][B][R]
    uint8_t *host;        // [n_req][H + max_new][R], device alias of pinned memory
};

// Shape constants every kernel needs.
struct Shape {
    int32_t n_req, n_layers, H, max_new, P, T, B, R;
    int32_t sel_cap, n_pages, full_rows;  // full_rows = (H / P) * P
    int64_t pool_rows;                    // pool_pages * P
    int64_t host_rows;                    // H + max_new
};

// Launch timing of one context (kvr_timing_begin / kvr_timing_end).
struct LaunchLog {
    int32_t cap = 0;            // event pairs created
    int32_t limit = 0;          // pairs this recording may use
    int32_t n = 0;              // launches recorded
    int32_t missed = 0;         // launches past the limit
    bool on = false;
    hipEvent_t *ev = nullptr;   // [2 * cap]: start, stop of each launch
    int32_t *kind = nullptr;    // [cap] kvr_kernel
};

}  // namespace kvr

struct kvr_ctx {
    kvr_config cfg;
    kvr::Shape shape;
    int device;
    // metadata (device)
    int32_t *L;
    int32_t *page_map;
    uint8_t *host_valid;
    int32_t *tag;
    uint32_t *stamp;
    uint32_t *clock;
    bool meta_bound;
    // per-layer pointers: host-side mirror and device table
    kvr::LayerPtrs *layers_h;
    kvr::LayerPtrs *layers_d;
    bool *layer_bound;
    size_t resolve_lds;
    kvr::LaunchLog *timing;  // null until kvr_timing_begin
};

namespace kvr {

// Record a message for kvr_last_error() and return `code` / clear it and
// return KVR_OK (for entry points outside kvr_api.hip).
int api_fail(int code, const char *fmt, ...);
int api_ok();

// The next start/stop event pair for a launch of `kind`, when the context is
// recording and the stream is not being captured.
bool next_timing_events(const kvr_ctx *c, int32_t kind, hipStream_t s, hipEvent_t *start,
                        hipEvent_t *stop);

// Every kernel of the library is launched here: plainly, or with the events
// of a timing recording attached to its dispatch.
template <typename... P, typename... A>
hipError_t launch(const kvr_ctx *c, int32_t kind, void (*kernel)(P...), dim3 grid, dim3 block,
                  size_t lds, hipStream_t s, A... args)
{
    static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
    std::tuple<P...> vals{static_cast<P>(args)...};
    void *argv[sizeof...(P) > 0 ? sizeof...(P) : 1];
    std::apply([&argv](auto &...v) {
        int i = 0;
        ((argv[i++] = static_cast<void *>(&v)), ...);
    }, vals);
    hipEvent_t a = nullptr, b = nullptr;
    const void *fn = reinterpret_cast<const void *>(kernel);
    hipError_t e = next_timing_events(c, kind, s, &a, &b)
                       ? hipExtLaunchKernel(fn, grid, block, argv, lds, s, a, b, 0)
                       : hipLaunchKernel(fn, grid, block, argv, lds, s);
    if (e != hipSuccess)
        (void)hipGetLastError();  // the error is returned; do not leave it sticky
    return e;
}

// Launchers (return a hipError_t of the launch).
// new_rows non-null: the append of kvr_append_rows for the same requests runs
// first, in the same launch (append_status as its status, may be null).
// append_pos non-null: the append is deferred (host row and L only; the tail
// slot is left to a gather launch) and append_pos receives the positions.
hipError_t launch_resolve(const kvr_ctx *c, int32_t n, const int32_t *req_ids, const int32_t *sel,
                          const int32_t *sel_count, int32_t stride, uint32_t *loc, kvr_fill *fills,
                          int32_t *fill_count, int32_t *status, kvr_stats *stats,
                          int32_t count_host_bytes, const uint8_t *new_rows,
                          int32_t *append_status, int32_t *append_pos, hipStream_t s);
size_t resolve_lds_bytes(const Shape &sh);
// The resolve workgroup's dynamic LDS: victim keys (vc entries), hash (hs
// entries) and miss bitmap (bw words); 0 when the shape does not fit.
size_t resolve_lds_layout(const Shape &sh, int32_t *vc, int32_t *hs, int32_t *bw);
hipError_t prepare_resolve_kernel();

// Copies the fills of each request from the host store into the hot cache of
// every listed layer.
hipError_t launch_refill(const kvr_ctx *c, const int32_t *layers, int32_t n_layers, int32_t n,
                         const int32_t *req_ids, const kvr_fill *fills, const int32_t *fill_count,
                         int32_t *status, hipStream_t s);

struct GatherTarget {
    int32_t layer;
    uint8_t *out;
};
constexpr int32_t kGatherAll = 0;       // every valid word
constexpr int32_t kGatherResident = 1;  // every valid word but fresh hot-cache rows
constexpr int32_t kGatherFill = 2;      // fresh hot-cache rows, from host into slot and out
constexpr int32_t kGatherFused = 3;     // fill and resident in one launch
// new_rows/append_pos non-null (fused mode only): the launch also completes
// deferred appends of the same entries: it writes each appended row of every
// target layer into its tail slot and serves tail words naming that slot
// from new_rows.
hipError_t launch_gather(const kvr_ctx *c, int32_t mode, const GatherTarget *targets,
                         int32_t n_targets, int32_t n, const int32_t *req_ids, const uint32_t *loc,
                         const int32_t *sel, const int32_t *count, int32_t stride, int32_t *status,
                         hipStream_t s, const uint8_t *new_rows = nullptr,
                         const int32_t *append_pos = nullptr);

// One launch: the fused gather g (its first nt layers, targets) beside the
// resolve r (no host fill; an append must be deferred).
hipError_t launch_step(const kvr_ctx *c, const kvr_gather_call &g, const GatherTarget *targets,
                       int32_t nt, const kvr_resolve_call &r, hipStream_t s);
hipError_t prepare_step_kernel();

hipError_t launch_append(const kvr_ctx *c, int32_t n, const int32_t *req_ids,
                         const uint8_t *new_rows, int32_t *status, hipStream_t s);

hipError_t launch_init_state(const kvr_ctx *c, hipStream_t s);

hipError_t launch_copy_loc(const kvr_ctx *c, int32_t n, const uint32_t *src, uint32_t *dst,
                           const int32_t *count, int32_t stride, hipStream_t s);

hipError_t launch_dedup(const kvr_ctx *c, int32_t n, int32_t q, int32_t k, const int32_t *sel, int32_t *union_rows,
                        int32_t *union_count, int32_t *map, hipStream_t s);
hipError_t prepare_dedup_kernel();
hipError_t launch_reclaim(const kvr_ctx *c, int32_t n, const int32_t *req, const int32_t *page,
                          int32_t *freed, int32_t *status, hipStream_t s);
hipError_t launch_restore(const kvr_ctx *c, int32_t n, const int32_t *req, const int32_t *page,
                          const int32_t *phys, int32_t *status, hipStream_t s);

}  // namespace kvr
