/*
 * kvr.h - C ABI of the MI355X (gfx950) per-decode-step sparse KV row resolver.
 *
 * The method is the resolver of "Adaptive DHiSparse: Speculative Decoding over
 * a Load-Adaptive KV Hierarchy" (section "How it works"):
 *   - Memory split: each request has, per KV source, its own B-slot hot
 *     cache, a writable tail and its metadata; whole pages of the history it
 *     was admitted with may in addition be kept ready in an optional pool that
 *     all requests share.
 *   - Resolution: a selected row is taken from the first of three places that
 *     holds it: (1) the tail, else a ready page found through the optional
 *     page map; (2) the hot cache, whose lookup examines no more than B slots
 *     and which is managed LRU; (3) the pinned host store, from which the row
 *     is copied into a hot-cache slot.
 *   - Speculative state: the queries of one verification block fetch each
 *     missing row once between them.
 *   - Model-specific reuse: Reuse layers inherit a location vector when they
 *     share one physical KV source; layers that share sparse indices but own
 *     distinct payloads fetch the same positions for their own payload.
 *
 * One context serves one KV source: n_req requests and n_layers payload
 * layers that share the source's metadata (history length, page map, hot-cache
 * tags and stamps).
 *
 * Conventions
 *   - Every buffer is caller-owned.  Pointers marked (device) are device
 *     memory; (host) is ordinary host memory read during the call; (pinned) is
 *     page-locked host memory from hipHostMalloc (for example kvr_host_alloc or
 *     a pinned torch tensor), which kernels read and write directly over the
 *     host link.  The library keeps bound pointers until kvr_destroy and never
 *     frees them.
 *   - Calls that take a stream enqueue work on it (a hipStream_t; NULL is the
 *     default stream) and return without waiting for the device.  They never
 *     synchronise the host and allocate nothing.  Their return value reports
 *     argument errors only.
 *   - Data-dependent errors (a selected row outside [0, L), more distinct
 *     pending rows than B, a missing row without a host copy) are written per
 *     request into a device status array, stream-ordered.  A request that fails
 *     changes nothing: L, tags, stamps, clock and hot payload stay as they were
 *     and its locations read KVR_LOC_INVALID.  The other requests of the call
 *     complete normally.
 *   - Return codes are kvr_status values; kvr_last_error() gives a message for
 *     the calling thread's last failure.  No C++ exception leaves the library.
 *   - Threads and streams: the calls that launch work only read the context,
 *     so several host threads may issue them at once, except while launch
 *     timing is on (kvr_timing_begin to kvr_timing_end records into the
 *     context); kvr_bind_*, kvr_timing_* and kvr_destroy need the caller to
 *     keep every other call on that context out meanwhile.  On the device,
 *     calls that touch the same request must be ordered (one stream, or
 *     events between streams): two resolves of one request in flight at once
 *     race on its tags, stamps and clock.
 *
 * Location word (uint32): bits 31..30 give the place (kvr_place), bits 29..0
 * the index in it: the tail ring slot (pos mod T), the optional-pool row
 * (physical page * P + pos mod P) or the hot-cache slot.  A hot-cache word
 * carries KVR_LOC_FRESH (bit 29) when its row was copied from host memory by
 * the call that wrote the word; its slot is then in bits 28..0.
 */
#ifndef KVR_H
#define KVR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvr_status {
    KVR_OK = 0,
    KVR_E_ARG = -1,          /* bad argument, shape or unbound buffer            */
    KVR_E_RANGE = -2,        /* selected row outside [0, L), or a bad location   */
    KVR_E_CAPACITY = -3,     /* more distinct pending rows than B; history full  */
    KVR_E_NO_HOST_COPY = -4, /* a missing row is neither on device nor on host   */
    KVR_E_HIP = -5,          /* the HIP runtime reported an error               */
    KVR_E_STATE = -6,        /* the LRU clock would wrap                         */
} kvr_status;

typedef enum kvr_place {
    KVR_PLACE_TAIL = 0,
    KVR_PLACE_PAGE = 1,
    KVR_PLACE_HOT = 2,
    KVR_PLACE_INVALID = 3,
} kvr_place;

#define KVR_LOC_INVALID 0xFFFFFFFFu
#define KVR_LOC_FRESH (1u << 29)  /* hot-cache word: filled from host by this call */

typedef enum kvr_reuse_mode {
    /* Reuse layers of one physical KV source: the location vector is inherited
     * as is (dst_loc NULL = alias, zero bytes moved; else a copy of it). */
    KVR_REUSE_SHARED_SOURCE = 0,
    /* Shared indices, distinct per-layer payloads: the rows filled from host
     * for one layer are fetched into the same hot slots of every destination
     * layer from that layer's host store; dst_loc (optional) receives a copy
     * of src_loc. */
    KVR_REUSE_DISTINCT_PAYLOAD = 1,
} kvr_reuse_mode;

/* Shape of one KV source.  Limits: 1 <= hot_slots <= 8192,
 * 1 <= sel_cap <= 8192, row_bytes a positive multiple of 16,
 * pool_pages * page_rows < 2^30, history_rows + max_new_rows < 2^31. */
typedef struct kvr_config {
    int32_t n_req;        /* requests of the source                           */
    int32_t n_layers;     /* payload layers sharing the source's metadata     */
    int32_t history_rows; /* H: imported history rows per request             */
    int32_t max_new_rows; /* decoded rows a request may append                */
    int32_t page_rows;    /* P: rows per optional-history page                */
    int32_t tail_rows;    /* T: rows in the mutable tail ring (0 = no tail)   */
    int32_t hot_slots;    /* B: hot-cache slots per request                   */
    int32_t row_bytes;    /* R: bytes per row (opaque payload)                */
    int32_t sel_cap;      /* most selection entries one request passes to one
                             resolve call (the union capacity for verify)     */
    int32_t reserved;     /* must be 0                                        */
    int64_t pool_pages;   /* pages in the global optional pool, per layer     */
} kvr_config;

/* One host refill: `row` was copied into hot slot `slot`. */
typedef struct kvr_fill {
    int32_t row;
    int32_t slot;
} kvr_fill;

/* Resolution counters, added to (device atomics) by every resolve call.
 * tail/page/hit/miss count selection entries by where they were found; fill
 * counts distinct rows copied from host and host_bytes their bytes. */
typedef struct kvr_stats {
    uint64_t calls, tail, page, hit, miss, fill, host_bytes, error;
} kvr_stats;

typedef struct kvr_ctx kvr_ctx;

/* Validate `cfg` and create a context on the current HIP device.  Allocates
 * only a small device table of layer pointers.  *out is NULL on failure. */
int kvr_create(const kvr_config *cfg, kvr_ctx **out);

/* Free the context (not the bound buffers).  NULL is accepted. */
int kvr_destroy(kvr_ctx *ctx);

/* Message for the calling thread's last non-OK return ("" if none). */
const char *kvr_last_error(void);

/* Bind the source's metadata (all device):
 *   L         int32  [n_req]              rows held: H + decoded rows
 *   page_map  int32  [n_req][ceil(H/P)]   physical page of a ready complete
 *                                          page, else -1 (a trailing partial
 *                                          page is never ready)
 *   host_valid uint8 [n_req][ceil(H/P)]   1 if the imported page has a host copy
 *   tag       int32  [n_req][B]           row held by a hot slot, -1 = empty
 *   stamp     uint32 [n_req][B]           LRU stamp of a hot slot
 *   clock     uint32 [n_req]              last LRU tick of the request
 * page_map and host_valid change only in kvr_reclaim_pages and
 * kvr_restore_pages. */
int kvr_bind_metadata(kvr_ctx *ctx, int32_t *L, int32_t *page_map, uint8_t *host_valid,
                      int32_t *tag, uint32_t *stamp, uint32_t *clock);

/* Bind one payload layer:
 *   tail (device) [n_req][T][R], pool (device) [pool_pages][P][R] (written
 *   only by kvr_restore_pages),
 *   hot (device) [n_req][B][R], host (pinned) [n_req][H + max_new][R].
 * tail may be NULL when T = 0 and pool when pool_pages = 0. */
int kvr_bind_layer(kvr_ctx *ctx, int32_t layer, void *tail, void *pool, void *hot,
                   void *host);

/* Fresh admission: L = H, every tag -1, every stamp 0, every clock 0. */
int kvr_init_state(kvr_ctx *ctx, void *stream);

/* Append one decoded row to each listed request, for every layer: the row
 * goes to tail slot L mod T and, written through, to host row L; then L += 1.
 * Decoded rows never enter optional pages (section "Limits": they follow
 * hot-cache rules), which is why they get a host copy.
 *   req_ids  (device) int32 [n] or NULL (= 0..n-1); distinct
 *   new_rows (device) [n_layers][n][R]
 *   status   (device) int32 [n] or NULL: KVR_OK, or KVR_E_CAPACITY when the
 *            request already holds H + max_new rows (nothing written). */
int kvr_append_rows(kvr_ctx *ctx, int32_t n, const int32_t *req_ids, const void *new_rows,
                    int32_t *status, void *stream);

/* Resolve one selection per listed request ("Resolution", steps 1-3).
 *   sel       (device) int32 [n][stride], rows of request i in sel[i][0..cnt)
 *   sel_count (device) int32 [n] or NULL (= stride); 0 <= cnt <= stride <= sel_cap
 *   loc       (device) uint32 [n][stride] out; entries >= cnt untouched
 *   fills     (device) kvr_fill [n][B] out: the rows copied from host, by
 *             ascending row; fill_count (device) int32 [n] out
 *   fill_layer payload layer refilled from host now, or -1 for none (the
 *             fills can be replayed into any layers with kvr_reuse_locations)
 *   status    (device) int32 [n] out, required
 *   stats     (device) kvr_stats or NULL, added to
 * Per request, with now = clock + 1 (one tick per call):
 *   1. a row in [max(0, L - T), L) is in the tail; else a row of a ready
 *      complete page is in the optional pool; else it is pending;
 *   2. each distinct pending row is looked for among the B tags; a hit
 *      stamps its slot with now;
 *   3. misses, by ascending row, take the slots not hit in this call with the
 *      smallest (stamp, slot), which get the row's tag and stamp now, and the
 *      host copy is fetched into them.
 * Repeated rows in one selection share one location. */
int kvr_resolve_rows(kvr_ctx *ctx, int32_t n, const int32_t *req_ids, const int32_t *sel,
                     const int32_t *sel_count, int32_t stride, uint32_t *loc, kvr_fill *fills,
                     int32_t *fill_count, int32_t fill_layer, int32_t *status, kvr_stats *stats,
                     void *stream);

/* kvr_append_rows followed by kvr_resolve_rows for the same requests, in one
 * launch: each request's row is appended (tail slot L mod T, host row L,
 * L += 1) before its selection is resolved against the new length.  The
 * arguments are those of the two calls (new_rows and append_status as in
 * kvr_append_rows; append_status may be NULL).  An append that fails
 * (KVR_E_CAPACITY) changes nothing and the resolve still runs, as with the
 * two calls; an entry whose request id is out of range fails both; one whose
 * selection count is out of range fails its resolve (KVR_E_ARG) after its
 * append. */
int kvr_append_resolve_rows(kvr_ctx *ctx, int32_t n, const int32_t *req_ids, const void *new_rows,
                            int32_t *append_status, const int32_t *sel, const int32_t *sel_count,
                            int32_t stride, uint32_t *loc, kvr_fill *fills, int32_t *fill_count,
                            int32_t fill_layer, int32_t *status, kvr_stats *stats, void *stream);

/* kvr_append_resolve_rows with the tail write of the append deferred, so
 * that the resolve of the next decode step may run while the previous step's
 * rows are still being gathered (the step's KV write, "Memory split": the
 * tail is the writable part; "Limits": decoded rows get a host copy).  The
 * launch writes each appended row's host copy and advances L, but leaves its
 * tail slot (L mod T) alone: that slot still holds the row L - T, which a
 * gather of the previous step may be reading.  append_pos (device) int32 [n]
 * receives, per entry, the position appended, or -1 when the entry appended
 * nothing (a failed append or a bad request id).  The resolve itself sees
 * the new length, exactly as after kvr_append_resolve_rows.  The appends are
 * completed by kvr_fused_gather_append_rows with the same entries, new_rows
 * and append_pos; until then a gather other than that one must not read the
 * tail slot of an appended row.  Other arguments and errors as for
 * kvr_append_resolve_rows. */
int kvr_append_resolve_rows_deferred(kvr_ctx *ctx, int32_t n, const int32_t *req_ids,
                                     const void *new_rows, int32_t *append_status,
                                     int32_t *append_pos, const int32_t *sel,
                                     const int32_t *sel_count, int32_t stride, uint32_t *loc,
                                     kvr_fill *fills, int32_t *fill_count, int32_t fill_layer,
                                     int32_t *status, kvr_stats *stats, void *stream);

/* Gather resolved rows into contiguous per-request buffers, for several
 * payload layers sharing one location vector ("Adaptive DHiSparse", section
 * "How it works", paragraph "Model-specific reuse": a layer reads its rows
 * where the location vector says; layers with shared sparse indices but
 * their own payloads each read their own bytes at the same locations):
 *   out[l] (device) [n][stride][R] for layers[l]; row j < cnt of request i is
 *   the R bytes at loc[i][j] in that layer (a fresh hot-cache row is read
 *   from its slot, so its fill must have run).  Invalid locations leave the
 *   row untouched.
 *   layers (host) int32 [n_layers]; out (host) array of n_layers device pointers
 *   loc (device) uint32 [n][stride]; count (device) int32 [n] or NULL (= stride)
 *   status (device) int32 [n] or NULL: set to KVR_E_RANGE for a request with a
 *   location outside its place, otherwise not written (clear it beforehand). */
int kvr_gather_rows(kvr_ctx *ctx, int32_t n_layers, const int32_t *layers, int32_t n,
                    const int32_t *req_ids, const uint32_t *loc, const int32_t *count,
                    int32_t stride, void *const *out, int32_t *status, void *stream);

/* The same gather split in two so that host fills and HBM gathers overlap
 * (same arguments as kvr_gather_rows; together the two write what
 * kvr_gather_rows writes after the fills):
 *   kvr_gather_resident_rows copies every row whose location is not a fresh
 *     hot-cache word (tail, page, hot-cache hit).  It reads no slot a fill of
 *     the same call writes, so it may run while those fills are in flight.
 *   kvr_fill_gather_rows copies every fresh row once from the layer's pinned
 *     host store into both the layer's hot-cache slot and the output: the
 *     host fill of that layer and its gather in one pass over the host link.
 *     sel (device) int32 [n][stride] is the selection the resolve call took
 *     (entry j's row); it reads no tag, so a later resolve of the same
 *     requests may run beside it.  Use it instead of fill_layer and
 *     kvr_reuse_locations(KVR_REUSE_DISTINCT_PAYLOAD) for these layers;
 *     repeated rows fetch their host copy once per repeat. */
int kvr_gather_resident_rows(kvr_ctx *ctx, int32_t n_layers, const int32_t *layers, int32_t n,
                             const int32_t *req_ids, const uint32_t *loc, const int32_t *count,
                             int32_t stride, void *const *out, int32_t *status, void *stream);
int kvr_fill_gather_rows(kvr_ctx *ctx, int32_t n_layers, const int32_t *layers, int32_t n,
                         const int32_t *req_ids, const uint32_t *loc, const int32_t *sel,
                         const int32_t *count, int32_t stride, void *const *out, int32_t *status,
                         void *stream);

/* kvr_fill_gather_rows and kvr_gather_resident_rows as one launch (same
 * arguments as kvr_fill_gather_rows; writes what the two write together):
 * part of the grid fills fresh rows from host while the rest gathers the
 * resident rows, with no wait between two launches on two streams.  Errors as
 * for the two calls. */
int kvr_fused_gather_rows(kvr_ctx *ctx, int32_t n_layers, const int32_t *layers, int32_t n,
                          const int32_t *req_ids, const uint32_t *loc, const int32_t *sel,
                          const int32_t *count, int32_t stride, void *const *out, int32_t *status,
                          void *stream);

/* kvr_fused_gather_rows that also completes the appends a
 * kvr_append_resolve_rows_deferred call left pending for the same entries
 * (same req_ids and n): for each entry with append_pos[i] >= 0, new_rows
 * (device) [n_layers of the context][n][R] row i of every layer goes into
 * tail slot append_pos[i] mod T, and a tail word of that entry naming that
 * slot is gathered from new_rows (the same bytes).  The call must name every
 * payload layer of the context exactly once (KVR_E_ARG otherwise), so every
 * layer's tail receives its row; with an empty selection (stride 0 or
 * counts 0) it still writes the rows.  Outputs and errors as for
 * kvr_fused_gather_rows. */
int kvr_fused_gather_append_rows(kvr_ctx *ctx, int32_t n_layers, const int32_t *layers, int32_t n,
                                 const int32_t *req_ids, const uint32_t *loc, const int32_t *sel,
                                 const int32_t *count, int32_t stride, void *const *out,
                                 int32_t *status, const void *new_rows, const int32_t *append_pos,
                                 void *stream);

/* One fused gather, as the arguments of kvr_fused_gather_append_rows
 * (new_rows and append_pos NULL: of kvr_fused_gather_rows).  layers and out
 * are host arrays of n_layers entries; the other pointers as documented
 * there. */
typedef struct kvr_gather_call {
    int32_t n_layers;
    const int32_t *layers;
    int32_t n;
    const int32_t *req_ids;
    const uint32_t *loc;
    const int32_t *sel;
    const int32_t *count;
    int32_t stride;
    void *const *out;
    int32_t *status;
    const void *new_rows;
    const int32_t *append_pos;
} kvr_gather_call;

/* One resolve, as the arguments of kvr_append_resolve_rows_deferred
 * (new_rows, append_status and append_pos NULL: of kvr_resolve_rows), with
 * no host fill (fill_layer -1). */
typedef struct kvr_resolve_call {
    int32_t n;
    const int32_t *req_ids;
    const void *new_rows;
    int32_t *append_status;
    int32_t *append_pos;
    const int32_t *sel;
    const int32_t *sel_count;
    int32_t stride;
    uint32_t *loc;
    kvr_fill *fills;
    int32_t *fill_count;
    int32_t *status;
    kvr_stats *stats;
} kvr_resolve_call;

/* The gather of one resolved selection and the resolve of the next one (the
 * next resolving layer's, or the next decode step's) in one launch ("How it
 * works": the resolve of "Resolution" and the gather the location vector of
 * "Model-specific reuse" feeds), so that the resolve leaves the critical
 * path without a wait between two queues.  Same results as
 * kvr_fused_gather_append_rows (or kvr_fused_gather_rows) with `gather`
 * followed by kvr_append_resolve_rows_deferred (or kvr_resolve_rows) with
 * `resolve`, provided the resolve writes none of the buffers the gather
 * reads (its loc, sel, count, new_rows and append_pos: give the two calls
 * different buffers, e.g. two sets used in turn).  The two never touch the
 * same state otherwise: the resolve reads and writes metadata and writes the
 * host copy of appended rows (beyond every row the gather fetches); the
 * gather writes hot-cache slots, tails and outputs.  An append in `resolve`
 * must be deferred (append_pos given): its tail slot may still be read by the
 * gather.  Either call may be NULL (then this is the other call alone);
 * argument errors of either half are returned before anything is launched.
 * Calls on one stream run in order, so a decode loop issues, per resolving
 * layer, this call with the previous layer's gather and this layer's
 * resolve, and ends with the last gather alone. */
int kvr_gather_resolve_rows(kvr_ctx *ctx, const kvr_gather_call *gather,
                            const kvr_resolve_call *resolve, void *stream);

/* Verification block dedup ("Speculative state": queries share missing-row
 * retrieval).  Per request: union_rows[i][0..u) = the distinct rows of the q
 * selections, ascending; map[i][qi][j] = index of sel[i][qi][j] in it.
 *   sel (device) int32 [n][q][k]; union_rows (device) int32 [n][q*k];
 *   union_count (device) int32 [n]; map (device) int32 [n][q][k].
 *   Requires q * k <= 8192.  The union is then resolved once. */
int kvr_dedup_verify_selections(kvr_ctx *ctx, int32_t n, int32_t q, int32_t k, const int32_t *sel,
                                int32_t *union_rows, int32_t *union_count, int32_t *map,
                                void *stream);

/* Location reuse across layers ("Model-specific reuse"); see kvr_reuse_mode.
 *   SHARED_SOURCE: dst_layers may be NULL; dst_loc (optional) gets src_loc.
 *   DISTINCT_PAYLOAD: the fills are replayed into every listed layer, all in
 *     one launch per 24 layers: row `row` of that layer's host store is copied
 *     into hot slot `slot` of that layer.
 *   dst_layers (host) int32 [n_layers]
 *   src_loc/dst_loc (device) uint32 [n][stride]; count (device) int32 [n] or NULL
 *   fills/fill_count (device): from the resolve call (DISTINCT_PAYLOAD only)
 *   status (device) int32 [n] or NULL: set to KVR_E_RANGE if a fill names a
 *   row or slot out of range, otherwise not written. */
int kvr_reuse_locations(kvr_ctx *ctx, int32_t mode, int32_t n_layers, const int32_t *dst_layers,
                        int32_t n, const int32_t *req_ids, const uint32_t *src_loc,
                        uint32_t *dst_loc, const int32_t *count, int32_t stride,
                        const kvr_fill *fills, const int32_t *fill_count, int32_t *status,
                        void *stream);

/* Optional-pool residency ("Adaptive DHiSparse", section "How it works",
 * paragraph "Reclamation and refill"): no row is ever lost, since a page
 * leaves the GPU only with a host backup in place and only once the kernels
 * that read it earlier are done; pages taken away are brought back later.
 *
 * kvr_reclaim_pages: the listed (req_ids[i], pages[i]) optional pages stop
 * being ready.  A page without a host copy first gets one (its P rows of
 * every payload layer are written from the pool to the host store over the
 * host link), then page_map becomes -1 and host_valid 1.  Stream order makes
 * the release wait for the kernels enqueued before it (earlier readers), and
 * every later kernel sees the page released.
 *   req_ids, pages (device) int32 [n]
 *   freed_phys (device) int32 [n]: the physical page entry i released, or -1
 *     if that page was not ready (also for a repeat of an earlier entry)
 *   status (device) int32 [n] or NULL: KVR_E_ARG for a request or page index
 *     out of range, KVR_E_STATE for a corrupt map entry (a physical page
 *     outside the pool, or an incomplete page marked ready; nothing moves),
 *     else KVR_OK.
 * kvr_restore_pages: the listed pages become ready in physical pages phys[i]:
 * their host rows of every layer are copied into the pool, then page_map
 * points at them.
 *   req_ids, pages, phys (device) int32 [n]; the caller hands out physical
 *     pages that no ready page maps (kvr_residency_refill does)
 *   status (device) int32 [n] or NULL: KVR_E_ARG for a request or page index
 *     out of range, a page that is not complete imported history, or a page
 *     or physical page that an earlier entry names; else KVR_E_RANGE for a
 *     physical page outside the pool; else KVR_E_STATE if the page is ready;
 *     else KVR_E_NO_HOST_COPY if it has no host copy; a failed entry changes
 *     nothing.
 * Both enqueue one kernel on `stream`; n = 0 is a no-op; n is at most
 * n_req * ceil(H/P). */
int kvr_reclaim_pages(kvr_ctx *ctx, int32_t n, const int32_t *req_ids, const int32_t *pages,
                      int32_t *freed_phys, int32_t *status, void *stream);
int kvr_restore_pages(kvr_ctx *ctx, int32_t n, const int32_t *req_ids, const int32_t *pages,
                      const int32_t *phys, int32_t *status, void *stream);

/* Host-side residency policy of one KV source's optional pool (no device
 * work; the caller applies its decisions with the two calls above).
 *
 * kvr_residency_create: page_map (host) int32 [n_req][n_pages] the initial
 *   map, of which the first n_complete pages per request may be optional;
 *   pool_pages physical pages in the pool, those no page maps are free.
 * kvr_residency_admit: an admission needing `need` physical pages.  Free
 *   pages are used first; the pages still missing (the shortfall) come from
 *   requests that give up every ready page they hold, one request at a time
 *   in `order` (n_order request ids, the reclaim order), until enough are
 *   free; the requests after that keep theirs.  The lowest free page ids are
 *   reserved for the admission.  Writes the (request, page) list to reclaim,
 *   in that order (at most `cap` entries), and a handle.  Returns
 *   KVR_E_CAPACITY when the shortfall is larger than all optional pages
 *   together (the admission waits; nothing changes, *n_out = 0),
 *   KVR_E_ARG when the list would exceed `cap` (nothing changes).
 * kvr_residency_release: the admission drained; its pages are free again.
 * kvr_residency_refill: bounded round-robin refill of the pages that
 *   reclamation took (residency repopulates as load drains): requests are
 *   visited cyclically from a cursor kept between calls, each visit giving
 *   one request its lowest-index reclaimed page not yet back and the lowest
 *   free physical page, until `bound` pages (at most `cap`), no free page, or
 *   a whole cycle without such a page; the cursor then points after the last
 *   request served.  Pages not ready at creation are never refilled.  Writes
 *   (request, page, physical page) triples.
 * kvr_residency_counts: free, ready and reserved physical pages.
 * The object is not thread-safe. */
typedef struct kvr_residency kvr_residency;

int kvr_residency_create(int32_t n_req, int32_t n_pages, int32_t n_complete, int64_t pool_pages,
                         const int32_t *page_map, kvr_residency **out);
int kvr_residency_destroy(kvr_residency *res);
int kvr_residency_admit(kvr_residency *res, int64_t need, int32_t n_order, const int32_t *order,
                        int32_t cap, int32_t *req_out, int32_t *page_out, int32_t *n_out,
                        int32_t *handle);
int kvr_residency_release(kvr_residency *res, int32_t handle);
int kvr_residency_refill(kvr_residency *res, int32_t bound, int32_t cap, int32_t *req_out,
                         int32_t *page_out, int32_t *phys_out, int32_t *n_out);
int kvr_residency_counts(const kvr_residency *res, int64_t *free_pages, int64_t *ready_pages,
                         int64_t *reserved_pages);

/* Speculative state ("Adaptive DHiSparse", section "How it works",
 * paragraph "Speculative state").
 *
 * Drafter visible-window ring: the drafter stores no more than the rows it can
 * still see.  Per
 * request, drafter rows are numbered by position; row p lives in slot p mod C
 * of a ring of C >= W slots; the visible window is the last min(W, length)
 * positions.  The C - W extra slots let rows that verification rejects be
 * dropped: a rollback to a shorter length is allowed while no position
 * written since (kept or dropped) has overwritten the window it leaves
 * visible, i.e. for keep >= (highest position ever written + 1) - (C - W).
 *   kvr_draft_create: ring (device) [n_req][C][row_bytes] (row_bytes a
 *     multiple of 16), length and high (device) int32 [n_req] (rows kept, and
 *     highest position ever written + 1); all caller-owned; the current device
 *     is the ring's.  kvr_draft_reset zeroes length and high (stream-ordered).
 *   kvr_draft_append: rows (device) [n][rows_each][row_bytes], rows_each <= C,
 *     appended at positions length .. length + rows_each - 1.
 *   kvr_draft_rollback: keep (device) int32 [n]; status KVR_E_RANGE (nothing
 *     changes) when keep is above the length or below the rollback limit.
 *   kvr_draft_window: out (device) [n][W][row_bytes] receives the visible rows
 *     oldest first (rows past the window are untouched); visible (device)
 *     int32 [n] or NULL receives their number.
 *   status (device) int32 [n] or NULL: KVR_E_ARG for a request out of range.
 * req_ids (device) int32 [n] or NULL (= 0 .. n-1) name each request at most
 * once per call.  All calls enqueue one kernel on `stream` and never
 * synchronise the host. */
typedef struct kvr_draft kvr_draft;

int kvr_draft_create(int32_t n_req, int32_t window, int32_t capacity, int32_t row_bytes,
                     void *ring, int32_t *length, int32_t *high, kvr_draft **out);
int kvr_draft_destroy(kvr_draft *d);
int kvr_draft_reset(kvr_draft *d, void *stream);
int kvr_draft_append(kvr_draft *d, int32_t n, const int32_t *req_ids, int32_t rows_each,
                     const void *rows, int32_t *status, void *stream);
int kvr_draft_rollback(kvr_draft *d, int32_t n, const int32_t *req_ids, const int32_t *keep,
                       int32_t *status, void *stream);
int kvr_draft_window(kvr_draft *d, int32_t n, const int32_t *req_ids, void *out,
                     int32_t *visible, int32_t *status, void *stream);

/* Verification staging reuse: a target layer's staging buffer is handed out
 * again only after the kernels that read it have finished.  A pool of n_buffers caller-owned buffers, named by
 * index and handed out round-robin.  kvr_staging_acquire makes `stream` wait
 * until the buffer's previous consumer has released it; kvr_staging_release
 * records that release on the consumer's stream after its last read of the
 * buffer.  Host object, not thread-safe; acquire and release enqueue only an
 * event wait or record.  Not meant for graph capture (a release recorded
 * before the capture is not visible to it). */
typedef struct kvr_staging kvr_staging;

int kvr_staging_create(int32_t n_buffers, kvr_staging **out);
int kvr_staging_destroy(kvr_staging *p);
int kvr_staging_acquire(kvr_staging *p, void *stream, int32_t *index);
int kvr_staging_release(kvr_staging *p, int32_t index, void *stream);

/* Host helper, after the caller has synchronised and copied status to host:
 * number of failed requests; *first_bad = index of the first (or -1). */
int kvr_status_summary(const int32_t *status, int32_t n, int32_t *first_bad);

/* Page-locked, device-mapped host memory for host stores (hipHostMalloc).
 * Returns KVR_E_HIP on failure. */
int kvr_host_alloc(size_t bytes, void **out);
int kvr_host_free(void *ptr);

/* Kernel launch timing (measurement aid, not part of the method).
 *
 * Between kvr_timing_begin and kvr_timing_end every kernel the context
 * launches carries a start and a stop event of its own dispatch
 * (hipExtLaunchKernel), so each recorded duration is the kernel's execution
 * alone, the interval a kernel-trace profiler reports, without the gaps
 * between launches.  Launches on a stream that is being captured into a graph
 * are not recorded.
 *
 * kvr_timing_begin: capacity = most launches to record (1 .. 1048576).
 *   Creates the events when the context has fewer than that (this is the
 *   only call here that allocates), then starts recording; launches past the
 *   capacity run untimed and are counted.
 * kvr_timing_end: stops recording, waits for the recorded launches and
 *   writes, for each in launch order, kinds[i] (kvr_kernel) and ms[i] (host
 *   arrays of `capacity` entries); *n_recorded = launches recorded.  Returns
 *   KVR_E_CAPACITY if launches went untimed or did not fit the arrays (the
 *   entries that fit are still written), KVR_E_ARG if recording was not on. */
typedef enum kvr_kernel {
    KVR_KERNEL_APPEND = 0,
    KVR_KERNEL_RESOLVE = 1,
    KVR_KERNEL_REFILL = 2,   /* host refill and per-layer replays */
    KVR_KERNEL_GATHER = 3,
    KVR_KERNEL_DEDUP = 4,
    KVR_KERNEL_STATE = 5,    /* state initialisation, location copies */
    KVR_KERNEL_FUSED = 6,    /* fill pass and resident gather in one launch */
    KVR_KERNEL_STEP = 7,     /* a fused gather beside the next resolve */
} kvr_kernel;

int kvr_timing_begin(kvr_ctx *ctx, int32_t capacity);
int kvr_timing_end(kvr_ctx *ctx, int32_t capacity, int32_t *kinds, float *ms,
                   int32_t *n_recorded);

#ifdef __cplusplus
}
#endif

#endif /* KVR_H */
