/*
 * CPU reference ("the oracle") for the per-decode-step sparse KV row resolver.
 *
 * TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's
 * CPU-baseline leg call this; the product path never does.  It shares no code,
 * header or constant table with the GPU library: every rule is written out
 * here again, plainly and slowly, from "Adaptive DHiSparse: Speculative
 * Decoding over a Load-Adaptive KV Hierarchy" (page 1 of the source pages).
 *
 * What the page fixes (section "How it works"):
 *   - Memory split: per KV source, a request has its own B-slot hot cache,
 *     a writable tail and its metadata; whole pages of the history it arrived
 *     with may also be kept in an optional pool that can be taken back.
 *   - Reclamation and refill: no row is ever only in a released page: it is
 *     ready on the GPU, in host memory, or both.
 *   - Resolution: for each selected row try, in this order, (1) the tail,
 *     then the ready pages through the optional map, (2) the hot cache, where
 *     a lookup examines at most B slots and replacement is LRU, (3) the
 *     pinned host store, whose row is copied into a hot-cache slot; the first
 *     place that has the row wins.
 *   - Speculative state: the queries of one verification block fetch each
 *     missing row once between them.
 *   - Model-specific reuse: Reuse layers inherit a location vector (one
 *     physical source); shared indices with distinct payloads replay the same
 *     positions per layer.
 *   - Limits: rows produced by decoding follow hot-cache rules (they never
 *     enter optional pages).
 *
 * Where the page is silent this file takes one reading, stated at the place
 * it is used: one LRU tick per resolve call, victims ordered by ascending
 * (stamp, slot), ascending missing rows paired with ascending victims, slots
 * hit in a call never chosen as victims, the tail checked before pages, and a
 * failed request committing nothing.
 *
 * Location word: bits 31..30 hold the place (0 tail, 1 optional page, 2 hot
 * cache, 3 invalid) and bits 29..0 the index there (ring slot, global pool row
 * = physical page * P + offset, or hot slot).  In a hot-cache word bit 29 is
 * the fresh flag: the row was copied from host memory by this call (a
 * consumer can take those bytes as they arrive); bits 28..0 are the slot.
 * 0xFFFFFFFF marks a row of a failed request.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum {
    ORC_OK = 0,
    ORC_E_ARG = -1,
    ORC_E_RANGE = -2,
    ORC_E_CAPACITY = -3,
    ORC_E_NO_HOST_COPY = -4,
    ORC_E_STATE = -6,
};

#define ORC_INVALID 0xFFFFFFFFu
#define ORC_FRESH (1u << 29) /* hot-cache word: the row was copied from host in this call */

/* statistics slots, added to by every call */
enum { ST_CALLS, ST_TAIL, ST_PAGE, ST_HIT, ST_MISS, ST_FILL, ST_HOST_BYTES, ST_ERROR, ST_N };

typedef struct orc_source {
    int32_t n_req, n_layers, H, max_new, P, T, B, R;
    int64_t pool_pages;
    int32_t *L;                 /* [n_req] rows held (imported + decoded)        */
    int32_t *page_map;          /* [n_req][n_pages] physical page or -1           */
    uint8_t *host_valid;        /* [n_req][n_pages] imported page has host copy   */
    int32_t *tag;               /* [n_req][B] row held by the slot, -1 = empty    */
    uint32_t *stamp;            /* [n_req][B] LRU stamp                           */
    uint32_t *clock;            /* [n_req]    last tick                           */
    uint8_t **tail;             /* per layer [n_req][T][R]                        */
    uint8_t **pool;             /* per layer [pool_pages][P][R]                   */
    uint8_t **hot;              /* per layer [n_req][B][R]                        */
    uint8_t **host;             /* per layer [n_req][H + max_new][R]              */
} orc_source;

static int32_t n_pages_of(const orc_source *s) { return (s->H + s->P - 1) / s->P; }
static int64_t host_rows_of(const orc_source *s) { return (int64_t)s->H + s->max_new; }

/* ---------------------------------------------------------------- append */

/* A decoded row joins the tail ring at position L mod T and is written
 * through to the host store (it follows hot-cache rules once it leaves the
 * tail, so it needs a host copy: the page's "Limits" and the invariant of
 * "Reclamation and refill").  new_rows: [n_layers][n_req][R]. */
int orc_append_one(const orc_source *s, int32_t r, const uint8_t *new_rows)
{
    int32_t L = s->L[r];
    if (L < 0 || (int64_t)L >= host_rows_of(s))
        return ORC_E_CAPACITY;
    for (int32_t l = 0; l < s->n_layers; ++l) {
        const uint8_t *row = new_rows + ((int64_t)l * s->n_req + r) * s->R;
        if (s->T > 0)
            memcpy(s->tail[l] + ((int64_t)r * s->T + L % s->T) * s->R, row, (size_t)s->R);
        memcpy(s->host[l] + ((int64_t)r * host_rows_of(s) + L) * s->R, row, (size_t)s->R);
    }
    s->L[r] = L + 1;
    return ORC_OK;
}

/* ---------------------------------------------------------------- resolve */

static int cmp_i32(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

typedef struct { uint32_t stamp; int32_t slot; } cand_t;

static int cmp_cand(const void *a, const void *b)
{
    const cand_t *x = (const cand_t *)a, *y = (const cand_t *)b;
    if (x->stamp != y->stamp)
        return x->stamp < y->stamp ? -1 : 1;
    return (x->slot > y->slot) - (x->slot < y->slot);
}

/* index of v in the ascending array a[0..n), or -1 */
static int32_t find_sorted(const int32_t *a, int32_t n, int32_t v)
{
    int32_t lo = 0, hi = n;
    while (lo < hi) {
        int32_t mid = lo + (hi - lo) / 2;
        if (a[mid] < v)
            lo = mid + 1;
        else
            hi = mid;
    }
    return (lo < n && a[lo] == v) ? lo : -1;
}

/*
 * Resolve one selection of request r (k entries) against its KV source.
 *   loc[k]            out: location word per entry
 *   fills[2 * B]      out: (row, slot) pairs filled from host, ascending row
 *   fill_count        out
 *   fill_layer        payload layer copied host -> hot (-1: none)
 *   stats[ST_N]       added to
 * Returns the request's status.  On any error nothing is committed (tags,
 * stamps, clock and hot payload are untouched) and every loc is 0xFFFFFFFF.
 */
int orc_resolve_one(const orc_source *s, int32_t r, const int32_t *sel, int32_t k,
                    int32_t fill_layer, uint32_t *loc, int32_t *fills, int32_t *fill_count,
                    uint64_t *stats)
{
    const int32_t B = s->B, T = s->T, P = s->P, H = s->H;
    const int32_t L = s->L[r];
    int32_t *tag = s->tag + (int64_t)r * B;
    uint32_t *stamp = s->stamp + (int64_t)r * B;
    const int32_t *pmap = s->page_map + (int64_t)r * n_pages_of(s);
    const uint8_t *hvalid = s->host_valid + (int64_t)r * n_pages_of(s);
    int status = ORC_OK;

    *fill_count = 0;
    stats[ST_CALLS] += 1;

    /* every selected row must exist */
    for (int32_t j = 0; j < k; ++j)
        if (sel[j] < 0 || sel[j] >= L)
            status = ORC_E_RANGE;
    if (status == ORC_OK && s->clock[r] == UINT32_MAX)
        status = ORC_E_STATE;
    if (status != ORC_OK) {
        for (int32_t j = 0; j < k; ++j)
            loc[j] = ORC_INVALID;
        stats[ST_ERROR] += 1;
        return status;
    }
    /* one LRU tick per call: everything touched by this call shares it */
    const uint32_t now = s->clock[r] + 1;

    /* Step 1: the tail holds rows [max(0, L - T), L); a complete imported page
     * is "ready" when the page map gives it a physical page.  The tail is
     * looked at first. */
    const int32_t tail_lo = (T > 0) ? (L - T > 0 ? L - T : 0) : L;
    const int32_t full_rows = (H / P) * P;
    uint8_t *kind = (uint8_t *)malloc((size_t)(k > 0 ? k : 1));
    int32_t *pend = (int32_t *)malloc(sizeof(int32_t) * (size_t)(k > 0 ? k : 1));
    int32_t n_pend = 0;
    for (int32_t j = 0; j < k; ++j) {
        int32_t pos = sel[j];
        if (pos >= tail_lo) {
            kind[j] = 0;
        } else if (pos < full_rows && pmap[pos / P] >= 0) {
            kind[j] = 1;
        } else {
            kind[j] = 2;
            pend[n_pend++] = pos;
        }
    }

    /* U: the distinct pending rows, ascending */
    qsort(pend, (size_t)n_pend, sizeof(int32_t), cmp_i32);
    int32_t nU = 0;
    for (int32_t i = 0; i < n_pend; ++i)
        if (nU == 0 || pend[nU - 1] != pend[i])
            pend[nU++] = pend[i];
    int32_t *U = pend;

    /* Step 2: for every pending row, compare it with the B tags of the hot
     * cache (the scan never looks beyond B slots, however long the history). */
    int32_t *slot_of = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nU > 0 ? nU : 1));
    uint8_t *hit_slot = (uint8_t *)calloc((size_t)B, 1);
    int32_t n_hit = 0, n_miss = 0;
    for (int32_t i = 0; i < nU; ++i) {
        slot_of[i] = -1;
        for (int32_t b = 0; b < B; ++b) {
            if (tag[b] == U[i]) {
                slot_of[i] = b;
                break;
            }
        }
        if (slot_of[i] >= 0) {
            hit_slot[slot_of[i]] = 1;
            ++n_hit;
        } else {
            ++n_miss;
        }
    }

    /* every missing row needs a free-able slot and a host copy */
    if (n_hit + n_miss > B) {
        status = ORC_E_CAPACITY;
    } else {
        for (int32_t i = 0; i < nU; ++i) {
            int32_t u = U[i];
            if (slot_of[i] < 0 && u < H && !hvalid[u / P])
                status = ORC_E_NO_HOST_COPY;
        }
    }
    if (status != ORC_OK) {
        for (int32_t j = 0; j < k; ++j)
            loc[j] = ORC_INVALID;
        stats[ST_ERROR] += 1;
        free(kind), free(pend), free(slot_of), free(hit_slot);
        return status;
    }

    /* Step 3: least recently used first.  Candidates are the slots not hit in
     * this call, ordered by (stamp, slot); the i-th smallest missing row takes
     * the i-th candidate.  Empty slots carry stamp 0 and so go first. */
    cand_t *cand = (cand_t *)malloc(sizeof(cand_t) * (size_t)B);
    int32_t n_cand = 0;
    for (int32_t b = 0; b < B; ++b)
        if (!hit_slot[b])
            cand[n_cand++] = (cand_t){stamp[b], b};
    qsort(cand, (size_t)n_cand, sizeof(cand_t), cmp_cand);

    /* commit */
    s->clock[r] = now;
    for (int32_t i = 0; i < nU; ++i)
        if (slot_of[i] >= 0)
            stamp[slot_of[i]] = now;
    int32_t m = 0;
    for (int32_t i = 0; i < nU; ++i) {
        if (slot_of[i] >= 0)
            continue;
        int32_t v = cand[m].slot;
        tag[v] = U[i];
        stamp[v] = now;
        slot_of[i] = v;
        fills[2 * m] = U[i];
        fills[2 * m + 1] = v;
        if (fill_layer >= 0) {
            const uint8_t *src = s->host[fill_layer] + ((int64_t)r * host_rows_of(s) + U[i]) * s->R;
            uint8_t *dst = s->hot[fill_layer] + ((int64_t)r * B + v) * s->R;
            memcpy(dst, src, (size_t)s->R);
        }
        ++m;
    }
    *fill_count = m;

    /* location words, in selection order; repeated rows share one location */
    for (int32_t j = 0; j < k; ++j) {
        int32_t pos = sel[j];
        if (kind[j] == 0) {
            loc[j] = (0u << 30) | (uint32_t)(pos % T);
            stats[ST_TAIL] += 1;
        } else if (kind[j] == 1) {
            loc[j] = (1u << 30) | (uint32_t)((int64_t)pmap[pos / P] * P + pos % P);
            stats[ST_PAGE] += 1;
        } else {
            int32_t i = find_sorted(U, nU, pos);
            /* a row is a hit if its slot was already holding it before this call */
            int filled_now = 0;
            for (int32_t f = 0; f < m; ++f)
                if (fills[2 * f] == pos)
                    filled_now = 1;
            /* a row copied from host in this call carries the fresh flag */
            loc[j] = (2u << 30) | (filled_now ? ORC_FRESH : 0u) | (uint32_t)slot_of[i];
            stats[filled_now ? ST_MISS : ST_HIT] += 1;
        }
    }
    stats[ST_FILL] += (uint64_t)m;
    if (fill_layer >= 0)
        stats[ST_HOST_BYTES] += (uint64_t)m * (uint64_t)s->R;

    free(kind), free(pend), free(slot_of), free(hit_slot), free(cand);
    return ORC_OK;
}

/* ---------------------------------------------------------------- replay */

/* Shared indices, distinct payload: the rows filled for one layer are fetched
 * again for another layer from that layer's host store into the same slots. */
int orc_replay_one(const orc_source *s, int32_t layer, int32_t r, const int32_t *fills,
                   int32_t fill_count)
{
    for (int32_t i = 0; i < fill_count; ++i) {
        int32_t row = fills[2 * i], slot = fills[2 * i + 1];
        if (row < 0 || (int64_t)row >= host_rows_of(s) || slot < 0 || slot >= s->B)
            return ORC_E_RANGE;
        memcpy(s->hot[layer] + ((int64_t)r * s->B + slot) * s->R,
               s->host[layer] + ((int64_t)r * host_rows_of(s) + row) * s->R, (size_t)s->R);
    }
    return ORC_OK;
}

/* ---------------------------------------------------------------- gather */

/* out[j] = the R bytes at loc[j] of payload layer `layer`, for j < count.
 * Entries marked invalid are left as they are.  Returns ORC_E_RANGE if some
 * location points outside its place (that row is left as it is too). */
int orc_gather_one(const orc_source *s, int32_t layer, int32_t r, const uint32_t *loc,
                   int32_t count, uint8_t *out)
{
    int status = ORC_OK;
    for (int32_t j = 0; j < count; ++j) {
        uint32_t w = loc[j];
        if (w == ORC_INVALID)
            continue;
        uint32_t place = w >> 30, idx = w & 0x3FFFFFFFu;
        const uint8_t *src = NULL;
        if (place == 0 && idx < (uint32_t)s->T)
            src = s->tail[layer] + ((int64_t)r * s->T + idx) * s->R;
        else if (place == 1 && (int64_t)idx < s->pool_pages * s->P)
            src = s->pool[layer] + (int64_t)idx * s->R;
        else if (place == 2 && (idx & ~ORC_FRESH) < (uint32_t)s->B)
            src = s->hot[layer] + ((int64_t)r * s->B + (idx & ~ORC_FRESH)) * s->R;
        if (!src) {
            status = ORC_E_RANGE;
            continue;
        }
        memcpy(out + (int64_t)j * s->R, src, (size_t)s->R);
    }
    return status;
}

/* ---------------------------------------------------------------- dedup */

/* The q selections of one verification block fetch each missing row once:
 * their union (ascending, distinct) is resolved once, and map[qi][j] is the
 * union index of sel[qi][j].  sel, map: [q][k]; union_rows: [q * k]. */
int orc_dedup_one(int32_t q, int32_t k, const int32_t *sel, int32_t *union_rows,
                  int32_t *union_count, int32_t *map)
{
    int64_t n = (int64_t)q * k;
    memcpy(union_rows, sel, sizeof(int32_t) * (size_t)n);
    qsort(union_rows, (size_t)n, sizeof(int32_t), cmp_i32);
    int32_t u = 0;
    for (int64_t i = 0; i < n; ++i)
        if (u == 0 || union_rows[u - 1] != union_rows[i])
            union_rows[u++] = union_rows[i];
    *union_count = u;
    for (int64_t i = 0; i < n; ++i)
        map[i] = find_sorted(union_rows, u, sel[i]);
    return ORC_OK;
}

/* ---------------------------------------------------------------- residency */

/* Reclamation (section "How it works", paragraph "Reclamation and refill"):
 * the listed optional pages stop being ready.  A page without a host copy
 * (resident-first admission deferred its backup) first gets one: its P rows
 * of every layer are copied from the pool to the host store, so that every
 * row stays either ready or backed up; only then is the page released.
 * The list is taken in order.  freed[i] = the physical page released by entry
 * i, or -1 when that page was not ready (a repeat of an earlier entry
 * included); status[i] = ORC_E_ARG for a request or page index out of range,
 * ORC_E_STATE for a map entry outside the pool or on an incomplete page. */
void orc_reclaim_pages(orc_source *s, int32_t n, const int32_t *req, const int32_t *page,
                       int32_t *freed, int32_t *status)
{
    const int32_t np = n_pages_of(s);
    for (int32_t i = 0; i < n; ++i) {
        const int32_t r = req[i], p = page[i];
        freed[i] = -1;
        status[i] = ORC_OK;
        if (r < 0 || r >= s->n_req || p < 0 || p >= np) {
            status[i] = ORC_E_ARG;
            continue;
        }
        const int32_t phys = s->page_map[(int64_t)r * np + p];
        if (phys < 0)
            continue;
        if ((int64_t)phys >= s->pool_pages || p >= s->H / s->P) {
            status[i] = ORC_E_STATE;  /* a corrupt map entry: nothing moves */
            continue;
        }
        if (!s->host_valid[(int64_t)r * np + p]) {
            for (int32_t l = 0; l < s->n_layers; ++l) {
                uint8_t *dst = s->host[l] + ((int64_t)r * host_rows_of(s) + (int64_t)p * s->P) * s->R;
                const uint8_t *src = s->pool[l] + (int64_t)phys * s->P * s->R;
                memcpy(dst, src, (size_t)s->P * s->R);
            }
            s->host_valid[(int64_t)r * np + p] = 1;
        }
        s->page_map[(int64_t)r * np + p] = -1;
        freed[i] = phys;
    }
}

/* Refill ("Reclamation and refill"): the listed pages become ready again in
 * the given physical pages: the host rows of every layer are copied into the
 * pool, then the page map points at them.  The list is taken in order.
 * status[i]: ORC_E_ARG for a request or page index out of range, a page that
 * is not complete imported history, or a request/page or physical page that
 * an earlier entry already names; else ORC_E_RANGE for a physical page outside
 * the pool; else ORC_E_STATE if the page is already ready; else
 * ORC_E_NO_HOST_COPY if it has no host copy.  A failed entry changes nothing.
 * The caller hands out physical pages that no page maps. */
void orc_restore_pages(orc_source *s, int32_t n, const int32_t *req, const int32_t *page,
                       const int32_t *phys, int32_t *status)
{
    const int32_t np = n_pages_of(s);
    const int32_t complete = s->H / s->P;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t r = req[i], p = page[i], ph = phys[i];
        int st = ORC_OK;
        if (r < 0 || r >= s->n_req || p < 0 || p >= complete)
            st = ORC_E_ARG;
        for (int32_t j = 0; j < i && st == ORC_OK; ++j)
            if ((req[j] == r && page[j] == p) || phys[j] == ph)
                st = ORC_E_ARG;
        if (st == ORC_OK && (ph < 0 || (int64_t)ph >= s->pool_pages))
            st = ORC_E_RANGE;
        if (st == ORC_OK && s->page_map[(int64_t)r * np + p] >= 0)
            st = ORC_E_STATE;
        if (st == ORC_OK && !s->host_valid[(int64_t)r * np + p])
            st = ORC_E_NO_HOST_COPY;
        status[i] = st;
        if (st != ORC_OK)
            continue;
        for (int32_t l = 0; l < s->n_layers; ++l) {
            const uint8_t *src = s->host[l] + ((int64_t)r * host_rows_of(s) + (int64_t)p * s->P) * s->R;
            uint8_t *dst = s->pool[l] + (int64_t)ph * s->P * s->R;
            memcpy(dst, src, (size_t)s->P * s->R);
        }
        s->page_map[(int64_t)r * np + p] = ph;
    }
}

/* ---------------------------------------------------------------- invariants */

/* Bit mask of violated state invariants of request r:
 *   1: some row in [0, L) is neither in the tail, nor in a ready page, nor has
 *      a host copy (the page's residency invariant);
 *   2: a valid tag is outside [0, L) or two slots hold the same row;
 *   4: a stamp is newer than the request's clock. */
int orc_check_one(const orc_source *s, int32_t r)
{
    int bad = 0;
    const int32_t L = s->L[r], B = s->B, P = s->P, T = s->T;
    const int32_t *pmap = s->page_map + (int64_t)r * n_pages_of(s);
    const uint8_t *hvalid = s->host_valid + (int64_t)r * n_pages_of(s);
    const int32_t tail_lo = (T > 0) ? (L - T > 0 ? L - T : 0) : L;
    const int32_t full_rows = (s->H / P) * P;
    for (int32_t pos = 0; pos < L && pos < s->H; ++pos) {
        int in_tail = pos >= tail_lo;
        int ready = pos < full_rows && pmap[pos / P] >= 0;
        if (!in_tail && !ready && !hvalid[pos / P])
            bad |= 1;
    }
    const int32_t *tag = s->tag + (int64_t)r * B;
    const uint32_t *stamp = s->stamp + (int64_t)r * B;
    for (int32_t b = 0; b < B; ++b) {
        if (tag[b] >= 0) {
            if (tag[b] >= L)
                bad |= 2;
            for (int32_t c = b + 1; c < B; ++c)
                if (tag[c] == tag[b])
                    bad |= 2;
        } else if (tag[b] != -1) {
            bad |= 2;
        }
        if (stamp[b] > s->clock[r])
            bad |= 4;
    }
    return bad;
}

/* ---------------------------------------------------------------- batches */

/* Requests are independent, so a batch is the per-request functions above
 * run over request shards on host threads. */
typedef struct batch {
    const orc_source *s;
    int op;
    int32_t n;
    const int32_t *req_ids;
    const int32_t *sel;
    const int32_t *count;
    int32_t stride;
    int32_t layer;
    uint32_t *loc;
    const uint32_t *loc_in;
    int32_t *fills;
    int32_t *fill_count;
    int32_t *status;
    uint8_t *out;
    const uint8_t *rows;
    int32_t q;
    int32_t *union_rows;
    int32_t *map;
    uint64_t stats[ST_N];
    int tid, nthreads;
} batch;

enum { OP_RESOLVE, OP_GATHER, OP_REPLAY, OP_DEDUP, OP_APPEND };

static void *run_batch(void *arg)
{
    batch *b = (batch *)arg;
    const orc_source *s = b->s;
    for (int32_t i = b->tid; i < b->n; i += b->nthreads) {
        int32_t r = b->req_ids ? b->req_ids[i] : i;
        int st;
        if (r < 0 || r >= s->n_req) {
            st = ORC_E_ARG;
        } else if (b->op == OP_RESOLVE) {
            int32_t k = b->count ? b->count[i] : b->stride;
            st = orc_resolve_one(s, r, b->sel + (int64_t)i * b->stride, k, b->layer,
                                 b->loc + (int64_t)i * b->stride, b->fills + (int64_t)i * 2 * s->B,
                                 b->fill_count + i, b->stats);
        } else if (b->op == OP_GATHER) {
            int32_t k = b->count ? b->count[i] : b->stride;
            st = orc_gather_one(s, b->layer, r, b->loc_in + (int64_t)i * b->stride, k,
                                b->out + (int64_t)i * b->stride * s->R);
        } else if (b->op == OP_REPLAY) {
            st = orc_replay_one(s, b->layer, r, b->fills + (int64_t)i * 2 * s->B, b->fill_count[i]);
        } else if (b->op == OP_DEDUP) {
            int64_t qk = (int64_t)b->q * b->stride;
            st = orc_dedup_one(b->q, b->stride, b->sel + i * qk, b->union_rows + i * qk,
                               b->fill_count + i, b->map + i * qk);
        } else {
            st = orc_append_one(s, r, b->rows);
        }
        if (b->status)
            b->status[i] = st;
    }
    return NULL;
}

static void run_threads(batch *proto, int32_t nthreads, uint64_t *stats)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 64)
        nthreads = 64;
    if (proto->n < nthreads)
        nthreads = proto->n > 0 ? proto->n : 1;
    batch b[64];
    pthread_t th[64];
    for (int t = 0; t < nthreads; ++t) {
        b[t] = *proto;
        memset(b[t].stats, 0, sizeof(b[t].stats));
        b[t].tid = t;
        b[t].nthreads = nthreads;
    }
    for (int t = 1; t < nthreads; ++t)
        pthread_create(&th[t], NULL, run_batch, &b[t]);
    run_batch(&b[0]);
    for (int t = 1; t < nthreads; ++t)
        pthread_join(th[t], NULL);
    if (stats)
        for (int t = 0; t < nthreads; ++t)
            for (int i = 0; i < ST_N; ++i)
                stats[i] += b[t].stats[i];
}

/* sel, loc: [n][stride]; count: [n] or NULL (= stride); fills: [n][B][2] */
void orc_resolve(const orc_source *s, int32_t n, const int32_t *req_ids, const int32_t *sel,
                 const int32_t *count, int32_t stride, int32_t fill_layer, uint32_t *loc,
                 int32_t *fills, int32_t *fill_count, int32_t *status, uint64_t *stats,
                 int32_t nthreads)
{
    batch b = {0};
    b.s = s, b.op = OP_RESOLVE, b.n = n, b.req_ids = req_ids, b.sel = sel, b.count = count;
    b.stride = stride, b.layer = fill_layer, b.loc = loc, b.fills = fills;
    b.fill_count = fill_count, b.status = status;
    run_threads(&b, nthreads, stats);
}

/* out: [n][stride][R] */
void orc_gather(const orc_source *s, int32_t layer, int32_t n, const int32_t *req_ids,
                const uint32_t *loc, const int32_t *count, int32_t stride, uint8_t *out,
                int32_t *status, int32_t nthreads)
{
    batch b = {0};
    b.s = s, b.op = OP_GATHER, b.n = n, b.req_ids = req_ids, b.loc_in = loc, b.count = count;
    b.stride = stride, b.layer = layer, b.out = out, b.status = status;
    run_threads(&b, nthreads, NULL);
}

void orc_replay(const orc_source *s, int32_t layer, int32_t n, const int32_t *req_ids,
                const int32_t *fills, const int32_t *fill_count, int32_t *status, int32_t nthreads)
{
    batch b = {0};
    b.s = s, b.op = OP_REPLAY, b.n = n, b.req_ids = req_ids, b.layer = layer;
    b.fills = (int32_t *)fills, b.fill_count = (int32_t *)fill_count, b.status = status;
    run_threads(&b, nthreads, NULL);
}

/* sel, map: [n][q][k]; union_rows: [n][q*k]; union_count: [n] */
void orc_dedup(const orc_source *s, int32_t n, int32_t q, int32_t k, const int32_t *sel,
               int32_t *union_rows, int32_t *union_count, int32_t *map, int32_t nthreads)
{
    batch b = {0};
    b.s = s, b.op = OP_DEDUP, b.n = n, b.q = q, b.stride = k, b.sel = sel;
    b.union_rows = union_rows, b.fill_count = union_count, b.map = map;
    run_threads(&b, nthreads, NULL);
}

/* new_rows: [n_layers][n_req][R]; appends to the listed requests */
void orc_append(const orc_source *s, int32_t n, const int32_t *req_ids, const uint8_t *new_rows,
                int32_t *status, int32_t nthreads)
{
    batch b = {0};
    b.s = s, b.op = OP_APPEND, b.n = n, b.req_ids = req_ids, b.rows = new_rows, b.status = status;
    run_threads(&b, nthreads, NULL);
}
