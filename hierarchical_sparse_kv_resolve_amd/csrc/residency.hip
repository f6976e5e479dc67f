// Optional-pool residency ("Adaptive DHiSparse: Speculative Decoding over a
// Load-Adaptive KV Hierarchy", section "How it works", paragraphs "Memory
// split", "Resident-first admission" and "Reclamation and refill").
//
// Device side: pages of imported history leave and re-enter the optional
// pool.  One workgroup per listed page moves the page's P rows of every
// payload layer (16-byte chunks, several loads in flight per lane) and then
// updates the page's metadata, so the release or the publication is ordered
// after the copy by the end of the kernel; stream order orders it after the
// readers enqueued earlier.
//
// Host side: the policy that decides which pages move: an admission covers
// its deficit with whole requests' ready pages in reclaim order (or waits),
// and refill hands free physical pages back to the pages reclamation took,
// bounded, in round-robin over requests.
#include <map>
#include <new>
#include <set>
#include <vector>

#include "kvr_internal.h"

namespace kvr {
namespace {

constexpr int NT = 256;
constexpr int kPageUnroll = 4;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct PageArgs {
    Shape sh;
    const LayerPtrs *layers;  // device table
    int32_t *page_map;
    uint8_t *host_valid;
    const int32_t *req;
    const int32_t *page;
    const int32_t *phys;      // restore only
    int32_t *freed;           // reclaim only
    int32_t *status;
};

// Copies P rows (P * R contiguous bytes) of every layer from a page of one
// side to the other: pool page -> host rows (to_host) or back.
__device__ void move_page(const PageArgs &a, int32_t r, int32_t p, int32_t ph, bool to_host)
{
    const int64_t chunks = (int64_t)a.sh.P * a.sh.R / 16;
    const int64_t host_off = ((int64_t)r * a.sh.host_rows + (int64_t)p * a.sh.P) * a.sh.R;
    const int64_t pool_off = (int64_t)ph * a.sh.P * a.sh.R;
    for (int l = 0; l < a.sh.n_layers; ++l) {
        const LayerPtrs lp = a.layers[l];
        const uint8_t *src = to_host ? lp.pool + pool_off : lp.host + host_off;
        uint8_t *dst = to_host ? lp.host + host_off : lp.pool + pool_off;
        for (int64_t c0 = 0; c0 < chunks; c0 += (int64_t)NT * kPageUnroll) {
            u32x4 v[kPageUnroll];
#pragma unroll
            for (int u = 0; u < kPageUnroll; ++u) {
                const int64_t c = c0 + u * NT + threadIdx.x;
                if (c < chunks)
                    v[u] = *reinterpret_cast<const u32x4 *>(src + c * 16);
            }
#pragma unroll
            for (int u = 0; u < kPageUnroll; ++u) {
                const int64_t c = c0 + u * NT + threadIdx.x;
                if (c < chunks)
                    *reinterpret_cast<u32x4 *>(dst + c * 16) = v[u];
            }
        }
    }
}

// Whether an entry before i names the same page (or, with phys, the same
// physical page).  Every thread scans a share of the earlier entries.
__device__ bool earlier_repeat(const PageArgs &a, int i, int32_t r, int32_t p, bool with_phys,
                               int32_t ph)
{
    __shared__ int sRepeat;
    if (threadIdx.x == 0)
        sRepeat = 0;
    __syncthreads();
    bool hit = false;
    for (int j = threadIdx.x; j < i; j += NT)
        hit |= (a.req[j] == r && a.page[j] == p) || (with_phys && a.phys[j] == ph);
    if (hit)
        sRepeat = 1;  // every writer stores the same value
    __syncthreads();
    return sRepeat != 0;
}

__global__ __launch_bounds__(NT) void reclaim_kernel(PageArgs a)
{
    const int i = blockIdx.x;
    const int32_t r = a.req[i], p = a.page[i];
    const bool bad = r < 0 || r >= a.sh.n_req || p < 0 || p >= a.sh.n_pages;
    const bool repeat = earlier_repeat(a, i, r, p, false, 0);
    int32_t ph = -1;
    int st = bad ? KVR_E_ARG : KVR_OK;
    if (!bad && !repeat) {
        const int64_t e = (int64_t)r * a.sh.n_pages + p;
        ph = a.page_map[e];
        // a map entry outside the pool or on an incomplete page is corrupt
        if (ph >= 0 && ((int64_t)ph * a.sh.P >= a.sh.pool_rows || p >= a.sh.H / a.sh.P)) {
            st = KVR_E_STATE;
            ph = -1;
        }
        if (ph >= 0) {
            if (!a.host_valid[e])
                move_page(a, r, p, ph, true);
            __syncthreads();
            if (threadIdx.x == 0) {
                a.host_valid[e] = 1;
                a.page_map[e] = -1;
            }
        }
    }
    if (threadIdx.x == 0) {
        a.freed[i] = ph;
        if (a.status)
            a.status[i] = st;
    }
}

__global__ __launch_bounds__(NT) void restore_kernel(PageArgs a)
{
    const int i = blockIdx.x;
    const int32_t r = a.req[i], p = a.page[i], ph = a.phys[i];
    const int complete = a.sh.H / a.sh.P;
    int st = (r < 0 || r >= a.sh.n_req || p < 0 || p >= complete) ? KVR_E_ARG : KVR_OK;
    if (earlier_repeat(a, i, r, p, true, ph) && st == KVR_OK)
        st = KVR_E_ARG;
    const int64_t e = (int64_t)r * a.sh.n_pages + p;
    if (st == KVR_OK && (ph < 0 || (int64_t)ph * a.sh.P >= a.sh.pool_rows))
        st = KVR_E_RANGE;
    if (st == KVR_OK && a.page_map[e] >= 0)
        st = KVR_E_STATE;
    if (st == KVR_OK && !a.host_valid[e])
        st = KVR_E_NO_HOST_COPY;
    if (st == KVR_OK) {
        move_page(a, r, p, ph, false);
        __syncthreads();
        if (threadIdx.x == 0)
            a.page_map[e] = ph;
    }
    if (threadIdx.x == 0 && a.status)
        a.status[i] = st;
}

PageArgs page_args(const kvr_ctx *c, const int32_t *req, const int32_t *page)
{
    PageArgs a{};
    a.sh = c->shape;
    a.layers = c->layers_d;
    a.page_map = c->page_map;
    a.host_valid = c->host_valid;
    a.req = req;
    a.page = page;
    return a;
}

}  // namespace

hipError_t launch_reclaim(const kvr_ctx *c, int32_t n, const int32_t *req, const int32_t *page,
                          int32_t *freed, int32_t *status, hipStream_t s)
{
    PageArgs a = page_args(c, req, page);
    a.freed = freed;
    a.status = status;
    return launch(c, KVR_KERNEL_STATE, reclaim_kernel, dim3(n), dim3(NT), 0, s, a);
}

hipError_t launch_restore(const kvr_ctx *c, int32_t n, const int32_t *req, const int32_t *page,
                          const int32_t *phys, int32_t *status, hipStream_t s)
{
    PageArgs a = page_args(c, req, page);
    a.phys = phys;
    a.status = status;
    return launch(c, KVR_KERNEL_STATE, restore_kernel, dim3(n), dim3(NT), 0, s, a);
}

}  // namespace kvr

// ---------------------------------------------------------------- host policy

struct kvr_residency {
    int32_t n_req = 0;
    int32_t n_complete = 0;
    int64_t pool_pages = 0;
    std::vector<int32_t> ready;  // [n_req][n_complete]: physical page or -1
    std::set<int32_t> free;      // free physical pages, lowest first
    std::map<int32_t, std::vector<int32_t>> reserved;
    std::vector<std::set<int32_t>> reclaimed;  // per request: taken, not yet back
    int32_t next_handle = 0;
    int32_t cursor = 0;

    int32_t &at(int32_t r, int32_t p) { return ready[(size_t)r * n_complete + p]; }
};

extern "C" {

int kvr_residency_create(int32_t n_req, int32_t n_pages, int32_t n_complete, int64_t pool_pages,
                         const int32_t *page_map, kvr_residency **out)
{
    if (!out)
        return kvr::api_fail(KVR_E_ARG, "out is required");
    *out = nullptr;
    if (n_req < 1 || n_pages < 0 || n_complete < 0 || n_complete > n_pages || pool_pages < 0 ||
        pool_pages >= ((int64_t)1 << 31))
        return kvr::api_fail(KVR_E_ARG, "bad residency shape");
    if (n_complete > 0 && !page_map)
        return kvr::api_fail(KVR_E_ARG, "page_map is required");
    kvr_residency *res = new (std::nothrow) kvr_residency();
    if (!res)
        return kvr::api_fail(KVR_E_ARG, "out of host memory");
    res->n_req = n_req;
    res->n_complete = n_complete;
    res->pool_pages = pool_pages;
    std::vector<char> used(pool_pages, 0);
    try {
        res->ready.assign((size_t)n_req * n_complete, -1);
        res->reclaimed.assign(n_req, std::set<int32_t>());
        for (int32_t r = 0; r < n_req; ++r) {
            for (int32_t p = 0; p < n_complete; ++p) {
                const int32_t ph = page_map[(int64_t)r * n_pages + p];
                if (ph < -1 || ph >= pool_pages || (ph >= 0 && used[ph])) {
                    delete res;
                    return kvr::api_fail(KVR_E_ARG, "page_map names an invalid or repeated "
                                                    "physical page");
                }
                if (ph >= 0)
                    used[ph] = 1;
                res->at(r, p) = ph;
            }
        }
        for (int64_t ph = 0; ph < pool_pages; ++ph)
            if (!used[ph])
                res->free.insert((int32_t)ph);
    } catch (...) {
        delete res;
        return kvr::api_fail(KVR_E_ARG, "out of host memory");
    }
    *out = res;
    return kvr::api_ok();
}

int kvr_residency_destroy(kvr_residency *res)
{
    delete res;
    return kvr::api_ok();
}

int kvr_residency_admit(kvr_residency *res, int64_t need, int32_t n_order, const int32_t *order,
                        int32_t cap, int32_t *req_out, int32_t *page_out, int32_t *n_out,
                        int32_t *handle)
{
    if (!res || !n_out || !handle)
        return kvr::api_fail(KVR_E_ARG, "res, n_out and handle are required");
    *n_out = 0;
    *handle = -1;
    if (need < 0 || n_order < 0 || cap < 0 || (n_order > 0 && !order) ||
        (cap > 0 && (!req_out || !page_out)))
        return kvr::api_fail(KVR_E_ARG, "bad admission arguments");
    std::vector<char> seen(res->n_req, 0);
    for (int32_t i = 0; i < n_order; ++i) {
        if (order[i] < 0 || order[i] >= res->n_req || seen[order[i]])
            return kvr::api_fail(KVR_E_ARG, "reclaim order entry %d is out of range or repeated", i);
        seen[order[i]] = 1;
    }
    // the requests whose pages cover the deficit, in reclaim order
    int64_t deficit = need - (int64_t)res->free.size();
    std::vector<int32_t> taken;
    int64_t planned = 0;
    for (int32_t i = 0; i < n_order && deficit > 0; ++i) {
        int64_t cnt = 0;
        for (int32_t p = 0; p < res->n_complete; ++p)
            cnt += res->at(order[i], p) >= 0;
        if (cnt == 0)
            continue;
        taken.push_back(order[i]);
        planned += cnt;
        deficit -= cnt;
    }
    if (deficit > 0)
        return kvr::api_fail(KVR_E_CAPACITY, "the shortfall is larger than all optional pages");
    if (planned > cap)
        return kvr::api_fail(KVR_E_ARG, "the reclaim list needs %lld entries, cap is %d",
                             (long long)planned, cap);
    int32_t k = 0;
    for (int32_t r : taken) {
        for (int32_t p = 0; p < res->n_complete; ++p) {
            int32_t &ph = res->at(r, p);
            if (ph < 0)
                continue;
            res->free.insert(ph);
            ph = -1;
            res->reclaimed[r].insert(p);
            req_out[k] = r;
            page_out[k] = p;
            ++k;
        }
    }
    std::vector<int32_t> mine;
    mine.reserve((size_t)need);
    for (int64_t t = 0; t < need; ++t) {
        mine.push_back(*res->free.begin());
        res->free.erase(res->free.begin());
    }
    *n_out = k;
    *handle = res->next_handle++;
    res->reserved[*handle] = std::move(mine);
    return kvr::api_ok();
}

int kvr_residency_release(kvr_residency *res, int32_t handle)
{
    if (!res)
        return kvr::api_fail(KVR_E_ARG, "res is required");
    auto it = res->reserved.find(handle);
    if (it == res->reserved.end())
        return kvr::api_fail(KVR_E_ARG, "unknown admission handle %d", handle);
    for (int32_t ph : it->second)
        res->free.insert(ph);
    res->reserved.erase(it);
    return kvr::api_ok();
}

int kvr_residency_refill(kvr_residency *res, int32_t bound, int32_t cap, int32_t *req_out,
                         int32_t *page_out, int32_t *phys_out, int32_t *n_out)
{
    if (!res || !n_out)
        return kvr::api_fail(KVR_E_ARG, "res and n_out are required");
    *n_out = 0;
    if (bound < 0 || cap < 0 || (cap > 0 && (!req_out || !page_out || !phys_out)))
        return kvr::api_fail(KVR_E_ARG, "bad refill arguments");
    const int32_t limit = bound < cap ? bound : cap;
    int32_t k = 0, idle = 0, r = res->cursor;
    while (k < limit && !res->free.empty() && idle < res->n_req) {
        std::set<int32_t> &back = res->reclaimed[r];
        if (!back.empty()) {
            const int32_t p = *back.begin();
            back.erase(back.begin());
            const int32_t ph = *res->free.begin();
            res->free.erase(res->free.begin());
            res->at(r, p) = ph;
            req_out[k] = r;
            page_out[k] = p;
            phys_out[k] = ph;
            ++k;
            idle = 0;
            res->cursor = (r + 1) % res->n_req;
        } else {
            ++idle;
        }
        r = (r + 1) % res->n_req;
    }
    *n_out = k;
    return kvr::api_ok();
}

int kvr_residency_counts(const kvr_residency *res, int64_t *free_pages, int64_t *ready_pages,
                         int64_t *reserved_pages)
{
    if (!res)
        return kvr::api_fail(KVR_E_ARG, "res is required");
    int64_t ready = 0, reserved = 0;
    for (int32_t ph : res->ready)
        ready += ph >= 0;
    for (const auto &kv : res->reserved)
        reserved += (int64_t)kv.second.size();
    if (free_pages)
        *free_pages = (int64_t)res->free.size();
    if (ready_pages)
        *ready_pages = ready;
    if (reserved_pages)
        *reserved_pages = reserved;
    return kvr::api_ok();
}

}  // extern "C"
