// Speculative state ("Adaptive DHiSparse: Speculative Decoding over a
// Load-Adaptive KV Hierarchy", section "How it works", paragraph "Speculative
// state"): the drafter stores just the rows it can still see, in a ring, and
// the target layers hand a verification staging buffer out again only after
// the kernels that read it have finished.
//
// Drafter ring: per request a ring of C rows (slot = position mod C) of which
// the last W positions are visible; C - W extra slots let drafted rows that
// verification rejects be dropped again.  One workgroup per request moves its
// rows as 16-byte chunks; lengths and the high-water mark (highest position
// ever written + 1, which bounds how far a rollback may go) live on the
// device, so no call synchronises the host.
//
// Staging pool: buffer indices handed out round-robin; acquiring one makes
// the stream wait for that buffer's last release, which the consumer records
// on its own stream once it has read the buffer.
#include <new>
#include <vector>

#include "kvr_internal.h"

struct kvr_draft {
    int32_t n_req, W, C, R;
    uint8_t *ring;    // [n_req][C][R]
    int32_t *length;  // [n_req]
    int32_t *high;    // [n_req]
    int device;
};

struct kvr_staging {
    int32_t n;
    uint32_t next;
    std::vector<hipEvent_t> released;
    std::vector<char> pending;  // a release was recorded and not yet waited for
};

namespace kvr {
namespace {

constexpr int NT = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct DraftArgs {
    int32_t n_req, W, C, R;
    uint8_t *ring;
    int32_t *length;
    int32_t *high;
    const int32_t *req_ids;
    const uint8_t *rows;      // append: [n][a][R]
    int32_t a;
    const int32_t *keep;      // rollback: [n]
    uint8_t *out;             // window: [n][W][R]
    int32_t *visible;         // window: [n] or null
    int32_t *status;          // [n] or null
};

__device__ __forceinline__ int req_of(const DraftArgs &d, int i)
{
    const int r = d.req_ids ? d.req_ids[i] : i;
    return (r >= 0 && r < d.n_req) ? r : -1;
}

__global__ __launch_bounds__(NT) void draft_append_kernel(DraftArgs d)
{
    const int i = blockIdx.x;
    const int r = req_of(d, i);
    if (r < 0) {
        if (threadIdx.x == 0 && d.status)
            d.status[i] = KVR_E_ARG;
        return;
    }
    const int32_t len = d.length[r];
    const int C16 = d.R / 16;
    const int64_t total = (int64_t)d.a * C16;
    for (int64_t c = threadIdx.x; c < total; c += NT) {
        const int t = (int)(c / C16);
        const int off = (int)(c - (int64_t)t * C16) * 16;
        const int64_t slot = ((int64_t)len + t) % d.C;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(d.rows + ((int64_t)i * d.a + t) * d.R + off);
        *reinterpret_cast<u32x4 *>(d.ring + ((int64_t)r * d.C + slot) * d.R + off) = v;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const int32_t nl = len + d.a;
        d.length[r] = nl;
        if (nl > d.high[r])
            d.high[r] = nl;
        if (d.status)
            d.status[i] = KVR_OK;
    }
}

__global__ void draft_rollback_kernel(DraftArgs d, int32_t n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n)
        return;
    const int r = req_of(d, i);
    int st = KVR_OK;
    if (r < 0) {
        st = KVR_E_ARG;
    } else {
        const int32_t keep = d.keep[i];
        const int32_t lo = d.high[r] - (d.C - d.W);
        if (keep < (lo > 0 ? lo : 0) || keep > d.length[r])
            st = KVR_E_RANGE;
        else
            d.length[r] = keep;
    }
    if (d.status)
        d.status[i] = st;
}

__global__ __launch_bounds__(NT) void draft_window_kernel(DraftArgs d)
{
    const int i = blockIdx.x;
    const int r = req_of(d, i);
    if (r < 0) {
        if (threadIdx.x == 0 && d.status)
            d.status[i] = KVR_E_ARG;
        return;
    }
    const int32_t len = d.length[r];
    const int32_t first = len > d.W ? len - d.W : 0;
    const int vis = len - first;
    const int C16 = d.R / 16;
    const int64_t total = (int64_t)vis * C16;
    for (int64_t c = threadIdx.x; c < total; c += NT) {
        const int t = (int)(c / C16);
        const int off = (int)(c - (int64_t)t * C16) * 16;
        const int64_t slot = ((int64_t)first + t) % d.C;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(d.ring + ((int64_t)r * d.C + slot) * d.R + off);
        *reinterpret_cast<u32x4 *>(d.out + ((int64_t)i * d.W + t) * d.R + off) = v;
    }
    if (threadIdx.x == 0) {
        if (d.visible)
            d.visible[i] = vis;
        if (d.status)
            d.status[i] = KVR_OK;
    }
}

__global__ void draft_reset_kernel(int32_t *length, int32_t *high, int32_t n_req)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n_req) {
        length[i] = 0;
        high[i] = 0;
    }
}

DraftArgs draft_args(const kvr_draft *dr, const int32_t *req_ids)
{
    DraftArgs d{};
    d.n_req = dr->n_req;
    d.W = dr->W;
    d.C = dr->C;
    d.R = dr->R;
    d.ring = dr->ring;
    d.length = dr->length;
    d.high = dr->high;
    d.req_ids = req_ids;
    return d;
}

int draft_prologue(const kvr_draft *d, int32_t n, hipStream_t s)
{
    (void)s;
    if (!d)
        return api_fail(KVR_E_ARG, "null drafter ring");
    if (n < 0 || n > d->n_req)
        return api_fail(KVR_E_ARG, "request count %d outside [0, %d]", n, d->n_req);
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != d->device)
        return api_fail(KVR_E_ARG, "the current device is not the ring's device");
    return KVR_OK;
}

int launch_result(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        return api_fail(KVR_E_HIP, "%s: %s", what, hipGetErrorString(e));
    return api_ok();
}

}  // namespace
}  // namespace kvr

extern "C" {

int kvr_draft_create(int32_t n_req, int32_t window, int32_t capacity, int32_t row_bytes,
                     void *ring, int32_t *length, int32_t *high, kvr_draft **out)
{
    if (!out)
        return kvr::api_fail(KVR_E_ARG, "out is required");
    *out = nullptr;
    if (n_req < 1 || window < 1 || capacity < window || row_bytes < 16 || row_bytes % 16 ||
        (int64_t)capacity * row_bytes > ((int64_t)1 << 31))
        return kvr::api_fail(KVR_E_ARG, "bad drafter ring shape");
    if (!ring || !length || !high)
        return kvr::api_fail(KVR_E_ARG, "ring, length and high are required");
    kvr_draft *d = new (std::nothrow) kvr_draft();
    if (!d)
        return kvr::api_fail(KVR_E_ARG, "out of host memory");
    hipError_t e = hipGetDevice(&d->device);
    if (e != hipSuccess) {
        delete d;
        return kvr::api_fail(KVR_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    }
    d->n_req = n_req;
    d->W = window;
    d->C = capacity;
    d->R = row_bytes;
    d->ring = static_cast<uint8_t *>(ring);
    d->length = length;
    d->high = high;
    *out = d;
    return kvr::api_ok();
}

int kvr_draft_destroy(kvr_draft *d)
{
    delete d;
    return kvr::api_ok();
}

int kvr_draft_reset(kvr_draft *d, void *stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (int rc = kvr::draft_prologue(d, 0, s))
        return rc;
    hipLaunchKernelGGL(kvr::draft_reset_kernel, dim3((d->n_req + 255) / 256), dim3(256), 0, s,
                       d->length, d->high, d->n_req);
    return kvr::launch_result(hipGetLastError(), "drafter reset launch");
}

int kvr_draft_append(kvr_draft *d, int32_t n, const int32_t *req_ids, int32_t rows_each,
                     const void *rows, int32_t *status, void *stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (int rc = kvr::draft_prologue(d, n, s))
        return rc;
    // at most C rows, so one call never writes a slot twice
    if (rows_each < 0 || rows_each > d->C || (n > 0 && rows_each > 0 && !rows))
        return kvr::api_fail(KVR_E_ARG, "rows_each must be in [0, capacity] with rows given");
    if (n == 0 || rows_each == 0)
        return kvr::api_ok();
    kvr::DraftArgs a = kvr::draft_args(d, req_ids);
    a.rows = static_cast<const uint8_t *>(rows);
    a.a = rows_each;
    a.status = status;
    hipLaunchKernelGGL(kvr::draft_append_kernel, dim3(n), dim3(kvr::NT), 0, s, a);
    return kvr::launch_result(hipGetLastError(), "drafter append launch");
}

int kvr_draft_rollback(kvr_draft *d, int32_t n, const int32_t *req_ids, const int32_t *keep,
                       int32_t *status, void *stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (int rc = kvr::draft_prologue(d, n, s))
        return rc;
    if (n > 0 && !keep)
        return kvr::api_fail(KVR_E_ARG, "keep is required");
    if (n == 0)
        return kvr::api_ok();
    kvr::DraftArgs a = kvr::draft_args(d, req_ids);
    a.keep = keep;
    a.status = status;
    hipLaunchKernelGGL(kvr::draft_rollback_kernel, dim3((n + 255) / 256), dim3(256), 0, s, a, n);
    return kvr::launch_result(hipGetLastError(), "drafter rollback launch");
}

int kvr_draft_window(kvr_draft *d, int32_t n, const int32_t *req_ids, void *out,
                     int32_t *visible, int32_t *status, void *stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (int rc = kvr::draft_prologue(d, n, s))
        return rc;
    if (n > 0 && !out)
        return kvr::api_fail(KVR_E_ARG, "out is required");
    if (n == 0)
        return kvr::api_ok();
    kvr::DraftArgs a = kvr::draft_args(d, req_ids);
    a.out = static_cast<uint8_t *>(out);
    a.visible = visible;
    a.status = status;
    hipLaunchKernelGGL(kvr::draft_window_kernel, dim3(n), dim3(kvr::NT), 0, s, a);
    return kvr::launch_result(hipGetLastError(), "drafter window launch");
}

int kvr_staging_create(int32_t n_buffers, kvr_staging **out)
{
    if (!out)
        return kvr::api_fail(KVR_E_ARG, "out is required");
    *out = nullptr;
    if (n_buffers < 1 || n_buffers > 1024)
        return kvr::api_fail(KVR_E_ARG, "buffer count %d outside [1, 1024]", n_buffers);
    kvr_staging *p = new (std::nothrow) kvr_staging();
    if (!p)
        return kvr::api_fail(KVR_E_ARG, "out of host memory");
    p->n = n_buffers;
    p->next = 0;
    p->released.assign(n_buffers, nullptr);
    p->pending.assign(n_buffers, 0);
    for (int32_t b = 0; b < n_buffers; ++b) {
        hipError_t e = hipEventCreateWithFlags(&p->released[b], hipEventDisableTiming);
        if (e != hipSuccess) {
            for (int32_t c = 0; c < b; ++c)
                (void)hipEventDestroy(p->released[c]);
            delete p;
            return kvr::api_fail(KVR_E_HIP, "hipEventCreate: %s", hipGetErrorString(e));
        }
    }
    *out = p;
    return kvr::api_ok();
}

int kvr_staging_destroy(kvr_staging *p)
{
    if (!p)
        return kvr::api_ok();
    for (hipEvent_t e : p->released)
        (void)hipEventDestroy(e);
    delete p;
    return kvr::api_ok();
}

int kvr_staging_acquire(kvr_staging *p, void *stream, int32_t *index)
{
    if (!p || !index)
        return kvr::api_fail(KVR_E_ARG, "pool and index are required");
    const int32_t b = (int32_t)(p->next++ % (uint32_t)p->n);
    if (p->pending[b]) {
        hipError_t e = hipStreamWaitEvent(static_cast<hipStream_t>(stream), p->released[b], 0);
        if (e != hipSuccess)
            return kvr::api_fail(KVR_E_HIP, "hipStreamWaitEvent: %s", hipGetErrorString(e));
        p->pending[b] = 0;
    }
    *index = b;
    return kvr::api_ok();
}

int kvr_staging_release(kvr_staging *p, int32_t index, void *stream)
{
    if (!p || index < 0 || index >= p->n)
        return kvr::api_fail(KVR_E_ARG, "bad staging buffer index");
    hipError_t e = hipEventRecord(p->released[index], static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return kvr::api_fail(KVR_E_HIP, "hipEventRecord: %s", hipGetErrorString(e));
    p->pending[index] = 1;
    return kvr::api_ok();
}

}  // extern "C"
