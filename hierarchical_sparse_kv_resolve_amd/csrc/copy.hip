// Byte-moving kernels of the resolver besides the gather: the host refill of
// hot-cache slots (also the per-layer replay for shared indices with distinct
// payloads), the tail append, and small state kernels.  Host rows are read
// straight from pinned memory through its device mapping (zero copy over the
// host link), in tiles of whole rows like the gather's (sized for more loads
// in flight per lane, as host reads wait longer).
#include "kvr_internal.h"
#include "rows.h"

namespace kvr {
namespace {

constexpr int NT = kRowThreads;

// ------------------------------------------------------------------ refill

struct RefillArgs {
    Shape sh;
    TileShape ts;
    uint8_t *hot[kGatherLayersPerLaunch];
    const uint8_t *host[kGatherLayersPerLaunch];
    const int32_t *req_ids;
    const kvr_fill *fills;
    const int32_t *fill_count;
    int32_t *status;
};

// grid: (workers, layers).  Host rows arrive over the host link, so a few
// workers with many loads in flight keep it busy; a bounded grid leaves the
// other compute units free for kernels that run beside the fills (the next
// resolve, gathers of other layers).  Each worker strides over the
// (request, tile of fill rows) pairs and skips tiles beyond a request's fills.
__global__ __launch_bounds__(NT) void refill_kernel(RefillArgs a, int32_t n, int32_t tiles_per_req)
{
    __shared__ const uint8_t *sSrc[kMaxTileRows];
    __shared__ uint8_t *sDst[kMaxTileRows];
    const int t = blockIdx.y;
    const int R = a.sh.R;
    const int C = a.ts.chunks;
    for (int64_t job = blockIdx.x; job < (int64_t)n * tiles_per_req; job += gridDim.x) {
        const int i = (int)(job / tiles_per_req);
        const int tile = (int)(job - (int64_t)i * tiles_per_req);
        const int r = a.req_ids ? a.req_ids[i] : i;
        int fc = a.fill_count[i];
        fc = fc < 0 ? 0 : (fc > a.sh.B ? a.sh.B : fc);
        const int j0 = tile * a.ts.rows;
        if (j0 >= fc || r < 0 || r >= a.sh.n_req)
            continue;  // uniform across the workgroup
        const int nrows = min(a.ts.rows, fc - j0);
        __syncthreads();  // the previous tile's readers are done with sSrc/sDst
        if ((int)threadIdx.x < nrows) {
            const kvr_fill f = a.fills[(int64_t)i * a.sh.B + j0 + threadIdx.x];
            const bool ok =
                f.row >= 0 && (int64_t)f.row < a.sh.host_rows && f.slot >= 0 && f.slot < a.sh.B;
            sSrc[threadIdx.x] = ok ? a.host[t] + ((int64_t)r * a.sh.host_rows + f.row) * R : nullptr;
            sDst[threadIdx.x] = ok ? a.hot[t] + ((int64_t)r * a.sh.B + f.slot) * R : nullptr;
            if (!ok && a.status)
                a.status[i] = KVR_E_RANGE;
        }
        __syncthreads();
        const int total = nrows * C;
        for (int c0 = 0; c0 < total; c0 += NT * kUnroll) {
            u32x4 v[kUnroll];
            uint8_t *dsts[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int c = c0 + u * NT + threadIdx.x;
                dsts[u] = nullptr;
                if (c < total) {
                    const int row = (int)(((uint64_t)(uint32_t)c * a.ts.magic) >> 32);
                    const uint8_t *src = sSrc[row];
                    if (src) {
                        const int off = (c - row * C) * 16;
                        dsts[u] = sDst[row] + off;
                        load_chunk(v[u], src + off);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                if (dsts[u])
                    store_chunk(dsts[u], v[u]);
        }
    }
}

// ------------------------------------------------------------------ append

struct AppendArgs {
    Shape sh;
    const LayerPtrs *layers;
    int32_t *L;
    int32_t n;
    const int32_t *req_ids;
    const uint8_t *new_rows;  // [n_layers][n][R]
    int32_t *status;
};

__global__ __launch_bounds__(NT) void append_kernel(AppendArgs a)
{
    const int i = blockIdx.x;
    const int r = a.req_ids ? a.req_ids[i] : i;
    if (r < 0 || r >= a.sh.n_req) {
        if (threadIdx.x == 0 && a.status)
            a.status[i] = KVR_E_ARG;
        return;
    }
    const int32_t L = a.L[r];
    if (L < 0 || (int64_t)L >= a.sh.host_rows) {
        if (threadIdx.x == 0 && a.status)
            a.status[i] = KVR_E_CAPACITY;
        return;
    }
    const int C = a.sh.R / 16;
    const int per_layer = C * (a.sh.T > 0 ? 2 : 1);
    for (int c = threadIdx.x; c < per_layer * a.sh.n_layers; c += NT) {
        const int l = c / per_layer;
        const int e = c - l * per_layer;
        const int off = (e % C) * 16;
        const LayerPtrs lp = a.layers[l];
        u32x4 v;
        load_chunk(v, a.new_rows + ((int64_t)l * a.n + i) * a.sh.R + off);
        uint8_t *dst = (e < C) ? lp.host + ((int64_t)r * a.sh.host_rows + L) * a.sh.R + off
                               : lp.tail + ((int64_t)r * a.sh.T + L % a.sh.T) * a.sh.R + off;
        store_chunk(dst, v);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        a.L[r] = L + 1;
        if (a.status)
            a.status[i] = KVR_OK;
    }
}

// ------------------------------------------------------------------ small state kernels

__global__ void init_state_kernel(Shape sh, int32_t *L, int32_t *tag, uint32_t *stamp,
                                  uint32_t *clock)
{
    const int64_t n = (int64_t)sh.n_req * sh.B;
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n;
         e += (int64_t)gridDim.x * blockDim.x) {
        tag[e] = -1;
        stamp[e] = 0;
        if (e < sh.n_req) {
            L[e] = sh.H;
            clock[e] = 0;
        }
    }
}

__global__ void copy_loc_kernel(const uint32_t *src, uint32_t *dst, const int32_t *count,
                                int32_t stride)
{
    const int i = blockIdx.y;
    int cnt = count ? count[i] : stride;
    cnt = cnt < 0 ? 0 : (cnt > stride ? stride : cnt);
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j < cnt)
        dst[(int64_t)i * stride + j] = src[(int64_t)i * stride + j];
}

}  // namespace

bool tile_magic_exact(int32_t row_bytes)
{
    Shape sh{};
    sh.R = row_bytes;
    // the tiles of 256-thread workgroups (host and device unrolls) and of the
    // 1024-thread workgroups that gather beside a resolve
    const int shapes[3][2] = {{kUnroll, kRowThreads}, {kGatherUnroll, kRowThreads},
                              {kGatherUnroll, 1024}};
    for (const auto &u : shapes) {
        const TileShape ts = tile_for(sh, u[0], u[1]);
        for (uint32_t c = 0; c < (uint32_t)(ts.rows * ts.chunks); ++c)
            if ((uint32_t)(((uint64_t)c * ts.magic) >> 32) != c / (uint32_t)ts.chunks)
                return false;
    }
    return true;
}

// Workers per refill launch, over all its layers.
constexpr int kRefillWorkers = 128;

hipError_t launch_refill(const kvr_ctx *c, const int32_t *layers, int32_t n_layers, int32_t n,
                         const int32_t *req_ids, const kvr_fill *fills, const int32_t *fill_count,
                         int32_t *status, hipStream_t s)
{
    RefillArgs a;
    a.sh = c->shape;
    a.ts = tile_for(c->shape, kUnroll);
    a.req_ids = req_ids;
    a.fills = fills;
    a.fill_count = fill_count;
    a.status = status;
    const int tiles_per_req = (c->shape.B + a.ts.rows - 1) / a.ts.rows;
    for (int32_t t0 = 0; t0 < n_layers; t0 += kGatherLayersPerLaunch) {
        const int nt = n_layers - t0 < kGatherLayersPerLaunch ? n_layers - t0 : kGatherLayersPerLaunch;
        for (int t = 0; t < nt; ++t) {
            a.hot[t] = c->layers_h[layers[t0 + t]].hot;
            a.host[t] = c->layers_h[layers[t0 + t]].host;
        }
        const int64_t jobs = (int64_t)n * tiles_per_req;
        int64_t workers = (kRefillWorkers + nt - 1) / nt;
        workers = workers < jobs ? workers : jobs;
        dim3 grid((unsigned)(workers > 0 ? workers : 1), nt);
        hipError_t e = launch(c, KVR_KERNEL_REFILL, refill_kernel, grid, dim3(NT), 0, s, a, n,
                              tiles_per_req);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

hipError_t launch_append(const kvr_ctx *c, int32_t n, const int32_t *req_ids,
                         const uint8_t *new_rows, int32_t *status, hipStream_t s)
{
    AppendArgs a;
    a.sh = c->shape;
    a.layers = c->layers_d;
    a.L = c->L;
    a.n = n;
    a.req_ids = req_ids;
    a.new_rows = new_rows;
    a.status = status;
    return launch(c, KVR_KERNEL_APPEND, append_kernel, dim3(n), dim3(NT), 0, s, a);
}

hipError_t launch_init_state(const kvr_ctx *c, hipStream_t s)
{
    const int64_t n = (int64_t)c->shape.n_req * c->shape.B;
    int blocks = (int)((n + 255) / 256);
    blocks = blocks < 1 ? 1 : (blocks > 4096 ? 4096 : blocks);
    return launch(c, KVR_KERNEL_STATE, init_state_kernel, dim3(blocks), dim3(256), 0, s, c->shape,
                  c->L, c->tag, c->stamp, c->clock);
}

hipError_t launch_copy_loc(const kvr_ctx *c, int32_t n, const uint32_t *src, uint32_t *dst,
                           const int32_t *count, int32_t stride, hipStream_t s)
{
    dim3 grid((stride + 255) / 256, n);
    return launch(c, KVR_KERNEL_STATE, copy_loc_kernel, grid, dim3(256), 0, s, src, dst, count,
                  stride);
}

}  // namespace kvr
