// Gather of resolved rows into contiguous per-request buffers ("Adaptive
// DHiSparse: Speculative Decoding over a Load-Adaptive KV Hierarchy", section
// "How it works", paragraph "Model-specific reuse": attention consumes the
// rows named by the location vector).  out[layer][i][j] receives the R bytes
// that location word j of request i names in that layer's tail, optional
// pool or hot cache.  One launch serves every payload layer that shares the
// location vector (grid z = layer).
#include "kvr_internal.h"
#include "rows.h"

namespace kvr {
namespace {

constexpr int NT = kRowThreads;

struct GatherArgs {
    Shape sh;
    TileShape ts;
    const LayerPtrs *layers;  // device table
    int32_t layer[kGatherLayersPerLaunch];
    uint8_t *out[kGatherLayersPerLaunch];
    const int32_t *req_ids;
    const uint32_t *loc;
    const int32_t *count;
    int32_t stride;
    int32_t *status;
};

__global__ __launch_bounds__(NT) void gather_kernel(GatherArgs a)
{
    __shared__ const uint8_t *sSrc[kMaxTileRows];
    const int i = blockIdx.y;
    const int t = blockIdx.z;
    const int r = a.req_ids ? a.req_ids[i] : i;
    int cnt = a.count ? a.count[i] : a.stride;
    cnt = cnt < 0 ? 0 : (cnt > a.stride ? a.stride : cnt);
    const int j0 = blockIdx.x * a.ts.rows;
    if (j0 >= cnt || r < 0 || r >= a.sh.n_req)
        return;
    const int nrows = min(a.ts.rows, cnt - j0);
    const LayerPtrs lp = a.layers[a.layer[t]];
    const int R = a.sh.R;
    if ((int)threadIdx.x < nrows) {
        const uint32_t w = a.loc[(int64_t)i * a.stride + j0 + threadIdx.x];
        const uint32_t place = w >> kPlaceShift, idx = w & kIndexMask;
        const uint8_t *src = nullptr;
        if (w != KVR_LOC_INVALID) {
            if (place == KVR_PLACE_TAIL && idx < (uint32_t)a.sh.T)
                src = lp.tail + ((int64_t)r * a.sh.T + idx) * R;
            else if (place == KVR_PLACE_PAGE && (int64_t)idx < a.sh.pool_rows)
                src = lp.pool + (int64_t)idx * R;
            else if (place == KVR_PLACE_HOT && idx < (uint32_t)a.sh.B)
                src = lp.hot + ((int64_t)r * a.sh.B + idx) * R;
            else if (a.status)
                a.status[i] = KVR_E_RANGE;
        }
        sSrc[threadIdx.x] = src;
    }
    __syncthreads();
    uint8_t *dst = a.out[t] + ((int64_t)i * a.stride + j0) * R;
    const int C = a.ts.chunks;
    const int total = nrows * C;
    for (int c0 = 0; c0 < total; c0 += NT * kUnroll) {
        u32x4 v[kUnroll];
        const uint8_t *srcs[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int c = c0 + u * NT + threadIdx.x;
            srcs[u] = nullptr;
            if (c < total) {
                const int row = (int)(((uint64_t)(uint32_t)c * a.ts.magic) >> 32);
                const uint8_t *s = sSrc[row];
                if (s) {
                    srcs[u] = s;
                    load_chunk(v[u], s + (c - row * C) * 16);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int c = c0 + u * NT + threadIdx.x;
            if (srcs[u])
                store_chunk_nt(dst + (int64_t)c * 16, v[u]);
        }
    }
}

}  // namespace

hipError_t launch_gather(const kvr_ctx *c, const GatherTarget *targets, int32_t n_targets,
                         int32_t n, const int32_t *req_ids, const uint32_t *loc,
                         const int32_t *count, int32_t stride, int32_t *status, hipStream_t s)
{
    GatherArgs a;
    a.sh = c->shape;
    a.ts = tile_for(c->shape);
    a.layers = c->layers_d;
    a.req_ids = req_ids;
    a.loc = loc;
    a.count = count;
    a.stride = stride;
    a.status = status;
    for (int32_t t0 = 0; t0 < n_targets; t0 += kGatherLayersPerLaunch) {
        const int nt = n_targets - t0 < kGatherLayersPerLaunch ? n_targets - t0 : kGatherLayersPerLaunch;
        for (int t = 0; t < nt; ++t) {
            a.layer[t] = targets[t0 + t].layer;
            a.out[t] = targets[t0 + t].out;
        }
        dim3 grid((stride + a.ts.rows - 1) / a.ts.rows, n, nt);
        hipError_t e = launch(c, KVR_KERNEL_GATHER, gather_kernel, grid, dim3(NT), 0, s, a);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace kvr
