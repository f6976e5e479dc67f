// Device code of the gather, the fill pass and the completion of deferred
// appends, shared by the gather kernels and the launch that gathers one
// selection while resolving the next.  Each function is written for a
// workgroup of NTH threads (256 in the gather kernels, 1024 beside the
// resolve) whose threads all take part in every barrier.
#pragma once

#include "kvr_internal.h"
#include "rows.h"

namespace kvr {
namespace {

// Fill workers per launch, over all its layers (at most one per job): enough
// jobs in flight to keep the host link busy, few enough that the resident
// gather running beside them keeps its compute units.
constexpr int kFillWorkers = 128;

struct GatherArgs {
    Shape sh;
    TileShape ts;
    const LayerPtrs *layers;  // device table
    int32_t layer[kGatherLayersPerLaunch];
    uint8_t *out[kGatherLayersPerLaunch];
    const int32_t *req_ids;
    const uint32_t *loc;
    const int32_t *count;
    const int32_t *sel;       // [n][stride] the resolved selection (fill mode)
    int32_t stride;
    int32_t *status;
    int32_t fill_tile;        // entries per fill job (at most kFillTile)
    int32_t n;                // request entries of the call
    const uint8_t *new_rows;  // deferred appends: [context layers][n][R], or null
    const int32_t *append_pos;  // [n] appended position per entry, -1 for none
};

// Source of a word in the all and resident modes (null: nothing to copy).
__device__ __forceinline__ const uint8_t *resident_src(const GatherArgs &a, const LayerPtrs &lp,
                                                       int r, uint32_t w, bool skip_fresh,
                                                       bool &bad)
{
    bad = false;
    if (w == KVR_LOC_INVALID)
        return nullptr;
    const uint32_t place = w >> kPlaceShift, idx = w & kIndexMask;
    if (place == KVR_PLACE_TAIL && idx < (uint32_t)a.sh.T)
        return lp.tail + ((int64_t)r * a.sh.T + idx) * a.sh.R;
    if (place == KVR_PLACE_PAGE && (int64_t)idx < a.sh.pool_rows)
        return lp.pool + (int64_t)idx * a.sh.R;
    if (place == KVR_PLACE_HOT && (idx & kSlotMask) < (uint32_t)a.sh.B) {
        if (skip_fresh && (idx & kFreshBit))
            return nullptr;
        return lp.hot + ((int64_t)r * a.sh.B + (idx & kSlotMask)) * a.sh.R;
    }
    bad = true;
    return nullptr;
}

// Tile x (kMaxTileRows or fewer whole rows) of request entry i into target t.
template <int MODE, int NTH>
__device__ __forceinline__ void gather_tile(const GatherArgs &a, int x, int i, int t,
                                            const uint8_t **sSrc)
{
    const int r = a.req_ids ? a.req_ids[i] : i;
    int cnt = a.count ? a.count[i] : a.stride;
    cnt = cnt < 0 ? 0 : (cnt > a.stride ? a.stride : cnt);
    const int j0 = x * a.ts.rows;
    if (j0 >= cnt || r < 0 || r >= a.sh.n_req)
        return;  // uniform across the workgroup
    const int nrows = min(a.ts.rows, cnt - j0);
    const LayerPtrs lp = a.layers[a.layer[t]];
    const int R = a.sh.R;
    uint8_t *dst = a.out[t] + ((int64_t)i * a.stride + j0) * R;
    if ((int)threadIdx.x < nrows) {
        const uint32_t w = a.loc[(int64_t)i * a.stride + j0 + threadIdx.x];
        bool bad;
        const uint8_t *src = resident_src(a, lp, r, w, MODE == kGatherResident, bad);
        if (a.append_pos && src && (w >> kPlaceShift) == KVR_PLACE_TAIL) {
            // the slot of a deferred append is being written in this launch:
            // its row comes from the new rows
            const int32_t apos = a.append_pos[i];
            if (apos >= 0 && (w & kIndexMask) == (uint32_t)(apos % a.sh.T))
                src = a.new_rows + ((int64_t)a.layer[t] * a.n + i) * R;
        }
        sSrc[threadIdx.x] = src;
        if (bad && a.status)
            a.status[i] = KVR_E_RANGE;
    }
    __syncthreads();
    const int C = a.ts.chunks;
    const int total = nrows * C;
    for (int c0 = 0; c0 < total; c0 += NTH * kGatherUnroll) {
        u32x4 v[kGatherUnroll];
        int rr[kGatherUnroll];
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u) {
            const int c = c0 + u * NTH + threadIdx.x;
            rr[u] = -1;
            if (c < total) {
                const int row = (int)(((uint64_t)(uint32_t)c * a.ts.magic) >> 32);
                const uint8_t *s = sSrc[row];
                if (s) {
                    rr[u] = row;
                    load_chunk(v[u], s + (c - row * C) * 16);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u) {
            if (rr[u] < 0)
                continue;
            const int c = c0 + u * NTH + threadIdx.x;
            store_chunk_nt(dst + (int64_t)c * 16, v[u]);
        }
    }
}

// Fill pass: a bounded set of workers (per layer) strides over (request, tile
// of fill_tile entries) jobs, so the host link is kept busy by a few workers
// with many loads in flight while the other compute units gather resident
// rows.  Each job compacts its fresh rows in LDS (their order does not matter:
// each row has its own two destinations), then streams them.  Jobs take 1024
// entries, or fewer when a call has fewer than 16 such jobs' worth of entries
// per layer (down to 16 entries), so that a small call still has 16 workers
// per layer drawing on the host link.
constexpr int kFillTile = 1024;
// 16-byte host loads in flight per lane in the copy loop: twice the refill's,
// so a worker keeps 64 KiB of host reads in flight and the last workers of a
// launch drain it faster (measured best of 8, 12, 16, 20 and 24 for the GLM
// shape; 20 and 24 are marginally better only at the verify and long-context
// shapes).  It costs occupancy (3 waves per SIMD), which the resident tiles of
// the fused launch do not miss.
constexpr int kFillUnroll = 16;
constexpr int kFillTileMin = 16;
constexpr int kFillJobsMin = 16;

struct FillList {
    int32_t row[kFillTile];   // host row (the selection entry's row)
    int32_t slot[kFillTile];  // hot-cache slot
    int32_t j[kFillTile];     // selection entry (output row)
    int32_t n;
};

template <int NTH, int UNROLL = kFillUnroll>
__device__ __forceinline__ void fill_jobs(const GatherArgs &a, int t, int worker, int workers,
                                          int32_t n, int32_t tiles_per_req, FillList &fl)
{
    constexpr int kFillPer = kFillTile / NTH;  // entries per thread of a full job
    const LayerPtrs lp = a.layers[a.layer[t]];
    const int R = a.sh.R;
    const int C = a.ts.chunks;
    // jobs in tile-major order: a worker's jobs (worker, worker + workers, ...)
    // spread over tiles, so that when counts fall short of the stride (a
    // verify union) the empty last tiles do not all land on the same workers
    for (int64_t job = worker; job < (int64_t)n * tiles_per_req; job += workers) {
        const int tile = (int)(job / n);
        const int i = (int)(job - (int64_t)tile * n);
        const int j0 = tile * a.fill_tile;
        const int r = a.req_ids ? a.req_ids[i] : i;
        int cnt = a.count ? a.count[i] : a.stride;
        cnt = cnt < 0 ? 0 : (cnt > a.stride ? a.stride : cnt);
        if (j0 >= cnt || r < 0 || r >= a.sh.n_req)
            continue;  // uniform across the workgroup
        const int j1 = min(j0 + a.fill_tile, cnt);
        // every location word and selection row of the job is loaded before
        // any is used (one memory round trip, not one per pass), and before
        // the barriers, which it overlaps
        uint32_t wv[kFillPer];
        int32_t rv[kFillPer];
#pragma unroll
        for (int u = 0; u < kFillPer; ++u) {
            const int j = j0 + u * NTH + (int)threadIdx.x;
            wv[u] = j < j1 ? a.loc[(int64_t)i * a.stride + j] : KVR_LOC_INVALID;
            rv[u] = j < j1 ? a.sel[(int64_t)i * a.stride + j] : -1;
        }
        __syncthreads();  // the previous job is done with the list
        if (threadIdx.x == 0)
            fl.n = 0;
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kFillPer; ++u) {
            const uint32_t w = wv[u];
            const uint32_t place = w >> kPlaceShift, idx = w & kIndexMask;
            if (w == KVR_LOC_INVALID || place != KVR_PLACE_HOT || !(idx & kFreshBit))
                continue;
            const uint32_t slot = idx & kSlotMask;
            const int32_t row = rv[u];
            if (slot < (uint32_t)a.sh.B && row >= 0 && (int64_t)row < a.sh.host_rows) {
                const int k = atomicAdd(&fl.n, 1);
                fl.row[k] = row;
                fl.slot[k] = (int32_t)slot;
                fl.j[k] = j0 + u * NTH + (int)threadIdx.x;
            } else if (a.status) {
                a.status[i] = KVR_E_RANGE;
            }
        }
        __syncthreads();
        const uint8_t *src = lp.host + (int64_t)r * a.sh.host_rows * R;
        uint8_t *hot = lp.hot + (int64_t)r * a.sh.B * R;
        uint8_t *out = a.out[t] + (int64_t)i * a.stride * R;
        const int total = fl.n * C;
        for (int c0 = 0; c0 < total; c0 += NTH * UNROLL) {
            u32x4 v[UNROLL];
            int rr[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int c = c0 + u * NTH + threadIdx.x;
                rr[u] = c < total ? c / C : -1;
                if (rr[u] >= 0)
                    load_chunk(v[u], src + (int64_t)fl.row[rr[u]] * R + (c - rr[u] * C) * 16);
            }
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                if (rr[u] < 0)
                    continue;
                const int off = (c0 + u * NTH + (int)threadIdx.x - rr[u] * C) * 16;
                store_chunk(hot + (int64_t)fl.slot[rr[u]] * R + off, v[u]);
                store_chunk_nt(out + (int64_t)fl.j[rr[u]] * R + off, v[u]);
            }
        }
    }
}

// The appended row of entry i of every target layer into its tail slot
// (deferred appends), by one workgroup.
template <int NTH>
__device__ __forceinline__ void write_appended(const GatherArgs &a, int i, int nt)
{
    const int32_t apos = a.append_pos[i];
    const int r = a.req_ids ? a.req_ids[i] : i;
    if (apos < 0 || a.sh.T <= 0 || r < 0 || r >= a.sh.n_req)
        return;
    const int R = a.sh.R;
    const int C = R / 16;
    for (int c = threadIdx.x; c < nt * C; c += NTH) {
        const int t = c / C;
        const int off = (c - t * C) * 16;
        const int l = a.layer[t];
        u32x4 v;
        load_chunk(v, a.new_rows + ((int64_t)l * a.n + i) * R + off);
        store_chunk(a.layers[l].tail + ((int64_t)r * a.sh.T + apos % a.sh.T) * R + off, v);
    }
}

}  // namespace
}  // namespace kvr
