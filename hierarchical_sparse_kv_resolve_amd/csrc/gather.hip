// Gather of resolved rows into contiguous per-request buffers ("Adaptive
// DHiSparse: Speculative Decoding over a Load-Adaptive KV Hierarchy", section
// "How it works", paragraph "Model-specific reuse": attention consumes the
// rows named by the location vector).  out[layer][i][j] receives the R bytes
// that location word j of request i names in that layer's tail, optional
// pool or hot cache.  One launch serves every payload layer that shares the
// location vector (grid z = layer).
//
// Modes (the first two of one kernel):
//   all       every valid word (fresh hot-cache rows read from their slots);
//   resident  every valid word except fresh hot-cache rows; it reads no slot
//             a fill of the same call writes, so it runs beside the fills;
//   fill      (fill_kernel) only fresh hot-cache rows: each is read once from
//             the layer's pinned host store (its row is the selection
//             entry's) and written both to the slot (the host fill of step 3
//             of "Resolution") and to the output, one pass over the host link
//             for both.  It reads the selection, not the tags, so a later
//             resolve of the same requests may already be rewriting tags.
//   fused     (fused_gather_kernel) fill and resident in one launch: the
//             first workgroups of the grid are fill workers, the rest gather
//             resident tiles, so the two share the chip without the
//             cross-queue waits that two concurrent launches need.
//             It may also complete deferred appends (the decoded row of
//             each entry, whose host copy and length a resolve launch has
//             already written): a few workgroups write each appended row
//             into its tail slot, and resident tiles read a tail word naming
//             that slot from the new rows instead, so no tile reads the slot
//             while it is written.  The row it replaces left the tail window
//             with the append, so no word of this launch names it.
#include "gather_body.h"

namespace kvr {
namespace {

constexpr int NT = kRowThreads;

template <int MODE>
__global__ __launch_bounds__(NT) void gather_kernel(GatherArgs a)
{
    __shared__ const uint8_t *sSrc[kMaxTileRows];
    gather_tile<MODE, NT>(a, blockIdx.x, blockIdx.y, blockIdx.z, sSrc);
}

__global__ __launch_bounds__(NT) void fill_kernel(GatherArgs a, int32_t n, int32_t tiles_per_req)
{
    __shared__ FillList fl;
    fill_jobs<NT>(a, blockIdx.y, blockIdx.x, gridDim.x, n, tiles_per_req, fl);
}

// Fill and resident gather in one 1-D grid: workgroups [0, nt * workers) are
// the fill workers of every target (so all of them start first), then, with
// deferred appends, one workgroup per request entry writes its appended rows,
// the rest are resident tiles, x fastest, then request entry, then target.
__global__ __launch_bounds__(NT) void fused_gather_kernel(GatherArgs a, int32_t n,
                                                          int32_t tiles_per_req, int32_t workers,
                                                          int32_t nt, int32_t tiles_x)
{
    __shared__ union {
        const uint8_t *src[kMaxTileRows];
        FillList fill;
    } sm;
    const int64_t b = blockIdx.x;
    const int64_t n_fill = (int64_t)workers * nt;
    const int64_t n_app = a.append_pos ? n : 0;
    if (b < n_fill) {
        fill_jobs<NT>(a, (int)(b / workers), (int)(b % workers), workers, n, tiles_per_req, sm.fill);
    } else if (b < n_fill + n_app) {
        write_appended<NT>(a, (int)(b - n_fill), nt);
    } else {
        const int64_t g = b - n_fill - n_app;
        const int64_t per_t = (int64_t)tiles_x * n;
        const int t = (int)(g / per_t);
        const int64_t rem = g - (int64_t)t * per_t;
        gather_tile<kGatherResident, NT>(a, (int)(rem % tiles_x), (int)(rem / tiles_x), t, sm.src);
    }
}

}  // namespace

hipError_t launch_gather(const kvr_ctx *c, int32_t mode, const GatherTarget *targets,
                         int32_t n_targets, int32_t n, const int32_t *req_ids, const uint32_t *loc,
                         const int32_t *sel, const int32_t *count, int32_t stride, int32_t *status,
                         hipStream_t s, const uint8_t *new_rows, const int32_t *append_pos)
{
    GatherArgs a;
    a.sh = c->shape;
    a.ts = tile_for(c->shape, kGatherUnroll);
    a.layers = c->layers_d;
    a.req_ids = req_ids;
    a.loc = loc;
    a.count = count;
    a.sel = sel;
    a.stride = stride;
    a.status = status;
    a.n = n;
    const bool deferred = mode == kGatherFused && append_pos != nullptr && new_rows != nullptr;
    a.new_rows = deferred ? new_rows : nullptr;
    a.append_pos = deferred ? append_pos : nullptr;
    for (int32_t t0 = 0; t0 < n_targets; t0 += kGatherLayersPerLaunch) {
        const int nt = n_targets - t0 < kGatherLayersPerLaunch ? n_targets - t0 : kGatherLayersPerLaunch;
        for (int t = 0; t < nt; ++t) {
            a.layer[t] = targets[t0 + t].layer;
            a.out[t] = targets[t0 + t].out;
        }
        const int tiles_x = (stride + a.ts.rows - 1) / a.ts.rows;
        dim3 grid(tiles_x, n, nt);
        // fill workers per target: at most one per job
        int ft = kFillTileMin;
        while (ft < kFillTile && (int64_t)ft * kFillJobsMin < (int64_t)n * stride)
            ft *= 2;
        a.fill_tile = ft;
        const int tiles_per_req = (stride + ft - 1) / ft;
        const int64_t jobs = (int64_t)n * tiles_per_req;
        int64_t workers = (kFillWorkers + nt - 1) / nt;
        workers = workers < jobs ? workers : jobs;
        workers = workers > 0 ? workers : 1;
        hipError_t e;
        if (mode == kGatherFill) {
            dim3 fgrid((unsigned)workers, nt);
            e = launch(c, KVR_KERNEL_REFILL, fill_kernel, fgrid, dim3(NT), 0, s, a, n, tiles_per_req);
        } else if (mode == kGatherFused) {
            const int64_t blocks = workers * nt + (deferred ? n : 0) + (int64_t)tiles_x * n * nt;
            if (blocks > 0x7FFFFFFF)
                return hipErrorInvalidConfiguration;
            e = launch(c, KVR_KERNEL_FUSED, fused_gather_kernel, dim3((unsigned)blocks), dim3(NT), 0,
                       s, a, n, tiles_per_req, (int32_t)workers, (int32_t)nt, (int32_t)tiles_x);
        } else if (mode == kGatherResident)
            e = launch(c, KVR_KERNEL_GATHER, gather_kernel<kGatherResident>, grid, dim3(NT), 0, s, a);
        else
            e = launch(c, KVR_KERNEL_GATHER, gather_kernel<kGatherAll>, grid, dim3(NT), 0, s, a);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace kvr
