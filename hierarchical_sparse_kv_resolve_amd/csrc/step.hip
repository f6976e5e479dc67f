// One launch that gathers the rows of one resolved selection and resolves
// the next selection ("Adaptive DHiSparse: Speculative Decoding over a
// Load-Adaptive KV Hierarchy", section "How it works", paragraphs
// "Resolution" and "Model-specific reuse").
//
// The resolve of the next selection (the next resolving layer's, or the next
// decode step's) needs only metadata -- lengths, page maps, tags, stamps --
// which the gather of the previous selection neither reads nor writes, and
// the gather needs only its own location words, selection and payload, which
// the resolve does not write (its append is deferred: the tail slot it
// replaces is written by the gather that follows it).  So the two run side
// by side in one grid, with no wait between two queues: workgroups of 1024
// threads take, by block index, the fill workers of the gather (first, so the
// host link starts at once), one resolve workgroup per request entry, the
// writers of deferred appends, then the resident tiles.  The gather parts
// are the code of the fused gather kernel run by 1024-thread workgroups (the
// tile and the fill job of a workgroup grow accordingly), sharing the
// dynamic LDS the resolve needs.
#include "gather_body.h"
#include "resolve_body.h"

namespace kvr {
namespace {

constexpr int NTS = 1024;
// Fill workers per launch (over all its layers) and 16-byte host loads in
// flight per lane, within the 128 registers a lane of a 1024-thread
// workgroup has (16 loads spill).  Measured on the long-context and GLM
// shapes (ms per step / us per step): 32 workers with 8 loads 2.939 / 221.1,
// 48 x 8 2.913 / 221.0, 64 x 8 2.908 / 220.7, 32 x 12 2.920 / 220.6,
// 48 x 12 2.915 / 220.8, 64 x 12 2.887-2.889 / 221.0-221.6, 96 x 12 2.922 /
// 238.3, 128 x 12 2.974 / 262.1: more workers than 64 take compute units the
// resident tiles and the resolve need (one 1024-thread workgroup fits a
// compute unit beside the resolve's LDS).
constexpr int kStepFillWorkers = 64;
constexpr int kStepFillUnroll = 12;

struct StepLayout {
    int32_t n_fill;         // fill workers: workers * nt
    int32_t workers;        // fill workers per target layer
    int32_t nt;             // target layers of the gather
    int32_t n_res;          // resolve workgroups: request entries of the resolve
    int32_t n_app;          // deferred-append writers: gather entries, or 0
    int32_t n_g;            // request entries of the gather
    int32_t tiles_per_req;  // fill jobs per request entry
    int32_t tiles_x;        // resident tiles per request entry
};

template <int EK, int EB>
__global__ __launch_bounds__(NTS) void step_kernel(ResolveArgs ra, GatherArgs ga, StepLayout lay)
{
    extern __shared__ __align__(16) uint8_t lds[];
    int64_t b = blockIdx.x;
    if (b < lay.n_fill) {
        fill_jobs<NTS, kStepFillUnroll>(ga, (int)(b / lay.workers), (int)(b % lay.workers),
                                        lay.workers, lay.n_g, lay.tiles_per_req,
                                        *reinterpret_cast<FillList *>(lds));
        return;
    }
    b -= lay.n_fill;
    if (b < lay.n_res) {
        resolve_body<EK, EB>(ra, (int)b, lds);
        return;
    }
    b -= lay.n_res;
    if (b < lay.n_app) {
        write_appended<NTS>(ga, (int)b, lay.nt);
        return;
    }
    b -= lay.n_app;
    const int64_t per_t = (int64_t)lay.tiles_x * lay.n_g;
    const int t = (int)(b / per_t);
    const int64_t rem = b - (int64_t)t * per_t;
    gather_tile<kGatherResident, NTS>(ga, (int)(rem % lay.tiles_x), (int)(rem / lay.tiles_x), t,
                                      reinterpret_cast<const uint8_t **>(lds));
}

using StepFn = void (*)(ResolveArgs, GatherArgs, StepLayout);

template <int EK>
StepFn step_pick_eb(int eb)
{
    switch (eb) {
    case 1: return &step_kernel<EK, 1>;
    case 2: return &step_kernel<EK, 2>;
    case 4: return &step_kernel<EK, 4>;
    default: return &step_kernel<EK, 8>;
    }
}

StepFn step_pick(const Shape &sh)
{
    const int eb = resolve_per_thread(sh.B);
    switch (resolve_per_thread(sh.sel_cap)) {
    case 1: return step_pick_eb<1>(eb);
    case 2: return step_pick_eb<2>(eb);
    case 4: return step_pick_eb<4>(eb);
    default: return step_pick_eb<8>(eb);
    }
}

}  // namespace

hipError_t prepare_step_kernel()
{
    const int most = (int)(kLdsPerCu - kStaticLdsBound);
    for (int ek = 1; ek <= 8; ek *= 2) {
        for (int eb = 1; eb <= 8; eb *= 2) {
            Shape sh{};
            sh.sel_cap = ek * NTS;
            sh.B = eb * NTS;
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(step_pick(sh)),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, most);
            if (e != hipSuccess)
                return e;
        }
    }
    return hipSuccess;
}

hipError_t launch_step(const kvr_ctx *c, const kvr_gather_call &g, const GatherTarget *targets,
                       int32_t nt, const kvr_resolve_call &r, hipStream_t s)
{
    ResolveArgs ra;
    const size_t res_lds = resolve_args(ra, c, r.n, r.req_ids, r.sel, r.sel_count, r.stride, r.loc,
                                        r.fills, r.fill_count, r.status, r.stats, 0,
                                        static_cast<const uint8_t *>(r.new_rows),
                                        r.append_status, r.append_pos);
    GatherArgs ga;
    ga.sh = c->shape;
    ga.ts = tile_for(c->shape, kGatherUnroll, NTS);
    ga.layers = c->layers_d;
    ga.req_ids = g.req_ids;
    ga.loc = g.loc;
    ga.count = g.count;
    ga.sel = g.sel;
    ga.stride = g.stride;
    ga.status = g.status;
    ga.n = g.n;
    const bool deferred = g.append_pos != nullptr && g.new_rows != nullptr;
    ga.new_rows = deferred ? static_cast<const uint8_t *>(g.new_rows) : nullptr;
    ga.append_pos = deferred ? g.append_pos : nullptr;
    for (int t = 0; t < nt; ++t) {
        ga.layer[t] = targets[t].layer;
        ga.out[t] = targets[t].out;
    }
    StepLayout lay;
    lay.nt = nt;
    lay.n_g = g.n;
    lay.n_res = r.n;
    lay.n_app = deferred ? g.n : 0;
    lay.tiles_x = (g.stride + ga.ts.rows - 1) / ga.ts.rows;
    // fill jobs as in the fused kernel: 1024 entries, fewer for small calls
    int ft = kFillTileMin;
    while (ft < kFillTile && (int64_t)ft * kFillJobsMin < (int64_t)g.n * g.stride)
        ft *= 2;
    ga.fill_tile = ft;
    lay.tiles_per_req = (g.stride + ft - 1) / ft;
    const int64_t jobs = (int64_t)g.n * lay.tiles_per_req;
    int64_t workers = (kStepFillWorkers + nt - 1) / nt;
    workers = workers < jobs ? workers : jobs;
    workers = workers > 0 ? workers : 1;
    lay.workers = (int32_t)workers;
    lay.n_fill = (int32_t)(workers * nt);
    const int64_t blocks = (int64_t)lay.n_fill + lay.n_res + lay.n_app + (int64_t)lay.tiles_x * g.n * nt;
    if (blocks > 0x7FFFFFFF)
        return hipErrorInvalidConfiguration;
    size_t lds = res_lds;
    lds = lds > sizeof(FillList) ? lds : sizeof(FillList);
    lds = lds > sizeof(const uint8_t *) * kMaxTileRows ? lds : sizeof(const uint8_t *) * kMaxTileRows;
    return launch(c, KVR_KERNEL_STEP, step_pick(c->shape), dim3((unsigned)blocks), dim3(NTS), lds,
                  s, ra, ga, lay);
}

}  // namespace kvr
