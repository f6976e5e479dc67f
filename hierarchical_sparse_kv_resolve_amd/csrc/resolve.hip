// Resolution of one selection per request against its KV source.
//
// Follows "Adaptive DHiSparse: Speculative Decoding over a Load-Adaptive KV
// Hierarchy", section "How it works", paragraph "Resolution": a selected row
// is taken from the tail or a ready optional-history page if it is there,
// else from the B-slot hot cache (with LRU stamps), else its host-store copy
// is brought into an LRU victim slot.  The host copy itself is done
// by the refill or fill kernels (copy.hip, gather.hip) from the fill list or
// the location words written here.  On request the same launch first appends
// each request's decoded row (the tail write of "Memory split").
//
// One workgroup of 1024 threads (16 waves) owns one request for the whole
// call, so every decision about that request's hot cache is made in one place
// and LDS holds all of it:
//   hkey/hval  an open-addressing hash of the distinct pending rows (insert
//              if absent dedups them; each thread keeps the entries of its
//              selection entries in registers); hval holds the row's hot
//              slot, the rank of the miss, or the filled slot,
//   bm         a bitmap over the request's rows marking the misses (when it
//              fits beside the hash): a miss's rank is the number of set
//              bits below it, from a block scan of the words' popcounts,
//   sKey       the victims' (stamp << 32 | slot) keys in victim order (and,
//              without the bitmap, first the misses to be sorted).
// The hot-cache scan looks each of the B tags up once in the hash, so the
// work per call is bounded by B and by the selection size, never by the
// history length.  Tags and stamps are loaded at kernel start so their
// latency hides behind step 1.
//
// Victims are the m smallest (stamp, slot) keys among the slots not hit in the
// call.  A radix select over stamp digits finds the threshold stamp tau (when
// all stamps lie within 64 values, by ballot counts per value); every
// candidate older than tau is a victim, and the youngest victims are the
// first candidates stamped tau in slot order (ordered compaction with wave
// ballots).  Only the candidates older than tau are sorted, and only when
// their stamps differ.  Misses take victims in ascending row order.  Up to
// 256 keys are put in order by counting ranks; more by sorting a run per wave
// in registers and merging the runs by rank (block_merge_sort).
#include <climits>

#include "block.h"
#include "kvr_internal.h"

#include "resolve_body.h"

namespace kvr {
namespace {

// One workgroup per request entry of the call.
template <int EK, int EB>
__global__ __launch_bounds__(NT) void resolve_kernel(ResolveArgs a)
{
    extern __shared__ __align__(16) uint8_t lds[];
    resolve_body<EK, EB>(a, blockIdx.x, lds);
}

}  // namespace

// Dynamic LDS layout of one resolve workgroup: victim keys then the hash
// (keys and values).  Returns 0 when the shape does not fit in LDS.
size_t resolve_lds_layout(const Shape &sh, int32_t *vc, int32_t *hs, int32_t *bw)
{
    const int m_cap = sh.B < sh.sel_cap ? sh.B : sh.sel_cap;
    const int v = next_pow2(m_cap > NT ? m_cap : NT);
    const size_t budget = kLdsPerCu - kStaticLdsBound;
    if ((size_t)v * 8 >= budget)
        return 0;
    size_t avail = budget - (size_t)v * 8;
    // keep the hash's load factor at most 0.8 and at least one empty entry
    const size_t h_min = (size_t)sh.sel_cap + (size_t)sh.sel_cap / 4 + 64;
    // the miss bitmap (and the scan's run offsets) when it leaves the hash
    // its minimum
    const size_t words = (size_t)((sh.host_rows + 31) / 32);
    const size_t bm_bytes = words * 4 + (size_t)NT * 4;
    size_t b = 0;
    if (words > 0 && avail >= bm_bytes + (h_min + 63) / 64 * 64 * 8) {
        b = words;
        avail -= bm_bytes;
    }
    size_t h = avail / 8;
    const size_t want = (size_t)4 * sh.sel_cap > 256 ? (size_t)4 * sh.sel_cap : 256;
    if (h > want)
        h = want;
    h = h / 64 * 64;
    if (h < h_min)
        return 0;
    *vc = v;
    *hs = (int32_t)h;
    *bw = (int32_t)b;
    return (size_t)v * 8 + h * 8 + (b > 0 ? bm_bytes : 0);
}

size_t resolve_lds_bytes(const Shape &sh)
{
    int32_t vc, hs, bw;
    return resolve_lds_layout(sh, &vc, &hs, &bw);
}

namespace {

using ResolveFn = void (*)(ResolveArgs);

template <int EK, int EB>
ResolveFn kernel_ptr()
{
    return &resolve_kernel<EK, EB>;
}


template <int EK>
ResolveFn pick_eb(int eb)
{
    switch (eb) {
    case 1: return kernel_ptr<EK, 1>();
    case 2: return kernel_ptr<EK, 2>();
    case 4: return kernel_ptr<EK, 4>();
    default: return kernel_ptr<EK, 8>();
    }
}

ResolveFn pick_kernel(const Shape &sh)
{
    const int eb = resolve_per_thread(sh.B);
    switch (resolve_per_thread(sh.sel_cap)) {
    case 1: return pick_eb<1>(eb);
    case 2: return pick_eb<2>(eb);
    case 4: return pick_eb<4>(eb);
    default: return pick_eb<8>(eb);
    }
}

}  // namespace

// The limit is a per-kernel attribute shared by every context, so it is set
// to the largest dynamic LDS any shape may use, on every instance.
hipError_t prepare_resolve_kernel()
{
    const int most = (int)(kLdsPerCu - kStaticLdsBound);
    for (int ek = 1; ek <= 8; ek *= 2) {
        for (int eb = 1; eb <= 8; eb *= 2) {
            Shape sh{};
            sh.sel_cap = ek * NT;
            sh.B = eb * NT;
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(pick_kernel(sh)),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, most);
            if (e != hipSuccess)
                return e;
        }
    }
    return hipSuccess;
}

hipError_t launch_resolve(const kvr_ctx *c, int32_t n, const int32_t *req_ids, const int32_t *sel,
                          const int32_t *sel_count, int32_t stride, uint32_t *loc, kvr_fill *fills,
                          int32_t *fill_count, int32_t *status, kvr_stats *stats,
                          int32_t count_host_bytes, const uint8_t *new_rows,
                          int32_t *append_status, int32_t *append_pos, hipStream_t s)
{
    ResolveArgs a;
    const size_t lds = resolve_args(a, c, n, req_ids, sel, sel_count, stride, loc, fills,
                                    fill_count, status, stats, count_host_bytes, new_rows,
                                    append_status, append_pos);
    return launch(c, KVR_KERNEL_RESOLVE, pick_kernel(c->shape), dim3(n), dim3(NT), lds, s, a);
}

}  // namespace kvr
