// Resolution of one selection per request against its KV source.
//
// Follows "Adaptive DHiSparse: Speculative Decoding over a Load-Adaptive KV
// Hierarchy", section "How it works", paragraph "Resolution": a selected row
// is taken from the tail or a ready optional-history page if it is there,
// else from the B-slot hot cache (with LRU stamps), else it is copied from
// pinned host memory into an LRU victim slot.  The host copy itself is done
// by the refill kernel (copy.hip) from the fill list written here.
//
// One workgroup of 1024 threads (16 waves) owns one request for the whole
// call, so every decision about that request's hot cache is made in one place
// and LDS holds all of it:
//   sU    the distinct pending rows, ascending (bitonic sort + ballot/scan
//         compaction),
//   sSlot per pending row: its hot slot, or the rank of the miss,
//   sKey  victim keys (stamp << 32 | slot) of the slots not hit in the call.
// The hot-cache scan touches each of the B tags exactly once (a binary search
// of the tag among the sorted pending rows), so the work per call is bounded
// by B and by the selection size, never by the history length.
#include <climits>

#include "block.h"
#include "kvr_internal.h"

namespace kvr {
namespace {

constexpr int NT = 1024;
constexpr int NW = NT / kWave;
constexpr int kPerThreadU = kMaxSelCap / NT;  // pending rows per thread in a compaction
constexpr int kPerThreadB = kMaxHotSlots / NT;
constexpr int32_t kNoSlot = INT_MAX;
constexpr int32_t kFilledBit = 1 << 30;

struct ResolveArgs {
    Shape sh;
    int32_t *L;
    const int32_t *page_map;
    const uint8_t *host_valid;
    int32_t *tag;
    uint32_t *stamp;
    uint32_t *clock;
    const int32_t *req_ids;
    const int32_t *sel;
    const int32_t *sel_count;
    int32_t stride;
    int32_t count_host_bytes;
    uint32_t *loc;
    kvr_fill *fills;
    int32_t *fill_count;
    int32_t *status;
    kvr_stats *stats;
    int32_t u_cap;  // power of two >= sel_cap
    int32_t b_cap;  // power of two >= B
};

__device__ __forceinline__ void fail_request(const ResolveArgs &a, int i, int k, int code)
{
    uint32_t *loc = a.loc + (int64_t)i * a.stride;
    for (int j = threadIdx.x; j < k; j += NT)
        loc[j] = KVR_LOC_INVALID;
    if (threadIdx.x == 0) {
        a.fill_count[i] = 0;
        a.status[i] = code;
        if (a.stats) {
            atomicAdd((unsigned long long *)&a.stats->calls, 1ull);
            atomicAdd((unsigned long long *)&a.stats->error, 1ull);
        }
    }
}

__global__ __launch_bounds__(NT) void resolve_kernel(ResolveArgs a)
{
    extern __shared__ __align__(16) uint8_t lds[];
    uint64_t *sKey = reinterpret_cast<uint64_t *>(lds);
    int32_t *sU = reinterpret_cast<int32_t *>(sKey + a.b_cap);
    int32_t *sSlot = sU + a.u_cap;
    __shared__ int sScan[NW];
    __shared__ unsigned long long sRed[NW];
    __shared__ int sPend;
    __shared__ int sRangeErr;
    __shared__ int sHostErr;

    const Shape &sh = a.sh;
    const int i = blockIdx.x;
    const int tid = threadIdx.x;
    const int r = a.req_ids ? a.req_ids[i] : i;
    int k = a.sel_count ? a.sel_count[i] : a.stride;
    if (r < 0 || r >= sh.n_req || k < 0 || k > a.stride) {
        fail_request(a, i, k < 0 ? 0 : (k > a.stride ? a.stride : k), KVR_E_ARG);
        return;
    }
    const int32_t *sel = a.sel + (int64_t)i * a.stride;
    uint32_t *loc = a.loc + (int64_t)i * a.stride;
    const int32_t L = a.L[r];
    const uint32_t clk = a.clock[r];
    const int32_t tail_lo = sh.T > 0 ? max(L - sh.T, 0) : L;
    const int32_t *pmap = a.page_map + (int64_t)r * sh.n_pages;
    const uint8_t *hvalid = a.host_valid + (int64_t)r * sh.n_pages;
    int32_t *tag = a.tag + (int64_t)r * sh.B;
    uint32_t *stamp = a.stamp + (int64_t)r * sh.B;

    if (tid == 0) {
        sPend = 0;
        sRangeErr = 0;
        sHostErr = 0;
    }
    __syncthreads();

    // Step 1 and range check: rows in the tail window or in a ready complete
    // page are found; the others are compacted into sU by wave ballots.
    for (int base = 0; base < k; base += NT) {
        const int j = base + tid;
        bool pending = false;
        int32_t pos = 0;
        if (j < k) {
            pos = sel[j];
            if (pos < 0 || pos >= L)
                sRangeErr = 1;
            else if (pos < tail_lo && !(pos < sh.full_rows && pmap[pos / sh.P] >= 0))
                pending = true;
        }
        const uint64_t m = __ballot(pending);
        int wbase = 0;
        if (lane_id() == 0 && m)
            wbase = atomicAdd(&sPend, __popcll(m));
        wbase = __shfl(wbase, 0, kWave);
        if (pending)
            sU[wbase + ballot_rank(m)] = pos;
    }
    __syncthreads();
    if (sRangeErr) {
        fail_request(a, i, k, KVR_E_RANGE);
        return;
    }
    if (clk == 0xFFFFFFFFu) {
        fail_request(a, i, k, KVR_E_STATE);
        return;
    }
    const uint32_t now = clk + 1;
    const int n_pend = sPend;

    // Distinct pending rows, ascending.
    const int np2 = next_pow2(n_pend > 0 ? n_pend : 1);
    for (int t = n_pend + tid; t < np2; t += NT)
        sU[t] = INT_MAX;
    __syncthreads();
    bitonic_sort<NT>(sU, np2);
    int nU;
    {
        const int per = (n_pend + NT - 1) / NT;
        const int beg = tid * per;
        int32_t v[kPerThreadU];
        int keep = 0, cnt = 0;
#pragma unroll
        for (int e = 0; e < kPerThreadU; ++e) {
            const int idx = beg + e;
            if (e < per && idx < n_pend) {
                v[e] = sU[idx];
                if (idx == 0 || sU[idx - 1] != v[e]) {
                    keep |= 1 << e;
                    ++cnt;
                }
            }
        }
        int total;
        int off = block_exclusive_scan<NT>(cnt, sScan, total);
#pragma unroll
        for (int e = 0; e < kPerThreadU; ++e)
            if (keep & (1 << e))
                sU[off++] = v[e];
        nU = total;
    }
    for (int t = tid; t < nU; t += NT)
        sSlot[t] = kNoSlot;
    __syncthreads();

    // Step 2: each of the B tags is looked up once among the pending rows.
    // If two slots ever held one row, the lower slot is the hit.
    int fidx[kPerThreadB];
#pragma unroll
    for (int e = 0; e < kPerThreadB; ++e) {
        const int b = tid + e * NT;
        fidx[e] = -1;
        if (b < sh.B && nU > 0) {
            const int32_t t = tag[b];
            if (t >= 0) {
                fidx[e] = lds_find(sU, nU, t);
                if (fidx[e] >= 0)
                    atomicMin(&sSlot[fidx[e]], b);
            }
        }
    }
    __syncthreads();

    // Misses: rank them in ascending row order; check host copies.
    int m_total;
    {
        const int per = (nU + NT - 1) / NT;
        const int beg = tid * per;
        int cnt = 0;
        for (int e = 0; e < per; ++e) {
            const int idx = beg + e;
            if (idx < nU && sSlot[idx] == kNoSlot) {
                ++cnt;
                const int32_t u = sU[idx];
                if (u < sh.H && !hvalid[u / sh.P])
                    sHostErr = 1;
            }
        }
        int off = block_exclusive_scan<NT>(cnt, sScan, m_total);
        for (int e = 0; e < per; ++e) {
            const int idx = beg + e;
            if (idx < nU && sSlot[idx] == kNoSlot)
                sSlot[idx] = -1 - off++;  // miss rank, negative
        }
    }
    __syncthreads();
    if (nU > sh.B) {
        fail_request(a, i, k, KVR_E_CAPACITY);
        return;
    }
    if (sHostErr) {
        fail_request(a, i, k, KVR_E_NO_HOST_COPY);
        return;
    }

    // Step 3: the m least recently used slots not hit in this call, ordered by
    // (stamp, slot), become the victims of the m misses in ascending row order.
    if (m_total > 0) {
#pragma unroll
        for (int e = 0; e < kPerThreadB; ++e) {
            const int b = tid + e * NT;
            if (b < a.b_cap) {
                uint64_t key = ~0ull;
                if (b < sh.B) {
                    const bool hit = fidx[e] >= 0 && sSlot[fidx[e]] == b;
                    if (!hit)
                        key = ((uint64_t)stamp[b] << 32) | (uint32_t)b;
                }
                sKey[b] = key;
            }
        }
        __syncthreads();
        bitonic_sort<NT>(sKey, a.b_cap);
    }

    // Commit: hits take the new stamp, victims the missing row and the stamp.
    kvr_fill *fills = a.fills + (int64_t)i * sh.B;
    for (int idx = tid; idx < nU; idx += NT) {
        const int32_t s = sSlot[idx];
        if (s >= 0) {
            stamp[s] = now;
        } else {
            const int rank = -1 - s;
            const int32_t slot = (int32_t)(uint32_t)sKey[rank];
            const int32_t u = sU[idx];
            tag[slot] = u;
            stamp[slot] = now;
            fills[rank] = kvr_fill{u, slot};
            sSlot[idx] = slot | kFilledBit;
        }
    }
    __syncthreads();

    // Location words in selection order; count entries by where they were found.
    uint64_t counts = 0;  // 16-bit fields: tail, page, hit, miss
    for (int j = tid; j < k; j += NT) {
        const int32_t pos = sel[j];
        uint32_t w;
        if (pos >= tail_lo) {
            w = (uint32_t)(pos % sh.T);
            counts += 1ull;
        } else if (pos < sh.full_rows && pmap[pos / sh.P] >= 0) {
            w = (1u << kPlaceShift) | (uint32_t)((int64_t)pmap[pos / sh.P] * sh.P + pos % sh.P);
            counts += 1ull << 16;
        } else {
            const int32_t s = sSlot[lds_find(sU, nU, pos)];
            w = (2u << kPlaceShift) | (uint32_t)(s & kIndexMask);
            counts += (s & kFilledBit) ? (1ull << 48) : (1ull << 32);
        }
        loc[j] = w;
    }
    if (a.stats) {
        const uint64_t tot = block_sum<NT>((unsigned long long)counts, sRed);
        if (tid == 0) {
            unsigned long long *st = reinterpret_cast<unsigned long long *>(a.stats);
            atomicAdd(&st[0], 1ull);
            atomicAdd(&st[1], tot & 0xFFFF);
            atomicAdd(&st[2], (tot >> 16) & 0xFFFF);
            atomicAdd(&st[3], (tot >> 32) & 0xFFFF);
            atomicAdd(&st[4], (tot >> 48) & 0xFFFF);
            atomicAdd(&st[5], (unsigned long long)m_total);
            if (a.count_host_bytes)
                atomicAdd(&st[6], (unsigned long long)m_total * (unsigned long long)sh.R);
        }
    }
    if (tid == 0) {
        a.clock[r] = now;
        a.fill_count[i] = m_total;
        a.status[i] = KVR_OK;
    }
}

}  // namespace

size_t resolve_lds_bytes(const Shape &sh)
{
    return (size_t)next_pow2(sh.B) * 8 + (size_t)next_pow2(sh.sel_cap) * 8;
}

// The limit is a per-kernel attribute shared by every context, so it is set
// to the largest dynamic LDS any valid shape can ask for.
hipError_t prepare_resolve_kernel()
{
    const size_t most = (size_t)kMaxHotSlots * 8 + (size_t)kMaxSelCap * 8;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&resolve_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)most);
}

hipError_t launch_resolve(const kvr_ctx *c, int32_t n, const int32_t *req_ids, const int32_t *sel,
                          const int32_t *sel_count, int32_t stride, uint32_t *loc, kvr_fill *fills,
                          int32_t *fill_count, int32_t *status, kvr_stats *stats,
                          int32_t count_host_bytes, hipStream_t s)
{
    ResolveArgs a;
    a.sh = c->shape;
    a.L = c->L;
    a.page_map = c->page_map;
    a.host_valid = c->host_valid;
    a.tag = c->tag;
    a.stamp = c->stamp;
    a.clock = c->clock;
    a.req_ids = req_ids;
    a.sel = sel;
    a.sel_count = sel_count;
    a.stride = stride;
    a.count_host_bytes = count_host_bytes;
    a.loc = loc;
    a.fills = fills;
    a.fill_count = fill_count;
    a.status = status;
    a.stats = stats;
    a.u_cap = next_pow2(c->shape.sel_cap);
    a.b_cap = next_pow2(c->shape.B);
    hipLaunchKernelGGL(resolve_kernel, dim3(n), dim3(NT), c->resolve_lds, s, a);
    return hipGetLastError();
}

}  // namespace kvr
