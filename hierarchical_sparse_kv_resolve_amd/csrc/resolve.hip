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
//   sU    the distinct pending rows, ascending (wave-ballot compaction, a
//         register/shuffle bitonic sort, workgroup-scan dedup),
//   sSlot per pending row: its hot slot, or the rank of the miss,
//   sKey  the victims' (stamp << 32 | slot) keys in victim order.
// The hot-cache scan touches each of the B tags exactly once (a binary search
// of the tag among the sorted pending rows), so the work per call is bounded
// by B and by the selection size, never by the history length.
//
// Victims are the m smallest (stamp, slot) keys among the slots not hit in the
// call.  Instead of sorting all B keys, a radix select over stamp digits finds
// the threshold stamp tau; every candidate older than tau is a victim, and the
// youngest victims are the first candidates stamped tau in slot order.  Only
// the candidates older than tau are sorted, and only when their stamps differ.
#include <climits>

#include "block.h"
#include "kvr_internal.h"

namespace kvr {
namespace {

constexpr int NT = 1024;
constexpr int NW = NT / kWave;
constexpr int EK = kMaxSelCap / NT;    // selection entries per thread
constexpr int EB = kMaxHotSlots / NT;  // hot slots per thread
constexpr int32_t kNoSlot = INT_MAX;
constexpr int32_t kFilledBit = 1 << 30;
constexpr uint32_t kPending = 0xFFFFFFFEu;  // not a valid location word

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
    int32_t u_cap;  // LDS entries of sU and sSlot: max(NT, next_pow2(sel_cap))
    int32_t b_cap;  // LDS entries of sKey: max(NT, next_pow2(B))
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

// Digit of `rel` at bit `shift` (8-bit digits).
__device__ __forceinline__ int digit8(uint32_t rel, int shift) { return (rel >> shift) & 0xFF; }

__global__ __launch_bounds__(NT) void resolve_kernel(ResolveArgs a)
{
    extern __shared__ __align__(16) uint8_t lds[];
    uint64_t *sKey = reinterpret_cast<uint64_t *>(lds);
    int32_t *sU = reinterpret_cast<int32_t *>(sKey + a.b_cap);
    int32_t *sSlot = sU + a.u_cap;
    __shared__ int sScan[NW];
    __shared__ unsigned long long sScan64[NW];
    __shared__ unsigned long long sRed[NW];
    __shared__ uint32_t sRedU[2 * NW];
    __shared__ int sHist[256];
    __shared__ int sPick[2];
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

    // Step 1 and range check.  Entry e of this thread is selection j = e*NT+tid;
    // its row and location word stay in registers until the end.  Rows in the
    // tail window or in a ready complete page are found here; the others are
    // compacted into sU by wave ballots.
    int32_t pos[EK];
    uint32_t word[EK];
#pragma unroll
    for (int e = 0; e < EK; ++e) {
        pos[e] = -1;
        word[e] = 0;
    }
#pragma unroll
    for (int e = 0; e < EK; ++e) {
        const int j = e * NT + tid;
        if (e * NT >= k)
            break;  // uniform: no entry of this round exists
        bool pending = false;
        if (j < k) {
            const int32_t p = sel[j];
            pos[e] = p;
            if (p < 0 || p >= L) {
                sRangeErr = 1;
            } else if (p >= tail_lo) {
                word[e] = (uint32_t)(p % sh.T);
            } else {
                const int32_t phys = p < sh.full_rows ? pmap[p / sh.P] : -1;
                if (phys >= 0) {
                    word[e] = (1u << kPlaceShift) | (uint32_t)((int64_t)phys * sh.P + p % sh.P);
                } else {
                    word[e] = kPending;
                    pending = true;
                }
            }
        }
        const uint64_t m = __ballot(pending);
        int wbase = 0;
        if (lane_id() == 0 && m)
            wbase = atomicAdd(&sPend, __popcll(m));
        wbase = __shfl(wbase, 0, kWave);
        if (pending)
            sU[wbase + ballot_rank(m)] = pos[e];
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
    int nU = 0;
    if (n_pend > 0) {
        block_sort_lds<NT, int32_t>(sU, n_pend, INT_MAX);
        const int per = (n_pend + NT - 1) / NT;
        const int beg = tid * per;
        int32_t v[EK];
        int keep = 0, cnt = 0;
#pragma unroll
        for (int e = 0; e < EK; ++e) {
            const int idx = beg + e;
            if (e < per && idx < n_pend) {
                v[e] = sU[idx];
                if (idx == 0 || sU[idx - 1] != v[e]) {
                    keep |= 1 << e;
                    ++cnt;
                }
            }
        }
        int off = block_exclusive_scan<NT>(cnt, sScan, nU);
#pragma unroll
        for (int e = 0; e < EK; ++e)
            if (keep & (1 << e))
                sU[off++] = v[e];
        for (int t = tid; t < nU; t += NT)
            sSlot[t] = kNoSlot;
        __syncthreads();
    }

    // Step 2: each of the B tags is looked up once among the pending rows
    // (EB searches per thread run interleaved).  If two slots ever held one
    // row, the lower slot is the hit.
    int fidx[EB];
    uint32_t st[EB];
    {
        int32_t t[EB];
#pragma unroll
        for (int e = 0; e < EB; ++e) {
            const int b = e * NT + tid;
            t[e] = (b < sh.B) ? tag[b] : -1;
            st[e] = 0;
        }
        if (nU > 0) {
            lds_find_many<EB>(sU, nU, t, fidx);
#pragma unroll
            for (int e = 0; e < EB; ++e) {
                if (t[e] < 0)
                    fidx[e] = -1;
                if (fidx[e] >= 0)
                    atomicMin(&sSlot[fidx[e]], e * NT + tid);
            }
        } else {
#pragma unroll
            for (int e = 0; e < EB; ++e)
                fidx[e] = -1;
        }
    }
    __syncthreads();

    // Misses: rank them in ascending row order; check host copies.
    int m_total = 0;
    if (nU > 0) {
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
        __syncthreads();
    }
    if (nU > sh.B) {
        fail_request(a, i, k, KVR_E_CAPACITY);
        return;
    }
    if (sHostErr) {
        fail_request(a, i, k, KVR_E_NO_HOST_COPY);
        return;
    }

    // Step 3: victims = the m_total smallest (stamp, slot) among slots not hit.
    if (m_total > 0) {
        bool cand[EB];
        uint32_t lo = 0xFFFFFFFFu, hi = 0;
#pragma unroll
        for (int e = 0; e < EB; ++e) {
            const int b = e * NT + tid;
            cand[e] = b < sh.B && !(fidx[e] >= 0 && sSlot[fidx[e]] == b);
            if (cand[e]) {
                st[e] = stamp[b];
                lo = st[e] < lo ? st[e] : lo;
                hi = st[e] > hi ? st[e] : hi;
            }
        }
        lo = wave_min(lo);
        hi = wave_max(hi);
        if (lane_id() == 0) {
            sRedU[wave_id()] = lo;
            sRedU[NW + wave_id()] = hi;
        }
        __syncthreads();
        lo = 0xFFFFFFFFu;
        hi = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            lo = sRedU[w] < lo ? sRedU[w] : lo;
            hi = sRedU[NW + w] > hi ? sRedU[NW + w] : hi;
        }
        // Radix select of the threshold stamp over rel = stamp - lo, 8 bits at
        // a time from the highest digit that varies.
        const uint32_t span = hi - lo;
        int top = 0;
        while (top < 32 && (span >> top) > 0xFF)
            top += 8;
        uint32_t prefix = 0;      // digits chosen so far (above `shift + 8`)
        int m_rem = m_total;      // victims still to take at or above the prefix
        int c_lt = 0;             // candidates strictly older than the prefix bucket
        if (span > 0) {
            for (int shift = top; shift >= 0; shift -= 8) {
                for (int t = tid; t < 256; t += NT)
                    sHist[t] = 0;
                __syncthreads();
                const uint32_t hmask = (shift + 8 >= 32) ? 0u : (0xFFFFFFFFu << (shift + 8));
#pragma unroll
                for (int e = 0; e < EB; ++e) {
                    if (cand[e]) {
                        const uint32_t rel = st[e] - lo;
                        if ((rel & hmask) == prefix)
                            atomicAdd(&sHist[digit8(rel, shift)], 1);
                    }
                }
                __syncthreads();
                if (wave_id() == 0) {
                    // lane l holds bins 4l .. 4l+3
                    int c[4], sum = 0;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        c[q] = sHist[lane_id() * 4 + q];
                        sum += c[q];
                    }
                    const int incl = wave_inclusive_scan(sum);
                    int below = incl - sum;
                    // the bin where the running count first reaches m_rem
                    int pick = -1, pick_below = 0;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if (pick < 0 && below < m_rem && below + c[q] >= m_rem) {
                            pick = lane_id() * 4 + q;
                            pick_below = below;
                        }
                        below += c[q];
                    }
                    const uint64_t found = __ballot(pick >= 0);
                    const int src = __ffsll((unsigned long long)found) - 1;
                    pick = __shfl(pick, src, kWave);
                    pick_below = __shfl(pick_below, src, kWave);
                    if (lane_id() == 0) {
                        sPick[0] = pick;
                        sPick[1] = pick_below;
                    }
                }
                __syncthreads();
                prefix |= (uint32_t)sPick[0] << shift;
                m_rem -= sPick[1];
                c_lt += sPick[1];
                __syncthreads();
            }
        }
        const uint32_t tau = lo + prefix;

        // Ordered compaction in slot order: candidates older than tau become
        // sKey[0 .. c_lt) (then sorted), the first m_rem candidates stamped
        // tau fill sKey[c_lt .. m_total).  Slot b = e*NT + tid, so the order
        // is (e, tid); 16-bit fields pack the per-e counts of one thread.
        uint64_t lt_bits = 0, eq_bits = 0;
#pragma unroll
        for (int e = 0; e < EB; ++e) {
            if (cand[e]) {
                if (st[e] < tau)
                    lt_bits |= 1ull << (8 * e);
                else if (st[e] == tau)
                    eq_bits |= 1ull << (8 * e);
            }
        }
        // one scan of 8 byte-wide fields per kind would overflow (counts reach
        // NT), so scan 4 fields of 16 bits twice per kind
        int lt_rank[EB], eq_rank[EB];
        int lt_tot_before = 0, eq_tot_before = 0;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            uint64_t pl = 0, pe = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int e = half * 4 + q;
                pl |= (uint64_t)((lt_bits >> (8 * e)) & 1) << (16 * q);
                pe |= (uint64_t)((eq_bits >> (8 * e)) & 1) << (16 * q);
            }
            u64 tl, te;
            const u64 xl = block_exclusive_scan64<NT>(pl, sScan64, tl);
            const u64 xe = block_exclusive_scan64<NT>(pe, sScan64, te);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int e = half * 4 + q;
                lt_rank[e] = lt_tot_before + (int)((xl >> (16 * q)) & 0xFFFF);
                eq_rank[e] = eq_tot_before + (int)((xe >> (16 * q)) & 0xFFFF);
                lt_tot_before += (int)((tl >> (16 * q)) & 0xFFFF);
                eq_tot_before += (int)((te >> (16 * q)) & 0xFFFF);
            }
        }
#pragma unroll
        for (int e = 0; e < EB; ++e)
            if ((lt_bits >> (8 * e)) & 1)
                sKey[lt_rank[e]] = ((uint64_t)st[e] << 32) | (uint32_t)(e * NT + tid);
        __syncthreads();
        if (c_lt > 1) {
            // sort only when the older candidates carry different stamps
            uint32_t l2 = 0xFFFFFFFFu, h2 = 0;
            for (int t = tid; t < c_lt; t += NT) {
                const uint32_t sv = (uint32_t)(sKey[t] >> 32);
                l2 = sv < l2 ? sv : l2;
                h2 = sv > h2 ? sv : h2;
            }
            l2 = wave_min(l2);
            h2 = wave_max(h2);
            if (lane_id() == 0) {
                sRedU[wave_id()] = l2;
                sRedU[NW + wave_id()] = h2;
            }
            __syncthreads();
            uint32_t gl = 0xFFFFFFFFu, gh = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                gl = sRedU[w] < gl ? sRedU[w] : gl;
                gh = sRedU[NW + w] > gh ? sRedU[NW + w] : gh;
            }
            __syncthreads();
            if (gl != gh)  // uniform
                block_sort_lds<NT, uint64_t>(sKey, c_lt, ~0ull);
        }
        // the sort above uses sKey as its exchange buffer, so the youngest
        // victims are placed after it
#pragma unroll
        for (int e = 0; e < EB; ++e)
            if (((eq_bits >> (8 * e)) & 1) && eq_rank[e] < m_rem)
                sKey[c_lt + eq_rank[e]] = ((uint64_t)st[e] << 32) | (uint32_t)(e * NT + tid);
        __syncthreads();
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
            if ((uint32_t)slot >= (uint32_t)sh.B)
                continue;  // cannot happen: every rank below m_total has a victim
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
    {
        int32_t key[EK];
        int hidx[EK];
#pragma unroll
        for (int e = 0; e < EK; ++e)
            key[e] = (word[e] == kPending) ? pos[e] : INT_MIN;
        if (nU > 0)
            lds_find_many<EK>(sU, nU, key, hidx);
#pragma unroll
        for (int e = 0; e < EK; ++e) {
            const int j = e * NT + tid;
            if (j >= k)
                continue;
            uint32_t w = word[e];
            if (w == kPending) {
                const int32_t s = sSlot[hidx[e]];
                w = (2u << kPlaceShift) | (uint32_t)(s & kIndexMask);
                counts += (s & kFilledBit) ? (1ull << 48) : (1ull << 32);
            } else {
                counts += (w >> kPlaceShift) == 0 ? 1ull : (1ull << 16);
            }
            loc[j] = w;
        }
    }
    if (a.stats) {
        const uint64_t tot = block_sum<NT>((unsigned long long)counts, sRed);
        if (tid == 0) {
            unsigned long long *stp = reinterpret_cast<unsigned long long *>(a.stats);
            atomicAdd(&stp[0], 1ull);
            atomicAdd(&stp[1], tot & 0xFFFF);
            atomicAdd(&stp[2], (tot >> 16) & 0xFFFF);
            atomicAdd(&stp[3], (tot >> 32) & 0xFFFF);
            atomicAdd(&stp[4], (tot >> 48) & 0xFFFF);
            atomicAdd(&stp[5], (unsigned long long)m_total);
            if (a.count_host_bytes)
                atomicAdd(&stp[6], (unsigned long long)m_total * (unsigned long long)sh.R);
        }
    }
    if (tid == 0) {
        a.clock[r] = now;
        a.fill_count[i] = m_total;
        a.status[i] = KVR_OK;
    }
}

int lds_entries(int n) { return next_pow2(n > NT ? n : NT); }

}  // namespace

size_t resolve_lds_bytes(const Shape &sh)
{
    return (size_t)lds_entries(sh.B) * 8 + (size_t)lds_entries(sh.sel_cap) * 8;
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
    a.u_cap = lds_entries(c->shape.sel_cap);
    a.b_cap = lds_entries(c->shape.B);
    hipLaunchKernelGGL(resolve_kernel, dim3(n), dim3(NT), c->resolve_lds, s, a);
    return hipGetLastError();
}

}  // namespace kvr
