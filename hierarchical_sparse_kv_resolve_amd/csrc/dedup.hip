// Verification-block dedup: the q queries of a request share missing-row
// retrieval ("Adaptive DHiSparse: Speculative Decoding over a Load-Adaptive
// KV Hierarchy", section "How it works", paragraph "Speculative state"), so
// their selections are merged into one ascending union that is resolved
// once, plus a map from every query entry to its union index.
//
// One 1024-thread workgroup per request.  When every row lies in
// [0, history rows) and a bitmap over those rows fits in LDS, each entry sets
// its row's bit; a block scan of the words' popcounts gives each run of words
// its union offset, the set bits written out in order are the ascending
// union, and an entry's map value is the number of set bits below its row.
// Otherwise every entry goes into an LDS hash once (insert if absent; each
// entry keeps its hash slot in a register), the distinct rows are compacted
// with wave ballots and sorted (each wave sorts a run in registers, runs are
// merged by rank), each row's union index is written back into its hash
// entry, and every entry reads its map value from its own hash slot.
#include <climits>

#include "block.h"
#include "kvr_internal.h"

namespace kvr {
namespace {

constexpr int NT = 1024;
constexpr int EQ = kMaxUnion / NT;  // entries per thread
constexpr uint64_t kUsed = 1ull << 63;
constexpr int kRankShift = 40;     // union index in bits 40..62 of an entry

// Hash entries: 0 = empty, else kUsed | (union index << kRankShift) | key bits.
__device__ __forceinline__ int dslot(int32_t key, int hs)
{
    return (int)(((uint64_t)((uint32_t)key * 0x9E3779B1u) * (uint32_t)hs) >> 32);
}

__device__ __forceinline__ int dinsert(uint64_t *h, int hs, int32_t key, bool &fresh)
{
    const uint64_t mine = kUsed | (uint32_t)key;
    int idx = dslot(key, hs);
    while (true) {
        const uint64_t old =
            atomicCAS((unsigned long long *)&h[idx], 0ull, (unsigned long long)mine);
        if (old == 0 || (uint32_t)old == (uint32_t)key) {
            fresh = old == 0;
            return idx;
        }
        idx = idx + 1 == hs ? 0 : idx + 1;
    }
}

__device__ __forceinline__ int dfind(const uint64_t *h, int hs, int32_t key)
{
    int idx = dslot(key, hs);
    while (true) {
        const uint64_t v = h[idx];
        if (v == 0 || (uint32_t)v == (uint32_t)key)
            return v == 0 ? -1 : idx;
        idx = idx + 1 == hs ? 0 : idx + 1;
    }
}

__global__ __launch_bounds__(NT) void dedup_kernel(int32_t q, int32_t k, int32_t hs, int32_t bw,
                                                   const int32_t *sel, int32_t *union_rows,
                                                   int32_t *union_count, int32_t *map)
{
    extern __shared__ __align__(16) uint8_t lds[];
    uint64_t *h = reinterpret_cast<uint64_t *>(lds);
    int32_t *list = reinterpret_cast<int32_t *>(h + hs);
    // the bitmap path's arrays share the region: bm [bw] then run offsets [NT]
    uint32_t *bm = reinterpret_cast<uint32_t *>(lds);
    int32_t *sRun = reinterpret_cast<int32_t *>(bm + bw);
    __shared__ int sCount;
    __shared__ int sOut;
    __shared__ int sWave[NT / kWave];
    const int i = blockIdx.x;
    const int tid = threadIdx.x;
    const int n_all = q * k;
    const int32_t *in = sel + (int64_t)i * n_all;
    int32_t *uout = union_rows + (int64_t)i * n_all;
    int32_t *mout = map + (int64_t)i * n_all;
    int32_t key[EQ];
#pragma unroll
    for (int e = 0; e < EQ; ++e) {
        const int t = e * NT + tid;
        key[e] = t < n_all ? in[t] : 0;
    }

    if (bw > 0) {
        for (int x = tid; x < bw; x += NT)
            bm[x] = 0;
        if (tid == 0)
            sOut = 0;
        __syncthreads();
        const uint32_t bits = (uint32_t)bw * 32u;
        bool out = false;
#pragma unroll
        for (int e = 0; e < EQ; ++e) {
            if (e * NT + tid < n_all) {
                if ((uint32_t)key[e] < bits)
                    atomicOr(&bm[key[e] >> 5], 1u << (key[e] & 31));
                else
                    out = true;
            }
        }
        if (out)
            sOut = 1;
        __syncthreads();
        if (!sOut) {
            const int wpt = (bw + NT - 1) / NT;
            const int w0 = tid * wpt;
            int cnt = 0;
            for (int x = w0; x < w0 + wpt && x < bw; ++x)
                cnt += __popc(bm[x]);
            const int incl = wave_inclusive_scan(cnt);
            if (lane_id() == kWave - 1)
                sWave[wave_id()] = incl;
            __syncthreads();
            int base = 0, total = 0;
            for (int w = 0; w < NT / kWave; ++w) {
                base += w < wave_id() ? sWave[w] : 0;
                total += sWave[w];
            }
            base += incl - cnt;
            sRun[tid] = base;
            // the set bits of this thread's run, in order, are union entries
            // base, base + 1, ...
            int pos = base;
            for (int x = w0; x < w0 + wpt && x < bw; ++x) {
                uint32_t word = bm[x];
                while (word) {
                    const int b = __ffs(word) - 1;
                    uout[pos++] = x * 32 + b;
                    word &= word - 1;
                }
            }
            if (tid == 0)
                union_count[i] = total;
            __syncthreads();
#pragma unroll
            for (int e = 0; e < EQ; ++e) {
                const int t = e * NT + tid;
                if (t < n_all) {
                    const int row = key[e];
                    const int w = row >> 5;
                    const int c = w / wpt;
                    int rank = sRun[c] + __popc(bm[w] & ((1u << (row & 31)) - 1u));
                    for (int x = c * wpt; x < w; ++x)
                        rank += __popc(bm[x]);
                    mout[t] = rank;
                }
            }
            return;
        }
        __syncthreads();  // every thread is done with the bitmap before the hash
    }

    for (int x = tid; x < hs; x += NT)
        h[x] = 0;
    if (tid == 0)
        sCount = 0;
    __syncthreads();

    // every entry once into the hash; the inserting entry owns the row
    int slot[EQ];
    int owned = 0;
#pragma unroll
    for (int e = 0; e < EQ; ++e) {
        slot[e] = 0;
        if (e * NT + tid < n_all) {
            bool fresh;
            slot[e] = dinsert(h, hs, key[e], fresh);
            owned |= fresh ? (1 << e) : 0;
        }
    }
    // owners list their rows (wave-ballot compaction)
#pragma unroll
    for (int e = 0; e < EQ; ++e) {
        const bool own = (owned >> e) & 1;
        const uint64_t b = __ballot(own);
        int base = 0;
        if (lane_id() == 0 && b)
            base = atomicAdd(&sCount, __popcll(b));
        base = lane_value(base, 0);
        if (own)
            list[base + ballot_rank(b)] = key[e];
    }
    __syncthreads();
    const int u = sCount;
    if (u > 0)
        block_merge_sort<NT, EQ, int32_t>(list, u, INT_MAX);

    // union rows out; each row's union index into its hash entry
    for (int t = tid; t < u; t += NT) {
        const int32_t x = list[t];
        uout[t] = x;
        const int e = dfind(h, hs, x);
        if (e >= 0)
            h[e] |= (uint64_t)t << kRankShift;
    }
    if (tid == 0)
        union_count[i] = u;
    __syncthreads();

    uint64_t v[EQ];
#pragma unroll
    for (int e = 0; e < EQ; ++e)
        v[e] = h[slot[e]];
#pragma unroll
    for (int e = 0; e < EQ; ++e) {
        const int t = e * NT + tid;
        if (t < n_all)
            mout[t] = (int32_t)((v[e] & ~kUsed) >> kRankShift);
    }
}

constexpr size_t kDedupLdsMax = 160 * 1024 - 1024;  // beside the static counters

// LDS of one dedup workgroup: hash entries (load factor at most 2/3, at least
// one entry always empty) then the union list, as wide as the sort needs; the
// row bitmap (bw words over rows 0 .. host_rows-1, 0 when it does not fit)
// and its run offsets reuse the same region.
size_t dedup_layout(int n_all, int64_t host_rows, int32_t *hs, int32_t *bw)
{
    const int cap = next_pow2(n_all > NT ? n_all : NT);
    int h = n_all * 3 / 2 + 64;
    h = (h + 63) / 64 * 64;
    *hs = h;
    const size_t hash_bytes = (size_t)h * 8 + (size_t)cap * 4;
    const size_t words = (size_t)((host_rows + 31) / 32);
    const size_t bm_bytes = words * 4 + (size_t)NT * 4;
    *bw = 0;
    if (words > 0 && bm_bytes <= kDedupLdsMax) {
        *bw = (int32_t)words;
        return hash_bytes > bm_bytes ? hash_bytes : bm_bytes;
    }
    return hash_bytes;
}

}  // namespace

hipError_t prepare_dedup_kernel()
{
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&dedup_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)kDedupLdsMax);
}

hipError_t launch_dedup(const kvr_ctx *c, int32_t n, int32_t q, int32_t k, const int32_t *sel,
                        int32_t *union_rows, int32_t *union_count, int32_t *map, hipStream_t s)
{
    int32_t hs, bw;
    const size_t lds = dedup_layout(q * k, c->shape.host_rows, &hs, &bw);
    return launch(c, KVR_KERNEL_DEDUP, dedup_kernel, dim3(n), dim3(NT), lds, s, q, k, hs, bw, sel,
                  union_rows, union_count, map);
}

}  // namespace kvr
