// Verification-block dedup: the q queries of a request share missing-row
// retrieval ("Adaptive DHiSparse: Speculative Decoding over a Load-Adaptive
// KV Hierarchy", section "How it works", paragraph "Speculative state"), so
// their selections are merged into one ascending union that is resolved
// once, plus a map from every query entry to its union index.
//
// One 1024-thread workgroup per request.  Every entry goes into an LDS hash
// once (insert if absent; each entry keeps its hash slot in a register), the
// distinct rows are compacted with wave ballots and sorted (each wave sorts a
// run in registers, runs are merged by rank), each row's union index is
// written back into its hash entry, and every entry reads its map value from
// its own hash slot.  Only the union is sorted; there are no searches.
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

__global__ __launch_bounds__(NT) void dedup_kernel(int32_t q, int32_t k, int32_t hs,
                                                   const int32_t *sel, int32_t *union_rows,
                                                   int32_t *union_count, int32_t *map)
{
    extern __shared__ __align__(16) uint8_t lds[];
    uint64_t *h = reinterpret_cast<uint64_t *>(lds);
    int32_t *list = reinterpret_cast<int32_t *>(h + hs);
    __shared__ int sCount;
    const int i = blockIdx.x;
    const int tid = threadIdx.x;
    const int n_all = q * k;
    const int32_t *in = sel + (int64_t)i * n_all;
    int32_t key[EQ];
#pragma unroll
    for (int e = 0; e < EQ; ++e) {
        const int t = e * NT + tid;
        key[e] = t < n_all ? in[t] : 0;
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
        base = __shfl(base, 0, kWave);
        if (own)
            list[base + ballot_rank(b)] = key[e];
    }
    __syncthreads();
    const int u = sCount;
    if (u > 0)
        block_merge_sort<NT, EQ, int32_t>(list, u, INT_MAX);

    // union rows out; each row's union index into its hash entry
    int32_t *uout = union_rows + (int64_t)i * n_all;
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

    int32_t *mout = map + (int64_t)i * n_all;
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

// LDS of one dedup workgroup: hash entries (load factor at most 2/3, at least
// one entry always empty) then the union list, as wide as the sort needs.
size_t dedup_layout(int n_all, int32_t *hs)
{
    const int cap = next_pow2(n_all > NT ? n_all : NT);
    int h = n_all * 3 / 2 + 64;
    h = (h + 63) / 64 * 64;
    *hs = h;
    return (size_t)h * 8 + (size_t)cap * 4;
}

}  // namespace

hipError_t prepare_dedup_kernel()
{
    int32_t hs;
    const size_t most = dedup_layout(kMaxUnion, &hs);
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&dedup_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)most);
}

hipError_t launch_dedup(const kvr_ctx *c, int32_t n, int32_t q, int32_t k, const int32_t *sel,
                        int32_t *union_rows, int32_t *union_count, int32_t *map, hipStream_t s)
{
    int32_t hs;
    const size_t lds = dedup_layout(q * k, &hs);
    return launch(c, KVR_KERNEL_DEDUP, dedup_kernel, dim3(n), dim3(NT), lds, s, q, k, hs, sel,
                  union_rows, union_count, map);
}

}  // namespace kvr
