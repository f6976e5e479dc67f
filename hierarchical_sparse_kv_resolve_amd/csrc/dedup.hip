// Verification-block dedup: the q queries of a request share missing-row
// retrieval ("Adaptive DHiSparse: Speculative Decoding over a Load-Adaptive
// KV Hierarchy", section "How it works", paragraph "Speculative state"), so
// their selections are merged into one ascending union that is resolved
// once, plus a map from every query entry to its union index.
//
// One 1024-thread workgroup per request: the q*k entries are sorted in LDS
// (bitonic), duplicates are dropped with a workgroup scan, and each entry
// finds its union index by binary search in LDS.
#include <climits>

#include "block.h"
#include "kvr_internal.h"

namespace kvr {
namespace {

constexpr int NT = 1024;
constexpr int NW = NT / kWave;
constexpr int kPerThread = kMaxUnion / NT;

__global__ __launch_bounds__(NT) void dedup_kernel(int32_t q, int32_t k, const int32_t *sel,
                                                   int32_t *union_rows, int32_t *union_count,
                                                   int32_t *map)
{
    extern __shared__ __align__(16) uint8_t lds[];
    int32_t *s = reinterpret_cast<int32_t *>(lds);
    __shared__ int sScan[NW];
    const int i = blockIdx.x;
    const int n_all = q * k;
    const int np2 = next_pow2(n_all > 0 ? n_all : 1);
    const int32_t *in = sel + (int64_t)i * n_all;
    for (int t = threadIdx.x; t < np2; t += NT)
        s[t] = t < n_all ? in[t] : INT_MAX;
    __syncthreads();
    bitonic_sort<NT>(s, np2);

    const int per = (n_all + NT - 1) / NT;
    const int beg = threadIdx.x * per;
    int32_t v[kPerThread];
    int keep = 0, cnt = 0;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
        const int idx = beg + e;
        if (e < per && idx < n_all) {
            v[e] = s[idx];
            if (idx == 0 || s[idx - 1] != v[e]) {
                keep |= 1 << e;
                ++cnt;
            }
        }
    }
    int u;
    int off = block_exclusive_scan<NT>(cnt, sScan, u);
    int32_t *uout = union_rows + (int64_t)i * n_all;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
        if (keep & (1 << e)) {
            s[off] = v[e];
            uout[off] = v[e];
            ++off;
        }
    }
    __syncthreads();
    if (threadIdx.x == 0)
        union_count[i] = u;
    int32_t *mout = map + (int64_t)i * n_all;
    for (int t = threadIdx.x; t < n_all; t += NT)
        mout[t] = lds_find(s, u, in[t]);
}

}  // namespace

hipError_t prepare_dedup_kernel()
{
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&dedup_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, kMaxUnion * 4);
}

hipError_t launch_dedup(int32_t n, int32_t q, int32_t k, const int32_t *sel, int32_t *union_rows,
                        int32_t *union_count, int32_t *map, hipStream_t s)
{
    const size_t lds = (size_t)next_pow2(q * k > 0 ? q * k : 1) * 4;
    hipLaunchKernelGGL(dedup_kernel, dim3(n), dim3(NT), lds, s, q, k, sel, union_rows, union_count,
                       map);
    return hipGetLastError();
}

}  // namespace kvr
