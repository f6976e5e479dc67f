// Verification-block dedup: the q queries of a request share missing-row
// retrieval ("Adaptive DHiSparse: Speculative Decoding over a Load-Adaptive
// KV Hierarchy", section "How it works", paragraph "Speculative state"), so
// their selections are merged into one ascending union that is resolved
// once, plus a map from every query entry to its union index.
//
// One 1024-thread workgroup per request: the q*k entries are sorted with the
// register/shuffle bitonic network (LDS only for strides 64..512), duplicates
// are dropped with a workgroup scan, and each entry finds its union index by
// binary search in LDS, several searches per thread interleaved.
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
    const int32_t *in = sel + (int64_t)i * n_all;
    for (int t = threadIdx.x; t < n_all; t += NT)
        s[t] = in[t];
    __syncthreads();
    if (n_all > 0)
        block_sort_lds<NT, int32_t>(s, n_all, INT_MAX);

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
    // eight interleaved searches per round
    for (int base = 0; base < n_all; base += 8 * NT) {
        int32_t key[8];
        int idx[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int t = base + e * NT + threadIdx.x;
            key[e] = t < n_all ? in[t] : INT_MIN;
        }
        lds_find_many<8>(s, u, key, idx);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int t = base + e * NT + threadIdx.x;
            if (t < n_all)
                mout[t] = idx[e];
        }
    }
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
    // the sort works on max(NT, next power of two >= q*k) entries
    const int n_all = q * k;
    const size_t lds = (size_t)next_pow2(n_all > NT ? n_all : NT) * 4;
    hipLaunchKernelGGL(dedup_kernel, dim3(n), dim3(NT), lds, s, q, k, sel, union_rows, union_count,
                       map);
    return hipGetLastError();
}

}  // namespace kvr
