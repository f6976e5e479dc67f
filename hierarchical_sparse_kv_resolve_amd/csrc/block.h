// Workgroup-level building blocks for 64-lane gfx950 wavefronts: ballot
// compaction, scans, reductions and an LDS bitonic sort.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvr {

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

// Lanes below this one whose predicate is set.
__device__ __forceinline__ int ballot_rank(uint64_t mask)
{
    return __popcll(mask & ((1ull << lane_id()) - 1ull));
}

__device__ __forceinline__ int wave_inclusive_scan(int x)
{
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        int y = __shfl_up(x, d, kWave);
        if (lane_id() >= d)
            x += y;
    }
    return x;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T x)
{
#pragma unroll
    for (int d = kWave / 2; d > 0; d >>= 1)
        x += __shfl_xor(x, d, kWave);
    return x;
}

// Exclusive prefix sum over the workgroup in thread order; `total` gets the
// sum over all threads.  `scratch` holds NT/64 ints of LDS.  Every thread of
// the workgroup must call it.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int *scratch, int &total)
{
    constexpr int NW = NT / kWave;
    int incl = wave_inclusive_scan(v);
    if (lane_id() == kWave - 1)
        scratch[wave_id()] = incl;
    __syncthreads();
    if (wave_id() == 0) {
        int w = lane_id() < NW ? scratch[lane_id()] : 0;
        w = wave_inclusive_scan(w);
        if (lane_id() < NW)
            scratch[lane_id()] = w;
    }
    __syncthreads();
    int base = wave_id() > 0 ? scratch[wave_id() - 1] : 0;
    total = scratch[NW - 1];
    __syncthreads();
    return base + incl - v;
}

// Sum over the workgroup, returned to every thread.  `scratch`: NT/64 values.
template <int NT, typename T>
__device__ __forceinline__ T block_sum(T v, T *scratch)
{
    constexpr int NW = NT / kWave;
    T w = wave_sum(v);
    if (lane_id() == 0)
        scratch[wave_id()] = w;
    __syncthreads();
    T total = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i)
        total += scratch[i];
    __syncthreads();
    return total;
}

// Ascending bitonic sort of s[0..n) in LDS, n a power of two.  Ends with a
// barrier, so the sorted array is visible to every thread.
template <int NT, typename K>
__device__ void bitonic_sort(K *s, int n)
{
    for (int k = 2; k <= n; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int t = threadIdx.x; t < (n >> 1); t += NT) {
                const int i = ((t & ~(j - 1)) << 1) | (t & (j - 1));
                const int p = i | j;
                K a = s[i], b = s[p];
                const bool up = (i & k) == 0;
                if (up ? (a > b) : (a < b)) {
                    s[i] = b;
                    s[p] = a;
                }
            }
            __syncthreads();
        }
    }
}

// Index of v in the ascending s[0..n), or -1.
__device__ __forceinline__ int lds_find(const int32_t *s, int n, int32_t v)
{
    int lo = 0, hi = n;
    while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if (s[mid] < v)
            lo = mid + 1;
        else
            hi = mid;
    }
    return (lo < n && s[lo] == v) ? lo : -1;
}

__host__ __device__ __forceinline__ int next_pow2(int x)
{
    int p = 1;
    while (p < x)
        p <<= 1;
    return p;
}

}  // namespace kvr
