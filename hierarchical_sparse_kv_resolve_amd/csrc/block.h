// Workgroup-level building blocks for 64-lane gfx950 wavefronts: ballot
// compaction, wave scans and reductions, an LDS bitonic sort and a register
// sort of wave runs merged by rank.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvr {

constexpr int kWave = 64;

__host__ __device__ __forceinline__ int next_pow2(int x)
{
    int p = 1;
    while (p < x)
        p <<= 1;
    return p;
}

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

template <typename T>
__device__ __forceinline__ T wave_min(T x)
{
#pragma unroll
    for (int d = kWave / 2; d > 0; d >>= 1) {
        T y = __shfl_xor(x, d, kWave);
        x = y < x ? y : x;
    }
    return x;
}

template <typename T>
__device__ __forceinline__ T wave_max(T x)
{
#pragma unroll
    for (int d = kWave / 2; d > 0; d >>= 1) {
        T y = __shfl_xor(x, d, kWave);
        x = y > x ? y : x;
    }
    return x;
}

// ---------------------------------------------------------------------------
// Wave-sort + merge-by-rank: s[0..n) ascending in LDS (ties keep run order,
// so duplicate keys land in distinct places).  Each 64-lane wave sorts its
// own run of 64*E keys in registers (bitonic network: strides of 64 and more
// inside a thread, smaller ones through cross-lane shuffles, no barriers);
// then every key's final place is its position in its run plus, for every
// other run, the number of keys of that run that go before it (binary
// searches, all of a thread's searches interleaved).  `pad` must sort after
// every real key; keys at or beyond n are not written back.

template <int E, typename K>
__device__ __forceinline__ void wave_sort_run(K (&v)[E])
{
    constexpr int N = kWave * E;
    const int lane = lane_id();
#pragma unroll
    for (int k = 2; k <= N; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            if (j >= kWave) {
                const int je = j / kWave;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    if ((e & je) == 0) {
                        const int idx = e * kWave + lane;
                        const bool up = (idx & k) == 0;
                        K a = v[e], b = v[e | je];
                        if (up ? (a > b) : (a < b)) {
                            v[e] = b;
                            v[e | je] = a;
                        }
                    }
                }
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int idx = e * kWave + lane;
                    const K o = __shfl_xor(v[e], j, kWave);
                    const bool keep_min = ((idx & j) == 0) == ((idx & k) == 0);
                    v[e] = keep_min ? (o < v[e] ? o : v[e]) : (o > v[e] ? o : v[e]);
                }
            }
        }
    }
}

template <int NT, int E, typename K>
__device__ void block_merge_sort_e(K *s, int n, K pad)
{
    constexpr int NW = NT / kWave;
    constexpr int RUN = kWave * E;
    __shared__ int s_pads;  // real keys equal to pad
    const int w = wave_id(), lane = lane_id();
    if (threadIdx.x == 0)
        s_pads = 0;
    __syncthreads();
    K v[E];
    int pads = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int idx = w * RUN + e * kWave + lane;
        v[e] = idx < n ? s[idx] : pad;
        pads += (idx < n && !(v[e] < pad)) ? 1 : 0;
    }
    pads = wave_sum(pads);
    if (lane == 0 && pads)
        atomicAdd(&s_pads, pads);
    wave_sort_run<E>(v);
    __syncthreads();  // every thread has read its keys
#pragma unroll
    for (int e = 0; e < E; ++e)
        s[w * RUN + e * kWave + lane] = v[e];
    __syncthreads();
    int rank[E];
    // For every other run, the number of its keys that go before v: runs
    // before this one count keys <= v (ties go to earlier runs), runs after it
    // keys < v; "<= v" is "< v + 1" (keys equal to pad are never placed).
    // The searches into eight runs advance together (eight loads in flight);
    // one key and eight runs at a time bound the register footprint.
#pragma unroll 1
    for (int e = 0; e < E; ++e) {
        const K lt = v[e];
        const K le = v[e] < pad ? K(v[e] + 1) : v[e];
        int r = e * kWave + lane;
#pragma unroll 1
        for (int og = 0; og < NW; og += 8) {
            int lo[8];
#pragma unroll
            for (int o = 0; o < 8; ++o)
                lo[o] = 0;
#pragma unroll
            for (int step = RUN / 2; step > 0; step >>= 1) {
                K x[8];
#pragma unroll
                for (int o = 0; o < 8; ++o)
                    x[o] = s[(og + o) * RUN + lo[o] + step - 1];
#pragma unroll
                for (int o = 0; o < 8; ++o)
                    lo[o] += x[o] < (og + o < w ? le : lt) ? step : 0;
            }
#pragma unroll
            for (int o = 0; o < 8; ++o) {
                const K x = s[(og + o) * RUN + lo[o]];
                const int c = lo[o] + (x < (og + o < w ? le : lt) ? 1 : 0);
                r += og + o == w ? 0 : c;
            }
        }
        rank[e] = r;
    }
    const int n_less = n - s_pads;  // real keys below pad take places [0, n_less)
    __syncthreads();  // every search is done before keys move
#pragma unroll
    for (int e = 0; e < E; ++e)
        if (v[e] < pad && rank[e] < n_less)
            s[rank[e]] = v[e];
    for (int t = n_less + (int)threadIdx.x; t < n; t += NT)
        s[t] = pad;
    __syncthreads();
}

// s[0..n) ascending, n <= EMAX * NT; s must hold max(NT, next_pow2(n)) keys.
// Only run widths up to EMAX * 64 are instantiated (they set the register
// budget of the calling kernel).
template <int NT, int EMAX, typename K>
__device__ void block_merge_sort(K *s, int n, K pad)
{
    const int E = next_pow2(n > NT ? n : NT) / NT;
    if (EMAX <= 1 || E <= 1)
        block_merge_sort_e<NT, 1, K>(s, n, pad);
    else if (EMAX <= 2 || E <= 2)
        block_merge_sort_e<NT, (EMAX >= 2 ? 2 : 1), K>(s, n, pad);
    else if (EMAX <= 4 || E <= 4)
        block_merge_sort_e<NT, (EMAX >= 4 ? 4 : 1), K>(s, n, pad);
    else
        block_merge_sort_e<NT, (EMAX >= 8 ? 8 : 1), K>(s, n, pad);
}

}  // namespace kvr
