// Workgroup-level building blocks for 64-lane gfx950 wavefronts: ballot
// compaction, scans, reductions and an LDS bitonic sort.
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

template <typename T>
__device__ __forceinline__ T wave_inclusive_scan_t(T x)
{
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        T y = __shfl_up(x, d, kWave);
        if (lane_id() >= d)
            x += y;
    }
    return x;
}

// Exclusive prefix sum of 64-bit values over the workgroup in thread order.
// Used with several small counters packed into one word (each field must not
// overflow into the next).  `scratch`: NT/64 words of LDS.
typedef unsigned long long u64;

template <int NT>
__device__ __forceinline__ u64 block_exclusive_scan64(u64 v, u64 *scratch, u64 &total)
{
    constexpr int NW = NT / kWave;
    u64 incl = wave_inclusive_scan_t<u64>(v);
    if (lane_id() == kWave - 1)
        scratch[wave_id()] = incl;
    __syncthreads();
    if (wave_id() == 0) {
        u64 w = lane_id() < NW ? scratch[lane_id()] : 0;
        w = wave_inclusive_scan_t<u64>(w);
        if (lane_id() < NW)
            scratch[lane_id()] = w;
    }
    __syncthreads();
    u64 base = wave_id() > 0 ? scratch[wave_id() - 1] : 0;
    total = scratch[NW - 1];
    __syncthreads();
    return base + incl - v;
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

// One compare-exchange stage of a bitonic network whose partner lies in the
// same thread (stride j = JE * NT).  Element e of a thread sits at index
// e * NT + tid.
template <int NT, int E, int JE, typename K>
__device__ __forceinline__ void bitonic_stage_regs(K (&v)[E], int k)
{
#pragma unroll
    for (int e = 0; e < E; ++e) {
        if ((e & JE) == 0) {
            const int idx = e * NT + (int)threadIdx.x;
            const bool up = (idx & k) == 0;
            K a = v[e], b = v[e | JE];
            if (up ? (a > b) : (a < b)) {
                v[e] = b;
                v[e | JE] = a;
            }
        }
    }
}

// Ascending bitonic sort of NT * E keys held E per thread (element e of a
// thread is index e * NT + tid), the 64-lane wavefront way: strides below 64
// exchange through cross-lane shuffles, strides of 64 .. NT/2 through LDS
// (`xch`, NT * E keys), and strides of NT and more stay inside a thread.
// Every thread of the workgroup must call it.
template <int NT, int E, typename K>
__device__ void block_sort_regs(K (&v)[E], K *xch)
{
    constexpr int N = NT * E;
    const int tid = threadIdx.x;
    for (int k = 2; k <= N; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            if (j >= NT) {
                const int je = j / NT;
                if (E >= 2 && je == 1)
                    bitonic_stage_regs<NT, E, (E >= 2 ? 1 : 0)>(v, k);
                else if (E >= 4 && je == 2)
                    bitonic_stage_regs<NT, E, (E >= 4 ? 2 : 0)>(v, k);
                else if (E >= 8 && je == 4)
                    bitonic_stage_regs<NT, E, (E >= 8 ? 4 : 0)>(v, k);
            } else if (j >= kWave) {
#pragma unroll
                for (int e = 0; e < E; ++e)
                    xch[e * NT + tid] = v[e];
                __syncthreads();
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int idx = e * NT + tid;
                    const K o = xch[idx ^ j];
                    const bool keep_min = ((idx & j) == 0) == ((idx & k) == 0);
                    v[e] = keep_min ? (o < v[e] ? o : v[e]) : (o > v[e] ? o : v[e]);
                }
                __syncthreads();
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int idx = e * NT + tid;
                    const K o = __shfl_xor(v[e], j, kWave);
                    const bool keep_min = ((idx & j) == 0) == ((idx & k) == 0);
                    v[e] = keep_min ? (o < v[e] ? o : v[e]) : (o > v[e] ? o : v[e]);
                }
            }
        }
    }
}

// Sort s[0..n) ascending in LDS, with `pad` filling up to the sorting width
// (max(NT, next power of two >= n), at most 8 * NT entries of s).  Ends with
// a barrier.
template <int NT, typename K>
__device__ void block_sort_lds(K *s, int n, K pad)
{
    const int width = next_pow2(n > NT ? n : NT);
    const int E = width / NT;
    const int tid = threadIdx.x;
    if (E == 1) {
        K v[1];
        v[0] = tid < n ? s[tid] : pad;
        __syncthreads();
        block_sort_regs<NT, 1>(v, s);
        s[tid] = v[0];
    } else if (E == 2) {
        K v[2];
#pragma unroll
        for (int e = 0; e < 2; ++e)
            v[e] = e * NT + tid < n ? s[e * NT + tid] : pad;
        __syncthreads();
        block_sort_regs<NT, 2>(v, s);
#pragma unroll
        for (int e = 0; e < 2; ++e)
            s[e * NT + tid] = v[e];
    } else if (E == 4) {
        K v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            v[e] = e * NT + tid < n ? s[e * NT + tid] : pad;
        __syncthreads();
        block_sort_regs<NT, 4>(v, s);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            s[e * NT + tid] = v[e];
    } else {
        K v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            v[e] = e * NT + tid < n ? s[e * NT + tid] : pad;
        __syncthreads();
        block_sort_regs<NT, 8>(v, s);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            s[e * NT + tid] = v[e];
    }
    __syncthreads();
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

// E independent binary searches at once (their LDS reads overlap): idx[e] is
// the position of key[e] in the ascending s[0..n), or -1.
template <int E>
__device__ __forceinline__ void lds_find_many(const int32_t *s, int n, const int32_t (&key)[E],
                                              int (&idx)[E])
{
    int lo[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        lo[e] = 0;
    // loads are unconditional (indices clamped into the array) so that all E
    // of a round are in flight together
    for (int step = next_pow2(n + 1) >> 1; step > 0; step >>= 1) {
        int32_t x[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int probe = lo[e] + step - 1;
            x[e] = s[probe < n ? probe : 0];
        }
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int probe = lo[e] + step - 1;
            lo[e] += (probe < n && x[e] < key[e]) ? step : 0;
        }
    }
    int32_t x[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        x[e] = s[lo[e] < n ? lo[e] : 0];
#pragma unroll
    for (int e = 0; e < E; ++e)
        idx[e] = (lo[e] < n && x[e] == key[e]) ? lo[e] : -1;
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


}  // namespace kvr
