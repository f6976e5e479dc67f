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

// DPP controls of gfx9: within one instruction a lane reads another lane of
// its row of 16 (quad permutations, the mirror of each half row and of each
// row, shifts right inside a row) or the last lane of an earlier row, with no
// trip through LDS.  A lane whose source lies outside its row, and every lane
// of a row left out by the row mask, reads 0.
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppRowShr1 = 0x111;       // lane - 1 of the row
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowMirror = 0x140;     // lane 15 - i of the row
constexpr int kDppRowHalfMirror = 0x141; // lane 7 - i of the half row
constexpr int kDppRowBcast15 = 0x142;    // lane 15 of the row before
constexpr int kDppRowBcast31 = 0x143;    // lane 31, into rows 2 and 3

template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t dpp32(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROWS, 0xF, false);
}

template <int CTRL, typename T>
__device__ __forceinline__ T dpp_move(T x)
{
    static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit lanes");
    if constexpr (sizeof(T) == 8) {
        const uint64_t u = (uint64_t)x;
        return (T)(((uint64_t)dpp32<CTRL>((uint32_t)(u >> 32)) << 32) | dpp32<CTRL>((uint32_t)u));
    } else {
        return (T)dpp32<CTRL>((uint32_t)x);
    }
}

// The value of x in lane `lane` (uniform), for every lane.
template <typename T>
__device__ __forceinline__ T lane_value(T x, int lane)
{
    static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit lanes");
    if constexpr (sizeof(T) == 8) {
        const uint64_t u = (uint64_t)x;
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
        return (T)(((uint64_t)hi << 32) | lo);
    } else {
        return (T)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, lane);
    }
}

// Inclusive prefix sum over the 64 lanes of a full wave: a scan inside each
// row by shifts of 1, 2, 4 and 8 lanes, then each row adds the totals of the
// rows before it.
__device__ __forceinline__ int wave_inclusive_scan(int x)
{
    uint32_t v = (uint32_t)x;
    v += dpp32<kDppRowShr1>(v);
    v += dpp32<kDppRowShr2>(v);
    v += dpp32<kDppRowShr4>(v);
    v += dpp32<kDppRowShr8>(v);
    v += dpp32<kDppRowBcast15, 0xA>(v);
    v += dpp32<kDppRowBcast31, 0xC>(v);
    return (int)v;
}

// Reduction of a full wave by a commutative, associative op: inside each row
// (quads, then mirrored half rows, then mirrored rows), then over the four
// rows' results in scalar registers; every lane gets the result.
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T x, Op op)
{
    x = op(x, dpp_move<kDppQuadXor1>(x));
    x = op(x, dpp_move<kDppQuadXor2>(x));
    x = op(x, dpp_move<kDppRowHalfMirror>(x));
    x = op(x, dpp_move<kDppRowMirror>(x));
    return op(op(lane_value(x, 0), lane_value(x, 16)), op(lane_value(x, 32), lane_value(x, 48)));
}

template <typename T>
__device__ __forceinline__ T wave_sum(T x)
{
    return wave_reduce(x, [](T a, T b) { return a + b; });
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
    return wave_reduce(x, [](T a, T b) { return b < a ? b : a; });
}

template <typename T>
__device__ __forceinline__ T wave_max(T x)
{
    return wave_reduce(x, [](T a, T b) { return b > a ? b : a; });
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
                    const K o = j == 1   ? dpp_move<kDppQuadXor1>(v[e])
                                : j == 2 ? dpp_move<kDppQuadXor2>(v[e])
                                         : __shfl_xor(v[e], j, kWave);
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
