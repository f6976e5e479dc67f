// Device code of the resolve (steps 1 to 3 of "Resolution" for one request
// per workgroup of 1024 threads), shared by the resolve kernel and the
// launch that gathers one selection while resolving the next.
#pragma once

#include <climits>

#include "block.h"
#include "kvr_internal.h"

namespace kvr {
namespace {

constexpr int NT = 1024;
constexpr int NW = NT / kWave;
// Selection entries (EK) and hot slots (EB) per thread are template
// parameters: the launch picks the smallest of 1, 2, 4, 8 that covers sel_cap
// and B, so small shapes keep fewer live registers.
constexpr int kCntE = 8;  // hot-slot entries per thread the compaction counters cover
constexpr int32_t kEmpty = -1;
constexpr int32_t kNoSlot = INT_MAX;
constexpr int32_t kFilledBit = 1 << 30;
// A pending entry keeps its hash entry in its location word until the end:
// place bits 3 with an index below 2^30 is no valid word (invalid is all ones).
constexpr uint32_t kPendingTag = 3u << 30;
__device__ __forceinline__ bool is_pending(uint32_t w) { return (w >> 30) == 3u && w != 0xFFFFFFFFu; }

struct ResolveArgs {
    Shape sh;
    int32_t n;  // request entries of the call
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
    int32_t vc;  // sKey entries: max(NT, next_pow2(min(B, sel_cap)))
    int32_t hs;  // hash entries
    int32_t bw;  // words of the miss bitmap over rows 0 .. host_rows-1 (0: none)
    // append in the same launch (new_rows non-null): [n_layers][n][R]
    const LayerPtrs *layers;
    const uint8_t *new_rows;
    int32_t *append_status;
    // deferred append: the host row and L only; the tail slot is written by
    // the gather launch that consumes append_pos (the appended position, or
    // -1 when the entry appended nothing)
    int32_t *append_pos;
    int32_t defer_tail;
};

__device__ __forceinline__ int hslot(int32_t key, int hs)
{
    return (int)(((uint64_t)((uint32_t)key * 0x9E3779B1u) * (uint32_t)hs) >> 32);
}

__device__ __forceinline__ int hnext(int idx, int hs) { return idx + 1 == hs ? 0 : idx + 1; }

// Insert key (>= 0) if absent.  Returns the key's entry; `fresh` tells
// whether this call put it there.  The table always keeps an empty entry
// (more entries than keys), so probing ends.
__device__ __forceinline__ int hinsert(int32_t *hkey, int hs, int32_t key, bool &fresh)
{
    int idx = hslot(key, hs);
    while (true) {
        const int32_t old = atomicCAS(&hkey[idx], kEmpty, key);
        if (old == kEmpty || old == key) {
            fresh = old == kEmpty;
            return idx;
        }
        idx = hnext(idx, hs);
    }
}

// Ascending order of n <= 256 distinct keys s[0..n) in place, by counting for
// each key the keys below it.  P = NT / next_pow2(n) consecutive lanes share
// one key and split the count over contiguous chunks (eight independent LDS
// reads in flight per round); the partial counts meet through shuffles.
template <int NT, typename K>
__device__ __forceinline__ void rank_sort_small(K *s, int n)
{
    const int tid = threadIdx.x;
    int P = NT / next_pow2(n > 0 ? n : 1);
    P = P > kWave ? kWave : P;
    const int el = tid / P, part = tid % P;
    const K mine = el < n ? s[el] : K(0);
    const int chunk = (n + P - 1) / P;
    const int j0 = part * chunk;
    const int j1 = j0 + chunk < n ? j0 + chunk : n;
    int below = 0;
    int j = j0;
    for (; j + 8 <= j1; j += 8) {
        K v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            v[q] = s[j + q];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            below += v[q] < mine ? 1 : 0;
    }
    for (; j < j1; ++j)
        below += s[j] < mine ? 1 : 0;
    // the P lanes of one key add their counts: inside rows by DPP, across
    // rows by shuffles (P is uniform)
    if (P >= 2)
        below += dpp_move<kDppQuadXor1>(below);
    if (P >= 4)
        below += dpp_move<kDppQuadXor2>(below);
    if (P >= 8)
        below += dpp_move<kDppRowHalfMirror>(below);
    if (P >= 16)
        below += dpp_move<kDppRowMirror>(below);
    if (P >= 32)
        below += __shfl_xor(below, 16, kWave);
    if (P >= 64)
        below += __shfl_xor(below, 32, kWave);
    __syncthreads();
    if (el < n && part == 0)
        s[below] = mine;
    __syncthreads();
}

// E lookups with interleaved probes: idx[e] = entry of key[e], or -1 when it
// is absent or key[e] < 0.  Each round issues all E loads before using any
// (finished lookups re-read their last entry), so their latencies overlap.
template <int E>
__device__ __forceinline__ void hfind_many(const int32_t *hkey, int hs, const int32_t (&key)[E],
                                           int (&idx)[E])
{
    int cur[E];
    bool live[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        live[e] = key[e] >= 0;
        cur[e] = live[e] ? hslot(key[e], hs) : 0;
        idx[e] = -1;
    }
    while (true) {
        int32_t kk[E];
#pragma unroll
        for (int e = 0; e < E; ++e)
            kk[e] = hkey[cur[e]];
        bool any = false;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const bool hit = live[e] && kk[e] == key[e];
            const bool stop = hit || kk[e] == kEmpty;
            idx[e] = hit ? cur[e] : idx[e];
            live[e] = live[e] && !stop;
            const int nxt = cur[e] + 1 == hs ? 0 : cur[e] + 1;
            cur[e] = live[e] ? nxt : cur[e];
            any = any || live[e];
        }
        if (!any)
            break;
    }
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Chunks of the decoded rows a block appends: per layer, the host copy, then
// (unless the tail write is deferred) the tail copy, of R/16 chunks each.
__device__ __forceinline__ int append_per_layer(const ResolveArgs &a)
{
    return (a.sh.R / 16) * (a.sh.T > 0 && !a.defer_tail ? 2 : 1);
}

// A thread's first chunk to append (chunk threadIdx.x) and the store it goes
// to, loaded before the request's length is known: the chunk does not depend
// on it, so the append waits for one memory round trip instead of two.
struct AppendChunk {
    u32x4 v;
    uint8_t *base;  // the layer's host store or tail
};

__device__ __forceinline__ AppendChunk append_first(const ResolveArgs &a, int i)
{
    AppendChunk f;
    f.v = u32x4{0u, 0u, 0u, 0u};
    f.base = nullptr;
    const int per_layer = append_per_layer(a);
    const int c = threadIdx.x;
    if (a.new_rows && c < per_layer * a.sh.n_layers) {
        const int C = a.sh.R / 16;
        const int l = c / per_layer;
        const int e = c - l * per_layer;
        f.v = *reinterpret_cast<const u32x4 *>(a.new_rows + ((int64_t)l * a.n + i) * a.sh.R +
                                               (e % C) * 16);
        f.base = e < C ? a.layers[l].host : a.layers[l].tail;
    }
    return f;
}

// The request's decoded row of every layer into tail slot L mod T and, written
// through, host row L (what kvr_append_rows does), by all threads of the block.
// A deferred append writes the host row only.  `first` is append_first's.
__device__ __forceinline__ void append_row(const ResolveArgs &a, int i, int r, int32_t L,
                                           const AppendChunk &first)
{
    const Shape &sh = a.sh;
    const int C = sh.R / 16;
    const int per_layer = append_per_layer(a);
    for (int c = threadIdx.x; c < per_layer * sh.n_layers; c += NT) {
        const int l = c / per_layer;
        const int e = c - l * per_layer;
        const int off = (e % C) * 16;
        u32x4 v;
        uint8_t *base;
        if (c == (int)threadIdx.x) {
            v = first.v;
            base = first.base;
        } else {
            v = *reinterpret_cast<const u32x4 *>(a.new_rows + ((int64_t)l * a.n + i) * sh.R + off);
            base = e < C ? a.layers[l].host : a.layers[l].tail;
        }
        uint8_t *dst = (e < C) ? base + ((int64_t)r * sh.host_rows + L) * sh.R + off
                               : base + ((int64_t)r * sh.T + L % sh.T) * sh.R + off;
        *reinterpret_cast<u32x4 *>(dst) = v;
    }
}

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

template <int EK, int EB>
__device__ __forceinline__ void resolve_body(const ResolveArgs &a, int i, uint8_t *lds)
{
    static_assert(EB <= kCntE && 2 * kCntE * NW == 4 * kWave, "compaction counter layout");
    // the instances that spill unless the stamp-range reductions are pinned
    constexpr bool kPinRange = EK >= 8 || (EK >= 4 && EB >= 8);
    uint64_t *sKey = reinterpret_cast<uint64_t *>(lds);
    int32_t *hkey = reinterpret_cast<int32_t *>(sKey + a.vc);
    int32_t *hval = hkey + a.hs;
    uint32_t *bm = reinterpret_cast<uint32_t *>(hval + a.hs);  // [bw] miss rows
    int32_t *sChunk = reinterpret_cast<int32_t *>(bm + a.bw);  // [NT] when bw > 0
    __shared__ int sHist[256];
    __shared__ int sCnt[2 * kCntE * NW];  // [kind][e][wave]; e >= EB stays 0
    __shared__ uint32_t sRedU[2 * NW];
    __shared__ int sPick[2];
    __shared__ int sUnique;
    __shared__ int sMiss;
    __shared__ int sRangeErr;
    __shared__ int sHostErr;
    __shared__ unsigned long long sStat;

    const Shape &sh = a.sh;
    const int tid = threadIdx.x;
    const int hs = a.hs;
    const int r = a.req_ids ? a.req_ids[i] : i;
    int k = a.sel_count ? a.sel_count[i] : a.stride;
    const bool r_ok = r >= 0 && r < sh.n_req;
    const bool call_ok = r_ok && k >= 0 && k <= a.stride;
    const int32_t *sel = a.sel + (int64_t)i * a.stride;
    uint32_t *loc = a.loc + (int64_t)i * a.stride;
    int32_t *tag = a.tag + (int64_t)r * sh.B;
    uint32_t *stamp = a.stamp + (int64_t)r * sh.B;

    // Every load that needs only the call's arguments is issued before any
    // is used, so their round trips overlap: the request's length, this
    // thread's first chunk to append, its selection rows (the head of the
    // longest dependent chain: row -> page map), and the tags and stamps of
    // its slots (b = e*NT + tid).
    int32_t L = r_ok ? a.L[r] : 0;
    const AppendChunk first = append_first(a, i);
    int32_t p_in[EK];
#pragma unroll
    for (int e = 0; e < EK; ++e) {
        const int j = e * NT + tid;
        p_in[e] = call_ok && j < k ? sel[j] : 0;
    }
    int32_t t[EB];
    uint32_t st[EB];
#pragma unroll
    for (int e = 0; e < EB; ++e) {
        const int b = e * NT + tid;
        t[e] = call_ok && b < sh.B ? tag[b] : -1;
        st[e] = call_ok && b < sh.B ? stamp[b] : 0u;
    }
    const uint32_t clk = call_ok ? a.clock[r] : 0u;

    // Append first when asked (it fails alone, as the separate call would):
    // every thread has read L before thread 0 publishes L + 1 after a barrier.
    bool appended = false;
    if (a.new_rows) {
        int code = KVR_E_ARG;
        if (r_ok) {
            if (L < 0 || (int64_t)L >= sh.host_rows) {
                code = KVR_E_CAPACITY;
            } else {
                append_row(a, i, r, L, first);
                appended = true;
                code = KVR_OK;
                ++L;
            }
        }
        if (tid == 0 && a.append_status)
            a.append_status[i] = code;
        if (tid == 0 && a.append_pos)
            a.append_pos[i] = appended ? L - 1 : -1;
    }
    if (!call_ok) {
        if (appended) {
            __syncthreads();
            if (tid == 0)
                a.L[r] = L;
        }
        fail_request(a, i, k < 0 ? 0 : (k > a.stride ? a.stride : k), KVR_E_ARG);
        return;
    }
    const int32_t tail_lo = sh.T > 0 ? max(L - sh.T, 0) : L;
    const int32_t *pmap = a.page_map + (int64_t)r * sh.n_pages;
    const uint8_t *hvalid = a.host_valid + (int64_t)r * sh.n_pages;

    for (int x = tid; x < hs; x += NT) {
        hkey[x] = kEmpty;
        hval[x] = kNoSlot;
    }
    for (int x = tid; x < a.bw; x += NT)
        bm[x] = 0;
    for (int x = tid; x < 256; x += NT)
        sHist[x] = 0;
    for (int x = tid; x < 2 * kCntE * NW; x += NT)
        sCnt[x] = 0;
    if (tid == 0) {
        sUnique = 0;
        sMiss = 0;
        sRangeErr = 0;
        sHostErr = 0;
        sStat = 0;
    }
    __syncthreads();
    if (appended && tid == 0)
        a.L[r] = L;

    // Step 1 and range check.  Entry e of this thread is selection j = e*NT+tid;
    // its row and location word stay in registers until the end.  Rows in the
    // tail window or in a ready complete page are found here; the others go
    // into the hash once each.
    uint32_t word[EK];
    int owned = 0, nohost = 0, fresh_n = 0;
    // the page-map entry and the host-copy flag of every entry's page, all
    // loads issued before any is used
    int32_t phys[EK];
    uint8_t hostok[EK];
#pragma unroll
    for (int e = 0; e < EK; ++e) {
        word[e] = 0;
        const int32_t p = p_in[e];
        const bool paged = e * NT + tid < k && p >= 0 && p < tail_lo;
        phys[e] = paged && p < sh.full_rows ? pmap[p / sh.P] : -1;
        hostok[e] = paged && p < sh.H ? hvalid[p / sh.P] : (uint8_t)1;
    }
#pragma unroll
    for (int e = 0; e < EK; ++e) {
        const int j = e * NT + tid;
        if (j < k) {
            const int32_t p = p_in[e];
            if (p < 0 || p >= L) {
                sRangeErr = 1;
            } else if (p >= tail_lo) {
                word[e] = (uint32_t)(p % sh.T);
            } else if (phys[e] >= 0) {
                word[e] = (1u << kPlaceShift) | (uint32_t)((int64_t)phys[e] * sh.P + p % sh.P);
            } else {
                bool fresh;
                word[e] = kPendingTag | (uint32_t)hinsert(hkey, hs, p, fresh);
                if (fresh) {
                    owned |= 1 << e;
                    ++fresh_n;
                    if (!hostok[e])
                        nohost |= 1 << e;
                }
            }
        }
    }
    {
        const int wf = wave_sum(fresh_n);
        uint32_t lo = 0xFFFFFFFFu, hi = 0;
        int32_t tmax = -1;
#pragma unroll
        for (int e = 0; e < EB; ++e) {
            if (e * NT + tid < sh.B) {
                lo = st[e] < lo ? st[e] : lo;
                hi = st[e] > hi ? st[e] : hi;
            }
            tmax = t[e] > tmax ? t[e] : tmax;  // waits for the tags here, in step 1's shadow
        }
        lo = wave_min(lo);
        hi = wave_max(hi);
        // tmax is never used: consuming it here makes the tag loads complete
        // inside step 1 instead of being sunk to their first use
        asm volatile("; tags in %0" ::"v"(tmax));
        if (lane_id() == 0) {
            if (wf)
                atomicAdd(&sUnique, wf);
            sRedU[wave_id()] = lo;
            sRedU[NW + wave_id()] = hi;
        }
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
    const int nU = sUnique;
    if (nU > sh.B) {
        fail_request(a, i, k, KVR_E_CAPACITY);
        return;
    }
    const uint32_t now = clk + 1;
    // The block's stamp range.  The compiler loads the 2*NW per-wave values
    // here and reduces them at the range's first use in step 3, which hides
    // the reduction but keeps all of them live across step 2; in the largest
    // instances that spills registers to scratch (reloaded on step 3's
    // critical path, about 4 us), so there the empty asm makes the reduction
    // happen here.
    uint32_t lo = 0xFFFFFFFFu, hi = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        lo = sRedU[w] < lo ? sRedU[w] : lo;
        hi = sRedU[NW + w] > hi ? sRedU[NW + w] : hi;
    }
    if constexpr (kPinRange)
        asm volatile("" : "+v"(lo), "+v"(hi));

    // Step 2: every tag is looked up once among the pending rows.  If two
    // slots ever held one row, the lower slot is the hit.
    int fidx[EB];
    hfind_many<EB>(hkey, hs, t, fidx);
#pragma unroll
    for (int e = 0; e < EB; ++e)
        if (fidx[e] >= 0)
            atomicMin(&hval[fidx[e]], e * NT + tid);
    __syncthreads();

    // Misses: pending rows no slot holds (each checked once, by the entry that
    // inserted it); each needs a host copy.  They are marked in the row bitmap
    // or, without one, listed as packed (row, hash entry).
    uint64_t *sMissList = sKey;
    int32_t hv[EK];
#pragma unroll
    for (int e = 0; e < EK; ++e)
        hv[e] = hval[((owned >> e) & 1) ? (word[e] & kIndexMask) : 0];
#pragma unroll
    for (int e = 0; e < EK; ++e) {
        const uint32_t h = word[e] & kIndexMask;
        const bool miss = ((owned >> e) & 1) && hv[e] == kNoSlot;
        if (miss && ((nohost >> e) & 1))
            sHostErr = 1;
        const uint64_t mb = __ballot(miss);
        int wbase = 0;
        if (lane_id() == 0 && mb)
            wbase = atomicAdd(&sMiss, __popcll(mb));
        wbase = lane_value(wbase, 0);
        if (miss) {
            const int32_t row = hkey[h];
            if (a.bw > 0)
                atomicOr(&bm[row >> 5], 1u << (row & 31));
            else
                sMissList[wbase + ballot_rank(mb)] = ((uint64_t)(uint32_t)row << 32) | h;
        }
    }
    __syncthreads();
    if (sHostErr) {
        fail_request(a, i, k, KVR_E_NO_HOST_COPY);
        return;
    }
    const int m_total = sMiss;

    if (m_total > 0) {
        // Misses in ascending row order: a miss's rank is the number of miss
        // rows below it.  With the bitmap, each thread counts the bits of a
        // run of words, a block scan turns the counts into run offsets, and
        // each miss adds the bits below it inside its run.  Without it, the
        // list is sorted (wave-sorted runs merged by rank) and each miss
        // learns its rank through the hash entry packed with its row.
        if (a.bw > 0) {
            const int wpt = (a.bw + NT - 1) / NT;
            const int w0 = tid * wpt;
            int cnt = 0;
            for (int x = w0; x < w0 + wpt && x < a.bw; ++x)
                cnt += __popc(bm[x]);
            const int incl = wave_inclusive_scan(cnt);
            if (lane_id() == kWave - 1)
                sRedU[wave_id()] = (uint32_t)incl;
            __syncthreads();
            int base = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w)
                base += w < wave_id() ? (int)sRedU[w] : 0;
            sChunk[tid] = base + incl - cnt;
            __syncthreads();
#pragma unroll
            for (int e = 0; e < EK; ++e) {
                if (!((owned >> e) & 1) || hv[e] != kNoSlot)
                    continue;
                const uint32_t h = word[e] & kIndexMask;
                const int32_t row = hkey[h];
                const int w = row >> 5;
                const int c = w / wpt;
                int rank = sChunk[c] + __popc(bm[w] & ((1u << (row & 31)) - 1u));
                for (int x = c * wpt; x < w; ++x)
                    rank += __popc(bm[x]);
                hval[h] = -1 - rank;
            }
        } else if (m_total <= 256) {
            rank_sort_small<NT, uint64_t>(sMissList, m_total);
            for (int q = tid; q < m_total; q += NT)
                hval[(uint32_t)sMissList[q]] = -1 - q;
        } else {
            // plain rows sort cheaper; each then finds its entry in the hash
            int32_t *rows = reinterpret_cast<int32_t *>(sMissList);
            uint32_t own[EK];
#pragma unroll
            for (int e = 0; e < EK; ++e) {
                const int q = e * NT + tid;
                own[e] = q < m_total ? (uint32_t)(sMissList[q] >> 32) : 0u;
            }
            __syncthreads();
#pragma unroll
            for (int e = 0; e < EK; ++e) {
                const int q = e * NT + tid;
                if (q < m_total)
                    rows[q] = (int32_t)own[e];
            }
            __syncthreads();
            block_merge_sort<NT, (EK < EB ? EK : EB), int32_t>(rows, m_total, INT_MAX);
            int32_t key[EK];
            int idx[EK];
#pragma unroll
            for (int e = 0; e < EK; ++e) {
                const int q = e * NT + tid;
                key[e] = q < m_total ? rows[q] : -1;
            }
            hfind_many<EK>(hkey, hs, key, idx);
#pragma unroll
            for (int e = 0; e < EK; ++e)
                if (idx[e] >= 0)
                    hval[idx[e]] = -1 - (e * NT + tid);
        }
        __syncthreads();

        // Step 3: victims = the m_total smallest (stamp, slot) among the slots
        // whose tag is not a hit of this call.
        bool cand[EB];
        {
            int32_t hs_[EB];
#pragma unroll
            for (int e = 0; e < EB; ++e)
                hs_[e] = hval[fidx[e] >= 0 ? fidx[e] : 0];
#pragma unroll
            for (int e = 0; e < EB; ++e) {
                const int b = e * NT + tid;
                cand[e] = b < sh.B && !(fidx[e] >= 0 && hs_[e] == b);
            }
        }
        // Radix select of the threshold stamp over rel = stamp - lo, 8 bits
        // at a time from the highest digit that varies.
        const uint32_t span = hi - lo;
        int top = 0;
        while (top < 24 && (span >> top) > 0xFF)
            top += 8;
        uint32_t prefix = 0;
        int m_rem = m_total;
        int c_lt = 0;
        if (span > 0) {
            for (int shift = top; shift >= 0; shift -= 8) {
                const uint32_t hmask = (shift + 8 >= 32) ? 0u : (0xFFFFFFFFu << (shift + 8));
                if (span < (uint32_t)kWave) {
                    // one pass over at most 64 stamp values, which candidates
                    // share in large groups: each wave counts every value by
                    // ballots and lane v adds value v's count (same-address
                    // LDS atomics from one wave would be serialized)
                    // (non-candidates compare as a value above any v)
                    uint32_t rel[EB];
#pragma unroll
                    for (int e = 0; e < EB; ++e)
                        rel[e] = cand[e] ? st[e] - lo : 0xFFFFFFFFu;
                    int mine = 0;
                    const int vmax = __builtin_amdgcn_readfirstlane((int)span);  // uniform
                    for (int v = 0; v <= vmax; ++v) {
                        int c = 0;
#pragma unroll
                        for (int e = 0; e < EB; ++e)
                            c += __popcll(__builtin_amdgcn_uicmp(rel[e], (uint32_t)v, 32));  // ==
                        mine = lane_id() == v ? c : mine;
                    }
                    if (mine)
                        atomicAdd(&sHist[lane_id()], mine);
                } else {
#pragma unroll
                    for (int e = 0; e < EB; ++e) {
                        if (cand[e]) {
                            const uint32_t rel = st[e] - lo;
                            if ((rel & hmask) == prefix)
                                atomicAdd(&sHist[(rel >> shift) & 0xFF], 1);
                        }
                    }
                }
                __syncthreads();
                if (wave_id() == 0) {
                    // lane l holds bins 4l .. 4l+3; they are cleared for the next pass
                    int c[4], sum = 0;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        c[q] = sHist[lane_id() * 4 + q];
                        sHist[lane_id() * 4 + q] = 0;
                        sum += c[q];
                    }
                    const int incl = wave_inclusive_scan(sum);
                    int below = incl - sum;
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
                    const int src = found ? __ffsll((unsigned long long)found) - 1 : 0;
                    pick = lane_value(pick, src);
                    pick_below = lane_value(pick_below, src);
                    if (lane_id() == 0) {
                        sPick[0] = pick < 0 ? 0 : pick;
                        sPick[1] = pick_below;
                    }
                }
                __syncthreads();
                prefix |= (uint32_t)sPick[0] << shift;
                m_rem -= sPick[1];
                c_lt += sPick[1];
            }
        }
        const uint32_t tau = lo + prefix;

        // Ordered compaction in slot order (b = e*NT + tid, i.e. (e, wave,
        // lane)): wave ballots give the order inside a wave, one wave scans
        // the per-(e, wave) counts.  Candidates older than tau go to
        // sKey[0 .. c_lt), the first m_rem stamped tau to sKey[c_lt ..).
        uint64_t blt[EB], beq[EB];
        uint32_t l2 = 0xFFFFFFFFu, h2 = 0;
#pragma unroll
        for (int e = 0; e < EB; ++e) {
            const bool lt = cand[e] && st[e] < tau;
            const bool eq = cand[e] && st[e] == tau;
            blt[e] = __ballot(lt);
            beq[e] = __ballot(eq);
            if (lt) {
                l2 = st[e] < l2 ? st[e] : l2;
                h2 = st[e] > h2 ? st[e] : h2;
            }
            if (lane_id() == 0) {
                sCnt[e * NW + wave_id()] = __popcll(blt[e]);
                sCnt[kCntE * NW + e * NW + wave_id()] = __popcll(beq[e]);
            }
        }
        l2 = wave_min(l2);
        h2 = wave_max(h2);
        if (lane_id() == 0) {
            sRedU[wave_id()] = l2;
            sRedU[NW + wave_id()] = h2;
        }
        __syncthreads();
        if (wave_id() == 0) {
            // 2 * kCntE * NW = 256 counts, 4 per lane; lanes 0..31 hold the
            // older kind, lanes 32..63 the tau kind, each scanned on its own
            int c[4], sum = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                c[q] = sCnt[lane_id() * 4 + q];
                sum += c[q];
            }
            const int incl = wave_inclusive_scan(sum);
            const int half = lane_value(incl, kWave / 2 - 1);
            int run = incl - sum - (lane_id() >= kWave / 2 ? half : 0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                sCnt[lane_id() * 4 + q] = run;
                run += c[q];
            }
        }
        __syncthreads();
        uint32_t gl = 0xFFFFFFFFu, gh = 0;  // the same for the candidates older than tau
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            gl = sRedU[w] < gl ? sRedU[w] : gl;
            gh = sRedU[NW + w] > gh ? sRedU[NW + w] : gh;
        }
        if constexpr (kPinRange)
            asm volatile("" : "+v"(gl), "+v"(gh));
#pragma unroll
        for (int e = 0; e < EB; ++e) {
            if ((blt[e] >> lane_id()) & 1) {
                const int rank = sCnt[e * NW + wave_id()] + ballot_rank(blt[e]);
                sKey[rank] = ((uint64_t)st[e] << 32) | (uint32_t)(e * NT + tid);
            }
        }
        __syncthreads();
        if (c_lt > 1 && gl != gh) {  // uniform
            if (c_lt <= 256) {
                rank_sort_small<NT, uint64_t>(sKey, c_lt);
            } else if (gh - gl < (1u << 18)) {
                // (stamp - gl, slot) packs into 31 bits: sort those instead
                int32_t *k32 = reinterpret_cast<int32_t *>(sKey);
                uint64_t own[EB];
#pragma unroll
                for (int e = 0; e < EB; ++e) {
                    const int q = e * NT + tid;
                    own[e] = q < c_lt ? sKey[q] : 0ull;
                }
                __syncthreads();
#pragma unroll
                for (int e = 0; e < EB; ++e) {
                    const int q = e * NT + tid;
                    if (q < c_lt)
                        k32[q] = (int32_t)(((uint32_t)(own[e] >> 32) - gl) << 13 | (uint32_t)own[e]);
                }
                __syncthreads();
                block_merge_sort<NT, (EK < EB ? EK : EB), int32_t>(k32, c_lt, INT_MAX);
#pragma unroll
                for (int e = 0; e < EB; ++e) {
                    const int q = e * NT + tid;
                    own[e] = q < c_lt ? (uint64_t)(uint32_t)k32[q] : 0ull;
                }
                __syncthreads();
#pragma unroll
                for (int e = 0; e < EB; ++e) {
                    const int q = e * NT + tid;
                    if (q < c_lt)
                        sKey[q] = ((uint64_t)((uint32_t)(own[e] >> 13) + gl) << 32) |
                                  (uint32_t)(own[e] & 0x1FFF);
                }
                __syncthreads();
            } else {
                // stamps more than 2^18 ticks apart: the in-LDS network
                // (slow, rare, light on registers)
                const int width = next_pow2(c_lt);
                for (int q = c_lt + tid; q < width; q += NT)
                    sKey[q] = ~0ull;
                __syncthreads();
                bitonic_sort<NT>(sKey, width);
            }
        }
        // the sort uses sKey as its exchange buffer, so the youngest victims
        // are placed after it
#pragma unroll
        for (int e = 0; e < EB; ++e) {
            if ((beq[e] >> lane_id()) & 1) {
                const int rank = sCnt[kCntE * NW + e * NW + wave_id()] + ballot_rank(beq[e]);
                if (rank < m_rem)
                    sKey[c_lt + rank] = ((uint64_t)st[e] << 32) | (uint32_t)(e * NT + tid);
            }
        }
        __syncthreads();
    }

    // Commit: hits take the new stamp, victims the missing row and the stamp.
    kvr_fill *fills = a.fills + (int64_t)i * sh.B;
#pragma unroll
    for (int e = 0; e < EK; ++e)
        hv[e] = hval[((owned >> e) & 1) ? (word[e] & kIndexMask) : 0];
#pragma unroll
    for (int e = 0; e < EK; ++e) {
        if (!((owned >> e) & 1))
            continue;
        const uint32_t h = word[e] & kIndexMask;
        const int32_t s = hv[e];
        if (s >= 0) {
            stamp[s] = now;
        } else {
            const int rank = -1 - s;
            const int32_t slot = (int32_t)(uint32_t)sKey[rank];
            if ((uint32_t)slot >= (uint32_t)sh.B)
                continue;  // cannot happen: every rank below m_total has a victim
            const int32_t u = hkey[h];
            tag[slot] = u;
            stamp[slot] = now;
            fills[rank] = kvr_fill{u, slot};
            hval[h] = slot | kFilledBit;
        }
    }
    __syncthreads();

    // Location words in selection order; count entries by where they were found.
    uint64_t counts = 0;  // 16-bit fields: tail, page, hit, miss
#pragma unroll
    for (int e = 0; e < EK; ++e)
        hv[e] = hval[is_pending(word[e]) ? (word[e] & kIndexMask) : 0];
#pragma unroll
    for (int e = 0; e < EK; ++e) {
        const int j = e * NT + tid;
        if (j >= k)
            continue;
        uint32_t w = word[e];
        if (is_pending(w)) {
            const int32_t s = hv[e];
            w = (2u << kPlaceShift) | ((s & kFilledBit) ? kFreshBit : 0u) | (uint32_t)(s & kSlotMask);
            counts += (s & kFilledBit) ? (1ull << 48) : (1ull << 32);
        } else {
            counts += (w >> kPlaceShift) == 0 ? 1ull : (1ull << 16);
        }
        loc[j] = w;
    }
    if (a.stats) {
        // The counters are summed in LDS first and one thread per workgroup
        // adds them: device-scope atomics on one address from every wave of
        // every workgroup are serialized in the memory system and kept the
        // kernel from completing long after its last wave.  A workgroup's
        // fields stay below 2^16 (at most 8 * 1024 entries).
        const unsigned long long wsum = wave_sum((unsigned long long)counts);
        unsigned long long *stp = reinterpret_cast<unsigned long long *>(a.stats);
        if (lane_id() == 0 && wsum)
            atomicAdd(&sStat, wsum);
        __syncthreads();
        if (tid == 0) {
            const unsigned long long tot = sStat;
            atomicAdd(&stp[1], tot & 0xFFFF);
            atomicAdd(&stp[2], (tot >> 16) & 0xFFFF);
            atomicAdd(&stp[3], (tot >> 32) & 0xFFFF);
            atomicAdd(&stp[4], (tot >> 48) & 0xFFFF);
            atomicAdd(&stp[0], 1ull);
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

// Bound on the resolve's static LDS (histogram, compaction counts, scalars).
constexpr size_t kStaticLdsBound = 4096;
constexpr size_t kLdsPerCu = 160 * 1024;

// Entries per thread of the instance that covers n selection entries or
// slots: 1, 2, 4 or 8.
inline int resolve_per_thread(int n)
{
    const int e = (n + NT - 1) / NT;
    return e <= 1 ? 1 : (e <= 2 ? 2 : (e <= 4 ? 4 : 8));
}

// The arguments of one resolve call; returns the dynamic LDS it needs.
inline size_t resolve_args(ResolveArgs &a, const kvr_ctx *c, int32_t n, const int32_t *req_ids,
                           const int32_t *sel, const int32_t *sel_count, int32_t stride,
                           uint32_t *loc, kvr_fill *fills, int32_t *fill_count, int32_t *status,
                           kvr_stats *stats, int32_t count_host_bytes, const uint8_t *new_rows,
                           int32_t *append_status, int32_t *append_pos)
{
    a.n = n;
    a.layers = c->layers_d;
    a.new_rows = new_rows;
    a.append_status = append_status;
    a.append_pos = append_pos;
    a.defer_tail = append_pos != nullptr;
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
    return resolve_lds_layout(c->shape, &a.vc, &a.hs, &a.bw);
}

}  // namespace
}  // namespace kvr
