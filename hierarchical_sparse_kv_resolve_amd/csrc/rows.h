// Row movers' common pieces: the tile of whole rows a workgroup moves and
// 16-byte chunk loads and stores.
//
// Rows are opaque R-byte payloads (R a multiple of 16).  A workgroup owns a
// tile of whole rows; the rows' source and destination addresses are staged
// in LDS once, then the tile is moved as a flat run of 16-byte chunks spread
// over all lanes, with every load of a thread issued before its stores so
// that several 16-byte requests per lane are in flight.  Rows of 1152 B (72
// chunks) or 656 B (41 chunks) therefore never leave lanes idle the way a
// one-row-per-wave mapping would.
#pragma once

#include "kvr_internal.h"

namespace kvr {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowThreads = 256;  // threads per row-moving workgroup
constexpr int kUnroll = 8;        // 16-byte loads in flight per lane (host reads)
constexpr int kGatherUnroll = 6;  // the same for device gathers: smaller tiles, more of them
constexpr int kMaxTileRows = 128;

struct TileShape {
    int32_t rows;    // rows per workgroup tile
    int32_t chunks;  // 16-byte chunks per row
    uint64_t magic;  // row = (chunk * magic) >> 32 for chunk < rows * chunks
};

__device__ __forceinline__ void load_chunk(u32x4 &v, const uint8_t *p)
{
    v = *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ void store_chunk_nt(uint8_t *p, const u32x4 &v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}

__device__ __forceinline__ void store_chunk(uint8_t *p, const u32x4 &v)
{
    *reinterpret_cast<u32x4 *>(p) = v;
}

// As many whole rows as `unroll` chunks per lane of a workgroup of `threads`
// cover, and the multiplier that divides a chunk index by the row's chunk
// count.
inline TileShape tile_for(const Shape &sh, int unroll, int threads = kRowThreads)
{
    TileShape ts;
    ts.chunks = sh.R / 16;
    int rows = (threads * unroll) / ts.chunks;
    ts.rows = rows < 1 ? 1 : (rows > kMaxTileRows ? kMaxTileRows : rows);
    ts.magic = (((uint64_t)1 << 32) + ts.chunks - 1) / ts.chunks;
    return ts;
}

}  // namespace kvr
