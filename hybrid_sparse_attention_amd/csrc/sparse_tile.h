// Gathered-row tiles shared by the forward and backward kernels of the DSA sparse core
// attention: 256-wide bfloat16 latent rows, brought to LDS 32 at a time by LDS DMA, with the
// 32 16-byte chunks of each row rotated (chunk c of row r at position (c + 2r + 16 (r & 1))
// mod 32) so that row-wise reads (keys) and transposing reads (values) both run at the LDS's
// full rate on gfx950 (measured: the XOR swizzles tried before left both reads about 1.5x
// slower).
#pragma once

#include "common.h"

namespace lgsa {
namespace sparse_tile {

constexpr int D = 256;                  // head width of query/key and value
constexpr int KT = 32;                  // keys per tile
constexpr int TROW = 2 * D;             // bytes of one gathered row (no padding: rotated)
constexpr int TILE = KT * TROW;         // 16 KiB

// 16-byte position of chunk c (0..31) of tile row r, and the chunk held at position q
__device__ __forceinline__ int chunk_pos(int r, int c) { return (c + 2 * r + 16 * (r & 1)) & 31; }
__device__ __forceinline__ int chunk_at(int r, int q) { return (q - 2 * r - 16 * (r & 1)) & 31; }

// Gather one tile: DMA instruction i (of 16) loads tile rows 2i (lanes 0..31) and 2i + 1
// (lanes 32..63); wave w issues i = w, w + NW, ...  `ix` holds, in lane j < 32, the position
// of tile row j (-1 when skipped: the row is then read from position 0 and masked).
template <int NW>
__device__ __forceinline__ void gather_tile(const uint16_t* rows, long long stride, int ix,
                                            char* tile, int w, int lane) {
  const int hi = lane >> 5;
  for (int i = w; i < KT / 2; i += NW) {
    const int sa = __builtin_amdgcn_readlane(ix, 2 * i);
    const int sb = __builtin_amdgcn_readlane(ix, 2 * i + 1);
    const int s = max(hi ? sb : sa, 0);
    const int r = 2 * i + hi;
    const int chunk = chunk_at(r, lane & 31);
    lds_dma16(rows + (size_t)s * stride + 8 * chunk, tile + 2 * i * TROW);
  }
}

// raw list entries of tile rows j0 .. j0 + 31 (lane j < 32; -1 past j_end).  The range check
// is left to valid_ix, applied only once the load has been drained with the tile's transfers:
// using the loaded value earlier would make the wave wait for the gathers issued before it.
__device__ __forceinline__ int load_ix(const int32_t* idx, int j0, int j_end, int lane) {
  const int j = j0 + lane;
  return (lane < KT && j < j_end) ? idx[j] : -1;
}

// the entry as a position, or -1 when it is skipped (negative or beyond the rows held)
__device__ __forceinline__ int valid_ix(int s, int S) { return (s >= 0 && s < S) ? s : -1; }

}  // namespace sparse_tile
}  // namespace lgsa
