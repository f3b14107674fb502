// Geometry shared by every kernel of libpa and its host layer: the cache
// block, the head dimension and its 16-byte chunks, the 64-token tile.
#pragma once

namespace pa {

constexpr int kBlock = 256;      // tokens per cache block
constexpr int kDim = 128;        // head dim
constexpr int kChunks = kDim / 8;  // 16-byte chunks per row
constexpr int kTile = 64;        // decode tile: one token per lane

}  // namespace pa
