// Tile geometry of the gfx950 prefill kernel (prefill_mfma.hip): the LDS
// chunk swizzle of K and V tiles, the split of a 64-key tile into 1 KB blocks
// over the waves, and the softmax modes of a key tile.
#pragma once

#include "common.h"

namespace pva {

enum TileMode : int { kFirst = 0, kPlain = 1, kMasked = 2, kSafe = 3 };

// LDS chunk swizzle: 16-byte chunk c of key row r is stored at chunk
// c ^ chunk_perm<D>(r). gfx950's LDS serves 64 banks of 4 bytes per clock, so
// a 128-dim bf16 row (256 bytes) spans the banks exactly once and a 64-dim row
// half of them. The permutation makes both access patterns of the kernel
// conflict-free: 16 consecutive rows at one logical chunk (the K fragment
// reads) and 4 consecutive rows x 4 consecutive chunks (the transpose reads
// of V).
template <int D>
__host__ __device__ constexpr int chunk_perm(int r) {
  if constexpr (D == 128) {
    return 4 * (r & 3) + ((r >> 2) & 3);
  } else {
    return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
  }
}

// Tile geometry of one operand with rows of W 16-bit elements: a wave's 1 KB
// load covers 512 / W key rows, a 64-key tile splits into 1 KB blocks dealt
// round-robin to the NW waves.
template <int W, int NW>
struct TileShape {
  static constexpr int BN = 64;
  static constexpr int CH = W / 8;               // 16-byte chunks per key row
  static constexpr int TILE = BN * W;            // 16-bit elements per tile
  static constexpr int ROWS_PER_BLOCK = 512 / W;
  static constexpr int BLOCKS = BN / ROWS_PER_BLOCK;
  static constexpr int BPW = BLOCKS / NW;        // 1 KB blocks per wave per tile
  static_assert(BLOCKS % NW == 0, "tile blocks must split evenly over the waves");
};

}  // namespace pva
