// Tile geometry of the gfx950 prefill kernel (prefill_mfma.hip): the LDS
// layout of K and V tiles, their split into 1 KB load blocks over the waves,
// and the softmax modes of a key tile.
#pragma once

#include "common.h"

namespace pva {

enum TileMode : int { kFirst = 0, kPlain = 1, kMasked = 2, kSafe = 3, kFirstOpen = 4 };

// LDS layout of a 64-key tile whose rows hold W 16-bit elements (CH = W / 8
// chunks of 16 bytes). One global_load_lds instruction fills one 1 KB block
// of RB = 64 / CH rows, lane L landing in 16-byte slot L of the block. Inside
// a block the slots run over chunk quads, then rows, then the chunk within
// its quad: chunk c of the block's row r sits in slot
// (c / 4) * 4 * RB + 4 * r + ((c % 4) ^ g(r)), and blocks lie BSLOTS = 64 + PAD
// slots apart. Then
//  * each quad of lanes of a load fetches 64 contiguous bytes of one key row,
//    so the loads coalesce as well as row-major ones;
//  * the element offset of (row, chunk) is a per-lane base plus a constant
//    for every fragment the kernel reads (the 32-row and 16-row steps are
//    whole blocks, and g and the chunk steps leave each other alone), so
//    reads take immediate offsets and no address arithmetic per tile;
//  * gfx950's LDS serves 64 banks of 4 bytes per clock, and both read
//    patterns of the kernel are conflict-free: 16 consecutive rows at one
//    chunk (the 16-byte K fragment reads, 16 lanes per clock) and 4 rows x
//    4 chunks in 8-byte halves (the V transpose reads, 32 lanes per clock).
//    The rows of one block differ in their 4 * r, the blocks in their
//    padding shift, and for 8-row blocks g(r) separates rows r and r + 4.
// The properties are checked at compile time below.
template <int W>
struct TileLayout {
  static constexpr int BN = 64;
  static constexpr int CH = W / 8;
  static constexpr int RB = 64 / CH;            // rows per 1 KB block
  static constexpr int PAD = RB == 4 ? 1 : 2;   // padding slots per block
  static constexpr int BSLOTS = 64 + PAD;
  static constexpr int BLOCKS = BN / RB;
  static constexpr int BLOCK_ELEMS = BSLOTS * 8;
  static constexpr int TILE = BLOCKS * BLOCK_ELEMS;  // 16-bit elements per tile
  __host__ __device__ static constexpr int g(int r) { return RB == 8 ? (r >> 2) & 1 : 0; }
  __host__ __device__ static constexpr int slot(int row, int c) {
    const int r = row % RB;
    return (row / RB) * BSLOTS + (c / 4) * 4 * RB + 4 * r + ((c % 4) ^ g(r));
  }
  __host__ __device__ static constexpr int elem(int row, int c) { return slot(row, c) * 8; }
  // The (row, chunk) that lane L of the load of block b fetches.
  __host__ __device__ static constexpr int load_row(int b, int lane) { return b * RB + (lane / 4) % RB; }
  __host__ __device__ static constexpr int load_chunk(int lane) {
    return (lane / (4 * RB)) * 4 + ((lane % 4) ^ g((lane / 4) % RB));
  }
};

namespace tile_check {

template <class L>
constexpr bool layout_is_a_bijection_and_loads_are_contiguous() {
  bool seen[L::BLOCKS * L::BSLOTS] = {};
  for (int r = 0; r < L::BN; ++r) {
    for (int c = 0; c < L::CH; ++c) {
      const int s = L::slot(r, c);
      if (s < 0 || s >= L::BLOCKS * L::BSLOTS || s % L::BSLOTS >= 64 || seen[s]) return false;
      seen[s] = true;
    }
  }
  for (int b = 0; b < L::BLOCKS; ++b) {
    for (int lane = 0; lane < 64; ++lane) {
      if (L::slot(L::load_row(b, lane), L::load_chunk(lane)) != b * L::BSLOTS + lane) return false;
      // a lane quad reads the four chunks of one aligned 64-byte piece of a row
      const int q0 = lane & ~3;
      if (L::load_row(b, lane) != L::load_row(b, q0) || L::load_chunk(lane) / 4 != L::load_chunk(q0) / 4) return false;
    }
  }
  return true;
}

// K fragment reads: lane (l32, half) reads row 32*mt + l32, chunk 2*kk + half,
// 16 bytes; each group of 16 lanes must cover the 16 bank groups once.
template <class L>
constexpr bool k_reads_conflict_free() {
  for (int mt = 0; mt < 2; ++mt) {
    for (int c0 = 0; c0 < L::CH; c0 += 2) {
      for (int g = 0; g < 4; ++g) {
        bool used[16] = {};
        for (int i = 0; i < 16; ++i) {
          const int lane = 16 * g + i;
          const int row = 32 * mt + (lane & 31);
          const int bg = L::slot(row, c0 + (lane >> 5)) % 16;
          if (used[bg]) return false;
          used[bg] = true;
        }
      }
    }
  }
  return true;
}

// V transpose reads: lane with group G = lane / 16 and i = lane % 16 reads 8
// bytes of key row 16*kb + 8*h + 4*(G/2) + i/4 at head dims
// 32*mb + 16*(G%2) + 4*(i%4) .. +3; each half-wave must cover the 64 banks once.
template <class L>
constexpr bool v_reads_conflict_free() {
  for (int kb = 0; kb < L::BN / 16; ++kb) {
    for (int h = 0; h < 2; ++h) {
      for (int mb = 0; mb < L::CH / 4; ++mb) {
        for (int half = 0; half < 2; ++half) {
          bool used[64] = {};
          for (int j = 0; j < 32; ++j) {
            const int lane = 32 * half + j;
            const int grp = lane >> 4, i = lane & 15;
            const int row = 16 * kb + 8 * h + 4 * (grp >> 1) + (i >> 2);
            const int d = 32 * mb + 16 * (grp & 1) + 4 * (i & 3);
            const int byte = L::elem(row, d >> 3) * 2 + (d & 7) * 2;
            for (int w = 0; w < 2; ++w) {
              const int bank = (byte / 4 + w) % 64;
              if (used[bank]) return false;
              used[bank] = true;
            }
          }
        }
      }
    }
  }
  return true;
}

// The kernel reads every fragment at a per-lane base plus a constant: K at
// elem(l32, half) + (elem(32 mt, 2 kk) - elem(0, 0)), V at
// elem(key, chunk) + (elem(16 kb + 8 h, 4 mb) - elem(0, 0)) for the lane's
// key < 8 and chunk < 4 of the first block pair.
template <class L>
constexpr bool fragment_offsets_are_lane_constant() {
  for (int lane = 0; lane < 64; ++lane) {
    const int l32 = lane & 31, half = lane >> 5;
    for (int mt = 0; mt < 2; ++mt) {
      for (int kk = 0; kk < L::CH / 2; ++kk) {
        if (L::elem(32 * mt + l32, 2 * kk + half) != L::elem(l32, half) + L::elem(32 * mt, 2 * kk) - L::elem(0, 0))
          return false;
      }
    }
    const int grp = lane >> 4, i = lane & 15;
    const int key = 4 * (grp >> 1) + (i >> 2), chunk = (16 * (grp & 1) + 4 * (i & 3)) >> 3;
    for (int kb = 0; kb < L::BN / 16; ++kb) {
      for (int h = 0; h < 2; ++h) {
        for (int mb = 0; mb < L::CH / 4; ++mb) {
          if (L::elem(16 * kb + 8 * h + key, 4 * mb + chunk) !=
              L::elem(key, chunk) + L::elem(16 * kb + 8 * h, 4 * mb) - L::elem(0, 0))
            return false;
        }
      }
    }
  }
  return true;
}

static_assert(layout_is_a_bijection_and_loads_are_contiguous<TileLayout<128>>(), "layout, 128");
static_assert(layout_is_a_bijection_and_loads_are_contiguous<TileLayout<64>>(), "layout, 64");
static_assert(k_reads_conflict_free<TileLayout<128>>(), "K reads, 128");
static_assert(k_reads_conflict_free<TileLayout<64>>(), "K reads, 64");
static_assert(v_reads_conflict_free<TileLayout<128>>(), "V reads, 128");
static_assert(v_reads_conflict_free<TileLayout<64>>(), "V reads, 64");
static_assert(fragment_offsets_are_lane_constant<TileLayout<128>>(), "fragment offsets, 128");
static_assert(fragment_offsets_are_lane_constant<TileLayout<64>>(), "fragment offsets, 64");

}  // namespace tile_check

}  // namespace pva
