// Cooperative global -> register -> LDS copies of row tiles, split in two
// halves so the global loads of the next tile can be issued before the
// current tile is computed (software pipelining with double-buffered LDS).
#pragma once
#include "common.hpp"

namespace dmgqa {

// A [ROWS x D] bf16 tile copied by NT threads, 16 bytes per thread per step.
template <int ROWS, int D, int NT>
struct TileRegs {
  static constexpr int kChunks = ROWS * (D / 8);
  static constexpr int kPer = (kChunks + NT - 1) / NT;
  static_assert(kChunks % NT == 0, "tile must split evenly over the threads");
  u32x4 r[kPer];

  // rowptr(row) -> pointer to the row's first element in global memory
  template <class RowPtr>
  __device__ __forceinline__ void load(RowPtr rowptr) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int x = threadIdx.x + j * NT;
      const int row = x / (D / 8), col = (x % (D / 8)) * 8;
      r[j] = *reinterpret_cast<const u32x4*>(rowptr(row) + col);
    }
  }
  // into a swizzled LDS tile (see swz)
  __device__ __forceinline__ void store(u16* lds) const {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int x = threadIdx.x + j * NT;
      const int row = x / (D / 8), col = (x % (D / 8)) * 8;
      *reinterpret_cast<u32x4*>(lds + swz<D>(row, col)) = r[j];
    }
  }
};

}  // namespace dmgqa
