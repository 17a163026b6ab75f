// Direct global -> LDS tile loads (global_load_lds_dwordx4, gfx950).
//
// One instruction moves 16 bytes per lane and writes lane l's bytes at
// (wave-uniform LDS address) + 16*l, so a wave fills a contiguous 1 KiB of
// LDS while each lane picks its global address freely.  For a swizzled tile
// (see swz) LDS chunk slot x = row*(D/8) + p holds logical chunk p ^ f(row)
// of that row, so the lane writing slot x fetches exactly that chunk.
//
// The loads count against vmcnt.  Callers wait with an explicit
// s_waitcnt vmcnt(..) and s_barrier (not __syncthreads, whose workgroup
// fence would drain every outstanding load), and keep each ring stage in
// its own __shared__ array so the compiler can tell a stage being filled
// from the stage being read.
#pragma once
#include "common.hpp"

namespace dmgqa {

__device__ __forceinline__ void dma16(const void* g, u16* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base,
                                   16, 0, 0);
}

// s_waitcnt vmcnt(n) with expcnt / lgkmcnt left unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Swizzle function of swz<D>, as an XOR on the chunk index.
template <int D>
__device__ __forceinline__ int swz_f(int row) {
  return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3))
                  : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}

// Loader of a [ROWS x D] bf16 tile whose rows are `stride` elements apart in
// global memory, by NW waves.  Element offsets within one tensor slice are
// 32-bit (the host checks that they fit), so the address is a wave-uniform
// 64-bit base plus a 32-bit per-lane offset.
template <int ROWS, int D, int NW>
struct TileDma {
  static constexpr int kChunksPerRow = D / 8;
  static constexpr int kInstr = ROWS * kChunksPerRow / 64;   // per tile
  static constexpr int kPerWave = kInstr / NW;
  static_assert(kInstr % NW == 0, "tile must split evenly over the waves");

  // rows first_row + r of `base` (clamped to max_row) into LDS tile `lds`
  __device__ __forceinline__ static void issue(const u16* base, unsigned stride, int first_row,
                                               int max_row, u16* lds, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < kPerWave; ++j) {
      const int x = (wave * kPerWave + j) * 64 + lane;
      const int row = x / kChunksPerRow;
      const int col = ((x % kChunksPerRow) ^ swz_f<D>(row)) * 8;
      const unsigned r = (unsigned)min(first_row + row, max_row);
      dma16(base + (r * stride + (unsigned)col), lds + (wave * kPerWave + j) * 512);
    }
  }
};

// Loader of a [ROWS x D] bf16 tile into a padded row-major LDS tile with row
// stride LDS_LD elements (LDS_LD % 8 == 0, LDS_LD >= D).  LDS chunk slot
// x = row * (LDS_LD/8) + p holds chunk p of the row; lanes writing padding
// slots (p >= D/8) fetch a duplicate of an in-bounds chunk instead of being
// masked off.  Per-lane offsets are computed once; per tile only the
// wave-uniform base moves, and rows are clamped (per lane) only for a tile
// that runs past the last valid row.
template <int ROWS, int D, int LDS_LD, int NW>
struct PadTileDma {
  static constexpr int kChunksPerRow = D / 8;
  static constexpr int kSlotsPerRow = LDS_LD / 8;
  static constexpr int kInstr = (ROWS * kSlotsPerRow + 63) / 64;
  static constexpr int kPerWave = (kInstr + NW - 1) / NW;
  static_assert(ROWS * kSlotsPerRow % 64 == 0, "whole instructions must fill the LDS tile");
  int row[kPerWave];     // tile row of this lane's slot (clamped into the tile)
  unsigned off[kPerWave];  // element offset of its chunk within the row block

  __device__ __forceinline__ void init(unsigned stride, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < kPerWave; ++j) {
      const int x = (j * NW + wave) * 64 + lane;
      const int r = min(x / kSlotsPerRow, ROWS - 1);
      const int p = (x % kSlotsPerRow) % kChunksPerRow;
      row[j] = r;
      off[j] = (unsigned)r * stride + (unsigned)(p * 8);
    }
  }
  // rows first_row .. first_row + ROWS - 1 of `base` (rows > max_row are
  // clamped to max_row) into LDS tile `lds`
  __device__ __forceinline__ void issue(const u16* base, unsigned stride, int first_row,
                                        int max_row, u16* lds, int wave, int lane) const {
    const u16* tb = base + (size_t)first_row * stride;
    if (first_row + ROWS - 1 <= max_row) {
#pragma unroll
      for (int j = 0; j < kPerWave; ++j)
        if (j * NW + wave < kInstr) dma16(tb + off[j], lds + (j * NW + wave) * 512);
    } else {
#pragma unroll
      for (int j = 0; j < kPerWave; ++j) {
        if (j * NW + wave < kInstr) {
          const int dr = min(first_row + row[j], max_row) - (first_row + row[j]);
          dma16(tb + off[j] + (int)(dr * (int)stride), lds + (j * NW + wave) * 512);
        }
      }
    }
  }
};

}  // namespace dmgqa
