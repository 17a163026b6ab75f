// Shared device helpers for the gfx950 document-masked GQA attention kernels.
//
// MFMA conventions used throughout (v_mfma_f32_32x32x16_bf16, wave64):
//   lane l = 32*h + i  (h = l/32 in {0,1}, i = l%32)
//   A operand [32 x 16]: lane l holds A[m = i][k = 8h .. 8h+7]
//   B operand [16 x 32]: lane l holds B[k = 8h .. 8h+7][n = i]
//   C/D [32 x 32] fp32:  lane l, register r holds C[m = 8(r/4) + 4h + r%4][n = i]
// A kernel keeps the score tile as S^T (kv along m, queries along n) so each
// lane owns one query row; the 16 registers then hold 16 key columns of that
// row.  Feeding those registers back as the B operand of the next product
// (P^T, dS^T) pairs register slot (h, e) of a 16-wide k-step ks with key
// index 16*ks + 8*(e/4) + 4*h + e%4; the other operand is read from LDS in the
// same key order with ds_read_b64_tr_b16 (see tr_operand below).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

#include "index.hpp"

namespace dmgqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;

// Cache-policy operand of the buffer load / store builtins: the
// non-temporal bit (streaming data that is not reused soon).
constexpr int kCachePolicyNT = 2;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

// 16-byte global load of 8 bf16.
__device__ __forceinline__ bf16x8 ld_bf16x8(const u16* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

// 16-byte LDS load of 8 bf16.
__device__ __forceinline__ bf16x8 lds_bf16x8(const u16* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

// ds_read_b64_tr_b16: within each group of 16 lanes, result lane j element e
// is element (j % 4) of the 4 bf16 that source lane 4*e + j/4 addresses.
// So if source lane s (s = lane % 16) points at row (k0 + s/4), column
// (n0 + 4*(s%4)) of a row-major tile, lane j receives rows k0..k0+3 of column
// n0 + j: four consecutive k values of one column.
__device__ __forceinline__ i16x4 ds_read_tr(const u16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
}

// LDS tiles are row-major with D bf16 per row (no padding) and the 16-byte
// chunks of each row permuted by an XOR with a function f(row).  Measured on
// gfx950 (SQ_LDS_BANK_CONFLICT), the LDS serves these reads as 64 four-byte
// banks; f is chosen so that both access patterns of the kernels are
// conflict-free:
//  - ds_read_b128 of one chunk from 16 consecutive rows (16 lanes a cycle);
//  - ds_read_b64_tr_b16 of 4 adjacent chunks (the first a multiple of 4) from
//    4 consecutive rows starting at a multiple of 4 (32 lanes a cycle).
// D = 128 (256-byte rows, one bank line): f = 4*(row%4) + (row/4)%4 takes 16
// distinct values on 16 consecutive rows, and f/4 differs on the 4 rows of a
// transposed read, so their 4-chunk blocks land in different banks.
// D = 64 (128-byte rows, half a bank line; row parity picks the half):
// f = 4*((row/2)%2) + (row/4)%4 gives 8 distinct values per parity on 16
// rows, and rows r, r+2 of a transposed read differ in bit 2 of f.
template <int D>
__device__ __forceinline__ int swz(int row, int col) {
  static_assert(D == 64 || D == 128, "head dim");
  const int f = D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3))
                         : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
  return row * D + ((((col >> 3) ^ f) << 3) | (col & 7));
}

// MFMA operand holding, for lane l = 32*h + i, column (n0 + i) of a swizzled
// row-major bf16 LDS tile `base` at the 8 rows that register slot (h, e)
// pairs with in k-step ks:
//   row = row0 + 16*ks + 8*(e/4) + 4*h + e%4.
// Two transposed reads, each giving four consecutive rows.
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const u16* base, int row0, int ks, int n0,
                                             int lane) {
  const int s = lane & 15;
  const int grp = lane >> 4;        // 0..3
  const int h = grp >> 1;
  const int col = n0 + 16 * (grp & 1) + 4 * (s & 3);
  const int row = row0 + 16 * ks + 4 * h + (s >> 2);
  i16x4 lo = ds_read_tr(base + swz<D>(row, col));
  i16x4 hi = ds_read_tr(base + swz<D>(row + 8, col));
  bf16x8 r;
  bf16x4 a = __builtin_bit_cast(bf16x4, lo);
  bf16x4 b = __builtin_bit_cast(bf16x4, hi);
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// Registers 8*(ks%2) .. 8*(ks%2)+7 of an S^T-shaped accumulator as a bf16
// MFMA operand (round to nearest even).
__device__ __forceinline__ bf16x8 pack_bf16(const f32x16& acc, int half) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)acc[8 * half + e];
  return r;
}

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

// max(a, b, c) as one v_max3_f32.  Written as an instruction so the compiler
// does not add NaN-quieting copies of MFMA results before each max (scores
// are finite or -inf here).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// acc + x0 + x1 for a bf16 pair, one v_dot2_f32_bf16 against (1, 1).
__device__ __forceinline__ float sum2_bf16(bf16x2 x, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(x, one, acc, false);
}

// x / G and x % G (x >= 0); shifts when G is a power of two.
__device__ __forceinline__ int div_g(int x, const Geo& g) {
  return g.g_log2 >= 0 ? (x >> g.g_log2) : x / g.G;
}
__device__ __forceinline__ int mod_g(int x, const Geo& g) {
  return g.g_log2 >= 0 ? (x & (g.G - 1)) : x % g.G;
}

// t / G for 0 <= t < 2^16 (and G < 2^16): with M = ceil(2^32/G) = (2^32+e)/G,
// 0 <= e < G, t*M / 2^32 = t/G + t*e/(G*2^32) and t*e < 2^32, so the excess
// never reaches the next multiple of 1/G and the high word is floor(t/G).
__device__ __forceinline__ int div_small(int t, const Geo& g) {
  return g.G == 1 ? t : (int)__umulhi((unsigned)t, g.g_magic);
}

// f(std::integral_constant<int, I>{}) for I = 0 .. N-1, unrolled at compile
// time (for operands that must be immediates).
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// A value the caller knows is the same in every lane, as a scalar.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

}  // namespace dmgqa
