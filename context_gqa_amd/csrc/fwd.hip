// Forward kernel: document-masked causal GQA attention for one CP rank.
//
// Method ("Training Infrastructure and Systems", "FlashAttention: never write
// the score matrix", sections "Online softmax" and "Tiling"): a workgroup
// keeps a tile of query rows in registers and walks the key/value tiles its
// rows can reach, never writing scores to HBM.  Per key tile it forms the
// raw scores with MFMA, masks them only when the tile is partial, updates the
// running row maximum m and sum l with the rescaling factor
// exp(scale*(m_old - m_new)), rescales the running output by the same factor
// and adds P V.  At the end it writes out = O / l and lse = scale*m + ln l.
//
// Layout on gfx950: 4 waves x 32 query rows, two workgroups per CU; rows
// are (token, head-in-group) pairs of one KV head, so one K/V tile in LDS
// serves all G query heads sharing it (GQA).
// Scores are held as S^T = K Q^T so that each lane owns one query row (two
// lanes per row, 16 keys each): the row max and sum need one cross-lane
// exchange.  P V is computed as O^T = V^T P^T with V read from LDS by
// transposed reads.
//
// K/V tiles (64 keys) stream through 2 LDS stages, filled by global->LDS
// DMA one tile ahead.  A tile holds 64 rows x D bf16 in groups
// of 4 sixteen-byte chunks: group c/4 of row r occupies the 64 bytes at
// (c/4) * 4096 + 64 * r, chunk c in slot (c % 4) ^ ((r / 4) % 4), so the
// 128-bit reads of K (32 rows of one chunk per 32-lane half) and the
// transposed reads of V (4 rows x 4 slots x 2 halves) are conflict-free on
// the 64 banks, and a DMA instruction moves 64 contiguous bytes of 16 rows.
#include "common.hpp"
#include "kernels.hpp"
#include "dma.hpp"

namespace dmgqa {

namespace {

constexpr int kRows = kFwdBM;             // query rows per workgroup
constexpr int kWaves = kRows / 32;
constexpr int kGroupBytes = kFwdBN * 64;  // one chunk group of a 64-row tile

typedef __attribute__((address_space(3))) char lds_char;

// Lazy rescaling: the running maximum used as the exponent reference is only
// raised when a row's new maximum exceeds it by more than 2^kRescaleLog2 (in
// exp2 units); otherwise P may reach 2^kRescaleLog2, which bf16 and fp32
// represent exactly as well as values below 1.  out = O / l is unchanged.
constexpr float kRescaleLog2 = 8.f;

// global_load_lds_dwordx4 as inline assembly: lane l's 16 bytes at
// sbase + voff + IMM go to LDS address lds + 16 * l (sbase, lds
// wave-uniform; voff a 32-bit per-lane byte offset).  The immediate offset
// moves the LDS address too, so M0 is lds - IMM.  Written as assembly so the
// compiler adds no waits of its own for these LDS writes; every read of a
// stage follows an explicit vmcnt wait and a barrier.
template <int IMM>
__device__ __forceinline__ void dma_lds16(const void* sbase, unsigned voff, unsigned lds) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds) - (unsigned)IMM;
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 offset:%3" ::"v"(voff),
               "s"(sbase), "s"(m0), "i"(IMM)
               : "memory");
}

// The value of lane l ^ 32 (the other half of the wave), by
// v_permlane32_swap on two copies: it moves lanes 0-31 of the second
// register into lanes 32-63 of the first and lanes 32-63 of the first into
// lanes 0-31 of the second.  Written as assembly on two distinct operands,
// with wait states around it (measured on gfx950: without them, lanes 32-63
// of the first register read a stale value; the compiler builtin, given the
// same value twice, returned the first result for both).  No LDS round trip,
// unlike a shuffle through ds_bpermute.
__device__ __forceinline__ float other_half(float x) {
  float a = x, b = x;
  asm volatile("s_nop 4\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 4" : "+v"(a), "+v"(b));
  // lanes 0-31: a = own, b = lane + 32; lanes 32-63: a = lane - 32, b = own
  return (threadIdx.x & 32) ? a : b;
}

__device__ __forceinline__ bf16x8 ld_lds_b128(const char* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// MFMA operand holding, for lane l = 32h + i, column 32*db + i of the tile
// rows that register slot (h, e) pairs with in k-step ks (rows 16ks +
// 8(e/4) + 4h + e%4), from a tile in the grouped layout; lane_off[hf] is the
// per-lane part of the address of rows 8*hf .. 8*hf+3 of the 16-row step.
__device__ __forceinline__ bf16x8 tr_group(const char* tile, const int (&lane_off)[2], int ks,
                                           int db) {
  const char* p = tile + db * kGroupBytes + 16 * ks * 64;
  const i16x4 lo = ds_read_tr(reinterpret_cast<const u16*>(p + lane_off[0]));
  const i16x4 hi = ds_read_tr(reinterpret_cast<const u16*>(p + lane_off[1]));
  const bf16x4 a = __builtin_bit_cast(bf16x4, lo);
  const bf16x4 b = __builtin_bit_cast(bf16x4, hi);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

}  // namespace

// CROSS: interval masks with explicit ends -- row p reaches keys dstart[p]
// .. dhi[p]-1 (both [B, S], indexed by query position, keys indexed on
// their own); otherwise keys dstart[p] .. p with dstart [B, Skv].
template <int D, bool CROSS>
__global__ __launch_bounds__(kRows * 2, 2) void fwd_kernel(const u16* __restrict__ q,
                                                          const u16* __restrict__ k,
                                                          const u16* __restrict__ v,
                                                          const int32_t* __restrict__ dstart,
                                                          const int32_t* __restrict__ dhi,
                                                          const int32_t* __restrict__ order,
                                                          u16* __restrict__ out,
                                                          float* __restrict__ lse, Geo g) {
  constexpr int BM = kRows, BN = kFwdBN, KK = D / 16, DB = D / 32;
  constexpr int kTile = D / 32 * kGroupBytes;   // bytes of a K (or V) tile
  constexpr int kStage = 2 * kTile;
  __shared__ __attribute__((aligned(1024))) char stg[2 * kStage];
  // LDS byte address of stg (the cast to the LDS address space checks for
  // null, so it is taken once; DMA addresses are offsets from it)
  const unsigned stg_lds = (unsigned)(uintptr_t)(lds_char*)stg;

  const int nrows = g.Sq * g.G;
  const int nt = (nrows + BM - 1) / BM;
  // (batch row, tile) items in the heaviest-first order, the KV heads of an
  // item consecutively (clamped: the order is a permutation of 0 .. B*nt-1)
  const int item = min(max(order[blockIdx.x / g.Hkv], 0), g.B * nt - 1);
  const int b = item / nt, tile = item - b * nt;
  const int kvh = blockIdx.x % g.Hkv;
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int h = lane >> 5, i = lane & 31;

  const int row0 = tile * BM;
  const int row = row0 + wave * 32 + i;
  const bool valid = row < nrows;
  const int rr = valid ? row : nrows - 1;
  const int tok = rr / g.G;
  const int head = kvh * g.G + rr % g.G;
  const int pos = local_pos(tok, g.c, g.cp, g.rank);
  const int32_t* ds = dstart + (size_t)b * (CROSS ? g.S : g.Skv);
  const int32_t* dh = CROSS ? dhi + (size_t)b * g.S : nullptr;
  const int lo = ds[pos];
  // last key this row reaches
  const int last = CROSS ? dh[pos] - 1 : pos;

  const size_t qoff = (((size_t)b * g.Sq + tok) * g.Hq + head) * D;
  bf16x8 qop[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) qop[kk] = ld_bf16x8(q + qoff + 8 * h + 16 * kk);

  const QTileKeys kr =
      CROSS ? qtile_keys_iv<BM, BN>(row0, ds, dh, g) : qtile_keys<BM, BN>(row0, ds, g);
  const int ntiles = kr.na + kr.nb;

  float m = -INFINITY, l = 0.f;
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = zero16();

  // K operand (A of S^T = K Q^T): lane (h, i) reads row i (and 32 + i),
  // chunk h + 2kk: slot (h + 2(kk&1)) ^ (i/4 % 4).
  const int off_b[2] = {64 * i + 16 * (h ^ ((i >> 2) & 3)),
                        64 * i + 16 * ((h ^ ((i >> 2) & 3)) ^ 2)};
  // V operand (transposed reads): source lane s of 16-lane group grp reads
  // row 4h + s/4 (+8 for the second half), chunk 2(grp&1) + (s&3)/2 of the
  // group, 8-byte half s&1; the row quad index is h (+2).
  const int s16 = lane & 15, grp = lane >> 4;
  int off_t[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
    off_t[hf] = (4 * h + (s16 >> 2) + 8 * hf) * 64 +
                16 * ((2 * (grp & 1) + ((s16 & 3) >> 1)) ^ ((h + 2 * hf) & 3)) + 8 * (s16 & 1);

  // DMA: wave w fills rows 16(w%4) .. +15 of chunk groups w/4 + 2m of the K
  // and V tiles (lane l: row 16(w%4) + l/4, slot l%4).  Every tile index
  // past the last re-loads the last tile, so each wave issues the same
  // number of instructions per tile and every wait is a plain vmcnt.
  const size_t kvstride = (size_t)g.Hkv * D;
  const u16* kbase = k + (size_t)b * g.Skv * kvstride + (size_t)kvh * D;
  const u16* vbase = v + (size_t)b * g.Skv * kvstride + (size_t)kvh * D;
  const int drow = 16 * wave + (lane >> 2);
  const unsigned coff = 8 * ((lane & 3) ^ ((drow >> 2) & 3));
  auto tile_start = [&](int it) __attribute__((always_inline)) {
    const int x = min(it, ntiles - 1);
    return uniform((x < kr.na ? kr.a0 + x : kr.b0 + (x - kr.na)) * BN);
  };
  // byte offset of this lane's row chunk from the batch / head base (K and
  // V share the layout; the host keeps each tensor below 2^31 elements)
  auto dma_off = [&](int it) __attribute__((always_inline)) {
    const int key = max(min(tile_start(it) + drow, g.Skv - 1), 0);
    return ((unsigned)key * (unsigned)kvstride + coff) * 2u;
  };
  auto issue_k = [&](unsigned off, char* st) __attribute__((always_inline)) {
    static_for<D / 32>([&](auto cc) __attribute__((always_inline)) {
      constexpr int C = decltype(cc)::value;
      dma_lds16<64 * C>(kbase, off,
                        stg_lds + (unsigned)(st - stg) + 64 * 16 * wave + C * kGroupBytes);
    });
  };
  auto issue_v = [&](unsigned off, char* st) __attribute__((always_inline)) {
    static_for<D / 32>([&](auto cc) __attribute__((always_inline)) {
      constexpr int C = decltype(cc)::value;
      dma_lds16<64 * C>(vbase, off,
                        stg_lds + (unsigned)(st - stg) + kTile + 64 * 16 * wave + C * kGroupBytes);
    });
  };

  auto step = [&](int it, const char* cK, auto&& mid) __attribute__((always_inline)) {
    const char* cV = cK + kTile;
    const int t0 = tile_start(it);
    // K operands for all k-steps are read up front (2*KK LDS reads in
    // flight), so LDS latency overlaps the MFMA chain.
    bf16x8 kf0[KK], kf1[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      kf0[kk] = ld_lds_b128(cK + (kk >> 1) * kGroupBytes + off_b[kk & 1]);
      kf1[kk] = ld_lds_b128(cK + (kk >> 1) * kGroupBytes + 32 * 64 + off_b[kk & 1]);
    }
    f32x16 s0 = zero16(), s1 = zero16();
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      s0 = mfma32(kf0[kk], qop[kk], s0);
      s1 = mfma32(kf1[kk], qop[kk], s1);
    }
    sched_reads_ahead<2 * KK, KK, 2>();
    // the next tile's V DMA, while the score products run
    mid();
    const bool full = qtile_full(kr, t0, BN);
    if (!full) {
      // allowed keys lo..last relative to this lane's first key t0 + 4h;
      // register r holds key offset 8*(r/4) + r%4 (+32 for s1)
      // key offset c is allowed iff lo_rel <= c <= hi_rel, one unsigned
      // compare (hi_rel >= lo_rel: a row always reaches at least one key)
      const int lo_rel = lo - (t0 + 4 * h);
      const unsigned span = (unsigned)(last - lo);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = 8 * (r >> 2) + (r & 3);
        if ((unsigned)(c - lo_rel) > span) s0[r] = -INFINITY;
        if ((unsigned)(c + 32 - lo_rel) > span) s1[r] = -INFINITY;
      }
    }
    // row maximum: two independent max3 chains, then the other half-wave
    float ma = max3f(s0[0], s0[1], s0[2]), mb = max3f(s1[0], s1[1], s1[2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) {
      ma = max3f(ma, s0[r], s0[r + 1]);
      mb = max3f(mb, s1[r], s1[r + 1]);
    }
    float mx = max3f(ma, mb, fmaxf(s0[15], s1[15]));
    mx = fmaxf(mx, other_half(mx));
    const bool need = mx != -INFINITY && (m == -INFINITY || (mx - m) * g.scale_log2 > kRescaleLog2);
    if (__any(need)) {
      const float mnew = need ? mx : m;
      const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m - mnew) * g.scale_log2);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      m = mnew;
    }
    const float msc = m == -INFINITY ? 0.f : m * g.scale_log2;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = __builtin_amdgcn_exp2f(fmaf(s0[r], g.scale_log2, -msc));
      s1[r] = __builtin_amdgcn_exp2f(fmaf(s1[r], g.scale_log2, -msc));
    }
    // the row sum is taken over the bf16 P that multiplies V
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int ks = 0; ks < BN / 16; ++ks) {
      const bf16x8 pop = pack_bf16(ks < 2 ? s0 : s1, ks & 1);
      float& rs = (ks & 1) ? rs1 : rs0;
#pragma unroll
      for (int e = 0; e < 8; e += 2) rs = sum2_bf16(bf16x2{pop[e], pop[e + 1]}, rs);
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] = mfma32(tr_group(cV, off_t, ks, db), pop, o[db]);
    }
    l += rs0 + rs1;
  };

  // Two stages: before tile it, wait for its DMA, barrier (every wave's
  // DMA of tile it is in, and every wave has finished tile it-1, whose
  // stage is refilled next), start tile it+1's K DMA, compute (tile it+1's
  // V DMA is issued once the score products are under way).
  if (ntiles > 0) {
    char* sA = stg;
    char* sB = stg + kStage;
    {
      const unsigned off0 = dma_off(0);
      issue_k(off0, sA);
      issue_v(off0, sA);
    }
    for (int it = 0; it < ntiles; ++it) {
      wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const bool more = it + 1 < ntiles;
      const unsigned offn = dma_off(it + 1);
      if (more) issue_k(offn, sB);
      step(it, sA, [&]() __attribute__((always_inline)) {
        if (more) issue_v(offn, sB);
      });
      char* t = sA;
      sA = sB;
      sB = t;
    }
  }

  const float lt = l + other_half(l);
  if (valid) {
    const float inv = 1.f / lt;
    u16* orow = out + qoff;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[db][4 * r4 + e] * inv);
        *reinterpret_cast<uint2*>(orow + 32 * db + 8 * r4 + 4 * h) = __builtin_bit_cast(uint2, w);
      }
    if (h == 0) lse[((size_t)b * g.Sq + tok) * g.Hq + head] = m * g.scale + logf(lt);
  }
}

hipError_t launch_fwd(int D, const u16* q, const u16* k, const u16* v, const int32_t* dstart,
                      const int32_t* dhi, const int32_t* order, u16* out, float* lse,
                      const Geo& g, hipStream_t st) {
  const int nt = (g.Sq * g.G + kRows - 1) / kRows;
  const unsigned grid = (unsigned)nt * g.B * g.Hkv;
#define DMGQA_FWD(DD, CC) \
  fwd_kernel<DD, CC><<<grid, kWaves * 64, 0, st>>>(q, k, v, dstart, dhi, order, out, lse, g)
  if (D == 128) {
    if (dhi) DMGQA_FWD(128, true); else DMGQA_FWD(128, false);
  } else {
    if (dhi) DMGQA_FWD(64, true); else DMGQA_FWD(64, false);
  }
#undef DMGQA_FWD
  return hipGetLastError();
}

}  // namespace dmgqa
