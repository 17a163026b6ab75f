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
// The loop is software-pipelined across key tiles: tile j+1's score
// products are issued while tile j's exponentials run (each vector
// instruction placed right after an MFMA executes in its shadow, measured on
// gfx950: up to about one MFMA's 32 cycles of vector work per MFMA is
// free), and tile j+1's row maximum is taken while tile j's P V products
// run.  What is left between two tiles is the barrier, the mask of a
// partial tile and the reference update.
//
// K/V tiles (64 keys) stream through 2 LDS stages, filled by global->LDS
// DMA (K two tiles ahead, V one).  A tile holds 64 rows x D bf16 in groups
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

  // ---- software pipeline: tile j's softmax under tile j+1's score products
  //
  // Iteration j holds S_j = K_j Q^T (computed in iteration j-1) and:
  //   1. masks S_j (partial tiles), takes the row maximum, moves the
  //      reference m (and rescales O and l) when needed;
  //   2. issues the 16 products S_{j+1} = K_{j+1} Q^T, each followed by a
  //      share of the exponentials of S_j, so the vector work runs while the
  //      matrix pipe is busy with the next tile (within one wave the vector
  //      instructions after an MFMA execute in its shadow);
  //   3. issues the 16 products O += P_j V_j, with the packing and row sums
  //      that remain and the row maximum of S_{j+1} in their shadow.
  // Stage s holds K and V tiles of 64 keys.  K_j and V_j live in stage j%2.
  // Iteration j starts with a barrier (every wave has finished iteration
  // j-1, so S_j's K reads and P_{j-1} V_{j-1}'s V reads are done); after it
  // the DMA loads K_{j+2} into stage j%2 and V_{j+1} into stage (j+1)%2,
  // which the barrier of iteration j+1 waits for.
  auto k_op = [&](const char* cK, int kk, int half) __attribute__((always_inline)) {
    return ld_lds_b128(cK + (kk >> 1) * kGroupBytes + 32 * 64 * half + off_b[kk & 1]);
  };
  // S = K Q^T of one tile with nothing interleaved (the first tile)
  auto s_plain = [&](const char* cK, f32x16& s0, f32x16& s1) __attribute__((always_inline)) {
    bf16x8 kf0[KK], kf1[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      kf0[kk] = k_op(cK, kk, 0);
      kf1[kk] = k_op(cK, kk, 1);
    }
    s0 = zero16();
    s1 = zero16();
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      s0 = mfma32(kf0[kk], qop[kk], s0);
      s1 = mfma32(kf1[kk], qop[kk], s1);
    }
  };
  // The row maximum of an unmasked tile (both lanes of a row combined).
  auto row_max = [&](const f32x16& s0, const f32x16& s1) __attribute__((always_inline)) {
    float ma = max3f(s0[0], s0[1], s0[2]), mb = max3f(s1[0], s1[1], s1[2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) {
      ma = max3f(ma, s0[r], s0[r + 1]);
      mb = max3f(mb, s1[r], s1[r + 1]);
    }
    const float mx = max3f(ma, mb, fmaxf(s0[15], s1[15]));
    return fmaxf(mx, other_half(mx));
  };
  // Step 1 for tile j (first key t0): mask, maximum, reference.  Returns the
  // exponent offset m * scale * log2(e) (0 while m is -inf).  mx_pre: the
  // row maximum of S_j taken during the previous iteration's P V products
  // (have_pre), valid when the tile needs no mask.
  auto prepare = [&](int t0, f32x16& s0, f32x16& s1, float mx_pre, bool have_pre)
                     __attribute__((always_inline)) {
    const bool full = qtile_full(kr, t0, BN);
    float mx = mx_pre;
    if (!full || !have_pre) {
      if (!full) {
        // allowed keys lo..last relative to this lane's first key t0 + 4h;
        // register r holds key offset 8*(r/4) + r%4 (+32 for s1); key
        // offset c is allowed iff lo_rel <= c <= hi_rel, one unsigned
        // compare (a row always reaches at least one key, so hi_rel >= lo_rel)
        const int lo_rel = lo - (t0 + 4 * h);
        const unsigned span = (unsigned)(last - lo);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = 8 * (r >> 2) + (r & 3);
          if ((unsigned)(c - lo_rel) > span) s0[r] = -INFINITY;
          if ((unsigned)(c + 32 - lo_rel) > span) s1[r] = -INFINITY;
        }
      }
      mx = row_max(s0, s1);
    }
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
    return m == -INFINITY ? 0.f : m * g.scale_log2;
  };
  // Steps 2 and 3 as NS + NP slots, each one MFMA and its share of the
  // vector work, fenced so the compiler keeps the order: slots 0 .. NS-1
  // the products of S_{j+1} (NEXT) and the exponentials of S_j, VPS values
  // per slot (value v is s0[v] for v < 16, else s1[v-16]); P_j in bf16 as
  // four k-step operands, each packed one slot after its last exponential,
  // its row sum one slot later; slots NS .. NS+NP-1 the products P_j V_j.
  // Operands are read two slots ahead of their MFMA.
  constexpr int NS = 2 * KK, NP = (BN / 16) * DB, VPS = 32 / NS;
  constexpr int kPackSlot[4] = {(7) / VPS + 1, (15) / VPS + 1, (23) / VPS + 1, (31) / VPS + 1};
  // With NEXT the slots also issue the DMA of V_{j+1} (into stage sn) and
  // K_{j+2} (into stage sj; past the last tile it re-loads the last one,
  // into a stage no later iteration reads), one instruction every other
  // slot: issued in one burst after the barrier, the eight waves of a CU
  // stalled on the vector memory queue.
  constexpr int NDMA = D / 32;   // DMA instructions per tile and wave
  // first slot of the next tile's row maximum (two slots after its last
  // score product; nine steps, kMaxPer per slot)
  constexpr int kMaxSlot = NS + 2;
  constexpr int kMaxPer = (9 + (NS + NP - kMaxSlot) - 1) / (NS + NP - kMaxSlot);
  // slots of the first V and K DMA instructions (then every other slot)
  constexpr int kDmaV = 1, kDmaK = 1 + 2 * NDMA;
  static_assert(kDmaV + 2 * NDMA <= NS + NP && kDmaK + 2 * NDMA <= NS + NP, "DMA slots");
  auto pipelined = [&](auto next_c, const char* cKn, const char* cV, float msc, f32x16& s0,
                       f32x16& s1, f32x16& n0, f32x16& n1, unsigned offV, unsigned offK,
                       const char* sj, const char* sn, float& mx_next)
                       __attribute__((always_inline)) {
    constexpr bool NEXT = decltype(next_c)::value;
    bf16x8 kb[3], vb[3], pop[4];
    float rs0 = 0.f, rs1 = 0.f;
    float ma = 0.f, mb = 0.f;
    auto read_for = [&](auto slot_c) __attribute__((always_inline)) {
      constexpr int S = decltype(slot_c)::value;
      if constexpr (S < NS) {
        if constexpr (NEXT) kb[S % 3] = k_op(cKn, S >> 1, S & 1);
      } else if constexpr (S < NS + NP) {
        constexpr int P = S - NS;
        vb[P % 3] = tr_group(cV, off_t, P / DB, P % DB);
      }
    };
    if constexpr (NEXT) {
      n0 = zero16();
      n1 = zero16();
    }
    read_for(std::integral_constant<int, 0>{});
    read_for(std::integral_constant<int, 1>{});
    static_for<NS + NP>([&](auto slot_c) __attribute__((always_inline)) {
      constexpr int S = decltype(slot_c)::value;
      read_for(std::integral_constant<int, S + 2>{});
      if constexpr (S < NS) {
        if constexpr (NEXT) {
          if constexpr ((S & 1) == 0)
            n0 = mfma32(kb[S % 3], qop[S >> 1], n0);
          else
            n1 = mfma32(kb[S % 3], qop[S >> 1], n1);
        }
        static_for<VPS>([&](auto e_c) __attribute__((always_inline)) {
          constexpr int V = VPS * S + decltype(e_c)::value;
          if constexpr (V < 16)
            s0[V] = __builtin_amdgcn_exp2f(fmaf(s0[V], g.scale_log2, -msc));
          else
            s1[V - 16] = __builtin_amdgcn_exp2f(fmaf(s1[V - 16], g.scale_log2, -msc));
        });
      } else {
        constexpr int P = S - NS;
        o[P % DB] = mfma32(vb[P % 3], pop[P / DB], o[P % DB]);
      }
      if constexpr (NEXT && S >= kDmaV && S < kDmaV + 2 * NDMA && (S - kDmaV) % 2 == 0) {
        constexpr int C = (S - kDmaV) / 2;
        dma_lds16<64 * C>(vbase, offV,
                          stg_lds + (unsigned)(sn - stg) + kTile + 64 * 16 * wave + C * kGroupBytes);
      }
      if constexpr (NEXT && S >= kDmaK && S < kDmaK + 2 * NDMA && (S - kDmaK) % 2 == 0) {
        constexpr int C = (S - kDmaK) / 2;
        dma_lds16<64 * C>(kbase, offK,
                          stg_lds + (unsigned)(sj - stg) + 64 * 16 * wave + C * kGroupBytes);
      }
      static_for<4>([&](auto q_c) __attribute__((always_inline)) {
        constexpr int Q = decltype(q_c)::value;
        if constexpr (S == kPackSlot[Q]) pop[Q] = pack_bf16(Q < 2 ? s0 : s1, Q & 1);
        if constexpr (S == kPackSlot[Q] + 1) {
          float& rs = (Q & 1) ? rs1 : rs0;
#pragma unroll
          for (int e = 0; e < 8; e += 2) rs = sum2_bf16(bf16x2{pop[Q][e], pop[Q][e + 1]}, rs);
        }
      });
      if constexpr (S == kPackSlot[3] + 2) l += rs0 + rs1;
      // NEXT: the row maximum of S_{j+1} (complete after the score
      // products), one step per slot from slot kMaxSlot on
      if constexpr (NEXT && S >= kMaxSlot) {
        static_for<kMaxPer>([&](auto t_c) __attribute__((always_inline)) {
          constexpr int T = (S - kMaxSlot) * kMaxPer + decltype(t_c)::value;
          if constexpr (T == 0) {
            ma = max3f(n0[0], n0[1], n0[2]);
            mb = max3f(n1[0], n1[1], n1[2]);
          } else if constexpr (T < 7) {
            ma = max3f(ma, n0[2 * T + 1], n0[2 * T + 2]);
            mb = max3f(mb, n1[2 * T + 1], n1[2 * T + 2]);
          } else if constexpr (T == 7) {
            ma = max3f(ma, mb, fmaxf(n0[15], n1[15]));
          } else if constexpr (T == 8) {
            mx_next = fmaxf(ma, other_half(ma));
          }
        });
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  static_assert(kPackSlot[3] + 2 < NS + NP, "row sums inside the slots");
  static_assert(kMaxPer * (NS + NP - kMaxSlot) >= 9, "row maximum inside the slots");
  // operand Q of P_j is first used by P V product Q * DB (slot NS + Q * DB)
  static_assert(kPackSlot[0] <= NS && kPackSlot[1] <= NS + DB && kPackSlot[2] <= NS + 2 * DB &&
                    kPackSlot[3] <= NS + 3 * DB,
                "each P operand packed before its first P V product");

  if (ntiles > 0) {
    // prologue: K_0, V_0 into stage 0 and K_1 into stage 1; S_0
    {
      const unsigned off0 = dma_off(0);
      issue_k(off0, stg);
      issue_v(off0, stg);
      if (ntiles > 1) issue_k(dma_off(1), stg + kStage);
    }
    f32x16 sa0, sa1, sb0, sb1;
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    s_plain(stg, sa0, sa1);
    // iteration j: S_j in (c0, c1), S_{j+1} into (n0, n1) unless j is the
    // last tile (NEXT false; the last tile is peeled off the loop so that
    // the two forms never share a branch, out of which the compiler would
    // hoist their common exponentials)
    float mx_pre = 0.f;
    auto iteration = [&](auto next_c, int j, f32x16& c0, f32x16& c1, f32x16& n0, f32x16& n1)
                         __attribute__((always_inline)) {
      wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      char* sj = stg + (j & 1) * kStage;
      char* sn = stg + ((j + 1) & 1) * kStage;
      unsigned offV = 0, offK = 0;
      if constexpr (decltype(next_c)::value) {
        offV = dma_off(j + 1);
        offK = dma_off(j + 2);
      }
      const float msc = prepare(tile_start(j), c0, c1, mx_pre, j > 0);
      pipelined(next_c, sn, sj + kTile, msc, c0, c1, n0, n1, offV, offK, sj, sn, mx_pre);
    };
    int j = 0;
    for (; j + 2 < ntiles; j += 2) {
      iteration(std::true_type{}, j, sa0, sa1, sb0, sb1);
      iteration(std::true_type{}, j + 1, sb0, sb1, sa0, sa1);
    }
    // one or two tiles left, S_j in sa
    if (j + 1 < ntiles) {
      iteration(std::true_type{}, j, sa0, sa1, sb0, sb1);
      iteration(std::false_type{}, j + 1, sb0, sb1, sa0, sa1);
    } else {
      iteration(std::false_type{}, j, sa0, sa1, sb0, sb1);
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
