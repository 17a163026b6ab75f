// dK and dV of document-masked causal GQA attention for one CP rank
// (key-stationary).
//
// For the gradients (chain rule of softmax attention, recomputing P from
// the saved log-sum-exp as the pages' FlashAttention discussion describes:
// "Training Infrastructure and Systems", "FlashAttention: never write the
// score matrix"):
//   P = exp(scale * q k^T - lse),  dS = P * (dO v^T - D),  D = <dO, O>
//   dV = sum over rows of P^T dO,  dK = scale * sum over rows of dS^T Q
// where the rows are the (token, query head) pairs of the KV head's group
// that may attend to the key (GQA: the group's heads share the key).
//
// Work item: 128 keys of one KV head (wave w owns keys t0 + 32w .. +31) x a
// slice of the query rows that reach them.  Rows are streamed through LDS in
// blocks of 64 (3 stages, filled by global->LDS DMA two blocks ahead) and
// processed in sub-blocks of 32.  Per sub-block and wave:
//   S_j = Q_j K^T and dP_j = dO_j V^T  (MFMA; the accumulators start from
//       -lse/scale and -D, so P = exp2(scale*log2e * S_j) and dS = P * dP_j
//       take one multiply each)
//   P, dS and their bf16 operands        (VALU, next to independent MFMAs)
//   dV += P^T dO_j, dK += dS^T Q_j       (MFMA, transposed LDS reads)
//
// P enters dV as a bf16 hi + lo pair (16 significant bits): dV sums P over
// every row of the group, and one bf16 rounding of P is not accurate enough
// for the fp32 result there.
//
// LDS stage layout (bytes): [Q tile][dO tile][-lse/scale: 64 fp32][-D: 64 fp32].
// A tile holds 64 rows x D bf16 in groups of 4 sixteen-byte chunks (32
// elements): group c/4 of row r occupies the 64 bytes at
// (c/4) * 4096 + 64 * r, and inside them chunk c sits in slot
// (c % 4) ^ ((r / 4) % 4).  On the 64 four-byte banks this makes both
// access patterns conflict-free:
//   - ds_read_b128 of one chunk by 16 consecutive rows: bank =
//     16*(r%4) + 4*slot, and the slot differs across the four row quads;
//   - ds_read_b64_tr_b16 (rows r..r+3 of a quad x 4 chunks of a group x two
//     8-byte halves, 32 lanes a cycle): 4 rows x 4 slots x 2 halves.
// A DMA instruction fills one chunk group of 16 rows (lane l: row 16w + l/4,
// slot l % 4): every lane loads 16 bytes of its row from a 64-byte run, and
// each lane keeps the same row for all of a block's instructions.
#include "common.hpp"
#include "dma.hpp"

#include <stdint.h>
#include "kernels.hpp"

namespace dmgqa {

namespace {

constexpr int kBlkRows = kDkdvBM;                    // 64 query rows per LDS stage
constexpr int kGroupBytes = kBlkRows * 64;           // one chunk group of a tile

template <int D>
struct DkdvLds {
  static constexpr int kChunks = D / 8;
  static constexpr int kTile = kChunks / 4 * kGroupBytes;
  static constexpr int kL = 2 * kTile;               // -lse/scale per row
  static constexpr int kN = kL + kBlkRows * 4;       // -D per row
  static constexpr int kStage = kN + kBlkRows * 4;
  static constexpr int kDmaPerWave = kChunks / 2 + 1;  // per block: Q, dO share + one row stat
};

typedef __attribute__((address_space(3))) char lds_char;

// global_load_lds_dword{,x4} issued as inline assembly: lane l's 4 / 16
// bytes at sbase + voff + IMM go to LDS address lds + size * l (sbase and
// lds wave-uniform, voff a 32-bit per-lane byte offset, so only one VGPR per
// lane carries the address).  The instruction's immediate offset is added to
// the LDS address too, so M0 is set to lds - IMM.  The compiler does not see these as LDS
// writes, so it adds no waits of its own for them (its conservative merge of
// in-flight DMA state at loop heads would otherwise wait for the block just
// issued); the kernel orders every read of a stage after an explicit vmcnt
// wait and a barrier instead.
template <int IMM>
__device__ __forceinline__ void dma_lds16(const void* sbase, unsigned voff, char* lds) {
  const unsigned m0 =
      __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(lds_char*)lds) - (unsigned)IMM;
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 offset:%3" ::"v"(voff),
               "s"(sbase), "s"(m0), "i"(IMM)
               : "memory");
}
__device__ __forceinline__ void dma_lds4(const void* sbase, unsigned voff, char* lds) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(lds_char*)lds);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase),
               "s"(m0)
               : "memory");
}

__device__ __forceinline__ bf16x8 ld_lds_b128(const char* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ f32x4 ld_lds_f32x4(const char* p) {
  return *reinterpret_cast<const f32x4*>(p);
}

// Operand for lane l = 32h + i holding column (32*db + i) of the rows that
// register slot (h, e) pairs with in k-step ks (see common.hpp), from a tile
// in the grouped layout above; lane_off[hf] is the per-lane part of the
// address of the rows 8*hf .. 8*hf+3 of the 16-row step.
__device__ __forceinline__ bf16x8 tr_group(const char* tile, const int (&lane_off)[2], int q0,
                                           int ks, int db) {
  const char* p = tile + db * kGroupBytes + (q0 + 16 * ks) * 64;
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

// Token ranges of the query rows that reach key tile kt (same rule as the
// scheduler): positions [t0, dend(last key of the tile)).
__device__ __forceinline__ void dkdv_ranges(const int32_t* dend_b, int kt, const Geo& g, int& a0,
                                            int& na, int& b0, int& nb) {
  const int t0 = kt * kDkdvBN;
  const int tl = min(t0 + kDkdvBN - 1, g.Skv - 1);
  const int p1 = dend_b[tl];
  const int baseA = g.rank * g.c;
  const int baseB = (2 * g.cp - 1 - g.rank) * g.c;
  const int la = min(max(t0 - baseA, 0), g.c), ha = min(max(p1 - baseA, 0), g.c);
  const int lb = min(max(t0 - baseB, 0), g.c), hb = min(max(p1 - baseB, 0), g.c);
  a0 = la; na = max(0, ha - la);
  b0 = g.c + lb; nb = max(0, hb - lb);
}

// STASH: also store dS (bf16) for the dQ product kernel.  Each wave's
// 32 rows x 32 keys of dS are transposed through LDS (written key-major,
// read with the transposed read) into 16-byte chunks of one row and 8 keys
// in the MFMA slot order; chunk (key group kq of 16, lane 32h + i) of a
// stash block holds row i of the block and keys 16kq + 8(e/4) + 4h + e%4,
// so the dQ kernel loads each operand with one 16-byte read per lane.
template <int D, bool STASH>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    const u16* __restrict__ dout, const float* __restrict__ Lbuf, const float* __restrict__ Nbuf,
    const int32_t* __restrict__ dend, SchedHeader* __restrict__ hdr,
    const int2* __restrict__ tile_info, const int2* __restrict__ items,
    const int4* __restrict__ tile_rows, u16* __restrict__ stash, int stash_kvh_blocks,
    float* __restrict__ partial, float* __restrict__ dk, float* __restrict__ dv, Geo g, int nkt) {
  using Lds = DkdvLds<D>;
  constexpr int BN = kDkdvBN, KK = D / 16, DB = D / 32, NCH = D / 8;
  __shared__ __attribute__((aligned(1024))) char st0[Lds::kStage];
  __shared__ __attribute__((aligned(1024))) char st1[Lds::kStage];
  __shared__ __attribute__((aligned(1024))) char st2[Lds::kStage];
  __shared__ int s_item;
  // per-wave transpose scratch of the dS stash: [32 keys][32 rows] bf16
  // row stride 36: the key-major writes and the transposed reads are both
  // spread over the 64 banks
  constexpr int kTrLd = 36;
  __shared__ __attribute__((aligned(16))) u16 s_tr[STASH ? 4 * 32 * kTrLd : 1];

  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int h = lane >> 5, i = lane & 31;
  const int total = hdr->n_base_items * g.Hkv;
  const int rps = hdr->rows_per_split;
  const size_t kvstride = (size_t)g.Hkv * D;
  const float c2 = g.scale_log2;

  // per-lane parts of the LDS addresses.  b128 operand (row i, chunk
  // h + 2kk): slot (h + 2(kk&1)) ^ (i/4 % 4) = slot of even kk, ^2 for odd.
  const int off_b[2] = {64 * i + 16 * (h ^ ((i >> 2) & 3)),
                        64 * i + 16 * ((h ^ ((i >> 2) & 3)) ^ 2)};
  // transposed operand: source lane s of 16-lane group grp reads row
  // 4h + s/4 (+8 for the second half), chunk 2(grp&1) + (s&3)/2 of the
  // group, 8-byte half s&1; the row quad index is h (+2).
  const int s16 = lane & 15, grp = lane >> 4;
  int off_t[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
    off_t[hf] = (4 * h + (s16 >> 2) + 8 * hf) * 64 +
                16 * ((2 * (grp & 1) + ((s16 & 3) >> 1)) ^ ((h + 2 * hf) & 3)) + 8 * (s16 & 1);

  for (;;) {
    if (threadIdx.x == 0) s_item = atomicAdd(&hdr->counter, 1);
    __syncthreads();
    const int it = uniform(s_item);
    __syncthreads();
    if (it >= total) break;
    const int base = it / g.Hkv, kvh = it % g.Hkv;
    const int2 itm = items[base];
    const int x = itm.x, split = itm.y;
    const int b = x / nkt, kt = x % nkt;
    const int t0 = kt * BN;
    const int32_t* de = dend + (size_t)b * g.Skv;
    int a0, na, b0, nb;
    dkdv_ranges(de, kt, g, a0, na, b0, nb);
    const int rows_total = (na + nb) * g.G;
    const int r_begin = split * rps;
    const int r_end = min(r_begin + rps, rows_total);
    const int nsb = r_end > r_begin ? (r_end - r_begin + 31) / 32 : 0;
    const int nblk = (nsb + 1) / 2;

    // this lane's key and its K / V operands
    const int key = t0 + wave * 32 + i;
    const int kc = min(key, g.Skv - 1);
    const u16* krow = k + ((size_t)b * g.Skv + kc) * kvstride + (size_t)kvh * D;
    const u16* vrow = v + ((size_t)b * g.Skv + kc) * kvstride + (size_t)kvh * D;
    bf16x8 kop[KK], vop[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      kop[kk] = ld_bf16x8(krow + 8 * h + 16 * kk);
      vop[kk] = ld_bf16x8(vrow + 8 * h + 16 * kk);
    }

    // Rows allowed for this key: local tokens with position in
    // [key, dend(key)), a contiguous run [ti_lo, ti_hi) of the tile's token
    // list (run A then run B, positions increasing), i.e. virtual rows
    // [G*ti_lo, G*ti_hi), clipped to the item's rows.  Both ends grow with
    // the key, so the wave's common range is [lo of its last key, hi of its
    // first key).
    int vr_lo = r_end, vr_hi = r_end;
    {
      const int A = g.rank * g.c + a0;
      const int Bb = (2 * g.cp - 1 - g.rank) * g.c + (b0 - g.c);
      if (key < g.Skv) {
        const int e = de[key];
        const int ti_lo = min(max(key - A, 0), na) + min(max(key - Bb, 0), nb);
        const int ti_hi = min(max(e - A, 0), na) + min(max(e - Bb, 0), nb);
        vr_lo = min(max(ti_lo * g.G, r_begin), r_end);
        vr_hi = min(max(ti_hi * g.G, r_begin), r_end);
      }
    }
    const int w_lo = __builtin_amdgcn_readlane(vr_lo, 31);
    const int w_hi = __builtin_amdgcn_readlane(vr_hi, 0);

    f32x16 dka[DB], dva[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) { dka[db] = zero16(); dva[db] = zero16(); }

    // Row bookkeeping of the next block to load: virtual row nx_vr0 =
    // nx_ti * G + nx_hh (uniform), advanced by kBlkRows per block.  Every
    // block boundary issues the same number of DMA instructions: rows past
    // the item's end (including whole blocks past it) re-load its last row,
    // into a stage that is not read again.  The fixed count lets every wait
    // be a plain vmcnt of one block's instructions.
    int nx_ti = r_begin / g.G;
    int nx_hh = r_begin - nx_ti * g.G;
    const int step_ti = kBlkRows / g.G, step_hh = kBlkRows - step_ti * g.G;
    const int last_ti = (r_end - 1) / g.G, last_hh = (r_end - 1) - last_ti * g.G;
    int nx_blk = 0;
    auto row_index = [&](int r) __attribute__((always_inline)) -> unsigned {
      const bool ok = r_begin + nx_blk * kBlkRows + r < r_end;
      const int t = nx_hh + r;
      const int qd = div_small(t, g);
      const int ti = ok ? nx_ti + qd : last_ti;
      const int hh = ok ? t - qd * g.G : last_hh;
      const int tok = ti < na ? a0 + ti : b0 + (ti - na);
      return (unsigned)((b * g.Sq + tok) * g.Hq + kvh * g.G + hh);
    };
    auto issue_block = [&](char* st) __attribute__((always_inline)) {
      // tiles: wave w fills rows 16w .. 16w+15 of every chunk group
      const int rr = 16 * wave + (lane >> 2);
      const unsigned ridx = row_index(rr);
      const int slot = lane & 3, xr = (rr >> 2) & 3;
      // byte offset of the row's chunk (q and dout share the layout; both
      // stay below 4 GiB, which the host checks)
      const unsigned qoff = (ridx * (unsigned)D + 8 * (slot ^ xr)) * 2u;
      char* tq = st + 64 * 16 * wave;
      static_for<NCH / 4>([&](auto c) __attribute__((always_inline)) {
        dma_lds16<64 * decltype(c)::value>(q, qoff, tq + decltype(c)::value * kGroupBytes);
        dma_lds16<64 * decltype(c)::value>(dout, qoff,
                                           tq + Lds::kTile + decltype(c)::value * kGroupBytes);
      });
      // row statistics: lane = row (waves 0, 2: -lse/scale; 1, 3: -D)
      const unsigned ridm = row_index(lane);
      if (wave & 1)
        dma_lds4(Nbuf, ridm * 4u, st + Lds::kN);
      else
        dma_lds4(Lbuf, ridm * 4u, st + Lds::kL);
      ++nx_blk;
      nx_ti += step_ti;
      nx_hh += step_hh;
      if (nx_hh >= g.G) { nx_hh -= g.G; ++nx_ti; }
    };

    // dS stash of this item's tile: virtual row vr is query row tlo*G + vr
    // of the KV head (the tile's rows are the contiguous local tokens
    // [tlo, thi)); block b of the tile covers rows [32(J_lo + b), +32).
    // Stores go through a buffer resource spanning exactly the tile's
    // blocks: a lane whose row lies past the item's end gets an offset
    // beyond that range, which the hardware drops (no divergent branch).
    const int4 trow = tile_rows[x];
    const int tr_z = uniform(trow.z), tr_x = uniform(trow.x);
    const int tile_blocks = uniform((trow.y * g.G + kStashRows - 1) / kStashRows - trow.z);
    __amdgpu_buffer_rsrc_t srs;
    if constexpr (STASH)
      srs = __builtin_amdgcn_make_buffer_rsrc(
          stash + ((size_t)kvh * stash_kvh_blocks + uniform(trow.w)) * (kStashBlockBytes / 2), 0,
          tile_blocks * kStashBlockBytes, 0x00020000);
    // (1) dS to this wave's transpose scratch, key-major: lane (h, i) holds
    // key i at rows 16ks + 4h + 0..3 and 16ks + 8 + 4h + 0..3.
    auto stash_put = [&](const bf16x8 (&dsop)[2]) __attribute__((always_inline)) {
      u16* T = s_tr + wave * 32 * kTrLd;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x4 w = __builtin_bit_cast(u32x4, dsop[ks]);
        *reinterpret_cast<uint2*>(T + i * kTrLd + 16 * ks + 4 * h) = uint2{w[0], w[1]};
        *reinterpret_cast<uint2*>(T + i * kTrLd + 16 * ks + 8 + 4 * h) = uint2{w[2], w[3]};
      }
    };
    // (2) transposed read: lane (h, i) gets row i, keys 16kq + 8(e/4) + 4h +
    // e%4, stored as chunk (2*wave + kq, lane) of the row's stash block.
    // Done after the sub-block's products, when its operands are dead.
    auto stash_store = [&](int R) __attribute__((always_inline)) {
      const u16* T = s_tr + wave * 32 * kTrLd;
      const int grow = tr_x * g.G + R + i;
      const unsigned off = R + i < r_end ? (unsigned)(((grow >> 5) - tr_z) * kStashBlockBytes +
                                                      (32 * h + (grow & 31)) * 16 + wave * 2048)
                                         : 0x80000000u;
#pragma unroll
      for (int kq = 0; kq < 2; ++kq) {
        const bf16x8 op = tr_operand_pad<kTrLd>(T, 0, kq, 0, lane);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, op), srs, off + kq * 1024,
                                               0, 0);
      }
    };

    // One sub-block of 32 rows (rows q0.. of stage st, virtual rows from R).
    // Program order puts vector work next to matrix work it does not depend
    // on: P = exp2(..) and its operands while the dP chain runs, dS and its
    // operand while the dV products run.
    auto body = [&](auto masked, const char* st, int q0, int R) __attribute__((always_inline)) {
      // keeps the compiler from hoisting the loads both variants share above
      // the branch that picks the variant (which would make them all live at once)
      if constexpr (decltype(masked)::value)
        asm volatile("; masked sub-block" ::: "memory");
      else
        asm volatile("; full sub-block" ::: "memory");
      f32x16 sc, pc;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 l4 = ld_lds_f32x4(st + Lds::kL + 4 * (q0 + 8 * r4 + 4 * h));
        const f32x4 n4 = ld_lds_f32x4(st + Lds::kN + 4 * (q0 + 8 * r4 + 4 * h));
#pragma unroll
        for (int e = 0; e < 4; ++e) { sc[4 * r4 + e] = l4[e]; pc[4 * r4 + e] = n4[e]; }
      }
      // Each phase's LDS operands are read up front and the phases are fenced
      // (sched_barrier), so the reads are in flight while the previous
      // phase's products run instead of one read before each product.
      bf16x8 qa[KK], oa[KK];
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        qa[kk] = ld_lds_b128(st + (kk >> 1) * kGroupBytes + 64 * q0 + off_b[kk & 1]);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        oa[kk] = ld_lds_b128(st + Lds::kTile + (kk >> 1) * kGroupBytes + 64 * q0 + off_b[kk & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) sc = mfma32(qa[kk], kop[kk], sc);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) pc = mfma32(oa[kk], vop[kk], pc);

      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(sc[r] * c2);
      if constexpr (decltype(masked)::value) {
        // register r holds virtual row R + 4h + cr, cr = 8*(r/4) + r%4
        const int lo_rel = vr_lo - R - 4 * h;
        const unsigned span = (unsigned)max(vr_hi - vr_lo, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int cr = 8 * (r >> 2) + (r & 3);
          if ((unsigned)(cr - lo_rel) >= span) p[r] = 0.f;
        }
      }
      // hi = bf16(P) (round to nearest even, one conversion per pair), lo =
      // bf16(P - hi), with hi widened back to fp32 by a shift / mask
      bf16x8 pop[2], plo[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = p[8 * ks + e], p1 = p[8 * ks + e + 1];
          const bf16x2 hp = {(__bf16)p0, (__bf16)p1};
          const unsigned hw = __builtin_bit_cast(unsigned, hp);
          const float h0 = __builtin_bit_cast(float, hw << 16);
          const float h1 = __builtin_bit_cast(float, hw & 0xffff0000u);
          pop[ks][e] = hp[0];
          pop[ks][e + 1] = hp[1];
          plo[ks][e] = (__bf16)(p0 - h0);
          plo[ks][e + 1] = (__bf16)(p1 - h1);
        }
      const char* tQ = st;
      const char* tO = st + Lds::kTile;
      bf16x8 dot[2][DB];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int db = 0; db < DB; ++db) dot[ks][db] = tr_group(tO, off_t, q0, ks, db);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          dva[db] = mfma32(pop[ks], dot[ks][db], dva[db]);
          dva[db] = mfma32(plo[ks], dot[ks][db], dva[db]);
        }
      bf16x8 dsop[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) dsop[ks][e] = (__bf16)(p[8 * ks + e] * pc[8 * ks + e]);
      if constexpr (STASH) stash_put(dsop);
      bf16x8 qt[2][DB];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int db = 0; db < DB; ++db) qt[ks][db] = tr_group(tQ, off_t, q0, ks, db);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int db = 0; db < DB; ++db)
          dka[db] = mfma32(dsop[ks], qt[ks][db], dka[db]);
      if constexpr (STASH) stash_store(R);
    };

    // The first sub-block of block n waits for its DMA (issued two blocks
    // earlier; only block n+1's may still be in flight), then - past the
    // barrier, which also retires every read of block n-1 - starts the DMA
    // of block n+2 into block n-1's stage.  K/V operands and the key bounds
    // must have arrived before the DMA stream starts, so that no wait inside
    // the loop has to count them.
    wait_vmcnt<0>();
    if (nblk > 0) {
      issue_block(st0);
      issue_block(st1);
    }
    int j = 0;
    auto step = [&](const char* st, int q0, char* dst, auto first) __attribute__((always_inline)) {
      if constexpr (decltype(first)::value) {
        wait_vmcnt<Lds::kDmaPerWave>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        issue_block(dst);
      }
      const int R = r_begin + 32 * j;
      if (w_lo <= R && R + 32 <= w_hi)
        body(std::false_type{}, st, q0, R);
      else
        body(std::true_type{}, st, q0, R);
      ++j;
    };
    while (j < nsb) {
      step(st0, 0, st2, std::true_type{});
      if (j >= nsb) break;
      step(st0, 32, st2, std::false_type{});
      if (j >= nsb) break;
      step(st1, 0, st0, std::true_type{});
      if (j >= nsb) break;
      step(st1, 32, st0, std::false_type{});
      if (j >= nsb) break;
      step(st2, 0, st1, std::true_type{});
      if (j >= nsb) break;
      step(st2, 32, st1, std::false_type{});
    }

    // No DMA (including the re-loads past the item's end) may still be
    // writing LDS once the item is done.
    wait_vmcnt<0>();

    // Write this wave's 32 keys: directly (dK scaled) if the tile was not
    // split, else to the item's partial-sum slot.
    const int2 info = tile_info[x];
    const bool split_tile = info.x > 1;
    float* dst_k;
    float* dst_v;
    size_t rstride;
    if (split_tile) {
      const size_t slot = (size_t)(info.y + split) * g.Hkv + kvh;
      dst_k = partial + slot * 2 * BN * D;
      dst_v = dst_k + BN * D;
      rstride = D;
    } else {
      dst_k = dk + ((size_t)b * g.Skv + t0) * kvstride + (size_t)kvh * D;
      dst_v = dv + ((size_t)b * g.Skv + t0) * kvstride + (size_t)kvh * D;
      rstride = kvstride;
    }
    const float kscale = split_tile ? 1.f : g.scale;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kvloc = wave * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (split_tile || t0 + kvloc < g.Skv) {
          dst_k[(size_t)kvloc * rstride + 32 * db + i] = dka[db][r] * kscale;
          dst_v[(size_t)kvloc * rstride + 32 * db + i] = dva[db][r];
        }
      }
  }
}

hipError_t launch_bwd_dkdv(int D, const u16* q, const u16* k, const u16* v, const u16* dout,
                           const float* Lbuf, const float* Nbuf, const int32_t* dend,
                           SchedHeader* hdr, const int2* tile_info, const int2* items,
                           const int4* tile_rows, u16* stash, int stash_kvh_blocks,
                           float* partial, float* dk, float* dv, const Geo& g, int nkt,
                           hipStream_t st) {
#define DMGQA_DKDV(DD, SS)                                                                   \
  bwd_dkdv_kernel<DD, SS><<<kDkdvGrid, 256, 0, st>>>(q, k, v, dout, Lbuf, Nbuf, dend, hdr,   \
                                                     tile_info, items, tile_rows, stash,     \
                                                     stash_kvh_blocks, partial, dk, dv, g, nkt)
  if (D == 128) {
    if (stash) DMGQA_DKDV(128, true); else DMGQA_DKDV(128, false);
  } else {
    if (stash) DMGQA_DKDV(64, true); else DMGQA_DKDV(64, false);
  }
#undef DMGQA_DKDV
  return hipGetLastError();
}

}  // namespace dmgqa
