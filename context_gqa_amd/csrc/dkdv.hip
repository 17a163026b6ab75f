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
// Work item: 128 keys of one KV head x a slice of the query rows that reach
// them.  Eight waves (two per SIMD, so one wave's vector work runs under the
// other's matrix work) each own 16 keys, t0 + 16w .. +15, and use
// 16x16x32 MFMAs.  Rows are streamed through LDS in blocks of 64 (a ring of
// 4 stages, filled by global->LDS DMA two blocks ahead, the DMA
// instructions spread over the sub-blocks) and processed in sub-blocks of
// 32.  Per sub-block and wave:
//   S = Q K^T and dP' = dO' V'^T   (MFMA; the accumulators start from
//       -lse/scale and -D' = -D * 2^(eo+ev), so P = exp2(scale*log2e * S)
//       and dS' = P * dP' take one multiply each)
//   P (fp16), dS' (bf16)           (VALU)
//   dV' += P^T dO', dK += dS'^T Q  (MFMA, transposed LDS reads)
// Each LDS operand read is issued a fixed number of products ahead of the
// MFMA that consumes it, through a small ring of registers, in program order
// (scheduling fences: left to itself the compiler placed each read just
// before its product, and every MFMA waited out the LDS latency); dS' is
// formed under the dV products, and the previous sub-block's stash read and
// store bracket the score products.
//
// Lane layout (lane l = 16*g4 + j): the S / dP tiles are C[row][key] with
// key = j; lane group g4 holds the rows 16t + 4*g4 + r (t = 0, 1, r = 0..3).
// Those 8 values are the A operand (P^T, dS^T: key j, k-slot 8*g4 + e <->
// row 16(e/4) + 4*g4 + e%4) of the dV / dK products with no data movement.
//
// dP' and dV' are fp16 products: dV sums P over every row of the group, and
// one bf16 rounding of P (8 significant bits) is not accurate enough for the
// fp32 result there; fp16 carries 11.  dO and V enter as dO' = dO * 2^eo (in
// fp16 from the row-statistics pass) and V' = V * 2^ev (converted per work
// item), exact power-of-two scales chosen per call so that fp16's exponent
// range holds them (the exponent scan in prep.hip); dK, dV and the dS stash
// are scaled back exactly at the end.
//
// LDS stage layout (bytes): [Q tile][dO' tile][-lse/scale: 64 fp32][-D': 64 fp32].
// A tile holds 64 rows x D bf16 in groups of 4 sixteen-byte chunks (32
// elements): group c/4 of row r occupies the 64 bytes at
// (c/4) * 4096 + 64 * r, and inside them chunk c sits in slot
// (c % 4) ^ f(r), f(r) = 2 * ((r / 4) % 2).  Both read patterns of the
// kernel are conflict-free with this f (SQ_LDS_BANK_CONFLICT 0, measured
// over the 256 slot functions linear in the row's low four bits):
//   - ds_read_b128 of the S / dP operands: each 16-lane group reads one
//     chunk of 16 consecutive rows, the four groups four chunks;
//   - ds_read_b64_tr_b16 of the dV / dK operands: each 16-lane group reads
//     4 rows of a quad x 2 chunks x two 8-byte halves.
// (The earlier f(r) = (r / 4) % 4 left the first pattern 2-way
// conflicting.)
// A DMA instruction fills one chunk group of 16 rows (lane l: row
// 16*(w%4) + l/4, slot l % 4): every lane loads 16 bytes of its row from a
// 64-byte run, and each lane keeps the same row for all of a block's
// instructions.
#include "common.hpp"
#include "dma.hpp"

#include <stdint.h>
#include "kernels.hpp"

namespace dmgqa {

namespace {

constexpr int kBlkRows = kDkdvBM;                    // 64 query rows per LDS stage
constexpr int kGroupBytes = kBlkRows * 64;           // one chunk group of a tile
constexpr int kWaves = 8;
constexpr int kWaveKeys = kDkdvBN / kWaves;          // 16 keys per wave

template <int D>
struct DkdvLds {
  static constexpr int kChunks = D / 8;
  static constexpr int kTile = kChunks / 4 * kGroupBytes;
  static constexpr int kL = 2 * kTile;               // -lse/scale per row
  static constexpr int kN = kL + kBlkRows * 4;       // -D per row
  static constexpr int kStage = kN + kBlkRows * 4;
  // DMA instructions per block and wave: D/64 chunk groups each of Q and
  // dO, and one row-statistics load (16 lanes)
  static constexpr int kDmaPerWave = 2 * (D / 64) + 1;
};

typedef __attribute__((address_space(3))) char lds_char;

// global_load_lds_dword{,x4} issued as inline assembly: lane l's 4 / 16
// bytes at sbase + voff + IMM go to LDS address lds + size * l (sbase and
// lds wave-uniform, voff a 32-bit per-lane byte offset, so only one VGPR per
// lane carries the address).  The instruction's immediate offset is added to
// the LDS address too, so M0 is set to lds - IMM.  The compiler does not see
// these as LDS writes, so it adds no waits of its own for them (its
// conservative merge of in-flight DMA state at loop heads would otherwise
// wait for the block just issued); the kernel orders every read of a stage
// after an explicit vmcnt wait and a barrier instead.
template <int IMM>
__device__ __forceinline__ void dma_lds16(const void* sbase, unsigned voff, unsigned lds) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds) - (unsigned)IMM;
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 offset:%3" ::"v"(voff),
               "s"(sbase), "s"(m0), "i"(IMM)
               : "memory");
}
__device__ __forceinline__ void dma_lds4(const void* sbase, unsigned voff, unsigned lds) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds);
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

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// The same product with fp16 operands (the bits of the bf16-typed registers
// that hold them reinterpreted).
__device__ __forceinline__ f32x4 mfma16h(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                               __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// B operand of 32 rows x 16 columns from a tile in the grouped layout: two
// transposed reads, at p (rows 4*g4 + 0..3 of the sub-block) and 16 rows
// further.
__device__ __forceinline__ bf16x8 tr_pair(const char* p) {
  const i16x4 lo = ds_read_tr(reinterpret_cast<const u16*>(p));
  const i16x4 hi = ds_read_tr(reinterpret_cast<const u16*>(p + 16 * 64));
  const bf16x4 a = __builtin_bit_cast(bf16x4, lo);
  const bf16x4 b = __builtin_bit_cast(bf16x4, hi);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

}  // namespace

// STASH: also store dS (bf16) for the dQ product kernel.  Each wave's
// 32 rows x 16 keys of dS are transposed through LDS (written key-major,
// read with the transposed read) into one 16-byte chunk per lane: chunk
// (key group w, lane 32h + i) of a stash block holds row i of the block and
// keys 16w + 8(e/4) + 4h + e%4, so the dQ kernel loads each operand with
// one 16-byte read per lane.
template <int D, bool STASH>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    const u16* __restrict__ dout16, const float* __restrict__ Lbuf, const float* __restrict__ Nbuf,
    const int32_t* __restrict__ kfirst, const int32_t* __restrict__ dend,
    SchedHeader* __restrict__ hdr,
    const int2* __restrict__ tile_info, const int2* __restrict__ items,
    const int4* __restrict__ tile_rows, u16* __restrict__ stash, int stash_kvh_blocks,
    float* __restrict__ partial, float* __restrict__ dk, float* __restrict__ dv, Geo g, int nkt) {
  using Lds = DkdvLds<D>;
  constexpr int BN = kDkdvBN, KS = D / 32, ND = D / 16;
  // ring of 4 stages (kStage is a multiple of 256 bytes)
  static_assert(Lds::kStage % 256 == 0, "stage alignment");
  __shared__ __attribute__((aligned(1024))) char stg[4 * Lds::kStage];
  // LDS byte address of stg, taken once (the cast checks for null); DMA
  // addresses are offsets from it
  const unsigned stg_lds = (unsigned)(uintptr_t)(lds_char*)stg;
  auto lds_of = [&](const char* p) __attribute__((always_inline)) {
    return stg_lds + (unsigned)(p - stg);
  };
  __shared__ int s_item;
  // per-wave transpose scratch of the dS stash: [16 keys][32 rows] bf16,
  // 64 bytes per key, its eight 8-byte pieces (4 rows each) permuted by
  // piece ^ tr_swz(key): the transposed read of a 32-lane half covers four
  // whole keys (all 64 banks once), and the four keys whose rows share a
  // bank window write disjoint pieces (SQ_LDS_BANK_CONFLICT: the earlier
  // padded rows of 40 elements cost ~4 conflict cycles per access)
  constexpr int kTrLd = 32;
  __shared__ __attribute__((aligned(16))) u16 s_tr[STASH ? kWaves * kWaveKeys * kTrLd : 1];

  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int g4 = lane >> 4, j = lane & 15;
  const int total = hdr->n_base_items * g.Hkv;
  const int rps = hdr->rows_per_split;
  const size_t kvstride = (size_t)g.Hkv * D;
  const float c2 = g.scale_log2;

  // b128 operand (A of S = Q K^T): lane l reads row j of a 16-row step,
  // chunk 4ks + g4 (slot g4 ^ f(j); f depends on row bit 2 only, so the
  // 16-row steps all share these offsets).
  const int off_b = 64 * j + 16 * (g4 ^ (((j >> 2) & 1) << 1));
  // transposed operand (B of dV, dK) for d tile nd: source lane j of group
  // g4 reads row 4*g4 + j/4 (+16), chunk 2(nd&1) + (j&3)/2 of chunk group
  // nd/2, 8-byte half j&1 (f of those rows is 2*(g4 % 2)).
  int off_t[2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
    off_t[par] = 64 * (4 * g4 + (j >> 2)) + 16 * ((2 * par + ((j & 3) >> 1)) ^ ((g4 & 1) << 1)) +
                 8 * (j & 1);

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
    const int32_t* kf = kfirst ? kfirst + (size_t)b * g.Skv : nullptr;
    int a0, na, b0, nb;
    key_tile_tokens(kf, de, kt, g, a0, na, b0, nb);
    const int rows_total = (na + nb) * g.G;
    const int r_begin = split * rps;
    const int r_end = min(r_begin + rps, rows_total);
    const int nsb = r_end > r_begin ? (r_end - r_begin + 31) / 32 : 0;

    // this lane's key and its K / V operands (B of S = Q K^T, dP = dO V^T:
    // lane l holds key j, elements 32ks + 8*g4 .. +7)
    const int key = t0 + wave * kWaveKeys + j;
    const int kc = min(key, g.Skv - 1);
    const u16* krow = k + ((size_t)b * g.Skv + kc) * kvstride + (size_t)kvh * D;
    const u16* vrow = v + ((size_t)b * g.Skv + kc) * kvstride + (size_t)kvh * D;
    // V' = V * 2^ev in fp16 (exact power-of-two scale), for dP' = dO' V'^T
    bf16x8 kop[KS], vop[KS];
    const float sv = __builtin_amdgcn_ldexpf(1.f, hdr->ev);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kop[ks] = ld_bf16x8(krow + 32 * ks + 8 * g4);
      const bf16x8 vb = ld_bf16x8(vrow + 32 * ks + 8 * g4);
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f16x2 hv = {(_Float16)((float)vb[2 * e] * sv), (_Float16)((float)vb[2 * e + 1] * sv)};
        w[e] = __builtin_bit_cast(unsigned, hv);
      }
      vop[ks] = __builtin_bit_cast(bf16x8, w);
    }

    // Rows allowed for this key (key_rows: a contiguous range of the item's
    // virtual rows).  Both ends grow with the key, so the wave's common
    // range is [lo of its last key, hi of its first key).
    int vr_lo, vr_hi;
    key_rows(key, kf, de, a0, na, b0, nb, g, r_begin, r_end, vr_lo, vr_hi);
    const int w_lo = __builtin_amdgcn_readlane(vr_lo, kWaveKeys - 1);
    const int w_hi = __builtin_amdgcn_readlane(vr_hi, 0);

    f32x4 dka[ND], dva[ND];
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) {
      dka[nd] = f32x4{0.f, 0.f, 0.f, 0.f};
      dva[nd] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

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
    // DMA of one block, in two parts so that its instructions can be spread
    // over the block's two sub-blocks: prep_block computes this lane's row
    // offsets and advances the row bookkeeping, issue_q starts Q and the row
    // statistics, issue_o dO.
    unsigned nx_qoff = 0, nx_ridm = 0;
    auto prep_block = [&]() __attribute__((always_inline)) {
      // tiles: wave w fills rows 16(w%4) .. +15 of chunk groups w/4 + 2m
      const int rq = wave & 3, c0 = wave >> 2;
      const int rr = 16 * rq + (lane >> 2);
      const unsigned ridx = row_index(rr);
      const int slot = lane & 3, xr = ((rr >> 2) & 1) << 1;
      // byte offset of the row's chunk (q and dout share the layout; both
      // stay below 4 GiB, which the host checks)
      nx_qoff = (ridx * (unsigned)D + 32 * c0 + 8 * (slot ^ xr)) * 2u;
      nx_ridm = row_index(16 * rq + (lane & 15));
      ++nx_blk;
      nx_ti += step_ti;
      nx_hh += step_hh;
      if (nx_hh >= g.G) { nx_hh -= g.G; ++nx_ti; }
    };
    auto issue_q = [&](char* st) __attribute__((always_inline)) {
      const int rq = wave & 3, c0 = wave >> 2;
      char* tq = st + 64 * 16 * rq + c0 * kGroupBytes;
      static_for<D / 64>([&](auto m) __attribute__((always_inline)) {
        constexpr int M = decltype(m)::value;
        dma_lds16<128 * M>(q, nx_qoff, lds_of(tq) + 2 * M * kGroupBytes);
      });
      // row statistics, lanes 0..15: rows 16(w%4) + lane; waves 0-3 load
      // -lse/scale, waves 4-7 -D
      if (lane < 16) {
        if (wave < 4)
          dma_lds4(Lbuf, nx_ridm * 4u, lds_of(st) + Lds::kL + 64 * rq);
        else
          dma_lds4(Nbuf, nx_ridm * 4u, lds_of(st) + Lds::kN + 64 * rq);
      }
    };
    auto issue_o = [&](char* st) __attribute__((always_inline)) {
      const int rq = wave & 3, c0 = wave >> 2;
      char* tq = st + Lds::kTile + 64 * 16 * rq + c0 * kGroupBytes;
      static_for<D / 64>([&](auto m) __attribute__((always_inline)) {
        constexpr int M = decltype(m)::value;
        dma_lds16<128 * M>(dout16, nx_qoff, lds_of(tq) + 2 * M * kGroupBytes);
      });
    };

    // dS stash of this item's tile: virtual row vr is query row tlo*G + vr
    // of the KV head (the tile's rows are the contiguous local tokens
    // [tlo, thi)); block b of the tile covers rows [32(J_lo + b), +32).
    // Stores go through a buffer resource spanning exactly the tile's
    // blocks: a lane whose row lies past the item's end gets an offset
    // beyond that range, which the hardware drops (no divergent branch).
    // A tile left out of the stash (trow.w < 0: its blocks did not fit in
    // the budget) gets an empty range, so its stores are all dropped.
    const int4 trow = tile_rows[x];
    const int tr_z = uniform(trow.z), tr_x = uniform(trow.x), tr_w = uniform(trow.w);
    const int tile_blocks =
        tr_w >= 0 ? uniform((trow.y * g.G + kStashRows - 1) / kStashRows - trow.z) : 0;
    __amdgpu_buffer_rsrc_t srs;
    if constexpr (STASH)
      srs = __builtin_amdgcn_make_buffer_rsrc(
          stash + ((size_t)kvh * stash_kvh_blocks + max(tr_w, 0)) * (kStashBlockBytes / 2), 0,
          tile_blocks * kStashBlockBytes, 0x00020000);
    // (1) dS to this wave's transpose scratch, key-major: lane (g4, j) holds
    // key j at rows 16t + 4*g4 + 0..3.
    auto tr_swz = [](int key) __attribute__((always_inline)) { return 2 * ((key >> 2) & 3); };
    auto stash_put = [&](const bf16x8& dsop) __attribute__((always_inline)) {
      u16* T = s_tr + wave * kWaveKeys * kTrLd;
      const u32x4 w4 = __builtin_bit_cast(u32x4, dsop);
      *reinterpret_cast<uint2*>(T + j * kTrLd + 4 * (g4 ^ tr_swz(j))) = uint2{w4[0], w4[1]};
      *reinterpret_cast<uint2*>(T + j * kTrLd + 4 * ((4 + g4) ^ tr_swz(j))) =
          uint2{w4[2], w4[3]};
    };
    // (2) transposed read: lane (h, i) gets row i, keys 8(e/4) + 4h + e%4
    // of the wave's 16, stored as chunk (w, lane) of the row's stash block.
    // Read at the start of the next sub-block (and once after the last),
    // before that sub-block's (1) rewrites the scratch, and stored once its
    // score products are issued, so they run between the read and the store.
    auto stash_read = [&]() __attribute__((always_inline)) {
      const u16* T = s_tr + wave * kWaveKeys * kTrLd;
      // transposed read (as a padded-tile operand read, with the pieces
      // permuted): 16-lane group grp reads keys 4(grp/2) + s/4 (+8),
      // rows 16(grp%2) + 4(s%4) .. +3
      const int s4 = lane & 15, grp = lane >> 4;
      const int k0 = 4 * (grp >> 1) + (s4 >> 2), k1 = k0 + 8;
      const int pc = 4 * (grp & 1) + (s4 & 3);
      const i16x4 lo = ds_read_tr(T + k0 * kTrLd + 4 * (pc ^ tr_swz(k0)));
      const i16x4 hi = ds_read_tr(T + k1 * kTrLd + 4 * (pc ^ tr_swz(k1)));
      const bf16x4 la = __builtin_bit_cast(bf16x4, lo), ha = __builtin_bit_cast(bf16x4, hi);
      return bf16x8{la[0], la[1], la[2], la[3], ha[0], ha[1], ha[2], ha[3]};
    };
    // store of the sub-block from virtual row R (none when `valid` is
    // false: the offset then lies past the buffer, which drops the store)
    auto stash_write = [&](const bf16x8& op, int R, bool valid) __attribute__((always_inline)) {
      const int i = lane & 31, h = lane >> 5;
      const int grow = tr_x * g.G + R + i;
      const unsigned off = valid && R + i < r_end
                               ? (unsigned)(((grow >> 5) - tr_z) * kStashBlockBytes + wave * 1024 +
                                            (32 * h + (grow & 31)) * 16)
                               : 0x80000000u;
      // non-temporal: the stash is read once, by the dQ kernel, long after
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, op), srs, off, 0,
                                             kCachePolicyNT);
    };

    // S = Q K^T and dP = dO V^T of one sub-block (rows q0.. of stage st):
    // the accumulators start at -lse/scale and -D of their rows.
    auto sdp = [&](const char* st, int q0, f32x4 (&sc)[2], f32x4 (&pc)[2])
                   __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        sc[t] = ld_lds_f32x4(st + Lds::kL + 4 * (q0 + 16 * t + 4 * g4));
        pc[t] = ld_lds_f32x4(st + Lds::kN + 4 * (q0 + 16 * t + 4 * g4));
      }
      // product p: S (p < 2KS: rows 16t, t = p%2, k-step p/2) then dP; its
      // operand read kAhead products before it, through a ring of
      // registers, in program order (fenced)
      constexpr int NPR = 4 * KS, kAhead = 4;
      auto read_op = [&](auto p_c) __attribute__((always_inline)) {
        constexpr int P = decltype(p_c)::value;
        constexpr int T = P & 1, KSI = (P % (2 * KS)) >> 1;
        constexpr int base = P < 2 * KS ? 0 : Lds::kTile;
        return ld_lds_b128(st + base + KSI * kGroupBytes + 64 * (q0 + 16 * T) + off_b);
      };
      bf16x8 ring[kAhead + 1];
      static_for<kAhead>([&](auto p_c) __attribute__((always_inline)) {
        ring[decltype(p_c)::value] = read_op(p_c);
      });
      static_for<NPR>([&](auto p_c) __attribute__((always_inline)) {
        constexpr int P = decltype(p_c)::value;
        if constexpr (P + kAhead < NPR)
          ring[(P + kAhead) % (kAhead + 1)] = read_op(std::integral_constant<int, P + kAhead>{});
        constexpr int T = P & 1, KSI = (P % (2 * KS)) >> 1;
        if constexpr (P < 2 * KS)
          sc[T] = mfma16(ring[P % (kAhead + 1)], kop[KSI], sc[T]);
        else
          pc[T] = mfma16h(ring[P % (kAhead + 1)], vop[KSI], pc[T]);
        __builtin_amdgcn_sched_barrier(0);
      });
    };

    // The rest of a sub-block (virtual rows from R, rows q0.. of stage st)
    // from its S and dP: P, dV += P^T dO, dS, dK += dS^T Q.
    auto rest = [&](auto masked, const char* st, int q0, int R, const f32x4 (&sc)[2],
                    const f32x4 (&pc)[2]) __attribute__((always_inline)) {
      const char* tQ = st + 64 * q0;
      const char* tO = st + Lds::kTile + 64 * q0;
      // product r: dV' += P^T dO' (r < ND, d tile r) then dK += dS'^T Q
      // (d tile r - ND); its transposed operand read kAheadT products
      // before it through a ring, in program order (fenced); the first
      // reads are issued before P is formed, and dS' is formed under the dV
      // products
      constexpr int kAheadT = 3;
      auto read_t = [&](auto r_c) __attribute__((always_inline)) {
        constexpr int R_ = decltype(r_c)::value;
        constexpr int nd = R_ % ND;
        const char* tile = R_ < ND ? tO : tQ;
        return tr_pair(tile + (nd >> 1) * kGroupBytes + off_t[nd & 1]);
      };
      bf16x8 rg[kAheadT + 1];
      static_for<kAheadT>([&](auto r_c) __attribute__((always_inline)) {
        rg[decltype(r_c)::value] = read_t(r_c);
      });
      // p[4t + r]: row 16t + 4*g4 + r of the sub-block, key j
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(sc[e >> 2][e & 3] * c2);
      if constexpr (decltype(masked)::value) {
        const int lo_rel = vr_lo - R - 4 * g4;
        const unsigned span = (unsigned)max(vr_hi - vr_lo, 0);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int cr = 16 * (e >> 2) + (e & 3);
          if ((unsigned)(cr - lo_rel) >= span) p[e] = 0.f;
        }
      }
      // P in fp16 (round to nearest even, one conversion per pair) for
      // dV' += P^T dO' (the dO' tile is fp16)
      u32x4 pw;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f16x2 hp = {(_Float16)p[2 * e], (_Float16)p[2 * e + 1]};
        pw[e] = __builtin_bit_cast(unsigned, hp);
      }
      const bf16x8 pop = __builtin_bit_cast(bf16x8, pw);
      bf16x8 dsop;
      __builtin_amdgcn_sched_barrier(0);
      static_for<2 * ND>([&](auto r_c) __attribute__((always_inline)) {
        constexpr int R_ = decltype(r_c)::value;
        if constexpr (R_ + kAheadT < 2 * ND)
          rg[(R_ + kAheadT) % (kAheadT + 1)] = read_t(std::integral_constant<int, R_ + kAheadT>{});
        if constexpr (R_ < ND) {
          dva[R_] = mfma16h(pop, rg[R_ % (kAheadT + 1)], dva[R_]);
          // dS' = P * dP' (bf16), two values per dV product (ND >= 4)
          if constexpr (R_ < 4) {
            dsop[2 * R_] = (__bf16)(p[2 * R_] * pc[(2 * R_) >> 2][(2 * R_) & 3]);
            dsop[2 * R_ + 1] = (__bf16)(p[2 * R_ + 1] * pc[(2 * R_ + 1) >> 2][(2 * R_ + 1) & 3]);
          }
        } else {
          dka[R_ - ND] = mfma16(dsop, rg[R_ % (kAheadT + 1)], dka[R_ - ND]);
        }
        // dS' (complete after slot 3) to the transpose scratch
        if constexpr (STASH && R_ == 4) stash_put(dsop);
        __builtin_amdgcn_sched_barrier(0);
      });
    };

    // Sub-block j lives in stage (j/2) % 4 at row 32*(j%2).  Block n+2's
    // DMA is issued during block n, after the barrier that opens it (Q and
    // row statistics in its first sub-block, dO in its second); that
    // barrier also guarantees every wave has finished block n-1.  Every
    // wait counts one block's instructions: block n's DMA must be done,
    // block n+1's may be in flight.  A last block with a single sub-block
    // skips the dO part; no wait follows it.
    auto stage = [&](int blk) __attribute__((always_inline)) -> char* {
      return stg + (blk & 3) * Lds::kStage;
    };
    wait_vmcnt<0>();
    if (nsb > 0) {
      prep_block();
      issue_q(stage(0));
      issue_o(stage(0));
      prep_block();
      issue_q(stage(1));
      issue_o(stage(1));
    }
    for (int jb = 0; 2 * jb < nsb; ++jb) {
      wait_vmcnt<Lds::kDmaPerWave>();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      prep_block();
      const char* st = stage(jb);
      char* nx = stage(jb + 2);
      auto sub_block = [&](auto second) __attribute__((always_inline)) {
        constexpr int h2 = decltype(second)::value ? 1 : 0;
        const int R = r_begin + 64 * jb + 32 * h2;
        f32x4 sc[2], pc[2];
        // the previous sub-block's dS (if any) from the transpose scratch,
        // stored once the score products are issued
        bf16x8 prev;
        if constexpr (STASH) prev = stash_read();
        sdp(st, 32 * h2, sc, pc);
        // DMA instructions of a later block, while the products run
        if constexpr (h2 == 0)
          issue_q(nx);
        else
          issue_o(nx);
        if constexpr (STASH) stash_write(prev, R - 32, R > r_begin);
        if (w_lo <= R && R + 32 <= w_hi)
          rest(std::false_type{}, st, 32 * h2, R, sc, pc);
        else
          rest(std::true_type{}, st, 32 * h2, R, sc, pc);
      };
      sub_block(std::false_type{});
      if (2 * jb + 1 < nsb) sub_block(std::true_type{});
    }
    if constexpr (STASH)
      if (nsb > 0) stash_write(stash_read(), r_begin + 32 * (nsb - 1), true);

    // No DMA (including the re-loads past the item's end) may still be
    // writing LDS once the item is done.
    wait_vmcnt<0>();

    // Write this wave's 16 keys: directly (dK scaled) if the tile was not
    // split, else to the item's partial-sum slot.  Register r of d tile nd
    // holds key 16w + 4*g4 + r, element 16nd + j.
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
    // dS' and dV' carry 2^(eo+ev) and 2^eo (fp16 scales); split tiles'
    // partial sums are scaled by the reduce
    const float kscale = split_tile ? 1.f : g.scale * hdr->dk_mul;
    const float vscale = split_tile ? 1.f : hdr->dv_mul;
#pragma unroll
    for (int nd = 0; nd < ND; ++nd)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kvloc = wave * kWaveKeys + 4 * g4 + r;
        if (split_tile || t0 + kvloc < g.Skv) {
          dst_k[(size_t)kvloc * rstride + 16 * nd + j] = dka[nd][r] * kscale;
          dst_v[(size_t)kvloc * rstride + 16 * nd + j] = dva[nd][r] * vscale;
        }
      }
  }
}

hipError_t launch_bwd_dkdv(int D, const u16* q, const u16* k, const u16* v, const u16* dout16,
                           const float* Lbuf, const float* Nbuf, const int32_t* kfirst,
                           const int32_t* dend, SchedHeader* hdr, const int2* tile_info, const int2* items,
                           const int4* tile_rows, u16* stash, int stash_kvh_blocks,
                           float* partial, float* dk, float* dv, const Geo& g, int nkt,
                           hipStream_t st) {
#define DMGQA_DKDV(DD, SS)                                                                  \
  bwd_dkdv_kernel<DD, SS><<<kDkdvGrid, kWaves * 64, 0, st>>>(                               \
      q, k, v, dout16, Lbuf, Nbuf, kfirst, dend, hdr, tile_info, items, tile_rows, stash,             \
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
