// dQ of document-masked causal GQA attention from the dS stash.
//
// dQ = scale * dS K ("Training Infrastructure and Systems", "FlashAttention:
// never write the score matrix" for the recomputation it replaces; the chain
// rule as in the other backward kernels).  The dK/dV kernel, which computes
// dS for every (query row, key) pair it visits, stores it as bf16 in stash
// blocks of 32 query rows x 128 keys; this kernel is then a plain product
// per KV head: for each 32-row block of query rows, the sum over the key
// tiles that reach it of dS_block K_tile.  Without the stash, dQ has to
// recompute S, P and dP (three products instead of one).
#include "common.hpp"
#include "dma.hpp"
#include "kernels.hpp"
#include "reduce.hpp"

namespace dmgqa {

namespace {

// K tile of 128 keys in LDS: two halves of 64 keys, each in groups of four
// 16-byte chunks (32 elements): group c/4 of key row r at (c/4)*4096 + 64*r,
// chunk c in slot (c % 4) ^ ((r / 4) % 4) -- conflict-free for the
// transposed reads (4 rows x 4 slots x two 8-byte halves per 32 lanes).
constexpr int kHalfRows = 64;
constexpr int kGroupBytes = kHalfRows * 64;

template <int D>
struct KTile {
  static constexpr int kHalf = D / 32 * kGroupBytes;   // bytes of one 64-key half
  static constexpr int kBytes = 2 * kHalf;
};

// K^T operand (lane 32h + i: column d = 32 db + i, keys of k-step ks of the
// half in the MFMA slot order) from a half tile.
__device__ __forceinline__ bf16x8 kt_operand(const char* half, const int (&off)[2], int ks,
                                             int db) {
  const char* p = half + db * kGroupBytes + 16 * ks * 64;
  const i16x4 lo = ds_read_tr(reinterpret_cast<const u16*>(p + off[0]));
  const i16x4 hi = ds_read_tr(reinterpret_cast<const u16*>(p + off[1]));
  const bf16x4 a = __builtin_bit_cast(bf16x4, lo);
  const bf16x4 b = __builtin_bit_cast(bf16x4, hi);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

typedef __attribute__((address_space(3))) char lds_char;

// global_load_lds_dwordx4 as inline assembly: lane l's 16 bytes at
// sbase + voff + IMM go to LDS address lds + 16 * l (sbase, lds
// wave-uniform).  The immediate offset moves the LDS address too, so M0 is
// lds - IMM.
template <int IMM>
__device__ __forceinline__ void dma_asm16(const void* sbase, unsigned voff, unsigned lds) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds) - (unsigned)IMM;
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 offset:%3" ::"v"(voff),
               "s"(sbase), "s"(m0), "i"(IMM)
               : "memory");
}

}  // namespace

// One workgroup = 4 stash blocks (128 query rows of one KV head): wave w
// owns block J = 4*qb + w.  Workgroups past the dQ grid (dq_grid onwards)
// add the partial dK/dV slots of the split key tiles instead: dispatched
// after every dQ workgroup, they run in the launch's tail, where the long
// row blocks leave memory bandwidth unused.  Key tiles of 128 are those reaching any of the
// 128 rows; their K tiles stream through two LDS stages (DMA one tile
// ahead), and the wave's dS operands are loaded into registers two tiles
// ahead.  Rows of a block outside the tile's reach hold
// no stash data and are zeroed.  CROSS: query position p reaches keys
// dstart[p] .. dhi[p]-1 (both [B, S], keys indexed on their own); else keys
// dstart[p] .. p (dstart [B, Skv]).
template <int D, bool CROSS>
__global__ __launch_bounds__(256, 2) void bwd_dq_stash_kernel(
    const u16* __restrict__ k, const int32_t* __restrict__ dstart,
    const int32_t* __restrict__ dhi, const int4* __restrict__ tile_rows, const u16* __restrict__ stash, int stash_kvh_blocks,
    const int32_t* __restrict__ order, u16* __restrict__ dq, float* __restrict__ dq_part,
    const int2* __restrict__ tile_info, const float* __restrict__ partial,
    float* __restrict__ dk, float* __restrict__ dv, const SchedHeader* __restrict__ hdr, Geo g,
    int nkt, int dq_grid) {
  if ((int)blockIdx.x >= dq_grid) {
    reduce_partials<D>(tile_info, partial, dk, dv, hdr, g, nkt, (int)blockIdx.x - dq_grid);
    return;
  }
  using KT = KTile<D>;
  constexpr int DB = D / 32, NCH = D / 8, BN = kDkdvBN;
  __shared__ __attribute__((aligned(1024))) char sk[2 * KT::kBytes];
  char* const sk0 = sk;
  char* const sk1 = sk + KT::kBytes;
  // LDS byte address of sk, taken once (the cast checks for null)
  const unsigned sk_lds = (unsigned)(uintptr_t)(lds_char*)sk;

  const int nrows = g.Sq * g.G;
  const int nqb = (nrows + 127) / 128;
  // (batch row, row block) items in the heaviest-first order, the KV heads
  // of an item consecutively (clamped: the order is a permutation)
  const int item = min(max(order[blockIdx.x / g.Hkv], 0), g.B * nqb - 1);
  const int b = item / nqb, qb = item - b * nqb;
  const int kvh = blockIdx.x % g.Hkv;
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int h = lane >> 5, i = lane & 31;
  const int J = 4 * qb + wave;                 // this wave's 32-row block
  const int grow = 32 * J + i;                 // this lane's query row (in the KV head)

  // transposed-read offsets (row quad index h, +2 for the second half)
  const int s16 = lane & 15, grp = lane >> 4;
  int off_t[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
    off_t[hf] = (4 * h + (s16 >> 2) + 8 * hf) * 64 +
                16 * ((2 * (grp & 1) + ((s16 & 3) >> 1)) ^ ((h + 2 * hf) & 3)) + 8 * (s16 & 1);

  const int32_t* ds = dstart + (size_t)b * (CROSS ? g.S : g.Skv);
  const QTileKeys kr =
      CROSS ? qtile_keys_iv<128, BN>(128 * qb, ds, dhi + (size_t)b * g.S, g)
            : qtile_keys<128, BN>(128 * qb, ds, g);
  const int ntiles = kr.na + kr.nb;
  const size_t kvstride = (size_t)g.Hkv * D;
  const u16* kbase = k + (size_t)b * g.Skv * kvstride + (size_t)kvh * D;
  const int4* trow_b = tile_rows + (size_t)b * nkt;
  const u16* stash_h = stash + (size_t)kvh * stash_kvh_blocks * (kStashBlockBytes / 2);

  // K tile DMA: wave w fills key rows 16w .. 16w+15 of both halves (lane
  // l: row 16w + l/4, slot l%4), as assembly with a scalar base and a 32-bit
  // per-lane offset (K below 2^31 elements, which the host checks), so the
  // compiler adds no waits of its own for these LDS writes.
  const int kr_row = 16 * wave + (lane >> 2);
  const unsigned coff = 8 * ((lane & 3) ^ ((kr_row >> 2) & 3));
  // per-lane byte offsets of the two halves' rows within a full tile
  const unsigned koff[2] = {((unsigned)kr_row * (unsigned)kvstride + coff) * 2u,
                            ((unsigned)(kr_row + 64) * (unsigned)kvstride + coff) * 2u};
  auto issue = [&](int it, char* st) __attribute__((always_inline)) {
    const int kt = uniform(it < kr.na ? kr.a0 + it : kr.b0 + (it - kr.na));
    // the tile's rows as a scalar base; a tile running past the last key
    // clamps its rows per lane
    const u16* tb = kbase + (size_t)kt * BN * kvstride;
    const bool partial = kt * BN + BN > g.Skv;
    auto half = [&](int hf, unsigned off) __attribute__((always_inline)) {
      char* dst = st + hf * KT::kHalf + 64 * 16 * wave;
      static_for<NCH / 4>([&](auto cc) __attribute__((always_inline)) {
        constexpr int C = decltype(cc)::value;
        dma_asm16<64 * C>(tb, off, sk_lds + (unsigned)(dst - sk) + C * kGroupBytes);
      });
    };
    if (!partial) {
      half(0, koff[0]);
      half(1, koff[1]);
    } else {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int key = min(64 * hf + kr_row, g.Skv - 1 - kt * BN);
        half(hf, ((unsigned)key * (unsigned)kvstride + coff) * 2u);
      }
    }
  };
  // dS operands of this wave's block for tile `it`, loaded two tiles ahead
  // of their use.  `have`: the tile's stash holds block J; `part`: some rows
  // of the block lie outside the tile's reach (their stash rows are never
  // written and are replaced by zeros at use); `ok`: this lane's row does not.
  // Past the last tile the loads still happen (from this head's first stash
  // block, never used), so every step issues the same number of them.
  struct DsOps {
    u32x4 op[8];
    int4 tr;     // the tile's row range (tile_rows entry)
    bool in;     // a tile of this workgroup (not a load past the last)
  };
  auto load_ds = [&](int it, DsOps& d) __attribute__((always_inline)) {
    const int x = min(it, ntiles - 1);
    const int kt = uniform(x < kr.na ? kr.a0 + x : kr.b0 + (x - kr.na));
    const int4 tr = trow_b[kt];
    d.tr = tr;
    d.in = it < ntiles;
    const int nblk = tr.y > tr.x ? (tr.y * g.G + kStashRows - 1) / kStashRows - tr.z : 0;
    const int rel = J - tr.z;
    const bool have = d.in && tr.w >= 0 && rel >= 0 && rel < nblk;
    // one block through a buffer resource (wave-uniform base) and a fixed
    // per-lane offset; non-temporal (the stash is read once: keeping it out
    // of the caches took the kernel from 138 to 117 us on the 405B share)
    const u16* blk = stash_h + (have ? (size_t)(tr.w + rel) * (kStashBlockBytes / 2) : 0);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u16*>(blk), 0, kStashBlockBytes, 0x00020000);
#pragma unroll
    for (int kq = 0; kq < 8; ++kq)
      d.op[kq] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16 + kq * 1024, 0, kCachePolicyNT));
  };
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = zero16();

  // One barrier per key tile.  Issue order: K(it+1) DMA, then dS(it+2)
  // loads, so when tile it starts only the 8 dS loads of tile it+1 may be
  // outstanding: wait for the rest (tile it's K and dS), barrier (every
  // wave's K loads are in and every wave is done with tile it-1, whose
  // stage the next DMA refills), start the next loads, multiply.
  auto step = [&](int it, const char* cur, char* nxt, DsOps& dc, DsOps& dn)
                  __attribute__((always_inline)) {
    wait_vmcnt<8>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (it + 1 < ntiles) issue(it + 1, nxt);
    load_ds(it + 2, dn);
    const int4 tr = dc.tr;
    const int nblk = tr.y > tr.x ? (tr.y * g.G + kStashRows - 1) / kStashRows - tr.z : 0;
    const int rel = J - tr.z;
    const bool have = dc.in && tr.w >= 0 && rel >= 0 && rel < nblk;
    // rows of the block outside the tile's reach: never written, zeroed here
    const bool part = !(tr.x * g.G <= 32 * J && 32 * J + 32 <= tr.y * g.G);
    const bool ok = grow >= tr.x * g.G && grow < tr.y * g.G;
    if (have) {
      if (part && !ok) {
#pragma unroll
        for (int kq = 0; kq < 8; ++kq) dc.op[kq] = u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int db = 0; db < DB; ++db)
            acc[db] = mfma32(kt_operand(cur + hf * KT::kHalf, off_t, ks, db),
                             __builtin_bit_cast(bf16x8, dc.op[4 * hf + ks]), acc[db]);
    }
  };
  if (ntiles > 0) {
    DsOps d0, d1, d2;
    issue(0, sk0);
    load_ds(0, d0);
    load_ds(1, d1);
    // K stages alternate with the tile index, dS register sets cycle by 3
    for (int it = 0; it < ntiles; it += 6) {
      step(it, sk0, sk1, d0, d2);
      if (it + 1 >= ntiles) break;
      step(it + 1, sk1, sk0, d1, d0);
      if (it + 2 >= ntiles) break;
      step(it + 2, sk0, sk1, d2, d1);
      if (it + 3 >= ntiles) break;
      step(it + 3, sk1, sk0, d0, d2);
      if (it + 4 >= ntiles) break;
      step(it + 4, sk0, sk1, d1, d0);
      if (it + 5 >= ntiles) break;
      step(it + 5, sk1, sk0, d2, d1);
    }
    wait_vmcnt<0>();
  }

  // Stashed tiles are a prefix in (batch row, key tile) order, so the
  // query tile reaches a tile without stash iff its last key tile has none;
  // then the recompute kernel adds those tiles' share to the unscaled fp32
  // sums left here and writes dq.
  const int kt_last = kr.nb > 0 ? kr.b0 + kr.nb - 1 : kr.a0 + kr.na - 1;
  const bool mixed = dq_part != nullptr && ntiles > 0 && trow_b[kt_last].w < 0;
  // the stash holds dS * 2^(eo+ev) (fp16 scales of the dK/dV kernel)
  const float dsmul = hdr->dk_mul;
  if (mixed) {
    if (grow < nrows) {
      const int tok = grow / g.G, hh = grow - tok * g.G;
      float* prow = dq_part + (((size_t)b * g.Sq + tok) * g.Hq + kvh * g.G + hh) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 w = {acc[db][4 * r4] * dsmul, acc[db][4 * r4 + 1] * dsmul,
                           acc[db][4 * r4 + 2] * dsmul, acc[db][4 * r4 + 3] * dsmul};
          *reinterpret_cast<f32x4*>(prow + 32 * db + 8 * r4 + 4 * h) = w;
        }
    }
  } else if (grow < nrows) {
    const int tok = grow / g.G, hh = grow - tok * g.G;
    u16* orow = dq + (((size_t)b * g.Sq + tok) * g.Hq + kvh * g.G + hh) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc[db][4 * r4 + e] * (g.scale * dsmul));
        *reinterpret_cast<uint2*>(orow + 32 * db + 8 * r4 + 4 * h) = __builtin_bit_cast(uint2, w);
      }
  }
}

hipError_t launch_bwd_dq_stash(int D, const u16* k, const int32_t* dstart, const int32_t* dhi,
                               const int4* tile_rows, const u16* stash, int stash_kvh_blocks,
                               const int32_t* order, u16* dq, float* dq_part,
                               const int2* tile_info, const float* partial, float* dk, float* dv,
                               const SchedHeader* hdr, const Geo& g, int nkt, hipStream_t st) {
  const int nqb = (g.Sq * g.G + 127) / 128;
  const unsigned grid = (unsigned)nqb * g.B * g.Hkv;
#define DMGQA_DQS(DD, CC)                                                                      \
  bwd_dq_stash_kernel<DD, CC><<<grid + reduce_grid<DD>(g, nkt), 256, 0, st>>>(                 \
      k, dstart, dhi, tile_rows, stash, stash_kvh_blocks, order, dq, dq_part, tile_info, partial, \
      dk, dv, hdr, g, nkt, (int)grid)
  if (D == 128) {
    if (dhi) DMGQA_DQS(128, true); else DMGQA_DQS(128, false);
  } else {
    if (dhi) DMGQA_DQS(64, true); else DMGQA_DQS(64, false);
  }
#undef DMGQA_DQS
  return hipGetLastError();
}

}  // namespace dmgqa
