// Backward kernels: dQ, dK and dV of document-masked causal GQA attention for
// one CP rank.
//
// The pages say only that the backward pass recomputes the scores instead of
// storing them ("Training Infrastructure and Systems", "FlashAttention: never
// write the score matrix", "Tiling").  The gradients are the chain rule of
// softmax attention with P = exp(scale * q k^T - lse) on allowed pairs:
//   D_i  = <dO_i, O_i>
//   dP   = dO V^T,  dS = P * (dP - D)
//   dQ   = scale * dS K
//   dK   = scale * dS^T Q,  dV = P^T dO   (summed over the G query heads of
//                                          each KV head, GQA)
// dK and dV are accumulated and returned in fp32, following the pages' use of
// FP32 gradient accumulation ("The Llama 3 Herd of Models", section 3.3.2,
// "Numerical stability").
//
// Three kernels:
//   bwd_dq    query-stationary, same tiling as the forward; it also computes
//             D for its rows and stores it for the dK/dV kernel.
//   bwd_dkdv  key-stationary work items (64 keys x a slice of the query rows
//             that reach them); persistent workgroups take items from a
//             counter.  Items of a key tile that was split write fp32 partial
//             sums to their own slots.
//   bwd_reduce adds the partial sums of split key tiles in item order, so the
//             result does not depend on which workgroup ran which item.
#include "common.hpp"
#include "kernels.hpp"
#include "qtile.hpp"
#include "tileload.hpp"

namespace dmgqa {

template <int D>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    const u16* __restrict__ out, const u16* __restrict__ dout, const float* __restrict__ lse,
    const int32_t* __restrict__ dstart, u16* __restrict__ dq, float* __restrict__ Dbuf, Geo g) {
  constexpr int BM = kFwdBM, BN = kFwdBN, LD = D, KK = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(16))) u16 sK[2][BN * LD];
  __shared__ __attribute__((aligned(16))) u16 sV[2][BN * LD];

  const int nrows = g.Sq * g.G;
  const int nt = (nrows + BM - 1) / BM;
  const int nbg = g.B * g.Hkv;
  const int tile = nt - 1 - (int)(blockIdx.x / nbg);
  const int bg = blockIdx.x % nbg;
  const int b = bg / g.Hkv, kvh = bg % g.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, i = lane & 31;

  const int row0 = tile * BM;
  const int row = row0 + wave * 32 + i;
  const bool valid = row < nrows;
  const int rr = valid ? row : nrows - 1;
  const int tok = rr / g.G;
  const int head = kvh * g.G + rr % g.G;
  const int pos = local_pos(tok, g.c, g.cp, g.rank);
  const int32_t* ds = dstart + (size_t)b * g.Skv;
  const int lo = ds[pos];

  const size_t roff = ((size_t)b * g.Sq + tok) * g.Hq + head;
  const size_t qoff = roff * D;
  bf16x8 qop[KK], dop[KK];
  float dsum = 0.f;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    qop[kk] = ld_bf16x8(q + qoff + 8 * h + 16 * kk);
    dop[kk] = ld_bf16x8(dout + qoff + 8 * h + 16 * kk);
    const bf16x8 ov = ld_bf16x8(out + qoff + 8 * h + 16 * kk);
#pragma unroll
    for (int e = 0; e < 8; ++e) dsum = fmaf((float)dop[kk][e], (float)ov[e], dsum);
  }
  const float Dv = dsum + xor32(dsum);
  if (valid && h == 0) Dbuf[roff] = Dv;
  const float lse2 = lse[roff] * kLog2e;

  const QTileKeys kr = qtile_keys<BM, BN>(row0, ds, g);
  const int ntiles = kr.na + kr.nb;

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = zero16();

  const size_t kvstride = (size_t)g.Hkv * D;
  const u16* kbase = k + (size_t)b * g.Skv * kvstride + (size_t)kvh * D;
  const u16* vbase = v + (size_t)b * g.Skv * kvstride + (size_t)kvh * D;
  TileRegs<BN, D, 256> rk, rv;
  auto fetch = [&](int it) __attribute__((always_inline)) {
    const int t0 = (it < kr.na ? kr.a0 + it : kr.b0 + (it - kr.na)) * BN;
    rk.load([&](int r) { return kbase + (size_t)min(t0 + r, g.Skv - 1) * kvstride; });
    rv.load([&](int r) { return vbase + (size_t)min(t0 + r, g.Skv - 1) * kvstride; });
  };
  fetch(0);
  rk.store(sK[0]);
  rv.store(sV[0]);
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int t0 = (it < kr.na ? kr.a0 + it : kr.b0 + (it - kr.na)) * BN;
    const int cur = it & 1;
    if (it + 1 < ntiles) fetch(it + 1);
    const u16* cK = sK[cur];
    const u16* cV = sV[cur];

    const bool full = kr.max_lo <= t0 && t0 + BN - 1 <= kr.min_pos;
    // two 32-key halves, to keep the score/dP accumulators at 32 registers
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      f32x16 s0 = zero16(), p0 = zero16();
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        s0 = mfma32(lds_bf16x8(&cK[swz<D>(32 * half + i, 8 * h + 16 * kk)]), qop[kk], s0);
        p0 = mfma32(lds_bf16x8(&cV[swz<D>(32 * half + i, 8 * h + 16 * kk)]), dop[kk], p0);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float e0 = __builtin_amdgcn_exp2f(fmaf(s0[r], g.scale_log2, -lse2));
        if (!full) {
          const int kv = t0 + 32 * half + 8 * (r >> 2) + 4 * h + (r & 3);
          if (kv < lo || kv > pos) e0 = 0.f;
        }
        s0[r] = e0 * (p0[r] - Dv);
      }
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const bf16x8 dsop = pack_bf16(s0, kh);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          acc[db] = mfma32(tr_operand<D>(cK, 0, 2 * half + kh, 32 * db, lane), dsop, acc[db]);
      }
    }
    if (it + 1 < ntiles) {
      rk.store(sK[cur ^ 1]);
      rv.store(sV[cur ^ 1]);
    }
    __syncthreads();
  }

  if (valid) {
    u16* orow = dq + qoff;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc[db][4 * r4 + e] * g.scale);
        *reinterpret_cast<uint2*>(orow + 32 * db + 8 * r4 + 4 * h) = __builtin_bit_cast(uint2, w);
      }
  }
}

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

template <int D>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    const u16* __restrict__ dout, const float* __restrict__ lse,
    const int32_t* __restrict__ dstart, const int32_t* __restrict__ dend,
    const float* __restrict__ Dbuf, SchedHeader* __restrict__ hdr,
    const int2* __restrict__ tile_info, const int2* __restrict__ items,
    float* __restrict__ partial, float* __restrict__ dk, float* __restrict__ dv, Geo g,
    int nkt) {
  // Work item: 128 keys (wave w owns keys t0 + 32w .. t0 + 32w + 31) x one
  // slice of the query rows reaching them.  Query rows stream through two LDS
  // stages in blocks of BM = 64 (every wave uses every row, as two sub-blocks
  // of 32); the global loads of block n+1 are issued before block n is
  // computed and written to the other stage after it.
  constexpr int BN = kDkdvBN, BM = kDkdvBM, KK = D / 16, DB = D / 32;
  constexpr int kTile = BM * D;                     // elements of one Q or dO block
  __shared__ __attribute__((aligned(16))) u16 sQ[2][kTile];
  __shared__ __attribute__((aligned(16))) u16 sdO[2][kTile];
  __shared__ __attribute__((aligned(16))) float s_lse2[2][BM];
  __shared__ __attribute__((aligned(16))) float s_D[2][BM];
  __shared__ __attribute__((aligned(16))) int s_lo[2][BM];
  __shared__ __attribute__((aligned(16))) int s_pos[2][BM];
  __shared__ int s_item;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, i = lane & 31;
  const int total = hdr->n_base_items * g.Hkv;
  const int rps = hdr->rows_per_split;
  const size_t kvstride = (size_t)g.Hkv * D;

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
    const int32_t* ds = dstart + (size_t)b * g.Skv;
    int a0, na, b0, nb;
    dkdv_ranges(dend + (size_t)b * g.Skv, kt, g, a0, na, b0, nb);
    const int rows_total = (na + nb) * g.G;
    const int r_begin = split * rps;
    const int r_end = min(r_begin + rps, rows_total);
    const int nblk = r_end > r_begin ? (r_end - r_begin + BM - 1) / BM : 0;

    const int kv_l = t0 + wave * 32 + i;
    const int kv_c = min(kv_l, g.Skv - 1);
    const u16* krow = k + ((size_t)b * g.Skv + kv_c) * kvstride + (size_t)kvh * D;
    const u16* vrow = v + ((size_t)b * g.Skv + kv_c) * kvstride + (size_t)kvh * D;
    bf16x8 kop[KK], vop[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      kop[kk] = ld_bf16x8(krow + 8 * h + 16 * kk);
      vop[kk] = ld_bf16x8(vrow + 8 * h + 16 * kk);
    }
    f32x16 dka[DB], dva[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) { dka[db] = zero16(); dva[db] = zero16(); }

    // Query rows of a block: virtual row vr0 + r (r < BM) is head-in-group
    // (hh0 + r) % G of token index ti0 + (hh0 + r) / G of the reaching
    // token run; vr0, ti0, hh0 are uniform.  Offsets are 32-bit (checked on
    // the host).
    TileRegs<BM, D, 256> rq, rdo;
    float m_lse2 = 0.f, m_D = 0.f;
    int m_lo = 0, m_pos = -1;
    auto fetch = [&](int blk) __attribute__((always_inline)) {
      const int vr0 = r_begin + blk * BM;
      const int ti0 = vr0 / g.G, hh0 = vr0 - ti0 * g.G;
      const int nrow = r_end - vr0;   // rows of this block that exist
      auto row_of = [&](int r) __attribute__((always_inline)) -> unsigned {
        const int t = hh0 + min(r, nrow - 1);
        const int qd = div_small(t, g);
        const int ti = ti0 + qd;
        const int tok = ti < na ? a0 + ti : b0 + (ti - na);
        return (unsigned)((b * g.Sq + tok) * g.Hq + kvh * g.G + (t - qd * g.G));
      };
      rq.load([&](int r) { return q + row_of(r) * (unsigned)D; });
      rdo.load([&](int r) { return dout + row_of(r) * (unsigned)D; });
      if (threadIdx.x < BM) {
        const int r = threadIdx.x;
        const bool ok = r < nrow;
        const int t = hh0 + min(r, nrow - 1);
        const int qd = div_small(t, g);
        const int ti = ti0 + qd;
        const int tok = ti < na ? a0 + ti : b0 + (ti - na);
        const int p = local_pos(tok, g.c, g.cp, g.rank);
        const unsigned ro = (unsigned)((b * g.Sq + tok) * g.Hq + kvh * g.G + (t - qd * g.G));
        m_pos = ok ? p : -1;
        m_lo = ok ? ds[p] : 0;
        m_lse2 = lse[ro] * kLog2e;
        m_D = Dbuf[ro];
      }
    };
    auto stash = [&](int st) __attribute__((always_inline)) {
      rq.store(sQ[st]);
      rdo.store(sdO[st]);
      if (threadIdx.x < BM) {
        s_pos[st][threadIdx.x] = m_pos;
        s_lo[st][threadIdx.x] = m_lo;
        s_lse2[st][threadIdx.x] = m_lse2;
        s_D[st][threadIdx.x] = m_D;
      }
    };
    if (nblk > 0) {
      fetch(0);
      stash(0);
    }
    __syncthreads();

    for (int blk = 0; blk < nblk; ++blk) {
      const int st = blk & 1;
      const int vr0 = r_begin + blk * BM;
      if (blk + 1 < nblk) fetch(blk + 1);
      const u16* cQ = sQ[st];
      const u16* cdO = sdO[st];
#pragma unroll
      for (int sb = 0; sb < BM / 32; ++sb) {
        const int q0 = 32 * sb;
        const bool full = vr0 + q0 + 32 <= r_end && s_lo[st][q0 + 31] <= t0 &&
                          t0 + BN - 1 <= s_pos[st][q0];
        f32x16 s = zero16(), dp = zero16();
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          s = mfma32(lds_bf16x8(cQ + swz<D>(q0 + i, 8 * h + 16 * kk)), kop[kk], s);
          dp = mfma32(lds_bf16x8(cdO + swz<D>(q0 + i, 8 * h + 16 * kk)), vop[kk], dp);
        }
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int qb = q0 + 8 * r4 + 4 * h;
          const f32x4 L = *reinterpret_cast<const f32x4*>(&s_lse2[st][qb]);
          const f32x4 Dd = *reinterpret_cast<const f32x4*>(&s_D[st][qb]);
          int4 LO = make_int4(0, 0, 0, 0), PO = make_int4(0, 0, 0, 0);
          if (!full) {
            LO = *reinterpret_cast<const int4*>(&s_lo[st][qb]);
            PO = *reinterpret_cast<const int4*>(&s_pos[st][qb]);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * r4 + e;
            float p = __builtin_amdgcn_exp2f(fmaf(s[r], g.scale_log2, -L[e]));
            if (!full) {
              const int lo_e = e == 0 ? LO.x : e == 1 ? LO.y : e == 2 ? LO.z : LO.w;
              const int po_e = e == 0 ? PO.x : e == 1 ? PO.y : e == 2 ? PO.z : PO.w;
              if (kv_l < lo_e || kv_l > po_e) p = 0.f;
            }
            s[r] = p;
            dp[r] = p * (dp[r] - Dd[e]);
          }
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          // P enters dV = P^T dO as bf16 hi + lo parts (16 significant bits):
          // dV sums P over every query row and head of the group, and a single
          // bf16 rounding of P (8 bits) is not accurate enough there.
          const bf16x8 pop = pack_bf16(s, ks);
          bf16x8 plo;
#pragma unroll
          for (int e = 0; e < 8; ++e) plo[e] = (__bf16)(s[8 * ks + e] - (float)pop[e]);
          const bf16x8 dsop = pack_bf16(dp, ks);
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const bf16x8 dot = tr_operand<D>(cdO, q0, ks, 32 * db, lane);
            dva[db] = mfma32(pop, dot, dva[db]);
            dva[db] = mfma32(plo, dot, dva[db]);
            dka[db] = mfma32(dsop, tr_operand<D>(cQ, q0, ks, 32 * db, lane), dka[db]);
          }
        }
      }
      if (blk + 1 < nblk) stash(st ^ 1);
      __syncthreads();
    }

    // Write this wave's 32 keys: directly (scaled) if the tile was not
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

// Sum of the partial slots of each split key tile, in item order.  One
// workgroup per (key tile, KV head, 1024-float chunk).
template <int D>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const int2* __restrict__ tile_info,
                                                         const float* __restrict__ partial,
                                                         float* __restrict__ dk,
                                                         float* __restrict__ dv, Geo g, int nkt) {
  constexpr int BN = kDkdvBN;
  constexpr int kChunks = 2 * BN * D / 1024;
  const int chunk = blockIdx.x % kChunks;
  const int th = blockIdx.x / kChunks;
  const int x = th / g.Hkv, kvh = th % g.Hkv;
  const int2 info = tile_info[x];
  if (info.x <= 1) return;
  const int b = x / nkt, kt = x % nkt;
  const int t0 = kt * BN;
  const size_t kvstride = (size_t)g.Hkv * D;
  const int e = chunk * 1024 + threadIdx.x * 4;
  const int which = e / (BN * D);
  const int kvloc = (e % (BN * D)) / D, col = e % D;
  if (t0 + kvloc >= g.Skv) return;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < info.x; ++sp) {
    const size_t slot = (size_t)(info.y + sp) * g.Hkv + kvh;
    s += *reinterpret_cast<const f32x4*>(partial + slot * 2 * BN * D + e);
  }
  if (which == 0) s *= g.scale;
  float* dst = (which == 0 ? dk : dv) + ((size_t)b * g.Skv + t0 + kvloc) * kvstride +
               (size_t)kvh * D + col;
  *reinterpret_cast<f32x4*>(dst) = s;
}

hipError_t launch_bwd_dq(int D, const u16* q, const u16* k, const u16* v, const u16* out,
                         const u16* dout, const float* lse, const int32_t* dstart, u16* dq,
                         float* Dbuf, const Geo& g, hipStream_t st) {
  const int nt = (g.Sq * g.G + kFwdBM - 1) / kFwdBM;
  const unsigned grid = (unsigned)nt * g.B * g.Hkv;
  if (D == 128)
    bwd_dq_kernel<128><<<grid, 256, 0, st>>>(q, k, v, out, dout, lse, dstart, dq, Dbuf, g);
  else
    bwd_dq_kernel<64><<<grid, 256, 0, st>>>(q, k, v, out, dout, lse, dstart, dq, Dbuf, g);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(int D, const u16* q, const u16* k, const u16* v, const u16* dout,
                           const float* lse, const int32_t* dstart, const int32_t* dend,
                           const float* Dbuf, SchedHeader* hdr, const int2* tile_info,
                           const int2* items, float* partial, float* dk, float* dv, const Geo& g,
                           int nkt, hipStream_t st) {
  if (D == 128)
    bwd_dkdv_kernel<128><<<kDkdvGrid, 256, 0, st>>>(q, k, v, dout, lse, dstart, dend, Dbuf, hdr,
                                                    tile_info, items, partial, dk, dv, g, nkt);
  else
    bwd_dkdv_kernel<64><<<kDkdvGrid, 256, 0, st>>>(q, k, v, dout, lse, dstart, dend, Dbuf, hdr,
                                                   tile_info, items, partial, dk, dv, g, nkt);
  return hipGetLastError();
}

hipError_t launch_bwd_reduce(int D, const int2* tile_info, const float* partial, float* dk,
                             float* dv, const Geo& g, int nkt, hipStream_t st) {
  const unsigned rgrid = (unsigned)g.B * nkt * g.Hkv * (2 * kDkdvBN * D / 1024);
  if (D == 128)
    bwd_reduce_kernel<128><<<rgrid, 256, 0, st>>>(tile_info, partial, dk, dv, g, nkt);
  else
    bwd_reduce_kernel<64><<<rgrid, 256, 0, st>>>(tile_info, partial, dk, dv, g, nkt);
  return hipGetLastError();
}

}  // namespace dmgqa
