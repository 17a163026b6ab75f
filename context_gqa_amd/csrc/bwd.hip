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
// Two kernels here (the dK/dV kernel has its own file):
//   bwd_dq    query-stationary, same tiling as the forward: dQ of every
//             query tile (no stash), or of the key tiles the dS stash does
//             not cover (stash with a budget).
//   bwd_reduce adds the partial sums of split key tiles in item order, so the
//             result does not depend on which workgroup ran which item.
#include "common.hpp"
#include "kernels.hpp"
#include "reduce.hpp"
#include "tileload.hpp"

namespace dmgqa {

// CROSS: query position p reaches keys dstart[p] .. dhi[p]-1 (both [B, S]);
// else keys dstart[p] .. p (dstart [B, Skv]).
// Mixed stash mode (dq_part != null): only query tiles whose last 128-key
// tile has no stash run (the same test as the stash kernel, which then left
// its unscaled sums in dq_part), over the 64-key tiles whose 128-key tile
// has no stash, starting from dq_part.
template <int D, bool CROSS>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    const u16* __restrict__ out, const u16* __restrict__ dout, const float* __restrict__ lse,
    const int32_t* __restrict__ dstart, const int32_t* __restrict__ dhi, u16* __restrict__ dq,
    const int4* __restrict__ tile_rows,
    const float* __restrict__ dq_part, Geo g, int nkt) {
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
  const int32_t* ds = dstart + (size_t)b * (CROSS ? g.S : g.Skv);
  const int32_t* dh = CROSS ? dhi + (size_t)b * g.S : nullptr;
  const int4* trow_b = tile_rows + (size_t)b * nkt;
  if (dq_part != nullptr) {
    const QTileKeys k2 =
        CROSS ? qtile_keys_iv<BM, kDkdvBN>(row0, ds, dh, g) : qtile_keys<BM, kDkdvBN>(row0, ds, g);
    const int kt_last = k2.nb > 0 ? k2.b0 + k2.nb - 1 : k2.a0 + k2.na - 1;
    if (k2.na + k2.nb == 0 || trow_b[kt_last].w >= 0) return;
  }
  const int row = row0 + wave * 32 + i;
  const bool valid = row < nrows;
  const int rr = valid ? row : nrows - 1;
  const int tok = rr / g.G;
  const int head = kvh * g.G + rr % g.G;
  const int pos = local_pos(tok, g.c, g.cp, g.rank);
  const int lo = ds[pos];
  // last key this row reaches
  const int last = CROSS ? dh[pos] - 1 : pos;

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
  const float lse2 = lse[roff] * kLog2e;

  const QTileKeys kr =
      CROSS ? qtile_keys_iv<BM, BN>(row0, ds, dh, g) : qtile_keys<BM, BN>(row0, ds, g);
  const int ntiles = kr.na + kr.nb;

  // accumulator layout: register r of d block db holds column
  // 32 db + 8 (r / 4) + 4 h + r % 4 of this lane's row
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = zero16();
  if (dq_part != nullptr) {
    const float* prow = dq_part + qoff;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 w = *reinterpret_cast<const f32x4*>(prow + 32 * db + 8 * r4 + 4 * h);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[db][4 * r4 + e] = w[e];
      }
  }

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

    // in mixed stash mode the stash kernel has covered the stashed tiles
    const bool skip = dq_part != nullptr && trow_b[t0 / kDkdvBN].w >= 0;
    const bool full = qtile_full(kr, t0, BN);
    // two 32-key halves, to keep the score/dP accumulators at 32 registers
    if (!skip) {
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
          if (kv < lo || kv > last) e0 = 0.f;
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

// Sum of the partial slots of each split key tile, in item order.
template <int D>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const int2* __restrict__ tile_info,
                                                         const float* __restrict__ partial,
                                                         float* __restrict__ dk,
                                                         float* __restrict__ dv,
                                                         const SchedHeader* __restrict__ hdr,
                                                         Geo g, int nkt) {
  reduce_partials<D>(tile_info, partial, dk, dv, hdr, g, nkt, (int)blockIdx.x);
}

hipError_t launch_bwd_dq(int D, const u16* q, const u16* k, const u16* v, const u16* out,
                         const u16* dout, const float* lse, const int32_t* dstart,
                         const int32_t* dhi, u16* dq,
                         const int4* tile_rows, const float* dq_part, const Geo& g, int nkt,
                         hipStream_t st) {
  const int nt = (g.Sq * g.G + kFwdBM - 1) / kFwdBM;
  const unsigned grid = (unsigned)nt * g.B * g.Hkv;
#define DMGQA_DQ(DD, CC)                                                                     \
  bwd_dq_kernel<DD, CC><<<grid, 256, 0, st>>>(q, k, v, out, dout, lse, dstart, dhi, dq,       \
                                              tile_rows, dq_part, g, nkt)
  if (D == 128) {
    if (dhi) DMGQA_DQ(128, true); else DMGQA_DQ(128, false);
  } else {
    if (dhi) DMGQA_DQ(64, true); else DMGQA_DQ(64, false);
  }
#undef DMGQA_DQ
  return hipGetLastError();
}

hipError_t launch_bwd_reduce(int D, const int2* tile_info, const float* partial, float* dk,
                             float* dv, const SchedHeader* hdr, const Geo& g, int nkt,
                             hipStream_t st) {
  if (D == 128)
    bwd_reduce_kernel<128><<<reduce_grid<128>(g, nkt), 256, 0, st>>>(tile_info, partial, dk, dv,
                                                                      hdr, g, nkt);
  else
    bwd_reduce_kernel<64><<<reduce_grid<64>(g, nkt), 256, 0, st>>>(tile_info, partial, dk, dv,
                                                                    hdr, g, nkt);
  return hipGetLastError();
}

}  // namespace dmgqa
