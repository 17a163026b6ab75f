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
//   bwd_dq    query-stationary, same tiling as the forward; it also stores
//             -D and -lse/scale per row for the dK/dV kernel.
//   bwd_reduce adds the partial sums of split key tiles in item order, so the
//             result does not depend on which workgroup ran which item.
#include "common.hpp"
#include "kernels.hpp"
#include "qtile.hpp"
#include "reduce.hpp"
#include "tileload.hpp"

namespace dmgqa {

template <int D>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    const u16* __restrict__ out, const u16* __restrict__ dout, const float* __restrict__ lse,
    const int32_t* __restrict__ dstart, u16* __restrict__ dq, float* __restrict__ Lbuf,
    float* __restrict__ Nbuf, Geo g) {
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
  const float lse_v = lse[roff];
  if (valid && h == 0) {   // row statistics for the dK/dV kernel
    Nbuf[roff] = -Dv;
    Lbuf[roff] = -lse_v / g.scale;
  }
  const float lse2 = lse_v * kLog2e;

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

// Sum of the partial slots of each split key tile, in item order.
template <int D>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const int2* __restrict__ tile_info,
                                                         const float* __restrict__ partial,
                                                         float* __restrict__ dk,
                                                         float* __restrict__ dv, Geo g, int nkt) {
  reduce_partials<D>(tile_info, partial, dk, dv, g, nkt, (int)blockIdx.x);
}

hipError_t launch_bwd_dq(int D, const u16* q, const u16* k, const u16* v, const u16* out,
                         const u16* dout, const float* lse, const int32_t* dstart, u16* dq,
                         float* Lbuf, float* Nbuf, const Geo& g, hipStream_t st) {
  const int nt = (g.Sq * g.G + kFwdBM - 1) / kFwdBM;
  const unsigned grid = (unsigned)nt * g.B * g.Hkv;
  if (D == 128)
    bwd_dq_kernel<128><<<grid, 256, 0, st>>>(q, k, v, out, dout, lse, dstart, dq, Lbuf, Nbuf, g);
  else
    bwd_dq_kernel<64><<<grid, 256, 0, st>>>(q, k, v, out, dout, lse, dstart, dq, Lbuf, Nbuf, g);
  return hipGetLastError();
}

hipError_t launch_bwd_reduce(int D, const int2* tile_info, const float* partial, float* dk,
                             float* dv, const Geo& g, int nkt, hipStream_t st) {
  if (D == 128)
    bwd_reduce_kernel<128><<<reduce_grid<128>(g, nkt), 256, 0, st>>>(tile_info, partial, dk, dv,
                                                                      g, nkt);
  else
    bwd_reduce_kernel<64><<<reduce_grid<64>(g, nkt), 256, 0, st>>>(tile_info, partial, dk, dv, g,
                                                                    nkt);
  return hipGetLastError();
}

}  // namespace dmgqa
