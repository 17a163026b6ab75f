// Sum of the partial dK/dV slots of the split key tiles (device part,
// shared by the reduce kernel and the dQ-from-stash kernel, which runs the
// same work in workgroups appended to its grid).
#pragma once
#include "common.hpp"
#include "kernels.hpp"

namespace dmgqa {

// Workgroups (256 threads) of the reduce: one per (key tile, KV head,
// 1024-float chunk of its dK and dV).
template <int D>
__host__ __device__ constexpr int reduce_chunks() { return 2 * kDkdvBN * D / 1024; }
template <int D>
inline unsigned reduce_grid(const Geo& g, int nkt) {
  return (unsigned)g.B * nkt * g.Hkv * reduce_chunks<D>();
}

// Workgroup `blk`: adds the tile's partial slots in item order (so the
// result does not depend on timing) and writes dK or dV (scaled).
template <int D>
__device__ __forceinline__ void reduce_partials(const int2* __restrict__ tile_info,
                                                const float* __restrict__ partial,
                                                float* __restrict__ dk, float* __restrict__ dv,
                                                const SchedHeader* __restrict__ hdr,
                                                const Geo& g, int nkt, int blk) {
  constexpr int BN = kDkdvBN;
  constexpr int kChunks = reduce_chunks<D>();
  const int chunk = blk % kChunks;
  const int th = blk / kChunks;
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
  // the partial sums of dK and dV carry the fp16 scales (SchedHeader)
  s *= which == 0 ? g.scale * hdr->dk_mul : hdr->dv_mul;
  float* dst = (which == 0 ? dk : dv) + ((size_t)b * g.Skv + t0 + kvloc) * kvstride +
               (size_t)kvh * D + col;
  *reinterpret_cast<f32x4*>(dst) = s;
}

}  // namespace dmgqa
