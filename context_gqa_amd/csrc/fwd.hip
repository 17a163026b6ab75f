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
// Layout on gfx950: 4 waves x 32 query rows; rows are (token, head-in-group)
// pairs of one KV head, so one K/V tile in LDS serves all G query heads
// sharing it (GQA).  Scores are held as S^T = K Q^T so that each lane owns
// one query row (two lanes per row, 16 keys each): the row max and sum need
// one cross-lane exchange.  P V is computed as O^T = V^T P^T with V read
// from LDS by transposed reads.
#include "common.hpp"
#include "kernels.hpp"
#include "qtile.hpp"
#include "dma.hpp"

namespace dmgqa {

// Lazy rescaling: the running maximum used as the exponent reference is only
// raised when a row's new maximum exceeds it by more than 2^kRescaleLog2 (in
// exp2 units); otherwise P may reach 2^kRescaleLog2, which bf16 and fp32
// represent exactly as well as values below 1.  out = O / l is unchanged.
constexpr float kRescaleLog2 = 8.f;

template <int D>
__global__ __launch_bounds__(256, 2) void fwd_kernel(const u16* __restrict__ q,
                                                     const u16* __restrict__ k,
                                                     const u16* __restrict__ v,
                                                     const int32_t* __restrict__ dstart,
                                                     u16* __restrict__ out,
                                                     float* __restrict__ lse, Geo g) {
  constexpr int BM = kFwdBM, BN = kFwdBN, KK = D / 16, DB = D / 32;
  // Padded layouts, each conflict-free for its one access pattern on the
  // 64-bank LDS: K is read by ds_read_b128 (16 consecutive rows, one chunk)
  // -> row stride D + 8; V by ds_read_b64_tr_b16 (4 rows x 4 chunks) -> row
  // stride D + 32.  Two stages, each its own array (see dma.hpp).
  constexpr int LDK = D + 8, LDV = D + 32;
  __shared__ __attribute__((aligned(1024))) u16 sK0[BN * LDK];
  __shared__ __attribute__((aligned(1024))) u16 sK1[BN * LDK];
  __shared__ __attribute__((aligned(1024))) u16 sV0[BN * LDV];
  __shared__ __attribute__((aligned(1024))) u16 sV1[BN * LDV];

  const int nrows = g.Sq * g.G;
  const int nt = (nrows + BM - 1) / BM;
  const int nbg = g.B * g.Hkv;
  // heaviest tiles (latest positions) are dispatched first
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

  const size_t qoff = (((size_t)b * g.Sq + tok) * g.Hq + head) * D;
  bf16x8 qop[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) qop[kk] = ld_bf16x8(q + qoff + 8 * h + 16 * kk);

  const QTileKeys kr = qtile_keys<BM, BN>(row0, ds, g);
  const int ntiles = kr.na + kr.nb;

  float m = -INFINITY, l = 0.f;
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = zero16();

  const size_t kvstride = (size_t)g.Hkv * D;
  const u16* kbase = k + (size_t)b * g.Skv * kvstride + (size_t)kvh * D;
  const u16* vbase = v + (size_t)b * g.Skv * kvstride + (size_t)kvh * D;
  PadTileDma<BN, D, LDK, 4> dmak;
  PadTileDma<BN, D, LDV, 4> dmav;
  dmak.init((unsigned)kvstride, wave, lane);
  dmav.init((unsigned)kvstride, wave, lane);
  auto issue = [&](int it, u16* dK, u16* dV) __attribute__((always_inline)) {
    const int t0 = uniform((it < kr.na ? kr.a0 + it : kr.b0 + (it - kr.na)) * BN);
    dmak.issue(kbase, (unsigned)kvstride, t0, g.Skv - 1, dK, wave, lane);
    dmav.issue(vbase, (unsigned)kvstride, t0, g.Skv - 1, dV, wave, lane);
  };
  issue(0, sK0, sV0);
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();

  auto step = [&](int it, const u16* cK, const u16* cV, u16* nK, u16* nV)
                  __attribute__((always_inline)) {
    const int t0 = (it < kr.na ? kr.a0 + it : kr.b0 + (it - kr.na)) * BN;
    if (it + 1 < ntiles) issue(it + 1, nK, nV);

    // K operands for all k-steps are read up front (2*KK LDS reads in
    // flight), so LDS latency overlaps the MFMA chain.
    bf16x8 kf0[KK], kf1[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      kf0[kk] = lds_bf16x8(&cK[i * LDK + 8 * h + 16 * kk]);
      kf1[kk] = lds_bf16x8(&cK[(32 + i) * LDK + 8 * h + 16 * kk]);
    }
    f32x16 s0 = zero16(), s1 = zero16();
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      s0 = mfma32(kf0[kk], qop[kk], s0);
      s1 = mfma32(kf1[kk], qop[kk], s1);
    }
    sched_reads_ahead<2 * KK, KK, 2>();
    const bool full = kr.max_lo <= t0 && t0 + BN - 1 <= kr.min_pos;
    if (!full) {
      // allowed keys lo..pos relative to this lane's first key t0 + 4h;
      // register r holds key offset 8*(r/4) + r%4 (+32 for s1)
      const int lo_rel = lo - (t0 + 4 * h), hi_rel = pos - (t0 + 4 * h);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = 8 * (r >> 2) + (r & 3);
        if (c < lo_rel || c > hi_rel) s0[r] = -INFINITY;
        if (c + 32 < lo_rel || c + 32 > hi_rel) s1[r] = -INFINITY;
      }
    }
    float mx = max3f(s0[0], s1[0], s0[1]);
#pragma unroll
    for (int r = 1; r < 15; ++r) mx = max3f(mx, s1[r], s0[r + 1]);
    mx = max3f(mx, s1[15], s1[15]);
    mx = fmaxf(mx, xor32(mx));
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
      for (int db = 0; db < DB; ++db)
        o[db] = mfma32(tr_operand_pad<LDV>(cV, 0, ks, 32 * db, lane), pop, o[db]);
    }
    l += rs0 + rs1;
    // this wave's loads of the next tile are done; after the barrier every
    // wave's are, and every wave has finished reading the current stage
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
  };
  for (int it = 0; it < ntiles; it += 2) {
    step(it, sK0, sV0, sK1, sV1);
    if (it + 1 < ntiles) step(it + 1, sK1, sV1, sK0, sV0);
  }

  const float lt = l + xor32(l);
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
                      u16* out, float* lse, const Geo& g, hipStream_t st) {
  const int nt = (g.Sq * g.G + kFwdBM - 1) / kFwdBM;
  const unsigned grid = (unsigned)nt * g.B * g.Hkv;
  if (D == 128)
    fwd_kernel<128><<<grid, 256, 0, st>>>(q, k, v, dstart, out, lse, g);
  else
    fwd_kernel<64><<<grid, 256, 0, st>>>(q, k, v, dstart, out, lse, g);
  return hipGetLastError();
}

}  // namespace dmgqa
