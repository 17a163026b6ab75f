// Document bounds and the dK/dV work schedule.
//
// For every key position t < Skv of every batch row the prep kernels write
//   dstart[t] = first position of t's document
//   dend[t]   = one past the last position of t's document, capped at Skv.
// With packed documents (each id one contiguous run) the document mask of
// "Paper notes: The Llama 3 Herd of Models" ("Two architectural choices",
// no attention across document boundaries) together with the causal mask
// becomes an interval per query position p: keys dstart[p] .. p.  The
// attention kernels read these arrays instead of comparing document ids.
#include "common.hpp"
#include "kernels.hpp"

namespace dmgqa {

constexpr int kScanThreads = 1024;

// Inclusive block-wide scan with max (forward) of `v`.
__device__ int block_scan_max(int v, int* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int u = __shfl_up(v, o);
    if (lane >= o) v = max(v, u);
  }
  if (lane == 63) sh[wave] = v;
  __syncthreads();
  if (wave == 0) {
    int w = lane < (kScanThreads / 64) ? sh[lane] : INT32_MIN;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      int u = __shfl_up(w, o);
      if (lane >= o) w = max(w, u);
    }
    if (lane < kScanThreads / 64) sh[16 + lane] = w;
  }
  __syncthreads();
  if (wave > 0) v = max(v, sh[16 + wave - 1]);
  __syncthreads();
  return v;
}

// Inclusive block-wide suffix scan with min of `v` (from the last thread).
__device__ int block_rscan_min(int v, int* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int u = __shfl_down(v, o);
    if (lane + o < 64) v = min(v, u);
  }
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  if (wave == 0) {
    int w = lane < (kScanThreads / 64) ? sh[lane] : INT32_MAX;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      int u = __shfl_down(w, o);
      if (lane + o < 16) w = min(w, u);
    }
    if (lane < kScanThreads / 64) sh[16 + lane] = w;
  }
  __syncthreads();
  if (wave < kScanThreads / 64 - 1) v = min(v, sh[16 + wave + 1]);
  __syncthreads();
  return v;
}

// Pass 1: per 1024-position block, the latest document start at or before t
// and the earliest document end after t, within the block; plus the block
// aggregates.  grid = (nblk, B).
__global__ __launch_bounds__(kScanThreads) void prep_scan_local(
    const int32_t* __restrict__ doc, int S, int Skv, int nblk,
    int32_t* __restrict__ dstart, int32_t* __restrict__ dend,
    int32_t* __restrict__ agg_start, int32_t* __restrict__ agg_end) {
  __shared__ int sh[32];
  const int b = blockIdx.y;
  const int t = blockIdx.x * kScanThreads + threadIdx.x;
  const int32_t* d = doc + (size_t)b * S;
  int vs = -1, ve = INT32_MAX;
  if (t < Skv) {
    const int cur = d[t];
    if (t == 0 || d[t - 1] != cur) vs = t;
    if (t == Skv - 1 || d[t + 1] != cur) ve = t + 1;
  }
  const int s = block_scan_max(vs, sh);
  const int e = block_rscan_min(ve, sh);
  if (t < Skv) {
    dstart[(size_t)b * Skv + t] = s;
    dend[(size_t)b * Skv + t] = e;
  }
  if (threadIdx.x == kScanThreads - 1) agg_start[b * nblk + blockIdx.x] = s;
  if (threadIdx.x == 0) agg_end[b * nblk + blockIdx.x] = e;
}

// Pass 2: combine with the aggregates of the other blocks.
__global__ __launch_bounds__(kScanThreads) void prep_scan_fix(
    int Skv, int nblk, int32_t* __restrict__ dstart, int32_t* __restrict__ dend,
    const int32_t* __restrict__ agg_start, const int32_t* __restrict__ agg_end) {
  __shared__ int red[2][16];
  const int b = blockIdx.y, blk = blockIdx.x;
  int ps = -1, se = INT32_MAX;
  for (int x = threadIdx.x; x < nblk; x += kScanThreads) {
    if (x < blk) ps = max(ps, agg_start[b * nblk + x]);
    if (x > blk) se = min(se, agg_end[b * nblk + x]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    ps = max(ps, __shfl_xor(ps, o));
    se = min(se, __shfl_xor(se, o));
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) { red[0][wave] = ps; red[1][wave] = se; }
  __syncthreads();
  ps = -1; se = INT32_MAX;
#pragma unroll
  for (int w = 0; w < kScanThreads / 64; ++w) { ps = max(ps, red[0][w]); se = min(se, red[1][w]); }
  const int t = blk * kScanThreads + threadIdx.x;
  if (t < Skv) {
    const size_t i = (size_t)b * Skv + t;
    dstart[i] = max(dstart[i], ps);
    dend[i] = min(dend[i], se);
  }
}

// cu_seqlens form (B == 1): binary search of each position's document.
__global__ __launch_bounds__(256) void prep_cu(const int32_t* __restrict__ cu, int n_docs,
                                               int Skv, int32_t* __restrict__ dstart,
                                               int32_t* __restrict__ dend) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= Skv) return;
  int lo = 0, hi = n_docs - 1;  // find the last i with cu[i] <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  dstart[t] = cu[lo];
  dend[t] = min(cu[lo + 1], Skv);
}

// Interval masks: query position p attends to keys lo[p] .. p, lo
// non-decreasing with 0 <= lo[p] <= p (the all-gathered K/V let a CP rank
// apply any mask of this kind: "Scaling Llama 3 Training with Efficient
// Parallelism Strategies", section "Context Parallelism (CP)", Figure 7).
// The document mask is lo = first position of p's document; a sliding
// window of W keys inside documents is lo = max(document start, p - W + 1).
// The attention kernels need the same two arrays as for documents:
//   dstart[t] = lo[t]
//   dend[t]   = one past the last query position p with lo[p] <= t, capped
//               at Skv (lo non-decreasing: the first p > t with lo[p] > t,
//               by binary search over (t, S)).
// grid = (ceil(Skv / 256), B).
__global__ __launch_bounds__(256) void prep_interval(const int32_t* __restrict__ lo, int S,
                                                     int Skv, int32_t* __restrict__ dstart,
                                                     int32_t* __restrict__ dend) {
  const int b = blockIdx.y;
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= Skv) return;
  const int32_t* l = lo + (size_t)b * S;
  dstart[(size_t)b * Skv + t] = l[t];
  int a = t + 1, z = S;   // first p in [t+1, S) with l[p] > t, or S
  while (a < z) {
    const int mid = (a + z) >> 1;
    if (l[mid] > t) z = mid; else a = mid + 1;
  }
  dend[(size_t)b * Skv + t] = min(a, Skv);
}

// One block (kScanThreads threads).  For every (batch, key tile): the
// number of query rows (local tokens x group heads) that reach it; then a
// split of those rows into pieces of `rows_per_split` (chosen so the total
// stays under kMaxSplitBase), the work-item list and the partial-sum slots.
__device__ void sched_body(const int32_t* __restrict__ kfirst, const int32_t* __restrict__ dend,
                           const Geo& g, int nkt, int max_split_base, int stash_budget,
                           SchedHeader* __restrict__ hdr,
                           int2* __restrict__ tile_info, int2* __restrict__ items,
                           int4* __restrict__ tile_rows) {
  __shared__ int sh[32];
  __shared__ long long red[16];
  const int ntiles = g.B * nkt;
  const int per = (ntiles + kScanThreads - 1) / kScanThreads;
  const int first = threadIdx.x * per;
  // 1. rows per tile and the total
  long long tot = 0;
  for (int x = first; x < min(first + per, ntiles); ++x) {
    const int b = x / nkt, kt = x % nkt;
    int a0, na, b0, nb;
    key_tile_tokens(kfirst ? kfirst + (size_t)b * g.Skv : nullptr, dend + (size_t)b * g.Skv, kt,
                    g, a0, na, b0, nb);
    tot += (long long)(na + nb) * g.G;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) tot += __shfl_xor(tot, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = tot;
  __syncthreads();
  long long total = 0;
  for (int w = 0; w < kScanThreads / 64; ++w) total += red[w];
  long long rps = (total + max_split_base - 1) / max_split_base;
  if (rps < kMinRowsPerSplit) rps = kMinRowsPerSplit;
  rps = (rps + kDkdvBM - 1) / kDkdvBM * kDkdvBM;
  // 2. splits per tile: rows / rps full splits and at most one shorter
  //    remainder (a tile no row reaches gets one empty item, which writes
  //    its zero gradients).  Items are listed largest first, so that the
  //    persistent workgroups, taking them in order, end close together: all
  //    full splits in tile order, then the remainders by decreasing size
  //    (64 size classes; order within a class is arbitrary and does not
  //    affect results, which depend only on (tile, split)).
  __shared__ int bucket_cnt[64], bucket_base[64];
  if (threadIdx.x < 64) bucket_cnt[threadIdx.x] = 0;
  __syncthreads();
  auto remainder_class = [&](long long rem) { return 63 - (int)min(63LL, rem * 64 / rps); };
  int my_full = 0, my_slots = 0, my_blocks = 0;
  for (int x = first; x < min(first + per, ntiles); ++x) {
    const int b = x / nkt, kt = x % nkt;
    int a0, na, b0, nb;
    key_tile_tokens(kfirst ? kfirst + (size_t)b * g.Skv : nullptr, dend + (size_t)b * g.Skv, kt,
                    g, a0, na, b0, nb);
    const long long rows = (long long)(na + nb) * g.G;
    const int nf = (int)(rows / rps);
    const long long rem = rows - (long long)nf * rps;
    const int ns = nf + ((rem > 0 || rows == 0) ? 1 : 0);
    my_full += nf;
    my_slots += ns > 1 ? ns : 0;
    // (without a stash nothing is counted: the host bounds the block sums
    // below 2^31 only when it reserves one)
    if (stash_budget > 0) my_blocks += stash_blocks(a0, na, b0, nb, g);
    if (rem > 0 || rows == 0) atomicAdd(&bucket_cnt[remainder_class(rem)], 1);
  }
  __shared__ int scan_i[kScanThreads], scan_s[kScanThreads], scan_b[kScanThreads];
  scan_i[threadIdx.x] = my_full;
  scan_s[threadIdx.x] = my_slots;
  scan_b[threadIdx.x] = my_blocks;
  __syncthreads();
  const int tx = threadIdx.x;
  for (int o = 1; o < kScanThreads; o <<= 1) {
    int vi = tx >= o ? scan_i[tx - o] : 0;
    int vs = tx >= o ? scan_s[tx - o] : 0;
    int vb = tx >= o ? scan_b[tx - o] : 0;
    __syncthreads();
    scan_i[threadIdx.x] += vi;
    scan_s[threadIdx.x] += vs;
    scan_b[threadIdx.x] += vb;
    __syncthreads();
  }
  const int n_full = scan_i[kScanThreads - 1];
  if (threadIdx.x == 0) {
    int acc = n_full;
    for (int c = 0; c < 64; ++c) {
      bucket_base[c] = acc;
      acc += bucket_cnt[c];
      bucket_cnt[c] = 0;
    }
  }
  __syncthreads();
  int item = scan_i[threadIdx.x] - my_full;
  int slot = scan_s[threadIdx.x] - my_slots;
  int sblk = scan_b[threadIdx.x] - my_blocks;
  int n_items_mine = 0;
  for (int x = first; x < min(first + per, ntiles); ++x) {
    const int b = x / nkt, kt = x % nkt;
    int a0, na, b0, nb;
    key_tile_tokens(kfirst ? kfirst + (size_t)b * g.Skv : nullptr, dend + (size_t)b * g.Skv, kt,
                    g, a0, na, b0, nb);
    const long long rows = (long long)(na + nb) * g.G;
    const int nf = (int)(rows / rps);
    const long long rem = rows - (long long)nf * rps;
    const bool has_rem = rem > 0 || rows == 0;
    const int ns = nf + (has_rem ? 1 : 0);
    tile_info[x] = make_int2(ns, ns > 1 ? slot : -1);
    {
      // stashed while the tile's blocks fit in the budget: a prefix of the
      // tiles in (batch row, key tile) order, since sblk only grows
      const int tlo = na > 0 ? a0 : b0, thi = nb > 0 ? b0 + nb : a0 + na;
      const int nblk = stash_budget > 0 ? stash_blocks(a0, na, b0, nb, g) : 0;
      const bool fits = stash_budget > 0 && (long long)sblk + nblk <= (long long)stash_budget;
      tile_rows[x] = make_int4(tlo, thi, tlo * g.G / kStashRows, fits ? sblk : -1);
      sblk += nblk;
    }
    for (int s = 0; s < nf; ++s) items[item + s] = make_int2(x, s);
    item += nf;
    if (has_rem) {
      const int c = remainder_class(rem);
      items[bucket_base[c] + atomicAdd(&bucket_cnt[c], 1)] = make_int2(x, nf);
    }
    n_items_mine += ns;
    slot += ns > 1 ? ns : 0;
  }
  // total item count
  scan_i[threadIdx.x] = n_items_mine;
  __syncthreads();
  for (int o = kScanThreads / 2; o > 0; o >>= 1) {
    if (tx < o) scan_i[tx] += scan_i[tx + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    hdr->n_base_items = scan_i[0];
    hdr->rows_per_split = (int)rps;
    hdr->n_slots_base = scan_s[kScanThreads - 1];
    hdr->counter = 0;
  }
  (void)sh;
}

// Cross-attention: query position p attends to keys lo[p] .. hi[p]-1 with lo
// and hi non-decreasing and lo[p] < hi[p] (keys indexed apart from the
// queries).  The positions that reach key t are then one contiguous run:
// {p : hi[p] > t} is a suffix of the positions and {p : lo[p] <= t} a
// prefix, so the run is [kfirst[t], kend[t]) with kfirst[t] the first p with
// hi[p] > t and kend[t] the first p with lo[p] > t (S if none); empty when
// kfirst[t] >= kend[t].  Two binary searches per key.  grid = (ceil(Skv /
// 256), B).
__global__ __launch_bounds__(256) void prep_cross_keys(const int32_t* __restrict__ lo,
                                                       const int32_t* __restrict__ hi, int S,
                                                       int Skv, int32_t* __restrict__ kfirst,
                                                       int32_t* __restrict__ kend) {
  const int b = blockIdx.y;
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= Skv) return;
  const int32_t* l = lo + (size_t)b * S;
  const int32_t* h = hi + (size_t)b * S;
  int a = 0, z = S;   // first p with h[p] > t
  while (a < z) {
    const int mid = (a + z) >> 1;
    if (h[mid] > t) z = mid; else a = mid + 1;
  }
  kfirst[(size_t)b * Skv + t] = a;
  a = 0; z = S;       // first p with l[p] > t
  while (a < z) {
    const int mid = (a + z) >> 1;
    if (l[mid] > t) z = mid; else a = mid + 1;
  }
  kend[(size_t)b * Skv + t] = a;
}

// ---------------------------------------------------------------- fp16 scales
//
// The dK/dV kernel multiplies dO with V (dP) and P with dO (dV) in fp16:
// fp16 carries 11 significant bits (bf16: 8), enough for P in the dV sum
// over every row of a KV group, but only 5 exponent bits.  dO and V are
// therefore scaled by powers of two chosen per call, eo and ev, so that the
// largest magnitude of each lies in [2^14, 2^15): bf16 values down to
// 2^-28 of the maximum stay exact, smaller ones keep an absolute error
// below 2^-39 of the maximum.  The scales are exact, and undone exactly at
// the end (dk_mul, dv_mul of SchedHeader).

// Partial maxima of the bf16 magnitude bits (sign cleared: for finite values
// the bit order is the value order) of dO and V: kScaleParts blocks of
// kScaleThreads threads, each thread keeping eight 16-byte loads in flight
// over its strided share of each tensor.
constexpr int kScaleThreads = 256;
constexpr int kScaleUnroll = 8;

__device__ __forceinline__ unsigned max_mag8(uint4 w, unsigned m) {
  const unsigned ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) m = max(m, max(ws[e] & 0x7fffu, (ws[e] >> 16) & 0x7fffu));
  return m;
}

__global__ __launch_bounds__(kScaleThreads) void scale_scan(const u16* __restrict__ dout,
                                                            long long n_dout,
                                                            const u16* __restrict__ v,
                                                            long long n_v,
                                                            int2* __restrict__ parts) {
  __shared__ int red[2][kScaleThreads / 64];
  const long long step = (long long)kScaleParts * kScaleThreads * 8;   // elements per pass
  const long long first = ((long long)blockIdx.x * kScaleThreads + threadIdx.x) * 8;
  auto scan = [&](const u16* x, long long n) {
    unsigned m = 0;
    long long i = first;
    // whole groups of kScaleUnroll loads
    for (; i + (kScaleUnroll - 1) * step + 8 <= n; i += kScaleUnroll * step) {
      uint4 w[kScaleUnroll];
#pragma unroll
      for (int u = 0; u < kScaleUnroll; ++u)
        w[u] = *reinterpret_cast<const uint4*>(x + i + u * step);
#pragma unroll
      for (int u = 0; u < kScaleUnroll; ++u) m = max_mag8(w[u], m);
    }
    for (; i < n; i += step) {
      if (i + 8 <= n)
        m = max_mag8(*reinterpret_cast<const uint4*>(x + i), m);
      else
        for (long long t = i; t < n; ++t) m = max(m, (unsigned)(x[t] & 0x7fffu));
    }
    return m;
  };
  unsigned mo = scan(dout, n_dout);
  unsigned mv = scan(v, n_v);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mo = max(mo, (unsigned)__shfl_xor((int)mo, o));
    mv = max(mv, (unsigned)__shfl_xor((int)mv, o));
  }
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = (int)mo;
    red[1][threadIdx.x >> 6] = (int)mv;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int a = 0, b = 0;
    for (int w = 0; w < kScaleThreads / 64; ++w) { a = max(a, red[0][w]); b = max(b, red[1][w]); }
    parts[blockIdx.x] = make_int2(a, b);
  }
}

// 2^e placing the largest magnitude (bf16 bits m, sign cleared) in
// [2^14, 2^15): e = 14 - floor(log2 max); 0 for an all-zero tensor; the
// exponent field of a subnormal counts as -126.  Kept within [-100, 100].
__device__ __forceinline__ int scale_exp(unsigned m) {
  if (m == 0) return 0;
  const int e = (int)(m >> 7) - 127;
  return min(max(14 - max(e, -126), -100), 100);
}

// (eo, ev) from the partial maxima, reduced by the first wave; every thread
// of the block gets them.
static_assert(kScaleParts % 64 == 0, "partial maxima per lane");
__device__ int2 scale_exponents(const int2* __restrict__ parts) {
  __shared__ int2 ex;
  if (threadIdx.x < 64) {
    unsigned mo = 0, mv = 0;
#pragma unroll
    for (int k = 0; k < kScaleParts / 64; ++k) {
      const int2 p = parts[threadIdx.x + 64 * k];
      mo = max(mo, (unsigned)p.x);
      mv = max(mv, (unsigned)p.y);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      mo = max(mo, (unsigned)__shfl_xor((int)mo, o));
      mv = max(mv, (unsigned)__shfl_xor((int)mv, o));
    }
    if (threadIdx.x == 0) ex = make_int2(scale_exp(mo), scale_exp(mv));
  }
  __syncthreads();
  return ex;
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Per query row: -lse/scale (start value of the S accumulators of the dK/dV
// kernel, so that P = exp2(scale*log2e * S)), -D * 2^(eo+ev) with
// D = <dO, O> (start value of its dP' accumulators, so that dS' = P * dP'),
// and the row of dO' = dO * 2^eo in fp16.  D/8 lanes per row, one 16-byte
// chunk of out and dout each, kRowstatPasses rows per lane; `blk` indexes
// groups of kRowstatPasses * kScanThreads / (D/8) rows.
constexpr int kRowstatPasses = 4;
template <int D>
__device__ void rowstat_rows(const u16* __restrict__ out, const u16* __restrict__ dout,
                             const float* __restrict__ lse, float* __restrict__ Lbuf,
                             float* __restrict__ Nbuf, u16* __restrict__ dout16, int nrows,
                             float inv_scale, const int2* __restrict__ scale_parts, int blk) {
  constexpr int kLanes = D / 8;
  constexpr int kRowsPass = kScanThreads / kLanes;
  const int j = threadIdx.x % kLanes;
  const int row0 = blk * (kRowsPass * kRowstatPasses) + (int)(threadIdx.x / kLanes);
  // every load of the block's rows is issued before the exponents are read
  bf16x8 o[kRowstatPasses], d[kRowstatPasses];
#pragma unroll
  for (int p = 0; p < kRowstatPasses; ++p) {
    const int rr = min(row0 + p * kRowsPass, nrows - 1);
    o[p] = ld_bf16x8(out + (size_t)rr * D + 8 * j);
    d[p] = ld_bf16x8(dout + (size_t)rr * D + 8 * j);
  }
  const int2 ex = scale_exponents(scale_parts);
  const float so = __builtin_amdgcn_ldexpf(1.f, ex.x);
  const float sn = -__builtin_amdgcn_ldexpf(1.f, ex.x + ex.y);
#pragma unroll
  for (int p = 0; p < kRowstatPasses; ++p) {
    const int row = row0 + p * kRowsPass;
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)o[p][e], (float)d[p][e], acc);
#pragma unroll
    for (int o2 = kLanes / 2; o2 > 0; o2 >>= 1) acc += __shfl_xor(acc, o2, kLanes);
    if (row < nrows) {
      unsigned w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f16x2 hp = {(_Float16)((float)d[p][2 * e] * so),
                          (_Float16)((float)d[p][2 * e + 1] * so)};
        w[e] = __builtin_bit_cast(unsigned, hp);
      }
      *reinterpret_cast<uint4*>(dout16 + (size_t)row * D + 8 * j) =
          make_uint4(w[0], w[1], w[2], w[3]);
      if (j == 0) {
        Nbuf[row] = acc * sn;
        Lbuf[row] = -lse[row] * inv_scale;
      }
    }
  }
}

// Inclusive block-wide scan with + of `v`.
__device__ int block_scan_add(int v, int* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  if (lane == 63) sh[wave] = v;
  __syncthreads();
  if (wave == 0) {
    int w = lane < (kScanThreads / 64) ? sh[lane] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      int u = __shfl_up(w, o);
      if (lane >= o) w += u;
    }
    if (lane < kScanThreads / 64) sh[16 + lane] = w;
  }
  __syncthreads();
  if (wave > 0) v += sh[16 + wave - 1];
  __syncthreads();
  return v;
}

// Dispatch order of the query tiles of the forward (BN = kFwdBN) or dQ
// (BN = kDkdvBN) kernel: the B * nt items (batch row, tile) sorted by
// decreasing cost, the number of BN-key tiles the tile's rows reach
// (heaviest first, the longest-processing-time rule, so that the long tiles
// of long documents do not start last).  A counting sort over kOrderBins
// cost classes (costs beyond the last class share it); items of one class
// keep no particular order.  Only which workgroup computes a tile changes,
// never its result.  One block of kScanThreads threads.
constexpr int kOrderBins = 4096;
static_assert(kOrderBins % kScanThreads == 0, "bins per thread");

template <int BN, bool CROSS = false>
__device__ void tile_order_body(const int32_t* __restrict__ dstart, const Geo& g,
                                int32_t* __restrict__ order,
                                const int32_t* __restrict__ dhi = nullptr) {
  __shared__ int cnt[kOrderBins];
  __shared__ int sh[32];
  constexpr int BM = kFwdBM;
  const int nt = (g.Sq * g.G + BM - 1) / BM;
  const int n = g.B * nt;
  for (int i = threadIdx.x; i < kOrderBins; i += kScanThreads) cnt[i] = 0;
  __syncthreads();
  // class 0 holds the heaviest items
  auto cls = [&](int x) {
    const int b = x / nt, t = x - b * nt;
    const QTileKeys kr =
        CROSS ? qtile_keys_iv<BM, BN>(t * BM, dstart + (size_t)b * g.S, dhi + (size_t)b * g.S, g)
              : qtile_keys<BM, BN>(t * BM, dstart + (size_t)b * g.Skv, g);
    return kOrderBins - 1 - min(kr.na + kr.nb, kOrderBins - 1);
  };
  // the classes of the first kKeep items of each thread stay in registers
  constexpr int kKeep = 4;
  int keep[kKeep];
#pragma unroll
  for (int e = 0; e < kKeep; ++e) {
    const int x = threadIdx.x + e * kScanThreads;
    keep[e] = x < n ? cls(x) : 0;
  }
#pragma unroll
  for (int e = 0; e < kKeep; ++e)
    if ((int)threadIdx.x + e * kScanThreads < n) atomicAdd(&cnt[keep[e]], 1);
  for (int x = threadIdx.x + kKeep * kScanThreads; x < n; x += kScanThreads)
    atomicAdd(&cnt[cls(x)], 1);
  __syncthreads();
  // exclusive prefix sum over the classes (thread i owns classes per*i ..)
  constexpr int per = kOrderBins / kScanThreads;
  int loc[per];
  int tot = 0;
#pragma unroll
  for (int e = 0; e < per; ++e) {
    loc[e] = tot;
    tot += cnt[per * threadIdx.x + e];
  }
  const int base = block_scan_add(tot, sh) - tot;
#pragma unroll
  for (int e = 0; e < per; ++e) cnt[per * threadIdx.x + e] = base + loc[e];
  __syncthreads();
#pragma unroll
  for (int e = 0; e < kKeep; ++e) {
    const int x = threadIdx.x + e * kScanThreads;
    if (x < n) order[atomicAdd(&cnt[keep[e]], 1)] = x;
  }
  for (int x = threadIdx.x + kKeep * kScanThreads; x < n; x += kScanThreads)
    order[atomicAdd(&cnt[cls(x)], 1)] = x;
}

__global__ __launch_bounds__(kScanThreads) void tile_order_fwd(const int32_t* __restrict__ dstart,
                                                               Geo g, int32_t* __restrict__ order) {
  tile_order_body<kFwdBN>(dstart, g, order);
}

// The same for interval masks with explicit ends (dstart, dhi [B, S]).
__global__ __launch_bounds__(kScanThreads) void tile_order_fwd_iv(
    const int32_t* __restrict__ dstart, const int32_t* __restrict__ dhi, Geo g,
    int32_t* __restrict__ order) {
  tile_order_body<kFwdBN, true>(dstart, g, order, dhi);
}

// Plan of one batch layout: the bounds (the scans above) and both query-tile
// orders (forward, BN = kFwdBN; dQ, BN = kDkdvBN) that the attention calls
// read instead of computing them per call.  (Single-workgroup kernels for
// bounds and orders together measured 19 us, with strided reads of the ids,
// and 23 us, with eight ids per thread scanned in registers and the bounds
// kept in LDS for the orders, against 17 us for the scans and this launch:
// the two counting sorts, which run side by side here, then run one after
// the other.)

// Both orders from bounds already written (any B): block 0 the forward's,
// block 1 the dQ kernel's.
__global__ __launch_bounds__(kScanThreads) void plan_orders(const int32_t* __restrict__ dstart,
                                                            Geo g, int32_t* __restrict__ fwd_order,
                                                            int32_t* __restrict__ dq_order) {
  if (blockIdx.x == 0)
    tile_order_body<kFwdBN>(dstart, g, fwd_order);
  else
    tile_order_body<kDkdvBN>(dstart, g, dq_order);
}

// The dK/dV schedule and the fp16 scales (block 0), the dQ tile order
// (block 1, unless dq_order is null) and the row statistics (the other
// blocks) in one launch: the single-block parts run beside the row
// statistics.
template <int D, bool CROSS>
__global__ __launch_bounds__(kScanThreads) void sched_rowstat(
    const int32_t* __restrict__ kfirst, const int32_t* __restrict__ dstart,
    const int32_t* __restrict__ dhi,
    const int32_t* __restrict__ dend, Geo g, int nkt, int max_split_base, int stash_budget,
    SchedHeader* __restrict__ hdr, int2* __restrict__ tile_info, int2* __restrict__ items,
    int4* __restrict__ tile_rows, int32_t* __restrict__ dq_order, const u16* __restrict__ out,
    const u16* __restrict__ dout, const float* __restrict__ lse,
    const int2* __restrict__ scale_parts, float* __restrict__ Lbuf, float* __restrict__ Nbuf,
    u16* __restrict__ dout16) {
  if (blockIdx.x == 0) {
    const int2 ex = scale_exponents(scale_parts);
    sched_body(kfirst, dend, g, nkt, max_split_base, stash_budget, hdr, tile_info, items,
               tile_rows);
    if (threadIdx.x == 0) {
      hdr->eo = ex.x;
      hdr->ev = ex.y;
      hdr->dk_mul = __builtin_amdgcn_ldexpf(1.f, -(ex.x + ex.y));
      hdr->dv_mul = __builtin_amdgcn_ldexpf(1.f, -ex.x);
    }
  } else if (blockIdx.x == 1) {
    if (dq_order != nullptr) tile_order_body<kDkdvBN, CROSS>(dstart, g, dq_order, dhi);
  } else {
    rowstat_rows<D>(out, dout, lse, Lbuf, Nbuf, dout16, g.B * g.Sq * g.Hq, 1.f / g.scale,
                    scale_parts, (int)blockIdx.x - 2);
  }
}

// ---------------------------------------------------------------- launchers

hipError_t launch_prep_docs(const int32_t* doc, int B, int S, int Skv, int32_t* dstart,
                            int32_t* dend, int32_t* agg, hipStream_t st) {
  const int nblk = (Skv + kScanThreads - 1) / kScanThreads;
  dim3 grid(nblk, B);
  prep_scan_local<<<grid, kScanThreads, 0, st>>>(doc, S, Skv, nblk, dstart, dend, agg,
                                                 agg + (size_t)B * nblk);
  prep_scan_fix<<<grid, kScanThreads, 0, st>>>(Skv, nblk, dstart, dend, agg,
                                               agg + (size_t)B * nblk);
  return hipGetLastError();
}

hipError_t launch_prep_interval(const int32_t* lo, int B, int S, int Skv, int32_t* dstart,
                                int32_t* dend, hipStream_t st) {
  dim3 grid((Skv + 255) / 256, B);
  prep_interval<<<grid, 256, 0, st>>>(lo, S, Skv, dstart, dend);
  return hipGetLastError();
}

hipError_t launch_prep_cu(const int32_t* cu, int n_docs, int Skv, int32_t* dstart, int32_t* dend,
                          hipStream_t st) {
  prep_cu<<<(Skv + 255) / 256, 256, 0, st>>>(cu, n_docs, Skv, dstart, dend);
  return hipGetLastError();
}

hipError_t launch_prep_cross_keys(const int32_t* lo, const int32_t* hi, int B, int S, int Skv,
                                  int32_t* kfirst, int32_t* kend, hipStream_t st) {
  dim3 grid((Skv + 255) / 256, B);
  prep_cross_keys<<<grid, 256, 0, st>>>(lo, hi, S, Skv, kfirst, kend);
  return hipGetLastError();
}

hipError_t launch_sched_rowstat(int D, const int32_t* kfirst, const int32_t* dstart,
                                const int32_t* dhi, const int32_t* dend, const Geo& g, int nkt,
                                int max_split_base, int stash_budget, SchedHeader* hdr,
                                int2* tile_info, int2* items, int4* tile_rows, int32_t* dq_order,
                                const u16* out, const u16* dout, const float* lse,
                                const int2* scale_parts, float* Lbuf, float* Nbuf, u16* dout16,
                                hipStream_t st) {
  const int nrows = g.B * g.Sq * g.Hq;
  const int rows_per_block = kScanThreads / (D / 8) * kRowstatPasses;
  const unsigned grid = 2u + (unsigned)((nrows + rows_per_block - 1) / rows_per_block);
#define DMGQA_RS(DD, CC)                                                                      \
  sched_rowstat<DD, CC><<<grid, kScanThreads, 0, st>>>(                                      \
      kfirst, dstart, dhi, dend, g, nkt, max_split_base, stash_budget, hdr, tile_info, items, \
      tile_rows, dq_order, out, dout, lse, scale_parts, Lbuf, Nbuf, dout16)
  if (D == 128) {
    if (dhi) DMGQA_RS(128, true); else DMGQA_RS(128, false);
  } else {
    if (dhi) DMGQA_RS(64, true); else DMGQA_RS(64, false);
  }
#undef DMGQA_RS
  return hipGetLastError();
}

hipError_t launch_scale_scan(const u16* dout, long long n_dout, const u16* v, long long n_v,
                             int2* parts, hipStream_t st) {
  scale_scan<<<kScaleParts, kScaleThreads, 0, st>>>(dout, n_dout, v, n_v, parts);
  return hipGetLastError();
}

hipError_t launch_plan_orders(const int32_t* dstart, const Geo& g, int32_t* fwd_order,
                              int32_t* dq_order, hipStream_t st) {
  plan_orders<<<2, kScanThreads, 0, st>>>(dstart, g, fwd_order, dq_order);
  return hipGetLastError();
}

hipError_t launch_tile_order_fwd(const int32_t* dstart, const int32_t* dhi, const Geo& g,
                                 int32_t* order, hipStream_t st) {
  if (dhi)
    tile_order_fwd_iv<<<1, kScanThreads, 0, st>>>(dstart, dhi, g, order);
  else
    tile_order_fwd<<<1, kScanThreads, 0, st>>>(dstart, g, order);
  return hipGetLastError();
}

}  // namespace dmgqa
