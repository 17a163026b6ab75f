// Tile sizes, workspace records and launcher declarations shared by the
// kernels and the C-ABI entry points.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace dmgqa {

// Tile sizes kFwdBM / kFwdBN (forward and dQ kernels: 128 query rows per
// workgroup of 4 waves, 64 keys per step), kDkdvBN / kDkdvBM (dK/dV kernel:
// 128 keys per work item, 8 waves x 16, query rows streamed 64 at a time)
// and kStashRows are in index.hpp.
// Split of the query rows reaching one key tile into work items: at least
// this many rows per item, and about kMaxSplitTotal split items per call.
// With one split per persistent workgroup a full split is one workgroup's
// even share of the rows, and the remainders fill the rest; on the 405B TP
// share this beat 512 splits (fewer partial slots to add: reduce 22 -> 13
// us) and lost badly at 320 or 384 (a second round of full splits on some
// workgroups).
constexpr int kDkdvGrid = 256;  // persistent workgroups of the dK/dV kernel
constexpr int kMinRowsPerSplit = 512;
constexpr int kMaxSplitTotal = kDkdvGrid;
// dS stash block: kStashRows query rows x kDkdvBN keys, bf16.
constexpr int kStashBlockBytes = kStashRows * kDkdvBN * 2;

struct SchedHeader {
  int n_base_items;    // work items per KV head
  int rows_per_split;  // query rows per item
  int n_slots_base;    // partial-sum slots per KV head
  int counter;         // work counter of the persistent dK/dV kernel
  // Power-of-two scales of the backward's fp16 operands (see
  // launch_scale_scan): dO' = dO * 2^eo and V' = V * 2^ev, so dP' = dO' V'^T
  // and dS' = P (dP' - D') carry 2^(eo+ev); dk_mul = 2^-(eo+ev) and
  // dv_mul = 2^-eo undo them (dK, dQ from dS'; dV from P dO').
  int eo, ev;
  float dk_mul, dv_mul;
  int pad[8];
};

// Per-call exponent scan of the backward: partial maxima of |dO| and |V|
// (bf16 magnitude bits), one int2 per block of kScaleParts blocks; the
// consumers reduce them (scale_exponents in prep.hip).
constexpr int kScaleParts = 512;
hipError_t launch_scale_scan(const u16* dout, long long n_dout, const u16* v, long long n_v,
                             int2* parts, hipStream_t st);

hipError_t launch_prep_docs(const int32_t* doc, int B, int S, int Skv, int32_t* dstart,
                            int32_t* dend, int32_t* agg, hipStream_t st);
hipError_t launch_prep_cu(const int32_t* cu, int n_docs, int Skv, int32_t* dstart, int32_t* dend,
                          hipStream_t st);
// Bounds of an interval mask (keys lo[p] .. p) from lo [B, S].
hipError_t launch_prep_interval(const int32_t* lo, int B, int S, int Skv, int32_t* dstart,
                                int32_t* dend, hipStream_t st);
// Cross-attention key ranges: for every key t of batch row b, the query
// positions that reach it are [kfirst[t], kend[t]) (kfirst = the first p with
// hi[p] > t, kend = the first p with lo[p] > t; lo, hi [B, S] non-decreasing).
hipError_t launch_prep_cross_keys(const int32_t* lo, const int32_t* hi, int B, int S, int Skv,
                                  int32_t* kfirst, int32_t* kend, hipStream_t st);
// The dK/dV schedule (launch_sched_rowstat, block 0) takes the query
// positions that reach key t as [t, dend[t]) (causal interval masks, kfirst
// == nullptr) or [kfirst[t], dend[t]).  stash_budget: dS stash blocks per KV
// head; key tiles are stashed in tile order while their blocks fit
// (tile_rows[x].w = first block, else -1).
// dhi == nullptr: causal interval masks (keys dstart[p] .. p, dstart [B, Skv]);
// else keys dstart[p] .. dhi[p]-1 with dstart, dhi [B, S].
hipError_t launch_fwd(int D, const u16* q, const u16* k, const u16* v, const int32_t* dstart,
                      const int32_t* dhi, const int32_t* order, u16* out, float* lse,
                      const Geo& g, hipStream_t st);
// dQ recomputing S, P and dP.  dhi as for launch_fwd.  With
// dq_part != null only the query tiles that reach a key tile without stash
// (tile_rows[b*nkt + kt].w < 0) run, over those key tiles only, adding to
// the partial sums the stash kernel left in dq_part (fp32 [B, Sq, Hq, D]).
hipError_t launch_bwd_dq(int D, const u16* q, const u16* k, const u16* v, const u16* out,
                         const u16* dout, const float* lse, const int32_t* dstart,
                         const int32_t* dhi, u16* dq,
                         const int4* tile_rows, const float* dq_part, const Geo& g, int nkt,
                         hipStream_t st);
// dout16: dO' in fp16 (the row-statistics pass writes it); Nbuf holds
// -D * 2^(eo+ev).
hipError_t launch_bwd_dkdv(int D, const u16* q, const u16* k, const u16* v, const u16* dout16,
                           const float* Lbuf, const float* Nbuf, const int32_t* kfirst,
                           const int32_t* dend,
                           SchedHeader* hdr, const int2* tile_info, const int2* items,
                           const int4* tile_rows, u16* stash, int stash_kvh_blocks,
                           float* partial, float* dk, float* dv, const Geo& g, int nkt,
                           hipStream_t st);
// Schedule (one block) and per-row statistics (stash path) in one launch.
// Schedule (block 0, with the fp16 scales into hdr), the dQ tile order
// (block 1; skipped when dq_order is null) and the row statistics (the other
// blocks: -lse/scale, -D * 2^(eo+ev), and dO' = dO * 2^eo in fp16 into
// dout16) in one launch.  kfirst: see the schedule note above.  The dQ
// order takes dstart (and dhi, the explicit ends, for cross attention; null
// for causal interval masks) as the forward's order does.
hipError_t launch_sched_rowstat(int D, const int32_t* kfirst, const int32_t* dstart,
                                const int32_t* dhi, const int32_t* dend, const Geo& g, int nkt,
                                int max_split_base, int stash_budget, SchedHeader* hdr,
                                int2* tile_info, int2* items, int4* tile_rows, int32_t* dq_order,
                                const u16* out, const u16* dout, const float* lse,
                                const int2* scale_parts, float* Lbuf, float* Nbuf, u16* dout16,
                                hipStream_t st);
// Heaviest-first dispatch order of the forward's query tiles (one block):
// order[i] = b * nt + tile for B * nt items, nt = ceil(Sq * G / kFwdBM).
// Both query-tile orders of a batch plan from its bounds (two workgroups).
hipError_t launch_plan_orders(const int32_t* dstart, const Geo& g, int32_t* fwd_order,
                              int32_t* dq_order, hipStream_t st);
hipError_t launch_tile_order_fwd(const int32_t* dstart, const int32_t* dhi, const Geo& g,
                                 int32_t* order, hipStream_t st);
// dQ from the dS stash, and (in workgroups appended to its grid) the sum of
// the partial dK/dV slots.  A query tile that also reaches key tiles without
// stash writes its unscaled fp32 partial sums to dq_part instead of dq (only
// when dq_part is not null), for launch_bwd_dq to finish.  dhi as for
// launch_fwd.
hipError_t launch_bwd_dq_stash(int D, const u16* k, const int32_t* dstart, const int32_t* dhi,
                               const int4* tile_rows,
                               const u16* stash, int stash_kvh_blocks, const int32_t* order, u16* dq,
                               float* dq_part, const int2* tile_info, const float* partial,
                               float* dk, float* dv, const SchedHeader* hdr, const Geo& g, int nkt,
                               hipStream_t st);
hipError_t launch_bwd_reduce(int D, const int2* tile_info, const float* partial, float* dk,
                             float* dv, const SchedHeader* hdr, const Geo& g, int nkt,
                             hipStream_t st);

// Kernel timing (benchmark use): when enabled, each launch below is
// bracketed by HIP events recorded on the launch stream.
enum KernelId {
  kKPrep = 0, kKFwd, kKDq, kKDkdv, kKReduce, kKSchedRowstat, kKOrder,
  kKDqRest,   // dQ of the key tiles beyond the stash budget (recomputed)
  kKScale,    // exponent scan of dO and V (fp16 scales)
  kNumKernels
};
void timing_begin(int kernel, hipStream_t st);
void timing_end(int kernel, hipStream_t st);

}  // namespace dmgqa
