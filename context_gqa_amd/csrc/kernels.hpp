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
  int pad[12];
};

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
// dK/dV schedule.  The query positions that reach key t are [t, dend[t])
// (causal interval masks, kfirst == nullptr) or [kfirst[t], dend[t]).
// stash_budget: dS stash blocks per KV head; key tiles are stashed in tile
// order while their blocks fit (tile_rows[x].w = first block, else -1).
hipError_t launch_sched_dkdv(const int32_t* kfirst, const int32_t* dend, const Geo& g, int nkt,
                             int max_split_base, int stash_budget, SchedHeader* hdr,
                             int2* tile_info, int2* items, int4* tile_rows, hipStream_t st);
// dhi == nullptr: causal interval masks (keys dstart[p] .. p, dstart [B, Skv]);
// else keys dstart[p] .. dhi[p]-1 with dstart, dhi [B, S].
hipError_t launch_fwd(int D, const u16* q, const u16* k, const u16* v, const int32_t* dstart,
                      const int32_t* dhi, const int32_t* order, u16* out, float* lse,
                      const Geo& g, hipStream_t st);
// dQ recomputing S, P and dP.  dhi as for launch_fwd.  Lbuf / Nbuf (may be
// null): the row statistics for the dK/dV kernel are stored there.  With
// dq_part != null only the query tiles that reach a key tile without stash
// (tile_rows[b*nkt + kt].w < 0) run, over those key tiles only, adding to
// the partial sums the stash kernel left in dq_part (fp32 [B, Sq, Hq, D]).
hipError_t launch_bwd_dq(int D, const u16* q, const u16* k, const u16* v, const u16* out,
                         const u16* dout, const float* lse, const int32_t* dstart,
                         const int32_t* dhi, u16* dq, float* Lbuf, float* Nbuf,
                         const int4* tile_rows, const float* dq_part, const Geo& g, int nkt,
                         hipStream_t st);
hipError_t launch_bwd_dkdv(int D, const u16* q, const u16* k, const u16* v, const u16* dout,
                           const float* Lbuf, const float* Nbuf, const int32_t* kfirst,
                           const int32_t* dend,
                           SchedHeader* hdr, const int2* tile_info, const int2* items,
                           const int4* tile_rows, u16* stash, int stash_kvh_blocks,
                           float* partial, float* dk, float* dv, const Geo& g, int nkt,
                           hipStream_t st);
// Schedule (one block) and per-row statistics (stash path) in one launch.
hipError_t launch_sched_rowstat(int D, const int32_t* dstart, const int32_t* dend, const Geo& g,
                                int nkt, int max_split_base, int stash_budget,
                                SchedHeader* hdr, int2* tile_info,
                                int2* items, int4* tile_rows, int32_t* dq_order, const u16* out,
                                const u16* dout, const float* lse, float* Lbuf, float* Nbuf,
                                hipStream_t st);
// Heaviest-first dispatch order of the forward's query tiles (one block):
// order[i] = b * nt + tile for B * nt items, nt = ceil(Sq * G / kFwdBM).
hipError_t launch_tile_order_fwd(const int32_t* dstart, const int32_t* dhi, const Geo& g,
                                 int32_t* order, hipStream_t st);
// dQ from the dS stash, and (in workgroups appended to its grid) the sum of
// the partial dK/dV slots.  A query tile that also reaches key tiles without
// stash writes its unscaled fp32 partial sums to dq_part instead of dq (only
// when dq_part is not null), for launch_bwd_dq to finish.
hipError_t launch_bwd_dq_stash(int D, const u16* k, const int32_t* dstart, const int4* tile_rows,
                               const u16* stash, int stash_kvh_blocks, const int32_t* order, u16* dq,
                               float* dq_part, const int2* tile_info, const float* partial,
                               float* dk, float* dv, const Geo& g, int nkt, hipStream_t st);
hipError_t launch_bwd_reduce(int D, const int2* tile_info, const float* partial, float* dk,
                             float* dv, const Geo& g, int nkt, hipStream_t st);

// Kernel timing (benchmark use): when enabled, each launch below is
// bracketed by HIP events recorded on the launch stream.
enum KernelId {
  kKPrep = 0, kKFwd, kKSched, kKDq, kKDkdv, kKReduce, kKSchedRowstat, kKOrder,
  kKDqRest,   // dQ of the key tiles beyond the stash budget (recomputed)
  kNumKernels
};
void timing_begin(int kernel, hipStream_t st);
void timing_end(int kernel, hipStream_t st);

}  // namespace dmgqa
