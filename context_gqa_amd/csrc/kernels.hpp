// Tile sizes, workspace records and launcher declarations shared by the
// kernels and the C-ABI entry points.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace dmgqa {

// Forward and dQ kernels: 128 query rows (tokens x group heads) per
// workgroup of 4 waves (32 rows per wave), 64 keys per step.
constexpr int kFwdBM = 128;
constexpr int kFwdBN = 64;
// dK/dV kernel: 128 keys per work item (8 waves x 16), query rows streamed
// 64 at a time.
constexpr int kDkdvBN = 128;
constexpr int kDkdvBM = 64;
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
// dS stash: blocks of kStashRows query rows (aligned within each KV head's
// row index tok*G + head) x kDkdvBN keys of one key tile, bf16.
constexpr int kStashRows = 32;
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
hipError_t launch_sched_dkdv(const int32_t* dend, const Geo& g, int nkt, int max_split_base,
                             SchedHeader* hdr, int2* tile_info, int2* items, int4* tile_rows,
                             hipStream_t st);
// dhi == nullptr: causal interval masks (keys dstart[p] .. p, dstart [B, Skv]);
// else keys dstart[p] .. dhi[p]-1 with dstart, dhi [B, S].
hipError_t launch_fwd(int D, const u16* q, const u16* k, const u16* v, const int32_t* dstart,
                      const int32_t* dhi, const int32_t* order, u16* out, float* lse,
                      const Geo& g, hipStream_t st);
hipError_t launch_bwd_dq(int D, const u16* q, const u16* k, const u16* v, const u16* out,
                         const u16* dout, const float* lse, const int32_t* dstart, u16* dq,
                         float* Lbuf, float* Nbuf, const Geo& g, hipStream_t st);
hipError_t launch_bwd_dkdv(int D, const u16* q, const u16* k, const u16* v, const u16* dout,
                           const float* Lbuf, const float* Nbuf, const int32_t* dend,
                           SchedHeader* hdr, const int2* tile_info, const int2* items,
                           const int4* tile_rows, u16* stash, int stash_kvh_blocks,
                           float* partial, float* dk, float* dv, const Geo& g, int nkt,
                           hipStream_t st);
// Schedule (one block) and per-row statistics (stash path) in one launch.
hipError_t launch_sched_rowstat(int D, const int32_t* dstart, const int32_t* dend, const Geo& g,
                                int nkt, int max_split_base, SchedHeader* hdr, int2* tile_info,
                                int2* items, int4* tile_rows, int32_t* dq_order, const u16* out,
                                const u16* dout, const float* lse, float* Lbuf, float* Nbuf,
                                hipStream_t st);
// Heaviest-first dispatch order of the forward's query tiles (one block):
// order[i] = b * nt + tile for B * nt items, nt = ceil(Sq * G / kFwdBM).
hipError_t launch_tile_order_fwd(const int32_t* dstart, const int32_t* dhi, const Geo& g,
                                 int32_t* order, hipStream_t st);
// dQ from the dS stash, and (in workgroups appended to its grid) the sum of
// the partial dK/dV slots.
hipError_t launch_bwd_dq_stash(int D, const u16* k, const int32_t* dstart, const int4* tile_rows,
                               const u16* stash, int stash_kvh_blocks, const int32_t* order, u16* dq,
                               const int2* tile_info, const float* partial, float* dk, float* dv,
                               const Geo& g, int nkt, hipStream_t st);
hipError_t launch_bwd_reduce(int D, const int2* tile_info, const float* partial, float* dk,
                             float* dv, const Geo& g, int nkt, hipStream_t st);

// Kernel timing (benchmark use): when enabled, each launch below is
// bracketed by HIP events recorded on the launch stream.
enum KernelId {
  kKPrep = 0, kKFwd, kKSched, kKDq, kKDkdv, kKReduce, kKSchedRowstat, kKOrder, kNumKernels
};
void timing_begin(int kernel, hipStream_t st);
void timing_end(int kernel, hipStream_t st);

}  // namespace dmgqa
