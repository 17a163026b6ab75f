// C-ABI entry points of libdocmask_gqa: argument validation (before any HIP
// call), workspace layout and kernel launches.  The operation and the
// argument contract are documented in include/docmask_gqa.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <unordered_set>
#include <vector>

#include "../../include/docmask_gqa.h"
#include "kernels.hpp"

namespace dmgqa {
namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Shape {
  int B, S, Skv, Hq, Hkv, D, cp, rank;
  int G, c, Sq;
  bool empty;
};

// Scalar checks shared by both passes.  Returns DMGQA_OK or an error.
int check_shape(int B, int S, int Skv, int Hq, int Hkv, int D, int cp, int rank, Shape* sh) {
  if (B < 0 || S < 0 || Skv < 0 || Hq <= 0 || Hkv <= 0 || cp <= 0) return DMGQA_ERR_INVALID_ARG;
  if (rank < 0 || rank >= cp) return DMGQA_ERR_INVALID_ARG;
  if (S % (2 * cp) != 0) return DMGQA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return DMGQA_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return DMGQA_ERR_UNSUPPORTED;
  const int c = S / (2 * cp);
  const long long need = (long long)(2 * cp - rank) * c;
  if ((long long)Skv < need || Skv > S) return DMGQA_ERR_INVALID_ARG;
  const int G = Hq / Hkv;
  const long long Sq = 2LL * c;
  // row index within a KV group and grid sizes are 32-bit
  if (Sq * G >= (1LL << 30) || (long long)Skv * 2 >= (1LL << 31)) return DMGQA_ERR_UNSUPPORTED;
  const long long tiles = (Sq * G + kFwdBM - 1) / kFwdBM * (long long)B * Hkv;
  if (tiles >= (1LL << 31)) return DMGQA_ERR_UNSUPPORTED;
  // element offsets inside q/out/dout/dq and k/v/dk/dv are 32-bit
  if ((long long)B * Sq * Hq * D >= (1LL << 31) || (long long)B * Skv * Hkv * D >= (1LL << 31) ||
      G >= (1 << 15))
    return DMGQA_ERR_UNSUPPORTED;
  sh->B = B; sh->S = S; sh->Skv = Skv; sh->Hq = Hq; sh->Hkv = Hkv; sh->D = D;
  sh->cp = cp; sh->rank = rank; sh->G = G; sh->c = c; sh->Sq = (int)Sq;
  sh->empty = (B == 0 || S == 0);
  return DMGQA_OK;
}

// Debug mode (environment variable DMGQA_DEBUG set to anything but "0",
// read at every call): each call validates its masking input with the
// synchronous checkers below before any launch -- a copy to the host and a
// synchronisation of the stream, so not for graph capture or timed runs --
// and returns DMGQA_ERR_INVALID_ARG on a violated precondition.
bool debug_mode() {
  const char* e = std::getenv("DMGQA_DEBUG");
  return e != nullptr && e[0] != '\0' && std::strcmp(e, "0") != 0;
}

// Checker result (0 valid, 1 violated, negative status) as a call status.
int debug_status(int r) { return r == 0 ? DMGQA_OK : (r > 0 ? DMGQA_ERR_INVALID_ARG : r); }

int debug_check_docs(const int32_t* doc_ids, const int32_t* cu, int n_docs, int B, int S,
                     hipStream_t st) {
  if (!debug_mode()) return DMGQA_OK;
  if (doc_ids) return debug_status(docmask_gqa_check_docs(doc_ids, B, S, st));
  if (cu) return debug_status(docmask_gqa_check_cu_seqlens(cu, n_docs, S, st));
  return DMGQA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// The kernels track the running maximum of the raw scores and rescale only
// when it grows, which assumes the scale is positive; a finite positive
// scale is required.
bool scale_ok(float x) { return std::isfinite(x) && x > 0.f; }

int check_docs_args(const int32_t* doc_ids, const int32_t* cu, int n_docs, const Shape& s) {
  if ((doc_ids == nullptr) == (cu == nullptr)) return DMGQA_ERR_INVALID_ARG;
  if (doc_ids && !aligned(doc_ids, 4)) return DMGQA_ERR_INVALID_ARG;
  if (cu) {
    if (s.B > 1) return DMGQA_ERR_UNSUPPORTED;
    if (n_docs < 1 || n_docs > s.S || !aligned(cu, 4)) return DMGQA_ERR_INVALID_ARG;
  }
  return DMGQA_OK;
}

// Workspace layout.  Up to total_min: what every backward path needs (the
// bounds, the schedule, the row statistics and the partial-sum slots); the
// dS stash and the partial dQ buffer follow (see plan_stash).
struct Layout {
  size_t dstart, dend, agg, order, rowstat, hdr, tile_info, items, tile_rows, partial, dout16,
      scale_parts, total_min;
  int nkt, max_split_base;
};

// Default budget of the dS stash (all KV heads together) in the workspace
// that docmask_gqa_bwd_workspace_size asks for.
constexpr long long kDefaultStashBudget = 2LL << 30;

// Upper bound, over all document layouts, of the dS stash blocks of one KV
// head for the shape's rank and Skv: a key tile starting at t0 reaches at
// most the local tokens with positions in [t0, S), a contiguous range
// [tlo, thi) of local tokens, i.e. query rows [tlo*G, thi*G) covered by
// blocks of kStashRows rows.
long long stash_blocks_bound(const Shape& s, int nkt) {
  const long long baseA = (long long)s.rank * s.c;
  const long long baseB = (long long)(2 * s.cp - 1 - s.rank) * s.c;
  long long total = 0;
  for (int kt = 0; kt < nkt; ++kt) {
    const long long t0 = (long long)kt * kDkdvBN;
    const long long la = std::min<long long>(std::max<long long>(t0 - baseA, 0), s.c);
    const long long lb = std::min<long long>(std::max<long long>(t0 - baseB, 0), s.c);
    const long long na = s.c - la, nb = s.c - lb;
    const long long tlo = na > 0 ? la : s.c + lb;
    const long long thi = nb > 0 ? 2LL * s.c : la + na;
    if (thi > tlo) total += (thi * s.G + kStashRows - 1) / kStashRows - tlo * s.G / kStashRows;
  }
  return total * s.B;
}

// The same bound for cross attention (keys indexed apart from the queries):
// a key tile's reaching queries are one range of at most the S query tokens.
long long cross_stash_blocks_bound(const Shape& s, int nkt) {
  return (long long)s.B * nkt * (((long long)s.S * s.G + kStashRows - 1) / kStashRows + 1);
}

// The same bound for any rank that may pass this Skv (the size queries take
// no rank): the maximum over those ranks, or, for more than 64 ranks, every
// key tile reaching every local row.
long long stash_blocks_any_rank(Shape s, int nkt) {
  if (s.cp > 64)
    return (long long)s.B * nkt * (((long long)s.Sq * s.G + kStashRows - 1) / kStashRows + 1);
  long long m = 0;
  for (int r = 0; r < s.cp; ++r) {
    if ((long long)(2 * s.cp - r) * s.c > s.Skv) continue;   // needs a longer K/V prefix
    s.rank = r;
    m = std::max(m, stash_blocks_bound(s, nkt));
  }
  return m;
}

Layout layout(const Shape& s, bool backward) {
  Layout L{};
  size_t off = 0;
  const size_t pos = (size_t)s.B * s.Skv * sizeof(int32_t);
  const int nblk = (s.Skv + 1023) / 1024;
  L.dstart = off; off = align_up(off + pos);
  L.dend = off; off = align_up(off + pos);
  L.agg = off; off = align_up(off + 2 * (size_t)s.B * nblk * sizeof(int32_t));
  // dispatch order of the query tiles (forward, or dQ from the stash)
  const size_t nt = ((size_t)s.Sq * s.G + kFwdBM - 1) / kFwdBM;
  L.order = off; off = align_up(off + (size_t)s.B * nt * sizeof(int32_t));
  if (backward) {
    L.nkt = (s.Skv + kDkdvBN - 1) / kDkdvBN;
    L.max_split_base = kMaxSplitTotal / s.Hkv > 1 ? kMaxSplitTotal / s.Hkv : 1;
    const size_t ntiles = (size_t)s.B * L.nkt;
    L.rowstat = off; off = align_up(off + 2 * (size_t)s.B * s.Sq * s.Hq * sizeof(float));
    L.hdr = off; off = align_up(off + sizeof(SchedHeader));
    L.tile_info = off; off = align_up(off + ntiles * sizeof(int2));
    L.items = off; off = align_up(off + (ntiles + L.max_split_base) * sizeof(int2));
    L.tile_rows = off; off = align_up(off + ntiles * sizeof(int4));
    const size_t slots = 2 * (size_t)L.max_split_base * s.Hkv;
    L.partial = off; off = align_up(off + slots * 2 * kDkdvBN * s.D * sizeof(float));
    // dO' = dO * 2^eo in fp16, and the partial maxima of the exponent scan
    L.dout16 = off; off = align_up(off + (size_t)s.B * s.Sq * s.Hq * s.D * 2);
    L.scale_parts = off; off = align_up(off + kScaleParts * sizeof(int2));
  }
  L.total_min = off;
  return L;
}

// How the backward forms dQ, from the workspace it was given:
//  - kStash: the dS stash holds every key tile the rank's layout can reach
//    (the worst-case bound fits); dQ is one product per key tile.
//  - kMixed: a stash of `budget` blocks per KV head (at least one) plus an
//    fp32 partial-dQ buffer; key tiles are stashed in order while they fit,
//    and the query tiles that reach the rest recompute those tiles' share.
//  - kRecompute: no stash; dQ recomputes S, P and dP for every key tile.
enum StashMode { kRecompute = 0, kStash = 1, kMixed = 2 };
struct StashPlan {
  StashMode mode;
  size_t stash, dq_part;   // byte offsets in the workspace
  int budget;              // stash blocks per KV head
};

size_t dq_part_bytes(const Shape& s) {
  return align_up((size_t)s.B * s.Sq * s.Hq * s.D * sizeof(float));
}

// The dK/dV kernel addresses one tile's stash with 32-bit byte offsets (a
// tile holds at most ceil(Sq*G/32) + 1 blocks).
bool stash_addressable(const Shape& s) {
  return ((long long)s.Sq * s.G / kStashRows + 2) * (long long)kStashBlockBytes < (1LL << 31);
}

// bound: stash blocks per KV head that the layout can need at most.
StashPlan plan_stash(const Shape& s, const Layout& L, size_t workspace_bytes, long long bound) {
  StashPlan p{kRecompute, L.total_min, 0, 0};
  if (!stash_addressable(s) || workspace_bytes <= L.total_min) return p;
  const long long per_block = (long long)s.Hkv * kStashBlockBytes;
  const size_t avail = workspace_bytes - L.total_min;
  if (bound < (1LL << 31) && (long long)avail >= bound * per_block) {
    p.mode = kStash;
    p.budget = (int)bound;
    return p;
  }
  const size_t dqb = dq_part_bytes(s);
  if (avail <= dqb) return p;
  const long long blocks = std::min<long long>(
      std::min<long long>((long long)(avail - dqb) / per_block, bound), (1LL << 31) - 1);
  if (blocks < 1) return p;
  p.mode = kMixed;
  p.dq_part = L.total_min;
  p.stash = L.total_min + dqb;
  p.budget = (int)blocks;
  return p;
}

// Workspace of the default backward: the whole worst-case stash (`worst`
// blocks per KV head) if it fits in kDefaultStashBudget, else that budget
// plus the partial-dQ buffer (or the whole stash, if that is smaller).
size_t default_bwd_bytes(const Shape& s, const Layout& L, long long worst) {
  if (!stash_addressable(s)) return L.total_min;
  const long long per_block = (long long)s.Hkv * kStashBlockBytes;
  const size_t full = worst < (1LL << 31) ? L.total_min + align_up((size_t)(worst * per_block))
                                          : SIZE_MAX;
  if (worst * per_block <= kDefaultStashBudget) return full;
  const long long blocks = std::min<long long>(kDefaultStashBudget / per_block, (1LL << 31) - 1);
  return std::min(full, L.total_min + dq_part_bytes(s) + align_up((size_t)(blocks * per_block)));
}

Geo make_geo(const Shape& s, float scale) {
  Geo g;
  g.B = s.B; g.S = s.S; g.Skv = s.Skv; g.Hq = s.Hq; g.Hkv = s.Hkv; g.G = s.G;
  g.Sq = s.Sq; g.c = s.c; g.cp = s.cp; g.rank = s.rank;
  g.g_magic = s.G >= 2 ? (unsigned)((((uint64_t)1 << 32) + (uint64_t)s.G - 1) / (uint64_t)s.G) : 0u;
  g.g_log2 = -1;
  for (int e = 0; e < 31; ++e)
    if ((1 << e) == s.G) g.g_log2 = e;
  g.scale = scale;
  g.scale_log2 = scale * kLog2e;
  return g;
}

// Document bounds dstart, dend [B, Skv] (agg: the scan's block aggregates,
// 2 * B * ceil(Skv / 1024) ints; unused with cu_seqlens).
int prep_bounds(const int32_t* doc_ids, const int32_t* cu, int n_docs, int B, int S, int Skv,
                int32_t* dstart, int32_t* dend, int32_t* agg, hipStream_t st) {
  timing_begin(kKPrep, st);
  hipError_t e = doc_ids ? launch_prep_docs(doc_ids, B, S, Skv, dstart, dend, agg, st)
                         : launch_prep_cu(cu, n_docs, Skv, dstart, dend, st);
  timing_end(kKPrep, st);
  return e == hipSuccess ? DMGQA_OK : DMGQA_ERR_HIP;
}

// Bounds for one call: from the caller's precomputed array, or computed into
// the workspace.
int call_bounds(const int32_t* doc_ids, const int32_t* cu, int n_docs, const int32_t* bounds,
                const Shape& s, char* ws, const Layout& L, hipStream_t st,
                const int32_t** dstart, const int32_t** dend) {
  if (bounds) {
    *dstart = bounds;
    *dend = bounds + (size_t)s.B * s.Skv;
    return DMGQA_OK;
  }
  int32_t* ds = reinterpret_cast<int32_t*>(ws + L.dstart);
  int32_t* de = reinterpret_cast<int32_t*>(ws + L.dend);
  *dstart = ds;
  *dend = de;
  return prep_bounds(doc_ids, cu, n_docs, s.B, s.S, s.Skv, ds, de,
                     reinterpret_cast<int32_t*>(ws + L.agg), st);
}

// Masking arguments: document ids / offsets, or a bounds array (exactly one
// form).
int check_mask_args(const int32_t* doc_ids, const int32_t* cu, int n_docs, const int32_t* bounds,
                    const Shape& s) {
  if (bounds) {
    if (doc_ids || cu || !aligned(bounds, 4)) return DMGQA_ERR_INVALID_ARG;
    return DMGQA_OK;
  }
  return check_docs_args(doc_ids, cu, n_docs, s);
}

int fwd_impl(const void* q, const void* k, const void* v, const int32_t* doc_ids,
             const int32_t* cu_seqlens, int32_t n_docs, const int32_t* bounds, int32_t B,
             int32_t S, int32_t Skv, int32_t Hq, int32_t Hkv, int32_t D, int32_t cp_size,
             int32_t cp_rank, float softmax_scale, void* out, float* lse, void* workspace,
             size_t workspace_bytes, void* stream, const int32_t* order_in = nullptr) {
  Shape s;
  int rc = check_shape(B, S, Skv, Hq, Hkv, D, cp_size, cp_rank, &s);
  if (rc != DMGQA_OK) return rc;
  if (!scale_ok(softmax_scale)) return DMGQA_ERR_INVALID_ARG;
  if (s.empty) return DMGQA_OK;
  if (!q || !k || !v || !out || !lse || !workspace) return DMGQA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(lse, 4) || !aligned(workspace, 16))
    return DMGQA_ERR_INVALID_ARG;
  rc = check_mask_args(doc_ids, cu_seqlens, n_docs, bounds, s);
  if (rc != DMGQA_OK) return rc;
  const Layout L = layout(s, false);
  if (workspace_bytes < L.total_min) return DMGQA_ERR_WORKSPACE;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  rc = debug_check_docs(doc_ids, cu_seqlens, n_docs, s.B, s.S, st);
  if (rc != DMGQA_OK) return rc;
  char* ws = static_cast<char*>(workspace);
  const int32_t* dstart;
  const int32_t* dend;
  rc = call_bounds(doc_ids, cu_seqlens, n_docs, bounds, s, ws, L, st, &dstart, &dend);
  if (rc != DMGQA_OK) return rc;
  const Geo g = make_geo(s, softmax_scale);
  // the query-tile order: the plan's, or built here
  const int32_t* order = order_in;
  hipError_t e = hipSuccess;
  if (!order) {
    int32_t* o = reinterpret_cast<int32_t*>(ws + L.order);
    timing_begin(kKOrder, st);
    e = launch_tile_order_fwd(dstart, nullptr, g, o, st);
    timing_end(kKOrder, st);
    if (e != hipSuccess) return DMGQA_ERR_HIP;
    order = o;
  }
  timing_begin(kKFwd, st);
  e = launch_fwd(D, static_cast<const u16*>(q), static_cast<const u16*>(k),
                 static_cast<const u16*>(v), dstart, nullptr, order, static_cast<u16*>(out), lse, g,
                 st);
  timing_end(kKFwd, st);
  return e == hipSuccess ? DMGQA_OK : DMGQA_ERR_HIP;
}

// Shape of a cross-attention call: S query tokens against Skv keys indexed
// on their own.  There is no context parallelism, so S may be any size: the
// geometry is one "chunk" of c = S rows (the local row map is then the
// identity) and no second chunk.
int check_cross_shape(int B, int S, int Skv, int Hq, int Hkv, int D, Shape* s) {
  if (B < 0 || S < 0 || Skv < 0 || Hq <= 0 || Hkv <= 0) return DMGQA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return DMGQA_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return DMGQA_ERR_UNSUPPORTED;
  const bool empty = B == 0 || S == 0;
  if (Skv == 0 && !empty) return DMGQA_ERR_INVALID_ARG;
  const long long G = Hq / Hkv;
  if ((long long)S * G >= (1LL << 30) || (long long)Skv * 2 >= (1LL << 31) ||
      (long long)S * 2 >= (1LL << 31))
    return DMGQA_ERR_UNSUPPORTED;
  const long long tiles = ((long long)S * G + kFwdBM - 1) / kFwdBM * (long long)B * Hkv;
  if (tiles >= (1LL << 31)) return DMGQA_ERR_UNSUPPORTED;
  if ((long long)B * S * Hq * D >= (1LL << 31) || (long long)B * Skv * Hkv * D >= (1LL << 31) ||
      G >= (1 << 15))
    return DMGQA_ERR_UNSUPPORTED;
  s->B = B; s->S = S; s->Skv = Skv; s->Hq = Hq; s->Hkv = Hkv; s->D = D;
  s->cp = 1; s->rank = 0; s->G = (int)G; s->c = S; s->Sq = S;
  s->empty = empty;
  return DMGQA_OK;
}

size_t cross_workspace_bytes(const Shape& s) {
  const size_t nt = ((size_t)s.Sq * s.G + kFwdBM - 1) / kFwdBM;
  return align_up((size_t)s.B * nt * sizeof(int32_t));
}

// Scratch of the allocation-free forward (docmask_gqa_attn_fwd_noalloc): the
// forward's workspace (document bounds, scan aggregates, tile order) in a
// fixed device array instead of caller memory.  Each GPU the library runs on
// holds its own copy until the process ends.  In host code `scratch` is only
// a stand-in for the symbol: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
constexpr size_t kNoAllocScratchBytes = 8u << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch (the device of `st`, or the
// current one for the null stream), looked up on the device's first call.
int scratch_for(hipStream_t st, char** out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return DMGQA_ERR_HIP;
  int dev = cur;
  if (st != nullptr) {
    hipDevice_t d;
    if (hipStreamGetDevice(st, &d) != hipSuccess) return DMGQA_ERR_HIP;
    dev = (int)d;
  }
  if (dev < 0 || dev >= kMaxDevices) return DMGQA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return DMGQA_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return DMGQA_ERR_HIP;
    if (e != hipSuccess || p == nullptr) return DMGQA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<char*>(g_scratch_ptr[dev]);
  return DMGQA_OK;
}

}  // namespace
}  // namespace dmgqa

using namespace dmgqa;

extern "C" {

size_t docmask_gqa_fwd_workspace_size(int32_t B, int32_t S, int32_t Skv, int32_t Hq, int32_t Hkv,
                                      int32_t D, int32_t cp_size) {
  Shape s;
  // the rank does not change the size; rank 0 needs the longest prefix, so
  // validate against the largest Skv any rank may pass
  if (check_shape(B, S, S, Hq, Hkv, D, cp_size, 0, &s) != DMGQA_OK) return 0;
  s.Skv = Skv > 0 && Skv <= S ? Skv : S;
  if (s.empty) return 0;
  return layout(s, false).total_min;
}

size_t docmask_gqa_bwd_workspace_size(int32_t B, int32_t S, int32_t Skv, int32_t Hq, int32_t Hkv,
                                      int32_t D, int32_t cp_size) {
  Shape s;
  if (check_shape(B, S, S, Hq, Hkv, D, cp_size, 0, &s) != DMGQA_OK) return 0;
  s.Skv = Skv > 0 && Skv <= S ? Skv : S;
  if (s.empty) return 0;
  const Layout L = layout(s, true);
  return default_bwd_bytes(s, L, stash_blocks_any_rank(s, L.nkt));
}

size_t docmask_gqa_bwd_workspace_size_min(int32_t B, int32_t S, int32_t Skv, int32_t Hq,
                                          int32_t Hkv, int32_t D, int32_t cp_size) {
  Shape s;
  if (check_shape(B, S, S, Hq, Hkv, D, cp_size, 0, &s) != DMGQA_OK) return 0;
  s.Skv = Skv > 0 && Skv <= S ? Skv : S;
  if (s.empty) return 0;
  return layout(s, true).total_min;
}

int docmask_gqa_bwd_path(int32_t B, int32_t S, int32_t Skv, int32_t Hq, int32_t Hkv, int32_t D,
                         int32_t cp_size, int32_t cp_rank, size_t workspace_bytes) {
  Shape s;
  const int rc = check_shape(B, S, Skv, Hq, Hkv, D, cp_size, cp_rank, &s);
  if (rc != DMGQA_OK) return rc;
  if (s.empty) return DMGQA_BWD_PATH_RECOMPUTE;
  const Layout L = layout(s, true);
  if (workspace_bytes < L.total_min) return DMGQA_ERR_WORKSPACE;
  switch (plan_stash(s, L, workspace_bytes, stash_blocks_bound(s, L.nkt)).mode) {
    case kStash: return DMGQA_BWD_PATH_STASH;
    case kMixed: return DMGQA_BWD_PATH_MIXED;
    default: return DMGQA_BWD_PATH_RECOMPUTE;
  }
}

size_t docmask_gqa_bwd_workspace_size_full(int32_t B, int32_t S, int32_t Skv, int32_t Hq,
                                           int32_t Hkv, int32_t D, int32_t cp_size) {
  Shape s;
  if (check_shape(B, S, S, Hq, Hkv, D, cp_size, 0, &s) != DMGQA_OK) return 0;
  s.Skv = Skv > 0 && Skv <= S ? Skv : S;
  if (s.empty) return 0;
  const Layout L = layout(s, true);
  const long long worst = stash_blocks_any_rank(s, L.nkt);
  if (!stash_addressable(s) || worst >= (1LL << 31)) return L.total_min;
  return L.total_min + align_up((size_t)worst * s.Hkv * kStashBlockBytes);
}

int docmask_gqa_attn_fwd(const void* q, const void* k, const void* v, const int32_t* doc_ids,
                         const int32_t* cu_seqlens, int32_t n_docs, int32_t B, int32_t S,
                         int32_t Skv, int32_t Hq, int32_t Hkv, int32_t D, int32_t cp_size,
                         int32_t cp_rank, float softmax_scale, void* out, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_impl(q, k, v, doc_ids, cu_seqlens, n_docs, nullptr, B, S, Skv, Hq, Hkv, D, cp_size,
                  cp_rank, softmax_scale, out, lse, workspace, workspace_bytes, stream);
}

int docmask_gqa_attn_fwd_noalloc(const void* q, const void* k, const void* v,
                                 const int32_t* doc_ids, const int32_t* cu_seqlens,
                                 int32_t n_docs, int32_t B, int32_t S, int32_t Skv, int32_t Hq,
                                 int32_t Hkv, int32_t D, int32_t cp_size, int32_t cp_rank,
                                 float softmax_scale, void* out, float* lse, void* stream) {
  // The scalar checks of the forward, and the size limit of the scratch,
  // come before any HIP call.
  Shape s;
  int rc = check_shape(B, S, Skv, Hq, Hkv, D, cp_size, cp_rank, &s);
  if (rc != DMGQA_OK) return rc;
  if (!scale_ok(softmax_scale)) return DMGQA_ERR_INVALID_ARG;
  if (s.empty) return DMGQA_OK;
  const size_t need = layout(s, false).total_min;
  if (need > kNoAllocScratchBytes) return DMGQA_ERR_WORKSPACE;
  char* ws = nullptr;
  rc = scratch_for(reinterpret_cast<hipStream_t>(stream), &ws);
  if (rc != DMGQA_OK) return rc;
  return fwd_impl(q, k, v, doc_ids, cu_seqlens, n_docs, nullptr, B, S, Skv, Hq, Hkv, D, cp_size,
                  cp_rank, softmax_scale, out, lse, ws, kNoAllocScratchBytes, stream);
}

int docmask_gqa_attn_fwd_bounds(const void* q, const void* k, const void* v,
                                const int32_t* bounds, int32_t B, int32_t S, int32_t Skv,
                                int32_t Hq, int32_t Hkv, int32_t D, int32_t cp_size,
                                int32_t cp_rank, float softmax_scale, void* out, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (!bounds) return DMGQA_ERR_INVALID_ARG;
  return fwd_impl(q, k, v, nullptr, nullptr, 0, bounds, B, S, Skv, Hq, Hkv, D, cp_size, cp_rank,
                  softmax_scale, out, lse, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace dmgqa {
namespace {

int bwd_impl(const void* q, const void* k, const void* v, const void* out, const void* dout,
             const float* lse, const int32_t* doc_ids, const int32_t* cu_seqlens, int32_t n_docs,
             const int32_t* bounds, int32_t B, int32_t S, int32_t Skv, int32_t Hq, int32_t Hkv,
             int32_t D, int32_t cp_size, int32_t cp_rank, float softmax_scale, void* dq,
             float* dk, float* dv, void* workspace, size_t workspace_bytes, void* stream,
             const int32_t* dq_order_in = nullptr) {
  Shape s;
  int rc = check_shape(B, S, Skv, Hq, Hkv, D, cp_size, cp_rank, &s);
  if (rc != DMGQA_OK) return rc;
  if (!scale_ok(softmax_scale)) return DMGQA_ERR_INVALID_ARG;
  if (s.empty) return DMGQA_OK;
  if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv || !workspace)
    return DMGQA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(lse, 4) || !aligned(dk, 16) ||
      !aligned(dv, 16) || !aligned(workspace, 16))
    return DMGQA_ERR_INVALID_ARG;
  rc = check_mask_args(doc_ids, cu_seqlens, n_docs, bounds, s);
  if (rc != DMGQA_OK) return rc;
  const Layout L = layout(s, true);
  if (workspace_bytes < L.total_min) return DMGQA_ERR_WORKSPACE;
  const StashPlan plan = plan_stash(s, L, workspace_bytes, stash_blocks_bound(s, L.nkt));

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  rc = debug_check_docs(doc_ids, cu_seqlens, n_docs, s.B, s.S, st);
  if (rc != DMGQA_OK) return rc;
  char* ws = static_cast<char*>(workspace);
  const int32_t* dstart;
  const int32_t* dend;
  rc = call_bounds(doc_ids, cu_seqlens, n_docs, bounds, s, ws, L, st, &dstart, &dend);
  if (rc != DMGQA_OK) return rc;
  const Geo g = make_geo(s, softmax_scale);
  // per query row: -lse/scale, then -D
  float* Lbuf = reinterpret_cast<float*>(ws + L.rowstat);
  float* Nbuf = Lbuf + (size_t)s.B * s.Sq * s.Hq;
  SchedHeader* hdr = reinterpret_cast<SchedHeader*>(ws + L.hdr);
  int2* tile_info = reinterpret_cast<int2*>(ws + L.tile_info);
  int2* items = reinterpret_cast<int2*>(ws + L.items);
  int4* tile_rows = reinterpret_cast<int4*>(ws + L.tile_rows);
  float* partial = reinterpret_cast<float*>(ws + L.partial);
  // the dQ kernel's query-tile order: the plan's, or built beside the row
  // statistics
  int32_t* dq_order_ws = dq_order_in ? nullptr : reinterpret_cast<int32_t*>(ws + L.order);
  const int32_t* dq_order = dq_order_in ? dq_order_in : dq_order_ws;
  const u16* qh = static_cast<const u16*>(q);
  const u16* kh = static_cast<const u16*>(k);
  const u16* vh = static_cast<const u16*>(v);
  const u16* oh = static_cast<const u16*>(out);
  const u16* doh = static_cast<const u16*>(dout);
  u16* dqh = static_cast<u16*>(dq);

  u16* dout16 = reinterpret_cast<u16*>(ws + L.dout16);
  int2* scale_parts = reinterpret_cast<int2*>(ws + L.scale_parts);

  // Every path: the exponent scan of dO and V, then the schedule with the
  // row statistics (and dO' in fp16) for the dK/dV kernel.
  timing_begin(kKScale, st);
  hipError_t e = launch_scale_scan(doh, (long long)s.B * s.Sq * s.Hq * D, vh,
                                   (long long)s.B * s.Skv * s.Hkv * D, scale_parts, st);
  timing_end(kKScale, st);
  if (e != hipSuccess) return DMGQA_ERR_HIP;
  timing_begin(kKSchedRowstat, st);
  e = launch_sched_rowstat(D, nullptr, dstart, nullptr, dend, g, L.nkt, L.max_split_base,
                           plan.mode == kRecompute ? 0 : plan.budget, hdr, tile_info, items,
                           tile_rows, plan.mode == kRecompute ? nullptr : dq_order_ws, oh, doh, lse,
                           scale_parts, Lbuf, Nbuf, dout16, st);
  timing_end(kKSchedRowstat, st);
  if (e != hipSuccess) return DMGQA_ERR_HIP;
  if (plan.mode != kRecompute) {
    // The dK/dV kernel stores dS of the stashed key tiles; dQ is then one
    // product per stashed key tile, and (mixed) the query tiles that also
    // reach key tiles beyond the budget recompute those tiles' share.
    u16* stash = reinterpret_cast<u16*>(ws + plan.stash);
    float* dq_part =
        plan.mode == kMixed ? reinterpret_cast<float*>(ws + plan.dq_part) : nullptr;
    timing_begin(kKDkdv, st);
    e = launch_bwd_dkdv(D, qh, kh, vh, dout16, Lbuf, Nbuf, nullptr, dend, hdr, tile_info, items,
                        tile_rows, stash, plan.budget, partial, dk, dv, g, L.nkt, st);
    timing_end(kKDkdv, st);
    if (e != hipSuccess) return DMGQA_ERR_HIP;
    timing_begin(kKDq, st);
    e = launch_bwd_dq_stash(D, kh, dstart, nullptr, tile_rows, stash, plan.budget, dq_order, dqh,
                            dq_part,
                            tile_info, partial, dk, dv, hdr, g, L.nkt, st);
    timing_end(kKDq, st);
    if (e != hipSuccess || plan.mode == kStash) return e == hipSuccess ? DMGQA_OK : DMGQA_ERR_HIP;
    timing_begin(kKDqRest, st);
    e = launch_bwd_dq(D, qh, kh, vh, oh, doh, lse, dstart, nullptr, dqh, tile_rows, dq_part, g,
                      L.nkt, st);
    timing_end(kKDqRest, st);
    return e == hipSuccess ? DMGQA_OK : DMGQA_ERR_HIP;
  }
  timing_begin(kKDq, st);
  e = launch_bwd_dq(D, qh, kh, vh, oh, doh, lse, dstart, nullptr, dqh, tile_rows, nullptr, g,
                    L.nkt, st);
  timing_end(kKDq, st);
  if (e != hipSuccess) return DMGQA_ERR_HIP;
  timing_begin(kKDkdv, st);
  e = launch_bwd_dkdv(D, qh, kh, vh, dout16, Lbuf, Nbuf, nullptr, dend, hdr, tile_info, items,
                      tile_rows, nullptr, 0, partial, dk, dv, g, L.nkt, st);
  timing_end(kKDkdv, st);
  if (e != hipSuccess) return DMGQA_ERR_HIP;
  timing_begin(kKReduce, st);
  e = launch_bwd_reduce(D, tile_info, partial, dk, dv, hdr, g, L.nkt, st);
  timing_end(kKReduce, st);
  return e == hipSuccess ? DMGQA_OK : DMGQA_ERR_HIP;
}

// Cross-attention backward: key ranges from lo / hi, the exponent scan, the
// schedule with the row statistics, then as the causal backward: with room
// for a dS stash beyond the minimum workspace, dK/dV storing dS and dQ from
// the stash (with the split tiles' partial slots added in its tail; mixed:
// the key tiles past the budget recomputed by the dQ kernel); without it, dQ
// recomputing the scores, dK/dV and the sum of the partial slots.
int bwd_cross_impl(const void* q, const void* k, const void* v, const void* out,
                   const void* dout, const float* lse, const int32_t* lo, const int32_t* hi,
                   int32_t B, int32_t S, int32_t Skv, int32_t Hq, int32_t Hkv, int32_t D,
                   float softmax_scale, void* dq, float* dk, float* dv, void* workspace,
                   size_t workspace_bytes, void* stream) {
  Shape s;
  int rc = check_cross_shape(B, S, Skv, Hq, Hkv, D, &s);
  if (rc != DMGQA_OK) return rc;
  if (!scale_ok(softmax_scale)) return DMGQA_ERR_INVALID_ARG;
  if (s.empty) return DMGQA_OK;
  if (!q || !k || !v || !out || !dout || !lse || !lo || !hi || !dq || !dk || !dv || !workspace)
    return DMGQA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(lse, 4) || !aligned(lo, 4) ||
      !aligned(hi, 4) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(workspace, 16))
    return DMGQA_ERR_INVALID_ARG;
  const Layout L = layout(s, true);
  if (workspace_bytes < L.total_min) return DMGQA_ERR_WORKSPACE;
  const StashPlan plan =
      plan_stash(s, L, workspace_bytes, cross_stash_blocks_bound(s, L.nkt));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (debug_mode()) {
    const int drc = debug_status(docmask_gqa_check_cross_intervals(lo, hi, B, S, Skv, st));
    if (drc != DMGQA_OK) return drc;
  }
  char* ws = static_cast<char*>(workspace);
  // per key: the first query position that reaches it and one past the last
  int32_t* kfirst = reinterpret_cast<int32_t*>(ws + L.dstart);
  int32_t* kend = reinterpret_cast<int32_t*>(ws + L.dend);
  float* Lbuf = reinterpret_cast<float*>(ws + L.rowstat);
  float* Nbuf = Lbuf + (size_t)s.B * s.Sq * s.Hq;
  SchedHeader* hdr = reinterpret_cast<SchedHeader*>(ws + L.hdr);
  int2* tile_info = reinterpret_cast<int2*>(ws + L.tile_info);
  int2* items = reinterpret_cast<int2*>(ws + L.items);
  int4* tile_rows = reinterpret_cast<int4*>(ws + L.tile_rows);
  float* partial = reinterpret_cast<float*>(ws + L.partial);
  const u16* qh = static_cast<const u16*>(q);
  const u16* kh = static_cast<const u16*>(k);
  const u16* vh = static_cast<const u16*>(v);
  const Geo g = make_geo(s, softmax_scale);

  const u16* oh = static_cast<const u16*>(out);
  const u16* doh = static_cast<const u16*>(dout);
  u16* dout16 = reinterpret_cast<u16*>(ws + L.dout16);
  int2* scale_parts = reinterpret_cast<int2*>(ws + L.scale_parts);

  timing_begin(kKPrep, st);
  hipError_t e = launch_prep_cross_keys(lo, hi, s.B, s.S, s.Skv, kfirst, kend, st);
  timing_end(kKPrep, st);
  if (e != hipSuccess) return DMGQA_ERR_HIP;
  timing_begin(kKScale, st);
  e = launch_scale_scan(doh, (long long)s.B * s.Sq * s.Hq * D, vh,
                        (long long)s.B * s.Skv * s.Hkv * D, scale_parts, st);
  timing_end(kKScale, st);
  if (e != hipSuccess) return DMGQA_ERR_HIP;
  // the dQ stash kernel's query-tile order, built beside the row statistics
  int32_t* dq_order = reinterpret_cast<int32_t*>(ws + L.order);
  timing_begin(kKSchedRowstat, st);
  e = launch_sched_rowstat(D, kfirst, lo, hi, kend, g, L.nkt, L.max_split_base,
                           plan.mode == kRecompute ? 0 : plan.budget, hdr, tile_info, items,
                           tile_rows, plan.mode == kRecompute ? nullptr : dq_order, oh, doh, lse,
                           scale_parts, Lbuf, Nbuf, dout16, st);
  timing_end(kKSchedRowstat, st);
  if (e != hipSuccess) return DMGQA_ERR_HIP;
  u16* dqh = static_cast<u16*>(dq);
  if (plan.mode != kRecompute) {
    u16* stash = reinterpret_cast<u16*>(ws + plan.stash);
    float* dq_part =
        plan.mode == kMixed ? reinterpret_cast<float*>(ws + plan.dq_part) : nullptr;
    timing_begin(kKDkdv, st);
    e = launch_bwd_dkdv(D, qh, kh, vh, dout16, Lbuf, Nbuf, kfirst, kend, hdr, tile_info, items,
                        tile_rows, stash, plan.budget, partial, dk, dv, g, L.nkt, st);
    timing_end(kKDkdv, st);
    if (e != hipSuccess) return DMGQA_ERR_HIP;
    timing_begin(kKDq, st);
    e = launch_bwd_dq_stash(D, kh, lo, hi, tile_rows, stash, plan.budget, dq_order, dqh, dq_part,
                            tile_info, partial, dk, dv, hdr, g, L.nkt, st);
    timing_end(kKDq, st);
    if (e != hipSuccess || plan.mode == kStash) return e == hipSuccess ? DMGQA_OK : DMGQA_ERR_HIP;
    timing_begin(kKDqRest, st);
    e = launch_bwd_dq(D, qh, kh, vh, oh, doh, lse, lo, hi, dqh, tile_rows, dq_part, g, L.nkt, st);
    timing_end(kKDqRest, st);
    return e == hipSuccess ? DMGQA_OK : DMGQA_ERR_HIP;
  }
  timing_begin(kKDq, st);
  e = launch_bwd_dq(D, qh, kh, vh, oh, doh, lse, lo, hi, dqh, tile_rows, nullptr, g, L.nkt, st);
  timing_end(kKDq, st);
  if (e != hipSuccess) return DMGQA_ERR_HIP;
  timing_begin(kKDkdv, st);
  e = launch_bwd_dkdv(D, qh, kh, vh, dout16, Lbuf, Nbuf, kfirst, kend, hdr, tile_info, items,
                      tile_rows, nullptr, 0, partial, dk, dv, g, L.nkt, st);
  timing_end(kKDkdv, st);
  if (e != hipSuccess) return DMGQA_ERR_HIP;
  timing_begin(kKReduce, st);
  e = launch_bwd_reduce(D, tile_info, partial, dk, dv, hdr, g, L.nkt, st);
  timing_end(kKReduce, st);
  return e == hipSuccess ? DMGQA_OK : DMGQA_ERR_HIP;
}

}  // namespace
}  // namespace dmgqa

extern "C" {

int docmask_gqa_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                         const void* dout, const float* lse, const int32_t* doc_ids,
                         const int32_t* cu_seqlens, int32_t n_docs, int32_t B, int32_t S,
                         int32_t Skv, int32_t Hq, int32_t Hkv, int32_t D, int32_t cp_size,
                         int32_t cp_rank, float softmax_scale, void* dq, float* dk, float* dv,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(q, k, v, out, dout, lse, doc_ids, cu_seqlens, n_docs, nullptr, B, S, Skv, Hq,
                  Hkv, D, cp_size, cp_rank, softmax_scale, dq, dk, dv, workspace,
                  workspace_bytes, stream);
}

int docmask_gqa_attn_bwd_bounds(const void* q, const void* k, const void* v, const void* out,
                                const void* dout, const float* lse, const int32_t* bounds,
                                int32_t B, int32_t S, int32_t Skv, int32_t Hq, int32_t Hkv,
                                int32_t D, int32_t cp_size, int32_t cp_rank,
                                float softmax_scale, void* dq, float* dk, float* dv,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (!bounds) return DMGQA_ERR_INVALID_ARG;
  return bwd_impl(q, k, v, out, dout, lse, nullptr, nullptr, 0, bounds, B, S, Skv, Hq, Hkv, D,
                  cp_size, cp_rank, softmax_scale, dq, dk, dv, workspace, workspace_bytes,
                  stream);
}

size_t docmask_gqa_doc_bounds_size(int32_t B, int32_t S, int32_t Skv) {
  if (B <= 0 || S <= 0 || Skv <= 0 || Skv > S) return 0;
  const size_t nblk = ((size_t)Skv + 1023) / 1024;
  return (2 * (size_t)B * Skv + 2 * (size_t)B * nblk) * sizeof(int32_t);
}

int docmask_gqa_doc_bounds(const int32_t* doc_ids, const int32_t* cu_seqlens, int32_t n_docs,
                           int32_t B, int32_t S, int32_t Skv, int32_t* bounds,
                           size_t bounds_bytes, void* stream) {
  if (B < 0 || S < 0 || Skv < 0 || Skv > S) return DMGQA_ERR_INVALID_ARG;
  if (B == 0 || Skv == 0) return DMGQA_OK;
  if ((long long)B * S >= (1LL << 31)) return DMGQA_ERR_UNSUPPORTED;
  if ((doc_ids == nullptr) == (cu_seqlens == nullptr)) return DMGQA_ERR_INVALID_ARG;
  if (doc_ids && !aligned(doc_ids, 4)) return DMGQA_ERR_INVALID_ARG;
  if (cu_seqlens) {
    if (B > 1) return DMGQA_ERR_UNSUPPORTED;
    if (n_docs < 1 || n_docs > S || !aligned(cu_seqlens, 4)) return DMGQA_ERR_INVALID_ARG;
  }
  if (!bounds || !aligned(bounds, 4)) return DMGQA_ERR_INVALID_ARG;
  if (bounds_bytes < docmask_gqa_doc_bounds_size(B, S, Skv)) return DMGQA_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int drc = debug_check_docs(doc_ids, cu_seqlens, n_docs, B, S, st);
  if (drc != DMGQA_OK) return drc;
  int32_t* dstart = bounds;
  int32_t* dend = bounds + (size_t)B * Skv;
  return prep_bounds(doc_ids, cu_seqlens, n_docs, B, S, Skv, dstart, dend,
                     bounds + 2 * (size_t)B * Skv, st);
}

}  // extern "C"

namespace dmgqa {

// Batch plan layout (int32 offsets): the bounds as in a bounds array
// (dstart [B, Skv] then dend [B, Skv]), the forward's and the dQ kernel's
// query-tile orders (B * nt each, nt query tiles of kFwdBM rows per batch
// row), then the bounds scan's block aggregates (scratch of the multi-launch
// path).
struct BatchPlanLayout {
  size_t fwd_order, dq_order, agg, total_ints;
};

BatchPlanLayout batch_plan_layout(const Shape& s) {
  BatchPlanLayout P;
  const size_t nt = ((size_t)s.Sq * s.G + kFwdBM - 1) / kFwdBM;
  P.fwd_order = 2 * (size_t)s.B * s.Skv;
  P.dq_order = P.fwd_order + (size_t)s.B * nt;
  P.agg = P.dq_order + (size_t)s.B * nt;
  P.total_ints = P.agg + 2 * (size_t)s.B * (((size_t)s.Skv + 1023) / 1024);
  return P;
}

}  // namespace dmgqa

extern "C" {

size_t docmask_gqa_batch_plan_size(int32_t B, int32_t S, int32_t Skv, int32_t Hq, int32_t Hkv,
                                   int32_t D, int32_t cp_size) {
  Shape s;
  if (check_shape(B, S, S, Hq, Hkv, D, cp_size, 0, &s) != DMGQA_OK) return 0;
  if (Skv <= 0 || Skv > S || s.empty) return 0;
  s.Skv = Skv;
  return batch_plan_layout(s).total_ints * sizeof(int32_t);
}

int docmask_gqa_batch_plan(const int32_t* doc_ids, const int32_t* cu_seqlens, int32_t n_docs,
                           int32_t B, int32_t S, int32_t Skv, int32_t Hq, int32_t Hkv, int32_t D,
                           int32_t cp_size, int32_t cp_rank, int32_t* plan, size_t plan_bytes,
                           void* stream) {
  Shape s;
  int rc = check_shape(B, S, Skv, Hq, Hkv, D, cp_size, cp_rank, &s);
  if (rc != DMGQA_OK) return rc;
  if (s.empty) return DMGQA_OK;
  rc = check_docs_args(doc_ids, cu_seqlens, n_docs, s);
  if (rc != DMGQA_OK) return rc;
  if (!plan || !aligned(plan, 4)) return DMGQA_ERR_INVALID_ARG;
  const BatchPlanLayout P = batch_plan_layout(s);
  if (plan_bytes < P.total_ints * sizeof(int32_t)) return DMGQA_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  rc = debug_check_docs(doc_ids, cu_seqlens, n_docs, s.B, s.S, st);
  if (rc != DMGQA_OK) return rc;
  const Geo g = make_geo(s, 1.f);   // the orders do not depend on the scale
  int32_t* dstart = plan;
  int32_t* dend = plan + (size_t)s.B * s.Skv;
  rc = prep_bounds(doc_ids, cu_seqlens, n_docs, s.B, s.S, s.Skv, dstart, dend, plan + P.agg, st);
  if (rc != DMGQA_OK) return rc;
  timing_begin(kKOrder, st);
  const hipError_t e = launch_plan_orders(dstart, g, plan + P.fwd_order, plan + P.dq_order, st);
  timing_end(kKOrder, st);
  return e == hipSuccess ? DMGQA_OK : DMGQA_ERR_HIP;
}

int docmask_gqa_attn_fwd_plan(const void* q, const void* k, const void* v, const int32_t* plan,
                              int32_t B, int32_t S, int32_t Skv, int32_t Hq, int32_t Hkv,
                              int32_t D, int32_t cp_size, int32_t cp_rank, float softmax_scale,
                              void* out, float* lse, void* workspace, size_t workspace_bytes,
                              void* stream) {
  Shape s;
  const int rc = check_shape(B, S, Skv, Hq, Hkv, D, cp_size, cp_rank, &s);
  if (rc != DMGQA_OK) return rc;
  if (s.empty) return fwd_impl(q, k, v, nullptr, nullptr, 0, plan, B, S, Skv, Hq, Hkv, D,
                               cp_size, cp_rank, softmax_scale, out, lse, workspace,
                               workspace_bytes, stream);
  if (!plan) return DMGQA_ERR_INVALID_ARG;
  return fwd_impl(q, k, v, nullptr, nullptr, 0, plan, B, S, Skv, Hq, Hkv, D, cp_size, cp_rank,
                  softmax_scale, out, lse, workspace, workspace_bytes, stream,
                  plan + batch_plan_layout(s).fwd_order);
}

int docmask_gqa_attn_bwd_plan(const void* q, const void* k, const void* v, const void* out,
                              const void* dout, const float* lse, const int32_t* plan,
                              int32_t B, int32_t S, int32_t Skv, int32_t Hq, int32_t Hkv,
                              int32_t D, int32_t cp_size, int32_t cp_rank, float softmax_scale,
                              void* dq, float* dk, float* dv, void* workspace,
                              size_t workspace_bytes, void* stream) {
  Shape s;
  const int rc = check_shape(B, S, Skv, Hq, Hkv, D, cp_size, cp_rank, &s);
  if (rc != DMGQA_OK) return rc;
  if (s.empty) return bwd_impl(q, k, v, out, dout, lse, nullptr, nullptr, 0, plan, B, S, Skv, Hq,
                               Hkv, D, cp_size, cp_rank, softmax_scale, dq, dk, dv, workspace,
                               workspace_bytes, stream);
  if (!plan) return DMGQA_ERR_INVALID_ARG;
  return bwd_impl(q, k, v, out, dout, lse, nullptr, nullptr, 0, plan, B, S, Skv, Hq, Hkv, D,
                  cp_size, cp_rank, softmax_scale, dq, dk, dv, workspace, workspace_bytes, stream,
                  plan + batch_plan_layout(s).dq_order);
}

int docmask_gqa_interval_bounds(const int32_t* lo, int32_t B, int32_t S, int32_t Skv,
                                int32_t* bounds, size_t bounds_bytes, void* stream) {
  if (B < 0 || S < 0 || Skv < 0 || Skv > S) return DMGQA_ERR_INVALID_ARG;
  if (B == 0 || Skv == 0) return DMGQA_OK;
  if ((long long)B * S >= (1LL << 31)) return DMGQA_ERR_UNSUPPORTED;
  if (!lo || !aligned(lo, 4)) return DMGQA_ERR_INVALID_ARG;
  if (!bounds || !aligned(bounds, 4)) return DMGQA_ERR_INVALID_ARG;
  if (bounds_bytes < docmask_gqa_doc_bounds_size(B, S, Skv)) return DMGQA_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (debug_mode()) {
    const int drc = debug_status(docmask_gqa_check_intervals(lo, B, S, st));
    if (drc != DMGQA_OK) return drc;
  }
  timing_begin(kKPrep, st);
  const hipError_t e = launch_prep_interval(lo, B, S, Skv, bounds, bounds + (size_t)B * Skv, st);
  timing_end(kKPrep, st);
  return e == hipSuccess ? DMGQA_OK : DMGQA_ERR_HIP;
}

size_t docmask_gqa_fwd_cross_workspace_size(int32_t B, int32_t S, int32_t Skv, int32_t Hq,
                                            int32_t Hkv, int32_t D) {
  Shape s;
  if (check_cross_shape(B, S, Skv, Hq, Hkv, D, &s) != DMGQA_OK || s.empty) return 0;
  return cross_workspace_bytes(s);
}

int docmask_gqa_attn_fwd_cross(const void* q, const void* k, const void* v, const int32_t* lo,
                               const int32_t* hi, int32_t B, int32_t S, int32_t Skv, int32_t Hq,
                               int32_t Hkv, int32_t D, float softmax_scale, void* out, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream) {
  Shape s;
  int rc = check_cross_shape(B, S, Skv, Hq, Hkv, D, &s);
  if (rc != DMGQA_OK) return rc;
  if (!scale_ok(softmax_scale)) return DMGQA_ERR_INVALID_ARG;
  if (s.empty) return DMGQA_OK;
  if (!q || !k || !v || !lo || !hi || !out || !lse || !workspace) return DMGQA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(lse, 4) || !aligned(lo, 4) || !aligned(hi, 4) || !aligned(workspace, 16))
    return DMGQA_ERR_INVALID_ARG;
  if (workspace_bytes < cross_workspace_bytes(s)) return DMGQA_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (debug_mode()) {
    const int drc = debug_status(docmask_gqa_check_cross_intervals(lo, hi, B, S, Skv, st));
    if (drc != DMGQA_OK) return drc;
  }
  const Geo g = make_geo(s, softmax_scale);
  int32_t* order = static_cast<int32_t*>(workspace);
  timing_begin(kKOrder, st);
  hipError_t e = launch_tile_order_fwd(lo, hi, g, order, st);
  timing_end(kKOrder, st);
  if (e != hipSuccess) return DMGQA_ERR_HIP;
  timing_begin(kKFwd, st);
  e = launch_fwd(D, static_cast<const u16*>(q), static_cast<const u16*>(k),
                 static_cast<const u16*>(v), lo, hi, order, static_cast<u16*>(out), lse, g, st);
  timing_end(kKFwd, st);
  return e == hipSuccess ? DMGQA_OK : DMGQA_ERR_HIP;
}

size_t docmask_gqa_bwd_cross_workspace_size(int32_t B, int32_t S, int32_t Skv, int32_t Hq,
                                            int32_t Hkv, int32_t D) {
  Shape s;
  if (check_cross_shape(B, S, Skv, Hq, Hkv, D, &s) != DMGQA_OK || s.empty) return 0;
  const Layout L = layout(s, true);
  return default_bwd_bytes(s, L, cross_stash_blocks_bound(s, L.nkt));
}

size_t docmask_gqa_bwd_cross_workspace_size_min(int32_t B, int32_t S, int32_t Skv, int32_t Hq,
                                                int32_t Hkv, int32_t D) {
  Shape s;
  if (check_cross_shape(B, S, Skv, Hq, Hkv, D, &s) != DMGQA_OK || s.empty) return 0;
  return layout(s, true).total_min;
}

int docmask_gqa_bwd_cross_path(int32_t B, int32_t S, int32_t Skv, int32_t Hq, int32_t Hkv,
                               int32_t D, size_t workspace_bytes) {
  Shape s;
  const int rc = check_cross_shape(B, S, Skv, Hq, Hkv, D, &s);
  if (rc != DMGQA_OK) return rc;
  if (s.empty) return DMGQA_BWD_PATH_RECOMPUTE;
  const Layout L = layout(s, true);
  if (workspace_bytes < L.total_min) return DMGQA_ERR_WORKSPACE;
  switch (plan_stash(s, L, workspace_bytes, cross_stash_blocks_bound(s, L.nkt)).mode) {
    case kStash: return DMGQA_BWD_PATH_STASH;
    case kMixed: return DMGQA_BWD_PATH_MIXED;
    default: return DMGQA_BWD_PATH_RECOMPUTE;
  }
}

int docmask_gqa_attn_bwd_cross(const void* q, const void* k, const void* v, const void* out,
                               const void* dout, const float* lse, const int32_t* lo,
                               const int32_t* hi, int32_t B, int32_t S, int32_t Skv, int32_t Hq,
                               int32_t Hkv, int32_t D, float softmax_scale, void* dq, float* dk,
                               float* dv, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return bwd_cross_impl(q, k, v, out, dout, lse, lo, hi, B, S, Skv, Hq, Hkv, D, softmax_scale, dq,
                        dk, dv, workspace, workspace_bytes, stream);
}

int docmask_gqa_check_cross_intervals(const int32_t* lo, const int32_t* hi, int32_t B, int32_t S,
                                      int32_t Skv, void* stream) {
  if (B < 0 || S < 0 || Skv < 0) return DMGQA_ERR_INVALID_ARG;
  if (B == 0 || S == 0) return 0;
  if (!lo || !hi) return DMGQA_ERR_INVALID_ARG;
  std::vector<int32_t> hl((size_t)B * S), hh((size_t)B * S);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(hl.data(), lo, hl.size() * sizeof(int32_t), hipMemcpyDeviceToHost, st) !=
          hipSuccess ||
      hipMemcpyAsync(hh.data(), hi, hh.size() * sizeof(int32_t), hipMemcpyDeviceToHost, st) !=
          hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return DMGQA_ERR_HIP;
  for (int b = 0; b < B; ++b) {
    const int32_t* l = hl.data() + (size_t)b * S;
    const int32_t* h = hh.data() + (size_t)b * S;
    for (int p = 0; p < S; ++p) {
      if (l[p] < 0 || l[p] >= h[p] || h[p] > Skv) return 1;
      if (p > 0 && (l[p] < l[p - 1] || h[p] < h[p - 1])) return 1;
    }
  }
  return 0;
}

int docmask_gqa_check_intervals(const int32_t* lo, int32_t B, int32_t S, void* stream) {
  if (B < 0 || S < 0) return DMGQA_ERR_INVALID_ARG;
  if (B == 0 || S == 0) return 0;
  if (!lo) return DMGQA_ERR_INVALID_ARG;
  std::vector<int32_t> h((size_t)B * S);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(h.data(), lo, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, st) !=
          hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return DMGQA_ERR_HIP;
  for (int b = 0; b < B; ++b) {
    const int32_t* l = h.data() + (size_t)b * S;
    for (int p = 0; p < S; ++p)
      if (l[p] < 0 || l[p] > p || (p > 0 && l[p] < l[p - 1])) return 1;
  }
  return 0;
}

int docmask_gqa_check_docs(const int32_t* doc_ids, int32_t B, int32_t S, void* stream) {
  if (B < 0 || S < 0) return DMGQA_ERR_INVALID_ARG;
  if (B == 0 || S == 0) return 0;
  if (!doc_ids) return DMGQA_ERR_INVALID_ARG;
  std::vector<int32_t> h((size_t)B * S);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(h.data(), doc_ids, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, st) !=
          hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return DMGQA_ERR_HIP;
  for (int b = 0; b < B; ++b) {
    std::unordered_set<int32_t> seen;
    const int32_t* d = h.data() + (size_t)b * S;
    for (int t = 0; t < S; ++t) {
      if (t > 0 && d[t] == d[t - 1]) continue;
      if (!seen.insert(d[t]).second) return 1;
    }
  }
  return 0;
}

int docmask_gqa_check_cu_seqlens(const int32_t* cu_seqlens, int32_t n_docs, int32_t S,
                                 void* stream) {
  if (n_docs < 1 || S < 0 || !cu_seqlens) return DMGQA_ERR_INVALID_ARG;
  std::vector<int32_t> h((size_t)n_docs + 1);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(h.data(), cu_seqlens, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost,
                     st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return DMGQA_ERR_HIP;
  if (h[0] != 0 || h[n_docs] != S) return 1;
  for (int i = 0; i < n_docs; ++i)
    if (h[i + 1] <= h[i]) return 1;
  return 0;
}

const char* docmask_gqa_status_string(int status) {
  switch (status) {
    case DMGQA_OK: return "ok";
    case DMGQA_ERR_INVALID_ARG: return "invalid argument";
    case DMGQA_ERR_UNSUPPORTED: return "unsupported configuration";
    case DMGQA_ERR_WORKSPACE: return "workspace too small";
    case DMGQA_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

int docmask_gqa_version(void) { return 100; }

}  // extern "C"
