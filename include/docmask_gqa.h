/*
 * docmask_gqa.h -- document-masked causal grouped-query attention for one
 * context-parallel (CP) rank, forward and backward, on AMD Instinct MI355X
 * (gfx950).  C ABI: plain pointers and sizes only.
 *
 * The operation (from the pages this library follows):
 *
 *  - Context parallelism ("The Llama 3 Herd of Models", section 3.3.2,
 *    "Context parallelism for long sequences"): the sequence of S tokens is
 *    cut into 2*cp_size equal chunks of c = S/(2*cp_size) tokens; rank i holds
 *    chunk i and chunk 2*cp_size-1-i.  K and V of the whole sequence are
 *    all-gathered first and attention is computed for the rank's local
 *    queries.  Here the gathered K/V are already in device memory.
 *  - Document mask ("Paper notes: The Llama 3 Herd of Models", "Two
 *    architectural choices"): a token never attends across a document
 *    boundary.  With the causal mask of a decoder, key position t is allowed
 *    for query position p iff t <= p and doc(t) == doc(p).
 *  - GQA (same sections): query head h uses KV head h / (Hq/Hkv).
 *  - Attention ("Training Infrastructure and Systems", "FlashAttention: never
 *    write the score matrix"): out = softmax(scale * Q K^T) V over the allowed
 *    keys, computed tile by tile with an online softmax; only out and one
 *    per-row statistic are written.  The statistic is
 *    lse = ln(sum over allowed t of exp(scale * <q, k_t>)), natural log.
 *  - Backward: the scores are recomputed; dq, dk, dv follow the chain rule of
 *    softmax attention.  dk and dv are summed over the Hq/Hkv query heads of
 *    each KV head and returned in fp32 (the pages accumulate gradients in
 *    FP32, Herd section 3.3.2, "Numerical stability").
 *
 * Local row layout.  q, out, dout, dq hold Sq = 2*c rows per batch entry:
 * rows 0..c-1 are chunk cp_rank (global positions cp_rank*c + j), rows
 * c..2c-1 are chunk 2*cp_size-1-cp_rank, both in ascending position order.
 *
 * Tensor layouts (all contiguous, row-major, device memory):
 *   q, out, dout, dq : bf16  [B, Sq, Hq, D]
 *   k, v             : bf16  [B, Skv, Hkv, D]  global sequence order 0..Skv-1
 *   dk, dv           : fp32  [B, Skv, Hkv, D]
 *   lse              : fp32  [B, Sq, Hq]
 *   doc_ids          : int32 [B, S]   per-token document id
 *   cu_seqlens       : int32 [n_docs+1] document offsets 0 = cu[0] < ... <
 *                      cu[n_docs] = S (B == 1 only)
 * bf16 tensors must be 16-byte aligned; fp32 and int32 tensors 4-byte aligned.
 *
 * Preconditions that are not checked by the calls (see
 * docmask_gqa_check_docs for a synchronous debug check): equal document ids
 * form one contiguous run of positions; cu_seqlens is strictly increasing.
 * |dout| must be finite.
 *
 * Ownership.  The caller allocates and frees every buffer, including the
 * workspace (size from the *_workspace_size queries).  The library allocates
 * no device memory and keeps no state between calls; calls are asynchronous
 * on `stream` (a hipStream_t; NULL = the default stream) and re-entrant when
 * different calls use different workspaces.  Every element of out, lse, dq,
 * dk and dv is written, including zeros for dk/dv rows that no local query
 * reaches.  The workspace contents are not needed after a call returns.
 *
 * Errors.  Every function returns 0 on success or a negative status.  All
 * argument checks happen before any HIP call, so a rejected call touches no
 * memory.  Device-side faults surface at the caller's next synchronisation.
 */
#ifndef DOCMASK_GQA_H
#define DOCMASK_GQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  DMGQA_OK = 0,
  DMGQA_ERR_INVALID_ARG = -1,  /* null pointer, misalignment, bad rank,
                                  S % (2*cp_size) != 0, Hq % Hkv != 0, Skv
                                  outside [(2*cp_size-cp_rank)*c, S], both or
                                  neither of doc_ids / cu_seqlens,
                                  softmax_scale not finite and positive,
                                  negative sizes */
  DMGQA_ERR_UNSUPPORTED = -2,  /* D not in {64, 128}; cu_seqlens with B > 1;
                                  sizes whose element offsets overflow */
  DMGQA_ERR_WORKSPACE = -3,    /* workspace_bytes below the required size
                                  (for the backward: below the minimum) */
  DMGQA_ERR_HIP = -4           /* a HIP launch or runtime call failed */
};

/* Bytes of workspace the forward call needs.  Depends only on the sizes;
 * 0 when there is nothing to compute. */
size_t docmask_gqa_fwd_workspace_size(int32_t B, int32_t S, int32_t Skv,
                                      int32_t Hq, int32_t Hkv, int32_t D,
                                      int32_t cp_size);

/* The forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same computation and arguments as
 * docmask_gqa_attn_fwd, with the workspace in a fixed array of 8 MiB that
 * the library holds on each GPU it runs on until the process ends.  The
 * call allocates nothing; its first call on a device looks up that device's
 * array.  Shapes whose forward workspace (docmask_gqa_fwd_workspace_size)
 * exceeds 8 MiB are rejected with DMGQA_ERR_WORKSPACE before any HIP call
 * (about B * Skv <= 10^6 key positions at 16 query heads per KV head).
 * Every call on one GPU uses that GPU's single array, so calls that overlap
 * in time on one GPU (different streams or host threads) race and must be
 * ordered by the caller. */
int docmask_gqa_attn_fwd_noalloc(const void* q, const void* k, const void* v,
                                 const int32_t* doc_ids,
                                 const int32_t* cu_seqlens, int32_t n_docs,
                                 int32_t B, int32_t S, int32_t Skv, int32_t Hq,
                                 int32_t Hkv, int32_t D, int32_t cp_size,
                                 int32_t cp_rank, float softmax_scale,
                                 void* out, float* lse, void* stream);

/* Backward workspace.  Besides the scheduling arrays (the minimum below),
 * the backward can use a stash for dS in bf16 (blocks of 32 query rows x 128
 * keys of one key tile): the dK/dV kernel, which forms dS anyway, stores it,
 * and dQ = scale * dS K becomes one product per key tile instead of
 * recomputing the scores, P and dP.  The stash a batch needs depends on its
 * documents (about 2 bytes per allowed (query row, key) pair and query head),
 * so the call plans it from the workspace it is given:
 *  - room for the worst case over all document layouts of this rank's shape
 *    (docmask_gqa_bwd_workspace_size_full): every key tile is stashed;
 *  - less, but more than the minimum plus an fp32 buffer of B*Sq*Hq*D floats
 *    (partial dQ) and one stash block per KV head: key tiles are stashed in
 *    order (batch row, then key position) while their blocks fit, and the
 *    query tiles that reach the others recompute those tiles' share of dQ;
 *  - otherwise no stash: dQ recomputes the scores for every key tile.
 * All three give the same results up to the order of rounding.
 *
 * docmask_gqa_bwd_workspace_size: the default.  The worst-case stash if it
 * fits in a budget of 2 GiB (all KV heads together), else the smaller of
 * that worst case and the minimum plus the partial-dQ buffer plus a 2 GiB
 * stash.  For an 8K-token share with 16
 * query heads per KV head (d = 128) that is about 1.1 GiB; the stash does
 * not grow past the budget for longer sequences.
 * docmask_gqa_bwd_workspace_size_full: the minimum plus the worst-case stash
 * (quadratic in the sequence: about Sq * Hq * Skv bytes).
 * docmask_gqa_bwd_workspace_size_min: the smallest workspace the backward
 * accepts (no stash).
 * The sizes depend only on the arguments; they hold for every cp_rank
 * whose K/V prefix fits in Skv.  0 when there is nothing to compute or the
 * sizes are invalid. */
size_t docmask_gqa_bwd_workspace_size(int32_t B, int32_t S, int32_t Skv,
                                      int32_t Hq, int32_t Hkv, int32_t D,
                                      int32_t cp_size);
size_t docmask_gqa_bwd_workspace_size_full(int32_t B, int32_t S, int32_t Skv,
                                           int32_t Hq, int32_t Hkv, int32_t D,
                                           int32_t cp_size);
size_t docmask_gqa_bwd_workspace_size_min(int32_t B, int32_t S, int32_t Skv,
                                          int32_t Hq, int32_t Hkv, int32_t D,
                                          int32_t cp_size);

/* Which way the backward will form dQ with a workspace of workspace_bytes
 * for these arguments (no HIP call): DMGQA_BWD_PATH_STASH (every key tile
 * stashed), DMGQA_BWD_PATH_MIXED (stash with a budget, the rest
 * recomputed), DMGQA_BWD_PATH_RECOMPUTE, or a negative status for arguments
 * the backward would reject (DMGQA_ERR_WORKSPACE below the minimum). */
enum {
  DMGQA_BWD_PATH_RECOMPUTE = 0,
  DMGQA_BWD_PATH_STASH = 1,
  DMGQA_BWD_PATH_MIXED = 2
};
int docmask_gqa_bwd_path(int32_t B, int32_t S, int32_t Skv, int32_t Hq,
                         int32_t Hkv, int32_t D, int32_t cp_size,
                         int32_t cp_rank, size_t workspace_bytes);

/* Forward: out = softmax(scale * q k^T, masked) v and lse for the rank's
 * local rows.  Exactly one of doc_ids / cu_seqlens is non-NULL; n_docs is
 * read only with cu_seqlens.  softmax_scale must be finite and positive,
 * normally 1/sqrt(D). */
int docmask_gqa_attn_fwd(const void* q, const void* k, const void* v,
                         const int32_t* doc_ids, const int32_t* cu_seqlens,
                         int32_t n_docs, int32_t B, int32_t S, int32_t Skv,
                         int32_t Hq, int32_t Hkv, int32_t D, int32_t cp_size,
                         int32_t cp_rank, float softmax_scale, void* out,
                         float* lse, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Backward: given the forward's out and lse and the output gradient dout,
 * writes dq (bf16), dk and dv (fp32, summed over each KV head's query
 * heads).  Same masking arguments as the forward. */
int docmask_gqa_attn_bwd(const void* q, const void* k, const void* v,
                         const void* out, const void* dout, const float* lse,
                         const int32_t* doc_ids, const int32_t* cu_seqlens,
                         int32_t n_docs, int32_t B, int32_t S, int32_t Skv,
                         int32_t Hq, int32_t Hkv, int32_t D, int32_t cp_size,
                         int32_t cp_rank, float softmax_scale, void* dq,
                         float* dk, float* dv, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Document bounds of every key position, for callers that run several
 * calls on the same batch (the forward and the backward of every layer):
 *   bounds[0][b][t] = first position of t's document,
 *   bounds[1][b][t] = one past its last position, capped at Skv,
 * int32 [2, B, Skv] at the start of `bounds`, followed by scratch.  With the
 * causal mask, query position p may attend to keys bounds[0][b][p] .. p
 * (the document mask of "Paper notes: The Llama 3 Herd of Models", "Two
 * architectural choices", as an interval per position).  Exactly one of
 * doc_ids / cu_seqlens, as for the attention calls.  The caller allocates
 * `bounds` (docmask_gqa_doc_bounds_size bytes, 4-byte aligned) and keeps it
 * while later calls read it; the call is asynchronous on `stream`.
 * docmask_gqa_doc_bounds_size returns 0 for invalid sizes. */
size_t docmask_gqa_doc_bounds_size(int32_t B, int32_t S, int32_t Skv);
int docmask_gqa_doc_bounds(const int32_t* doc_ids, const int32_t* cu_seqlens,
                           int32_t n_docs, int32_t B, int32_t S, int32_t Skv,
                           int32_t* bounds, size_t bounds_bytes, void* stream);

/* Bounds of a causal interval mask: query position p (global, 0 <= p < S)
 * attends to keys lo[b][p] .. p, where lo (int32 [B, S], device, 4-byte
 * aligned) is non-decreasing along p with 0 <= lo[p] <= p.  The all-gathered
 * K/V let each CP rank apply such masks ("Scaling Llama 3 Training with
 * Efficient Parallelism Strategies", section "Context Parallelism (CP)",
 * Figure 7: causal, document and CP-document masks); besides the document
 * mask (lo = first position of p's document) this covers a sliding window
 * of W keys, also inside documents (lo = max(document start, p - W + 1)).
 * Writes the same bounds array as docmask_gqa_doc_bounds (same size:
 * docmask_gqa_doc_bounds_size(B, S, Skv)), for the *_bounds calls:
 *   bounds[0][b][t] = lo[b][t],
 *   bounds[1][b][t] = one past the last p with lo[b][p] <= t, capped at Skv.
 * Asynchronous on `stream`; lo is not validated (precondition; see
 * docmask_gqa_check_intervals): other lo arrays give undefined results. */
int docmask_gqa_interval_bounds(const int32_t* lo, int32_t B, int32_t S,
                                int32_t Skv, int32_t* bounds,
                                size_t bounds_bytes, void* stream);

/* Cross-attention forward and backward: non-causal intervals with explicit
 * ends.  From
 * "Scaling Llama 3 Training with Efficient Parallelism Strategies", the
 * section on pipeline parallelism for multimodal training (Figure 5 and its
 * second challenge): cross-attention layers take image sequences of 1.2K-3K
 * tokens next to text of under 200 tokens.  Query token p (no context
 * parallelism: the rows of q are the S tokens in order) attends to keys
 * lo[b][p] .. hi[b][p]-1 of k and v, whose rows are indexed on their own
 * (for example the image tokens of p's sample).
 *   q, out, dout, dq : bf16 [B, S, Hq, D] (any S >= 0);
 *   k, v : bf16 [B, Skv, Hkv, D];  dk, dv : fp32 [B, Skv, Hkv, D];
 *   lse    : fp32 [B, S, Hq];
 *   lo, hi : int32 [B, S] device arrays, non-decreasing in p, with
 *            0 <= lo[b][p] < hi[b][p] <= Skv.  These are preconditions the
 *            call does not check; docmask_gqa_check_cross_intervals checks
 *            them synchronously and returns 0 (valid) or 1.
 * Forward workspace: docmask_gqa_fwd_cross_workspace_size bytes (the tile
 * order).  The backward takes the forward's out and lse and dout, and writes
 * dq and dk, dv (summed over each KV head's query heads, zero for keys no
 * query reaches) as the causal backward does, with the same three ways of
 * forming dQ, chosen from workspace_bytes:
 *  - docmask_gqa_bwd_cross_workspace_size_min bytes (the keys' query ranges,
 *    the schedule, the row statistics and the partial sums): no stash, dQ
 *    recomputes the scores;
 *  - more: a bf16 dS stash in the rest, key tiles stashed in order while
 *    their blocks fit (every tile when the rest holds the worst case, in
 *    which each key tile reaches all S query tokens; otherwise the mixed
 *    form, which also needs an fp32 [B, S, Hq, D] partial-dQ buffer and
 *    recomputes the key tiles past the budget);
 *  - docmask_gqa_bwd_cross_workspace_size: the minimum plus the worst-case
 *    stash, or the partial-dQ buffer plus a 2 GiB stash budget when the
 *    worst case is larger (at the multimodal sizes above the blocks the
 *    samples actually reach, a few hundred MiB, fit in that budget).
 * Only the image encoder and the cross-attention layers are trained in that
 * setting (same section), so this is the backward that runs.  Errors and
 * ownership as above. */
size_t docmask_gqa_fwd_cross_workspace_size(int32_t B, int32_t S, int32_t Skv,
                                            int32_t Hq, int32_t Hkv, int32_t D);
int docmask_gqa_attn_fwd_cross(const void* q, const void* k, const void* v,
                               const int32_t* lo, const int32_t* hi, int32_t B,
                               int32_t S, int32_t Skv, int32_t Hq, int32_t Hkv,
                               int32_t D, float softmax_scale, void* out,
                               float* lse, void* workspace,
                               size_t workspace_bytes, void* stream);
size_t docmask_gqa_bwd_cross_workspace_size(int32_t B, int32_t S, int32_t Skv,
                                            int32_t Hq, int32_t Hkv, int32_t D);
size_t docmask_gqa_bwd_cross_workspace_size_min(int32_t B, int32_t S, int32_t Skv,
                                                int32_t Hq, int32_t Hkv, int32_t D);
/* Which way the cross-attention backward will form dQ with a workspace of
 * workspace_bytes (no HIP call): the DMGQA_BWD_PATH_* values of
 * docmask_gqa_bwd_path, or a negative status for shapes the backward would
 * reject (DMGQA_ERR_WORKSPACE below the minimum).  The stash path needs
 * the worst case above; smaller workspaces past the minimum and the
 * partial-dQ buffer give the mixed path. */
int docmask_gqa_bwd_cross_path(int32_t B, int32_t S, int32_t Skv, int32_t Hq,
                               int32_t Hkv, int32_t D, size_t workspace_bytes);
int docmask_gqa_attn_bwd_cross(const void* q, const void* k, const void* v,
                               const void* out, const void* dout,
                               const float* lse, const int32_t* lo,
                               const int32_t* hi, int32_t B, int32_t S,
                               int32_t Skv, int32_t Hq, int32_t Hkv, int32_t D,
                               float softmax_scale, void* dq, float* dk,
                               float* dv, void* workspace,
                               size_t workspace_bytes, void* stream);
int docmask_gqa_check_cross_intervals(const int32_t* lo, const int32_t* hi,
                                      int32_t B, int32_t S, int32_t Skv,
                                      void* stream);

/* The forward and backward with the masking given as a bounds array from
 * docmask_gqa_doc_bounds or docmask_gqa_interval_bounds (same B, S and
 * Skv; its writes ordered before these calls) instead of doc_ids /
 * cu_seqlens; everything else as in docmask_gqa_attn_fwd /
 * docmask_gqa_attn_bwd, with the same workspace sizes.  The bounds are not validated against the sizes beyond alignment:
 * a bounds array of other sizes is undefined behaviour. */
int docmask_gqa_attn_fwd_bounds(const void* q, const void* k, const void* v,
                                const int32_t* bounds, int32_t B, int32_t S,
                                int32_t Skv, int32_t Hq, int32_t Hkv, int32_t D,
                                int32_t cp_size, int32_t cp_rank,
                                float softmax_scale, void* out, float* lse,
                                void* workspace, size_t workspace_bytes,
                                void* stream);
int docmask_gqa_attn_bwd_bounds(const void* q, const void* k, const void* v,
                                const void* out, const void* dout,
                                const float* lse, const int32_t* bounds,
                                int32_t B, int32_t S, int32_t Skv, int32_t Hq,
                                int32_t Hkv, int32_t D, int32_t cp_size,
                                int32_t cp_rank, float softmax_scale, void* dq,
                                float* dk, float* dv, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Batch plan: the bounds of docmask_gqa_doc_bounds together with the
 * query-tile orders that the forward and the backward's dQ kernel
 * otherwise build in every call (query tiles of 128 rows by decreasing
 * number of key tiles they reach, so that the longest tiles start first).
 * The bounds and orders depend only on the document layout and on (B, S,
 * Skv, Hq, Hkv, cp_size, cp_rank), not on q, k, v: the same layout serves
 * every layer of a training step ("Paper notes: The Llama 3 Herd of
 * Models", "Two architectural choices": the document mask is a property of
 * the packed sequence), so a caller builds the plan once per batch and
 * passes it to each layer's *_plan calls.  The bounds scan of
 * docmask_gqa_doc_bounds, then one launch for both orders.
 *   docmask_gqa_batch_plan_size: bytes of the plan for any rank of the
 *     shape (0 for invalid sizes); D only enters the shape checks.
 *   docmask_gqa_batch_plan: doc_ids or cu_seqlens as for the attention
 *     calls; plan: device buffer of at least that many bytes, 4-byte aligned,
 *     owned by the caller and kept while later calls read it; asynchronous
 *     on `stream`.  Layout (int32): the bounds array [2, B, Skv] as written by
 *     docmask_gqa_doc_bounds (so the plan also serves as `bounds` of the
 *     *_bounds calls), the forward order, the dQ order, scratch.
 *   docmask_gqa_attn_fwd_plan / docmask_gqa_attn_bwd_plan: as the *_bounds
 *     calls, reading the plan's bounds and order; workspace sizes as for
 *     docmask_gqa_attn_fwd / docmask_gqa_attn_bwd.  The plan must come from
 *     docmask_gqa_batch_plan with the same B, S, Skv, Hq, Hkv, cp_size and
 *     cp_rank (not checked: another plan is undefined behaviour). */
size_t docmask_gqa_batch_plan_size(int32_t B, int32_t S, int32_t Skv,
                                   int32_t Hq, int32_t Hkv, int32_t D,
                                   int32_t cp_size);
int docmask_gqa_batch_plan(const int32_t* doc_ids, const int32_t* cu_seqlens,
                           int32_t n_docs, int32_t B, int32_t S, int32_t Skv,
                           int32_t Hq, int32_t Hkv, int32_t D, int32_t cp_size,
                           int32_t cp_rank, int32_t* plan, size_t plan_bytes,
                           void* stream);
int docmask_gqa_attn_fwd_plan(const void* q, const void* k, const void* v,
                              const int32_t* plan, int32_t B, int32_t S,
                              int32_t Skv, int32_t Hq, int32_t Hkv, int32_t D,
                              int32_t cp_size, int32_t cp_rank,
                              float softmax_scale, void* out, float* lse,
                              void* workspace, size_t workspace_bytes,
                              void* stream);
int docmask_gqa_attn_bwd_plan(const void* q, const void* k, const void* v,
                              const void* out, const void* dout,
                              const float* lse, const int32_t* plan, int32_t B,
                              int32_t S, int32_t Skv, int32_t Hq, int32_t Hkv,
                              int32_t D, int32_t cp_size, int32_t cp_rank,
                              float softmax_scale, void* dq, float* dk,
                              float* dv, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Debug mode: with the environment variable DMGQA_DEBUG set to a value
 * other than "0" (read at every call), each call that takes document ids,
 * cu_seqlens or interval arrays first runs the matching synchronous check
 * below on them and returns DMGQA_ERR_INVALID_ARG (launching nothing) if the
 * precondition does not hold.  The checks copy the arrays to the host and
 * synchronise the stream: for debugging, not for graph capture or timing. */

/* Debug check of the document-id precondition.  Copies doc_ids [B, S] to the
 * host, synchronising `stream`.  Returns 0 if every id forms one contiguous
 * run in each batch row, 1 if some id reappears after a different id,
 * or a negative status. */
int docmask_gqa_check_docs(const int32_t* doc_ids, int32_t B, int32_t S,
                           void* stream);

/* Debug check of the interval precondition: copies lo [B, S] to the host,
 * synchronising `stream`.  Returns 0 if every row is non-decreasing with
 * 0 <= lo[p] <= p, 1 otherwise, or a negative status. */
int docmask_gqa_check_intervals(const int32_t* lo, int32_t B, int32_t S,
                                void* stream);

/* Debug check of cu_seqlens [n_docs+1] (synchronises `stream`).  Returns 0
 * if cu[0] == 0, cu[n_docs] == S and the offsets strictly increase, 1
 * otherwise, or a negative status. */
int docmask_gqa_check_cu_seqlens(const int32_t* cu_seqlens, int32_t n_docs,
                                 int32_t S, void* stream);

/* Kernel timing, for benchmarks.  docmask_gqa_timing_enable(1) clears the
 * records and makes every later kernel launch of the library record a HIP
 * event before and after it on the call's stream (events are created on
 * first use and kept until the process ends); enable(0) stops recording.
 * docmask_gqa_timing_read(kernel, &ms, &n) waits for the recorded events and
 * returns the summed duration and launch count of one kernel since the last
 * enable.  Kernel ids are 0 .. docmask_gqa_kernel_count()-1 with names from
 * docmask_gqa_kernel_name().  Not thread-safe with concurrent calls that
 * also record. */
int docmask_gqa_timing_enable(int on);
int docmask_gqa_timing_read(int kernel, double* total_ms, int* launches);
int docmask_gqa_kernel_count(void);
const char* docmask_gqa_kernel_name(int kernel);

/* Static description of a status code. */
const char* docmask_gqa_status_string(int status);

/* Library version, major*10000 + minor*100 + patch. */
int docmask_gqa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DOCMASK_GQA_H */
