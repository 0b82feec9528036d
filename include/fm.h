/*
 * fm.h -- C ABI of the column-wise-mask (FlashMask) exact attention library for AMD MI355X (gfx950).
 *
 * What is computed.  Exact softmax attention, forward and backward, under a column-wise sparse mask:
 * each key column j carries four query-axis boundaries LTS_j, LTE_j, UTS_j, UTE_j (FlashMask abstract,
 * papers.pytorch.kr 2410.01359: a column-wise sparse representation with O(N) memory; FlashMask-3
 * summary, readmex.ai, abstract body: four query-axis boundary vectors, indexed by key position,
 * storing query-axis interval boundaries). Query row i is masked for key column j when
 *     (causal and i < j)  or  LTS_j <= i < LTE_j  or  UTS_j <= i < UTE_j
 * (half-open intervals; an interval with start >= end is empty; values outside [0, N) are clipped
 * by this set definition and are not an error). Masked scores are excluded from the softmax. A query
 * row with every key masked yields out = 0, lse = -inf, a zero dq row and no dk/dv contribution.
 *
 * Tiles whose every (row, column) is masked are skipped and tiles with no masked entry run without
 * the elementwise mask: the kernels use the mask's sparsity to drop work, at no cost in accuracy
 * (FlashMask abstract). The result does not depend on the classification: it only decides which work
 * is done.
 *
 * Conventions shared by every call:
 *  - All tensor pointers are DEVICE pointers owned by the caller. The library keeps no pointer after
 *    a call returns, allocates nothing and keeps no state between calls.
 *  - Every call is asynchronous on `stream` (0 = the null stream) and never synchronizes. Argument
 *    errors are detected on the host before any launch, so a failing call launches nothing.
 *  - Layout: q, k, v, out, dout, dq, dk, dv are contiguous row-major [B, H, N, d] of `dtype`
 *    (self-attention: N queries and N keys, the same H for queries and keys). lse is float32
 *    [B, H, N], natural log of the sum of exp(scale * q.k) over the unmasked keys.
 *  - Mask vectors are contiguous int32 [B, Hm, N] with Hm = 1 (shared by all heads) or Hm = H.
 *    A pair (LTS, LTE) or (UTS, UTE) may be NULL as a pair: that interval is empty. One NULL and one
 *    non-NULL pointer in a pair is FM_ERR_INVALID.
 *  - bounds is int32 [B, Hm, ceil(N / fm_kblock()), 8] as written by fm_tile_bounds for the same
 *    vectors. It may be NULL only when all four vectors are NULL. Bounds that do not belong to the
 *    vectors give wrong results but never out-of-range memory accesses.
 *  - sched is NULL or an int32 schedule written by fm_tile_schedule for the same bounds, sizes, q_off
 *    and causal flag. It changes only the order in which work units are dispatched, never a result
 *    (every unit is independent and accumulates on chip). A schedule array of the right size whose
 *    content does not belong to the problem gives wrong results but never out-of-range accesses.
 *  - Outputs must not alias inputs or each other.
 */
#ifndef FM_H
#define FM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FM_OK = 0,
  FM_ERR_INVALID = 1,     /* NULL required pointer, B/H/N out of range, Hm not in {1, H}, half-NULL pair,
                             scale not finite and positive, vectors without bounds, qblock not positive */
  FM_ERR_UNSUPPORTED = 2, /* d not in {64, 128} or unknown dtype */
  FM_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than fm_bwd_workspace_bytes() */
  FM_ERR_LAUNCH = 4,      /* the HIP runtime reported an error for a launch */
  /* range markers, never returned: every int is a value of the type, so a value the library does not
   * know (fm_status_str of an arbitrary int) is handled rather than undefined */
  FM_STATUS_RANGE_MIN_ = -2147483647 - 1,
  FM_STATUS_RANGE_MAX_ = 2147483647
} fm_status;

typedef enum {
  FM_BF16 = 0,
  FM_F32 = 1,
  /* range markers, not dtypes: an unknown dtype value is FM_ERR_UNSUPPORTED rather than undefined */
  FM_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  FM_DTYPE_RANGE_MAX_ = 2147483647
} fm_dtype;

/* Largest N accepted by every call (row and column indices stay within int32 arithmetic). */
#define FM_MAX_N (1 << 24)

/* Width in key columns of one bounds entry (64). */
int fm_kblock(void);

/* Query rows per forward tile for head dim d (the qblock at which the forward kernel classifies
   tiles), or 0 for an unsupported d. */
int fm_fwd_qblock(int d);

/* Number of int32 elements of the bounds array: B * Hm * ceil(N / kblock) * 8 (0 on bad sizes). */
size_t fm_bounds_elems(int B, int Hm, int N);

/* Per-key-tile bounds pre-pass.
 * For each (b, hm, key tile t) over the valid columns c in [t*kblock, min(N, (t+1)*kblock)) writes
 *   bounds[b][hm][t][0..7] = min LTS, max LTS, min LTE, max LTE, min UTS, max UTS, min UTE, max UTE.
 * A NULL pair writes the canonical empty values: LT -> N, N, N, N; UT -> 0, 0, 0, 0.
 * The pages name no such pass; it is the per-tile summary from which the tile classification is read.
 * The vectors need no alignment beyond int32; when every row starts on a 16-byte boundary (16-byte
 * aligned pointers and N a multiple of 4) they are read with 16-byte loads. HBM-bound: each vector
 * element is read once.
 * Errors: FM_ERR_INVALID (bounds NULL, sizes out of range, half-NULL pair). */
fm_status fm_tile_bounds(const int32_t* lts, const int32_t* lte, const int32_t* uts, const int32_t* ute,
                         int B, int Hm, int N, int32_t* bounds, hipStream_t stream);

/* Longest-first dispatch schedule (the single-GPU form of the sparsity-aware load balancing that the
 * FlashMask-3 summary, readmex.ai, applies to masked attention across workers). The kernels' work units
 * are query units of 128 rows (forward, dq) and key units of 128 columns (dk, dv); the work of a unit is
 * the number of tiles on its row of the tile grid (64-column key tiles) or its column (64-row query
 * tiles) that the tile classification does not mark fully masked, with rows q_off + i. For each
 * (b, hm) row of the mask, with nq = ceil(Nq / 128) and nk = ceil(Nk / 128), sched holds
 *   [0, nq)              the query units in decreasing order of work (equal work: latest unit first)
 *   [nq, nq + nk)        the key units in decreasing order of work (equal work: earliest unit first)
 *   [nq + nk, 2nq + nk)  the work of each query unit, then [2nq + nk, 2(nq + nk)) that of each key unit.
 * Workgroups are handed to the hardware in that order, which is the longest-processing-time-first list
 * rule; equal work keeps the order used without a schedule. bounds as for fm_fwd (NULL when there are no
 * vectors); sched is a caller-owned device array of fm_schedule_elems(B, Hm, Nq, Nk) int32.
 * Errors: FM_ERR_INVALID (sched NULL, sizes out of range), FM_ERR_LAUNCH. */
size_t fm_schedule_elems(int B, int Hm, int Nq, int Nk);
fm_status fm_tile_schedule(const int32_t* bounds, int B, int Hm, int Nq, int Nk, int q_off, int causal,
                           int32_t* sched, hipStream_t stream);

/* Forward pass (FlashMask abstract: exact attention with mask-driven skipping; FlashAttention-3
 * abstract, fugumt.com 2407.08608: tiled online softmax).
 *   out[b,h,i,:] = sum_j P_ij v[b,h,j,:],  P_ij = exp(S_ij - lse_i) on unmasked (i, j), 0 elsewhere,
 *   S_ij = scale * q[b,h,i,:] . k[b,h,j,:],  lse[b,h,i] = log(sum over unmasked j of exp(S_ij)).
 * Vectors for head h are read at [b, (Hm == H ? h : 0), :]. causal != 0 adds the i < j mask.
 * scale must be finite and positive (the usual 1 / sqrt(d)).
 * bf16 inputs use bf16 matrix products with float32 accumulation and a float32 softmax; out is
 * rounded to bf16 (nearest even). float32 inputs use float32 matrix products.
 * Errors: FM_ERR_INVALID, FM_ERR_UNSUPPORTED, FM_ERR_LAUNCH. */
fm_status fm_fwd(const void* q, const void* k, const void* v, fm_dtype dtype, int B, int H, int N, int d,
                 const int32_t* lts, const int32_t* lte, const int32_t* uts, const int32_t* ute, int Hm,
                 const int32_t* bounds, const int32_t* sched, int causal, float scale, void* out, float* lse,
                 hipStream_t stream);

/* Device workspace fm_bwd needs: the float32 [B, H, N] row term D_i = sum_k dout_ik out_ik, rounded up
 * to 256 bytes. 0 on bad sizes. */
size_t fm_bwd_workspace_bytes(fm_dtype dtype, int B, int H, int N, int d);

/* Backward pass: gradients of sum(out * dout) with out from fm_fwd on the same inputs and mask.
 *   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  dQ = scale dS K,  dK = scale dS^T Q,
 * with P recomputed from q, k and the forward's lse. A query-tile-parallel pass forms D and dq (each
 * query tile accumulates its dq rows on chip over the live key tiles); a key-tile-parallel pass then
 * forms dk and dv (each key tile accumulates on chip over the live query tiles). No atomics: the result
 * is bitwise reproducible. dq, dk, dv have `dtype`. The workspace receives D (its previous content does
 * not matter) and must not be shared by concurrent calls.
 * Errors: FM_ERR_INVALID, FM_ERR_UNSUPPORTED, FM_ERR_WORKSPACE, FM_ERR_LAUNCH. */
fm_status fm_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                 const float* lse, fm_dtype dtype, int B, int H, int N, int d,
                 const int32_t* lts, const int32_t* lte, const int32_t* uts, const int32_t* ute, int Hm,
                 const int32_t* bounds, const int32_t* sched, int causal, float scale, void* dq, void* dk,
                 void* dv, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Backward with stored dS tiles: the same gradients as fm_bwd, with dq formed from dS tiles that the
 * key-tile-parallel pass writes to the workspace instead of by a second pass that recomputes S, dP and dS
 * (4 d FLOP per unmasked pair less matrix work, for 2 bytes of HBM writes and reads per stored pair).
 * The pages do not describe the backward's work split; the tiles the mask covers completely are skipped
 * as in the forward (FlashMask abstract, papers.pytorch.kr 2410.01359). A stored tile is 64 query rows x
 * 128 keys of bf16 (fm_bwd_ds_workspace_bytes per tile: 16 KB); a head needs one tile per (128-key tile,
 * 64-row query tile) between the first and the last query tile that is not fully masked for that key tile,
 * so the space grows with the unmasked pairs (about 2 bytes each for the document masks), not with N^2.
 *
 * fm_bwd_plan_bytes(B, H, Hm, N): device bytes of a plan (0 on bad sizes).
 * fm_bwd_plan(bounds, B, H, Hm, N, causal, plan, stream): writes the plan of the mask into the caller's
 *   device buffer `plan` (8-byte aligned, fm_bwd_plan_bytes long): per key tile its first live query
 *   tile and its first slot, per head its region, and in the first 8 bytes the int64 number of tiles of
 *   the whole problem. bounds as for fm_bwd (NULL when there are no vectors). A plan depends only on the
 *   bounds, the sizes and the causal flag: recompute it when the mask changes. Asynchronous like every
 *   call: read the total back (after synchronising) to size the workspace.
 * fm_bwd_ds_workspace_bytes(dtype, B, H, N, d, tiles): fm_bwd_workspace_bytes plus `tiles` stored tiles
 *   (0 on bad sizes or overflow).
 * fm_bwd_ds(...): the arguments of fm_bwd plus the plan. The workspace holds D first (as fm_bwd) and
 *   stored tiles in the rest: a head whose region fits gets its dS stored and its dq streamed; a head
 *   that does not fit (or any head, for float32 inputs) runs as in fm_bwd. Every head meets the same
 *   accuracy; results are bitwise reproducible for a given workspace size. The plan must come from
 *   fm_bwd_plan with the same B, H, Hm and N (its size and layout follow from them); a plan of those sizes
 *   whose content belongs to other bounds or another causal flag gives wrong results but never accesses
 *   memory outside the plan, the workspace or the tensors.
 * Errors: as fm_bwd; FM_ERR_INVALID for a NULL or misaligned plan. */
size_t fm_bwd_plan_bytes(int B, int H, int Hm, int N);
fm_status fm_bwd_plan(const int32_t* bounds, int B, int H, int Hm, int N, int causal, void* plan,
                      hipStream_t stream);
size_t fm_bwd_ds_workspace_bytes(fm_dtype dtype, int B, int H, int N, int d, int64_t tiles);
fm_status fm_bwd_ds(const void* q, const void* k, const void* v, const void* out, const void* dout,
                    const float* lse, fm_dtype dtype, int B, int H, int N, int d, const int32_t* lts,
                    const int32_t* lte, const int32_t* uts, const int32_t* ute, int Hm, const int32_t* bounds,
                    const int32_t* sched, const void* plan, int causal, float scale, void* dq, void* dk, void* dv,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* fm_bwd that allocates nothing, for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same arguments, results and
 * errors as fm_bwd without the workspace, whose D row term lives instead in a fixed array of
 * FM_NOALLOC_SCRATCH_BYTES in the library's device memory (one per GPU, held until the process ends).
 * Limit: B * H * N * 4 <= FM_NOALLOC_SCRATCH_BYTES (B * H * N <= 4194304); larger problems get
 * FM_ERR_WORKSPACE. Every call on a GPU shares that GPU's array: calls that overlap on one GPU (on
 * different streams) race. Nothing in the array needs clearing: each call writes it before reading it.
 * FM_ERR_LAUNCH also when the array's address cannot be looked up on the current device. */
#define FM_NOALLOC_SCRATCH_BYTES (16u << 20)
fm_status fm_bwd_noalloc(const void* q, const void* k, const void* v, const void* out, const void* dout,
                         const float* lse, fm_dtype dtype, int B, int H, int N, int d, const int32_t* lts,
                         const int32_t* lte, const int32_t* uts, const int32_t* ute, int Hm, const int32_t* bounds,
                         const int32_t* sched, int causal, float scale, void* dq, void* dk, void* dv,
                         hipStream_t stream);

/* One block of query rows against all keys: the unit of work of one rank under context parallelism,
 * whose mask localisation is a zero-communication clip-shift-max on the boundary vectors that keeps the
 * single-GPU kernel (FlashMask-3 summary, readmex.ai, the quoted abstract in the "in-depth insights"
 * section). Here the kernels apply that shift to their own row indices: local query row i is global row
 * q_off + i, and the vectors, the tile bounds and the causal rule (q_off + i < j) are read in global
 * coordinates, so the caller passes the full vectors unchanged.
 *   q, out, dout, dq: [B, H, Nq, d]; lse: float32 [B, H, Nq]; k, v, dk, dv: [B, H, Nk, d];
 *   vectors: int32 [B, Hm, Nk] (values are global query rows); bounds from fm_tile_bounds(..., Nk, ...).
 * out, lse and dq are exactly those rows of the whole problem; dk and dv are the contributions of these
 * rows only (summing them over a partition of the rows gives the whole dk, dv). The workspace is
 * fm_bwd_workspace_bytes(dtype, B, H, Nq, d); a schedule comes from fm_tile_schedule(..., Nq, Nk, q_off, ...).
 * fm_fwd / fm_bwd are the case Nq = Nk = N, q_off = 0.
 * Errors as fm_fwd / fm_bwd; also FM_ERR_INVALID for q_off < 0 or q_off + Nq > FM_MAX_N. */
fm_status fm_fwd_rows(const void* q, const void* k, const void* v, fm_dtype dtype, int B, int H, int Nq, int Nk,
                      int q_off, int d, const int32_t* lts, const int32_t* lte, const int32_t* uts,
                      const int32_t* ute, int Hm, const int32_t* bounds, const int32_t* sched, int causal,
                      float scale, void* out, float* lse, hipStream_t stream);
fm_status fm_bwd_rows(const void* q, const void* k, const void* v, const void* out, const void* dout,
                      const float* lse, fm_dtype dtype, int B, int H, int Nq, int Nk, int q_off, int d,
                      const int32_t* lts, const int32_t* lte, const int32_t* uts, const int32_t* ute, int Hm,
                      const int32_t* bounds, const int32_t* sched, int causal, float scale, void* dq, void* dk,
                      void* dv, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Key compaction for masks that drop whole key columns (per-head key dropping with compute reduced in
 * proportion to the keys kept: SCFA review, nubint.ai, "proposed method"). A column is dropped when it
 * is masked for every query row i in [0, N) (its causal rows, LT and UT together cover [0, N)). For each
 * (b, hm) row of the mask vectors [B, Hm, N]:
 *   counts[b, hm]      number of kept columns K, or -1 if some kept column needs three disjoint row
 *                      intervals (causal rows [0, j) plus two disjoint, non-adjacent spans), which the
 *                      compacted mask cannot hold; the other outputs of that row are then unspecified;
 *   kidx[b, hm, r]     original index of the r-th kept column (increasing), -1 for r >= K;
 *   kpos[b, hm, j]     position of column j among the kept ones, -1 if dropped;
 *   lts2 .. ute2       the mask of the compacted problem, to be run with causal = 0: kept position r
 *                      holds column j's spans clipped to [0, N], with the causal rows [0, j) merged into
 *                      the UT span (or, if UT starts after j, into the LT span); positions r >= K mask
 *                      every row (LT = [0, N), UT empty). Empty spans are canonical (LT N, N; UT 0, 0).
 * Running fm_fwd / fm_bwd on K, V gathered by kidx (fm_gather_rows) with these vectors gives the same
 * out, lse and dq as the original problem; dk, dv come back by gathering with kpos. All outputs are
 * int32 device arrays owned by the caller; a NULL pair of inputs is an empty span.
 * Errors: FM_ERR_INVALID (NULL outputs, sizes out of range, half-NULL pair), FM_ERR_LAUNCH. */
fm_status fm_compact_keys(const int32_t* lts, const int32_t* lte, const int32_t* uts, const int32_t* ute, int B,
                          int Hm, int N, int causal, int32_t* kidx, int32_t* kpos, int32_t* counts, int32_t* lts2,
                          int32_t* lte2, int32_t* uts2, int32_t* ute2, hipStream_t stream);

/* Row gather: y[b, h, r, :] = x[b, h, idx[b, hm, r], :] with hm = (Hm == H ? h : 0), and zero where
 * idx is negative. x, y are contiguous [B, H, N, d] of dtype (16-byte aligned), idx is int32
 * [B, Hm, N] with values in [-1, N) (others give a zero row). With kidx it builds the compacted K and
 * V; with kpos it scatters the compacted dK and dV back to the original order. y must not alias x.
 * Errors: FM_ERR_INVALID, FM_ERR_UNSUPPORTED, FM_ERR_LAUNCH. */
fm_status fm_gather_rows(const void* x, fm_dtype dtype, int B, int H, int N, int d, const int32_t* idx, int Hm,
                         void* y, hipStream_t stream);

/* Hash-bucket sparse causal attention (SCFA review, nubint.ai, "proposed method" and Figure 3: exact
 * attention restricted to hash buckets, computed after reordering queries and keys by bucket, which gives
 * a non-triangular causal mask). Query i attends key j iff both have the same bucket and j <= i.
 *
 * fm_lsh_buckets: Reformer-style geometric hash of each row of x [B, H, N, d] (dtype, 16-byte aligned):
 *   buckets[b, h, i] = the first index of the maximum of the nb values [x_i R_h, -x_i R_h], with the
 *   rotation R_h = rot[h] (Hr = H) or rot[0] (Hr = 1), float32 [Hr, d, nb / 2] row-major, a random matrix
 *   the caller draws. Dot products are float32. bf16 rows use matrix-core products with R split into
 *   three bf16 parts (hi + mid + lo, within 2^-24 |R| of R), accumulated in float32. float32 rows use
 *   per-lane fused multiply-adds over 16-byte chunks of the row, combined by a fixed butterfly. Rows
 *   whose top two values differ by less than float32 rounding may get either bucket.
 *   Errors: FM_ERR_INVALID (NULL, sizes, Hr not in {1, H}, nb odd or outside [2, 64], x misaligned),
 *   FM_ERR_UNSUPPORTED (d, dtype), FM_ERR_LAUNCH.
 *
 * fm_bucket_sort: for query buckets qbucket and key buckets kbucket, int32 [B, H, N] (a value outside
 *   [0, nb) marks a dropped token, which attends and is attended by nothing), sorts queries and keys of
 *   each head stably by bucket, dropped tokens last, and writes int32 [B, H, N] arrays:
 *     qidx[r]  original query at sorted row r;     qpos[i]  sorted row of query i (inverse of qidx);
 *     kidx[c]  original key at sorted column c;    kpos[j]  sorted column of key j;
 *     lts .. ute  the sorted problem's mask (Hm = H, causal = 0): for the key at column c, of bucket b at
 *       position p, with bucket b's queries in rows [qs, qe): UT = [0, lo) where lo = qs + (bucket-b
 *       queries at positions < p), LT = [qe, N); a dropped key has UT = [0, N). Empty spans canonical.
 *   Running fm_fwd / fm_bwd (causal = 0) on Q, dO gathered by qidx and K, V gathered by kidx
 *   (fm_gather_rows) with these vectors computes the hash attention; out and dq come back by gathering
 *   with qpos, dk and dv with kpos; lse stays in sorted order (row qpos[i] holds query i's).
 *   Errors: FM_ERR_INVALID (NULL, sizes, nb outside [1, 512]), FM_ERR_LAUNCH. */
fm_status fm_lsh_buckets(const void* x, fm_dtype dtype, int B, int H, int N, int d, const float* rot, int Hr,
                         int nb, int32_t* buckets, hipStream_t stream);
fm_status fm_bucket_sort(const int32_t* qbucket, const int32_t* kbucket, int B, int H, int N, int nb, int32_t* qidx,
                         int32_t* qpos, int32_t* kidx, int32_t* kpos, int32_t* lts, int32_t* lte, int32_t* uts,
                         int32_t* ute, hipStream_t stream);

/* fm_fwd and fm_bwd on a reordered problem (the sorted one above), with the outputs stored in the
 * original order directly instead of gathered back (same SCFA passage: the hash attention's results are
 * the original tokens'). q, k, v, dout and lse are in the reordered order, exactly as for fm_fwd / fm_bwd.
 *   omap, qmap: int32 [B, H, N], reordered row r -> original row (fm_bucket_sort's qidx);
 *   kmap:       int32 [B, H, N], reordered key c -> original key (its kidx).
 *   fm_fwd_mapped writes out[b][h][omap[r]] = row r of the result; lse stays at row r.
 *   fm_bwd_mapped reads out through qmap (out as fm_fwd_mapped wrote it), writes dq[b][h][qmap[r]] and
 *   dk, dv [b][h][kmap[c]]. Values equal fm_fwd / fm_bwd followed by the gathers with qpos / kpos, bit for
 *   bit. A map entry outside [0, N) drops that row: nothing is written for it, and in the backward a
 *   query row whose qmap entry is out of range contributes nothing to dk and dv (as if its dout were
 *   zero). With a map that is
 *   not a permutation, rows not hit keep their previous contents, and two entries naming the same row
 *   race (which of the two values remains is unspecified). out, dq, dk, dv must not overlap the inputs.
 * bf16 and float32, as fm_fwd / fm_bwd. Errors: as fm_fwd / fm_bwd; FM_ERR_INVALID for a NULL map. */
fm_status fm_fwd_mapped(const void* q, const void* k, const void* v, fm_dtype dtype, int B, int H, int N, int d,
                        const int32_t* lts, const int32_t* lte, const int32_t* uts, const int32_t* ute, int Hm,
                        const int32_t* bounds, const int32_t* sched, int causal, float scale, const int32_t* omap,
                        void* out, float* lse, hipStream_t stream);
fm_status fm_bwd_mapped(const void* q, const void* k, const void* v, const void* out, const void* dout,
                        const float* lse, fm_dtype dtype, int B, int H, int N, int d, const int32_t* lts,
                        const int32_t* lte, const int32_t* uts, const int32_t* ute, int Hm, const int32_t* bounds,
                        const int32_t* sched, int causal, float scale, const int32_t* qmap, const int32_t* kmap,
                        void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Test hook: the tile classifier the kernels use, materialised. For each (b, hm, query tile of
 * qblock rows, key tile of kblock columns), clipped to N, writes classes[b][hm][qt][kt]:
 *   2 FULL    the causal triangle or one interval covers every (row, column) of the tile
 *   0 NONE    not FULL, and neither the causal triangle nor either interval reaches any row of it
 *   1 PARTIAL otherwise.
 * With bounds read as (mnLTS, mxLTS, mnLTE, mxLTE, mnUTS, mxUTS, mnUTE, mxUTE) and rows [r0, r1),
 * columns [c0, c1): causal FULL iff r1-1 < c0, causal NONE iff !causal or r0 >= c1-1;
 * interval FULL iff r0 >= mxS and r1 <= mnE; interval NONE iff r1 <= mnS or r0 >= mxE.
 * classes is uint8 [B, Hm, ceil(N/qblock), ceil(N/kblock)].
 * Errors: FM_ERR_INVALID (NULL pointers, sizes, qblock <= 0), FM_ERR_LAUNCH. */
fm_status fm_tile_classes(const int32_t* bounds, int B, int Hm, int N, int causal, int qblock,
                          uint8_t* classes, hipStream_t stream);

/* Static description of a status code (never NULL). */
const char* fm_status_str(fm_status s);

#ifdef __cplusplus
}
#endif
#endif /* FM_H */
