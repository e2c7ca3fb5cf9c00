/*
 * moe.h -- C ABI of libmoe.so: the one-rank hot path of a dynamic
 * redundant-expert MoE layer on AMD MI355X (gfx950).
 *
 * Pages cited by title and section:
 *   [ainovat]  "Moonshot AI Open-Sources MoonEP: A Perfectly Balanced Expert
 *              Parallelism Library for MoE Training" (ainovat.com)
 *   [repocard] "MoonEP" repository card (findrepo.work)
 *   [blog]     "MoonEP" code walkthrough (moses-y.github.io)
 *
 * The path, per MoE layer step on rank r:
 *   moe_plan              router outputs of all R ranks -> counts + replica plan
 *   moe_dispatch_layout   plan -> cu_seqlens[E+B+1], dest_pos, src_flat of rank r
 *   moe_prefetch          slot weight rows <- the experts they duplicate
 *   moe_permute           token rows -> expert-grouped rows (bitwise gather)
 *   moe_group_gemm        grouped GEMM over one [E+B, Kd, N] weight tensor
 *   moe_group_gemm_gather the same, its row operand gathered from the token
 *                         rows as it is loaded (permute fused into the GEMM)
 *   moe_combine           router-weighted sum of each token's K expert rows
 *   backward: moe_permute (weighted), moe_group_gemm DGRAD/WGRAD,
 *             moe_replica_grad_fold
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is DEVICE memory owned by the caller, except
 *     `dims` (host).  The library allocates nothing; its only state is a
 *     per-device cache of device properties and the static per-GPU scratch of
 *     moe_plan_noalloc.  Calls only enqueue work on `stream` (0 = the null
 *     stream) and never synchronise with the host.
 *   - Host-side argument checks run before anything is enqueued and return
 *     MOE_EINVAL / MOE_ENOSPACE with nothing launched.  MOE_EHIP reports a
 *     failed kernel launch.  Call moe_status_string() for a message.
 *   - Problems only the device can see (an expert id out of range, more
 *     replicas than slots) are reported in the plan's status word and in
 *     *dev_status; outputs downstream of such a plan are then unspecified
 *     but every access stays inside the buffers described here.
 *   - Results are deterministic: no floating-point atomics, fixed
 *     reduction order.
 *   - Copy ids: copy (p, s, k) of token s of rank p, k-th routed expert,
 *     has id c = (p*S + s)*K + k.  All index arrays are int32, row-major.
 *   - Shape limits: 1 <= R <= 512, E % R == 0, 1 <= E <= 1024, 1 <= K <= E,
 *     S >= 1, 0 <= B <= 64, R*S*K < 2^31.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t R; /* ranks (the executed rank's peers are simulated)          */
  int32_t S; /* tokens per rank                                          */
  int32_t K; /* routed experts per token (top-K)                         */
  int32_t E; /* routed experts; expert e lives on rank e / (E/R)          */
  int32_t B; /* replica (prefetch) slots per rank: weight rows E..E+B-1   */
} moe_dims;

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,   /* bad pointer, shape, dtype or op                     */
  MOE_ENOSPACE = 2, /* workspace smaller than the *_workspace_bytes query, or
                       a no-allocation call needing more than its static
                       scratch                                              */
  MOE_EHIP = 3      /* a HIP launch failed                                  */
} moe_status_t;

/* Bits of the plan status word (plan[0]) and of *dev_status. */
enum {
  MOE_DEV_BAD_EXPERT_ID = 1u, /* some topk_idx value was outside [0, E)       */
  MOE_DEV_SLOT_OVERFLOW = 2u  /* some rank needed more than B replicas         */
};

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef enum {
  MOE_GEMM_FWD = 0,   /* out[seg] = a[seg] @ W[rho]                          */
  MOE_GEMM_DGRAD = 1, /* out[seg] = a[seg] @ W[rho]^T                        */
  MOE_GEMM_WGRAD = 2  /* out[rho] += a[seg]^T @ b[seg]   (fp32 out)          */
} moe_gemm_op;

const char *moe_status_string(moe_status_t s);

/* ---------------------------------------------------------------------------
 * moe_plan -- online redundant-expert plan from this step's router outputs.
 * [ainovat] paragraphs on the skew metric, the exact S*K-per-rank invariant
 * and the mechanism (a few redundant experts planned online, directly from
 * the router outputs); [repocard] "Strengths" (negligible planning cost).
 *
 * Counts C[p][e] of copies routed to each expert, then a greedy placement:
 * rank loads L_r = sum of T_e over its home experts, excess d_r = L_r - S*K;
 * donors (d_r > 0) by (d_r desc, r asc) cut one piece from each of their
 * experts taken by (T_e desc, e asc) until the excess is gone; the pieces
 * are dealt out, in order, to receivers (d_r < 0) ordered by (-d_r desc,
 * r asc), each replica carrying min(piece left, deficit left) copies; a
 * receiver's replicas take slots 0, 1, ... in order.  When some receiver
 * would need more than B slots, a relay fallback re-places the walk's
 * replicas in order: a full receiver instead takes more copies of an expert
 * it already hosts while that expert's home (a donor) takes the piece, or one
 * of its replicas switches to the new expert while the new expert's home
 * takes the switched-out copies (first fit over the receiver's slots; a
 * "place" goes to the home's keep, an existing replica, or a free slot).
 * If it cannot place a replica and B >= 1, a bounded search looks for a plan
 * with at most one replica per rank: the receivers, by (deficit desc, r asc),
 * each take their whole deficit from one expert of a rank that takes no
 * copies (homes by (d desc, r asc), experts by (T desc, e asc); homes with
 * that much excess left first, then the others); a home that so sends out
 * more than its excess takes the difference the same way, in the next
 * generation; depth first, at most 512 placements.  If it finds none, the
 * relay fallback's plan stands and each replica it could not place is dropped
 * with MOE_DEV_SLOT_OVERFLOW.  The list is then gathered by expert (experts
 * by first entry, entries in pass order) and each expert's copies are tiled
 * home first, then its entries.  Plans the walk fits are the walk's.
 * Afterwards every rank processes exactly S*K copies (absent overflow and bad
 * ids).  The relay fallback is one thread's loop and the search one
 * wavefront's (64 candidates tested at a time); both run only on overflow.  A
 * search that spends its budget adds a few milliseconds to the plan (2.2 ms at
 * R=32 E=256, 3.4 ms at R=512 E=1024 on MI355X).
 *
 *   topk_idx   [R*S*K] int32, router top-K expert ids of every rank.
 *   counts     [R*E] int32 out, C[p][e] (ids outside [0,E) not counted).
 *   plan       [moe_plan_words(dims)] int32 out:
 *                [0] status bits  [1] replicas in the list  [2] most
 *                replicas the walk asked of one rank  [3] donors
 *                [4] receivers  [5] pieces  [6] replicas relayed or
 *                switched by the fallback  [7] placements tried by
 *                the bounded search (0: it did not run)
 *                T[E]  keep[E] (copies of e staying home)
 *                rep_first[E] rep_n[E] (e's replicas in the list; 0,0 if none)
 *                replica list, E+R entries each of expert[] rank[] slot[]
 *                  start[] count[], an expert's entries together; the replica takes the
 *                  copies of its expert at positions [start, start+count) of
 *                  that expert's copy-id order; unused entries -1,-1,-1,0,0;
 *                  slot -1 = dropped
 *                slot tables [R*B] each of expert[] start[] count[]
 *                  (empty slot: -1, 0, 0)
 *   dev_status nullable; when given, *dev_status = plan status bits.
 *   ws         >= moe_plan_workspace_bytes(dims) bytes of scratch.
 * ------------------------------------------------------------------------- */
size_t moe_plan_words(const moe_dims *dims);
size_t moe_plan_workspace_bytes(const moe_dims *dims);
moe_status_t moe_plan(const moe_dims *dims, const int32_t *topk_idx, int32_t *counts,
                      int32_t *plan, uint32_t *dev_status, void *ws, size_t ws_bytes,
                      hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_plan_noalloc -- moe_plan with no workspace argument and no allocation,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments (minus ws, ws_bytes), same outputs, bit for bit, as
 * moe_plan.  The scratch moe_plan takes from `ws` lives instead in one static
 * device array of MOE_PLAN_NOALLOC_SCRATCH_BYTES per GPU, which the library
 * holds from its load until the process ends.  Its device address is looked
 * up once per device, on the first call with that device current (MOE_EHIP if
 * the lookup fails).  Returns MOE_ENOSPACE, with nothing launched, when
 * moe_plan_workspace_bytes(dims) exceeds that size (e.g. R=64, S=8192, K=8,
 * E=384 needs 1.6 MB; R=32, S=4096, K=8, E=256 needs 0.26 MB).  Every scratch
 * word is written before it is read, so no call needs it cleared.
 * Calls on one GPU share its one array: calls that can overlap on one GPU
 * (on different streams, or from several host threads) race and give
 * unspecified plans; calls on one stream are ordered and do not.
 * ------------------------------------------------------------------------- */
#define MOE_PLAN_NOALLOC_SCRATCH_BYTES (4u << 20)
moe_status_t moe_plan_noalloc(const moe_dims *dims, const int32_t *topk_idx, int32_t *counts,
                              int32_t *plan, uint32_t *dev_status, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_dispatch_layout -- turn the plan into rank `rank`'s cu_seqlens and the
 * token-to-row maps.  [ainovat] contract paragraph (dispatch returns a
 * cu_seqlens over the E+B weight rows that selects the active rows);
 * [blog] "What This Does" (tokens go straight to their final
 * expert-grouped position).
 *
 * Row layout of rank q's buffer: segments in ascending weight row rho
 * (home experts at their global id, slot j at row E+j); inside expert e the
 * copies keep copy-id order; the first keep[e] stay home, replica m takes
 * positions [start_m, start_m + count_m).
 *
 *   cu_seqlens [E+B+1] int32 out, leading 0, cu_seqlens[E+B] = S*K.
 *   dest_pos   [R*S*K] int32 out, q*S*K + row on rank q of every copy, or
 *              -1 when the copy has no destination (bad id, dropped replica).
 *   src_flat   [S*K] int32 out, copy id filling each row of rank `rank`,
 *              -1 for rows past cu_seqlens[E+B].
 *   ws         >= moe_dispatch_layout_workspace_bytes(dims) bytes.
 * ------------------------------------------------------------------------- */
size_t moe_dispatch_layout_workspace_bytes(const moe_dims *dims);
moe_status_t moe_dispatch_layout(const moe_dims *dims, int32_t rank, const int32_t *topk_idx,
                                 const int32_t *plan, int32_t *cu_seqlens, int32_t *dest_pos,
                                 int32_t *src_flat, void *ws, size_t ws_bytes,
                                 hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_prefetch -- copy each used slot row of rank `rank` from the expert it
 * duplicates: w[E+j] = w[slot_expert[rank][j]].  [ainovat] mechanism
 * paragraph (duplicated experts are fetched before expert compute).  On one
 * GPU this is a device row copy; empty slots are left untouched.
 *   w          [E+B, row_bytes] bytes, row_bytes % 16 == 0.
 * ------------------------------------------------------------------------- */
moe_status_t moe_prefetch(const moe_dims *dims, int32_t rank, const int32_t *plan, void *w,
                          int64_t row_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_permute -- xp[i] = x_all[src_flat[i] / K], the gather into
 * expert-grouped order ([blog] "What This Does"; [repocard] "Strengths":
 * permute fused into dispatch).  Bitwise copy; rows with src_flat < 0 are
 * zero.  With row_scale (indexed by copy id, [R*S*K] fp32) each row is
 * multiplied by row_scale[src] in fp32 and rounded once (RNE) to the row
 * type: the backward of moe_combine.
 *   x_all [R*S, width], xp [S*K, width], width*elem % 16 == 0.
 * ------------------------------------------------------------------------- */
moe_status_t moe_permute(const moe_dims *dims, moe_dtype dtype, int64_t width,
                         const void *x_all, const int32_t *src_flat, const float *row_scale,
                         void *xp, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_group_gemm -- grouped GEMM over one contiguous weight tensor whose
 * groups are addressed purely by row index.  [ainovat] contract and
 * contiguity paragraphs.  Segment rho covers rows cu_seqlens[rho] ..
 * cu_seqlens[rho+1] of the row operands; empty segments are skipped; rows
 * outside every segment are not written.  bf16 runs on MFMA with fp32
 * accumulation and one RNE rounding; fp32 runs on the vector ALUs.
 *
 *   FWD:   a [M_total, Kd], b = W [G, Kd, N]        -> out [M_total, N]
 *   DGRAD: a [M_total, N],  b = W [G, Kd, N]        -> out [M_total, Kd]
 *   WGRAD: a [M_total, Kd], b [M_total, N]          -> out fp32 [G, Kd, N], +=
 *   cu_seqlens [G+1] int32, non-decreasing, cu_seqlens[G] <= M_total.
 *   Kd % 8 == 0, N % 8 == 0, Kd <= 2^22, N <= 2^22; WGRAD: N <= 2^20 (else
 *   MOE_EINVAL).
 *   ws: optional device scratch (NULL: none) of at least
 *   moe_group_gemm_workspace_bytes(op, dtype) bytes, else MOE_ENOSPACE.  With
 *   it, bf16 FWD and DGRAD may split the contraction of the output tiles of
 *   the persistent grid's last, partial round over all workgroups and add the
 *   fp32 parts in a second kernel (same stream): the result is then rounded
 *   from a sum in a different order than without the workspace (deterministic
 *   for given inputs).  Calls that share one workspace must not overlap.
 * ------------------------------------------------------------------------- */
size_t moe_group_gemm_workspace_bytes(moe_gemm_op op, moe_dtype dtype);
moe_status_t moe_group_gemm(moe_gemm_op op, moe_dtype dtype, int32_t G, int32_t M_total,
                            int32_t Kd, int32_t N, const void *a, const void *b,
                            const int32_t *cu_seqlens, void *out, void *ws, size_t ws_bytes,
                            hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_group_gemm_gather -- moe_group_gemm whose row operand is gathered from
 * the token rows while the GEMM loads it, so the tokens reach their
 * expert-grouped GEMM rows with no permute pass: the dispatch's permute fused
 * into the expert GEMM.  [blog] "What This Does" (tokens go straight to their
 * final expert-grouped position); [repocard] "Strengths" (permute fused into
 * dispatch, zero copy).
 *
 * Row m of the operand A is token row x_src[gather[m] / gather_div].  With
 * gather = src_flat of moe_dispatch_layout and gather_div = K, A is the xp
 * that moe_permute writes, and the result is that of moe_permute followed by
 * moe_group_gemm, bit for bit (same products, same summation order):
 *   FWD:   out [M_total, N] = A[seg] @ W[rho],   b = W [G, Kd, N] (the up
 *          projection's forward);
 *   WGRAD: out fp32 [G, Kd, N] += A[seg]^T @ b[seg],   b [M_total, N] (the up
 *          projection's weight gradient, b = its output gradient).
 *   x_src  [src_rows, Kd] bf16, rows of Kd elements; it may be larger than
 *          4 GB (the gathered loads take 64-bit addresses).  1 <= src_rows < 2^31.
 *   gather [M_total] int32, gather_div >= 1.  An entry outside
 *          [0, src_rows * gather_div) reads row 0 (FWD; that output row is then
 *          unspecified) or zeros (WGRAD); moe_dispatch_layout writes such entries
 *          (-1) only for rows past cu_seqlens[G], outside every segment.
 *   G, M_total, Kd, N, cu_seqlens, out, ws: as moe_group_gemm (FWD may split
 *   its last round with the workspace).  bf16 only; DGRAD (whose row operand is
 *   an output gradient, already in expert-grouped order) is MOE_EINVAL.
 * ------------------------------------------------------------------------- */
moe_status_t moe_group_gemm_gather(moe_gemm_op op, moe_dtype dtype, int32_t G, int32_t M_total,
                                   int32_t Kd, int32_t N, const void *x_src, int64_t src_rows,
                                   const int32_t *gather, int32_t gather_div, const void *b,
                                   const int32_t *cu_seqlens, void *out, void *ws,
                                   size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_group_gemm_swiglu -- the FWD grouped GEMM with a gated (SwiGLU) epilogue:
 * h = a @ W[rho] per segment as in moe_group_gemm(FWD), W's N columns taken as
 * (gate, up) pairs (column 2j is gate j, 2j+1 is up j), and
 * z[:, j] = silu(h[:, 2j]) * h[:, 2j+1], silu(x) = x / (1 + exp(-x)), computed in
 * fp32 from the fp32 accumulators and rounded once (RNE).  The pages name no
 * activation ([ainovat] contract names only the two projections); the gated
 * unit is the usual framework variant and the interleaved pairs keep it local
 * to the accumulators.  bf16 only.
 *   a [M_total, Kd], b = W [G, Kd, N] (N % 16 == 0), cu_seqlens as in
 *   moe_group_gemm, z [M_total, N/2] bf16, h [M_total, N] bf16 or NULL (the
 *   pre-activation, rounded once, kept for moe_swiglu_backward).  ws, ws_bytes
 *   as for moe_group_gemm(FWD).
 * ------------------------------------------------------------------------- */
moe_status_t moe_group_gemm_swiglu(moe_dtype dtype, int32_t G, int32_t M_total, int32_t Kd,
                                   int32_t N, const void *a, const void *b,
                                   const int32_t *cu_seqlens, void *z, void *h, void *ws,
                                   size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_swiglu_backward -- gradient of the gated unit with respect to its
 * pre-activation, elementwise over pairs: with (g, u) = (h[:, 2j], h[:, 2j+1])
 * and d = dz[:, j], dh[:, 2j] = d * u * silu'(g) and dh[:, 2j+1] = d * silu(g),
 * silu'(x) = s(x) (1 + x (1 - s(x))), s the logistic function; fp32, one RNE.
 *   h [rows, 2 n_pairs], dz [rows, n_pairs], dh [rows, 2 n_pairs], all of the
 *   given dtype, row-major without padding; n_pairs * elem % 16 == 0.
 * ------------------------------------------------------------------------- */
moe_status_t moe_swiglu_backward(moe_dtype dtype, int64_t rows, int64_t n_pairs, const void *h,
                                 const void *dz, void *dh, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_combine -- out[s] = sum_k topk_w[c] * y_all[dest_pos[c]], c = copy
 * (rank, s, k), fp32 accumulation in ascending k, one RNE rounding; copies
 * with dest_pos < 0 add nothing.  [blog] "What This Does" / "Real-World
 * Use" (combine gathers expert outputs back to the tokens).
 *   y_all [R*S*K, width] (rank q's expert outputs at rows q*S*K ..),
 *   topk_w [R*S*K] fp32, out [S, width], width*elem % 16 == 0.
 * ------------------------------------------------------------------------- */
moe_status_t moe_combine(const moe_dims *dims, moe_dtype dtype, int64_t width, int32_t rank,
                         const void *y_all, const int32_t *dest_pos, const float *topk_w,
                         void *out, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_unpermute_reduce -- dx[s] = sum_k dxp_all[dest_pos[c]], c = copy (rank,
 * s, k): the backward of the dispatch, which copied each token row to K
 * expert-grouped rows, so a token's input gradient is the sum of its copies'
 * gradients.  fp32 accumulation in ascending k, one RNE rounding to the row
 * type; copies with dest_pos < 0 add nothing.  [blog] "What This Does"
 * (dispatch places a token's K copies) and "Real-World Use" (the training
 * loop runs backward through the same path).
 *   dxp_all [R*S*K, width] (rank q's input-gradient rows at q*S*K ..,
 *   the layout's order), dest_pos from moe_dispatch_layout, dx [S, width],
 *   width*elem % 16 == 0.
 * ------------------------------------------------------------------------- */
moe_status_t moe_unpermute_reduce(const moe_dims *dims, moe_dtype dtype, int64_t width,
                                  int32_t rank, const void *dxp_all, const int32_t *dest_pos,
                                  void *dx, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_combine_weight_grad -- dw[s*K + k] = sum_h dout[s, h] * y_all[dest_pos[c], h],
 * c = copy (rank, s, k): the gradient of moe_combine with respect to rank
 * `rank`'s router weights (the combine is linear in each weight).  Products
 * and sums in fp32: each thread sums its 16-byte vectors of the row in row
 * order, then a fixed-order reduction over the block, so the result is
 * deterministic; 0 for copies with dest_pos < 0.  [blog] "Real-World Use".
 *   y_all [R*S*K, width] as in moe_combine, dout [S, width] (this rank's
 *   output-gradient rows), dw [S*K] fp32, width*elem % 16 == 0.
 * ------------------------------------------------------------------------- */
moe_status_t moe_combine_weight_grad(const moe_dims *dims, moe_dtype dtype, int64_t width,
                                     int32_t rank, const void *y_all, const int32_t *dest_pos,
                                     const void *dout, float *dw, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_replica_grad_fold -- fold rank `rank`'s replica weight-gradient rows
 * into their home expert rows: for each used slot j holding expert e,
 * dw[e] += dw[E+j] (fp32), then dw[E+j] = 0.  [ainovat] mechanism paragraph
 * and [blog] "Real-World Use" (replica gradients go back to their home).
 *   dw [E+B, row_elems] fp32, row_elems % 4 == 0.
 * ------------------------------------------------------------------------- */
moe_status_t moe_replica_grad_fold(const moe_dims *dims, int32_t rank, const int32_t *plan,
                                   float *dw, int64_t row_elems, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
