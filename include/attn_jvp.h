/*
 * attn_jvp.h -- fused attention forward-mode derivative (JVP) on AMD gfx950.
 *
 * One online-softmax pass computes, per batch b, head h and query row i,
 *
 *   S    = s * Q K^T                       (scores, s = scale)
 *   dS   = s * (dQ K^T + Q dK^T)           (score tangent)
 *   P    = softmax_row(S)                  (masked keys get S = -inf, dS = 0)
 *   O    = P V
 *   LSE  = log sum_j exp(S_ij)             (natural log)
 *   dLSE = sum_j P_ij dS_ij                (tangent of LSE)
 *   dO   = P dV + (P (.) dS) V - dLSE (.) O
 *
 * Definitions: page "带分数正则的一致性蒸馏" (gitcode.csdn.net), section
 * 注意力 -- the attention formula (普通注意力的实现), the chain rule
 * t_o = P t_v + t_p V with t_p = P (.) t_s - (P t_s^T) P and
 * t_s = t_q K^T + Q t_k^T, the streaming form with extra state r, A, B, and the
 * 前向 kernel's op contract (shape rules, tangents sharing the primals'
 * strides, default scale d^-1/2, outputs allocated by the caller, O and dO in
 * the input dtype, LSE in float32).  dLSE is the derivative of the stored
 * log-sum-exp; the pages' kernel computes it (r / l) but does not store it.
 * The optional frame-window mask follows the page "VDN-Minimax-H3 ... Stage
 * A1" (yfxerp.com): chunked window of `chunk_frames` frames, `radius_chunks`
 * chunks on each side, first/last frames as always-visible anchor keys.
 *
 * Conventions shared by every entry point:
 *   - Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE (and split partials and
 *     workspaces) are DEVICE pointers owned by the caller; the library
 *     allocates and frees no device memory.
 *   - Shapes follow the pages' op contract: Q, dQ are [B, H, Lq, d_qk];
 *     K, dK are [B, H, Lkv, d_qk]; V, dV are [B, H, Lkv, d_v]; O, dO are
 *     [B, H, Lq, d_v]; LSE, dLSE are [B, H, Lq].  The square entry points
 *     (attn_jvp_fwd, attn_jvp_fwd_strided) take Lq = Lkv = N and
 *     d_qk = d_v = d.  Built head dims: d_qk, d_v in {16, 32, 64, 128, 256}
 *     for bfloat16 and {16, 32, 64} for float32 (others: EUNSUPPORTED).
 *   - The last (d) dimension must be contiguous; the other strides are
 *     given in ELEMENTS.  Tangents must use exactly the strides of their
 *     primal (dQ of Q, dK of K, dV of V, dO of O), as the pages require.
 *   - Every row start must be 16-byte aligned: base pointers aligned to 16
 *     bytes and strides multiples of 8 elements (bf16) or 4 (float32).
 *   - LSE and dLSE are float32, contiguous [B, H, Lq].
 *   - O, dO, LSE, dLSE must not alias any input.
 *   - The call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  Arguments are validated on the host before anything is
 *     launched; on error nothing is launched and a negative status returns.
 *   - No C++ exception crosses this interface.  Apart from the static
 *     scratch address of the allocation-free entry point, cached per device
 *     on first use, the library keeps no state between calls, and it is
 *     safe to call from several host threads.
 *   - Calls that run concurrently on one device race only if their outputs
 *     overlap.
 */
#ifndef ATTN_JVP_H
#define ATTN_JVP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of Q, K, V, dQ, dK, dV, O and dO.  Accumulation is float32. */
typedef enum {
  ATTN_JVP_BF16 = 0, /* bfloat16 in and out; P and P (.) dS rounded to bf16
                        (round to nearest even) before the value products */
  ATTN_JVP_FP32 = 1  /* float32 throughout */
} attn_jvp_dtype;

typedef enum {
  ATTN_JVP_OK = 0,
  ATTN_JVP_EINVAL = -1,      /* null pointer, non-positive size, bad dtype  */
  ATTN_JVP_EUNSUPPORTED = -2,/* head dims not built for the dtype, or a
                                frame-window mask with d_qk != d_v          */
  ATTN_JVP_ESTRIDE = -3,     /* tangent strides differ from the primal's, a
                                misaligned pointer or stride, or overlap    */
  ATTN_JVP_EMASK = -4,       /* inconsistent mask descriptor                */
  ATTN_JVP_EHIP = -5,        /* the HIP runtime reported an error at launch */
  ATTN_JVP_ENOSCRATCH = -6   /* the call's split partials exceed the static
                                scratch of attn_jvp_fwd_splitkv_noalloc     */
} attn_jvp_status;

enum { ATTN_JVP_MASK_NONE = 0, ATTN_JVP_MASK_FRAME_WINDOW = 1 };

/* Optional key mask; pass NULL (or kind = ATTN_JVP_MASK_NONE) for dense,
 * non-causal attention.  For ATTN_JVP_MASK_FRAME_WINDOW the N tokens are
 * frames * tokens_per_frame tokens flattened frame-major (token i is in frame
 * i / tokens_per_frame); chunks are runs of chunk_frames frames from frame 0.
 * Key j is visible to query i iff
 *     |chunk(frame(i)) - chunk(frame(j))| <= radius_chunks
 *  or (anchor_first && frame(j) == 0) or (anchor_last && frame(j) == frames-1)
 *  or (anchor_queries_see_all && frame(i) is an enabled anchor frame).
 * Self-attention only: requires Lq == Lkv == N, frames * tokens_per_frame
 * == N, chunk_frames >= 1, radius_chunks >= 0, otherwise ATTN_JVP_EMASK
 * (and d_qk == d_v, otherwise ATTN_JVP_EUNSUPPORTED).  Every query sees its
 * own frame, so no row is empty.  Tiles of keys that no query of a query block
 * can see are neither loaded nor computed. */
typedef struct {
  int32_t kind;
  int32_t frames;
  int32_t tokens_per_frame;
  int32_t chunk_frames;
  int32_t radius_chunks;
  int32_t anchor_first;
  int32_t anchor_last;
  int32_t anchor_queries_see_all;
} attn_jvp_mask;

/* Element strides (batch, head, row) of each tensor; the d stride is 1. */
typedef struct {
  int64_t q[3], k[3], v[3];
  int64_t dq[3], dk[3], dv[3];
  int64_t o[3], dout[3];
} attn_jvp_layout;

/* Sizes of one call (see the shape convention above). */
typedef struct {
  int32_t batch;       /* B */
  int32_t heads;       /* H */
  int32_t seqlen_q;    /* Lq: query rows */
  int32_t seqlen_kv;   /* Lkv: key / value rows */
  int32_t head_dim_qk; /* d_qk: head dim of Q, K, dQ, dK */
  int32_t head_dim_v;  /* d_v: head dim of V, dV, O, dO */
} attn_jvp_shape;

/* General entry point: Lq may differ from Lkv (cross-attention, or a key
 * range of a longer sequence) and d_qk from d_v.  `layout` NULL means every
 * tensor is contiguous in its own shape.  scale <= 0 selects 1/sqrt(d_qk).
 * Returns an attn_jvp_status; nothing is launched unless it is ATTN_JVP_OK. */
int attn_jvp_fwd_ex(const void *Q, const void *K, const void *V,
                    const void *dQ, const void *dK, const void *dV,
                    void *O, void *dO, float *LSE, float *dLSE,
                    const attn_jvp_shape *shape, float scale, int dtype,
                    const attn_jvp_layout *layout, const attn_jvp_mask *mask,
                    void *stream);

/* Host-only argument check of attn_jvp_fwd_ex (never touches the GPU). */
int attn_jvp_check_ex(const void *Q, const void *K, const void *V,
                      const void *dQ, const void *dK, const void *dV,
                      void *O, void *dO, float *LSE, float *dLSE,
                      const attn_jvp_shape *shape, int dtype,
                      const attn_jvp_layout *layout, const attn_jvp_mask *mask);

/* ---- Key splits -------------------------------------------------------
 * Attention over a union of disjoint key sets combines from per-set results:
 * with (O_k, dO_k, LSE_k, dLSE_k) of set k over the same query rows,
 *   LSE  = log sum_k exp(LSE_k),   w_k = exp(LSE_k - LSE),
 *   O    = sum_k w_k O_k,          dLSE = sum_k w_k dLSE_k,
 *   dO   = sum_k w_k (dO_k + (dLSE_k - dLSE) O_k).
 * (Derived from the definition above; the pages do not state it.)  This is
 * what lets one query block's keys be split over several workgroups, or a
 * long sequence's keys over several calls (ring-style context parallelism),
 * and it is why dLSE is an output.
 *
 * Float32 partials of key set k are laid out contiguous: O_parts and
 * dO_parts [num_parts, B, H, Lq, d_v], LSE_parts and dLSE_parts
 * [num_parts, B, H, Lq].  A row that sees no key of a set has LSE_k = -inf,
 * dLSE_k = 0 and O_k = dO_k = 0. */

/* attn_jvp_fwd_ex restricted to the keys it is given (pass K, dK, V, dV
 * already offset to a key range and Lkv = its length), writing float32
 * partials O, dO [B, H, Lq, d_v] and LSE, dLSE [B, H, Lq], contiguous (the
 * o / dout strides of `layout` are ignored).  No mask.  Returns a status. */
int attn_jvp_fwd_partial(const void *Q, const void *K, const void *V,
                         const void *dQ, const void *dK, const void *dV,
                         float *O, float *dO, float *LSE, float *dLSE,
                         const attn_jvp_shape *shape, float scale, int dtype,
                         const attn_jvp_layout *layout, void *stream);

/* Merge num_parts float32 partials (layout above) into O, dO (the dtype,
 * [B, H, Lq, d_v] with element strides o_strides[3] = (b, h, row), NULL =
 * contiguous; strides multiples of 4) and LSE, dLSE (float32, contiguous
 * [B, H, Lq]).  d_v must be a multiple of 4.  Outputs must not overlap the
 * partials.  Asynchronous on `stream`.  Returns a status. */
int attn_jvp_merge(int num_parts, const float *O_parts, const float *dO_parts,
                   const float *LSE_parts, const float *dLSE_parts,
                   void *O, void *dO, float *LSE, float *dLSE,
                   int B, int H, int Lq, int d_v, int dtype,
                   const int64_t *o_strides, void *stream);

/* Host-only: the key splits attn_jvp_fwd_splitkv uses for a call and the
 * device workspace it needs.  *num_splits: in, the requested count (0 =
 * choose: enough workgroups to fill the chip about twice, each split
 * keeping at least two key tiles, at most 64); out, the count used.
 * *workspace_bytes is 0 when one split is used.  Returns a status. */
int attn_jvp_splitkv_plan(const attn_jvp_shape *shape, int dtype,
                          const attn_jvp_mask *mask, int *num_splits,
                          size_t *workspace_bytes);

/* attn_jvp_fwd_ex with each query block's visited key tiles divided over
 * num_splits workgroups (0 = the plan's choice): the splits write float32
 * partials into `workspace` (device memory owned by the caller, 256-byte
 * aligned, at least the plan's workspace_bytes, not overlapping any tensor),
 * then a merge kernel writes O, dO, LSE, dLSE.  Both launches go to
 * `stream`; the workspace is free again once they complete.  With one
 * split this is attn_jvp_fwd_ex and the workspace is unused (may be NULL).
 * For few query blocks and long key sequences.  Returns a status. */
int attn_jvp_fwd_splitkv(const void *Q, const void *K, const void *V,
                         const void *dQ, const void *dK, const void *dV,
                         void *O, void *dO, float *LSE, float *dLSE,
                         const attn_jvp_shape *shape, float scale, int dtype,
                         const attn_jvp_layout *layout,
                         const attn_jvp_mask *mask, int num_splits,
                         void *workspace, size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * attn_jvp_fwd_splitkv with the float32 partials in a static device buffer of
 * the library instead of a caller workspace.  The caller still passes every
 * input and output.  Same arguments, rules and results as
 * attn_jvp_fwd_splitkv without workspace/workspace_bytes; no allocating call
 * is made.
 *  - The buffer holds ATTN_JVP_NOALLOC_SCRATCH_BYTES (64 MiB) on each GPU the
 *    library runs on, until the process ends.  A call whose plan needs more
 *    (attn_jvp_splitkv_plan's workspace_bytes) returns ATTN_JVP_ENOSCRATCH
 *    when num_splits is given; with num_splits = 0 the plan takes the most
 *    splits that fit (one split needs no buffer).
 *  - Every call on a GPU shares that GPU's buffer: calls that overlap in
 *    time on one GPU (two streams, or two host threads) race and give wrong
 *    results; serialise them.  The buffer keeps the last call's partials;
 *    nothing in it needs to start at zero (every split writes all its rows).
 *  - The stream must belong to the current device (else ATTN_JVP_EINVAL).
 *    The first call on a device looks up that device's buffer address once
 *    (hipGetSymbolAddress); make that first call outside graph capture.
 * Returns a status; nothing is launched unless it is ATTN_JVP_OK. */
#define ATTN_JVP_NOALLOC_SCRATCH_BYTES (64u << 20)
int attn_jvp_fwd_splitkv_noalloc(const void *Q, const void *K, const void *V,
                                 const void *dQ, const void *dK, const void *dV,
                                 void *O, void *dO, float *LSE, float *dLSE,
                                 const attn_jvp_shape *shape, float scale,
                                 int dtype, const attn_jvp_layout *layout,
                                 const attn_jvp_mask *mask, int num_splits,
                                 void *stream);

/* ---- Primal backward --------------------------------------------------
 * Gradients of a loss L through O = softmax(s Q K^T) V, from the row
 * log-sum-exp the forward stored (page "带分数正则的一致性蒸馏", section 注意力,
 * subsection 反向): with gO = dL/dO,
 *   P = exp(s Q K^T - LSE),   gV = P^T gO,   dP = gO V^T,
 *   D = rowsum(gO (.) O),     dS = P (.) (dP - D),
 *   gQ = s dS K,              gK = s dS^T Q.
 * The tangents play no part (they are not trained).  As on the pages, the
 * backward is built for d_qk == d_v only (otherwise ATTN_JVP_EUNSUPPORTED);
 * Lq may differ from Lkv.  An optional frame-window mask (the forward's
 * attn_jvp_mask, same rules: Lq == Lkv == frames * tokens_per_frame) gives
 * the gradients of the masked attention: P = 0 for every pair the window
 * hides (page "VDN-Minimax-H3 ... Stage A1"); pass the LSE and O of the
 * forward with the same mask. */

/* Element strides (batch, head, row) of the backward's tensors. */
typedef struct {
  int64_t q[3], k[3], v[3], o[3], go[3];   /* inputs */
  int64_t gq[3], gk[3], gv[3];             /* outputs */
} attn_jvp_bwd_layout;

/* gQ [B,H,Lq,d], gK, gV [B,H,Lkv,d] (the dtype) from Q, K, V, O, gO (the
 * dtype) and LSE (float32 [B,H,Lq], as the forward wrote it).  delta is a
 * caller-owned float32 [B,H,Lq] buffer that receives D = rowsum(gO (.) O).
 * `layout` NULL means every tensor contiguous in its shape; `mask` NULL (or
 * kind ATTN_JVP_MASK_NONE) means dense.  scale <= 0 selects 1/sqrt(d).  Two
 * launches on `stream` (dQ and D, then dK and dV); deterministic (no
 * atomics).  Outputs must not overlap inputs or each other.  Returns a
 * status (ATTN_JVP_EMASK for a mask the forward would reject); nothing is
 * launched unless it is ATTN_JVP_OK. */
int attn_jvp_bwd(const void *Q, const void *K, const void *V, const void *O,
                 const void *gO, const float *LSE, void *gQ, void *gK, void *gV,
                 float *delta, const attn_jvp_shape *shape, float scale, int dtype,
                 const attn_jvp_bwd_layout *layout, const attn_jvp_mask *mask,
                 void *stream);

/* Host-only argument check of attn_jvp_bwd (never touches the GPU). */
int attn_jvp_bwd_check(const void *Q, const void *K, const void *V, const void *O,
                       const void *gO, const float *LSE, void *gQ, void *gK,
                       void *gV, float *delta, const attn_jvp_shape *shape,
                       int dtype, const attn_jvp_bwd_layout *layout,
                       const attn_jvp_mask *mask);

/* Contiguous [B, H, N, d] tensors.  scale <= 0 selects 1/sqrt(d).
 * Returns an attn_jvp_status. */
int attn_jvp_fwd(const void *Q, const void *K, const void *V,
                 const void *dQ, const void *dK, const void *dV,
                 void *O, void *dO, float *LSE, float *dLSE,
                 int B, int H, int N, int d, float scale, int dtype,
                 const attn_jvp_mask *mask, void *stream);

/* Same computation for strided views (e.g. a [B, N, H, d] buffer seen as
 * [B, H, N, d]); `layout` gives every tensor's strides and must not be NULL. */
int attn_jvp_fwd_strided(const void *Q, const void *K, const void *V,
                         const void *dQ, const void *dK, const void *dV,
                         void *O, void *dO, float *LSE, float *dLSE,
                         int B, int H, int N, int d, float scale, int dtype,
                         const attn_jvp_layout *layout,
                         const attn_jvp_mask *mask, void *stream);

/* Host-only argument check of attn_jvp_fwd_strided: the status that call
 * would return before launching (never touches the GPU; device pointers are
 * only inspected for NULL and alignment). */
int attn_jvp_check(const void *Q, const void *K, const void *V,
                   const void *dQ, const void *dK, const void *dV,
                   void *O, void *dO, float *LSE, float *dLSE,
                   int B, int H, int N, int d, int dtype,
                   const attn_jvp_layout *layout, const attn_jvp_mask *mask);

/* Host-only: the query-block rows (block_m) and key-tile length (block_n) the
 * library uses for (dtype, d_qk = d_v = d); returns a status.  This is the
 * geometry of every masked, key-split and partial launch, and of most
 * others (see attn_jvp_fwd_geometry). */
int attn_jvp_tile_shape(int dtype, int d, int *block_m, int *block_n);

/* The same for unequal head dims (dtype, d_qk, d_v). */
int attn_jvp_tile_shape_ex(int dtype, int d_qk, int d_v, int *block_m, int *block_n);

/* Host-only: the geometry (query-block rows, key-tile length) that
 * attn_jvp_fwd_ex launches for this call.  It is attn_jvp_tile_shape_ex's,
 * except for unmasked bfloat16 d_qk = d_v = 64 calls whose grid of 192-row
 * blocks would leave much of its last round of the chip idle: those take
 * 64-row blocks and 32-key tiles (three workgroups per compute unit).  The
 * choice depends on batch x heads and seqlen_q only.  Returns
 * ATTN_JVP_EINVAL for a NULL argument or a non-positive size,
 * ATTN_JVP_EUNSUPPORTED for head dims that are not built. */
int attn_jvp_fwd_geometry(const attn_jvp_shape *shape, int dtype, const attn_jvp_mask *mask,
                          int *block_m, int *block_n);

/* Host-only: the key tiles the scheduler visits for each query block of an
 * N-token sequence under `mask` (NULL = dense) with the tile shape of
 * (dtype, d).  Writes ceil(N / block_m) counts into tiles_per_block (host
 * memory, caller-owned) and returns a status.  This is the exact work list
 * the kernel walks. */
int attn_jvp_visible_tiles(int N, int dtype, int d, const attn_jvp_mask *mask,
                           int64_t *tiles_per_block);

/* Host-only: the streamed tiles the two backward launches walk under `mask`
 * (NULL = dense) for an N-token sequence whose owned rows are cut into blocks
 * of block_rows and whose streamed rows are cut into tiles of tile_rows:
 * keys == 0 gives, per query block, the key tiles of the dQ launch; keys != 0
 * gives, per key block, the query tiles of the dK/dV launch (a block holding
 * an anchor key is seen by every query).  Writes ceil(N / block_rows) counts
 * into tiles_per_block (host memory, caller-owned); returns a status.  With
 * the block and tile rows a launch uses, this is the exact work list it
 * walks. */
int attn_jvp_bwd_visible_tiles(int N, int block_rows, int tile_rows, int keys,
                               const attn_jvp_mask *mask, int64_t *tiles_per_block);

/* Static English text for a status code. */
const char *attn_jvp_status_string(int status);

/* Host-only: a static NUL-terminated hex string, the sha256 digest of the
 * sources and compiler flags this library was built from.  A loader compares
 * it with the digest of the sources beside it and refuses a stale build. */
const char *attn_jvp_build_id(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_JVP_H */
