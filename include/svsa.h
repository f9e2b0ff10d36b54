/*
 * svsa.h - C ABI of the MI355X (gfx950) block-sparse video attention library.
 *
 * The library computes training-free, input-adaptive block-sparse
 * self-attention over 3D video tokens in four stages, each a separate call:
 *
 *   1. svsa_tile_permute  reorder (T,H,W) tokens into contiguous tiles
 *   2. svsa_pool          mean-pool Q and K per block (block summaries)
 *      (svsa_tile_permute_pool does stages 1 and 2 for Q and K in one pass;
 *      svsa_attn_stage_v does stage 1 for V straight into stage 4's workspace)
 *   3. svsa_block_mask    softmax(Qbar Kbar^T * scale) per query block, keep the
 *                         top-p (or a fixed fraction of) key blocks plus a
 *                         diagonal band, emitted as CSR index lists
 *   4. svsa_block_sparse_attn
 *                         flash attention with online softmax over the kept
 *                         blocks only
 *
 * Sources (web pages, cited by title and section):
 *   [PSA]   "Parameterized Stripe Attention for Efficient Video Generation"
 *   [iCATS] "iCATS: Fast Video Generation via Interaction-Aware Sparse
 *           Attention and Timestep-Adaptive Sparsity"
 *   [SPADE] "SPADE: An Input-Adaptive Sparse Attention Engine for Fast Video
 *           Diffusion Models Inference"
 *   [SVOO]  "Attention Sparsity is Input-Stable: Training-Free Sparse
 *           Attention for Video Generation via Offline Sparsity Profiling and
 *           Online QK Co-Clustering"
 *
 * Conventions shared by every call
 *   - Tensor pointers are DEVICE pointers allocated and owned by the caller.
 *     The calls never allocate or free memory and keep no state between calls
 *     (the one exception: svsa_block_mask_noalloc's scratch array and the
 *     per-device address of it that the library looks up once).
 *   - Per-head parameter arrays (top_p, keep_frac) are HOST pointers, read
 *     during the call only.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call only enqueues work on it and returns without waiting.
 *   - Geometry: N = T*H*W tokens, Bk = tt*th*tw tokens per block,
 *     nb = ceil(N / Bk) blocks, N_pad = nb * Bk.  Tensors are
 *     [batch, heads, tokens, head_dim] row-major; natural token order is
 *     i = t*H*W + h*W + w ([PSA] App. D, Prop. 1).
 *   - Errors: argument errors are detected on the host before any work is
 *     enqueued and return a negative status; a failed launch returns
 *     SVSA_E_HIP.  No C++ exception crosses this interface.
 *   - Results are bitwise reproducible run to run (no floating-point atomics).
 */
#ifndef SVSA_H
#define SVSA_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define SVSA_API __attribute__((visibility("default")))
#else
#define SVSA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Latent grid (T,H,W), tile shape (tt,th,tw) (all >= 1) and block layout.
 * pad3d = 0: tiles walked row-major over the tile grid, tokens inside a tile
 *   row-major (t,h,w), edge tiles partial; the sequence is cut into
 *   consecutive blocks of Bk = tt*th*tw tokens, padding only at the tail:
 *   nb = ceil(N / Bk).
 * pad3d = 1: [PSA] App. C.2 ("3D-Padding"): one block per tile, nb = nT*nH*nW
 *   (tile grid ceil(T/tt) x ceil(H/th) x ceil(W/tw)); the tile's tokens fill
 *   the first slots of its block, the rest of the block is padding.
 * In both layouts every block's valid tokens are its first slots.
 */
typedef struct svsa_geom {
  int32_t T, H, W;
  int32_t tt, th, tw;
  int32_t pad3d;
} svsa_geom;

/*
 * Alignment (checked on the host, SVSA_E_INVALID otherwise): bf16 / f32 tensors
 * 16 bytes, float64 arrays 8, int32 arrays 4, workspaces 256 (every torch
 * allocation satisfies all of them).
 */
enum svsa_dtype { SVSA_BF16 = 0, SVSA_F32 = 1 };

enum svsa_status {
  SVSA_OK = 0,
  SVSA_E_INVALID = -1,     /* null pointer, non-positive size, bad value     */
  SVSA_E_UNSUPPORTED = -2, /* valid but not implemented (dtype, head_dim...) */
  SVSA_E_WORKSPACE = -3,   /* workspace smaller than the *_workspace_bytes   */
  SVSA_E_CAPACITY = -4,    /* col_idx capacity below the worst case          */
  SVSA_E_HIP = -5          /* a HIP launch failed                            */
};

/*
 * Stage 1 - tile reorder.  [PSA] Sec. 3.2 "Efficient and Flexible Kernel":
 * Q, K, V move from the (T,H,W) layout to a block-centric arrangement so that
 * every block is contiguous in memory.  [SVOO] lists a forward / inverse pair
 * of token reorders ("..._to_frame_major" / "..._to_token_major").
 *
 * Tile order: tiles are walked row-major over the tile grid
 * (ceil(T/tt), ceil(H/th), ceil(W/tw)), tokens inside a tile row-major in
 * (t,h,w); tiles at the grid edge are partial and keep their place.
 *
 *   inverse == 0: src [batch,heads,N,D] natural  -> dst [batch,heads,N_pad,D]
 *                 tiled; rows N..N_pad-1 of dst are written with zeros.
 *   inverse != 0: src [batch,heads,N_pad,D] tiled -> dst [batch,heads,N,D]
 *                 natural; the padded rows of src are not read.
 * dtype: SVSA_BF16 or SVSA_F32 (bit-exact copy either way).  head_dim * element
 * size must be a multiple of 16 bytes.  src and dst must not overlap.
 * Tile volume must be < 65536.
 */
SVSA_API int svsa_tile_permute(const void* src, void* dst, int32_t dtype, int32_t batch,
                      int32_t heads, int32_t head_dim, const svsa_geom* g,
                      int32_t inverse, void* stream);

/*
 * Stage 2 - block summaries.  [SPADE] abstract: dynamic masks are expressed
 * through a Summarizer and an Estimator; the summary used here is the mean of
 * a block's valid tokens (the tail block has n = N - (nb-1)*Bk of them).
 *
 * x_tiled: [batch,heads,N_pad,D] tiled (output of svsa_tile_permute), dtype
 * SVSA_BF16 or SVSA_F32.  out: float64 [batch,heads,nb,D];
 * out[i] = (sum of the valid rows of block i, accumulated in float64) / n_i.
 */
SVSA_API int svsa_pool(const void* x_tiled, int32_t dtype, double* out, int32_t batch,
              int32_t heads, int32_t head_dim, const svsa_geom* g, void* stream);

/*
 * Stages 1 and 2 in one pass, for Q and K: dst <- the forward tile reorder of
 * src (exactly what svsa_tile_permute with inverse == 0 writes, padding rows
 * zeroed) and means <- the block means of dst (exactly what svsa_pool writes
 * for it), without reading dst back.  [PSA] Sec. 3.2 (the reorder) and
 * [SPADE] abstract (the block summary) define the two results.
 *
 * src: [batch,heads,N,D] natural; dst: [batch,heads,N_pad,D] tiled; both of
 * dtype SVSA_BF16 or SVSA_F32.  means: float64 [batch,heads,nb,D].  The head
 * dimension limits of svsa_pool apply.  src, dst and means must not overlap.
 */
SVSA_API int svsa_tile_permute_pool(const void* src, void* dst, double* means, int32_t dtype,
                                    int32_t batch, int32_t heads, int32_t head_dim,
                                    const svsa_geom* g, void* stream);

/*
 * Workspace (device bytes) needed by svsa_block_mask for these sizes.
 * Returns 0 if the sizes are invalid.
 */
SVSA_API size_t svsa_block_mask_workspace_bytes(int32_t batch, int32_t heads, int32_t nb);

/*
 * Stage 3 - block mask.  Block-to-block importance is the row softmax of
 * L_ij = softmax_scale * <qbar_i, kbar_j> over all nb key blocks ([SPADE]
 * Estimator; [iCATS] Sec. 4, cluster-level scores).  Per (batch, head, query
 * block i) the kept set is
 *   top-p mode  (top_p != NULL): the shortest prefix of the key blocks sorted
 *               by score descending (ties: lower index first) whose summed
 *               score reaches top_p[h] (>=); top_p[h] == 1 keeps every block
 *               ([iCATS] abstract and Sec. 3.2, the fixed top-p rule);
 *   fixed mode  (keep_frac != NULL): the ceil(keep_frac[h] * nb) best blocks in
 *               the same order ([SVOO] abstract, per-layer pruning levels);
 * united with the diagonal band |i - j| <= band_width - 1 (the width convention
 * of [PSA] Alg. 1).  The band is added after selection and does not count
 * toward the mass.  All arithmetic of this stage is float64.
 *
 * qbar, kbar: float64 [batch,heads,nb,D] (svsa_pool outputs).
 * top_p, keep_frac: HOST float arrays [heads]; exactly one is non-NULL; every
 *   value must lie in (0, 1].
 * band_width >= 1.
 * row_ptr: int32 [batch*heads*nb + 1] (rows ordered (b, h, i)); col_idx: int32
 *   with col_capacity >= batch*heads*nb*nb entries (the worst case; the actual
 *   count is row_ptr[last]).  Each row's columns are ascending and unique.
 * workspace: device buffer of at least
 *   svsa_block_mask_workspace_bytes(batch, heads, nb) bytes.
 * Limits: nb <= 4096, heads <= 256, batch*heads*nb*nb < 2^31.
 */
SVSA_API int svsa_block_mask(const double* qbar, const double* kbar, int32_t batch,
                    int32_t heads, int32_t nb, int32_t head_dim,
                    double softmax_scale, const float* top_p,
                    const float* keep_frac, int32_t band_width,
                    int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                    void* workspace, size_t ws_bytes, void* stream);

/*
 * svsa_block_mask without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, rule, outputs and
 * checks as svsa_block_mask; it allocates and frees nothing.  Its scratch is
 * a fixed device array inside the library (80 MiB: 64 MiB for the float64
 * logits of a chunk of whole (batch, head) pairs, processed one chunk after
 * the other, and 16 MiB for the kept bitmaps and counts of all rows), which
 * every device the library runs on holds until the process ends.
 * Limits beyond svsa_block_mask's: nb * nb * 8 <= 64 MiB (nb <= 2896), and
 * batch*heads*nb * (4 * ceil(nb / 32) + 4) bytes (rounded up to 256 for the
 * bitmaps) <= 16 MiB; otherwise SVSA_E_WORKSPACE, before any launch.
 * Every call on a device uses that device's one array: calls that overlap in
 * time on one device (other streams, other host threads) race and must be
 * ordered by the caller.  The array keeps the last call's contents; every
 * call writes all of it that it reads.
 */
SVSA_API int svsa_block_mask_noalloc(const double* qbar, const double* kbar, int32_t batch,
                                     int32_t heads, int32_t nb, int32_t head_dim,
                                     double softmax_scale, const float* top_p,
                                     const float* keep_frac, int32_t band_width,
                                     int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                                     void* stream);

/*
 * Workspace (device bytes) needed by svsa_stripe_mask.  Returns 0 if the
 * sizes are invalid.
 */
SVSA_API size_t svsa_stripe_mask_workspace_bytes(int32_t batch, int32_t heads,
                                                 const svsa_geom* g);

/*
 * Stripe mask -> CSR.  [PSA] Sec. 3.2 "Unified Representation" and Alg. 1
 * "PSA Mask Definition": six integers M(Tw, To, Ts, Sw, So, Ss) per head;
 * position q attends to position k when
 *   ((|dt - To|) mod Ts) <= Tw - 1  and  ((|ds - So|) mod Ss) <= Sw - 1,
 * dt = t_k - t_q (frame distance), ds = s_k - s_q (in-frame distance); PSA
 * applies the mask per PSABlock.  Here positions are the tiles of the tile
 * grid (nT, nH, nW): t = tile t index, s = tile h index * nW + tile w index,
 * so the parameters are in tile units; a stride <= 0 means infinity (no
 * modulo).  Query block i keeps key block j when some tile of block i attends
 * to some tile of block j (blocks made of partial edge tiles hold several),
 * or |i - j| <= band_width - 1 (band_width 0: no band).
 *
 * params: HOST int32 [heads][6] (Tw, To, Ts, Sw, So, Ss); Tw, Sw >= 1, else
 *   SVSA_E_INVALID.  heads <= 128, nb <= 4096, tile volume <= 1024, else
 *   SVSA_E_UNSUPPORTED.
 * row_ptr / col_idx / col_capacity: as svsa_block_mask (rows (b, h, i),
 *   ascending columns, capacity >= batch*heads*nb*nb).
 * workspace: at least svsa_stripe_mask_workspace_bytes(batch, heads, g).
 * The CSR feeds svsa_block_sparse_attn unchanged.  Integer-only: the lists
 * are exact and deterministic.
 */
SVSA_API int svsa_stripe_mask(const svsa_geom* g, int32_t batch, int32_t heads,
                              const int32_t* params, int32_t band_width, int32_t* row_ptr,
                              int32_t* col_idx, int64_t col_capacity, void* workspace,
                              size_t ws_bytes, void* stream);

/*
 * Workspace (device bytes) needed by svsa_block_sparse_attn: the per-group
 * union lists (room for two words per key sub-block, as the step walk of
 * SVSA_ATTN_STEP_PAIRS needs) and work queues, plus a transposed copy of V
 * (sized for head_dim 128, so the figure does not depend on head_dim).
 * Returns 0 if the sizes are invalid.
 */
SVSA_API size_t svsa_attn_workspace_bytes(int32_t batch, int32_t heads, const svsa_geom* g);

/*
 * Stage 4 - block-sparse attention.  [PSA] App. B, Alg. 2: for each query
 * block, walk its KV-block list, S = Q K^T, invalid (padded) key positions set
 * to -inf, safe softmax, P V accumulated into the block's output; [SPADE]
 * "flash block-sparse attention".  Here the softmax is the online (running
 * max / running sum) form, so the result equals one softmax over all valid
 * keys of the kept blocks:
 *   out[q] = sum_t softmax_t(softmax_scale * <q, k_t>) v_t,
 *   t over the valid keys (index < N) of the blocks listed for q's block.
 *
 * q, k, v, out: bf16 [batch,heads,N_pad,D] in tile order.  Output rows of
 *   padding slots (positions >= N in the packed layout, a block's slots past
 *   its valid tokens in the 3D-padded one) are unspecified: they may be
 *   written with any value or left untouched.  out must not
 *   overlap q, k, v or the workspace.  A query block with an empty list gets
 *   zeros.  v may be NULL when svsa_attn_stage_v has written V into this
 *   workspace for the same batch, heads, head_dim and geometry, and nothing
 *   has written the workspace since (other svsa_block_sparse_attn calls with
 *   v == NULL leave it intact).
 * row_ptr / col_idx: CSR as produced by svsa_block_mask (rows (b,h,i); each
 *   column in [0, nb)).  Columns outside [0, nb) are ignored.
 * head_dim: 64 or 128; tile volume Bk: any multiple of 32 (blocks are run as
 *   consecutive sub-blocks of 64 tokens, or 32 when Bk is an odd multiple of
 *   32; a block's list applies to each of its sub-blocks); ceil(N / sub) <= 4096
 *   and N_pad * head_dim * 2 bytes per (b, h) below 2^31 (else
 *   SVSA_E_UNSUPPORTED).  Products are bf16 x bf16
 *   on the matrix cores with float32 accumulation; the softmax runs in
 *   float32.
 * Scheduling (no effect on what is computed): query blocks are processed in
 *   groups of four that stream the union of their lists.  With 64-token
 *   blocks (Bk = 64), nb <= 2048 and batch * heads * nb^2 * head_dim >= 2^32
 *   (work large enough to pay for the ~0.3 ms search) the groups are formed
 *   from each head's lists, per window of 256 consecutive blocks (a greedy
 *   choice of blocks whose lists overlap), so a key block's products are
 *   summed in another order than with positional groups: results agree with
 *   those to float32 rounding, not bitwise.  svsa_block_sparse_attn_ex can
 *   force either grouping.  Either way a call is bitwise reproducible.
 * workspace: at least svsa_attn_workspace_bytes(batch, heads, g) bytes.
 */
SVSA_API int svsa_block_sparse_attn(const void* q, const void* k, const void* v, void* out,
                           int32_t batch, int32_t heads, int32_t head_dim,
                           const svsa_geom* g, float softmax_scale,
                           const int32_t* row_ptr, const int32_t* col_idx,
                           void* workspace, size_t ws_bytes, void* stream);

/* Flags of svsa_block_sparse_attn_ex. */
enum {
  SVSA_ATTN_OUT_NATURAL = 1,
  SVSA_ATTN_POSITIONAL_GROUPS = 2,
  SVSA_ATTN_GROUPS_BY_LIST = 4,
  SVSA_ATTN_STEP_PAIRS = 8
};

/*
 * svsa_block_sparse_attn with flags.  flags = 0: the same call.
 * SVSA_ATTN_OUT_NATURAL: out is [batch,heads,N,D] in natural (t,h,w) order,
 * each valid query row written at its natural position (the inverse tile
 * reorder of [PSA] Sec. 3.2 done by the attention kernel's stores), so the
 * result equals svsa_tile_permute(inverse = 1) applied to the tile-order
 * output, bitwise.  SVSA_ATTN_POSITIONAL_GROUPS: query blocks grouped four
 * consecutive ones at a time, never by their lists; SVSA_ATTN_GROUPS_BY_LIST:
 * grouped by their lists whenever the blocks allow it (64-token blocks,
 * nb <= 2048), whatever the size of the work (see "Scheduling" above); both
 * together, or other bits: SVSA_E_INVALID.  SVSA_ATTN_STEP_PAIRS (blocks
 * that are whole 64-token sub-blocks, at most 4096 of them per head;
 * ignored otherwise): the four query blocks of a workgroup walk their union
 * list in steps of one or two key blocks, two when the sets of query blocks
 * keeping them are disjoint, each query block computing on the one it keeps
 * ([PSA] App. B, Alg. 2 per query block; the steps only change which
 * workgroup-wide interval a kept block is processed in).  It pays where
 * neighbouring query blocks keep different key blocks (fixed-fraction
 * masks) and costs a little where they keep mostly the same ones (top-p
 * masks), as its copy pipeline is one key block shallower. The same kept
 * pairs are computed, in another order: results agree to float32 rounding,
 * and a call is bitwise reproducible.  Everything else as above.
 */
SVSA_API int svsa_block_sparse_attn_ex(const void* q, const void* k, const void* v, void* out,
                                       int32_t batch, int32_t heads, int32_t head_dim,
                                       const svsa_geom* g, float softmax_scale,
                                       const int32_t* row_ptr, const int32_t* col_idx,
                                       int32_t flags, void* workspace, size_t ws_bytes,
                                       void* stream);

/*
 * Stage 1 for V fused with the layout change the attention kernel needs:
 * natural-order V ([batch,heads,N,D], bf16) is written into `workspace` as
 * the transposed key blocks svsa_block_sparse_attn reads, in tile order
 * ([PSA] Sec. 3.2), with zeros in padding slots.  The result is what
 * svsa_block_sparse_attn would build from svsa_tile_permute's tiled V, so a
 * following svsa_block_sparse_attn(..., v = NULL, ..., workspace) gives the
 * same output bitwise, and no tiled V has to be stored.
 *
 * head_dim, geometry and the workspace size: as for svsa_block_sparse_attn.
 * v must not overlap the workspace.
 */
SVSA_API int svsa_attn_stage_v(const void* v, int32_t batch, int32_t heads, int32_t head_dim,
                               const svsa_geom* g, void* workspace, size_t ws_bytes,
                               void* stream);

/* ------------------------------------------------------------------------
 * Variable-size blocks: query / key clustering ([iCATS] Sec. 3.1 and 4.1,
 * interaction-aware clustering; [SVOO] online bidirectional QK
 * co-clustering).  The pages describe the idea; this library's reading:
 * replacing a token x by a centroid c moves its logits against the other
 * side's tokens y by (x - c).y, with summed square (x - c)^T G (x - c),
 * G = sum_y y y^T, approximated from the other side's clusters as
 * G = sum_j n_j c_j c_j^T (svsa_cluster_metric).  Clustering is Lloyd's
 * k-means under that fixed metric (svsa_kmeans).  Clusters are then laid out
 * contiguously, each padded to a multiple of the block alignment
 * (svsa_cluster_layout, svsa_cluster_permute), scored and selected per
 * cluster pair (svsa_cluster_mask) and attended (svsa_cluster_attn).
 * ------------------------------------------------------------------------ */

/* Workspace (device bytes) for svsa_kmeans; 0 if the sizes are invalid. */
SVSA_API size_t svsa_kmeans_workspace_bytes(int32_t batch, int32_t heads, int32_t n,
                                            int32_t clusters, int32_t head_dim);

/*
 * `iters` Lloyd iterations per (batch, head).  Each iteration assigns every
 * token to the centroid c of least (x - c)^T G (x - c) (ties: lowest index)
 * and then moves every non-empty centroid to the mean of its members (an
 * empty cluster keeps its centroid).  On return `labels` is the last
 * assignment, `sizes` its cluster sizes and `centroids` the means of those
 * labels.  The distance comparison drops the common x^T G x term and is
 * evaluated as c^T G c - 2 x . (G c) with bf16 MFMA on x and on a two-term
 * bf16 split of G c (fp32 accumulation): choices between centroids whose
 * distances differ by less than about 1e-4 of |x| |G c| may differ from an
 * exact evaluation.  Means are float64 sums in token order.
 *
 * x: bf16 [batch, heads, n, head_dim] (natural token order), head_dim 64 or 128.
 * metric: float64 [batch, heads, head_dim, head_dim] symmetric positive
 *   semi-definite, or NULL for G = I (plain feature-space k-means).
 * centroids: float64 [batch, heads, clusters, head_dim], in: the initial
 *   centroids (e.g. seeded token picks, or the previous step's), out: final.
 * labels: int32 [batch, heads, n] (out); sizes: int32 [batch, heads, clusters] (out).
 * Limits: clusters <= 4096, batch*heads <= 65535, iters >= 1.
 */
SVSA_API int svsa_kmeans(const void* x, int32_t batch, int32_t heads, int32_t n,
                         int32_t head_dim, const double* metric, double* centroids,
                         int32_t clusters, int32_t iters, int32_t* labels, int32_t* sizes,
                         void* workspace, size_t ws_bytes, void* stream);

/* Workspace (device bytes) for svsa_cluster_means; 0 if the sizes are invalid. */
SVSA_API size_t svsa_cluster_means_workspace_bytes(int32_t batch, int32_t heads, int32_t n,
                                                   int32_t clusters);

/*
 * Cluster summaries from given labels (the block means of variable-size
 * blocks): centroids[b,h,c] = float64 mean of the tokens labelled c (summed in
 * token order), sizes[b,h,c] their count; centroids of empty clusters are
 * left unchanged.  x: bf16 [batch, heads, n, head_dim] (64 or 128); labels:
 * int32 [batch, heads, n] (labels outside [0, clusters) are ignored).
 */
SVSA_API int svsa_cluster_means(const void* x, const int32_t* labels, int32_t batch,
                                int32_t heads, int32_t n, int32_t head_dim, int32_t clusters,
                                double* centroids, int32_t* sizes, void* workspace,
                                size_t ws_bytes, void* stream);

/*
 * metric[b,h] = sum_c sizes[b,h,c] * centroids[b,h,c] centroids[b,h,c]^T
 * (float64 [batch, heads, head_dim, head_dim]): the quadratic form that one
 * side's clusters induce on the other side's tokens.  head_dim a multiple of
 * 16, at most 256.
 */
SVSA_API int svsa_cluster_metric(const double* centroids, const int32_t* sizes, int32_t batch,
                                 int32_t heads, int32_t clusters, int32_t head_dim,
                                 double* metric, void* stream);

/*
 * Rows of the padded cluster layout: n + clusters * (align - 1), rounded up to
 * align (every layout fits).  align: a power of two <= 1024.  0 if invalid.
 */
SVSA_API int64_t svsa_cluster_capacity(int32_t n, int32_t clusters, int32_t align);

/*
 * Padded cluster layout per (batch, head): cluster c owns the slots start[c]
 * .. start[c] + sizes[c] - 1, its members in ascending token order;
 * start[0] = 0, start[c+1] = start[c] + align * ceil(sizes[c] / align), so
 * start[clusters] is the padded length L (<= svsa_cluster_capacity).
 * labels: int32 [batch, heads, n] in [0, clusters) (others are not placed:
 *   their slot is -1).
 * start: int32 [batch, heads, clusters + 1]; sizes: int32 [batch, heads, clusters];
 * slot: int32 [batch, heads, n] (slot of each token; may be NULL);
 * token: int32 [batch, heads, capacity] (token in each slot s < L, -1 for padding).
 * workspace: device buffer of svsa_cluster_layout_workspace_bytes() bytes.
 */
SVSA_API size_t svsa_cluster_layout_workspace_bytes(int32_t batch, int32_t heads, int32_t n,
                                                    int32_t clusters);
SVSA_API int svsa_cluster_layout(const int32_t* labels, int32_t batch, int32_t heads, int32_t n,
                                 int32_t clusters, int32_t align, int32_t* start,
                                 int32_t* sizes, int32_t* slot, int32_t* token,
                                 void* workspace, size_t ws_bytes, void* stream);

/*
 * Rows into the cluster layout (inverse = 0: dst[s] = src[token[s]] for the
 * slots s < start[clusters], zero for padding; dst is [batch, heads,
 * capacity, head_dim]) or back to token order (inverse = 1: dst[t] =
 * src[slot[t]], zero for tokens without a slot; dst is [batch, heads, n,
 * head_dim]).  map = token (forward) or slot (inverse) from
 * svsa_cluster_layout with the same clusters and align.
 */
SVSA_API int svsa_cluster_permute(const void* src, void* dst, int32_t dtype, int32_t batch,
                                  int32_t heads, int32_t n, int32_t head_dim, int32_t clusters,
                                  int32_t align, const int32_t* map, const int32_t* start,
                                  int32_t inverse, void* stream);

/* Workspace (device bytes) for svsa_cluster_mask; 0 if the sizes are invalid. */
SVSA_API size_t svsa_cluster_mask_workspace_bytes(int32_t batch, int32_t heads, int32_t nq,
                                                  int32_t nk);

/*
 * Cluster-level mask: per (batch, head, query cluster i) the key clusters
 * kept by the rule of svsa_block_mask (top-p or fixed fraction, same
 * tie-break, float64 throughout) applied to the row softmax over key
 * clusters of  softmax_scale * <qbar_i, kbar_j> + ln ksizes_j  (the mass of
 * ksizes_j keys that all equal kbar_j; empty key clusters score 0).  No
 * diagonal band (query and key clusters are different partitions).
 * qbar: float64 [batch, heads, nq, D] (query cluster means), kbar: float64
 * [batch, heads, nk, D], ksizes: int32 [batch, heads, nk] (device).
 * row_ptr: int32 [batch*heads*nq + 1]; col_idx capacity >= batch*heads*nq*nk.
 * Limits: nq, nk <= 4096, heads <= 256.
 */
SVSA_API int svsa_cluster_mask(const double* qbar, const double* kbar, const int32_t* ksizes,
                               int32_t batch, int32_t heads, int32_t nq, int32_t nk,
                               int32_t head_dim, double softmax_scale, const float* top_p,
                               const float* keep_frac, int32_t* row_ptr, int32_t* col_idx,
                               int64_t col_capacity, void* workspace, size_t ws_bytes,
                               void* stream);

/* Workspace (device bytes) for svsa_cluster_attn; 0 if the sizes are invalid. */
SVSA_API size_t svsa_cluster_attn_workspace_bytes(int32_t batch, int32_t heads, int32_t n_q,
                                                  int32_t nq, int32_t n_k, int32_t nk,
                                                  int32_t align);

/*
 * Attention over variable-size blocks: every query token of query cluster i
 * attends, in one softmax, to every key token of the key clusters its CSR row
 * keeps (the blockwise accumulation of [PSA] App. B, Alg. 2, with blocks of
 * any size).  Inputs are in the padded cluster layouts of svsa_cluster_layout
 * with the same align (32 or 64: every cluster starts on a sub-block of that
 * many rows; padded key rows are masked).
 * q: bf16 [batch, heads, cap_q, D], k, v: bf16 [batch, heads, cap_k, D] with
 *   cap_q = svsa_cluster_capacity(n_q, nq, align), cap_k likewise.
 * out: bf16 [batch, heads, cap_q, D]; rows of query tokens are written, padded
 *   rows are unspecified; a query cluster with an empty row gets zeros.
 * q_start / q_size: int32 [batch, heads, nq + 1] / [batch, heads, nq] (device),
 *   k_start / k_size the same for the key clusters.
 * row_ptr: int32 [batch*heads*nq + 1] over rows (b, h, i); col_idx: key
 *   cluster indices (out-of-range entries are ignored).
 * Limits: head_dim 64 or 128; cap_k / align <= 8192; cap * D * 2 < 2^31.
 */
SVSA_API int svsa_cluster_attn(const void* q, const void* k, const void* v, void* out,
                               int32_t batch, int32_t heads, int32_t head_dim, int32_t n_q,
                               int32_t nq, const int32_t* q_start, const int32_t* q_size,
                               int32_t n_k, int32_t nk, const int32_t* k_start,
                               const int32_t* k_size, int32_t align, float softmax_scale,
                               const int32_t* row_ptr, const int32_t* col_idx, void* workspace,
                               size_t ws_bytes, void* stream);

/* Workspace (device bytes) for svsa_tail_merge; 0 if the sizes are invalid. */
SVSA_API size_t svsa_tail_merge_workspace_bytes(int32_t batch, int32_t heads, int32_t n,
                                                int32_t nq, int32_t nk);

/*
 * Tail merging of the query clusters ([iCATS] Sec. 4.3 and App. E.1), this
 * library's reading: (1) query clusters of one (b, h) whose kept key-cluster
 * sets are identical merge into the lowest such index (the attention pattern
 * is unchanged); (2) `rounds` times: every non-empty cluster whose size is
 * not a multiple of `block` (its tail: size mod block tokens) finds the other
 * such cluster with the most similar kept set (Jaccard |A n B| / |A u B|,
 * compared exactly; ties: lowest index); mutually nearest pairs whose tails
 * fit one block move the smaller tail (equal tails: the higher index's) - the
 * donor's last members in token order - to the other cluster, whose kept set
 * becomes the union of both.  Every token keeps at least the key clusters it
 * had; emptied clusters keep their index and own no rows.
 * labels: int32 [batch, heads, n], rewritten in place.
 * row_ptr / col_idx: the cluster mask (rows (b, h, i) over nq query
 *   clusters, columns key clusters < nk); row_ptr_out / col_idx_out: the
 *   merged mask (capacity >= batch*heads*nq*nk), ascending columns.
 * Limits: nq <= 4096, nk <= 4096, rounds <= 8.
 */
SVSA_API int svsa_tail_merge(int32_t* labels, int32_t batch, int32_t heads, int32_t n,
                             int32_t nq, int32_t nk, int32_t block, int32_t rounds,
                             const int32_t* row_ptr, const int32_t* col_idx,
                             int32_t* row_ptr_out, int32_t* col_idx_out, int64_t col_capacity,
                             void* workspace, size_t ws_bytes, void* stream);

/*
 * SNR-guided top-p schedule ([iCATS] Sec. 4.2 "SNR-Guided Sparsity" and
 * App. A; the per-model pmin and tau of App. B).  Host-only: no GPU call,
 * no allocation; the result feeds the top_p array of svsa_block_mask, one
 * denoising step at a time.
 * The pages fix the shape of the schedule (dense before the first sparse
 * step; top-p lowered through the middle of denoising and nearly flat early
 * and late; a smooth function of log-SNR, computed offline from the noise
 * schedule) but print no formula.  This library's reading, for the
 * flow-matching noise level s_k in [0, 1] (x = (1 - s) x0 + s eps):
 *   logSNR_k = 2 ln((1 - s_k) / s_k),  w_k = sigmoid(-logSNR_k)
 *                                          (1 at pure noise, 0 at clean data)
 *   top_p[k] = 1                                            k < first_sparse
 *   top_p[k] = p_min + (tau - p_min) * clamp((w_k - w_L) / (w_F - w_L), 0, 1)
 *                                                           otherwise,
 * F = first_sparse, L = steps - 1 (tau when w_F == w_L): tau is the top-p of
 * the first sparse step and p_min that of the last.
 * sigmas: host float64 [steps]; top_p: host float32 [steps] (output).
 * Errors (SVSA_E_INVALID, nothing written): NULL pointer, steps < 1,
 * first_sparse outside [0, steps], a sigma outside [0, 1] or NaN, or not
 * 0 < p_min <= tau <= 1.
 */
SVSA_API int svsa_snr_top_p(const double* sigmas, int32_t steps, int32_t first_sparse,
                            float p_min, float tau, float* top_p);

/* Static description of a status code (never NULL). */
SVSA_API const char* svsa_status_string(int status);

/* Library ABI version (major*100 + minor). */
SVSA_API int svsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SVSA_H */
