/*
 * bsa.h -- C ABI of the block-sparse video attention library (libbsa.so,
 * gfx950 / MI355X).
 *
 * The library computes, per attention head of a video diffusion transformer,
 *
 *   1. block summaries: the mean of the valid tokens of each query block and
 *      each key block  (bsa_pool_blocks);
 *   2. block scores, per-row selection and overrides: float32 block logits
 *      z_ij = (q̄_i·k̄_j)/sqrt(D) (+ ln n_j), per-row top-k or importance
 *      sampling, query blocks overlapping frame 0 forced dense, optional text
 *      columns, and the compacted per-row block lists  (bsa_build_mask);
 *   3. exact attention on the selected blocks only, with online softmax and
 *      an optional additive per-block log-weight  (bsa_forward);
 *   and, as a finer selector, block importance from k-means representatives
 *   of each query block (bsa_cluster_importance) with selection from any
 *   importance matrix (bsa_select_blocks); top-p selection over competition
 *   domains routed by per-head entropy (bsa_select_top_p); and structured
 *   lists of per-head frame contexts (bsa_frame_scores, bsa_classify_heads,
 *   bsa_structured_lists).
 *
 * Pages followed (title; section):
 *   - "Attention matrix view: make only frame-0 query rows dense": sec. 1
 *     token packing [text] + [frame0] + [frame1] + ...; sec. 2 frame-0 query
 *     rows attend to every key/value token; sec. 4 block-level override
 *     (first/last frame-0 query block formula); sec. 6 top-k mask built first,
 *     frame-0 rows overwritten after; sec. 7 always keep text blocks.
 *   - "Competition Domains Matter ... (EG-Sparse)": centroid-level softmax
 *     weighted by cluster size (its Eq. 2); at-least-one-key-per-row safeguard.
 *   - "AB-Attention: accurate block-sparse attention for video diffusion":
 *     TL;DR and flowchart -- exact attention on selected key/value blocks;
 *     blocks sampled in proportion to importance and reweighted by inverse
 *     inclusion probability; key blocks smaller than a tile gathered into
 *     full tiles.
 *
 * Conventions shared by every entry point
 *   - Tensors are caller-owned device pointers (allocated by any HIP
 *     allocator, e.g. PyTorch), contiguous, 16-byte aligned.  Q/K/V/O are
 *     [B, H, seq_alloc, D] with D innermost.  The library never allocates,
 *     frees or synchronizes; all work is enqueued on `stream` (a hipStream_t;
 *     NULL = the default stream) and runs asynchronously.
 *   - S = text_len + frames * latent_h * latent_w valid tokens;
 *     nqb = ceil(S / q_block), nkb = ceil(S / k_block).  Rows >= S of an
 *     input are never used as data (pad keys are excluded, pad query rows
 *     produce 0), so they may hold anything, NaN included.
 *   - Errors: every argument is validated on the host before any launch; a
 *     non-OK status means nothing was enqueued, except BSA_ERR_HIP from a
 *     failed launch.  bsa_last_error() gives a message (thread-local).  No
 *     C++ exception crosses this boundary and no call exits the process.
 *   - Entry points are reentrant.  Global state: the thread-local error
 *     message, and a per-device record that the importance kernels' dynamic
 *     LDS limit has been raised (set by the first bsa_cluster_importance
 *     call on each device).
 *   - Stream capture: apart from that first bsa_cluster_importance call on a
 *     device, an entry point makes no runtime call besides its kernel
 *     launches (no memset, copy, allocation or synchronization), so any
 *     sequence of calls on one stream can be captured in a HIP graph and
 *     replayed; make the first bsa_cluster_importance call on a device
 *     outside a capture.
 */
#ifndef BSA_H
#define BSA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSA_ABI_VERSION 1

typedef enum {
  BSA_OK = 0,
  BSA_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad size, inconsistent geometry */
  BSA_ERR_UNSUPPORTED = 2,      /* valid request outside what the kernels implement */
  BSA_ERR_HIP = 3               /* a HIP runtime call failed; see bsa_last_error() */
} bsa_status;

typedef enum { BSA_DTYPE_BF16 = 0, BSA_DTYPE_F32 = 1 } bsa_dtype;

typedef enum { BSA_SELECT_TOPK = 0, BSA_SELECT_SAMPLE = 1 } bsa_select_mode;

/* Problem statement of the frame-0 page (sec. 4): text_len, latent_H x
 * latent_W tokens per frame, q_block_size; plus batch, heads, head_dim, the
 * key block size and the padded row count of every [B,H,seq_alloc,D] buffer.
 * Supported: head_dim 64 or 128; q_block 32 or 64; k_block 16, 32 or 64;
 * seq_alloc >= max(nqb*q_block, nkb*k_block).
 * Every entry point checks its geometry first: a NULL geometry, B or H < 1,
 * a negative size, S < 1 or a short seq_alloc give BSA_ERR_INVALID_ARGUMENT;
 * an unsupported head_dim, q_block or k_block, B*H > 2^24, more than 2^30
 * blocks, or B*H*max(nqb, nkb) > 2^31 - 1 (the block rows of one launch)
 * give BSA_ERR_UNSUPPORTED. */
typedef struct {
  int32_t B, H;
  int32_t text_len, frames, latent_h, latent_w;
  int32_t head_dim;
  int32_t q_block, k_block;
  int32_t reserved;
  int64_t seq_alloc;
} bsa_geometry;

/* Selection policy.
 *   mode = BSA_SELECT_TOPK: each row keeps the k largest logits, larger
 *     first, equal logits -> lower block index first; k = topk if topk > 0,
 *     else ceil(keep_ratio * nkb) (in double) clamped to [1, nkb].
 *   mode = BSA_SELECT_SAMPLE: Poisson sampling; block j is kept with
 *     probability pi_j = min(1, c * e_j), e_j = exp(z_j - max z) (own float32
 *     exp, Cody-Waite reduction + degree-7 Taylor), c water-filled so that
 *     sum pi = fp32(keep_ratio * nkb); the uniform of block j of row
 *     r = (b*H + h)*nqb + i is word j%4 of Philox4x64-10 at counter
 *     (r, j/4, 0, 0), key (seed, 0), taken as (word >> 40) * 2^-24; kept iff
 *     u < pi.  A kept block's log-weight is -ln pi_j (0 when pi_j = 1).  A
 *     row with nothing drawn keeps its largest-logit block with weight 0.
 *   frame0_dense: query blocks overlapping frame 0 keep every key block
 *     (weight 0), applied after selection.
 *   text_columns: every row also keeps the key blocks overlapping
 *     [0, text_len) (weight 0), not counted against k.
 *   log_cluster: add fp32(ln n_j) (n_j = valid tokens of key block j) to
 *     the logits. */
typedef struct {
  int32_t mode;
  int32_t topk;
  double keep_ratio;
  int32_t frame0_dense;
  int32_t text_columns;
  int32_t log_cluster;
  int32_t reserved;
  uint64_t seed;
} bsa_mask_params;

/* Derived sizes of a geometry (host only, no device work).  `p` may be NULL,
 * then topk and expected are 0.  Errors: the geometry checks; a NULL `out`;
 * with `p`, an unknown mode, topk < 0 or keep_ratio outside (0, 1]
 * (BSA_ERR_INVALID_ARGUMENT). */
typedef struct {
  int64_t S;
  int32_t nqb, nkb;
  int32_t frame0_first, frame0_last; /* -1, -1 if no frame */
  int32_t text_last;                 /* last key block overlapping text, -1 if none */
  int32_t topk;                      /* k of a top-k policy */
  float expected;                    /* fp32(keep_ratio * nkb) of a sampling policy */
  int32_t reserved;
} bsa_derived;

bsa_status bsa_derive(const bsa_geometry* g, const bsa_mask_params* p, bsa_derived* out);

/* Block mean pooling (AB-Attention page, TL;DR "coarse summaries";
 * EG-Sparse page, cluster centroids).
 *   x:      [B, H, seq_alloc, D] of `dtype`.
 *   block:  rows per block (the geometry's q_block for Q, k_block for K).
 *   pooled: [B, H, ceil(S/block), D] float32, written.  For block i with
 *           n = min(block, S - i*block) rows and channel d:
 *           acc = 0; for t ascending: acc = fl32(acc + x[t][d]);
 *           pooled = fl32(acc / n).  Bit-reproducible.
 *   Errors: an unknown dtype, `block` other than q_block or k_block, NULL or
 *   misaligned buffers (BSA_ERR_INVALID_ARGUMENT, before any launch). */
bsa_status bsa_pool_blocks(const void* x, int32_t dtype, const bsa_geometry* g, int32_t block,
                           float* pooled, void* stream);

/* Pooling of Q and K in one launch: q_pooled as bsa_pool_blocks(q, ...,
 * q_block) and k_pooled as bsa_pool_blocks(k, ..., k_block) compute them,
 * bit for bit (same definition, same pages).  One launch instead of two
 * saves a launch and a drain between them.
 *   q, k:     [B, H, seq_alloc, D] of `dtype`.
 *   q_pooled: [B, H, nqb, D] float32, written.
 *   k_pooled: [B, H, nkb, D] float32, written.
 *   Errors: an unknown dtype, NULL or misaligned buffers
 *   (BSA_ERR_INVALID_ARGUMENT, before any launch). */
bsa_status bsa_pool_qk(const void* q, const void* k, int32_t dtype, const bsa_geometry* g, float* q_pooled,
                       float* k_pooled, void* stream);

/* Block logits, selection, overrides and compaction (frame-0 page secs. 4,
 * 6, 7; EG-Sparse page Eq. 2 and the one-key safeguard; AB-Attention page
 * sampling and reweighting).
 *   q_pooled: [B, H, nqb, D] float32 (bsa_pool_blocks with q_block).
 *   k_pooled: [B, H, nkb, D] float32 (bsa_pool_blocks with k_block).
 *   logits: z = fl32(fl32(sum_d in ascending d of fl32(q̄_d * k̄_d)) *
 *           fp32(1/sqrt(D))) (+ fp32(ln n_j), one more rounding), -0 -> +0.
 *   mask:   [B, H, nqb, nkb] uint8 (1 = block selected) or NULL.
 *   kv_cnt: [B, H, nqb] int32, number of selected blocks per row (>= 1).
 *   kv_idx: [B, H, nqb, nkb] int32, row stride nkb; the first kv_cnt
 *           entries of a row are its selected block indices, ascending; the
 *           rest are left unwritten.
 *   log_w:  [B, H, nqb, nkb] float32 or NULL (required for SAMPLE): the
 *           log-weight of list slot p of each row, 0 for top-k rows.
 *   nkb is limited to 8192 for top-k and 2048 for sampling
 *   (BSA_ERR_UNSUPPORTED beyond).
 *   Errors: the parameter checks of bsa_derive; NULL q_pooled, k_pooled,
 *   kv_cnt or kv_idx, a misaligned buffer, or SAMPLE without log_w
 *   (BSA_ERR_INVALID_ARGUMENT, before any launch). */
bsa_status bsa_build_mask(const float* q_pooled, const float* k_pooled, const bsa_geometry* g,
                          const bsa_mask_params* p, uint8_t* mask, int32_t* kv_cnt,
                          int32_t* kv_idx, float* log_w, void* stream);

/* Exact attention on the selected blocks (AB-Attention page, TL;DR and
 * "Gather kernel"/"Reweighted attention" flowchart nodes; frame-0 page sec. 2).
 *   q, k, v: [B, H, seq_alloc, D] of `dtype` (bf16 or f32).
 *   kv_cnt, kv_idx: row lists as written by bsa_build_mask (row stride nkb).
 *            Indices outside [0, nkb) are skipped.
 *   log_w:   NULL or [B, H, nqb, nkb] float32 per-slot log-weights.
 *   softmax_scale: 0 -> fp32(1/sqrt(D)).
 *   For query token t of block i: o_t = sum_u softmax_u(q_t·k_u * scale +
 *   log_w[i][p(u)]) v_u over the tokens u < S of the listed key blocks
 *   (p(u) = list slot of u's block); key blocks smaller than 64 tokens are
 *   gathered four/two per 64-key tile.  bf16: bf16 matrix products with
 *   float32 accumulation and softmax (P rounded to bf16 for the P V
 *   product); f32: float32 matrix products and softmax throughout.
 *   out:     [B, H, seq_alloc, D] of `dtype`; rows >= S and rows with an
 *            empty list are written as 0.
 *   lse:     NULL or [B, H, seq_alloc] float32, ln sum_u exp(logit_u);
 *            -inf for rows >= S and empty rows.
 *   Limits: nkb <= 8192 and one head of q/k/v below 2 GiB
 *   (BSA_ERR_UNSUPPORTED beyond).
 *   Errors: an unknown dtype, NULL q, k, v, kv_cnt, kv_idx or out, a
 *   misaligned buffer, or a softmax_scale that is negative or not finite
 *   (BSA_ERR_INVALID_ARGUMENT, before any launch). */
bsa_status bsa_forward(const void* q, const void* k, const void* v, int32_t dtype,
                       const bsa_geometry* g, const int32_t* kv_cnt, const int32_t* kv_idx,
                       const float* log_w, float softmax_scale, void* out, float* lse,
                       void* stream);

/* Launch order of the forward's work items.  Performance only: every row is
 * computed the same way, so the outputs are bit-identical under either. */
typedef enum {
  /* default: each XCD takes a contiguous run of (head, query block) items;
   * inside a head, query blocks at the same in-frame position of successive
   * frames run together (content-selected lists overlap most there) */
  BSA_ORDER_FRAME_POSITION = 0,
  /* each XCD takes the same run of frames of every head: for frame-banded
   * lists (bsa_structured_lists), whose length differs by head class, this
   * balances the XCDs and keeps each XCD's keys inside its frames */
  BSA_ORDER_FRAME_RUNS = 1
} bsa_launch_order;

typedef struct {
  int32_t launch_order;   /* bsa_launch_order */
  int32_t reserved[3];
} bsa_forward_options;

/* bsa_forward with options (NULL: the defaults).  An unknown launch order
 * gives BSA_ERR_INVALID_ARGUMENT before any launch; everything else as
 * bsa_forward. */
bsa_status bsa_forward_ex(const void* q, const void* k, const void* v, int32_t dtype,
                          const bsa_geometry* g, const int32_t* kv_cnt, const int32_t* kv_idx,
                          const float* log_w, float softmax_scale, void* out, float* lse,
                          const bsa_forward_options* opt, void* stream);

/* bsa_forward_ex with the key lists of the frame-0 query blocks split over
 * `dense_split` work items each (the rows the frame-0 override makes dense:
 * "Attention matrix view: make only frame-0 query rows dense", sec. 2 and 4).
 * Part p of such a row walks list entries floor(p*cnt/P) .. floor((p+1)*cnt/P)-1
 * and leaves its partial softmax state in `workspace`; a second kernel on the
 * same stream merges the parts into out and lse (the same exact softmax over
 * the union of the blocks, up to rounding: not bit-identical to the one-wave
 * row).  Worth it when there are few rows per SIMD, so that a frame-0 row
 * walking all nkb blocks alone would outlast the rest of the launch; the
 * other rows are unchanged.
 *   dense_split: 1..16 (1: exactly bsa_forward_ex; ignored if the geometry
 *                has no frame-0 rows).
 *   workspace:   caller-owned device memory of at least
 *                bsa_forward_split_workspace_bytes(g, dense_split) bytes,
 *                16-byte aligned (may be NULL when that size is 0); its
 *                contents on entry do not matter, and it holds partial
 *                states until the merge has run.  Calls that overlap on one
 *                workspace race.
 *   Errors: as bsa_forward_ex; also dense_split outside 1..16, or a NULL,
 *   misaligned or short workspace when one is needed
 *   (BSA_ERR_INVALID_ARGUMENT, before any launch). */
bsa_status bsa_forward_split(const void* q, const void* k, const void* v, int32_t dtype,
                             const bsa_geometry* g, const int32_t* kv_cnt, const int32_t* kv_idx,
                             const float* log_w, float softmax_scale, void* out, float* lse,
                             const bsa_forward_options* opt, int32_t dense_split, void* workspace,
                             int64_t workspace_bytes, void* stream);

/* Workspace bytes bsa_forward_split needs: B*H*(frame-0 query blocks)*
 * dense_split*(q_block*D + 2*q_block)*4, or 0 when dense_split is 1 or there
 * are no frame-0 rows.  Errors: NULL bytes, dense_split outside 1..16
 * (BSA_ERR_INVALID_ARGUMENT), or any geometry error. */
bsa_status bsa_forward_split_workspace_bytes(const bsa_geometry* g, int32_t dense_split, int64_t* bytes);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * bsa_forward_split with its workspace in scratch memory the library owns,
 * a static device array of BSA_SPLIT_STATIC_MAX_BYTES that each GPU holds
 * from the library's first use of it on that device until the process ends.
 * The call allocates nothing; the caller still owns every input and output.
 * The first call on a device looks the array's device address up (one HIP
 * runtime call, made outside a capture on that device); later calls make no
 * runtime call besides their launches.  Every call on a GPU shares that
 * GPU's array: calls whose launches overlap on one GPU (on different
 * streams, or from different threads) race, and must be ordered by the
 * caller.  Nothing in the array needs clearing: each call writes every
 * partial state it merges.
 *   Errors: as bsa_forward_split; a split that needs more than
 *   BSA_SPLIT_STATIC_MAX_BYTES (bsa_forward_split_workspace_bytes) gives
 *   BSA_ERR_UNSUPPORTED before any launch; a failed address lookup gives
 *   BSA_ERR_HIP. */
#define BSA_SPLIT_STATIC_MAX_BYTES 33554432
bsa_status bsa_forward_split_static(const void* q, const void* k, const void* v, int32_t dtype,
                                    const bsa_geometry* g, const int32_t* kv_cnt, const int32_t* kv_idx,
                                    const float* log_w, float softmax_scale, void* out, float* lse,
                                    const bsa_forward_options* opt, int32_t dense_split, void* stream);

/* Intra-block clustering selector, step 1: block importance (AB-Attention
 * page, TL;DR item 1 and the flowchart's intra-block cluster node: queries
 * are clustered only inside their own query block; EG-Sparse page Eq. 2 for
 * the cluster-size-weighted softmax of a representative).
 *   q:          [B, H, seq_alloc, D] of `dtype` (the raw queries).
 *   k_pooled:   [B, H, nkb, D] float32 (bsa_pool_blocks with k_block).
 *   n_clusters: C in 1..8; a block of n < C valid tokens uses n clusters.
 *   iters:      Lloyd rounds T in 0..16.
 *   log_cluster: add fp32(ln n_j) to every logit (nonzero) or not.
 *   importance: [B, H, nqb, nkb] float32, written.
 *   Per query block: k-means of its valid tokens (squared Euclidean
 *   distance, sequential non-fused float32 chain over the channels; initial
 *   centroid c = token floor(c n / C); a token joins the lowest-index nearest
 *   centroid; an update replaces each non-empty centroid by the mean of its
 *   tokens, summed in ascending token order; T rounds, then one final
 *   assignment gives the sizes m_c).  For each non-empty cluster, logits z
 *   against every k̄_j exactly as in bsa_build_mask, e_j = exp(z_j - max z)
 *   by a fixed float32 sequence (Cody-Waite reduction, degree-7 Taylor
 *   polynomial), P_c,j = e_j / (sum of e by a halving tree over the row
 *   padded to a power of two).  importance_j = sum over clusters, ascending,
 *   of fl32(fl32(m_c / n) * P_c,j): the expected attention mass a query of
 *   the block puts on key block j.  Bit-reproducible; each row sums to 1
 *   within rounding.  With C = 1 and T >= 1 it is P' of the pooled block.
 *   Limits: C * nkb <= 16384 and nkb <= 8192 (BSA_ERR_UNSUPPORTED beyond).
 *   Errors: an unknown dtype, NULL or misaligned buffers, C or T out of
 *   range (BSA_ERR_INVALID_ARGUMENT, before any launch). */
bsa_status bsa_cluster_importance(const void* q, int32_t dtype, const float* k_pooled,
                                  const bsa_geometry* g, int32_t n_clusters, int32_t iters,
                                  int32_t log_cluster, float* importance, void* stream);

/* Intra-block clustering selector, step 2: selection from an importance
 * matrix (AB-Attention page, TL;DR item 2: blocks sampled in proportion to
 * importance and reweighted by the inverse inclusion probability; frame-0
 * page secs. 4, 6, 7 for the overrides).
 *   importance: [B, H, nqb, nkb] float32, finite, >= 0 (e.g. from
 *               bsa_cluster_importance).
 *   p:          as for bsa_build_mask; log_cluster is ignored (already in
 *               the importance).  TOPK keeps the k largest importances of a
 *               row (lower index first among equals); SAMPLE draws each block
 *               with inclusion probability pi_j = min(1, c * importance_j),
 *               sum pi = keep_ratio * nkb, exactly as bsa_build_mask does
 *               from exp(z - max z); the safeguard keeps the first block of
 *               largest importance.
 *   mask, kv_cnt, kv_idx, log_w: as for bsa_build_mask.
 *   Limits and errors as for bsa_build_mask (with importance in place of
 *   q_pooled and k_pooled). */
bsa_status bsa_select_blocks(const float* importance, const bsa_geometry* g,
                             const bsa_mask_params* p, uint8_t* mask, int32_t* kv_cnt,
                             int32_t* kv_idx, float* log_w, void* stream);

/* Top-p selection over competition domains (EG-Sparse page: per-head
 * entropy, Eq. 3; the domain hierarchy of its Section 3.3; its deployed
 * routing of low-entropy heads to a shared pool; the value-aware score of
 * the cross-head pool; the one-key-per-row safeguard). */
typedef enum {
  BSA_DOMAIN_ROW = 0,    /* per-row local: each row keeps its own top-p */
  BSA_DOMAIN_HEAD = 1,   /* per-head global: all rows of a head share one pool */
  BSA_DOMAIN_SPLIT = 2,  /* grouped cross-head: low- and high-entropy heads, two pools */
  BSA_DOMAIN_ALL = 3,    /* all-head global: one pool per batch element */
  BSA_DOMAIN_EG = 4      /* low-entropy heads share a pool, the others per-row local */
} bsa_domain;

typedef struct {
  int32_t domain;        /* bsa_domain */
  int32_t value_aware;   /* pooled domains rank by fl32(P' * ||v̄_j||) (needs v_pooled) */
  double top_p;          /* in (0, 1] */
  float entropy_eps;     /* > 0: H_h = (1/nqb) sum_i sum_j -P' ln(P' + eps) */
  int32_t frame0_dense;  /* query blocks overlapping frame 0 keep every block */
  int32_t text_columns;  /* every row keeps the key blocks overlapping the text */
  int32_t reserved;
} bsa_topp_params;

/* Bytes of device workspace bsa_select_top_p needs for this geometry.
 * Errors: the geometry checks; a NULL `bytes` (BSA_ERR_INVALID_ARGUMENT). */
bsa_status bsa_top_p_workspace_bytes(const bsa_geometry* g, int64_t* bytes);

/*   scores:      [B, H, nqb, nkb] float32 P' (finite, >= 0, each row of mass
 *                about 1; e.g. bsa_cluster_importance with one cluster).
 *   v_pooled:    [B, H, nkb, D] float32 (bsa_pool_blocks of V with k_block)
 *                when value_aware, else ignored (may be NULL).
 *   head_entropy: [B, H] float64 written, or NULL.
 *   workspace:   device buffer of at least bsa_top_p_workspace_bytes bytes,
 *                owned by the caller, overwritten; calls that share one
 *                workspace must not overlap.
 *   mask, kv_cnt, kv_idx: as for bsa_build_mask.
 * Mass is counted in fixed point, m(s) = floor(s * 2^32) + 1, exact in any
 * order; a domain keeps every block whose score is at least T, the largest
 * score with mass(score >= T) >= ceil(top_p * mass(domain)).  The median
 * split puts the floor(H/2) lowest-entropy heads of each batch element
 * (lower head first among equals) in the low group.  In a pooled domain a
 * row left empty keeps its first block of largest score.  Frame-0 rows and
 * text columns are applied after.  Limits: nkb <= 2048 and H <= 4096
 * (BSA_ERR_UNSUPPORTED beyond); pooled value-aware scores should stay below
 * 2^16.
 * Errors: NULL params, an unknown domain, top_p outside (0, 1], an
 * entropy_eps that is not finite and > 0, NULL scores, workspace, kv_cnt or
 * kv_idx, value_aware without v_pooled, a misaligned buffer, or a workspace
 * smaller than bsa_top_p_workspace_bytes (BSA_ERR_INVALID_ARGUMENT, before
 * any launch). */
bsa_status bsa_select_top_p(const float* scores, const float* v_pooled, const bsa_geometry* g,
                            const bsa_topp_params* tp, double* head_entropy, void* workspace,
                            int64_t workspace_bytes, uint8_t* mask, int32_t* kv_cnt, int32_t* kv_idx,
                            void* stream);

/* Structured block lists: per-head frame contexts over the same forward
 * ("Efficient Autoregressive Video Diffusion with Dummy Head": frame
 * attention scores of its Step 0, Dynamic Head Programming of its Step 1 and
 * worked example, the per-class contexts of its Steps 2-3; the block-causal
 * frame mask of "Purpose of the block-causal mask ..."; frame-0 page sec. 1
 * token packing).  Token t is text (frame -1) if t < text_len, else in frame
 * (t - text_len) / (latent_h * latent_w); frame 0 is the sink frame. */
typedef enum {
  BSA_HEAD_FULL = 0,      /* every frame (frames <= the query's with block_causal) */
  BSA_HEAD_SINK = 1,      /* the sink frame and the query's frame */
  BSA_HEAD_NEIGHBOR = 2,  /* the last `window` frames, the query's included */
  BSA_HEAD_DUMMY = 3      /* the query's frame (and the one before with dummy_prev) */
} bsa_head_class;

typedef struct {
  int32_t window;         /* L >= 1 */
  int32_t dummy_prev;     /* dummy heads also see frame i-1 (packed dummy heads) */
  int32_t block_causal;   /* full heads see frames <= the query's only */
  int32_t frame0_dense;   /* query blocks overlapping frame 0 keep every block */
  int32_t text_columns;   /* every row keeps the key blocks overlapping the text */
  int32_t reserved;
} bsa_struct_params;

/* Frame attention scores of every head from block scores.
 *   scores: [B, H, nqb, nkb] float32 P' (e.g. bsa_cluster_importance, one
 *           cluster).
 *   window: L >= 1.
 *   alpha:  [B, H, 3] float64 device buffer, written: for every query block
 *           whose first token is in a frame f >= 1, the P' mass on key blocks
 *           whose first token is in frame 0 (sink), in frames max(1, f-L+1)
 *           .. f-1 (neighbor) and in frame f (current), normalized to sum 1;
 *           the mean over those query blocks (0 if there are none).
 *   Errors: NULL or misaligned buffers, window < 1, or no frames give
 *   BSA_ERR_INVALID_ARGUMENT, more than 4096 frames BSA_ERR_UNSUPPORTED,
 *   before any launch. */
bsa_status bsa_frame_scores(const float* scores, const bsa_geometry* g, int32_t window, double* alpha,
                            void* stream);

/* Dynamic Head Programming on the host (no device work).
 *   alpha:   host [B, H, 3] frame scores.  n_dummy: dummy heads per batch
 *            element, 0..H.
 *   classes: host [B, H] int32, written: the n_dummy heads of smallest
 *            max(a_sink, a_neighbor) (lower head first among equals) are
 *            BSA_HEAD_DUMMY, the others BSA_HEAD_SINK if a_sink > a_neighbor,
 *            else BSA_HEAD_NEIGHBOR.
 *   Errors: NULL pointers, B or H < 1, n_dummy outside 0..H, or a
 *   non-finite alpha give BSA_ERR_INVALID_ARGUMENT; classes is then not
 *   written. */
bsa_status bsa_classify_heads(const double* alpha, int32_t B, int32_t H, int32_t n_dummy, int32_t* classes);

/* Block lists of the per-head contexts.
 *   head_class: [B, H] int32 device buffer of bsa_head_class values.
 *   A query block's context is the union over the frames of its tokens of
 *   its head class's frames, plus the text; a query block holding text sees
 *   everything.  A key block is listed iff it holds a token of the context.
 *   Frame-0 rows and text columns are applied after.  A class value other
 *   than 0, 1 or 2 is read as BSA_HEAD_DUMMY.
 *   mask (optional, NULL to skip), kv_cnt, kv_idx: as for bsa_build_mask
 *   (lists ascending; entries past kv_cnt are not written).
 *   Errors: NULL params, head_class, kv_cnt or kv_idx, a buffer not 16-byte
 *   aligned or window < 1 give BSA_ERR_INVALID_ARGUMENT before any launch. */
bsa_status bsa_structured_lists(const int32_t* head_class, const bsa_geometry* g, const bsa_struct_params* sp,
                                uint8_t* mask, int32_t* kv_cnt, int32_t* kv_idx, void* stream);

const char* bsa_status_string(int32_t status);
const char* bsa_last_error(void);
int32_t bsa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H */
