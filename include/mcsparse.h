/*
 * libmcsparse: meta-cached token-level sparse attention (MC-Sparse) for
 * AMD Instinct MI355X (gfx950).
 *
 * The method (MC-Sparse, arXiv 2610.06801; summarised on the paper landing
 * page's Abstract and the research walkthrough page's method steps 1-5,
 * Figure 6) caches three pieces of metadata at an anchor denoising step and
 * reuses them at the following steps:
 *   - query groups      (mcs_pddp_group)          walkthrough step 1
 *   - KV indices chosen from exact probabilities
 *                       (mcs_anchor_dense_lse, mcs_anchor_select_topk)
 *                                                  walkthrough step 2
 *   - residual R = dense - sparse output at the anchor
 *                       (mcs_residual)            walkthrough step 3
 * and a reuse step computes sparse attention over the cached indices with
 * fresh Q/K/V and adds R (mcs_sparse_apply)       walkthrough step 4.
 * R, and the KV indices in bitmap form (mcs_kv_idx_encode / _decode), can
 * be offloaded to pinned host memory and prefetched one layer ahead
 * (mcs_rcache_*)                                  walkthrough step 5; Table 8.
 *
 * Conventions shared by every call
 * --------------------------------
 * Tensors q, k, v, o, o_dense, r: bf16, logical shape [B, N, H, d] with d
 *   contiguous; element (b, n, h, c) lives at
 *   base + b*stride_b + n*stride_n + h*stride_h + c   (strides in elements).
 *   All of them share the descriptor's strides. Base pointers must be 16-byte
 *   aligned and strides multiples of 8 elements.
 * Softmax scale: desc->scale (1/sqrt(d) in every workload); no mask.
 * Groups: G = ceil(N / T) per (b, h). perm is int32 [B][H][N]: group g holds
 *   the query tokens perm[b][h][g*T : min((g+1)*T, N)], ascending; only the
 *   last group may be short.
 * KV indices: int32 [B][H][G][K], each row ascending, values in [0, N).
 * lse: fp32 [B][H][N], natural log, indexed by token.
 * Pointers are device pointers unless stated. The caller owns every buffer;
 *   compute calls allocate nothing and keep no state between calls.
 * Streams: every compute call enqueues on `stream` (a hipStream_t; NULL = the
 *   null stream) and returns without synchronising the host.
 * Errors: arguments are validated before anything is enqueued. On a non-OK
 *   status nothing was enqueued and outputs are untouched (except
 *   MCS_ERR_HIP, which reports a failed launch); mcs_last_error() returns a
 *   thread-local message. There is no fallback path.
 * Determinism: identical inputs give bitwise identical outputs (no float
 *   atomics, fixed reduction orders).
 */
#ifndef MCSPARSE_H
#define MCSPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t mcs_status_t;
enum {
  MCS_OK = 0,
  MCS_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, misaligned pointer or stride, aliasing */
  MCS_ERR_UNSUPPORTED = 2,      /* valid but not built: d not in {64,128}, T not in {64,128} */
  MCS_ERR_WORKSPACE = 3,        /* workspace smaller than the size query returned */
  MCS_ERR_HIP = 4,              /* HIP runtime or launch error; text in mcs_last_error() */
  MCS_ERR_STATE = 5             /* rcache call out of order (layer never stored / prefetched) */
};

/* A hipStream_t, kept opaque so this header needs no HIP include. */
typedef void *mcs_stream_t;

/* Checked by every call (MCS_ERR_INVALID_ARGUMENT unless noted): B, H, N >= 1
 * with B*H*N <= 2^31-1; N <= 2^28 (else MCS_ERR_UNSUPPORTED); strides
 * non-negative multiples of 8; rows of the layout disjoint (taking the
 * dimensions of size > 1 by increasing stride, each stride covers the span
 * of the dimensions inside it, a d-element row innermost), within 2^56
 * elements; one head's rows within 4 GiB (MCS_ERR_UNSUPPORTED); scale
 * finite. */
typedef struct {
  int32_t batch;    /* B >= 1 */
  int32_t heads;    /* H >= 1 */
  int32_t seqlen;   /* N >= 1 */
  int32_t head_dim; /* d in {64, 128} */
  int64_t stride_b; /* element strides of q, k, v, o, o_dense and r */
  int64_t stride_n;
  int64_t stride_h;
  float scale;      /* softmax scale */
} mcs_attn_desc_t;

/* Library version: major*10000 + minor*100 + patch. */
int32_t mcs_version(void);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char *mcs_last_error(void);

/* ------------------------------------------------------------------------
 * Step 1: Fast PDDP query grouping (research walkthrough page, method step 1,
 * Figure 6 left; paper Abstract: "tile-aligned groups").
 * For each (b, h) independently: recursively split a node S of n tokens,
 * G_S = ceil(n/T): if G_S == 1 it is a group; otherwise centre its queries,
 * form the covariance, take the principal direction by `power_iters` power
 * iterations from the unit vector of the largest diagonal entry (lowest index
 * on ties), orient it so its largest-magnitude component is positive, project
 * the centred queries on it, and put the first floor(G_S/2)*T tokens in
 * (projection, token index) order into the left child; left groups first.
 * All of this arithmetic is float64, so the split decisions do not depend on
 * fp32 rounding.
 *   q         [B,N,H,d] bf16 queries of the anchor step.
 *   group_size T in {64, 128}; power_iters in [1, 64] (16 in every workload).
 *   perm      out, int32 [B][H][N].
 *   ws        device workspace of at least mcs_pddp_group_workspace_size()
 *             bytes; contents are scratch.
 * perm and ws must not overlap q or each other. batch * heads above 65535
 * is MCS_ERR_UNSUPPORTED (for this call, its workspace query, _ex and
 * _noalloc).
 * ------------------------------------------------------------------------ */
mcs_status_t mcs_pddp_group_workspace_size(const mcs_attn_desc_t *desc, int32_t group_size,
                                           size_t *bytes);
mcs_status_t mcs_pddp_group(const mcs_attn_desc_t *desc, const void *q, int32_t group_size,
                            int32_t power_iters, int32_t *perm, void *ws, size_t ws_bytes,
                            mcs_stream_t stream);

/* Step 1 with options. mcs_pddp_group is this call with flags = 0.
 *   MCS_PDDP_WHITEN: whitened grouping. Whitening is listed on the news page
 *     only as an open item of the authors, never defined; this library reads
 *     it as per-dimension standardization. Every query dimension is centred
 *     and scaled to unit variance over the head's N tokens (population
 *     variance, float64), and a zero-variance dimension is left unscaled.
 *     The recursion above then runs on the standardized queries, so each
 *     node's covariance becomes W C W with W = diag(1/sigma). The root's
 *     power iteration starts at the lowest dimension of nonzero variance:
 *     exact arithmetic ties every standardized root variance at 1. The
 *     workspace size is the same as without the flag.
 *   Other flag bits: MCS_ERR_INVALID_ARGUMENT.
 */
#define MCS_PDDP_WHITEN 1u
mcs_status_t mcs_pddp_group_ex(const mcs_attn_desc_t *desc, const void *q, int32_t group_size,
                               int32_t power_iters, uint32_t flags, int32_t *perm, void *ws,
                               size_t ws_bytes, mcs_stream_t stream);

/* Step 1 without any allocation, for callers that cannot call hipMalloc
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * it): the same grouping as mcs_pddp_group_ex, bitwise, with the workspace
 * taken from a device array the library owns (MCS_PDDP_SCRATCH_BYTES =
 * 64 MiB on each GPU it runs on, held until the process ends).
 *   The heads are grouped in chunks whose workspace fits the scratch (they
 *   are independent), one chunk after another on `stream`.
 *   MCS_ERR_UNSUPPORTED: one head's workspace (mcs_pddp_group_workspace_size
 *   with batch = heads = 1) exceeds the scratch; every workload shape here
 *   fits (N = 98,304 at d = 128 needs about 59 MiB).
 *   Every call on one GPU shares that GPU's scratch: calls that may overlap
 *   on one GPU (other streams, other host threads) race and must be ordered
 *   by the caller (one stream, or events). Nothing in the scratch needs to
 *   start at zero. Other arguments and errors as mcs_pddp_group_ex. */
#define MCS_PDDP_SCRATCH_BYTES ((size_t)64 << 20)
mcs_status_t mcs_pddp_group_noalloc(const mcs_attn_desc_t *desc, const void *q, int32_t group_size,
                                    int32_t power_iters, uint32_t flags, int32_t *perm,
                                    mcs_stream_t stream);

/* ------------------------------------------------------------------------
 * Step 2a: anchor dense attention with per-row log-sum-exp (research
 * walkthrough page, method step 2: dense attention and each row's LSE first).
 *   o   = softmax(scale * q k^T) v, bf16 [B,N,H,d] (round to nearest even).
 *   lse = ln sum_j exp(scale * q_i . k_j), fp32 [B][H][N]; NULL skips it (the
 *         plain dense path, used as the speedup denominator).
 * o and lse must not overlap q, k, v or each other.
 * ------------------------------------------------------------------------ */
mcs_status_t mcs_anchor_dense_lse(const mcs_attn_desc_t *desc, const void *q, const void *k,
                                  const void *v, void *o, float *lse, mcs_stream_t stream);

/* ------------------------------------------------------------------------
 * Step 2b: exact probabilities, per-group accumulation and top-K (research
 * walkthrough page, method step 2: a second QK pass recovers the
 * probabilities, sums them per query group and keeps the top-K single KV
 * tokens, across KV block boundaries).
 *   A[g][j] = sum_{i in group g} exp(scale * q_i . k_j - lse_i)   (fp32)
 *   kv_idx[b][h][g][:] = the `topk` keys with the largest A[g][j]; equal
 *   mass -> lower j; stored ascending.
 *   lse         fp32 [B][H][N] from mcs_anchor_dense_lse.
 *   perm        int32 [B][H][N] from mcs_pddp_group.
 *   topk        K in [1, N].
 *   group_mass  NULL, or out fp32 [B][H][G][N]: then A is kept there and the
 *               workspace may be NULL / 0 bytes.
 *   ws          holds A when group_mass is NULL: at least
 *               mcs_anchor_select_topk_workspace_size() bytes.
 * kv_idx and A (group_mass or ws) must not overlap any input or each other.
 * ------------------------------------------------------------------------ */
mcs_status_t mcs_anchor_select_topk_workspace_size(const mcs_attn_desc_t *desc, int32_t group_size,
                                                   int32_t topk, size_t *bytes);
mcs_status_t mcs_anchor_select_topk(const mcs_attn_desc_t *desc, const void *q, const void *k,
                                    const float *lse, const int32_t *perm, int32_t group_size,
                                    int32_t topk, int32_t *kv_idx, float *group_mass, void *ws,
                                    size_t ws_bytes, mcs_stream_t stream);

/* ------------------------------------------------------------------------
 * Step 2b at block granularity: the selection-granularity ablation of the
 * paper landing page (Tables 3-4: single KV tokens against KV blocks at a
 * matched density). A block is `block` consecutive keys; its mass is the sum
 * of the exact group mass A[g][j] of its keys. Only the floor(N / block) full
 * blocks are candidates (a short last block would keep fewer keys). The
 * `nblocks` blocks of largest mass are chosen, equal mass -> lower block,
 * and their keys written block by block, ascending:
 *   kv_idx[b][h][g][i*block + t] = c_i*block + t, with c_0 < c_1 < ...
 *   group_mass  fp32 [B][H][G][N] from mcs_anchor_select_topk.
 *   block       a multiple of 64 in [64, 4096] (else MCS_ERR_UNSUPPORTED);
 *               N must hold at least one full block.
 *   nblocks     in [1, floor(N / block)].
 *   kv_idx      out, int32 [B][H][G][nblocks * block]: a key list like
 *               mcs_anchor_select_topk's, for mcs_residual / mcs_sparse_apply
 *               with topk = nblocks * block.
 *   ws          at least mcs_select_blocks_workspace_size() bytes (block
 *               sums and chosen block ids), 16-byte aligned.
 * kv_idx and ws must not overlap group_mass or each other.
 * ------------------------------------------------------------------------ */
mcs_status_t mcs_select_blocks_workspace_size(const mcs_attn_desc_t *desc, int32_t group_size, int32_t block,
                                              int32_t nblocks, size_t *bytes);
mcs_status_t mcs_select_blocks(const mcs_attn_desc_t *desc, const float *group_mass, int32_t group_size,
                               int32_t block, int32_t nblocks, int32_t *kv_idx, void *ws, size_t ws_bytes,
                               mcs_stream_t stream);

/* ------------------------------------------------------------------------
 * Step 3: anchor residual (research walkthrough page, method step 3: run the
 * sparse attention once more at the same anchor; R = dense - sparse).
 *   O_sparse(i) = sum_{j in S_g} softmax_{S_g}(scale * q_i . k_j) v_j, with
 *   the softmax renormalised over the selected set S_g of i's group;
 *   r = bf16(o_dense - O_sparse), [B,N,H,d], rows by token.
 *   o_dense is the bf16 output of mcs_anchor_dense_lse; r must not overlap
 *   any input (tensors, perm, kv_idx).
 * ------------------------------------------------------------------------ */
mcs_status_t mcs_residual(const mcs_attn_desc_t *desc, const void *q, const void *k, const void *v,
                          const void *o_dense, const int32_t *perm, int32_t group_size,
                          const int32_t *kv_idx, int32_t topk, void *r, mcs_stream_t stream);

/* ------------------------------------------------------------------------
 * Step 4: reuse-step sparse attention plus cached residual (research
 * walkthrough page, method step 4: reuse query order, KV indices and R with
 * the current step's Q, K, V; add R to the sparse result).
 *   o = bf16(O_sparse(q, k, v; perm, kv_idx) + r); r may be NULL (plain
 *   sparse attention). o must not overlap any input (tensors, perm, kv_idx).
 * ------------------------------------------------------------------------ */
mcs_status_t mcs_sparse_apply(const mcs_attn_desc_t *desc, const void *q, const void *k,
                              const void *v, const int32_t *perm, int32_t group_size,
                              const int32_t *kv_idx, int32_t topk, const void *r, void *o,
                              mcs_stream_t stream);

/* ------------------------------------------------------------------------
 * Compact KV indices for offload (research walkthrough page, method step 5;
 * paper landing page, Table 8, which offloads the selected KV indices beside
 * the residuals): one bit per key.
 *   bitmap  uint32 [B][H][G][W], W = ceil(N/32); bit (j % 32) of word j / 32
 *           of a row is set iff key j is in that row of kv_idx.
 *   mcs_kv_idx_bitmap_bytes: B*H*G*W*4.
 *   encode: kv_idx int32 [B][H][G][topk] -> bitmap. Entries outside [0, N)
 *           are dropped, repeated entries collapse.
 *   decode: bitmap -> kv_idx, ascending; each row must hold exactly topk set
 *           bits (what encode makes from a list of distinct in-range keys):
 *           with more, the first topk are written; with fewer, the tail of
 *           the row is left as it was.
 *   seqlen above 2^19 is MCS_ERR_UNSUPPORTED; kv_idx and bitmap must not
 *   overlap. Both enqueue on `stream`.
 * ------------------------------------------------------------------------ */
mcs_status_t mcs_kv_idx_bitmap_bytes(const mcs_attn_desc_t *desc, int32_t group_size, size_t *bytes);
mcs_status_t mcs_kv_idx_encode(const mcs_attn_desc_t *desc, int32_t group_size, const int32_t *kv_idx,
                               int32_t topk, uint32_t *bitmap, mcs_stream_t stream);
mcs_status_t mcs_kv_idx_decode(const mcs_attn_desc_t *desc, int32_t group_size, const uint32_t *bitmap,
                               int32_t topk, int32_t *kv_idx, mcs_stream_t stream);

/* ------------------------------------------------------------------------
 * Step 5: host offload of cached metadata with a one-layer-ahead prefetch
 * (research walkthrough page, method step 5; paper landing page, Table 8).
 * A cache holds `n_layers` (1..65536) blobs of `bytes_per_layer` bytes in
 * pinned host memory and owns two device slots used in turn (layer l uses
 * slot l % 2), plus the events that order them (two per layer, two per slot). It allocates (hipHostMalloc, hipMalloc)
 * in create and frees in destroy (which synchronises the device).
 *   store(l, src, s):     D2H copy of `bytes_per_layer` bytes from device
 *                         `src` into layer l's host blob, enqueued on s.
 *                         It first waits for the last prefetch of layer l,
 *                         on whatever stream that ran, so the blob is not
 *                         overwritten while it is being uploaded.
 *   prefetch(l, s):       H2D copy of layer l's blob into slot l % 2 on s
 *                         (a side stream). It first waits for the last store
 *                         of layer l, on whatever stream that ran, so a
 *                         store and a prefetch of one layer may be enqueued
 *                         on different streams. It also waits for the
 *                         slot's previous prefetch, so two prefetches into
 *                         one slot never write it at once. If the slot was acquired
 *                         since its last prefetch, the copy also waits for
 *                         all work enqueued so far on the acquiring stream,
 *                         so enqueue the slot's reader kernels before the
 *                         next prefetch into that slot.
 *   acquire(l, s, &ptr):  makes stream s (the compute stream) wait for the
 *                         prefetch of layer l and returns the slot pointer,
 *                         valid until the next prefetch into the same slot.
 *   MCS_ERR_STATE: prefetch of a layer never stored, acquire of a layer
 *   that is not the last prefetch into its slot.
 * ------------------------------------------------------------------------ */
typedef struct mcs_rcache mcs_rcache_t;
mcs_status_t mcs_rcache_create(int32_t n_layers, size_t bytes_per_layer, mcs_rcache_t **out);
mcs_status_t mcs_rcache_store(mcs_rcache_t *cache, int32_t layer, const void *src,
                              mcs_stream_t stream);
mcs_status_t mcs_rcache_prefetch(mcs_rcache_t *cache, int32_t layer, mcs_stream_t stream);
mcs_status_t mcs_rcache_acquire(mcs_rcache_t *cache, int32_t layer, mcs_stream_t stream,
                                const void **dev_ptr);
/* Host pointer of a layer's pinned blob (for inspection once its store has completed). */
mcs_status_t mcs_rcache_host_ptr(mcs_rcache_t *cache, int32_t layer, const void **host_ptr);
mcs_status_t mcs_rcache_destroy(mcs_rcache_t *cache);

#ifdef __cplusplus
}
#endif

#endif /* MCSPARSE_H */
