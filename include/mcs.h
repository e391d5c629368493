/*
 * mcs.h — C ABI of the MC-Sparse attention hot path on AMD Instinct MI355X
 * (gfx950).
 *
 * The method (web pages on "MC-Sparse: Analyzing and Bridging the Dense-Sparse
 * Attention Gap in Diffusion Transformers"; the onedev.kr summary, sections
 * "what is different" and "how it is used", and the ai-feeds.com summary,
 * sections "method" and "integration interface"):
 *
 *   anchor step  tau:  O_full = dense attention (the layer output)
 *                      G     = tile-aligned query groups (Fast PDDP)
 *                      S     = per-group KV token indices chosen by exact
 *                              attention probabilities (two passes)
 *                      R     = O_full - SparseAttn(Q, K, V; G, S)
 *   reuse step   t:    O_t   = SparseAttn(Q_t, K_t, V_t; G, S) + R
 *
 * Calls, in the order a caller uses them:
 *   anchor: mcs_group -> mcs_anchor_select -> mcs_residual
 *   reuse : mcs_sparse_attn
 *   mcs_dense_attn is the in-house dense kernel (anchor pass 1, and the
 *   denominator of the sparse kernel's speed-up).
 *   Selection variants of the pages' oracle analysis: mcs_block_select, then
 *   mcs_residual_counts / mcs_sparse_attn_counts on the block rows it writes.
 *
 * Conventions shared by every call
 * --------------------------------
 * Tensors are device pointers to contiguous row-major arrays (Q, K, V and the
 * layer output may also be strided views: see the `_strided` calls at the
 * end).  bf16 values are passed as uint16_t bit patterns.  Shapes use the dims
 * struct:
 *   Q, K, V, O, O_full, R : bf16  [batch, heads, n_pad, head_dim]
 *   lse                   : fp32  [batch, heads, n_pad]   (natural log)
 *   perm                  : int32 [batch, heads, n_pad]   group g = perm[g*C .. g*C+C-1]
 *   kv_idx                : int32 [batch, heads, n_pad/C, topk], ascending per group
 * Rows n_valid .. n_pad-1 are padding: the caller zero-fills them in Q, K, V;
 * padded keys never take part in a softmax and are never selected; padded
 * query rows take part in grouping as all-zero rows and get O = R = 0, lse = 0.
 * Supported: head_dim in {64, 96, 128} (the k-means comparator and the block
 * selection variants: 64 and 128); group_size C in {64, 128}; n_pad a
 * multiple of C; 1 <= n_valid <= n_pad < 2^24; 1 <= topk <= n_valid;
 * batch*heads*n_pad*head_dim < 2^40.  Every pointer must be 16-byte aligned.
 *
 * Ownership: the caller allocates every buffer, workspaces included.  The
 * library never allocates, frees or keeps device memory and holds no state
 * between calls; the metadata (perm, kv_idx, R) is ordinary caller memory that
 * may be cached, offloaded to the host or reloaded between steps.
 *
 * Device data is not validated (checking it would cost a pass over it):
 *   - perm must be a permutation of 0 .. n_pad-1 per head, as mcs_group
 *     writes it.  Its entries address query and output rows, but every
 *     kernel range-checks them: an entry outside 0 .. n_pad-1 reads query row
 *     0, counts as a padding row in the group scores and has no output row
 *     written, so a corrupted perm gives wrong results, never an access
 *     outside the tensors.
 *   - kv_idx entries must lie in 0 .. n_valid-1.  The K/V gathers are
 *     buffer loads bounded by the head's rows, so an entry outside that range
 *     reads a padding row, another row of the head or zeros, never memory
 *     outside the head, and only the result is wrong.  Ascending order is what
 *     the selection writes and what keeps the gathers sweeping forward;
 *     another order gives the same result up to rounding, and a repeated key
 *     is counted twice.
 *
 * Asynchrony: every call only enqueues work on `stream` (a hipStream_t; NULL is
 * the default stream) and returns.  Outputs are valid once the stream reaches
 * that point.  Calls on one stream run in order.
 *
 * Errors: arguments are checked before anything is enqueued.  On a bad
 * argument the call returns MCS_ERR_INVALID_ARG / MCS_ERR_UNSUPPORTED /
 * MCS_ERR_WORKSPACE, enqueues nothing, leaves every output untouched and
 * records a message for mcs_last_error() (per calling thread).  A failed kernel
 * launch returns MCS_ERR_HIP.  Faults inside kernels surface at the caller's
 * next synchronisation.
 *
 * Determinism: no floating-point atomics are used; for identical inputs on the
 * same device every output is bitwise identical from run to run.
 */
#ifndef MCS_H
#define MCS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MCS_ABI_VERSION 2

typedef enum {
  MCS_OK = 0,
  MCS_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size, bad scale   */
  MCS_ERR_UNSUPPORTED = 2, /* shape outside the supported set above         */
  MCS_ERR_WORKSPACE = 3,   /* workspace pointer null or smaller than needed  */
  MCS_ERR_HIP = 4          /* a HIP launch or runtime call failed            */
} mcs_status;

typedef struct {
  int32_t batch;      /* B                                   */
  int32_t heads;      /* H                                   */
  int32_t n_valid;    /* N, real tokens                      */
  int32_t n_pad;      /* N rounded up to a multiple of C     */
  int32_t head_dim;   /* d                                   */
  int32_t group_size; /* C, the query tile = group size      */
} mcs_dims;

int32_t mcs_abi_version(void);
const char* mcs_status_string(int32_t status);
/* Message of this thread's last failed call ("" if none). */
const char* mcs_last_error(void);

/*
 * mcs_group — Fast PDDP grouping (onedev.kr summary, "how it is used",
 * component 2).  Builds, per (batch, head), a binary tree of C-aligned median
 * splits: a node of m groups is projected on the principal direction of its
 * centred query rows (power iteration from v0 = 1/sqrt(d), `power_iters`
 * steps, sign fixed so the largest-magnitude component is positive, lowest
 * index on ties) and its members ordered by (projection, token index); the
 * first floor(m/2)*C go to the left child, the rest to the right.  All nodes of
 * one depth, across all heads, are processed by the same launches and only the
 * index array moves between depths.  Arithmetic is fp64 on the bf16 inputs; the
 * iteration runs on each node's centred covariance (X^T X - n mu mu^T), the
 * same operator as on the rows, with X^T X formed for one child of every split
 * and taken for the other as the parent's minus it.
 *   q          : bf16 [B,H,n_pad,d], the anchor step's queries (padding rows 0)
 *   power_iters: 0 .. 1000 (20 in the method's configurations)
 *   max_levels : -1 = all ceil(log2(n_pad/C)) depths; 0..L = stop after that
 *                many depths (partial trees, for testing)
 *   perm       : out, int32 [B,H,n_pad]; group g = perm[g*C .. g*C+C-1], members
 *                ascending; groups numbered left to right in the tree.
 *   workspace  : at least mcs_group_workspace_bytes(dims) bytes, 256-aligned.
 */
size_t mcs_group_workspace_bytes(const mcs_dims* dims);
int32_t mcs_group(const mcs_dims* dims, const uint16_t* q, int32_t power_iters,
                  int32_t max_levels, int32_t* perm, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * mcs_group_kmeans — size-balanced k-means grouping, a comparator of Fast
 * PDDP with the same output (onedev.kr summary, "how it is used", component 2,
 * on why k-means alone does not give equal-size groups; the system paragraph
 * compares the grouping cost with Flash-KMeans).  Per (batch, head), starting
 * from contiguous token blocks of C (iters = 0 returns that identity
 * partition), each of `iters` iterations:
 *   1. mu_g = mean of group g's C rows (fp64, rounded once to bf16);
 *   2. label_i = the g minimising ||mu_g||^2 - 2 q_i . mu_g (the dot products
 *      on bf16 matrix cores with fp32 accumulation, ||mu_g||^2 exact, rounded
 *      to fp32; ties to the lower g);
 *   3. tokens ordered by (label, token index), group g = positions
 *      g*C .. g*C+C-1 of that order.
 * Padded rows take part as all-zero rows, as in mcs_group.
 *   q      : bf16 [B,H,n_pad,d];  iters : 0 .. 1000
 *   perm   : out, int32 [B,H,n_pad], groups of exactly C, in the order of step 3
 *   labels : out (nullable), int32 [B,H,n_pad], the last iteration's labels
 *            (not written when iters = 0)
 *   workspace: at least mcs_group_kmeans_workspace_bytes(dims), 256-aligned.
 * Supported: n_pad / C <= 8192 groups (MCS_ERR_UNSUPPORTED otherwise).
 */
size_t mcs_group_kmeans_workspace_bytes(const mcs_dims* dims);
int32_t mcs_group_kmeans(const mcs_dims* dims, const uint16_t* q, int32_t iters, int32_t* perm,
                         int32_t* labels, void* workspace, size_t workspace_bytes, void* stream);

/*
 * mcs_anchor_select — the two-pass exact selection (onedev.kr summary, "how it
 * is used", components 1 and 3): pass 1 is dense attention writing O_full and
 * lse; pass 2 recomputes the logits of every group's members and scores each
 * valid key j by a_g[j] = sum over valid members i of exp(s_ij - lse_i), the
 * group's aggregated exact attention probability; the `topk` largest scores
 * (ties to the lower key index) are written ascending to kv_idx.
 *   q, k, v : bf16 [B,H,n_pad,d] at the anchor step
 *   perm    : from mcs_group
 *   scale   : softmax scale (1/sqrt(d) in the method), finite and > 0
 *   o_full  : out, bf16 [B,H,n_pad,d]; lse: out, fp32 [B,H,n_pad]
 *   kv_idx  : out, int32 [B,H,G,topk]
 *   workspace: mcs_anchor_select_workspace_bytes(dims, topk) lets all heads
 *           run at once; any size >= mcs_anchor_select_min_workspace_bytes
 *           works (heads are then processed in chunks).
 * When the workspace holds all heads, it keeps after the call the fp32 group
 * scores the selection ranked, from its first byte on, as one row-major
 * [batch*heads, n_pad/C, n_valid] array (for inspection and testing; with a
 * smaller workspace only the last chunk of heads remains, at the start).
 */
size_t mcs_anchor_select_workspace_bytes(const mcs_dims* dims, int32_t topk);
size_t mcs_anchor_select_min_workspace_bytes(const mcs_dims* dims, int32_t topk);
int32_t mcs_anchor_select(const mcs_dims* dims, const uint16_t* q, const uint16_t* k,
                          const uint16_t* v, const int32_t* perm, int32_t topk, float scale,
                          uint16_t* o_full, float* lse, int32_t* kv_idx, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * mcs_anchor_select_noalloc — mcs_anchor_select for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments and results as
 * mcs_anchor_select without the workspace: the scores live in a fixed
 * MCS_NOALLOC_SCRATCH_BYTES array that the library's device code holds on
 * every GPU it runs on until the process ends; heads are processed in chunks
 * of as many as fit.  Shapes whose single head needs more than that
 * (mcs_anchor_select_min_workspace_bytes > MCS_NOALLOC_SCRATCH_BYTES) are
 * rejected with MCS_ERR_UNSUPPORTED.  The call allocates nothing; its first
 * call on a device looks up that device's array address (the device must be
 * current and `stream` must belong to it).  All calls on one GPU share the
 * array: calls whose work overlaps on one GPU (other streams, unordered host
 * threads) race; calls ordered on one stream do not.
 */
#define MCS_NOALLOC_SCRATCH_BYTES ((size_t)192 << 20)
int32_t mcs_anchor_select_noalloc(const mcs_dims* dims, const uint16_t* q, const uint16_t* k,
                                  const uint16_t* v, const int32_t* perm, int32_t topk,
                                  float scale, uint16_t* o_full, float* lse, int32_t* kv_idx,
                                  void* stream);

/*
 * mcs_residual — R = O_full - SparseAttn(Q, K, V; perm, kv_idx) at the anchor
 * (onedev.kr summary, "what is different").  The sparse softmax is normalised
 * over each group's own index set.  Padded rows of R are 0.
 *   o_full : in, bf16 [B,H,n_pad,d];  r : out, bf16 [B,H,n_pad,d]
 */
int32_t mcs_residual(const mcs_dims* dims, const uint16_t* q, const uint16_t* k,
                     const uint16_t* v, const int32_t* perm, const int32_t* kv_idx,
                     int32_t topk, float scale, const uint16_t* o_full, uint16_t* r,
                     void* stream);

/*
 * mcs_sparse_attn — the reuse step O_t = SparseAttn(Q_t, K_t, V_t; G, S) + R
 * (onedev.kr summary, "what is different"; "how it is used", component 1: K
 * and V rows are gathered on line from the cached indices).  Each group's C
 * queries attend to exactly its topk keys kv_idx[g]; the softmax is normalised
 * over that set; R (nullable: no residual) is added in the epilogue; the result
 * is written in token order.  Padded rows of O are 0.
 *   o : out, bf16 [B,H,n_pad,d]; must not alias q, k, v or r.
 */
int32_t mcs_sparse_attn(const mcs_dims* dims, const uint16_t* q, const uint16_t* k,
                        const uint16_t* v, const int32_t* perm, const int32_t* kv_idx,
                        int32_t topk, float scale, const uint16_t* r, uint16_t* o,
                        void* stream);

/*
 * mcs_dense_attn — dense softmax attention over the n_valid keys, with the
 * per-row log-sum-exp (nullable).  The dense baseline of the onedev.kr
 * summary ("assumptions and limits") and anchor pass 1.
 *   o : out, bf16 [B,H,n_pad,d];  lse : out, fp32 [B,H,n_pad] or NULL
 */
int32_t mcs_dense_attn(const mcs_dims* dims, const uint16_t* q, const uint16_t* k,
                       const uint16_t* v, float scale, uint16_t* o, float* lse,
                       void* stream);

/*
 * Selection variants of the oracle analysis (onedev.kr summary, "how it
 * works"): at one attention density, a block oracle picks whole KV blocks per
 * query group with exact dense probabilities, and vanilla block-sparse
 * attention (BSA) ranks the blocks by mean-pooled queries and keys.  KV block
 * b holds the `block` consecutive valid keys b*block .. (the last block may be
 * shorter).  Per group, the `nblocks` best blocks (higher score first, ties to
 * the lower block index) are expanded to their tokens, ascending, in a row of
 * nblocks*block entries of kv_idx; kv_count[g] is the number of tokens written
 * and the rest of the row is set to -1.
 *   mode MCS_BLOCK_EXACT    score(g, b) = sum over the block's keys of the
 *                           group's exact score a_g[j] (as in
 *                           mcs_anchor_select; needs lse from the dense pass)
 *   mode MCS_BLOCK_MEANPOOL score(g, b) = scale * mean(q of g's valid members)
 *                           . mean(k of block b); lse is not read (NULL ok)
 * Query groups are those of perm: the identity partition (token blocks of C)
 * gives the pages' query blocks, a PDDP partition the grouped variant.
 * Scores are accumulated in fp64 and ranked in fp32.
 *   block   : 1 .. n_valid;  nblocks : 1 .. min(1024, ceil(n_valid/block))
 *   kv_idx  : out, int32 [B,H,G,nblocks*block];  kv_count : out, int32 [B,H,G]
 *   workspace: mcs_block_select_workspace_bytes(...) for all heads at once;
 *           any size >= mcs_block_select_min_workspace_bytes(...) works.
 */
#define MCS_BLOCK_EXACT 0
#define MCS_BLOCK_MEANPOOL 1
size_t mcs_block_select_workspace_bytes(const mcs_dims* dims, int32_t mode, int32_t block,
                                        int32_t nblocks);
size_t mcs_block_select_min_workspace_bytes(const mcs_dims* dims, int32_t mode, int32_t block,
                                            int32_t nblocks);
int32_t mcs_block_select(const mcs_dims* dims, const uint16_t* q, const uint16_t* k,
                         const int32_t* perm, const float* lse, int32_t mode, int32_t block,
                         int32_t nblocks, float scale, int32_t* kv_idx, int32_t* kv_count,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * mcs_sparse_attn_counts / mcs_residual_counts — mcs_sparse_attn and
 * mcs_residual for index rows of stride kv_stride whose group g uses its first
 * kv_count[g] entries (counts outside 1 .. kv_stride are clamped into it).
 * Everything else is as in the fixed-count calls.
 *   kv_idx : int32 [B,H,G,kv_stride];  kv_count : int32 [B,H,G]
 */
int32_t mcs_sparse_attn_counts(const mcs_dims* dims, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, const int32_t* perm, const int32_t* kv_idx,
                               int32_t kv_stride, const int32_t* kv_count, float scale,
                               const uint16_t* r, uint16_t* o, void* stream);
int32_t mcs_residual_counts(const mcs_dims* dims, const uint16_t* q, const uint16_t* k,
                            const uint16_t* v, const int32_t* perm, const int32_t* kv_idx,
                            int32_t kv_stride, const int32_t* kv_count, float scale,
                            const uint16_t* o_full, uint16_t* r, void* stream);

/*
 * Strided inputs and outputs.  A DiT block usually produces Q, K and V as
 * [batch, tokens, heads, head_dim] (BNHD), often as slices of one fused QKV
 * projection, and consumes the attention output in that layout too.  The
 * `_strided` calls below are the calls above with Q, K, V and the layer output
 * given as strided views instead of contiguous [B,H,n_pad,d] arrays; results
 * are bitwise the same as for contiguous copies of the same values.
 *
 * mcs_strides: element strides of a bf16 tensor seen as [B, H, n_pad, d] whose
 * rows (d values) are contiguous: row (b, h, n) starts at element
 * b*batch + h*head + n*token of the pointer passed.  The stride of a dimension
 * of extent 1 is ignored.  Every other stride must be a multiple of 8 elements
 * (16-byte rows), 0 <= stride < 2^40, token < 2^23, one head's rows must span
 * less than 4 GiB ((n_pad-1)*token*2 + 2d bytes) and the whole view less than
 * 2^40 elements.  The tensors still hold n_pad rows per head, the padding rows
 * zero-filled in Q, K and V as above.
 *
 * mcs_layout: strides of q, k, v and of o, the layer output: O of
 * mcs_sparse_attn_strided and mcs_dense_attn_strided, O_full of
 * mcs_anchor_select_strided (and read back by mcs_residual_strided).  k and v
 * must share the token stride (MCS_ERR_UNSUPPORTED otherwise); the rows of o
 * must not overlap (MCS_ERR_INVALID_ARG).  lse, perm, kv_idx and R stay
 * contiguous as above.  A NULL layout means all contiguous, i.e. the
 * unstrided calls.
 */
typedef struct {
  int64_t batch;
  int64_t head;
  int64_t token;
} mcs_strides;

typedef struct {
  mcs_strides q;
  mcs_strides k;
  mcs_strides v;
  mcs_strides o;
} mcs_layout;

/* Fill `layout` for contiguous [B,H,n_pad,d] tensors (the unstrided calls). */
void mcs_layout_bhnd(const mcs_dims* dims, mcs_layout* layout);
/* Fill `layout` for four separate contiguous [B,n_pad,H,d] tensors. */
void mcs_layout_bnhd(const mcs_dims* dims, mcs_layout* layout);

int32_t mcs_group_strided(const mcs_dims* dims, const mcs_layout* layout, const uint16_t* q,
                          int32_t power_iters, int32_t max_levels, int32_t* perm,
                          void* workspace, size_t workspace_bytes, void* stream);
int32_t mcs_anchor_select_strided(const mcs_dims* dims, const mcs_layout* layout,
                                  const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                  const int32_t* perm, int32_t topk, float scale,
                                  uint16_t* o_full, float* lse, int32_t* kv_idx,
                                  void* workspace, size_t workspace_bytes, void* stream);
int32_t mcs_residual_strided(const mcs_dims* dims, const mcs_layout* layout, const uint16_t* q,
                             const uint16_t* k, const uint16_t* v, const int32_t* perm,
                             const int32_t* kv_idx, int32_t topk, float scale,
                             const uint16_t* o_full, uint16_t* r, void* stream);
int32_t mcs_sparse_attn_strided(const mcs_dims* dims, const mcs_layout* layout,
                                const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const int32_t* perm, const int32_t* kv_idx, int32_t topk,
                                float scale, const uint16_t* r, uint16_t* o, void* stream);
int32_t mcs_dense_attn_strided(const mcs_dims* dims, const mcs_layout* layout,
                               const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               float scale, uint16_t* o, float* lse, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MCS_H */
