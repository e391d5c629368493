// Internal launch interface between the C-ABI layer (mcs_api.cpp) and the
// gfx950 kernels (*.hip).  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mcs {

enum AttnMode : int { ATTN_DENSE = 0, ATTN_SPARSE = 1, ATTN_RESID = 2 };

// Element strides of a bf16 tensor viewed as [batch, heads, n_pad, d] whose
// rows (d values) are contiguous: row (b, h, n) starts at element
// b*s.b + h*s.h + n*s.n.  The C-ABI layer checks that every stride keeps rows
// 16-byte aligned and that a head's rows span less than 4 GiB (the reach of a
// buffer resource).
struct Strides {
  int64_t b, h, n;
};

// Element offset of head bh = b*heads + h (bh < 2^31).
__host__ __device__ __forceinline__ int64_t head_offset(const Strides& s, int64_t bh, int32_t heads) {
  const int32_t b = (int32_t)bh / heads;
  return (int64_t)b * s.b + (int64_t)((int32_t)bh - b * heads) * s.h;
}

// Bytes from a head's first row to the end of row n_pad - 1.
__host__ __device__ __forceinline__ uint32_t head_span_bytes(const Strides& s, int32_t n_pad, int d) {
  return (uint32_t)(((int64_t)(n_pad - 1) * s.n + d) * 2);
}

struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* perm;    // sparse / resid: query rows of each group
  const int32_t* kv_idx;  // sparse / resid: [BH, G, kv_stride]
  const int32_t* kv_count;  // sparse / resid: [BH, G] keys per group, or NULL (= topk)
  const uint16_t* aux;    // sparse: residual to add (nullable); resid: O_full
  uint16_t* out;          // O (dense, sparse) or R (resid)
  float* lse;             // dense: nullable
  Strides sq, sk, sv;     // q, k, v (k and v share the token stride)
  Strides so, sa;         // out, aux
  int64_t bh;             // batch * heads
  int32_t heads;
  int32_t n_valid, n_pad, groups, topk;
  int32_t kv_stride;      // row stride of kv_idx (>= every count)
  float scale;
};

struct ScoreParams {
  const uint16_t* q;
  const uint16_t* k;
  const int32_t* perm;
  const float* lse;
  float* scores;          // [bh_count, G, n_valid]
  int32_t* hist;          // [bh_count, G, 1024] top-10-bit histogram of each row, or NULL
  Strides sq, sk;
  int64_t bh0, bh_count;  // heads [bh0, bh0 + bh_count)
  int32_t heads;
  int32_t n_valid, n_pad, groups;
  float scale;
};

struct TopkParams {
  const float* scores;    // [bh_count, G, n_valid]
  int32_t* kv_idx;        // [BH, G, topk], written for heads bh0 ..
  int64_t bh0, bh_count;
  int32_t n_valid, groups, topk;
  int32_t signed_keys;    // 0: scores >= 0; 1: any finite scores
  const int32_t* hist0;   // [bh_count, G, 1024] histogram of the top 10 key bits
                          // from the score pass (unsigned keys), or NULL
};

// Block selection (variants of the oracle analysis): KV blocks of `block`
// consecutive valid keys, the last one possibly shorter.
struct BlockParams {
  const uint16_t* q;
  const uint16_t* k;
  const int32_t* perm;
  const float* token_scores;  // exact mode: [bh_count, G, n_valid]
  double* kbar;               // mean-pool mode: [bh_count, NB, d]
  float* block_scores;        // [bh_count, G, NB]
  const int32_t* block_idx;   // expansion: [bh_count, G, nblocks], ascending
  int32_t* kv_idx;            // expansion: [BH, G, nblocks*block] tokens
  int32_t* kv_count;          // expansion: [BH, G]
  Strides sq, sk;
  int64_t bh0, bh_count;
  int32_t heads;
  int32_t n_valid, n_pad, groups, block, nb, nblocks;
  float scale;
};

struct PddpParams {
  const uint16_t* q;
  int32_t* perm_cur;      // current partition (read)
  int32_t* perm_next;     // next partition (split writes)
  double* partial;        // [BH, G, d]
  double* mu;             // [BH, G, d]  indexed by node start group
  double* vec;            // [BH, G, d]
  double* proj;           // [BH, n_pad] by position
  Strides sq;
  int64_t bh;
  int32_t heads;
  int32_t n_pad, groups, level;
  // covariance path; an entry is the upper 16x16 tiles of X^T X then the d
  // row sums (gram_entry doubles)
  double* gram;           // chunk partials of the formed nodes [BH, parent slots, nch, entry]
  double* gnode_prev;     // entries of the previous depth's nodes [BH, 2^(level-1), entry]
  double* gnode_cur;      // entries of this depth's nodes kept for the next [BH, 2^level, entry]
  int32_t gram_store;     // keep this depth's entries (nodes of >= 3 groups) in gnode_cur
  int32_t nch;            // chunks of GRAM_CH blocks of the largest formed node at this depth
  int32_t power_iters;    // power iterations
};

// Blocks (of C rows) per work item of the Gram path.
constexpr int GRAM_CH = 8;

// Size-balanced k-means grouping (the comparator of Fast PDDP).
constexpr int KM_TILE = 1024;     // tokens per tile of the balancing sort
constexpr int KM_MAX_GROUPS = 8192;
struct KmeansParams {
  const uint16_t* q;
  Strides sq;
  const int32_t* perm_cur;  // [BH, n_pad] current partition
  int32_t* perm_next;       // [BH, n_pad] balanced partition of this iteration
  int32_t* labels;          // [BH, n_pad] nearest centroid of each token
  uint16_t* cent;           // [BH, G, d] bf16 centroids
  float* cnorm;             // [BH, G] squared norms of the bf16 centroids
  int32_t* counts;          // [BH, tiles, G] per-tile label counts, then run starts
  int64_t bh;
  int32_t heads, n_pad, groups, tiles, label_bits;
};

// Records `msg` as this thread's last error (mcs_last_error) and returns code.
int32_t api_fail(int32_t code, const char* msg);

hipError_t launch_attention(int mode, int head_dim, int group_size, const AttnParams& p,
                            hipStream_t s);
hipError_t launch_scores(int head_dim, int group_size, const ScoreParams& p, hipStream_t s);
hipError_t launch_topk(const TopkParams& p, hipStream_t s);
hipError_t launch_block_sums(const BlockParams& p, hipStream_t s);
hipError_t launch_key_pool(int head_dim, const BlockParams& p, hipStream_t s);
hipError_t launch_meanpool_scores(int head_dim, int group_size, const BlockParams& p, hipStream_t s);
hipError_t launch_expand_blocks(const BlockParams& p, hipStream_t s);

hipError_t launch_pddp_identity(const PddpParams& p, hipStream_t s);
// stage: 0 = per-block row sums (node means without power iterations),
// 2 = projections
hipError_t launch_pddp_partial(int head_dim, int group_size, int stage, const PddpParams& p,
                               hipStream_t s);
// node means from the stage-0 sums, v = v0 (no power iterations)
hipError_t launch_pddp_mean(int head_dim, int group_size, const PddpParams& p, hipStream_t s);
hipError_t launch_pddp_split(int group_size, const PddpParams& p, hipStream_t s);
// Covariance path of a depth: X^T X and the row sums of the formed nodes (the
// root, else the left children), chunk partials summed per node
// (launch_pddp_gram); then per node its entry (right children: parent minus
// left sibling), mean, centred matrix, power iterations and sign rule
// (launch_pddp_gram_power, writes mu and v)
hipError_t launch_pddp_gram(int head_dim, int group_size, const PddpParams& p, hipStream_t s);
hipError_t launch_pddp_gram_power(int head_dim, int group_size, const PddpParams& p, hipStream_t s);

hipError_t launch_km_centroids(int head_dim, int group_size, const KmeansParams& p, hipStream_t s);
hipError_t launch_km_assign(int head_dim, const KmeansParams& p, hipStream_t s);
// count, scan and stable scatter: labels -> perm_next
hipError_t launch_km_balance(const KmeansParams& p, hipStream_t s);

}  // namespace mcs
