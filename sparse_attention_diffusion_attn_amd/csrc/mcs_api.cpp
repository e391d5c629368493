// C ABI of the MC-Sparse hot path: argument checks, workspace carving and
// kernel launches.  Every check runs before anything is enqueued, so a bad
// call leaves outputs untouched and the stream unchanged; the library keeps no
// device memory and no state between calls.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/mcs.h"
#include "mcs_internal.h"

namespace {

thread_local std::string g_last_error;

int32_t fail(int32_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int32_t ok() {
  g_last_error.clear();
  return MCS_OK;
}

}  // namespace

namespace mcs {
int32_t api_fail(int32_t code, const char* msg) { return fail(code, "%s", msg); }
}  // namespace mcs

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int levels_for(int groups) {
  int l = 0;
  while ((1 << l) < groups) ++l;
  return l;
}

// Shape checks common to every call.
int32_t check_dims(const mcs_dims* d) {
  if (d == nullptr) return fail(MCS_ERR_INVALID_ARG, "dims is NULL");
  if (d->batch < 1 || d->heads < 1)
    return fail(MCS_ERR_INVALID_ARG, "batch (%d) and heads (%d) must be >= 1", d->batch, d->heads);
  if (d->head_dim != 64 && d->head_dim != 96 && d->head_dim != 128)
    return fail(MCS_ERR_UNSUPPORTED, "head_dim %d not supported (64, 96 or 128)", d->head_dim);
  if (d->group_size != 64 && d->group_size != 128)
    return fail(MCS_ERR_UNSUPPORTED, "group_size %d not supported (64 or 128)", d->group_size);
  if (d->n_pad < 1 || d->n_pad >= (1 << 24))
    return fail(MCS_ERR_UNSUPPORTED, "n_pad %d outside 1 .. 2^24 - 1", d->n_pad);
  if (d->n_pad % d->group_size != 0)
    return fail(MCS_ERR_INVALID_ARG, "n_pad %d is not a multiple of group_size %d", d->n_pad,
                d->group_size);
  if (d->n_valid < 1 || d->n_valid > d->n_pad)
    return fail(MCS_ERR_INVALID_ARG, "n_valid %d outside 1 .. n_pad (%d)", d->n_valid, d->n_pad);
  const double elems = (double)d->batch * d->heads * d->n_pad * d->head_dim;
  if (elems >= 1099511627776.0)
    return fail(MCS_ERR_UNSUPPORTED, "batch*heads*n_pad*head_dim too large");
  const double items = (double)d->batch * d->heads * (d->n_pad / d->group_size);
  if (items >= 2147483647.0) return fail(MCS_ERR_UNSUPPORTED, "too many groups for one launch");
  return MCS_OK;
}

int32_t check_ptr(const void* p, const char* name, bool nullable = false) {
  if (p == nullptr) {
    if (nullable) return MCS_OK;
    return fail(MCS_ERR_INVALID_ARG, "%s is NULL", name);
  }
  if (!aligned16(p)) return fail(MCS_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return MCS_OK;
}

int32_t check_topk(const mcs_dims* d, int32_t topk) {
  if (topk < 1 || topk > d->n_valid)
    return fail(MCS_ERR_INVALID_ARG, "topk %d outside 1 .. n_valid (%d)", topk, d->n_valid);
  const double idx = (double)d->batch * d->heads * (d->n_pad / d->group_size) * topk;
  if (idx >= 9.0e15) return fail(MCS_ERR_UNSUPPORTED, "kv_idx too large");
  return MCS_OK;
}

int32_t check_scale(float s) {
  if (!std::isfinite(s) || !(s > 0.f))
    return fail(MCS_ERR_INVALID_ARG, "scale must be finite and > 0");
  return MCS_OK;
}

int32_t hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MCS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return MCS_OK;
}

#define MCS_TRY(expr)            \
  do {                           \
    const int32_t _st = (expr);  \
    if (_st != MCS_OK) return _st; \
  } while (0)

// ---- tensor layouts ----
// Strides of q, k, v and the layer output (o / o_full) in the kernels' form.
struct Lay {
  mcs::Strides q, k, v, o;
};

mcs::Strides bhnd_strides(const mcs_dims* d) {
  return {(int64_t)d->heads * d->n_pad * d->head_dim, (int64_t)d->n_pad * d->head_dim,
          (int64_t)d->head_dim};
}

// A stride of a dimension of extent 1 is never used; it is taken as 0.
mcs_strides used_strides(const mcs_dims* d, mcs_strides s) {
  if (d->batch == 1) s.batch = 0;
  if (d->heads == 1) s.head = 0;
  if (d->n_pad == 1) s.token = 0;
  return s;
}

mcs::Strides to_strides(const mcs_strides& s) { return {s.batch, s.head, s.token}; }

int32_t check_strides(const mcs_dims* d, const mcs_strides& s, const char* name, bool written) {
  const int64_t st[3] = {s.batch, s.head, s.token};
  const int64_t ext[3] = {d->batch, d->heads, d->n_pad};
  static const char* what[3] = {"batch", "head", "token"};
  for (int i = 0; i < 3; ++i) {
    if (st[i] < 0 || st[i] >= ((int64_t)1 << 40))
      return fail(MCS_ERR_INVALID_ARG, "%s %s stride %lld outside 0 .. 2^40 - 1", name, what[i],
                  (long long)st[i]);
    if (st[i] % 8 != 0)
      return fail(MCS_ERR_INVALID_ARG, "%s %s stride %lld is not a multiple of 8 elements", name,
                  what[i], (long long)st[i]);
  }
  if (s.token >= ((int64_t)1 << 23))
    return fail(MCS_ERR_UNSUPPORTED, "%s token stride %lld too large (< 2^23)", name,
                (long long)s.token);
  // a head's rows are read through 32-bit byte offsets
  if (((__int128)(d->n_pad - 1) * s.token + d->head_dim) * 2 > (__int128)0xffffffffu)
    return fail(MCS_ERR_UNSUPPORTED, "%s: one head's rows span 4 GiB or more", name);
  __int128 reach = d->head_dim;
  for (int i = 0; i < 3; ++i) reach += (__int128)(ext[i] - 1) * st[i];
  if (reach >= ((__int128)1 << 40))
    return fail(MCS_ERR_UNSUPPORTED, "%s spans 2^40 elements or more", name);
  if (written) {
    // rows of an output must not overlap: order the dimensions of extent > 1
    // by stride; each must step over everything the smaller ones cover
    int64_t ss[3], ee[3];
    int n = 0;
    for (int i = 0; i < 3; ++i)
      if (ext[i] > 1) { ss[n] = st[i]; ee[n] = ext[i]; ++n; }
    for (int i = 1; i < n; ++i)
      for (int j = i; j > 0 && ss[j] < ss[j - 1]; --j) {
        std::swap(ss[j], ss[j - 1]);
        std::swap(ee[j], ee[j - 1]);
      }
    __int128 covered = d->head_dim;
    for (int i = 0; i < n; ++i) {
      if ((__int128)ss[i] < covered)
        return fail(MCS_ERR_INVALID_ARG, "%s rows overlap (strides %lld/%lld/%lld)", name,
                    (long long)s.batch, (long long)s.head, (long long)s.token);
      covered = (__int128)ss[i] * ee[i];
    }
  }
  return MCS_OK;
}

// NULL = every tensor contiguous [B, H, n_pad, d].
int32_t resolve_layout(const mcs_dims* d, const mcs_layout* l, Lay* out) {
  if (l == nullptr) {
    out->q = out->k = out->v = out->o = bhnd_strides(d);
    return MCS_OK;
  }
  const mcs_strides q = used_strides(d, l->q), k = used_strides(d, l->k);
  const mcs_strides v = used_strides(d, l->v), o = used_strides(d, l->o);
  MCS_TRY(check_strides(d, q, "q", false));
  MCS_TRY(check_strides(d, k, "k", false));
  MCS_TRY(check_strides(d, v, "v", false));
  MCS_TRY(check_strides(d, o, "o", true));
  if (k.token != v.token)
    return fail(MCS_ERR_UNSUPPORTED, "k and v must share the token stride (%lld vs %lld)",
                (long long)k.token, (long long)v.token);
  out->q = to_strides(q);
  out->k = to_strides(k);
  out->v = to_strides(v);
  out->o = to_strides(o);
  return MCS_OK;
}

// ---- workspace layouts ----
// With power iterations, every depth runs the covariance path: entries of
// the formed nodes (the root, then the left children of nodes of >= 3 groups)
// as chunk partials, and the entries of every depth's nodes of >= 3 groups
// kept for the next depth (two buffers, previous and current).
size_t gram_entry_doubles(int head_dim) {
  const size_t dt = (size_t)head_dim / 16;
  return dt * (dt + 1) / 2 * 256 + (size_t)head_dim;
}

int largest_node(int groups, int level) {  // ceil(G / 2^level)
  return (int)(((int64_t)groups + ((int64_t)1 << level) - 1) >> level);
}

// chunks of GRAM_CH blocks of the largest node formed at `level`
int gram_chunks(int groups, int level) {
  const int m = (level == 0) ? groups : largest_node(groups, level - 1) / 2;
  return (m + mcs::GRAM_CH - 1) / mcs::GRAM_CH;
}

struct GroupWs {
  size_t partial, mu, vec, proj, perm, gram, gnode0, gnode1, total;
};

GroupWs group_ws(const mcs_dims* d) {
  const size_t bh = (size_t)d->batch * d->heads;
  const size_t G = (size_t)(d->n_pad / d->group_size);
  const size_t e = gram_entry_doubles(d->head_dim);
  const int L = levels_for((int)G);
  size_t gram = 0;  // chunk partials, largest depth
  for (int l = 0; l < L; ++l) {
    const size_t pslots = l == 0 ? 1 : (size_t)1 << (l - 1);
    gram = std::max(gram, pslots * (size_t)gram_chunks((int)G, l) * e);
  }
  // entries kept at depth l <= L-2 (read at depth l+1)
  const size_t gnode = L >= 2 ? ((size_t)1 << (L - 2)) * e : 0;
  GroupWs w;
  size_t o = 0;
  w.partial = o; o = align256(o + bh * G * d->head_dim * sizeof(double));
  w.mu = o;      o = align256(o + bh * G * d->head_dim * sizeof(double));
  w.vec = o;     o = align256(o + bh * G * d->head_dim * sizeof(double));
  w.proj = o;    o = align256(o + bh * (size_t)d->n_pad * sizeof(double));
  w.perm = o;    o = align256(o + bh * (size_t)d->n_pad * sizeof(int32_t));
  w.gram = o;    o = align256(o + bh * gram * sizeof(double));
  w.gnode0 = o;  o = align256(o + bh * gnode * sizeof(double));
  w.gnode1 = o;  o = align256(o + bh * gnode * sizeof(double));
  w.total = o;
  return w;
}

// ---- size-balanced k-means grouping ----
int32_t check_kmeans(const mcs_dims* d) {
  if (d->head_dim == 96)
    return fail(MCS_ERR_UNSUPPORTED, "k-means grouping supports head_dim 64 and 128");
  const int G = d->n_pad / d->group_size;
  if (G > mcs::KM_MAX_GROUPS)
    return fail(MCS_ERR_UNSUPPORTED, "k-means grouping supports up to %d groups per head (got %d)",
                mcs::KM_MAX_GROUPS, G);
  return MCS_OK;
}

struct KmWs {
  size_t perm, labels, cent, cnorm, counts, total;
};

KmWs km_ws(const mcs_dims* d) {
  const size_t bh = (size_t)d->batch * d->heads;
  const size_t G = (size_t)(d->n_pad / d->group_size);
  const size_t tiles = (size_t)((d->n_pad + mcs::KM_TILE - 1) / mcs::KM_TILE);
  KmWs w;
  size_t o = 0;
  w.perm = o;   o = align256(o + bh * (size_t)d->n_pad * sizeof(int32_t));
  w.labels = o; o = align256(o + bh * (size_t)d->n_pad * sizeof(int32_t));
  w.cent = o;   o = align256(o + bh * G * d->head_dim * sizeof(uint16_t));
  w.cnorm = o;  o = align256(o + bh * G * sizeof(float));
  w.counts = o; o = align256(o + bh * tiles * G * sizeof(int32_t));
  w.total = o;
  return w;
}

// per head: the group scores [G, n_valid] fp32, then the top-10-bit histogram
// of each group's row [G, 1024] int32 written by the score pass
size_t scores_bytes(const mcs_dims* d) {
  return align256((size_t)(d->n_pad / d->group_size) * d->n_valid * sizeof(float));
}
size_t scores_per_head(const mcs_dims* d) {
  return scores_bytes(d) + align256((size_t)(d->n_pad / d->group_size) * 1024 * sizeof(int32_t));
}

// ---- block selection ----
int32_t check_blocks(const mcs_dims* d, int32_t mode, int32_t block, int32_t nblocks) {
  if (d->head_dim == 96)
    return fail(MCS_ERR_UNSUPPORTED, "block selection supports head_dim 64 and 128");
  if (mode != MCS_BLOCK_EXACT && mode != MCS_BLOCK_MEANPOOL)
    return fail(MCS_ERR_INVALID_ARG, "block selection mode %d unknown", mode);
  if (block < 1 || block > d->n_valid)
    return fail(MCS_ERR_INVALID_ARG, "block %d outside 1 .. n_valid (%d)", block, d->n_valid);
  const int nb = (d->n_valid + block - 1) / block;
  if (nblocks < 1 || nblocks > nb || nblocks > 1024)
    return fail(MCS_ERR_INVALID_ARG, "nblocks %d outside 1 .. min(1024, %d blocks)", nblocks, nb);
  if ((int64_t)nblocks * block > (int64_t)1 << 30)
    return fail(MCS_ERR_UNSUPPORTED, "nblocks * block too large");
  return MCS_OK;
}

struct BlockWs {
  size_t scores, kbar, bscores, bidx, per_head;
};

// Per-head workspace of block selection: exact token scores (exact mode) or
// pooled keys (mean-pool mode), block scores, selected block indices.
BlockWs block_ws(const mcs_dims* d, int32_t mode, int32_t block, int32_t nblocks) {
  const size_t G = (size_t)(d->n_pad / d->group_size);
  const size_t nb = (size_t)((d->n_valid + block - 1) / block);
  BlockWs w{};
  size_t o = 0;
  w.scores = o;
  if (mode == MCS_BLOCK_EXACT) o = align256(o + G * d->n_valid * sizeof(float));
  w.kbar = o;
  if (mode == MCS_BLOCK_MEANPOOL) o = align256(o + nb * d->head_dim * sizeof(double));
  w.bscores = o; o = align256(o + G * nb * sizeof(float));
  w.bidx = o;    o = align256(o + G * (size_t)nblocks * sizeof(int32_t));
  w.per_head = o;
  return w;
}

int32_t attn_varlen(int mode, const mcs_dims* dims, const uint16_t* q, const uint16_t* k,
                    const uint16_t* v, const int32_t* perm, const int32_t* kv_idx,
                    int32_t kv_stride, const int32_t* kv_count, float scale, const uint16_t* aux,
                    uint16_t* out, hipStream_t s) {
  mcs::AttnParams p{};
  p.q = q; p.k = k; p.v = v; p.perm = perm; p.kv_idx = kv_idx; p.kv_count = kv_count;
  p.aux = aux; p.out = out;
  p.sq = p.sk = p.sv = p.so = p.sa = bhnd_strides(dims);
  p.bh = (int64_t)dims->batch * dims->heads; p.heads = dims->heads;
  p.n_valid = dims->n_valid; p.n_pad = dims->n_pad;
  p.groups = dims->n_pad / dims->group_size; p.topk = kv_stride; p.kv_stride = kv_stride;
  p.scale = scale;
  return hip_status(mcs::launch_attention(mode, dims->head_dim, dims->group_size, p, s),
                    mode == mcs::ATTN_SPARSE ? "sparse attention (counts)" : "residual (counts)");
}

}  // namespace

extern "C" {

int32_t mcs_abi_version(void) { return MCS_ABI_VERSION; }

void mcs_layout_bhnd(const mcs_dims* dims, mcs_layout* layout) {
  if (dims == nullptr || layout == nullptr) return;
  const int64_t d = dims->head_dim, n = dims->n_pad, h = dims->heads;
  const mcs_strides s = {h * n * d, n * d, d};
  *layout = {s, s, s, s};
}

void mcs_layout_bnhd(const mcs_dims* dims, mcs_layout* layout) {
  if (dims == nullptr || layout == nullptr) return;
  const int64_t d = dims->head_dim, n = dims->n_pad, h = dims->heads;
  const mcs_strides s = {n * h * d, d, h * d};
  *layout = {s, s, s, s};
}

const char* mcs_status_string(int32_t s) {
  switch (s) {
    case MCS_OK: return "MCS_OK";
    case MCS_ERR_INVALID_ARG: return "MCS_ERR_INVALID_ARG";
    case MCS_ERR_UNSUPPORTED: return "MCS_ERR_UNSUPPORTED";
    case MCS_ERR_WORKSPACE: return "MCS_ERR_WORKSPACE";
    case MCS_ERR_HIP: return "MCS_ERR_HIP";
    default: return "MCS_ERR_UNKNOWN";
  }
}

const char* mcs_last_error(void) { return g_last_error.c_str(); }

size_t mcs_group_workspace_bytes(const mcs_dims* dims) {
  if (check_dims(dims) != MCS_OK) return 0;
  return group_ws(dims).total;
}

int32_t mcs_group(const mcs_dims* dims, const uint16_t* q, int32_t power_iters,
                  int32_t max_levels, int32_t* perm, void* workspace, size_t workspace_bytes,
                  void* stream) {
  return mcs_group_strided(dims, nullptr, q, power_iters, max_levels, perm, workspace,
                           workspace_bytes, stream);
}

int32_t mcs_group_strided(const mcs_dims* dims, const mcs_layout* layout, const uint16_t* q,
                          int32_t power_iters, int32_t max_levels, int32_t* perm, void* workspace,
                          size_t workspace_bytes, void* stream) {
  MCS_TRY(check_dims(dims));
  Lay lay;
  MCS_TRY(resolve_layout(dims, layout, &lay));
  MCS_TRY(check_ptr(q, "q"));
  MCS_TRY(check_ptr(perm, "perm"));
  if (power_iters < 0 || power_iters > 1000)
    return fail(MCS_ERR_INVALID_ARG, "power_iters %d outside 0 .. 1000", power_iters);
  const int G = dims->n_pad / dims->group_size;
  const int L = levels_for(G);
  if (max_levels < -1 || max_levels > L)
    return fail(MCS_ERR_INVALID_ARG, "max_levels %d outside -1 .. %d", max_levels, L);
  const GroupWs w = group_ws(dims);
  if (workspace == nullptr || workspace_bytes < w.total)
    return fail(MCS_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", w.total,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(MCS_ERR_WORKSPACE, "workspace is not 256-byte aligned");

  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const int levels = (max_levels < 0) ? L : max_levels;
  int32_t* bufs[2] = {perm, (int32_t*)(ws + w.perm)};
  // the last depth must land in `perm`
  int cur = (levels % 2 == 0) ? 0 : 1;
  mcs::PddpParams p{};
  p.q = q;
  p.partial = (double*)(ws + w.partial);
  p.mu = (double*)(ws + w.mu);
  p.vec = (double*)(ws + w.vec);
  p.proj = (double*)(ws + w.proj);
  p.gram = (double*)(ws + w.gram);
  double* gnode[2] = {(double*)(ws + w.gnode0), (double*)(ws + w.gnode1)};
  p.power_iters = power_iters;
  p.sq = lay.q;
  p.bh = (int64_t)dims->batch * dims->heads;
  p.heads = dims->heads;
  p.n_pad = dims->n_pad;
  p.groups = G;
  p.perm_cur = bufs[cur];
  p.perm_next = bufs[1 - cur];
  MCS_TRY(hip_status(mcs::launch_pddp_identity(p, s), "pddp identity"));
  const int d = dims->head_dim, c = dims->group_size;
  for (int lv = 0; lv < levels; ++lv) {
    p.level = lv;
    p.perm_cur = bufs[cur];
    p.perm_next = bufs[1 - cur];
    if (power_iters > 0) {
      // covariance path: entries of the formed nodes, then per node its
      // mean, centred matrix, power iterations and sign rule
      p.nch = gram_chunks(G, lv);
      p.gram_store = (lv + 1 < L) ? 1 : 0;
      p.gnode_prev = gnode[lv & 1];
      p.gnode_cur = gnode[(lv + 1) & 1];
      MCS_TRY(hip_status(mcs::launch_pddp_gram(d, c, p, s), "pddp covariance"));
      MCS_TRY(hip_status(mcs::launch_pddp_gram_power(d, c, p, s), "pddp covariance power"));
    } else {
      // no iterations: v stays v0; only the node means are needed
      MCS_TRY(hip_status(mcs::launch_pddp_partial(d, c, 0, p, s), "pddp mean"));
      MCS_TRY(hip_status(mcs::launch_pddp_mean(d, c, p, s), "pddp mean reduce"));
    }
    MCS_TRY(hip_status(mcs::launch_pddp_partial(d, c, 2, p, s), "pddp projection"));
    MCS_TRY(hip_status(mcs::launch_pddp_split(c, p, s), "pddp split"));
    cur = 1 - cur;
  }
  return ok();
}

size_t mcs_group_kmeans_workspace_bytes(const mcs_dims* dims) {
  if (check_dims(dims) != MCS_OK || check_kmeans(dims) != MCS_OK) return 0;
  return km_ws(dims).total;
}

int32_t mcs_group_kmeans(const mcs_dims* dims, const uint16_t* q, int32_t iters, int32_t* perm,
                         int32_t* labels, void* workspace, size_t workspace_bytes, void* stream) {
  MCS_TRY(check_dims(dims));
  MCS_TRY(check_kmeans(dims));
  MCS_TRY(check_ptr(q, "q"));
  MCS_TRY(check_ptr(perm, "perm"));
  MCS_TRY(check_ptr(labels, "labels", true));
  if (iters < 0 || iters > 1000)
    return fail(MCS_ERR_INVALID_ARG, "iters %d outside 0 .. 1000", iters);
  const KmWs w = km_ws(dims);
  if (workspace == nullptr || workspace_bytes < w.total)
    return fail(MCS_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", w.total,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(MCS_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const int G = dims->n_pad / dims->group_size;
  int32_t* bufs[2] = {perm, (int32_t*)(ws + w.perm)};
  int cur = iters % 2;  // the last iteration writes `perm`
  mcs::PddpParams ip{};
  ip.perm_cur = bufs[cur];
  ip.bh = (int64_t)dims->batch * dims->heads;
  ip.n_pad = dims->n_pad;
  MCS_TRY(hip_status(mcs::launch_pddp_identity(ip, s), "k-means initial partition"));
  mcs::KmeansParams p{};
  p.q = q;
  p.sq = bhnd_strides(dims);
  p.labels = labels != nullptr ? labels : (int32_t*)(ws + w.labels);
  p.cent = (uint16_t*)(ws + w.cent);
  p.cnorm = (float*)(ws + w.cnorm);
  p.counts = (int32_t*)(ws + w.counts);
  p.bh = (int64_t)dims->batch * dims->heads;
  p.heads = dims->heads;
  p.n_pad = dims->n_pad;
  p.groups = G;
  p.tiles = (dims->n_pad + mcs::KM_TILE - 1) / mcs::KM_TILE;
  p.label_bits = levels_for(G);
  for (int it = 0; it < iters; ++it) {
    p.perm_cur = bufs[cur];
    p.perm_next = bufs[1 - cur];
    MCS_TRY(hip_status(mcs::launch_km_centroids(dims->head_dim, dims->group_size, p, s),
                       "k-means centroids"));
    MCS_TRY(hip_status(mcs::launch_km_assign(dims->head_dim, p, s), "k-means assignment"));
    MCS_TRY(hip_status(mcs::launch_km_balance(p, s), "k-means balancing"));
    cur = 1 - cur;
  }
  return ok();
}

size_t mcs_anchor_select_workspace_bytes(const mcs_dims* dims, int32_t topk) {
  if (check_dims(dims) != MCS_OK || check_topk(dims, topk) != MCS_OK) return 0;
  return scores_per_head(dims) * (size_t)dims->batch * dims->heads;
}

size_t mcs_anchor_select_min_workspace_bytes(const mcs_dims* dims, int32_t topk) {
  if (check_dims(dims) != MCS_OK || check_topk(dims, topk) != MCS_OK) return 0;
  return scores_per_head(dims);
}

int32_t mcs_dense_attn(const mcs_dims* dims, const uint16_t* q, const uint16_t* k,
                       const uint16_t* v, float scale, uint16_t* o, float* lse, void* stream) {
  return mcs_dense_attn_strided(dims, nullptr, q, k, v, scale, o, lse, stream);
}

int32_t mcs_dense_attn_strided(const mcs_dims* dims, const mcs_layout* layout, const uint16_t* q,
                               const uint16_t* k, const uint16_t* v, float scale, uint16_t* o,
                               float* lse, void* stream) {
  MCS_TRY(check_dims(dims));
  Lay lay;
  MCS_TRY(resolve_layout(dims, layout, &lay));
  MCS_TRY(check_ptr(q, "q"));
  MCS_TRY(check_ptr(k, "k"));
  MCS_TRY(check_ptr(v, "v"));
  MCS_TRY(check_ptr(o, "o"));
  MCS_TRY(check_ptr(lse, "lse", true));
  MCS_TRY(check_scale(scale));
  if (o == q || o == k || o == v) return fail(MCS_ERR_INVALID_ARG, "o must not alias q, k or v");
  mcs::AttnParams p{};
  p.q = q; p.k = k; p.v = v; p.out = o; p.lse = lse;
  p.sq = lay.q; p.sk = lay.k; p.sv = lay.v; p.so = lay.o; p.sa = lay.o;
  p.bh = (int64_t)dims->batch * dims->heads; p.heads = dims->heads;
  p.n_valid = dims->n_valid; p.n_pad = dims->n_pad;
  p.groups = dims->n_pad / dims->group_size;
  p.scale = scale;
  MCS_TRY(hip_status(mcs::launch_attention(mcs::ATTN_DENSE, dims->head_dim, dims->group_size, p,
                                           (hipStream_t)stream),
                     "dense attention"));
  return ok();
}

int32_t mcs_anchor_select(const mcs_dims* dims, const uint16_t* q, const uint16_t* k,
                          const uint16_t* v, const int32_t* perm, int32_t topk, float scale,
                          uint16_t* o_full, float* lse, int32_t* kv_idx, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return mcs_anchor_select_strided(dims, nullptr, q, k, v, perm, topk, scale, o_full, lse, kv_idx,
                                   workspace, workspace_bytes, stream);
}

int32_t mcs_anchor_select_strided(const mcs_dims* dims, const mcs_layout* layout,
                                  const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                  const int32_t* perm, int32_t topk, float scale, uint16_t* o_full,
                                  float* lse, int32_t* kv_idx, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  MCS_TRY(check_dims(dims));
  Lay lay;
  MCS_TRY(resolve_layout(dims, layout, &lay));
  MCS_TRY(check_ptr(q, "q"));
  MCS_TRY(check_ptr(k, "k"));
  MCS_TRY(check_ptr(v, "v"));
  MCS_TRY(check_ptr(perm, "perm"));
  MCS_TRY(check_ptr(o_full, "o_full"));
  MCS_TRY(check_ptr(lse, "lse"));
  MCS_TRY(check_ptr(kv_idx, "kv_idx"));
  MCS_TRY(check_topk(dims, topk));
  MCS_TRY(check_scale(scale));
  if (o_full == q || o_full == k || o_full == v)
    return fail(MCS_ERR_INVALID_ARG, "o_full must not alias q, k or v");
  const size_t per_head = scores_per_head(dims);
  if (workspace == nullptr || workspace_bytes < per_head)
    return fail(MCS_ERR_WORKSPACE, "workspace needs at least %zu bytes, got %zu", per_head,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(MCS_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  const int64_t bh = (int64_t)dims->batch * dims->heads;
  const int G = dims->n_pad / dims->group_size;

  // pass 1: dense attention (O_full, lse)
  mcs::AttnParams a{};
  a.q = q; a.k = k; a.v = v; a.out = o_full; a.lse = lse;
  a.sq = lay.q; a.sk = lay.k; a.sv = lay.v; a.so = lay.o; a.sa = lay.o;
  a.bh = bh; a.heads = dims->heads;
  a.n_valid = dims->n_valid; a.n_pad = dims->n_pad; a.groups = G; a.scale = scale;
  MCS_TRY(hip_status(mcs::launch_attention(mcs::ATTN_DENSE, dims->head_dim, dims->group_size, a, s),
                     "anchor pass 1"));

  // pass 2 + top-k, as many heads at a time as the workspace holds
  const int64_t chunk = std::min<int64_t>(bh, (int64_t)(workspace_bytes / per_head));
  for (int64_t h0 = 0; h0 < bh; h0 += chunk) {
    const int64_t hc = std::min<int64_t>(chunk, bh - h0);
    // scores of hc heads, then their histograms
    int32_t* hist = (int32_t*)((char*)workspace + hc * scores_bytes(dims));
    mcs::ScoreParams sp{};
    sp.q = q; sp.k = k; sp.perm = perm; sp.lse = lse; sp.scores = (float*)workspace;
    sp.hist = hist;
    sp.sq = lay.q; sp.sk = lay.k; sp.heads = dims->heads;
    sp.bh0 = h0; sp.bh_count = hc; sp.n_valid = dims->n_valid; sp.n_pad = dims->n_pad;
    sp.groups = G; sp.scale = scale;
    MCS_TRY(hip_status(mcs::launch_scores(dims->head_dim, dims->group_size, sp, s), "anchor pass 2"));
    mcs::TopkParams tp{};
    tp.scores = (const float*)workspace; tp.kv_idx = kv_idx; tp.bh0 = h0; tp.bh_count = hc;
    tp.n_valid = dims->n_valid; tp.groups = G; tp.topk = topk; tp.hist0 = hist;
    MCS_TRY(hip_status(mcs::launch_topk(tp, s), "top-k"));
  }
  return ok();
}

static int32_t sparse_common(const mcs_dims* dims, const uint16_t* q, const uint16_t* k,
                             const uint16_t* v, const int32_t* perm, const int32_t* kv_idx,
                             int32_t topk, float scale) {
  MCS_TRY(check_dims(dims));
  MCS_TRY(check_ptr(q, "q"));
  MCS_TRY(check_ptr(k, "k"));
  MCS_TRY(check_ptr(v, "v"));
  MCS_TRY(check_ptr(perm, "perm"));
  MCS_TRY(check_ptr(kv_idx, "kv_idx"));
  MCS_TRY(check_topk(dims, topk));
  MCS_TRY(check_scale(scale));
  return MCS_OK;
}

int32_t mcs_residual(const mcs_dims* dims, const uint16_t* q, const uint16_t* k,
                     const uint16_t* v, const int32_t* perm, const int32_t* kv_idx, int32_t topk,
                     float scale, const uint16_t* o_full, uint16_t* r, void* stream) {
  return mcs_residual_strided(dims, nullptr, q, k, v, perm, kv_idx, topk, scale, o_full, r,
                              stream);
}

int32_t mcs_residual_strided(const mcs_dims* dims, const mcs_layout* layout, const uint16_t* q,
                             const uint16_t* k, const uint16_t* v, const int32_t* perm,
                             const int32_t* kv_idx, int32_t topk, float scale,
                             const uint16_t* o_full, uint16_t* r, void* stream) {
  MCS_TRY(sparse_common(dims, q, k, v, perm, kv_idx, topk, scale));
  Lay lay;
  MCS_TRY(resolve_layout(dims, layout, &lay));
  MCS_TRY(check_ptr(o_full, "o_full"));
  MCS_TRY(check_ptr(r, "r"));
  const mcs::Strides rs = bhnd_strides(dims);
  if (r == q || r == k || r == v)
    return fail(MCS_ERR_INVALID_ARG, "r must not alias q, k or v");
  // R may overwrite O_full in place (every element is read, then written, by
  // the same lane) only if both have the same layout
  const mcs_strides ru = used_strides(dims, {rs.b, rs.h, rs.n});
  const mcs_strides ou = used_strides(dims, {lay.o.b, lay.o.h, lay.o.n});
  if (r == o_full && (ou.batch != ru.batch || ou.head != ru.head || ou.token != ru.token))
    return fail(MCS_ERR_INVALID_ARG, "r may alias o_full only if o_full is contiguous");
  mcs::AttnParams p{};
  p.q = q; p.k = k; p.v = v; p.perm = perm; p.kv_idx = kv_idx; p.aux = o_full; p.out = r;
  p.sq = lay.q; p.sk = lay.k; p.sv = lay.v; p.so = rs; p.sa = lay.o;
  p.bh = (int64_t)dims->batch * dims->heads; p.heads = dims->heads;
  p.n_valid = dims->n_valid; p.n_pad = dims->n_pad;
  p.groups = dims->n_pad / dims->group_size; p.topk = topk; p.kv_stride = topk; p.scale = scale;
  MCS_TRY(hip_status(mcs::launch_attention(mcs::ATTN_RESID, dims->head_dim, dims->group_size, p,
                                           (hipStream_t)stream),
                     "residual"));
  return ok();
}

int32_t mcs_sparse_attn(const mcs_dims* dims, const uint16_t* q, const uint16_t* k,
                        const uint16_t* v, const int32_t* perm, const int32_t* kv_idx,
                        int32_t topk, float scale, const uint16_t* r, uint16_t* o, void* stream) {
  return mcs_sparse_attn_strided(dims, nullptr, q, k, v, perm, kv_idx, topk, scale, r, o, stream);
}

int32_t mcs_sparse_attn_strided(const mcs_dims* dims, const mcs_layout* layout,
                                const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const int32_t* perm, const int32_t* kv_idx, int32_t topk,
                                float scale, const uint16_t* r, uint16_t* o, void* stream) {
  MCS_TRY(sparse_common(dims, q, k, v, perm, kv_idx, topk, scale));
  Lay lay;
  MCS_TRY(resolve_layout(dims, layout, &lay));
  MCS_TRY(check_ptr(r, "r", true));
  MCS_TRY(check_ptr(o, "o"));
  if (o == q || o == k || o == v || (r != nullptr && o == r))
    return fail(MCS_ERR_INVALID_ARG, "o must not alias q, k, v or r");
  mcs::AttnParams p{};
  p.q = q; p.k = k; p.v = v; p.perm = perm; p.kv_idx = kv_idx; p.aux = r; p.out = o;
  p.sq = lay.q; p.sk = lay.k; p.sv = lay.v; p.so = lay.o; p.sa = bhnd_strides(dims);
  p.bh = (int64_t)dims->batch * dims->heads; p.heads = dims->heads;
  p.n_valid = dims->n_valid; p.n_pad = dims->n_pad;
  p.groups = dims->n_pad / dims->group_size; p.topk = topk; p.kv_stride = topk; p.scale = scale;
  MCS_TRY(hip_status(mcs::launch_attention(mcs::ATTN_SPARSE, dims->head_dim, dims->group_size, p,
                                           (hipStream_t)stream),
                     "sparse attention"));
  return ok();
}

size_t mcs_block_select_workspace_bytes(const mcs_dims* dims, int32_t mode, int32_t block,
                                        int32_t nblocks) {
  if (check_dims(dims) != MCS_OK || check_blocks(dims, mode, block, nblocks) != MCS_OK) return 0;
  return block_ws(dims, mode, block, nblocks).per_head * (size_t)dims->batch * dims->heads;
}

size_t mcs_block_select_min_workspace_bytes(const mcs_dims* dims, int32_t mode, int32_t block,
                                            int32_t nblocks) {
  if (check_dims(dims) != MCS_OK || check_blocks(dims, mode, block, nblocks) != MCS_OK) return 0;
  return block_ws(dims, mode, block, nblocks).per_head;
}

int32_t mcs_block_select(const mcs_dims* dims, const uint16_t* q, const uint16_t* k,
                         const int32_t* perm, const float* lse, int32_t mode, int32_t block,
                         int32_t nblocks, float scale, int32_t* kv_idx, int32_t* kv_count,
                         void* workspace, size_t workspace_bytes, void* stream) {
  MCS_TRY(check_dims(dims));
  MCS_TRY(check_ptr(q, "q"));
  MCS_TRY(check_ptr(k, "k"));
  MCS_TRY(check_ptr(perm, "perm"));
  MCS_TRY(check_blocks(dims, mode, block, nblocks));
  MCS_TRY(check_ptr(lse, "lse", mode != MCS_BLOCK_EXACT));
  MCS_TRY(check_ptr(kv_idx, "kv_idx"));
  MCS_TRY(check_ptr(kv_count, "kv_count"));
  MCS_TRY(check_scale(scale));
  const BlockWs w = block_ws(dims, mode, block, nblocks);
  if (workspace == nullptr || workspace_bytes < w.per_head)
    return fail(MCS_ERR_WORKSPACE, "workspace needs at least %zu bytes, got %zu", w.per_head,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(MCS_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  const int64_t bh = (int64_t)dims->batch * dims->heads;
  const int G = dims->n_pad / dims->group_size;
  const int nb = (dims->n_valid + block - 1) / block;
  const int64_t chunk = std::min<int64_t>(bh, (int64_t)(workspace_bytes / w.per_head));
  char* ws = (char*)workspace;
  for (int64_t h0 = 0; h0 < bh; h0 += chunk) {
    const int64_t hc = std::min<int64_t>(chunk, bh - h0);
    // per-chunk carve-up: each region sized for hc heads
    const size_t rs = hc * (w.kbar - w.scores), rk = hc * (w.bscores - w.kbar);
    const size_t rb = hc * (w.bidx - w.bscores);
    mcs::BlockParams bp{};
    bp.q = q; bp.k = k; bp.perm = perm;
    bp.token_scores = (const float*)ws;
    bp.kbar = (double*)(ws + rs);
    bp.block_scores = (float*)(ws + rs + rk);
    bp.block_idx = (const int32_t*)(ws + rs + rk + rb);
    bp.kv_idx = kv_idx; bp.kv_count = kv_count;
    bp.sq = bp.sk = bhnd_strides(dims); bp.heads = dims->heads;
    bp.bh0 = h0; bp.bh_count = hc;
    bp.n_valid = dims->n_valid; bp.n_pad = dims->n_pad; bp.groups = G;
    bp.block = block; bp.nb = nb; bp.nblocks = nblocks; bp.scale = scale;
    if (mode == MCS_BLOCK_EXACT) {
      mcs::ScoreParams sp{};
      sp.q = q; sp.k = k; sp.perm = perm; sp.lse = lse; sp.scores = (float*)ws;
      sp.sq = sp.sk = bhnd_strides(dims); sp.heads = dims->heads;
      sp.bh0 = h0; sp.bh_count = hc; sp.n_valid = dims->n_valid; sp.n_pad = dims->n_pad;
      sp.groups = G; sp.scale = scale;
      MCS_TRY(hip_status(mcs::launch_scores(dims->head_dim, dims->group_size, sp, s), "block scores pass"));
      MCS_TRY(hip_status(mcs::launch_block_sums(bp, s), "block sums"));
    } else {
      MCS_TRY(hip_status(mcs::launch_key_pool(dims->head_dim, bp, s), "key pooling"));
      MCS_TRY(hip_status(mcs::launch_meanpool_scores(dims->head_dim, dims->group_size, bp, s),
                         "mean-pooled scores"));
    }
    mcs::TopkParams tp{};
    tp.scores = bp.block_scores; tp.kv_idx = (int32_t*)bp.block_idx; tp.bh0 = 0; tp.bh_count = hc;
    tp.n_valid = nb; tp.groups = G; tp.topk = nblocks;
    tp.signed_keys = (mode == MCS_BLOCK_MEANPOOL) ? 1 : 0;
    MCS_TRY(hip_status(mcs::launch_topk(tp, s), "block top-k"));
    MCS_TRY(hip_status(mcs::launch_expand_blocks(bp, s), "block expansion"));
  }
  return ok();
}

static int32_t varlen_common(const mcs_dims* dims, const uint16_t* q, const uint16_t* k,
                             const uint16_t* v, const int32_t* perm, const int32_t* kv_idx,
                             int32_t kv_stride, const int32_t* kv_count, float scale) {
  MCS_TRY(check_dims(dims));
  MCS_TRY(check_ptr(q, "q"));
  MCS_TRY(check_ptr(k, "k"));
  MCS_TRY(check_ptr(v, "v"));
  MCS_TRY(check_ptr(perm, "perm"));
  MCS_TRY(check_ptr(kv_idx, "kv_idx"));
  MCS_TRY(check_ptr(kv_count, "kv_count"));
  if (kv_stride < 1)
    return fail(MCS_ERR_INVALID_ARG, "kv_stride %d must be >= 1", kv_stride);
  const double idx = (double)dims->batch * dims->heads * (dims->n_pad / dims->group_size) * kv_stride;
  if (idx >= 9.0e15) return fail(MCS_ERR_UNSUPPORTED, "kv_idx too large");
  MCS_TRY(check_scale(scale));
  return MCS_OK;
}

int32_t mcs_sparse_attn_counts(const mcs_dims* dims, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, const int32_t* perm, const int32_t* kv_idx,
                               int32_t kv_stride, const int32_t* kv_count, float scale,
                               const uint16_t* r, uint16_t* o, void* stream) {
  MCS_TRY(varlen_common(dims, q, k, v, perm, kv_idx, kv_stride, kv_count, scale));
  MCS_TRY(check_ptr(r, "r", true));
  MCS_TRY(check_ptr(o, "o"));
  if (o == q || o == k || o == v || (r != nullptr && o == r))
    return fail(MCS_ERR_INVALID_ARG, "o must not alias q, k, v or r");
  MCS_TRY(attn_varlen(mcs::ATTN_SPARSE, dims, q, k, v, perm, kv_idx, kv_stride, kv_count, scale, r,
                      o, (hipStream_t)stream));
  return ok();
}

int32_t mcs_residual_counts(const mcs_dims* dims, const uint16_t* q, const uint16_t* k,
                            const uint16_t* v, const int32_t* perm, const int32_t* kv_idx,
                            int32_t kv_stride, const int32_t* kv_count, float scale,
                            const uint16_t* o_full, uint16_t* r, void* stream) {
  MCS_TRY(varlen_common(dims, q, k, v, perm, kv_idx, kv_stride, kv_count, scale));
  MCS_TRY(check_ptr(o_full, "o_full"));
  MCS_TRY(check_ptr(r, "r"));
  if (r == q || r == k || r == v)
    return fail(MCS_ERR_INVALID_ARG, "r must not alias q, k or v");
  MCS_TRY(attn_varlen(mcs::ATTN_RESID, dims, q, k, v, perm, kv_idx, kv_stride, kv_count, scale,
                      o_full, r, (hipStream_t)stream));
  return ok();
}

}  // extern "C"
