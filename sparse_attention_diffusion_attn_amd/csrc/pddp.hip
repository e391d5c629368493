// Fast PDDP grouping on gfx950 (onedev.kr summary, "how it is used",
// component 2): equal-size groups of exactly C queries from recursive median
// splits along each node's principal direction.  All nodes of one tree depth,
// across all heads, are handled by the same launches, and only the index array
// (perm) is carried from one depth to the next.
//
// A node of m groups occupies perm[s*C .. (s+m)*C) with its members in
// ascending token order.  Because every node is a whole number of groups, the
// 1-group blocks of perm are natural work units: each per-row pass (mean, power
// iteration step, projection) runs one workgroup per block and writes a fixed
// fp64 partial; a per-node kernel sums the partials in block order, so every
// reduction has a fixed order and results are bitwise reproducible.  At the
// upper depths (large nodes) the power iteration runs instead on each node's
// d x d covariance, formed once on the fp64 matrix cores (the covariance path
// below).  The split is an exact radix select on the fp64 projections (64-bit
// order-preserving keys, ties broken by position = token index) followed by a
// stable partition.
#include <utility>

#include "mcs_common.h"
#include "mcs_internal.h"

namespace mcs {

// Node (start group s, size m groups) containing group g at tree depth `level`.
// A node of m groups splits into floor(m/2) (left) and the rest (right); a node
// of one group is a leaf and stays as it is.
__device__ __forceinline__ void node_of(int G, int level, int g, int& s, int& m) {
  s = 0;
  m = G;
  for (int l = 0; l < level && m >= 2; ++l) {
    const int hh = m >> 1;
    if (g < s + hh) {
      m = hh;
    } else {
      s += hh;
      m -= hh;
    }
  }
}

// Node numbered `slot` (0 .. 2^level - 1, the path bits from the root, left =
// 0) at tree depth `level`.  A one-group leaf is carried down as its own left
// child, so every node of the depth has exactly one slot; other slots are
// empty (returns false).
__device__ __forceinline__ bool node_of_slot(int G, int level, int slot, int& s, int& m) {
  s = 0;
  m = G;
  for (int b = level - 1; b >= 0; --b) {
    const int bit = (slot >> b) & 1;
    if (m < 2) {
      if (bit) return false;
      continue;
    }
    const int hh = m >> 1;
    if (bit == 0) {
      m = hh;
    } else {
      s += hh;
      m -= hh;
    }
  }
  return true;
}

__global__ void pddp_identity_kernel(int32_t* perm, int n_pad, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < total) perm[i] = (int32_t)(i % n_pad);
}

// fp64 value of another lane, moved by a DPP lane pattern (both 32-bit halves).
// Every pattern used here has a source lane inside the row for every lane,
// so no "old" value is needed (and none is materialised).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)u, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// Sum over aligned groups of N = 8 or 16 lanes, the same bits in every lane of
// a group: pairs (quad_perm 1,0,3,2), quads (quad_perm 2,3,0,1), halves of a
// 16-lane row (row_half_mirror), whole rows (row_mirror).  Each step adds a
// lane's value to its partner's in the other half of the block being merged,
// and the partner adds the same two numbers, so every lane ends with
// bitwise the same sum.
template <int N>
__device__ __forceinline__ double group_sum(double x) {
  x += dpp_f64<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f64<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f64<0x141>(x);  // row_half_mirror
  if (N == 16) x += dpp_f64<0x140>(x);  // row_mirror
  return x;
}
// x + (value of lane l ^ 16) and x + (value of lane l ^ 32), in the VALU.
__device__ __forceinline__ double add_xor16(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)u, (uint32_t)u, false, false);
  const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
  const double a = __longlong_as_double((long long)(((uint64_t)hi[0] << 32) | lo[0]));
  const double b = __longlong_as_double((long long)(((uint64_t)hi[1] << 32) | lo[1]));
  return a + b;
}
__device__ __forceinline__ double add_xor32(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)u, (uint32_t)u, false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
  const double a = __longlong_as_double((long long)(((uint64_t)hi[0] << 32) | lo[0]));
  const double b = __longlong_as_double((long long)(((uint64_t)hi[1] << 32) | lo[1]));
  return a + b;
}

// stage 0: partial[g] = sum of the block's rows (node means when no power
//          iterations run)
// stage 2: proj[pos] = (x_r - mu) . v (v with its sign already fixed)
//
// Persistent: workgroup i handles the C-row blocks i, i + P, i + 2P, ... (P =
// grid size, all resident), each block being one group of perm (block b =
// head b / G, group b % G).  Thread (dg, rg) owns dimensions DPL*dg ..
// DPL*dg + DPL-1 of the rows rg, rg + RG, ... of a block and keeps them in
// VGPRs (bf16; DPL = 8, or 12 for d = 96 with 8 lanes per row); the DG
// threads of a row are consecutive lanes.  While block b is computed, the
// rows of block b + P (and the perm indices of block b + 2P) are loading, and
// the node's mu / v of block b + P are copied into the other half of a
// double-buffered LDS pair, so the workgroup never waits on a dependent load
// chain.  Reductions: per-row dot products over the DG lanes of the row with
// DPP moves; per-dimension sums over a wavefront's row groups with lane swaps,
// then over the four wavefronts in LDS (fixed orders throughout).
//
// With c = mu . v, t_r = (x_r - mu) . v = x_r . v - c.
template <int D>
struct RowLayout {
  static constexpr int DPL = (D == 96) ? 12 : 8;  // dimensions per lane
  static constexpr int DG = D / DPL;              // lanes per row
  static constexpr int W4 = DPL / 2;              // 32-bit words per lane
};

template <int D, int C, int STAGE>
__global__ __launch_bounds__(256) void pddp_partial_kernel(PddpParams p) {
  constexpr int NT = 256;
  constexpr int DPL = RowLayout<D>::DPL, DG = RowLayout<D>::DG, W4 = RowLayout<D>::W4;
  constexpr int RG = NT / DG, RPT = C / RG;
  static_assert(DG == 8 || DG == 16, "row lanes");
  static_assert(STAGE == 0 || STAGE == 2, "stage");
  __shared__ __attribute__((aligned(16))) double muv[2][2][128];  // [buf][mu | v][d]
  __shared__ double part[NT / 64][D];
  const int G = p.groups;
  const int64_t nblk = p.bh * (int64_t)G;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int dg = tid % DG, rg = tid / DG;

  const __amdgpu_buffer_rsrc_t murs =
      make_rsrc(p.mu, (uint32_t)min<int64_t>(nblk * D * 8, 0xffffffffll));
  const __amdgpu_buffer_rsrc_t vrs =
      make_rsrc(p.vec, (uint32_t)min<int64_t>(nblk * D * 8, 0xffffffffll));

  // Block b = bh * G + g.  A workgroup takes blocks b, b + P, b + 2P, ... (P =
  // grid size); the (head, group) pairs of the next blocks are stepped with a
  // carry instead of divided out again (the divisions were most of the
  // per-block scalar work).
  struct Pos {
    int bh, g;
  };
  const int P = gridDim.x;
  const int dbh = P / G, dg_step = P - dbh * G;
  auto step = [&](Pos q) {
    q.g += dg_step;
    q.bh += dbh;
    if (q.g >= G) {
      q.g -= G;
      ++q.bh;
    }
    return q;
  };
  const int nbh = (int)p.bh;

  // perm indices of this thread's rows in block q
  auto load_idx = [&](Pos q, int (&ix)[RPT]) {
    const int32_t* pc = p.perm_cur + (int64_t)q.bh * p.n_pad + (int64_t)q.g * C;
#pragma unroll
    for (int k = 0; k < RPT; ++k) ix[k] = pc[rg + k * RG];
  };
  // this thread's DPL bf16 of each of its rows (16 bytes, or 16 + 8)
  struct Row {
    uint32_t u[W4];
  };
  auto load_rows = [&](Pos q, const int (&ix)[RPT], Row (&xr)[RPT]) {
    const uint16_t* Qb = p.q + head_offset(p.sq, q.bh, p.heads);
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const uint16_t* src = Qb + (int64_t)ix[k] * p.sq.n + DPL * dg;
      const uint4 a = *(const uint4*)src;
      xr[k].u[0] = a.x; xr[k].u[1] = a.y; xr[k].u[2] = a.z; xr[k].u[3] = a.w;
      if constexpr (W4 == 6) {
        const uint2 b = *(const uint2*)(src + 8);
        xr[k].u[4] = b.x; xr[k].u[5] = b.y;
      }
    }
  };
  // mu and v of the node starting at group s into LDS half `buf` (one 16-byte
  // copy per lane of waves 0 and 1; for D < 128 the upper part is not used)
  auto load_muv = [&](Pos q, int s, int buf) {
    if (STAGE == 0 || w > 1) return;
    const uint32_t off = (uint32_t)((((int64_t)q.bh * G + s) * D) * 8) + 16u * (uint32_t)lane;
    if (w == 0) gather16_buf(murs, &muv[buf][0][0], off, 0);
    else gather16_buf(vrs, &muv[buf][1][0], off, 0);
  };
  auto to_f64 = [&](const Row& xv, double (&x)[DPL]) {
#pragma unroll
    for (int e = 0; e < W4; ++e) {
      x[2 * e] = (double)__uint_as_float(xv.u[e] << 16);
      x[2 * e + 1] = (double)__uint_as_float(xv.u[e] & 0xffff0000u);
    }
  };
  // per-dimension block totals: acc[e] (dimension DPL*dg+e, this thread's
  // rows) summed over the wavefront's row groups, then over the wavefronts in
  // order
  auto store_totals = [&](int bh, int g, double (&acc)[DPL]) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      double x = acc[e];
      if (DG == 8) x += dpp_f64<0x128>(x);  // row_ror:8 = lane ^ 8 inside a 16-lane row
      x = add_xor16(x);
      x = add_xor32(x);
      acc[e] = x;
    }
    if (lane < DG) {
#pragma unroll
      for (int e = 0; e < DPL; ++e) part[w][DPL * dg + e] = acc[e];
    }
    __syncthreads();
    if (tid < D) {
      double tot = part[0][tid];
#pragma unroll
      for (int q = 1; q < NT / 64; ++q) tot += part[q][tid];
      p.partial[((size_t)bh * G + g) * D + tid] = tot;
    }
  };

  if ((int64_t)blockIdx.x >= nblk) return;
  Pos cur = {(int)(blockIdx.x / G), (int)(blockIdx.x % G)};
  Pos nxt = step(cur);
  Pos nxt2 = step(nxt);
  int s, m, s_n = 0, m_n = 0;
  node_of(G, p.level, cur.g, s, m);
  int idx_n[RPT];
  Row xr[RPT], xr_n[RPT];
  load_idx(cur, idx_n);
  wait_vm0();
  load_rows(cur, idx_n, xr);
  load_muv(cur, s, 0);
  if (nxt.bh < nbh) load_idx(nxt, idx_n);

  for (int it = 0; cur.bh < nbh; ++it) {
    wait_vm0();
    __syncthreads();
    const int buf = it & 1;
    // prefetch the next block (rows, mu / v) and the indices of the one after
    if (nxt.bh < nbh) {
      load_rows(nxt, idx_n, xr_n);
      node_of(G, p.level, nxt.g, s_n, m_n);
      load_muv(nxt, s_n, buf ^ 1);
      if (nxt2.bh < nbh) load_idx(nxt2, idx_n);
    }
    const int bh = cur.bh;
    const int g = cur.g;
    if (m >= 2) {
      if (STAGE == 0) {
        double acc[DPL];
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] = 0.0;
#pragma unroll
        for (int k = 0; k < RPT; ++k) {
          double x[DPL];
          to_f64(xr[k], x);
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc[e] += x[e];
        }
        store_totals(bh, g, acc);
      } else {
        double mu8[DPL], v8[DPL];
#pragma unroll
        for (int e = 0; e < DPL; ++e) {
          mu8[e] = muv[buf][0][DPL * dg + e];
          v8[e] = muv[buf][1][DPL * dg + e];
        }
        double c = 0.0;
#pragma unroll
        for (int e = 0; e < DPL; ++e) c = __builtin_fma(mu8[e], v8[e], c);
        // t_r = x_r . v - c summed over the DG lanes of row r
        double t[RPT];
#pragma unroll
        for (int k = 0; k < RPT; ++k) {
          double x[DPL];
          to_f64(xr[k], x);
          double a0 = 0.0, a1 = 0.0;
#pragma unroll
          for (int e = 0; e < DPL; e += 2) {
            a0 = __builtin_fma(x[e], v8[e], a0);
            a1 = __builtin_fma(x[e + 1], v8[e + 1], a1);
          }
          t[k] = group_sum<DG>((a0 + a1) - c);
        }
        if (dg == 0) {
          double* pr = p.proj + (size_t)bh * p.n_pad + (size_t)g * C;
#pragma unroll
          for (int k = 0; k < RPT; ++k) pr[rg + k * RG] = t[k];
        }
      }
    }
#pragma unroll
    for (int k = 0; k < RPT; ++k) xr[k] = xr_n[k];
    cur = nxt;
    nxt = nxt2;
    nxt2 = step(nxt2);
    s = s_n;
    m = m_n;
  }
}

// Node means when no power iterations run: mu = (sum of partials) / rows and
// v = v0 = 1/sqrt(D).  One workgroup of D*PARTS threads per node (PARTS
// chosen per depth from the largest node size): thread (d, part) sums the
// partials of groups s + part, s + part + PARTS, ... in that order
// (independent loads, one dependent add chain), then the PARTS sums of each d
// in order.
template <int D, int C, int PARTS>
__global__ __launch_bounds__(D * PARTS) void pddp_reduce_kernel(PddpParams p) {
  constexpr int NT = D * PARTS;
  __shared__ double part_sum[NT];
  const int G = p.groups;
  const int slots = 1 << p.level;
  const int64_t bh = blockIdx.x / slots;
  int s, m;
  if (!node_of_slot(G, p.level, blockIdx.x - (int)(bh * slots), s, m) || m < 2) return;
  const int tid = threadIdx.x;
  const int d = tid % D, part = tid / D;
  const double* src = p.partial + ((size_t)bh * G + s) * D + d;
  double acc = 0.0;
  int gg = part;
  for (; gg + 15 * PARTS < m; gg += 16 * PARTS) {
    double a[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) a[u] = src[(size_t)(gg + u * PARTS) * D];
#pragma unroll
    for (int u = 0; u < 16; ++u) acc += a[u];
  }
  for (; gg < m; gg += PARTS) acc += src[(size_t)gg * D];
  part_sum[tid] = acc;
  __syncthreads();
  if (tid < D) {
    double tot = part_sum[tid];
    for (int q = 1; q < PARTS; ++q) tot += part_sum[q * D + tid];
    p.mu[((size_t)bh * G + s) * D + tid] = tot / (double)(m * C);
    p.vec[((size_t)bh * G + s) * D + tid] = 1.0 / sqrt((double)D);
  }
}

template <int NT>
__device__ __forceinline__ int block_excl_scan_i(int v, int* sh, int* total) {
  constexpr int NWV = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[w] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NWV; ++i) {
    const int s = sh[i];
    base += (i < w) ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

__device__ __forceinline__ uint64_t order_key(double x) {
  if (x == 0.0) x = 0.0;  // -0 and +0 are the same value
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

template <int C>
__global__ __launch_bounds__(512) void pddp_split_kernel(PddpParams p) {
  constexpr int NT = 512;
  constexpr int NBIN = 2048;
  constexpr int BPT = NBIN / NT;
  __shared__ int hist[NBIN];
  __shared__ int scan_sh[NT / 64 + 1];
  __shared__ int found[2];
  const int G = p.groups;
  const int slots = 1 << p.level;
  const int64_t bh = blockIdx.x / slots;
  int s, m;
  if (!node_of_slot(G, p.level, blockIdx.x - (int)(bh * slots), s, m)) return;
  const int tid = threadIdx.x;
  const int32_t* pc = p.perm_cur + (size_t)bh * p.n_pad + (size_t)s * C;
  int32_t* pn = p.perm_next + (size_t)bh * p.n_pad + (size_t)s * C;
  if (m < 2) {
    for (int i = tid; i < C; i += NT) pn[i] = pc[i];
    return;
  }
  const int n = m * C;
  const int n_left = (m >> 1) * C;
  const double* pr = p.proj + (size_t)bh * p.n_pad + (size_t)s * C;

  // radix select of the n_left-th smallest key (1-based), digits from the top
  uint64_t prefix = 0ull, pmask = 0ull;
  int krem = n_left;
  const int shifts[6] = {53, 42, 31, 20, 9, 0};
  const int widths[6] = {11, 11, 11, 11, 11, 9};
#pragma unroll
  for (int pass = 0; pass < 6; ++pass) {
    const int sh = shifts[pass];
    const uint64_t dmask = (1ull << widths[pass]) - 1ull;
    for (int b = tid; b < NBIN; b += NT) hist[b] = 0;
    __syncthreads();
    // eight independent loads in flight per thread: the pass is bound by their
    // latency, not by the LDS atomics
    int i = tid;
    for (; i + 7 * NT < n; i += 8 * NT) {
      uint64_t u[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) u[e] = order_key(pr[i + e * NT]);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if ((u[e] & pmask) == prefix) atomicAdd(&hist[(int)((u[e] >> sh) & dmask)], 1);
    }
    for (; i < n; i += NT) {
      const uint64_t u = order_key(pr[i]);
      if ((u & pmask) == prefix) atomicAdd(&hist[(int)((u >> sh) & dmask)], 1);
    }
    __syncthreads();
    int loc[BPT];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      loc[i] = hist[BPT * tid + i];
      sum += loc[i];
    }
    int tot;
    int below = block_excl_scan_i<NT>(sum, scan_sh, &tot);
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      if (below < krem && below + loc[i] >= krem) {
        found[0] = BPT * tid + i;
        found[1] = krem - below;
      }
      below += loc[i];
    }
    __syncthreads();
    prefix |= (uint64_t)found[0] << sh;
    pmask |= dmask << sh;
    krem = found[1];
    __syncthreads();
  }
  const uint64_t T = prefix;
  // stable partition in position (= token) order
  constexpr int E = 2;
  int left_taken = 0, eq_seen = 0;
  for (int base = 0; base < n; base += NT * E) {
    uint64_t u[E];
    int neq = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = base + tid * E + e;
      u[e] = (i < n) ? order_key(pr[i]) : ~0ull;
      if (i < n && u[e] == T) ++neq;
    }
    int eq_tot;
    int eq_rank = eq_seen + block_excl_scan_i<NT>(neq, scan_sh, &eq_tot);
    bool lf[E];
    int nl = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = base + tid * E + e;
      bool l = false;
      if (i < n) {
        if (u[e] < T) {
          l = true;
        } else if (u[e] == T) {
          l = eq_rank < krem;
          ++eq_rank;
        }
      }
      lf[e] = l;
      nl += l ? 1 : 0;
    }
    int l_tot;
    int lpos = left_taken + block_excl_scan_i<NT>(nl, scan_sh, &l_tot);
    // right-child members before this thread: positions before it minus left ones
    int rpos = (base + tid * E) - lpos;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = base + tid * E + e;
      if (i < n) {
        if (lf[e]) {
          if (lpos < n_left) pn[lpos] = pc[i];
          ++lpos;
        } else {
          if (n_left + rpos < n) pn[n_left + rpos] = pc[i];
          ++rpos;
        }
      }
    }
    left_taken += l_tot;
    eq_seen += eq_tot;
  }
}

// ---- covariance path ----
// The power iteration runs on each node's centred covariance instead of on its
// rows:
//   Sigma = X^T X - n mu mu^T   (fp64, d x d, n = m*C rows, padding rows included)
// which is the same operator v -> sum_r ((x_r - mu) . v)(x_r - mu); the 20
// iterations then cost d^2 work per node instead of a pass over its rows each.
// X^T X and the row sum X^T 1 are additive over rows, so below the root only
// one child of every split is formed from its rows (the left one, the first
// floor(m/2) groups of the parent's segment, never larger than its sibling)
// and the other is the parent's minus it; the node mean comes from the row
// sum, so no separate mean pass is needed.
//
// A node's entry holds the upper-triangular 16 x 16 tiles of X^T X (I <= J,
// row-major inside a tile, tiles in row-major upper order) followed by the d
// row sums: GRAM_ENTRY(d) doubles.
//
// pddp_gram_kernel: one workgroup per (head, parent slot, chunk of GRAM_CH
// blocks of the left child; the root itself at depth 0); X^T X of the chunk's
// rows on v_mfma_f64_16x16x4_f64 and the row sums, written as a partial.
// pddp_gram_sum_kernel: the chunk partials of each left child summed in chunk
// order (depths whose left children span several chunks).
// pddp_gram_power_kernel: one workgroup per node; its entry (left child or
// root: the sum just formed; right child: parent entry minus left entry),
// kept for the next depth when the node will split again; the mean, the
// centred matrix held in registers, the power iterations (v0 = 1/sqrt(d), v
// kept when |Sigma v| = 0) and the sign rule.

template <int DT>
__host__ __device__ constexpr int gram_tile_i(int t) {
  int i = 0, len = DT;
  while (t >= len) {
    t -= len;
    ++i;
    --len;
  }
  return i;
}
template <int DT>
__host__ __device__ constexpr int gram_tile_j(int t) {
  int i = 0, len = DT;
  while (t >= len) {
    t -= len;
    ++i;
    --len;
  }
  return i + t;
}
// index of upper tile (I, J), I <= J, in row-major upper order
template <int DT>
__host__ __device__ constexpr int gram_tile_index(int I, int J) {
  return I * DT - (I * (I - 1)) / 2 + (J - I);
}

typedef double f64x4 __attribute__((ext_vector_type(4)));

// tile t = W + 4K of the wave's share: acc += X[:, 16I..] (A) x X[:, 16J..] (B)
template <int DT, int W, int K>
__device__ __forceinline__ void gram_mfma(const double (&xv)[DT], f64x4& acc) {
  constexpr int t = W + 4 * K;
  if constexpr (t < DT * (DT + 1) / 2) {
    constexpr int I = gram_tile_i<DT>(t);
    constexpr int J = gram_tile_j<DT>(t);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(xv[I], xv[J], acc, 0, 0, 0);
  }
}
template <int DT, int W, int... K>
__device__ __forceinline__ void gram_mfmas(const double (&xv)[DT], f64x4 (&acc)[sizeof...(K)],
                                           std::integer_sequence<int, K...>) {
  (gram_mfma<DT, W, K>(xv, acc[K]), ...);
}
// lane l holds D[i][j] of tile t for j = l % 16, i = l / 16 + 4r (r = 0..3);
// partial tile t is stored row-major (16 x 16)
template <int DT, int W, int K>
__device__ __forceinline__ void gram_store(double* dst, const f64x4& acc, int lane) {
  constexpr int t = W + 4 * K;
  if constexpr (t < DT * (DT + 1) / 2) {
    double* tile = dst + t * 256;
    static_assert(gram_tile_i<DT>(t) <= gram_tile_j<DT>(t), "upper tile");
#pragma unroll
    for (int r = 0; r < 4; ++r) tile[(lane / 16 + 4 * r) * 16 + (lane & 15)] = acc[r];
  }
}
template <int DT, int W, int... K>
__device__ __forceinline__ void gram_stores(double* dst, const f64x4 (&acc)[sizeof...(K)], int lane,
                                            std::integer_sequence<int, K...>) {
  (gram_store<DT, W, K>(dst, acc[K], lane), ...);
}

template <int D>
__host__ __device__ constexpr int gram_entry() {
  return (D / 16) * (D / 16 + 1) / 2 * 256 + D;
}

template <int D, int C, int W>
__device__ __forceinline__ void gram_body(const PddpParams& p, char (*rows)[64 * (2 * D + 32)],
                                          const int32_t* pc, const uint16_t* Qb, int nrows,
                                          double* dst) {
  constexpr int DT = D / 16, NT = DT * (DT + 1) / 2, TPW = (NT + 3) / 4;
  constexpr int SUB = 64;                 // rows staged in LDS at a time
  constexpr int PITCH = 2 * D + 32;       // bytes per staged row (rows 4 apart hit other banks)
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int LPT = SUB * CPR / 256;    // 16-byte loads per thread per stage
  const int tid = threadIdx.x, lane = tid & 63;
  f64x4 acc[TPW];
#pragma unroll
  for (int k = 0; k < TPW; ++k) acc[k] = (f64x4){0.0, 0.0, 0.0, 0.0};
  double sx[DT];  // wave 0: row sums of dimensions 16*blk + lane % 16, rows lane/16 + 4 st
#pragma unroll
  for (int blk = 0; blk < DT; ++blk) sx[blk] = 0.0;
  uint4 nx[LPT];
#pragma unroll
  for (int q = 0; q < LPT; ++q) {
    const int idx = tid + 256 * q;
    const int row = pc[idx / CPR];
    nx[q] = *(const uint4*)(Qb + (int64_t)row * p.sq.n + 8 * (idx % CPR));
  }
#pragma unroll
  for (int q = 0; q < LPT; ++q) {
    const int idx = tid + 256 * q;
    *(uint4*)(rows[0] + (idx / CPR) * PITCH + 16 * (idx % CPR)) = nx[q];
  }
  __syncthreads();
  for (int r0 = 0, it = 0; r0 < nrows; r0 += SUB, ++it) {
    const int buf = it & 1;
    // the next stage's rows (the last stage loads itself again: the unused
    // copy goes to the buffer no wave reads any more)
    const int rn = (r0 + SUB < nrows) ? r0 + SUB : r0;
#pragma unroll
    for (int q = 0; q < LPT; ++q) {
      const int idx = tid + 256 * q;
      const int row = pc[rn + idx / CPR];
      nx[q] = *(const uint4*)(Qb + (int64_t)row * p.sq.n + 8 * (idx % CPR));
    }
    const char* rb = rows[buf];
#pragma unroll 4
    for (int st = 0; st < SUB / 4; ++st) {
      // lane l: row 4*st + l/16 of the stage, dimension 16*blk + l%16
      const uint16_t* xr = (const uint16_t*)(rb + (4 * st + lane / 16) * PITCH) + (lane & 15);
      double xv[DT];
#pragma unroll
      for (int blk = 0; blk < DT; ++blk) xv[blk] = (double)bf16_to_f32(xr[16 * blk]);
      gram_mfmas<DT, W>(xv, acc, std::make_integer_sequence<int, TPW>{});
      if constexpr (W == 0) {
#pragma unroll
        for (int blk = 0; blk < DT; ++blk) sx[blk] += xv[blk];
      }
    }
#pragma unroll
    for (int q = 0; q < LPT; ++q) {
      const int idx = tid + 256 * q;
      *(uint4*)(rows[buf ^ 1] + (idx / CPR) * PITCH + 16 * (idx % CPR)) = nx[q];
    }
    __syncthreads();
  }
  gram_stores<DT, W>(dst, acc, lane, std::make_integer_sequence<int, TPW>{});
  if constexpr (W == 0) {
    // the four row lanes of each dimension (l, l^16, l^32, l^48), fixed order
#pragma unroll
    for (int blk = 0; blk < DT; ++blk) {
      const double x = add_xor32(add_xor16(sx[blk]));
      if (lane < 16) dst[NT * 256 + 16 * blk + lane] = x;
    }
  }
}

// Slots of the nodes whose left children are formed at `level` (1 at the
// root depth, else the parent depth's 2^(level-1)).
__device__ __forceinline__ int gram_parent_slots(int level) { return level == 0 ? 1 : 1 << (level - 1); }

// Rows formed for parent slot ps at `level`: the root (level 0), else the
// left child of a parent of m >= 3 groups (m = 2 splits into two leaves,
// which need no covariance).  Returns false if there is nothing to form.
__device__ __forceinline__ bool gram_formed_node(int G, int level, int ps, int& s, int& m) {
  if (level == 0) {
    s = 0;
    m = G;
    return m >= 2;
  }
  if (!node_of_slot(G, level - 1, ps, s, m) || m < 3) return false;
  m >>= 1;
  return true;
}

template <int D, int C>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) void pddp_gram_kernel(
    PddpParams p) {
  constexpr int E = gram_entry<D>();
  __shared__ __attribute__((aligned(16))) char rows[2][64 * (2 * D + 32)];
  const int G = p.groups;
  const int pslots = gram_parent_slots(p.level);
  const int per_bh = pslots * p.nch;
  const int bh = blockIdx.x / per_bh;
  const int rem = blockIdx.x - bh * per_bh;
  const int ps = rem / p.nch, j = rem - ps * p.nch;
  int s, m;
  if (!gram_formed_node(G, p.level, ps, s, m)) return;
  const int b0 = j * GRAM_CH;
  if (b0 >= m) return;
  const int nrows = (min(b0 + GRAM_CH, m) - b0) * C;
  const int32_t* pc = p.perm_cur + (int64_t)bh * p.n_pad + (int64_t)(s + b0) * C;
  const uint16_t* Qb = p.q + head_offset(p.sq, bh, p.heads);
  double* dst = p.gram + ((int64_t)(bh * pslots + ps) * p.nch + j) * E;
  switch (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) {
    case 0: gram_body<D, C, 0>(p, rows, pc, Qb, nrows, dst); break;
    case 1: gram_body<D, C, 1>(p, rows, pc, Qb, nrows, dst); break;
    case 2: gram_body<D, C, 2>(p, rows, pc, Qb, nrows, dst); break;
    default: gram_body<D, C, 3>(p, rows, pc, Qb, nrows, dst); break;
  }
}

// Sum of a formed node's chunk partials, in chunk order, written over chunk 0
// (one workgroup per (head, parent slot, segment): a segment is one tile of
// 256 entries or the d row sums; each thread owns one entry, so reading every
// chunk's value and then writing chunk 0's is safe in place).
template <int D>
__global__ __launch_bounds__(256) void pddp_gram_sum_kernel(PddpParams p) {
  constexpr int DT = D / 16, NT = DT * (DT + 1) / 2, E = gram_entry<D>();
  const int G = p.groups;
  const int pslots = gram_parent_slots(p.level);
  const int per_bh = pslots * (NT + 1);
  const int bh = blockIdx.x / per_bh;
  const int rem = blockIdx.x - bh * per_bh;
  const int ps = rem / (NT + 1), seg = rem - ps * (NT + 1);
  int s, m;
  if (!gram_formed_node(G, p.level, ps, s, m)) return;
  const int nck = (m + GRAM_CH - 1) / GRAM_CH;
  if (nck < 2 || (int)threadIdx.x >= (seg < NT ? 256 : D)) return;
  double* src = p.gram + (int64_t)(bh * pslots + ps) * p.nch * E + seg * 256 + threadIdx.x;
  double a = 0.0;
  int k = 0;
  for (; k + 8 <= nck; k += 8) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = src[(int64_t)(k + u) * E];
#pragma unroll
    for (int u = 0; u < 8; ++u) a += v[u];
  }
  for (; k < nck; ++k) a += src[(int64_t)k * E];
  src[0] = a;
}

// One workgroup of 256 threads per node.  The node's entry is staged through
// LDS (coalesced loads, one tile of 256 values per pass; inside a tile, entry
// (r, c) sits at r*16 + (c ^ r), so both the row reads and the mirrored column
// reads below are free of bank conflicts).  Thread (i, part), i = t % D, part
// = t / D, then holds row i, columns part*D/PARTS .. +D/PARTS-1 of the centred
// matrix in registers (64 values for d = 128, 16 for d = 64); upper tiles are
// read along their rows, lower ones as the mirrored upper tile's columns.
// One step: each thread's partial dot product with v (four interleaved
// accumulators, v read from LDS as a broadcast), the PARTS partials of row i
// summed in part order, |w|^2 summed over the wavefronts of part 0 (lane
// moves in the VALU, then the wavefronts in order), v = w / |w|.
template <int D, int C>
__global__ __launch_bounds__(256) void pddp_gram_power_kernel(PddpParams p) {
  constexpr int DT = D / 16, NT = DT * (DT + 1) / 2, E = gram_entry<D>();
  constexpr int PARTS = 256 / D, CW = D / PARTS, NWD = (D + 63) / 64;
  constexpr int P2 = D <= 64 ? 64 : 128;  // sign rule: tree over the next power of two
  static_assert(CW % 16 == 0 && CW * PARTS == D, "columns per thread");
  __shared__ double stage[NT * 256];   // the entry's tiles; later the sign rule's scratch
  __shared__ double vec[D];
  __shared__ double mus[D];
  __shared__ double red[PARTS - 1][D];
  __shared__ double nrm[NWD];
  const int G = p.groups;
  const int slots = 1 << p.level;
  const int bh = blockIdx.x / slots;
  const int slot = blockIdx.x - bh * slots;
  int s, m;
  if (!node_of_slot(G, p.level, slot, s, m) || m < 2) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // threads past PARTS*D (d = 96: the last 64) hold no matrix entries
  const int i = tid % D, part = tid / D;
  const bool active = part < PARTS;
  const int c0 = active ? part * CW : 0;
  // the node's entry: formed from its rows (root, left child), or the
  // parent's entry minus the left sibling's (right child)
  const int pslots = gram_parent_slots(p.level);
  const int ps = (p.level == 0) ? 0 : (slot >> 1);
  const double* a_src = p.gram + (int64_t)(bh * pslots + ps) * p.nch * E;
  const double* par_src =
      (p.level > 0 && (slot & 1)) ? p.gnode_prev + (int64_t)(bh * pslots + ps) * E : nullptr;
  // kept for the next depth if this node splits into children that need it
  double* keep = (p.gram_store && m >= 3) ? p.gnode_cur + (int64_t)(bh * slots + slot) * E : nullptr;
  const double n = (double)(m * C);
  double* mu = p.mu + ((size_t)bh * G + s) * D;
  double* vv = p.vec + ((size_t)bh * G + s) * D;
  {
    double x[NT];
#pragma unroll
    for (int k = 0; k < NT; ++k) x[k] = a_src[k * 256 + tid];
    if (par_src != nullptr) {
#pragma unroll
      for (int k = 0; k < NT; ++k) x[k] = par_src[k * 256 + tid] - x[k];
    }
    if (keep != nullptr) {
#pragma unroll
      for (int k = 0; k < NT; ++k) keep[k * 256 + tid] = x[k];
    }
    const int r = tid >> 4, c = tid & 15;
#pragma unroll
    for (int k = 0; k < NT; ++k) stage[k * 256 + r * 16 + (c ^ r)] = x[k];
  }
  if (tid < D) {
    double sx = a_src[NT * 256 + tid];
    if (par_src != nullptr) sx = par_src[NT * 256 + tid] - sx;
    if (keep != nullptr) keep[NT * 256 + tid] = sx;
    const double mv = sx / n;
    mus[tid] = mv;
    mu[tid] = mv;
    vec[tid] = 1.0 / sqrt((double)D);
  }
  __syncthreads();
  double sg[CW];
  {
    const int I = i >> 4, ii = i & 15;
#pragma unroll
    for (int jb = 0; jb < CW / 16; ++jb) {
      const int J = (c0 >> 4) + jb;
      if (I <= J) {
        // row ii of upper tile (I, J)
        const double* t = stage + gram_tile_index<DT>(I, J) * 256 + ii * 16;
#pragma unroll
        for (int c = 0; c < 16; ++c) sg[jb * 16 + c] = t[c ^ ii];
      } else {
        // column ii of upper tile (J, I)
        const double* t = stage + gram_tile_index<DT>(J, I) * 256;
#pragma unroll
        for (int c = 0; c < 16; ++c) sg[jb * 16 + c] = t[c * 16 + (ii ^ c)];
      }
    }
    const double ni = n * mus[i];
#pragma unroll
    for (int c = 0; c < CW; ++c) sg[c] = sg[c] - ni * mus[c0 + c];
  }
  for (int it = 0; it < p.power_iters; ++it) {
    double a[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int c = 0; c < CW; c += 4) {
#pragma unroll
      for (int u = 0; u < 4; ++u) a[u] = __builtin_fma(sg[c + u], vec[c0 + c + u], a[u]);
    }
    const double pw = (a[0] + a[1]) + (a[2] + a[3]);
    if (part > 0 && active) red[part - 1][i] = pw;
    __syncthreads();
    double wv = pw;
    if (part == 0) {
#pragma unroll
      for (int q = 1; q < PARTS; ++q) wv += red[q - 1][i];
    }
    // |w|^2 over the rows held by part 0 (whole wavefronts take part; the
    // others add zeros)
    if (w < NWD) {
      const double q2 = add_xor32(add_xor16(group_sum<16>(part == 0 ? wv * wv : 0.0)));
      if (lane == 0) nrm[w] = q2;
    }
    __syncthreads();
    double nrm2 = nrm[0];
#pragma unroll
    for (int q = 1; q < NWD; ++q) nrm2 += nrm[q];
    if (part == 0 && nrm2 > 0.0) vec[i] = wv / sqrt(nrm2);
    __syncthreads();
  }
  // sign rule: the component of largest magnitude (first on ties) positive
  double* vmag = stage;
  int* vidx = reinterpret_cast<int*>(stage + P2);
  double nv = (tid < D) ? vec[tid] : 0.0;
  if (tid < P2) {
    vmag[tid] = (tid < D) ? fabs(nv) : -1.0;  // padding entries never win
    vidx[tid] = tid;
  }
  __syncthreads();
  for (int o = P2 / 2; o > 0; o >>= 1) {
    if (tid < o) {
      const double x = vmag[tid], y = vmag[tid + o];
      const int ix = vidx[tid], iy = vidx[tid + o];
      if (y > x || (y == x && iy < ix)) {
        vmag[tid] = y;
        vidx[tid] = iy;
      }
    }
    __syncthreads();
  }
  if (tid == vidx[0]) nrm[0] = nv;
  __syncthreads();
  if (nrm[0] < 0.0) nv = -nv;
  if (tid < D) vv[tid] = nv;
}

hipError_t launch_pddp_identity(const PddpParams& p, hipStream_t s) {
  const int64_t total = p.bh * (int64_t)p.n_pad;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(pddp_identity_kernel, dim3(blocks), dim3(256), 0, s, p.perm_cur, p.n_pad, total);
  return hipGetLastError();
}

// Grid of a persistent kernel: as many workgroups as are resident at once on
// the current device (at most `work`).
template <typename K>
static unsigned resident_grid(K kernel, int threads, int64_t work) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
      cus < 1 || per_cu < 1) {
    cus = 1;
    per_cu = 1;
  }
  const int64_t r = (int64_t)cus * per_cu;
  return (unsigned)(work < r ? work : r);
}

template <int D, int C, int STAGE>
static hipError_t partial_one(const PddpParams& p, hipStream_t s) {
  const int64_t work = p.bh * (int64_t)p.groups;
  const unsigned grid = resident_grid(pddp_partial_kernel<D, C, STAGE>, 256, work);
  hipLaunchKernelGGL((pddp_partial_kernel<D, C, STAGE>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int D, int C>
static hipError_t partial_t(int stage, const PddpParams& p, hipStream_t s) {
  if (stage == 0) return partial_one<D, C, 0>(p, s);
  if (stage == 2) return partial_one<D, C, 2>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_pddp_partial(int d, int c, int stage, const PddpParams& p, hipStream_t s) {
  if (d == 128 && c == 128) return partial_t<128, 128>(stage, p, s);
  if (d == 128 && c == 64) return partial_t<128, 64>(stage, p, s);
  if (d == 96 && c == 128) return partial_t<96, 128>(stage, p, s);
  if (d == 96 && c == 64) return partial_t<96, 64>(stage, p, s);
  if (d == 64 && c == 128) return partial_t<64, 128>(stage, p, s);
  if (d == 64 && c == 64) return partial_t<64, 64>(stage, p, s);
  return hipErrorInvalidValue;
}

template <int D, int C>
static hipError_t mean_t(const PddpParams& p, hipStream_t s) {
  // about 8 partials per thread for the largest node of this depth
  const int m_max = (p.groups + (1 << p.level) - 1) >> p.level;
  int parts = 1;
  while (parts < 1024 / D && parts < 8 && parts * 8 < m_max) parts *= 2;
  const dim3 grid((unsigned)(p.bh << p.level));
  switch (parts) {
    case 1: hipLaunchKernelGGL((pddp_reduce_kernel<D, C, 1>), grid, dim3(D), 0, s, p); break;
    case 2: hipLaunchKernelGGL((pddp_reduce_kernel<D, C, 2>), grid, dim3(D * 2), 0, s, p); break;
    case 4: hipLaunchKernelGGL((pddp_reduce_kernel<D, C, 4>), grid, dim3(D * 4), 0, s, p); break;
    default: hipLaunchKernelGGL((pddp_reduce_kernel<D, C, 8>), grid, dim3(D * 8), 0, s, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_pddp_mean(int d, int c, const PddpParams& p, hipStream_t s) {
  if (d == 128 && c == 128) return mean_t<128, 128>(p, s);
  if (d == 128 && c == 64) return mean_t<128, 64>(p, s);
  if (d == 96 && c == 128) return mean_t<96, 128>(p, s);
  if (d == 96 && c == 64) return mean_t<96, 64>(p, s);
  if (d == 64 && c == 128) return mean_t<64, 128>(p, s);
  if (d == 64 && c == 64) return mean_t<64, 64>(p, s);
  return hipErrorInvalidValue;
}

template <int D, int C>
static hipError_t gram_t(const PddpParams& p, hipStream_t s) {
  const int pslots = p.level == 0 ? 1 : 1 << (p.level - 1);
  hipLaunchKernelGGL((pddp_gram_kernel<D, C>), dim3((unsigned)(p.bh * pslots * p.nch)), dim3(256), 0, s, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nch < 2) return e;
  constexpr int nt = (D / 16) * (D / 16 + 1) / 2;
  hipLaunchKernelGGL((pddp_gram_sum_kernel<D>), dim3((unsigned)(p.bh * pslots * (nt + 1))), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_pddp_gram(int d, int c, const PddpParams& p, hipStream_t s) {
  if (d == 128 && c == 128) return gram_t<128, 128>(p, s);
  if (d == 128 && c == 64) return gram_t<128, 64>(p, s);
  if (d == 96 && c == 128) return gram_t<96, 128>(p, s);
  if (d == 96 && c == 64) return gram_t<96, 64>(p, s);
  if (d == 64 && c == 128) return gram_t<64, 128>(p, s);
  if (d == 64 && c == 64) return gram_t<64, 64>(p, s);
  return hipErrorInvalidValue;
}

template <int D, int C>
static hipError_t power_t(const PddpParams& p, hipStream_t s) {
  hipLaunchKernelGGL((pddp_gram_power_kernel<D, C>), dim3((unsigned)(p.bh * ((int64_t)1 << p.level))), dim3(256),
                     0, s, p);
  return hipGetLastError();
}

hipError_t launch_pddp_gram_power(int d, int c, const PddpParams& p, hipStream_t s) {
  if (d == 128 && c == 128) return power_t<128, 128>(p, s);
  if (d == 128 && c == 64) return power_t<128, 64>(p, s);
  if (d == 96 && c == 128) return power_t<96, 128>(p, s);
  if (d == 96 && c == 64) return power_t<96, 64>(p, s);
  if (d == 64 && c == 128) return power_t<64, 128>(p, s);
  if (d == 64 && c == 64) return power_t<64, 64>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_pddp_split(int c, const PddpParams& p, hipStream_t s) {
  const dim3 grid((unsigned)(p.bh << p.level));
  if (c == 128) hipLaunchKernelGGL((pddp_split_kernel<128>), grid, dim3(512), 0, s, p);
  else if (c == 64) hipLaunchKernelGGL((pddp_split_kernel<64>), grid, dim3(512), 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace mcs
