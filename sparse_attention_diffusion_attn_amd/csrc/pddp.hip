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
// reduction has a fixed order and results are bitwise reproducible.  The split
// is an exact radix select on the fp64 projections (64-bit order-preserving
// keys, ties broken by position = token index) followed by a stable partition.
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

// stage 0: partial[g] = sum of the block's rows
// stage 1: partial[g] = sum_r ((x_r - mu) . v) (x_r - mu)
// stage 2: proj[pos] = (x_r - mu) . v', v' = v with its sign fixed
template <int D, int C, int STAGE>
__global__ __launch_bounds__(256) void pddp_partial_kernel(PddpParams p) {
  constexpr int NT = 256;
  // thread (dg, rg) works on dimensions 8dg .. 8dg+7 of rows rg, rg+RG, ...
  constexpr int DG = D / 8, RG = NT / DG, RPT = C / RG;
  constexpr int TP = DG + 1;  // padded row of per-row partial dot products
  __shared__ __attribute__((aligned(16))) uint16_t xs[C * D];
  __shared__ double mus[D], vs[D];
  __shared__ double ts[C];
  __shared__ double part[(C * TP > RG * D) ? C * TP : RG * D];
  __shared__ int flip;

  const int G = p.groups;
  const int work = blockIdx.x;
  const int64_t bh = work / G;
  const int g = work - (int)(bh * G);
  int s, m;
  node_of(G, p.level, g, s, m);
  if (m < 2) return;
  const int tid = threadIdx.x;
  const int dg = tid % DG, rg = tid / DG;
  const int32_t* pc = p.perm_cur + (size_t)bh * p.n_pad + (size_t)g * C;
  const uint16_t* Qb = p.q + (size_t)bh * p.n_pad * D;

  // stage the block's C rows (bf16) in LDS: all row indices first, then all
  // 16-byte loads, then the LDS stores (one round trip for each)
  {
    constexpr int NL = C * D / 8 / NT;
    int rows[NL];
#pragma unroll
    for (int k = 0; k < NL; ++k) rows[k] = pc[(tid + k * NT) / (D / 8)];
    uint4 vals[NL];
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const int c8 = (tid + k * NT) % (D / 8);
      vals[k] = *(const uint4*)(Qb + (size_t)rows[k] * D + c8 * 8);
    }
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const int e = tid + k * NT;
      *(uint4*)(xs + (e / (D / 8)) * D + (e % (D / 8)) * 8) = vals[k];
    }
  }
  if (STAGE > 0) {
    const double* mu = p.mu + ((size_t)bh * G + s) * D;
    const double* vv = p.vec + ((size_t)bh * G + s) * D;
    for (int d = tid; d < D; d += NT) {
      mus[d] = mu[d];
      vs[d] = vv[d];
    }
  }
  __syncthreads();

  // eight bf16 of row r, dimensions 8dg .. 8dg+7, as doubles
  auto row8 = [&](int r, double (&x)[8]) {
    const uint4 xv = *(const uint4*)(xs + r * D + 8 * dg);
    const uint32_t w4[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = (double)__uint_as_float(w4[e] << 16);
      x[2 * e + 1] = (double)__uint_as_float(w4[e] & 0xffff0000u);
    }
  };
  // column partials part[rg][d] -> fixed-order sum over rg, for d = tid < D
  auto column_total = [&]() {
    double tot = 0.0;
    if (tid < D) {
      tot = part[tid];
      for (int q = 1; q < RG; ++q) tot += part[q * D + tid];
    }
    return tot;
  };

  if (STAGE == 0) {
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      double x[8];
      row8(rg + k * RG, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += x[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[rg * D + 8 * dg + e] = acc[e];
    __syncthreads();
    const double tot = column_total();
    if (tid < D) p.partial[((size_t)bh * G + g) * D + tid] = tot;
    return;
  }

  if (STAGE == 2) {
    if (tid == 0) {
      int best = 0;
      double bv = fabs(vs[0]);
      for (int d = 1; d < D; ++d) {
        const double a = fabs(vs[d]);
        if (a > bv) { bv = a; best = d; }
      }
      flip = vs[best] < 0.0 ? 1 : 0;
    }
    __syncthreads();
    if (flip) {
      for (int d = tid; d < D; d += NT) vs[d] = -vs[d];
    }
    __syncthreads();
  }

  double mu8[8], v8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    mu8[e] = mus[8 * dg + e];
    v8[e] = vs[8 * dg + e];
  }
  // t_r = (x_r - mu) . v: partial dot products over each thread's 8
  // dimensions, then a fixed-order sum over the DG partials of each row
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    const int r = rg + k * RG;
    double x[8];
    row8(r, x);
    double a0 = 0.0, a1 = 0.0;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      a0 = __builtin_fma(x[e] - mu8[e], v8[e], a0);
      a1 = __builtin_fma(x[e + 1] - mu8[e + 1], v8[e + 1], a1);
    }
    part[r * TP + dg] = a0 + a1;
  }
  __syncthreads();
  if (tid < C) {
    double t = part[tid * TP];
    for (int q = 1; q < DG; ++q) t += part[tid * TP + q];
    ts[tid] = t;
  }
  __syncthreads();
  if (STAGE == 2) {
    if (tid < C) p.proj[(size_t)bh * p.n_pad + (size_t)g * C + tid] = ts[tid];
    return;
  }
  // w_d = sum_r t_r (x_rd - mu_d)
  {
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int r = rg + k * RG;
      const double t = ts[r];
      double x[8];
      row8(r, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = __builtin_fma(t, x[e] - mu8[e], acc[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[rg * D + 8 * dg + e] = acc[e];
    __syncthreads();
    const double tot = column_total();
    if (tid < D) p.partial[((size_t)bh * G + g) * D + tid] = tot;
  }
}

// stage 0: mu = (sum of partials) / rows, v = v0 = 1/sqrt(D)
// stage 1: w = sum of partials; v = w / |w| if |w| > 0
template <int D, int C, int STAGE>
__global__ __launch_bounds__(256) void pddp_reduce_kernel(PddpParams p) {
  constexpr int NT = 256;
  constexpr int PARTS = NT / D;
  __shared__ double part_sum[NT];
  __shared__ double sq[NT];
  const int G = p.groups;
  const int slots = 1 << p.level;
  const int64_t bh = blockIdx.x / slots;
  int s, m;
  if (!node_of_slot(G, p.level, blockIdx.x - (int)(bh * slots), s, m) || m < 2) return;
  const int tid = threadIdx.x;
  const int d = tid % D, part = tid / D;
  // groups s + part, s + part + PARTS, ... in order
  double acc = 0.0;
  for (int gg = s + part; gg < s + m; gg += PARTS) acc += p.partial[((size_t)bh * G + gg) * D + d];
  part_sum[tid] = acc;
  __syncthreads();
  double tot = 0.0;
  if (tid < D) {
    tot = part_sum[tid];
    for (int q = 1; q < PARTS; ++q) tot += part_sum[q * D + tid];
  }
  double* mu = p.mu + ((size_t)bh * G + s) * D;
  double* vv = p.vec + ((size_t)bh * G + s) * D;
  if (STAGE == 0) {
    if (tid < D) {
      mu[tid] = tot / (double)(m * C);
      vv[tid] = 1.0 / sqrt((double)D);
    }
    return;
  }
  sq[tid] = (tid < D) ? tot * tot : 0.0;
  __syncthreads();
  for (int o = NT / 2; o > 0; o >>= 1) {
    if (tid < o) sq[tid] += sq[tid + o];
    __syncthreads();
  }
  const double nrm2 = sq[0];
  if (tid < D && nrm2 > 0.0) vv[tid] = tot / sqrt(nrm2);
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
    for (int i = tid; i < n; i += NT) {
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

hipError_t launch_pddp_identity(const PddpParams& p, hipStream_t s) {
  const int64_t total = p.bh * (int64_t)p.n_pad;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(pddp_identity_kernel, dim3(blocks), dim3(256), 0, s, p.perm_cur, p.n_pad, total);
  return hipGetLastError();
}

template <int D, int C>
static hipError_t partial_t(int stage, const PddpParams& p, hipStream_t s) {
  const dim3 grid((unsigned)(p.bh * p.groups));
  if (stage == 0) hipLaunchKernelGGL((pddp_partial_kernel<D, C, 0>), grid, dim3(256), 0, s, p);
  else if (stage == 1) hipLaunchKernelGGL((pddp_partial_kernel<D, C, 1>), grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL((pddp_partial_kernel<D, C, 2>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_pddp_partial(int d, int c, int stage, const PddpParams& p, hipStream_t s) {
  if (d == 128 && c == 128) return partial_t<128, 128>(stage, p, s);
  if (d == 128 && c == 64) return partial_t<128, 64>(stage, p, s);
  if (d == 64 && c == 128) return partial_t<64, 128>(stage, p, s);
  if (d == 64 && c == 64) return partial_t<64, 64>(stage, p, s);
  return hipErrorInvalidValue;
}

template <int D, int C>
static hipError_t reduce_t(int stage, const PddpParams& p, hipStream_t s) {
  const dim3 grid((unsigned)(p.bh << p.level));
  if (stage == 0) hipLaunchKernelGGL((pddp_reduce_kernel<D, C, 0>), grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL((pddp_reduce_kernel<D, C, 1>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_pddp_reduce(int d, int c, int stage, const PddpParams& p, hipStream_t s) {
  if (d == 128 && c == 128) return reduce_t<128, 128>(stage, p, s);
  if (d == 128 && c == 64) return reduce_t<128, 64>(stage, p, s);
  if (d == 64 && c == 128) return reduce_t<64, 128>(stage, p, s);
  if (d == 64 && c == 64) return reduce_t<64, 64>(stage, p, s);
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
