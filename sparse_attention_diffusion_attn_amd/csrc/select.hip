// Anchor pass 2 of the two-pass exact selection (onedev.kr summary, "how it is
// used", component 3: the dense kernel does not expose its logits, so a second
// pass recomputes them and turns them into exact probabilities) and the
// per-group token-level top-k ("how it is used", component 1).
//
// score_kernel: one workgroup per (head, group).  The group's C query rows are
// gathered by perm and held in VGPRs; all key tiles stream through the same
// double-buffered LDS tile as the attention kernel.  S = Q . K^T runs on
// v_mfma_f32_32x32x16_bf16 with each lane owning one key column, so the sum
// over the group's queries of exp(s_ij - lse_i) is 16 in-register adds, one
// lane exchange and a fixed-order add of the wavefronts' partials in LDS.
//
// topk_kernel: one workgroup per (head, group).  Exact radix select on the
// fp32 bit patterns of the non-negative scores (10/11/11-bit digits, LDS
// histograms with integer atomics), then an order-preserving compaction that
// keeps every key above the threshold and the lowest-index keys equal to it,
// written in ascending key order.  Integer counts only, so it is exact and
// deterministic.
#include "mcs_common.h"
#include "mcs_internal.h"

namespace mcs {

template <int D, int C>
__global__ __launch_bounds__(256) void score_kernel(ScoreParams p) {
  // Four wavefronts.  C = 128: one per 32-query block.  C = 64 (SPLIT): two
  // per 32-query block, one per 32-key half of every tile.
  static_assert(C == 128 || C == 64, "group size");
  constexpr bool SPLIT = (C == 64);
  constexpr int NW = 4;
  constexpr int NRB = C / 32;          // 32-query blocks
  constexpr int KT = 64;
  constexpr int NPL = D / 32;
  constexpr int TILE = NPL * 4096;
  constexpr int IPM = TILE / 1024;
  constexpr int IPW = IPM / NW;
  constexpr int KS = D / 16;

  __shared__ __attribute__((aligned(1024))) char lds[2 * TILE];
  __shared__ float red[2][NRB][KT];
  __shared__ int hist_s[1024];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ql = lane & 31;
  const int h = lane >> 5;
  const int rb = SPLIT ? (w & 1) : w;   // this wavefront's 32-query block
  const int kh = SPLIT ? (w >> 1) : 0;  // its 32-key half of each tile (SPLIT)

  const int G = p.groups;
  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t bl = work / G;               // head within this chunk
  const int g = work - (int)(bl * G);
  const int64_t bh = p.bh0 + bl;
  const uint16_t* Qb = p.q + head_offset(p.sq, bh, p.heads);
  const uint16_t* Kb = p.k + head_offset(p.sk, bh, p.heads);
  const int32_t* permb = p.perm + (size_t)bh * p.n_pad + (size_t)g * C;

  // A operand of S = Q K^T: this lane's query row 32rb + ql.  A perm entry
  // outside 0 .. n_pad-1 is never used as an address: its lane reads row 0,
  // and below it counts as a padding row (no term in the scores).
  const int qraw = permb[32 * rb + ql];
  const int qrow = ((uint32_t)qraw < (uint32_t)p.n_pad) ? qraw : 0;
  bf16x8 qreg[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk)
    qreg[kk] = *(const bf16x8*)(Qb + (int64_t)qrow * p.sq.n + 16 * kk + 8 * h);

  // Accumulator j of S holds query 32rb + 8(j/4) + 4h + (j%4): its lse in log2
  // units (+inf for padded queries, whose terms then vanish).
  float lse2[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int r = permb[32 * rb + 8 * (j >> 2) + 4 * h + (j & 3)];
    lse2[j] = ((uint32_t)r < (uint32_t)p.n_valid) ? p.lse[(size_t)bh * p.n_pad + r] * kLog2e : INFINITY;
  }

  const int nk = p.n_valid;
  const int ntiles = (nk + KT - 1) / KT;
  // Copy instruction ins = w*IPW + i fills plane ins/4, rows 16*(ins%4) + l/4
  // (lane l), physical chunk l%4 = logical chunk (l%4)^((l/16)%4); rows are
  // read through a buffer resource with 32-bit offsets (row * row stride),
  // the per-instruction part of the offset in a scalar register.
  const uint32_t rsb = (uint32_t)p.sk.n * 2u;  // row stride of K in bytes
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(Kb, head_span_bytes(p.sk, p.n_pad, D));
  const uint32_t lane_off = (uint32_t)(lane >> 2) * rsb + 16u * (uint32_t)((lane ^ (lane >> 4)) & 3);
  auto issue = [&](int t, int buf) {
    char* kdst = lds + buf * TILE + w * IPW * 1024;
    const uint32_t voff = (uint32_t)(t * KT) * rsb + lane_off;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int ins = w * IPW + i;
      const uint32_t soff = (uint32_t)(16 * (ins & 3)) * rsb + 64u * (uint32_t)(ins >> 2);
      gather16_buf(krs, kdst + i * 1024, voff, soff);
    }
  };
  const int sq = (ql >> 2) & 3;
  const int koff_e = ql * 64 + ((h ^ sq) << 4);
  const int koff_o = ql * 64 + (((2 + h) ^ sq) << 4);
  const float c2 = p.scale * kLog2e;
  float* out = p.scores + ((size_t)bl * G + g) * (size_t)nk;

  // Column sums of tile t are finished (fixed wavefront order) by the first
  // KT threads after the barrier at the top of tile t+1; the partials are
  // double-buffered so one barrier per tile suffices.
  // With p.hist, the top 10 bits of every score (its fp32 pattern; scores are
  // >= 0) are also counted, so the top-k pass can skip its first scan.
  const bool want_hist = p.hist != nullptr;
  if (want_hist) {
    for (int b = threadIdx.x; b < 1024; b += blockDim.x) hist_s[b] = 0;
  }
  auto finish = [&](int t) {
    if (threadIdx.x < KT) {
      const int key = t * KT + threadIdx.x;
      float a = red[t & 1][0][threadIdx.x];
#pragma unroll
      for (int ww = 1; ww < NRB; ++ww) a += red[t & 1][ww][threadIdx.x];
      if (key < nk) {
        out[key] = a;
        if (want_hist) atomicAdd(&hist_s[__float_as_uint(a) >> 22], 1);
      }
    }
  };

  issue(0, 0);
  for (int t = 0; t < ntiles; ++t) {
    wait_vm0();
    __syncthreads();
    if (t > 0) finish(t - 1);
    // the copies of tile t+1 are spread over the k-steps of tile t
    const bool more = t + 1 < ntiles;
    char* kdst_n = lds + ((t + 1) & 1) * TILE + w * IPW * 1024;
    const uint32_t voff_n = (uint32_t)((t + 1) * KT) * rsb + lane_off;
    const char* kbuf = lds + (t & 1) * TILE;
    f32x16 s0, s1;
#pragma unroll
    for (int j = 0; j < 16; ++j) { s0[j] = 0.f; s1[j] = 0.f; }
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const char* kp = kbuf + ((kk & 1) ? koff_o : koff_e) + (kk >> 1) * 4096;
      const bf16x8 b0 = *(const bf16x8*)(kp + kh * 2048);
      s0 = mfma32(qreg[kk], b0, s0);
      if (!SPLIT) {
        const bf16x8 b1 = *(const bf16x8*)(kp + 2048);
        s1 = mfma32(qreg[kk], b1, s1);
      }
      if (more) {
        constexpr int PER = (IPW + KS - 1) / KS;
#pragma unroll
        for (int i = kk * PER; i < (kk + 1) * PER && i < IPW; ++i) {
          const int ins = w * IPW + i;
          const uint32_t soff = (uint32_t)(16 * (ins & 3)) * rsb + 64u * (uint32_t)(ins >> 2);
          gather16_buf(krs, kdst_n + i * 1024, voff_n, soff);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      a0 += __builtin_amdgcn_exp2f(__builtin_fmaf(s0[j], c2, -lse2[j]));
      if (!SPLIT) a1 += __builtin_amdgcn_exp2f(__builtin_fmaf(s1[j], c2, -lse2[j]));
    }
    a0 = sum_xor32(a0);
    if (!SPLIT) a1 = sum_xor32(a1);
    if (h == 0) {
      red[t & 1][rb][32 * kh + ql] = a0;
      if (!SPLIT) red[t & 1][rb][32 + ql] = a1;
    }
  }
  __syncthreads();
  finish(ntiles - 1);
  if (want_hist) {
    __syncthreads();
    int32_t* hg = p.hist + ((size_t)bl * G + g) * 1024;
    for (int b = threadIdx.x; b < 1024; b += blockDim.x) hg[b] = hist_s[b];
  }
}

// ---------------------------------------------------------------------------
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* sh, int* total) {
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

template <int NT>
__global__ __launch_bounds__(NT) void topk_kernel(TopkParams p) {
  constexpr int NBIN = 2048;
  constexpr int BPT = NBIN / NT;  // bins per thread
  __shared__ int hist[NBIN];
  __shared__ int scan_sh[NT / 64 + 1];
  __shared__ int found[2];

  const int G = p.groups;
  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t bl = work / G;
  const int g = work - (int)(bl * G);
  const int n = p.n_valid;
  const uint32_t* a = (const uint32_t*)(p.scores + ((size_t)bl * G + g) * (size_t)n);
  // order-preserving unsigned key of a score (the bit pattern itself for
  // non-negative scores; sign-folded, with -0 = +0, for signed ones)
  const bool sgn = p.signed_keys != 0;
  auto key = [sgn](uint32_t u) -> uint32_t {
    if (!sgn) return u;
    if (u == 0x80000000u) u = 0u;
    return (u >> 31) ? ~u : (u | 0x80000000u);
  };
  int32_t* out = p.kv_idx + ((size_t)(p.bh0 + bl) * G + g) * (size_t)p.topk;
  const int tid = threadIdx.x;

  uint32_t prefix = 0u, pmask = 0u;
  int krem = p.topk;
  const int shifts[3] = {22, 11, 0};
  const int widths[3] = {10, 11, 11};
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = shifts[pass];
    const uint32_t dmask = (1u << widths[pass]) - 1u;
    if (pass == 0 && p.hist0 != nullptr) {
      // the score pass already counted the top 10 bits of this row
      const int32_t* h0 = p.hist0 + ((size_t)bl * G + g) * 1024;
      for (int b = tid; b < NBIN; b += NT) hist[b] = (b < 1024) ? h0[b] : 0;
    } else {
      for (int b = tid; b < NBIN; b += NT) hist[b] = 0;
      __syncthreads();
      // eight independent loads in flight per thread
      int j = tid;
      for (; j + 7 * NT < n; j += 8 * NT) {
        uint32_t u[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = key(a[j + e * NT]);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if ((u[e] & pmask) == prefix) atomicAdd(&hist[(u[e] >> sh) & dmask], 1);
      }
      for (; j < n; j += NT) {
        const uint32_t u = key(a[j]);
        if ((u & pmask) == prefix) atomicAdd(&hist[(u >> sh) & dmask], 1);
      }
    }
    __syncthreads();
    // thread t owns bins, highest first: NBIN-1-BPT*t-i for i = 0..BPT-1
    int loc[BPT];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      loc[i] = hist[NBIN - 1 - BPT * tid - i];
      sum += loc[i];
    }
    int tot;
    int above = block_excl_scan<NT>(sum, scan_sh, &tot);  // elements in higher bins
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      if (above < krem && above + loc[i] >= krem) {
        found[0] = NBIN - 1 - BPT * tid - i;
        found[1] = krem - above;
      }
      above += loc[i];
    }
    __syncthreads();
    prefix |= (uint32_t)found[0] << sh;
    pmask |= dmask << sh;
    krem = found[1];
    __syncthreads();
  }

  // Compaction in key order: keep u > T, and the first `krem` keys with u == T.
  const uint32_t T = prefix;
  constexpr int E = 4;
  int taken = 0, eq_seen = 0;
  for (int base = 0; base < n; base += NT * E) {
    uint32_t u[E];
    int neq = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = base + tid * E + e;
      u[e] = (j < n) ? key(a[j]) : 0u;
      if (j < n && u[e] == T) ++neq;
    }
    int eq_tot;
    int eq_rank = eq_seen + block_excl_scan<NT>(neq, scan_sh, &eq_tot);
    bool sel[E];
    int nsel = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = base + tid * E + e;
      bool s = false;
      if (j < n) {
        if (u[e] > T) {
          s = true;
        } else if (u[e] == T) {
          s = eq_rank < krem;
          ++eq_rank;
        }
      }
      sel[e] = s;
      nsel += s ? 1 : 0;
    }
    int sel_tot;
    int pos = taken + block_excl_scan<NT>(nsel, scan_sh, &sel_tot);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (sel[e] && pos < p.topk) out[pos++] = base + tid * E + e;
    }
    taken += sel_tot;
    eq_seen += eq_tot;
  }
}

template <int D, int C>
static hipError_t launch_scores_t(const ScoreParams& p, hipStream_t s) {
  const int64_t items = p.bh_count * (int64_t)p.groups;
  hipLaunchKernelGGL((score_kernel<D, C>), dim3((unsigned)items), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_scores(int d, int c, const ScoreParams& p, hipStream_t s) {
  if (d == 128 && c == 128) return launch_scores_t<128, 128>(p, s);
  if (d == 128 && c == 64) return launch_scores_t<128, 64>(p, s);
  if (d == 96 && c == 128) return launch_scores_t<96, 128>(p, s);
  if (d == 96 && c == 64) return launch_scores_t<96, 64>(p, s);
  if (d == 64 && c == 128) return launch_scores_t<64, 128>(p, s);
  if (d == 64 && c == 64) return launch_scores_t<64, 64>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_topk(const TopkParams& p, hipStream_t s) {
  const int64_t items = p.bh_count * (int64_t)p.groups;
  hipLaunchKernelGGL((topk_kernel<512>), dim3((unsigned)items), dim3(512), 0, s, p);
  return hipGetLastError();
}

}  // namespace mcs
