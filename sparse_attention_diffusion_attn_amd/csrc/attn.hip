// Dense, token-sparse and residual attention on gfx950 (one kernel template).
//
// The token-sparse mode is the reuse step of MC-Sparse (onedev.kr summary,
// "what is different": O_t = SparseAttn(Q_t, K_t, V_t; G, S) + R; "how it is
// used", component 1: K/V rows are gathered on line from the cached indices).
// The dense mode is the dense baseline and anchor pass 1; the residual mode
// writes R = O_full - SparseAttn(...) at the anchor.
//
// One workgroup per (head, query group), four wavefronts: for C = 128 each owns
// 32 query rows; for C = 64 two share each 32-row block, one per 32-key half of
// every tile.  Key/value tiles of 64 rows are gathered by index with 16-byte
// buffer->LDS copies into a double-buffered LDS tile (column planes, chunks
// permuted per row against bank conflicts).  The copies of tile t+1 are
// issued one per k-step of tile t's QK^T product (spread out, so the vector
// memory queues never fill in a burst) and the indices of tile t+2 after it;
// both are in flight while tile t is consumed.  Both contractions run on v_mfma_f32_32x32x16_bf16:
//   S^T = K_tile . Q^T   (A = gathered K rows from LDS, B = Q held in VGPRs)
//   O^T += V_tile^T . P^T (A = V via transposing LDS reads, B = P from the S^T
//                          accumulators, converted to bf16)
// so every lane owns one query row for the whole online softmax (fp32, exp2
// with the scale folded in); the only cross-lane step, in the running-max
// pass, is one max exchange between the two 32-lane halves, done in the VALU.
// Softmax does not depend on the offset subtracted from the logits, so the
// first pass uses none: p = exp2(s * scale * log2 e) straight from the
// accumulators, with no row max at all.  That is exact while every row's
// probability sum stays inside [2^-60, 2^64] and O is finite; a row outside
// (logits beyond about +-60 in log2 units) makes the workgroup redo the group
// with the lazily raised running max, which a dense call that returns the
// log-sum-exp always uses.
// The dense mode runs the very same code with contiguous key rows, so the
// sparse/dense time ratio measures the cost of gathering alone.
#include <type_traits>

#include "mcs_common.h"
#include "mcs_internal.h"

namespace mcs {

// Headroom of the lazily updated running max, in log2 units.
constexpr float kLazyLog2 = 8.0f;
// Row sums the zero-offset pass accepts: up to 2^64, probabilities keep full
// fp32 / bf16 relative precision and O stays far from overflow; from 2^-60 up,
// the largest probability of a row of up to 2^24 keys is at least 2^-84, so
// the ones that underflow (each below 2^-126) weigh less than 2^-18 of the
// row all together.
constexpr float kZeroOffMaxSum = 18446744073709551616.0f;  // 2^64
constexpr float kZeroOffMinSum = 8.673617379884035e-19f;   // 2^-60
__device__ constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

template <int D, int C, int MODE>
__global__ __launch_bounds__(256) void attn_kernel(AttnParams p) {
  // Four wavefronts.  C = 128: one per 32-row block of the group.  C = 64:
  // two per 32-row block, one per half of every key tile (SPLIT); their
  // partial softmax states are merged in the epilogue.  Either way a CU holds
  // two workgroups, eight wavefronts.
  static_assert(C == 128 || C == 64, "group size");
  constexpr bool SPLIT = (C == 64);
  constexpr int NW = 4;
  constexpr int KT = 64;                // keys per tile
  constexpr int NPL = D / 32;           // column planes per tile (4 KiB each)
  constexpr int TILE = NPL * 4096;      // bytes per matrix tile
  constexpr int IPM = TILE / 1024;      // 1 KiB copy instructions per matrix tile
  constexpr int IPW = IPM / NW;         // ... per wavefront
  constexpr int KS = D / 16;            // k-steps of the QK^T product
  static_assert(IPW >= 1 && IPM % NW == 0, "tile split");

  __shared__ __attribute__((aligned(1024))) char lds[4 * TILE];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ql = lane & 31;
  const int h = lane >> 5;
  const int rb = SPLIT ? (w & 1) : w;   // this wavefront's 32-row block
  const int kh = SPLIT ? (w >> 1) : 0;  // its half of each key tile (SPLIT)

  const int G = p.groups;
  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t bh = work / G;
  const int g = work - (int)(bh * G);
  const uint16_t* Qb = p.q + head_offset(p.sq, bh, p.heads);
  const uint16_t* Kb = p.k + head_offset(p.sk, bh, p.heads);
  const uint16_t* Vb = p.v + head_offset(p.sv, bh, p.heads);

  // ---- query rows of this lane (B operand of S^T, resident in VGPRs) ----
  // A perm entry outside 0 .. n_pad-1 (perm is caller memory that may have
  // travelled through the host) is never used as an address: such a lane
  // reads row 0 and writes nothing.
  const int qpos = g * C + 32 * rb + ql;
  const int qraw = (MODE == ATTN_DENSE) ? qpos : p.perm[(size_t)bh * p.n_pad + qpos];
  const bool row_ok = (uint32_t)qraw < (uint32_t)p.n_pad;
  const int qrow = row_ok ? qraw : 0;
  bf16x8 qreg[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk)
    qreg[kk] = *(const bf16x8*)(Qb + (int64_t)qrow * p.sq.n + 16 * kk + 8 * h);

  // keys of this group: all valid keys (dense), or the first nk indices of
  // the group's row (a per-group count, clamped to 1 .. row stride, or topk)
  int nk = p.n_valid;
  if (MODE != ATTN_DENSE) {
    nk = p.topk;
    if (p.kv_count != nullptr) {
      const int c = p.kv_count[(size_t)bh * G + g];
      nk = c < 1 ? 1 : (c > p.kv_stride ? p.kv_stride : c);
    }
  }
  const int ntiles = (nk + KT - 1) / KT;
  const int32_t* idxrow =
      (MODE == ATTN_DENSE) ? nullptr : p.kv_idx + ((size_t)bh * G + g) * p.kv_stride;

  // ---- gather geometry ----
  // Copy instruction `ins` (the wavefront's i-th: ins = w*IPW + i) fills
  // plane ins/4, tile slots 16*(ins%4) .. +15; lane l writes slot
  // 16*(ins%4) + l/4, physical chunk l%4, i.e. logical chunk (l%4)^((l/16)%4)
  // of that plane.  Slot 16*r + j holds key 4*j + r of the tile, so a lane's
  // i-th copy needs key 4*(l/4) + (ins%4): one offset register serves all its
  // index loads, the wave-uniform key and plane parts coming from ins.  Any
  // fixed order of the keys inside a tile is valid, as K and V share it and
  // only the final-tile mask looks at key positions.  K, V and the index row
  // are read through buffer resources with 32-bit offsets (row * row stride,
  // a 24-bit multiply); reads past a resource's end return zero (dword by
  // dword, so a 16-byte index load that straddles the end still returns its
  // valid entries), which the final-tile mask covers for the index row.
  constexpr int NTOK = IPW < 4 ? IPW : 4;     // distinct keys per lane per tile
  auto ins_key = [&](int i) { return (w * IPW + i) & 3; };                  // key offset of copy i
  auto ins_plane = [&](int i) { return (uint32_t)((w * IPW + i) >> 2) * 64u; };  // its plane's byte offset
  const int j4 = 4 * (lane >> 2);
  const uint32_t gcb = 16u * (uint32_t)((lane ^ (lane >> 4)) & 3);
  const uint32_t rsb = (uint32_t)p.sk.n * 2u;  // row stride of K and V in bytes
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(Kb, head_span_bytes(p.sk, p.n_pad, D));
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(Vb, head_span_bytes(p.sv, p.n_pad, D));
  const __amdgpu_buffer_rsrc_t irs =
      (MODE == ATTN_DENSE) ? krs : make_rsrc(idxrow, (uint32_t)nk * 4u);
  int tok[NTOK];
  // A lane's keys are 4*(l/4) + ins_key(i).  With four copies per wavefront
  // (d = 128) they are the four consecutive keys from 4*(l/4), read with one
  // 16-byte load instead of four 4-byte ones (fewer wavefronts through the
  // vector-memory path, which the copies keep busy); otherwise one 4-byte
  // load each.
  auto fetch_idx = [&](int t) {
    const int key0 = t * KT + j4;
    if (MODE == ATTN_DENSE) {
#pragma unroll
      for (int i = 0; i < NTOK; ++i) tok[i] = key0 + ins_key(i);
    } else if constexpr (IPW == 4) {
      const i32x4 x = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(irs, (uint32_t)key0 * 4u, 0, 0));
#pragma unroll
      for (int i = 0; i < 4; ++i) tok[i] = x[i];
    } else {
#pragma unroll
      for (int i = 0; i < NTOK; ++i)
        tok[i] = __builtin_amdgcn_raw_buffer_load_b32(irs, (uint32_t)(key0 + ins_key(i)) * 4u, 0, 0);
    }
  };
  auto issue = [&](int buf) {
    char* kdst = lds + buf * 2 * TILE + w * IPW * 1024;
    char* vdst = kdst + TILE;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const uint32_t voff = __umul24((uint32_t)tok[i % NTOK], rsb) + gcb;
      gather16_buf(krs, kdst + i * 1024, voff, ins_plane(i));
      gather16_buf(vrs, vdst + i * 1024, voff, ins_plane(i));
    }
  };

  // ---- LDS read geometry (base + compile-time offsets) ----
  // QK^T operand: rows ql (+32), 16-byte chunk 2*kk+h = plane kk/2, in-plane
  // chunk 2*(kk%2)+h.
  const int sq = (ql >> 2) & 3;
  const int koff_e = ql * 64 + ((h ^ sq) << 4);
  const int koff_o = ql * 64 + (((2 + h) ^ sq) << 4);
  // PV operand: transposing reads of rows 16u + 4h + jj/4 (and +8) at plane
  // columns 16*(qq%2) + 4*(jj%4).
  const int jj = lane & 15, qq = lane >> 4;
  const int vrow = 4 * h + (jj >> 2);
  const int vchunk = 2 * (qq & 1) + ((jj & 3) >> 1);
  const int vhalf = 8 * (jj & 1);
  const int voff_a = vrow * 64 + ((vchunk ^ h) << 4) + vhalf;
  const int voff_b = (vrow + 8) * 64 + ((vchunk ^ h ^ 2) << 4) + vhalf;

  f32x16 o[NPL];
  float mrun, lrun;
  const float c2 = p.scale * kLog2e;
  __shared__ int redo;
  if (threadIdx.x == 0) redo = 0;

  // One key tile: the copies of tile t+1 go to kdst_n (the other buffer)
  // while kbuf/vbuf (this tile's K and V) are read.  The three pointers are
  // restrict-qualified: the compiler then knows that the LDS reads cannot
  // alias the copies in flight, and does not make the transposing V reads
  // wait for those copies (it would otherwise insert a vmcnt(0) before them).
  auto tile = [&](auto fixed, int t, char* __restrict__ kdst_n, const char* __restrict__ kbuf,
                  const char* __restrict__ vbuf) __attribute__((always_inline)) {
    constexpr bool FIXED = decltype(fixed)::value;
    const bool more = t + 1 < ntiles;

    // S^T = K . Q^T for the 64 keys of this tile (two 32-key blocks).  The K
    // operands of k-step kk+1 are read while the products of kk run, and
    // step kk also issues its share of tile t+1's copies.
    f32x16 s0, s1;
#pragma unroll
    for (int j = 0; j < 16; ++j) { s0[j] = 0.f; s1[j] = 0.f; }
    // (SPLIT: only the 32 keys of this wavefront's half, in s0)
    bf16x8 a0 = *(const bf16x8*)(kbuf + koff_e + kh * 2048);
    bf16x8 a1 = SPLIT ? a0 : *(const bf16x8*)(kbuf + koff_e + 2048);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      bf16x8 n0 = a0, n1 = a1;
      if (kk + 1 < KS) {
        const char* kp = kbuf + (((kk + 1) & 1) ? koff_o : koff_e) + ((kk + 1) >> 1) * 4096;
        n0 = *(const bf16x8*)(kp + kh * 2048);
        if (!SPLIT) n1 = *(const bf16x8*)(kp + 2048);
      }
      __builtin_amdgcn_sched_barrier(0);
      s0 = mfma32(a0, qreg[kk], s0);
      if (!SPLIT) s1 = mfma32(a1, qreg[kk], s1);
      a0 = n0;
      a1 = n1;
      if (more) {
        constexpr int PER = (2 * IPW + KS - 1) / KS;
#pragma unroll
        for (int c = kk * PER; c < (kk + 1) * PER && c < 2 * IPW; ++c) {
          const int i = c >> 1;
          const uint32_t voff = __umul24((uint32_t)tok[i % NTOK], rsb) + gcb;
          if (c & 1)
            gather16_buf(vrs, kdst_n + TILE + i * 1024, voff, ins_plane(i));
          else
            gather16_buf(krs, kdst_n + i * 1024, voff, ins_plane(i));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // The V operands of the whole tile (four 16-key blocks) are read right
    // after the QK^T products: they do not depend on the softmax, which then
    // hides their latency.
    constexpr int NU = SPLIT ? 2 : 4;   // 16-key blocks of this wavefront
    i32x2 vall[NU][2 * NPL];
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int T = 0; T < NPL; ++T) {
        const int ub = (SPLIT ? 2 * kh : 0) + u;
        vall[u][2 * T] = tr_read(vbuf + voff_a + ub * 1024 + T * 4096);
        vall[u][2 * T + 1] = tr_read(vbuf + voff_b + ub * 1024 + T * 4096);
      }
    if (t + 2 < ntiles) fetch_idx(t + 2);

    // mask keys past the end in the last tile (slot s holds key
    // 4*(s%16) + s/16; slots s and s+32 hold keys two apart)
    if ((t + 1) * KT > nk) {
      const int lim = nk - t * KT;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int slot = 8 * (j >> 2) + 4 * h + (j & 3);
        const int key = 4 * (slot & 15) + (slot >> 4);
        if (key + 2 * kh >= lim) s0[j] = -INFINITY;
        if (!SPLIT && key + 2 >= lim) s1[j] = -INFINITY;
      }
    }

    // online softmax (this lane owns query ql; its partner lane ql+32 holds
    // the other half of the tile's keys).  The running max is only raised when
    // the tile's max exceeds it by more than kLazyLog2 (in log2 units), so the
    // rescale of O and l is skipped on almost every tile; probabilities stay
    // below 2^kLazyLog2 and the final O / l is unchanged.  The zero-offset
    // pass skips it (mrun stays 0).
    if constexpr (!FIXED) {
      float mx = s0[0];
#pragma unroll
      for (int j = 1; j < 16; ++j) mx = fmaxf(mx, s0[j]);
      if (!SPLIT) {
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s1[j]);
      }
      mx = max_xor32(mx);
      const bool raise = (mx - mrun) * c2 > kLazyLog2;
      if (__any(raise)) {
        const float mnew = raise ? mx : mrun;
        const float alpha = __builtin_amdgcn_exp2f((mrun - mnew) * c2);
        mrun = mnew;
        lrun *= alpha;
#pragma unroll
        for (int T = 0; T < NPL; ++T)
#pragma unroll
          for (int j = 0; j < 16; ++j) o[T][j] *= alpha;
      }
    }
    // (SPLIT: a half that has seen no valid key yet keeps mrun = -inf; its
    // probabilities are then exp2(-inf) = 0 rather than NaN)
    const float mc = (FIXED || (SPLIT && mrun == -INFINITY)) ? 0.f : mrun * c2;
    bf16x8 pb[NU];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[j], c2, -mc));
      pb[j >> 3][j & 7] = (__bf16)e0;
      if (!SPLIT) {
        const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[j], c2, -mc));
        pb[(2 + (j >> 3)) % NU][j & 7] = (__bf16)e1;
      }
    }
    // row sum of the bf16 probabilities the PV product uses (so numerator and
    // denominator see the same rounded weights), two per dot2 instruction
    {
      float la = 0.f, lb = 0.f;
#pragma unroll
      for (int q = 0; q < NU; ++q) {
        const bf16x2 p01 = {pb[q][0], pb[q][1]}, p23 = {pb[q][2], pb[q][3]};
        const bf16x2 p45 = {pb[q][4], pb[q][5]}, p67 = {pb[q][6], pb[q][7]};
        la = __builtin_amdgcn_fdot2_f32_bf16(p01, kOnes2, la, false);
        lb = __builtin_amdgcn_fdot2_f32_bf16(p23, kOnes2, lb, false);
        la = __builtin_amdgcn_fdot2_f32_bf16(p45, kOnes2, la, false);
        lb = __builtin_amdgcn_fdot2_f32_bf16(p67, kOnes2, lb, false);
      }
      lrun += la + lb;
    }

    // O^T += V^T . P^T, 16 keys (one k-step) per block u.
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const i32x2* va = vall[u];
#pragma unroll
      for (int T = 0; T < NPL; ++T) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, (i32x4){va[2 * T][0], va[2 * T][1],
                                                           va[2 * T + 1][0], va[2 * T + 1][1]});
        o[T] = mfma32(a, pb[u], o[T]);
      }
    }
  };

  auto run = [&](auto fixed) {
    constexpr bool FIXED = decltype(fixed)::value;
#pragma unroll
    for (int T = 0; T < NPL; ++T)
#pragma unroll
      for (int j = 0; j < 16; ++j) o[T][j] = 0.f;
    mrun = FIXED ? 0.f : -INFINITY;
    lrun = 0.f;
    fetch_idx(0);
    issue(0);
    if (ntiles > 1) fetch_idx(1);
    for (int t = 0; t < ntiles; ++t) {
      wait_vm0();
      __syncthreads();
      tile(fixed, t, lds + ((t + 1) & 1) * 2 * TILE + w * IPW * 1024, lds + (t & 1) * 2 * TILE,
           lds + (t & 1) * 2 * TILE + TILE);
    }
  };

  // Row sum over the lane pair; with C = 64 the two key halves of each row
  // block are merged here: the kh = 1 wavefront hands its running max, row sum
  // and O to the kh = 0 one through LDS (the tile buffers are free once every
  // wavefront has passed the barrier; no copy is in flight after the last
  // tile), and the kh = 0 wavefront rescales both to the common max.
  auto finish = [&]() -> float {
    float lsum = sum_xor32(lrun);
    if constexpr (SPLIT) {
      constexpr int NV = NPL * 16 + 2;    // values per lane
      float* xo = reinterpret_cast<float*>(lds) + rb * NV * 64 + lane;
      __syncthreads();
      if (kh == 1) {
#pragma unroll
        for (int T = 0; T < NPL; ++T)
#pragma unroll
          for (int j = 0; j < 16; ++j) xo[(T * 16 + j) * 64] = o[T][j];
        xo[(NPL * 16) * 64] = mrun;
        xo[(NPL * 16 + 1) * 64] = lsum;
      }
      __syncthreads();
      if (kh == 0) {
        const float m1 = xo[(NPL * 16) * 64], l1 = xo[(NPL * 16 + 1) * 64];
        const float m = fmaxf(mrun, m1);  // mrun is finite: key 0 lies in half 0
        const float f0 = __builtin_amdgcn_exp2f((mrun - m) * c2);
        const float f1 = (m1 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m1 - m) * c2);
#pragma unroll
        for (int T = 0; T < NPL; ++T)
#pragma unroll
          for (int j = 0; j < 16; ++j) o[T][j] = o[T][j] * f0 + xo[(T * 16 + j) * 64] * f1;
        lsum = lsum * f0 + l1 * f1;
        mrun = m;
      }
    }
    return lsum;
  };

  // The row sums add the bf16-rounded probabilities, so a row's largest term
  // is exact only when the offset is the row max (it is then exp2(0) = 1).  A
  // log-sum-exp output (the anchor's dense pass, whose lse weighs every key of
  // the score pass) therefore always takes the running-max pass.
  float lsum;
  bool zero_pass = !(MODE == ATTN_DENSE && p.lse != nullptr);
  if (zero_pass) {
    run(std::true_type{});
    lsum = finish();
    // range check on the (merged) rows; any failing row redoes the whole group
    bool ok = lsum >= kZeroOffMinSum && lsum <= kZeroOffMaxSum;
#pragma unroll
    for (int T = 0; T < NPL; ++T)
#pragma unroll
      for (int j = 0; j < 16; ++j) ok = ok && __builtin_isfinite(o[T][j]);
    if (SPLIT && kh == 1) ok = true;    // its values live in the kh = 0 wavefront now
    if (__any(!ok) && lane == 0) redo = 1;
    __syncthreads();
    zero_pass = (redo == 0);
  }
  if (!zero_pass) {
    run(std::false_type{});
    lsum = finish();
  }
  if (SPLIT && kh == 1) return;         // no barrier follows

  // ---- epilogue ----
  const float inv = 1.f / lsum;
  const bool valid = qrow < p.n_valid;
  uint16_t* Ob = p.out + head_offset(p.so, bh, p.heads) + (int64_t)qrow * p.so.n;
  const uint16_t* Ab =
      (p.aux != nullptr) ? p.aux + head_offset(p.sa, bh, p.heads) + (int64_t)qrow * p.sa.n : nullptr;
#pragma unroll
  for (int T = 0; T < NPL; ++T) {
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int col = 32 * T + 8 * gq + 4 * h;
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = o[T][4 * gq + e] * inv;
      if (MODE == ATTN_SPARSE && Ab != nullptr) {
        const uint2 rv = *(const uint2*)(Ab + col);
        x[0] += bf16_to_f32(rv.x & 0xffff);
        x[1] += bf16_to_f32(rv.x >> 16);
        x[2] += bf16_to_f32(rv.y & 0xffff);
        x[3] += bf16_to_f32(rv.y >> 16);
      } else if (MODE == ATTN_RESID) {
        const uint2 ov = *(const uint2*)(Ab + col);
        x[0] = bf16_to_f32(ov.x & 0xffff) - x[0];
        x[1] = bf16_to_f32(ov.x >> 16) - x[1];
        x[2] = bf16_to_f32(ov.y & 0xffff) - x[2];
        x[3] = bf16_to_f32(ov.y >> 16) - x[3];
      }
      if (!row_ok) continue;
      uint2 st;
      if (valid) {
        st.x = (uint32_t)f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16);
        st.y = (uint32_t)f32_to_bf16(x[2]) | ((uint32_t)f32_to_bf16(x[3]) << 16);
      } else {
        st.x = 0u;
        st.y = 0u;
      }
      *(uint2*)(Ob + col) = st;
    }
  }
  if (MODE == ATTN_DENSE && p.lse != nullptr && h == 0) {
    p.lse[(size_t)bh * p.n_pad + qrow] = valid ? (mrun * p.scale + __logf(lsum)) : 0.f;
  }
}

template <int D, int C, int MODE>
static hipError_t launch_one(const AttnParams& p, hipStream_t s) {
  const int64_t items = p.bh * (int64_t)p.groups;
  hipLaunchKernelGGL((attn_kernel<D, C, MODE>), dim3((unsigned)items), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_mode(int d, int c, const AttnParams& p, hipStream_t s) {
  if (d == 128 && c == 128) return launch_one<128, 128, MODE>(p, s);
  if (d == 128 && c == 64) return launch_one<128, 64, MODE>(p, s);
  if (d == 96 && c == 128) return launch_one<96, 128, MODE>(p, s);
  if (d == 96 && c == 64) return launch_one<96, 64, MODE>(p, s);
  if (d == 64 && c == 128) return launch_one<64, 128, MODE>(p, s);
  if (d == 64 && c == 64) return launch_one<64, 64, MODE>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_attention(int mode, int head_dim, int group_size, const AttnParams& p,
                            hipStream_t s) {
  switch (mode) {
    case ATTN_DENSE: return launch_mode<ATTN_DENSE>(head_dim, group_size, p, s);
    case ATTN_SPARSE: return launch_mode<ATTN_SPARSE>(head_dim, group_size, p, s);
    case ATTN_RESID: return launch_mode<ATTN_RESID>(head_dim, group_size, p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mcs
