// Block selection for the variants of MC-Sparse's oracle analysis (onedev.kr
// summary, "how it works": at one density, a block oracle chooses KV blocks
// per query block with exact dense probabilities; vanilla block-sparse
// attention ranks the blocks by mean-pooled queries and keys).  The chosen
// blocks are expanded to token index rows that the token-gather attention
// kernel consumes unchanged (with a per-group key count).
//
// KV blocks: `block` consecutive valid keys, the last one possibly shorter.
// Scores are accumulated in fp64 and rounded once to fp32 for the top-k.
//
// block_sum_kernel   exact block score = sum of the group's exact token
//                    scores over the block (one wavefront per block).
// key_pool_kernel    kbar_b = mean of block b's keys (fp64).
// meanpool_kernel    qbar_g = mean of group g's valid member queries (fp64),
//                    score = scale * qbar_g . kbar_b.
// expand_kernel      selected blocks (ascending) -> their tokens, ascending;
//                    positions past the group's count are set to -1.
#include "mcs_common.h"
#include "mcs_internal.h"

namespace mcs {

__device__ __forceinline__ double wave_sum_f64(double x) {
  // butterfly over the 64 lanes; partners add the same two numbers, so every
  // lane ends with bitwise the same value
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x += __shfl_xor(x, o);
  return x;
}

__global__ __launch_bounds__(256) void block_sum_kernel(BlockParams p) {
  const int G = p.groups;
  const int64_t bl = blockIdx.x / G;
  const int g = (int)(blockIdx.x - bl * G);
  const float* a = p.token_scores + ((size_t)bl * G + g) * (size_t)p.n_valid;
  float* out = p.block_scores + ((size_t)bl * G + g) * (size_t)p.nb;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int b = w; b < p.nb; b += 4) {
    const int j0 = b * p.block;
    const int j1 = min(j0 + p.block, p.n_valid);
    double s = 0.0;
    for (int j = j0 + lane; j < j1; j += 64) s += (double)a[j];
    s = wave_sum_f64(s);
    if (lane == 0) out[b] = (float)s;
  }
}

template <int D>
__global__ __launch_bounds__(D) void key_pool_kernel(BlockParams p) {
  const int64_t bl = blockIdx.x / p.nb;
  const int b = (int)(blockIdx.x - bl * p.nb);
  const int d = threadIdx.x;
  const uint16_t* K = p.k + head_offset(p.sk, p.bh0 + bl, p.heads);
  const int j0 = b * p.block;
  const int j1 = min(j0 + p.block, p.n_valid);
  double s = 0.0;
  for (int j = j0; j < j1; ++j) s += (double)bf16_to_f32(K[(int64_t)j * p.sk.n + d]);
  double* kb = p.kbar + ((size_t)bl * p.nb + b) * D;
  kb[d] = s / (double)(j1 - j0);
}

template <int D, int C>
__global__ __launch_bounds__(256) void meanpool_kernel(BlockParams p) {
  constexpr int NT = 256, PARTS = NT / D;
  __shared__ double part[NT];
  __shared__ double qbar[D];
  __shared__ int valid_cnt[PARTS];
  const int G = p.groups;
  const int64_t bl = blockIdx.x / G;
  const int g = (int)(blockIdx.x - bl * G);
  const int64_t bh = p.bh0 + bl;
  const uint16_t* Q = p.q + head_offset(p.sq, bh, p.heads);
  const int32_t* mem = p.perm + (size_t)bh * p.n_pad + (size_t)g * C;
  const int tid = threadIdx.x, d = tid % D, pt = tid / D;
  double s = 0.0;
  int cnt = 0;
  for (int r = pt; r < C; r += PARTS) {
    const int row = mem[r];
    if ((uint32_t)row < (uint32_t)p.n_valid) {  // padding rows and bad entries excluded
      s += (double)bf16_to_f32(Q[(int64_t)row * p.sq.n + d]);
      ++cnt;
    }
  }
  part[tid] = s;
  if (d == 0) valid_cnt[pt] = cnt;
  __syncthreads();
  if (tid < D) {
    double t = part[tid];
    int c = valid_cnt[0];
    for (int q = 1; q < PARTS; ++q) {
      t += part[q * D + tid];
      c += valid_cnt[q];
    }
    qbar[tid] = (c > 0) ? t / (double)c : 0.0;
  }
  __syncthreads();
  const double* kb = p.kbar + (size_t)bl * p.nb * D;
  float* out = p.block_scores + ((size_t)bl * G + g) * (size_t)p.nb;
  for (int b = tid; b < p.nb; b += NT) {
    double dot = 0.0;
    for (int e = 0; e < D; ++e) dot = __builtin_fma(qbar[e], kb[(size_t)b * D + e], dot);
    out[b] = (float)((double)p.scale * dot);
  }
}

__global__ __launch_bounds__(256) void expand_kernel(BlockParams p) {
  __shared__ int sel[1024];
  __shared__ int start[1025];
  const int G = p.groups;
  const int64_t bl = blockIdx.x / G;
  const int g = (int)(blockIdx.x - bl * G);
  const int32_t* bi = p.block_idx + ((size_t)bl * G + g) * (size_t)p.nblocks;
  const int64_t row = (p.bh0 + bl) * G + g;
  const int stride = p.nblocks * p.block;
  int32_t* out = p.kv_idx + (size_t)row * stride;
  const int tid = threadIdx.x;
  // block starts of the selected blocks in output order (nblocks <= 1024)
  for (int i = tid; i < p.nblocks; i += 256) sel[i] = bi[i];
  __syncthreads();
  if (tid == 0) {
    int o = 0;
    for (int i = 0; i < p.nblocks; ++i) {
      start[i] = o;
      const int j0 = sel[i] * p.block;
      o += min(j0 + p.block, p.n_valid) - j0;
    }
    start[p.nblocks] = o;
    p.kv_count[row] = o;
  }
  __syncthreads();
  for (int i = 0; i < p.nblocks; ++i) {
    const int j0 = sel[i] * p.block;
    const int len = start[i + 1] - start[i];
    for (int t = tid; t < len; t += 256) out[start[i] + t] = j0 + t;
  }
  for (int t = start[p.nblocks] + tid; t < stride; t += 256) out[t] = -1;
}

hipError_t launch_block_sums(const BlockParams& p, hipStream_t s) {
  hipLaunchKernelGGL(block_sum_kernel, dim3((unsigned)(p.bh_count * p.groups)), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_key_pool(int d, const BlockParams& p, hipStream_t s) {
  const dim3 grid((unsigned)(p.bh_count * p.nb));
  if (d == 128) hipLaunchKernelGGL((key_pool_kernel<128>), grid, dim3(128), 0, s, p);
  else if (d == 64) hipLaunchKernelGGL((key_pool_kernel<64>), grid, dim3(64), 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_meanpool_scores(int d, int c, const BlockParams& p, hipStream_t s) {
  const dim3 grid((unsigned)(p.bh_count * p.groups));
  if (d == 128 && c == 128) hipLaunchKernelGGL((meanpool_kernel<128, 128>), grid, dim3(256), 0, s, p);
  else if (d == 128 && c == 64) hipLaunchKernelGGL((meanpool_kernel<128, 64>), grid, dim3(256), 0, s, p);
  else if (d == 64 && c == 128) hipLaunchKernelGGL((meanpool_kernel<64, 128>), grid, dim3(256), 0, s, p);
  else if (d == 64 && c == 64) hipLaunchKernelGGL((meanpool_kernel<64, 64>), grid, dim3(256), 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_expand_blocks(const BlockParams& p, hipStream_t s) {
  hipLaunchKernelGGL(expand_kernel, dim3((unsigned)(p.bh_count * p.groups)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mcs
