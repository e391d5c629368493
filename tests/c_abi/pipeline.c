/* A plain C99 program that runs the method end to end through the C ABI on a
 * GPU, with device buffers from the HIP runtime and no PyTorch: an anchor step
 * (grouping, two-pass selection, residual) and one reuse step, on seeded
 * synthetic inputs (clustered queries and keys; the reuse step's Q, K, V are
 * the anchor's plus a small drift).  It writes its inputs and every output as
 * raw little-endian arrays into the directory given as argv[1], prints "ok"
 * and exits 0; the calling test checks them against the oracle. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mcs.h"

enum { B = 1, H = 2, NV = 300, NP = 320, D = 64, C = 64, TOPK = 70, NCL = 4 };
#define NQ ((size_t)B * H * NP * D)
#define G (NP / C)

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static double uniform01(void) { /* splitmix64, 53-bit uniform in (0, 1) */
  uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  z ^= z >> 31;
  return ((double)(z >> 11) + 0.5) / 9007199254740992.0;
}
static double normal(void) { /* Box-Muller */
  const double u = uniform01(), v = uniform01();
  return sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v);
}
static uint16_t to_bf16(float f) { /* round to nearest even */
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static float from_bf16(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static int save(const char* dir, const char* name, const void* p, size_t bytes) {
  char path[1024];
  FILE* f;
  snprintf(path, sizeof path, "%s/%s", dir, name);
  f = fopen(path, "wb");
  if (!f || fwrite(p, 1, bytes, f) != bytes) {
    fprintf(stderr, "cannot write %s\n", path);
    return 1;
  }
  fclose(f);
  return 0;
}

#define HIP_OK(x)                                                         \
  do {                                                                    \
    hipError_t e_ = (x);                                                  \
    if (e_ != hipSuccess) {                                               \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));      \
      return 1;                                                           \
    }                                                                     \
  } while (0)
#define MCS_OK_(x)                                                        \
  do {                                                                    \
    int32_t s_ = (x);                                                     \
    if (s_ != MCS_OK) {                                                   \
      fprintf(stderr, "%s failed: %s\n", #x, mcs_last_error());           \
      return 1;                                                           \
    }                                                                     \
  } while (0)

int main(int argc, char** argv) {
  static uint16_t hq[2][NQ], hk[2][NQ], hv[2][NQ], ho_full[NQ], hr[NQ], ho[NQ];
  static int32_t hperm[B * H * NP], hkv[B * H * G * TOPK];
  static float hlse[B * H * NP];
  static float qc[H][NCL][D], kc[H][NCL][D];
  uint16_t *q[2], *k[2], *v[2], *o_full, *r, *o;
  int32_t *perm, *kv;
  float* lse;
  void *ws_g, *ws_a;
  size_t wsg, wsa, i;
  int s, h, n, c;
  mcs_dims d;
  const float scale = 1.0f / 8.0f; /* 1/sqrt(64) */
  const char* dir = argc > 1 ? argv[1] : ".";

  /* clustered queries and keys (cluster of token n: n % NCL), Gaussian values;
     padding rows stay zero; step 1 drifts every valid entry by 0.05 N(0,1) */
  for (h = 0; h < H; ++h)
    for (c = 0; c < NCL; ++c)
      for (i = 0; i < D; ++i) {
        qc[h][c][i] = (float)normal();
        kc[h][c][i] = (float)normal();
      }
  memset(hq, 0, sizeof hq);
  memset(hk, 0, sizeof hk);
  memset(hv, 0, sizeof hv);
  for (h = 0; h < H; ++h)
    for (n = 0; n < NV; ++n)
      for (i = 0; i < D; ++i) {
        const size_t e = ((size_t)h * NP + n) * D + i;
        const float x = qc[h][n % NCL][i] + 0.4f * (float)normal();
        const float y = kc[h][n % NCL][i] + 0.4f * (float)normal();
        const float z = (float)normal();
        hq[0][e] = to_bf16(x);
        hk[0][e] = to_bf16(y);
        hv[0][e] = to_bf16(z);
        hq[1][e] = to_bf16(from_bf16(hq[0][e]) + 0.05f * (float)normal());
        hk[1][e] = to_bf16(from_bf16(hk[0][e]) + 0.05f * (float)normal());
        hv[1][e] = to_bf16(from_bf16(hv[0][e]) + 0.05f * (float)normal());
      }

  d.batch = B; d.heads = H; d.n_valid = NV; d.n_pad = NP; d.head_dim = D; d.group_size = C;
  wsg = mcs_group_workspace_bytes(&d);
  wsa = mcs_anchor_select_workspace_bytes(&d, TOPK);
  for (s = 0; s < 2; ++s) {
    HIP_OK(hipMalloc((void**)&q[s], NQ * 2));
    HIP_OK(hipMalloc((void**)&k[s], NQ * 2));
    HIP_OK(hipMalloc((void**)&v[s], NQ * 2));
    HIP_OK(hipMemcpy(q[s], hq[s], NQ * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(k[s], hk[s], NQ * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(v[s], hv[s], NQ * 2, hipMemcpyHostToDevice));
  }
  HIP_OK(hipMalloc((void**)&o_full, NQ * 2));
  HIP_OK(hipMalloc((void**)&r, NQ * 2));
  HIP_OK(hipMalloc((void**)&o, NQ * 2));
  HIP_OK(hipMalloc((void**)&perm, sizeof hperm));
  HIP_OK(hipMalloc((void**)&kv, sizeof hkv));
  HIP_OK(hipMalloc((void**)&lse, sizeof hlse));
  HIP_OK(hipMalloc(&ws_g, wsg));
  HIP_OK(hipMalloc(&ws_a, wsa));

  /* anchor step, then one reuse step, all on the default stream */
  MCS_OK_(mcs_group(&d, q[0], 20, -1, perm, ws_g, wsg, NULL));
  MCS_OK_(mcs_anchor_select(&d, q[0], k[0], v[0], perm, TOPK, scale, o_full, lse, kv, ws_a, wsa, NULL));
  MCS_OK_(mcs_residual(&d, q[0], k[0], v[0], perm, kv, TOPK, scale, o_full, r, NULL));
  MCS_OK_(mcs_sparse_attn(&d, q[1], k[1], v[1], perm, kv, TOPK, scale, r, o, NULL));
  HIP_OK(hipDeviceSynchronize());

  HIP_OK(hipMemcpy(hperm, perm, sizeof hperm, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hkv, kv, sizeof hkv, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hlse, lse, sizeof hlse, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(ho_full, o_full, NQ * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hr, r, NQ * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(ho, o, NQ * 2, hipMemcpyDeviceToHost));
  if (save(dir, "q0.bin", hq[0], NQ * 2) || save(dir, "k0.bin", hk[0], NQ * 2) ||
      save(dir, "v0.bin", hv[0], NQ * 2) || save(dir, "q1.bin", hq[1], NQ * 2) ||
      save(dir, "k1.bin", hk[1], NQ * 2) || save(dir, "v1.bin", hv[1], NQ * 2) ||
      save(dir, "perm.bin", hperm, sizeof hperm) || save(dir, "kv.bin", hkv, sizeof hkv) ||
      save(dir, "lse.bin", hlse, sizeof hlse) || save(dir, "o_full.bin", ho_full, NQ * 2) ||
      save(dir, "r.bin", hr, NQ * 2) || save(dir, "o.bin", ho, NQ * 2))
    return 1;

  for (s = 0; s < 2; ++s) {
    HIP_OK(hipFree(q[s]));
    HIP_OK(hipFree(k[s]));
    HIP_OK(hipFree(v[s]));
  }
  HIP_OK(hipFree(o_full));
  HIP_OK(hipFree(r));
  HIP_OK(hipFree(o));
  HIP_OK(hipFree(perm));
  HIP_OK(hipFree(kv));
  HIP_OK(hipFree(lse));
  HIP_OK(hipFree(ws_g));
  HIP_OK(hipFree(ws_a));
  printf("ok\n");
  return 0;
}
