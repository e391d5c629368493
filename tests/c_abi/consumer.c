/* A plain C99 consumer of the C ABI (include/mcs.h), built with the host C
 * compiler and linked against libmcs.so.  It only calls what works without a
 * GPU: version and status strings, the layout helpers, workspace queries and
 * argument validation (every failing call returns before enqueuing work).
 * Prints "ok" and exits 0 on success. */
#include <stdio.h>
#include <string.h>

#include "mcs.h"

#define CHECK(cond)                                              \
  do {                                                           \
    if (!(cond)) {                                               \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                  \
    }                                                            \
  } while (0)

int main(void) {
  mcs_dims d;
  mcs_layout lay;
  size_t ws;
  uint16_t* fake = (uint16_t*)(uintptr_t)0x10000; /* aligned, never dereferenced */
  int32_t st;

  CHECK(mcs_abi_version() == MCS_ABI_VERSION);
  CHECK(strcmp(mcs_status_string(MCS_ERR_WORKSPACE), "MCS_ERR_WORKSPACE") == 0);

  d.batch = 2; d.heads = 3; d.n_valid = 1000; d.n_pad = 1024; d.head_dim = 128; d.group_size = 128;
  mcs_layout_bnhd(&d, &lay);
  CHECK(lay.q.token == 3 * 128 && lay.q.head == 128 && lay.o.batch == 1024 * 3 * 128);
  mcs_layout_bhnd(&d, &lay);
  CHECK(lay.k.token == 128 && lay.k.head == 1024 * 128);

  ws = mcs_group_workspace_bytes(&d);
  CHECK(ws > 0);
  CHECK(mcs_anchor_select_min_workspace_bytes(&d, 250) > 0);
  CHECK(mcs_group_kmeans_workspace_bytes(&d) > 0);

  /* validation failures: nothing is enqueued, a message is recorded */
  st = mcs_sparse_attn(&d, NULL, fake, fake, (const int32_t*)fake, (const int32_t*)fake, 5, 0.1f,
                       NULL, fake + 128, NULL);
  CHECK(st == MCS_ERR_INVALID_ARG);
  CHECK(strstr(mcs_last_error(), "q is NULL") != NULL);
  d.head_dim = 80;
  st = mcs_dense_attn(&d, fake, fake, fake, 0.1f, fake + 128, NULL, NULL);
  CHECK(st == MCS_ERR_UNSUPPORTED);
  d.head_dim = 128;
  mcs_layout_bnhd(&d, &lay);
  lay.v.token += 8; /* k and v must share the token stride */
  st = mcs_sparse_attn_strided(&d, &lay, fake, fake, fake, (const int32_t*)fake,
                               (const int32_t*)fake, 5, 0.1f, NULL, fake + 128, NULL);
  CHECK(st == MCS_ERR_UNSUPPORTED);
  st = mcs_group(&d, fake, 20, -1, (int32_t*)fake, (void*)fake, ws - 1, NULL);
  CHECK(st == MCS_ERR_WORKSPACE);
  printf("ok\n");
  return 0;
}
