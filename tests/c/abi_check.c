/* A C99 consumer of include/swr.h: compiles the header as C and calls the
 * host-only layout planner (no GPU needed).  Expected values are the closed
 * form of the flat layout (weight_sharding, section "one AllGather per layer:
 * flat layout"): items on 16-byte boundaries in order, the total rounded up to
 * a multiple of 16*N, C = |T| / N.  For BF16 [512 x 128], [128 x 256],
 * [100 x 128] at N = 4 the items are 131072, 65536 and 25600 bytes, so the
 * offsets are 0, 131072, 196608 and |T| = 222208, C = 55552. */
#include <stdio.h>
#include <string.h>

#include "swr.h"

static int fails = 0;
#define CHECK(cond)                                                \
  do {                                                             \
    if (!(cond)) {                                                 \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++fails;                                                     \
    }                                                              \
  } while (0)

int main(void) {
  swr_weight_desc w[3];
  swr_view_desc v[3];
  swr_layout lay;
  const int64_t shapes[3][2] = {{512, 128}, {128, 256}, {100, 128}};
  const int64_t offsets[3] = {0, 131072, 196608};
  int i;
  memset(w, 0, sizeof(w));
  for (i = 0; i < 3; ++i) {
    w[i].out_features = shapes[i][0];
    w[i].in_features = shapes[i][1];
    w[i].dtype = SWR_BF16;
  }
  CHECK(swr_plan_layer(w, 3, 4, v, &lay) == SWR_OK);
  for (i = 0; i < 3; ++i) {
    CHECK(v[i].offset == offsets[i]);
    CHECK(v[i].nbytes == shapes[i][0] * shapes[i][1] * 2);
  }
  CHECK(lay.payload_bytes == 222208);
  CHECK(lay.total_bytes == 222208);
  CHECK(lay.chunk_bytes == 55552);
  CHECK(lay.n_chunks == 4 && lay.n_weights == 3);
  /* an error comes back as a status with a message, before any work */
  CHECK(swr_plan_layer(w, 3, 0, v, &lay) == SWR_E_INVALID);
  CHECK(strlen(swr_last_error()) > 0);
  CHECK(strstr(swr_version(), "gfx950") != NULL);
  if (fails == 0) printf("c abi ok\n");
  return fails == 0 ? 0 : 1;
}
