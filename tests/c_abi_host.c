/* A plain C99 consumer of the C ABI (no C++ and no torch): includes
 * include/leank.h, links libleank.so and calls its host-only entry points.
 * Prints one line of values that tests/test_c_abi.py compares with the
 * Python binding. */
#include <stdio.h>

#include "leank.h"

int main(void) {
  const int32_t kept[4] = {32, 0, 64, 8};
  leank_layer_cache c, cq, cp, cpq;
  int st = leank_plan_layer(kept, 3, 8, 4, 128, 4, 61, 1000, &c);
  st |= leank_plan_layer_q(kept, 3, 8, 4, 128, 4, 61, 1000, 4, &cq);
  st |= leank_plan_layer_paged(kept, 3, 8, 4, 128, 4, 61, 1000, 50, &cp);
  st |= leank_plan_layer_paged_q(kept, 3, 8, 4, 128, 4, 61, 1000, 50, 8, &cpq);
  size_t ws = 0;
  int64_t bytes = 0, bytes_q = 0;
  st |= leank_workspace_bytes(&c, 1000, &ws);
  st |= leank_decode_bytes(&c, 1000, &bytes);
  st |= leank_decode_bytes(&cq, 1000, &bytes_q);
  /* a request the library must refuse: head_dim 64 */
  leank_layer_cache bad;
  const int bad_st = leank_plan_layer(kept, 3, 8, 4, 64, 4, 61, 1000, &bad);
  printf("abi=%d size=%zu status=%d ws=%zu bytes=%lld bytes_q=%lld page=%llu page_q=%llu bad=%d\n%s\n",
         leank_abi_version(), leank_layer_cache_size(), st, ws, (long long)bytes,
         (long long)bytes_q, (unsigned long long)cp.page_bytes, (unsigned long long)cpq.page_bytes,
         bad_st, leank_status_string(bad_st));
  return st != LEANK_OK || sizeof(leank_layer_cache) != leank_layer_cache_size();
}
