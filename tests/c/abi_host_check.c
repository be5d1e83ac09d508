/* A C99 program that includes libmoe.h and links libmoe.so: the header is
 * plain C, and host-side calls (queries, argument validation, error
 * strings) work without touching a GPU. Prints "ok" and exits 0 on success.
 * Built and run by tests/test_abi_c.py. */
#include <stdio.h>
#include <string.h>

#include "libmoe.h"

#define EXPECT(cond)                                                     \
  do {                                                                   \
    if (!(cond)) {                                                       \
      fprintf(stderr, "%s:%d: failed: %s (last error: %s)\n", __FILE__, \
              __LINE__, #cond, moe_last_error());                        \
      return 1;                                                          \
    }                                                                    \
  } while (0)

int main(void) {
  /* capacity = ceil(N * CF / E) */
  EXPECT(moe_capacity(256, 4, 5, 4) == 80);
  EXPECT(moe_capacity(16384, 64, 1, 1) == 256);
  EXPECT(moe_capacity(10, 3, 1, 1) == 4);
  EXPECT(moe_capacity(257, 4, 5, 4) == 81);
  EXPECT(moe_capacity(100, 10, 11, 10) == 11);
  EXPECT(moe_capacity(10, 3, 1, 0) == -1);
  EXPECT(moe_router_workspace_bytes(4096, 4096, 8, 0) > 0);
  EXPECT(moe_dispatch_workspace_bytes(8192, 256, 8) > 0);
  EXPECT(moe_router_backward_workspace_bytes(4096, 4096, 8) > 0);

  /* validation happens before any launch: a NULL params pointer, more than
   * 256 experts, and a dropping policy without a capacity */
  EXPECT(moe_router_topk(NULL, NULL, MOE_BF16, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                         0, NULL) == MOE_EINVAL);
  moe_router_params p;
  memset(&p, 0, sizeof p);
  p.n_tokens = 16;
  p.d_model = 64;
  p.n_experts = 300;
  p.top_k = 2;
  p.n_cand = 2;
  p.renormalize = 1;
  char fake[16];
  EXPECT(moe_router_topk(&p, fake, MOE_BF16, (const float*)fake, NULL, (int32_t*)fake,
                         (float*)fake, (float*)fake, NULL, NULL, fake, (size_t)1 << 30,
                         NULL) == MOE_EUNSUPPORTED);
  EXPECT(strstr(moe_last_error(), "256") != NULL);
  EXPECT(moe_dispatch(16, 4, 1, 1, MOE_DROP, -1, (const int32_t*)fake, (const float*)fake,
                      (float*)fake, NULL, MOE_BF16, 0, (int32_t*)fake, (int32_t*)fake,
                      (int32_t*)fake, (int32_t*)fake, (int32_t*)fake, (int32_t*)fake, NULL,
                      fake, (size_t)1 << 30, NULL) == MOE_EINVAL);
  /* router weight planes: 3 planes of E (or 2E) rows padded to 64 */
  EXPECT(moe_router_planes_bytes(8, 4096, 0) == (size_t)3 * 64 * 4096 * 2);
  EXPECT(moe_router_planes_bytes(64, 1024, 1) == (size_t)3 * 128 * 1024 * 2);
  EXPECT(moe_router_prepare((const float*)fake, NULL, 8, 100, fake, (size_t)1 << 30, NULL) ==
         MOE_EINVAL);
  EXPECT(moe_router_prepare((const float*)fake, NULL, 8, 64, fake, 16, NULL) == MOE_EWORKSPACE);
  EXPECT(moe_router_prepare((const float*)fake, NULL, 300, 64, fake, (size_t)1 << 30, NULL) ==
         MOE_EUNSUPPORTED);
  EXPECT(strlen(moe_status_string(MOE_EWORKSPACE)) > 0);
  EXPECT(strlen(moe_version()) > 0);
  printf("ok %s\n", moe_version());
  return 0;
}
