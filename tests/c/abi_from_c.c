/* The C ABI used from plain C11: include/vx.h compiles as C, the library
 * links, and host-side validation answers without a GPU (every call below
 * fails its argument checks before any HIP call). Exit 0 on success. */
#include <stdio.h>
#include <string.h>

#include "vx.h"

static int expect(vx_status got, vx_status want, const char* what) {
  if (got != want) {
    printf("%s: %s (%s), wanted %s\n", what, vx_status_string(got), vx_last_error(),
           vx_status_string(want));
    return 1;
  }
  return 0;
}

int main(void) {
  int bad = 0;
  vx_pages p;
  memset(&p, 0, sizeof p);
  vx_geom g = {16, 8, 128, 128, 0, VX_BF16, VX_BF16, 0, 0};
  p.page_size = 32;  /* unsupported page size */
  bad |= expect(vx_page_scores(&p, &g, NULL, NULL, 1.0f, NULL, NULL), VX_ERR_UNSUPPORTED,
                "page_scores P=32");
  p.page_size = 16;
  bad |= expect(vx_page_scores(NULL, &g, NULL, NULL, 1.0f, NULL, NULL), VX_ERR_INVALID_ARG,
                "page_scores pages NULL");
  vx_geom mla = {32, 1, 576, 512, 1, VX_BF16, VX_BF16, 0, 0};
  bad |= expect(vx_bounds_update(&p, &mla, NULL, NULL, NULL, NULL), VX_ERR_UNSUPPORTED,
                "bounds_update MLA");
  vx_geom cb = g;
  cb.score_bf16 = 2; /* only 0 or 1 */
  bad |= expect(vx_page_scores(&p, &cb, NULL, NULL, 1.0f, NULL, NULL), VX_ERR_INVALID_ARG,
                "page_scores score_bf16 2");
  /* an empty batch is a no-op */
  bad |= expect(vx_topk_pages(&p, 8, NULL, 4, 1, 1, VX_TOPK_EXACT, NULL, NULL, 6, NULL, NULL),
                VX_OK, "topk empty batch");
  if (vx_abi_version() < 1) bad = 1;
  if (strcmp(vx_status_string(VX_ERR_WORKSPACE), "VX_ERR_WORKSPACE") != 0) bad = 1;
  printf("%s\n", bad ? "FAIL" : "ok");
  return bad;
}
