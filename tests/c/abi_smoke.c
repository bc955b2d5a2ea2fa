/* Plain-C consumer of the library: the header compiles as C99 and the
 * entry points link and validate arguments without a GPU (every call below
 * fails validation before any launch). Built and run by tests/test_abi.py. */
#include <stdio.h>
#include <string.h>

#include "hsa.h"

int main(void) {
  int32_t n_pad = 0, nb = 0;
  if (hsa_abi_version() != HSA_ABI_VERSION) return 1;
  if (hsa_plan_size(21, 30, 52, HSA_ORDER_HILBERT3D, 128, &n_pad, &nb) != HSA_OK) return 2;
  if (n_pad != 32768 || nb != 256) return 3;
  if (hsa_plan_size(0, 30, 52, HSA_ORDER_ROW, 128, &n_pad, &nb) != HSA_ERR_BAD_SHAPE) return 4;
  if (strlen(hsa_last_error()) == 0) return 5;
  hsa_select_params_t p;
  memset(&p, 0, sizeof p);
  p.mode = HSA_SELECT_RADIAL;
  p.frames = 61;
  p.tiles_per_frame = 13;
  p.lam = 0.125;
  if (hsa_select_list_width(12, 793, &p) != 169) return 6;
  if (hsa_attn(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 4, 0, 2, 4, 64, 64, HSA_BF16,
               0.125f, NULL) != HSA_ERR_NULL_PTR)
    return 7;
  if (hsa_attn_tokens(NULL, NULL, NULL, NULL, 256, 0, 256, NULL, NULL, 100, NULL, NULL, NULL, NULL, 4,
                      0, 2, 4, 64, 64, HSA_BF16, 0.125f, NULL) != HSA_ERR_NULL_PTR)
    return 8;
  printf("ok %d %s\n", hsa_abi_version(), hsa_status_str(HSA_ERR_WORKSPACE));
  return 0;
}
