/* A C99 program that includes the library's header and links against libwqmlp.so, so the C ABI is
 * checked from C itself: the header compiles as strict C, the symbols resolve at link and load time,
 * and calls that fail the pure-argument checks return their codes without touching a GPU. */
#include <stdio.h>
#include <string.h>

#include "wqmlp.h"

int main(void) {
  if (wq_abi_version() != WQ_ABI_VERSION) return 1;
  /* a null x with M > 0 fails the argument checks, before any device call */
  if (mlp_fp8w_run(1, 64, 64, NULL, WQ_BF16, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL, 0, NULL) != WQ_EINVAL)
    return 2;
  if (mlp_nvfp4_run(1, 96, 64, NULL, WQ_BF16, NULL, 1.0f, NULL, 1.0f, NULL, 1.0f, NULL, 0, NULL, 0, NULL) != WQ_EINVAL)
    return 3;
  /* an unknown metadata layout has no bank size */
  if (awq_bank_bytes(1, 64, 64, 5) != 0) return 4;
  if (awq_bank_bytes(2, 64, 64, 3) == 0) return 5;
  if (strlen(wq_strerror(WQ_EALIGN)) == 0 || wq_last_hip_error() != 0) return 6;
  printf("c consumer ok\n");
  return 0;
}
