/* A plain C99 client of the library: includes the public header, links
 * libw4a4.so and calls entry points that need no GPU (the version, the
 * split-attention size query, and argument validation, which runs before
 * any device is touched).  Built and run by tests/test_abi_c_client.py;
 * prints "c client ok" and exits 0 when every check holds. */
#include <stdio.h>
#include <string.h>

#include "w4a4.h"

static int fails = 0;

static void check(int cond, const char* what) {
  if (!cond) {
    ++fails;
    printf("FAIL %s (%s)\n", what, w4a4_last_error());
  }
}

int main(void) {
  static _Alignas(16) unsigned char buf[1024];
  check(w4a4_abi_version() == W4A4_ABI_VERSION, "ABI version of the loaded library matches the header");
  check(kv4_attention_workspace_bytes(1, 8, 32768) == 8 * 32 * 528, "split workspace size");
  check(kv4_attention_workspace_bytes(8, 32, 4096) == 0, "single pass needs no workspace");
  check(kv4_attention_workspace_bytes(1, 8, 0) == -1 && strlen(w4a4_last_error()) > 0, "bad S is refused");
  /* NULL input: refused before any device call */
  check(rotate_quant_act(NULL, 4, 128, 128, W4A4_HAD_128, NULL, W4A4_ACT_SYM_TOKEN, buf, (float*)buf, NULL, NULL) ==
            W4A4_ERR_NULL,
        "rotate_quant_act NULL input");
  /* K not a multiple of 128 */
  check(rotate_quant_act((const uint16_t*)buf, 4, 100, 100, W4A4_HAD_128, NULL, W4A4_ACT_SYM_TOKEN, buf, (float*)buf,
                         NULL, NULL) == W4A4_ERR_SHAPE,
        "rotate_quant_act ragged K");
  /* an empty batch is a no-op that touches nothing */
  check(w4a4_gemm(NULL, NULL, NULL, W4A4_ACT_SYM_TOKEN, NULL, NULL, NULL, 0, 16, 128, NULL, 16, NULL) == W4A4_OK,
        "w4a4_gemm with M = 0");
  if (fails) {
    printf("c client: %d checks failed\n", fails);
    return 1;
  }
  printf("c client ok\n");
  return 0;
}
