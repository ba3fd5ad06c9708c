/* A plain C99 program against include/infv2.h and libinfv2.so: the header
 * compiles as C with every warning an error, the library links, and calls
 * that fail validation return their codes without touching the GPU. */
#include <stdio.h>
#include <string.h>

#include "infv2.h"

int main(void) {
  void* fake = (void*)0x10000; /* aligned, never dereferenced: validation fails first */
  if (infv2_abi_version() < 1) return 1;
  if (strcmp(infv2_status_string(INFV2_OK), "ok") != 0) return 2;
  if (infv2_compress_k(fake, fake, 1, 1, 64, 64, 64, NULL) != INFV2_ERR_UNSUPPORTED) return 3; /* D = 64 */
  if (infv2_compress_v(fake, NULL, 1, 1, 64, 128, 64, NULL) != INFV2_ERR_INVALID) return 4;
  if (infv2_sparse_workspace_bytes(1, 32, 2, 32768, 32768, 128, 64, 64) != 0) return 5;
  if (infv2_compressed_attn_fwd(fake, fake, fake, NULL, fake, NULL, 1, 32, 2, 10, 9, 128, 64, 0.0f, 0.0f, 1.0f,
                                NULL) != INFV2_ERR_INVALID) /* S_q > S_k */
    return 6;
  if (infv2_attn_path(4096, 4096) != INFV2_PATH_DENSE || infv2_attn_path(4097, 4096) != INFV2_PATH_SPARSE) return 7;
  printf("c abi ok\n");
  return 0;
}
