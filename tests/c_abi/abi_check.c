/* Plain C11 caller of the C ABI (no HIP compiler, no GPU): the header compiles as C, the library links, and the
 * host-side entry points answer. Prints the codebook as hex floats and the storage sizes; a rejected call shows
 * the validation path. Built and run by tests/test_abi.py. */
#include <stdio.h>

#include "qlora.h"

int main(void) {
  float c[16], t[15];
  qlora_nf4_codebook(c);
  qlora_nf4_thresholds(t);
  for (int j = 0; j < 16; ++j) printf("%a\n", (double)c[j]);
  for (int j = 0; j < 15; ++j) printf("%a\n", (double)t[j]);
  printf("%zu %zu %zu\n", qlora_storage_bytes(4096, 4096), qlora_storage_bytes_absmax(4096, 4096),
         qlora_workspace_bytes(4096, 4096, 16, 64));
  /* d_in = 100 is not a multiple of 64: refused on the host, nothing enqueued */
  qlora_nf4_weight w = {64, 100, (uint8_t *)0x10000, (uint8_t *)0x10000, (float *)0x10000};
  const int s = qlora_dequantize(&w, QLORA_BF16, (void *)0x10000, 0);
  printf("%d %s\n", s, qlora_status_string(s));
  return s == QLORA_ERR_SHAPE ? 0 : 1;
}
