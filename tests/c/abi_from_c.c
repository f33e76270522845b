/* A C99 caller of libdamp.so that needs no GPU: it includes the public header as plain C, links
 * the library, and prints what the host-side entry points return (sizes, statuses and the error
 * text of rejected calls). tests/test_abi.py builds it with gcc -std=c99 -pedantic -Werror and
 * compares each line with the same calls made through the Python binding. */
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>

#include "damp.h"

int main(void) {
  damp_layout L = {4096, 32, 128, 128, 24};
  damp_layout small = {64, 2, 16, 16, 2};
  damp_layout bad = {0, 32, 128, 128, 24};
  int32_t r_per_head[2] = {2, 5};
  uint8_t bits[2 * 16];
  damp_state* st = NULL;
  damp_status rc;
  int i;
  for (i = 0; i < 2 * 16; ++i) bits[i] = (uint8_t)(i % 16 < 2 ? 16 : (i % 16 < 6 ? 8 : (i % 16 < 11 ? 6 : 4)));
  printf("block_bytes %zu\n", damp_block_bytes(&L));
  printf("block_data_bytes %zu\n", damp_block_data_bytes(&L));
  printf("state_bytes %zu\n", damp_state_bytes(&L));
  printf("window_bytes_8 %zu\n", damp_window_bytes(&L, 8));
  printf("window_bytes_9 %zu\n", damp_window_bytes(&L, 9));
  printf("state_bytes_per_head %zu\n", damp_state_bytes_per_head(&small, r_per_head));
  printf("stq_state_bytes %zu\n", stq_state_bytes(64, 2, 16, bits));
  rc = damp_state_alloc(&bad, NULL, NULL, 0, &st);
  printf("alloc_bad %d %s\n", (int)rc, damp_last_error());
  rc = damp_decode_step(NULL, NULL, 1, NULL, NULL, NULL, DAMP_BF16, NULL, DAMP_DECAY_SCALAR, NULL,
                        NULL, NULL);
  printf("step_null %d %s\n", (int)rc, damp_last_error());
  return 0;
}
