/* The C ABI from plain C: include/uniprefill.h must compile as C99 with
 * -pedantic and no warnings, and a C program linked against libuniprefill.so
 * can size workspaces and gets the documented status codes for bad arguments.
 * Every call here returns before any HIP work, so no GPU is needed.  Prints one
 * "name value" line per check for the test that builds and runs it. */
#include <stdio.h>

#include "uniprefill.h"
#include "uniprefill_prof.h"

#define FAKE ((void*)(1u << 20)) /* nonzero, aligned, never dereferenced */

int main(void) {
  up_select_params prm;
  prm.num_heads_q = 32;
  prm.num_heads_kv = 8;
  prm.head_dim = 128;
  prm.block_size = 64;
  prm.num_sink = 128;
  prm.window = 128;
  prm.top_p = 0.99;
  prm.softmax_scale = 0.0f;
  prm.flags = 0u;

  printf("max_blocks %lld\n", (long long)up_max_blocks(64, 1, 131072));
  printf("select_ws_positive %d\n", up_select_workspace_bytes(&prm, 1, 131072) > 0);
  printf("compact_ws_positive %d\n", up_compact_workspace_bytes(1, 131072) > 0);
  printf("status_ok %s\n", up_status_string(UP_OK) != NULL ? "set" : "null");
  printf("select_null_params %d\n",
         (int)up_select_blocks(NULL, FAKE, 4096, FAKE, 1024, FAKE, 1, 4096, NULL, FAKE, FAKE, FAKE, FAKE, FAKE,
                               FAKE, (size_t)1 << 30, NULL));
  prm.top_p = 1.5;
  printf("select_bad_p %d\n",
         (int)up_select_blocks(&prm, FAKE, 4096, FAKE, 1024, FAKE, 1, 4096, NULL, FAKE, FAKE, FAKE, FAKE, FAKE,
                               FAKE, (size_t)1 << 30, NULL));
  printf("select_profiled_bad_p %d\n",
         (int)up_select_blocks_profiled(&prm, FAKE, 4096, FAKE, 1024, FAKE, 1, 4096, NULL, FAKE, FAKE, FAKE,
                                        FAKE, FAKE, FAKE, (size_t)1 << 30, NULL, NULL, NULL));
  prm.top_p = 0.99;
  printf("select_small_workspace %d\n",
         (int)up_select_blocks(&prm, FAKE, 4096, FAKE, 1024, FAKE, 1, 4096, NULL, FAKE, FAKE, FAKE, FAKE, FAKE,
                               FAKE, 16, NULL));
  printf("scatter_odd_rows %d\n", (int)up_scatter_back(FAKE, 3, FAKE, FAKE, 1, 10, FAKE, 10, NULL));
  printf("metadata_negative_layer %d\n",
         (int)up_update_metadata(-1, 4, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, NULL));
  return 0;
}
