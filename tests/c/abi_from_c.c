/* Plain C99 user of the C ABI: includes pa.h, links the library and calls its host-only entry
 * points (no GPU needed).  Prints one line per check; exits non-zero on the first failure. */
#include <stdio.h>
#include <string.h>

#include "pa.h"

#define CHECK(cond)                                       \
  do {                                                    \
    if (!(cond)) {                                        \
      printf("FAIL %s (line %d)\n", #cond, __LINE__);     \
      return 1;                                           \
    }                                                     \
    printf("ok %s\n", #cond);                             \
  } while (0)

int main(void) {
  pa_desc d;
  memset(&d, 0, sizeof d);
  d.num_seqs = 4;
  d.num_q_tokens = 4;
  d.num_q_heads = 32;
  d.num_kv_heads = 8;
  d.head_dim = 128;
  d.page_size = PA_PAGE_SIZE;
  d.num_pages = 64;
  d.max_pages_per_seq = 16;
  d.max_seq_len = 0;
  d.dtype = PA_BF16;
  d.scale = 0.0883883f;
  CHECK(pa_abi_version() == PA_ABI_VERSION);
  CHECK(pa_check_desc(&d) == PA_OK);
  CHECK(pa_check_desc(NULL) == PA_ERR_NULL_POINTER);
  d.head_dim = 96;
  CHECK(pa_check_desc(&d) == PA_ERR_UNSUPPORTED);
  CHECK(pa_workspace_bytes(&d) == 0);
  d.head_dim = 128;
  d.num_q_heads = 30; /* not a multiple of num_kv_heads */
  CHECK(pa_check_desc(&d) == PA_ERR_BAD_SHAPE);
  CHECK(strlen(pa_status_str(PA_ERR_WORKSPACE_TOO_SMALL)) > 0);
  CHECK(pa_status_str((pa_status)12345) != NULL);
  CHECK(pa_attention(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == PA_ERR_NULL_POINTER);
  CHECK(pa_read_stream(NULL, 1024, 4, NULL, NULL) == PA_ERR_NULL_POINTER);
  printf("done\n");
  return 0;
}
