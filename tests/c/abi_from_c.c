/* A plain C99 caller of the attention library: it includes the public header
 * with a C compiler, links against the shared library and exercises the calls
 * that need no GPU (version, status strings, workspace sizes, argument
 * rejection before any HIP call). Prints one "ok" line per check; any failed
 * check prints "FAIL" and the program exits with status 1. */
#include <stdio.h>
#include <string.h>

#include "tiled_attn.h"

static int failures = 0;

static void check(int cond, const char* what) {
  printf("%s %s\n", cond ? "ok" : "FAIL", what);
  if (!cond) ++failures;
}

int main(void) {
  check(attn_version() >= 1, "version");
  check(strlen(attn_status_string(ATTN_OK)) > 0, "status string of ATTN_OK");
  check(strlen(attn_status_string(ATTN_ERR_INVALID_ARGUMENT)) > 0, "status string of an error");

  /* one float per query row: B * H * N */
  check(attn_bwd_workspace_bytes(2, 16, 4096, 128, ATTN_BF16) == (size_t)2 * 16 * 4096 * 4, "workspace bytes");
  check(attn_bwd_workspace_bytes(2, 16, 4096, 96, ATTN_BF16) == 0, "workspace bytes of an unsupported d");

  /* invalid arguments are rejected before any HIP call, with a message */
  attn_status s = attn_fwd(NULL, NULL, NULL, NULL, NULL, 1, 1, 64, 64, 1.f, ATTN_BF16, NULL);
  check(s == ATTN_ERR_INVALID_ARGUMENT, "forward with null pointers");
  check(strlen(attn_last_error()) > 0, "last error message");
  float dummy[64];
  s = attn_fwd(dummy, dummy, dummy, dummy, dummy, 1, 1, 64, 96, 1.f, ATTN_BF16, NULL);
  check(s == ATTN_ERR_UNSUPPORTED, "forward with d = 96");
  s = attn_bwd_ex_noalloc(dummy, dummy, dummy, dummy, dummy, dummy, dummy, dummy, dummy, 1, 1, 8, 8, 64, -1.f,
                          ATTN_MASK_NONE, ATTN_BF16, NULL);
  check(s == ATTN_ERR_INVALID_ARGUMENT, "allocation-free backward with a negative scale");
  return failures ? 1 : 0;
}
