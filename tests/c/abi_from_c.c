/*
 * The C ABI used from plain C (C11, no C++ and no Python): include the
 * header, link the library, make the host-side calls that need no GPU
 * (workspace sizes, pyramid budgets, status strings, argument errors) and
 * print one line per check.  Exit status 0 when every check holds.
 */
#include <stdio.h>
#include <string.h>

#include "triattn.h"

static int failures = 0;

static void check(int ok, const char* what) {
  printf("%s %s\n", ok ? "ok  " : "FAIL", what);
  if (!ok) ++failures;
}

int main(void) {
  tri_shape sh;
  memset(&sh, 0, sizeof sh);
  sh.head_dim = 128;
  sh.num_q_heads = 28;
  sh.num_kv_heads = 4;
  sh.num_layers = 28;
  sh.rope_theta = 10000.0;
  sh.rope_layout = TRI_ROPE_INTERLEAVED;

  const int64_t cu[3] = {0, 32768, 65536};
  const size_t ws = tri_workspace_bytes(&sh, 2, cu);
  check(ws > 0, "tri_workspace_bytes > 0 for two 32768-key sequences");
  check(tri_workspace_bytes(&sh, 2, NULL) == 0, "tri_workspace_bytes without cu_len is 0");

  int32_t b[28];
  check(tri_pyramid_budgets(28, 2048.0, 3.0, b) == TRI_OK, "tri_pyramid_budgets succeeds");
  long sum = 0;
  for (int l = 0; l < 28; ++l) sum += b[l];
  check(b[0] < b[27] && sum >= 28 * 2048 - 28 && sum <= 28 * 2048 + 28,
        "pyramid budgets rise and keep the mean");

  check(strcmp(tri_status_string(TRI_OK), "TRI_OK") == 0, "tri_status_string(TRI_OK)");
  check(strcmp(tri_status_string(TRI_ERR_WORKSPACE), "TRI_ERR_WORKSPACE") == 0,
        "tri_status_string(TRI_ERR_WORKSPACE)");

  /* argument errors return before any device work: no GPU needed */
  tri_shape bad = sh;
  bad.head_dim = 130;
  check(tri_workspace_bytes(&bad, 2, cu) == 0, "head_dim 130 is rejected");
  const int32_t budget[2] = {2048, -1};
  tri_status st = tri_select_compact(&sh, 2, cu, budget, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                                     NULL, NULL, 0, NULL);
  check(st == TRI_ERR_INVALID_ARGUMENT, "a negative budget is an invalid argument");
  check(strlen(tri_last_error()) > 0, "tri_last_error explains it");

  printf("%d failure(s)\n", failures);
  return failures == 0 ? 0 : 1;
}
