/* Plain C99 use of the C ABI without a GPU: the header compiles as C, the
   library links, and the host-only calls and argument checks behave as
   documented.  Prints one line per check; exit status 0 when all pass. */
#include <stdio.h>
#include <string.h>

#include "dlc.h"

static int failures = 0;

static void check(int ok, const char* what) {
  printf("%s %s\n", ok ? "ok  " : "FAIL", what);
  if (!ok) ++failures;
}

int main(void) {
  /* greedy bin-packing: 7 5 4 3 3 2 into 2 fragments -> loads 12 and 12 */
  const int64_t numel[6] = {7, 5, 4, 3, 3, 2};
  int32_t frag[6];
  int64_t load[2];
  check(dlc_fragment_plan(numel, 6, 2, frag, load) == DLC_OK, "dlc_fragment_plan returns DLC_OK");
  check(load[0] == 12 && load[1] == 12, "fragment loads 12 and 12");
  check(frag[0] == 0 && frag[1] == 1 && frag[2] == 1 && frag[3] == 0 && frag[4] == 1 && frag[5] == 0,
        "fragment of each tensor");

  dlc_tensor t[2] = {{0, 0, 1 << 20}, {1 << 20, 1 << 20, 4097}};
  size_t bytes = 0;
  check(dlc_workspace_bytes(8, t, 2, &bytes) == DLC_OK && bytes > 0 && bytes % 256 == 0,
        "dlc_workspace_bytes is positive and 256-aligned");
  check(dlc_workspace_bytes(0, t, 2, &bytes) == DLC_ERR_INVALID_ARGUMENT, "zero learners rejected");
  check(strlen(dlc_last_error()) > 0, "dlc_last_error describes the failure");
  check(dlc_ring_workspace_bytes(4, t, 2, &bytes) == DLC_OK && bytes > 0, "dlc_ring_workspace_bytes");
  check(dlc_rda_workspace_bytes(4, t, 2, &bytes) == DLC_OK && bytes > 0, "dlc_rda_workspace_bytes");

  /* merge weights: quorum 2 met at t = 2, grace 0.5 -> learners 0 and 2 */
  const double tokens[4] = {100, 200, 300, 0};
  const double arrival[4] = {1.0, 3.0, 2.0, 1.0 / 0.0};
  double w[4], when = 0.0;
  check(dlc_merge_weights(4, tokens, arrival, 2, 0.5, w, &when) == DLC_OK, "dlc_merge_weights returns DLC_OK");
  check(w[0] == 100 && w[1] == 0 && w[2] == 300 && w[3] == 0 && when == 2.5, "token weights and merge time");

  /* argument errors come back before anything touches a device */
  const double none[2] = {0.0, 0.0};
  check(dlc_merge_outer_step((float*)0x100000, (float*)0x100000, (const uint8_t*)0x100000, 4096, 2,
                             (const float*)0x100000, none, t, 1, 0.7, 0.9, 0, NULL) == DLC_ERR_NO_QUORUM,
        "all-zero weights are a failed quorum");
  check(strstr(dlc_version(), "gfx950") != NULL, "dlc_version names gfx950");
  return failures == 0 ? 0 : 1;
}
