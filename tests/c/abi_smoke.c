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

  /* plans and workspace sizes of the other calls: many tensors (several launches),
     ragged sizes (empty ring chunks), the largest tensor, empty fragments */
  enum { kMany = 3000 };
  static int64_t many_numel[kMany];
  static int32_t many_frag[kMany];
  static dlc_tensor many[kMany];
  int64_t pos = 0, total = 0;
  for (int i = 0; i < kMany; ++i) {
    many_numel[i] = i < 2000 ? 4096 : i < 2900 ? 1024 * 1024 : i < 2990 ? 4096 * 11008 : 4096;
    many[i].offset = many[i].loffset = pos;
    many[i].numel = many_numel[i];
    pos += (many_numel[i] + 63) / 64 * 64;
    total += many_numel[i];
  }
  int64_t loads24[24];
  check(dlc_fragment_plan(many_numel, kMany, 24, many_frag, loads24) == DLC_OK, "plan of 3000 tensors");
  int64_t sum = 0;
  for (int f = 0; f < 24; ++f) sum += loads24[f];
  check(sum == total, "the 24 fragment loads add up to the set");
  check(dlc_workspace_bytes(16, many, kMany, &bytes) == DLC_OK && bytes > 0, "workspace of 3000 tensors, K = 16");
  check(dlc_rda_workspace_bytes(64, many, 400, &bytes) == DLC_OK && bytes > 0, "RDA workspace of 400 tensors, K = 64");
  const dlc_tensor ragged[5] = {{0, 0, 1}, {64, 64, 63}, {128, 128, 65}, {256, 256, 4097},
                                {4416, 4416, 100003}};
  const int32_t ks[4] = {1, 2, 7, 64};
  for (int j = 0; j < 4; ++j) {
    char what[64];
    snprintf(what, sizeof what, "ring workspace of ragged tensors, K = %d", (int)ks[j]);
    check(dlc_ring_workspace_bytes(ks[j], ragged, 5, &bytes) == DLC_OK && bytes > 0, what);
  }
  const dlc_tensor big[1] = {{0, 0, 4294967295LL}};
  check(dlc_workspace_bytes(1, big, 1, &bytes) == DLC_OK && bytes > 0, "workspace of a 2^32 - 1 tensor");
  const int32_t first[5] = {0, 2, 2, 5, 5};
  check(dlc_cycle_workspace_bytes(4, ragged, first, 4, &bytes) == DLC_OK && bytes > 0,
        "cycle workspace with empty fragments");
  size_t rda_bytes = 0;
  check(dlc_cycle_rda_workspace_bytes(4, ragged, first, 4, &rda_bytes) == DLC_OK && rda_bytes > bytes,
        "RDA cycle workspace exceeds the cycle's");
  const int32_t bad_first[3] = {0, 3, 2};
  check(dlc_cycle_workspace_bytes(4, ragged, bad_first, 2, &bytes) == DLC_ERR_INVALID_ARGUMENT,
        "decreasing fragment_first rejected");

  /* argument errors of every call that launches work: each returns before anything
     is enqueued (the pointers are never dereferenced) */
  float* const F = (float*)0x100000;
  uint8_t* const U = (uint8_t*)0x100000;
  void* const W = (void*)0x100000;
  const double ones[4] = {1.0, 1.0, 1.0, 1.0};
  const dlc_tensor overlap[2] = {{0, 0, 128}, {64, 128, 64}};
  const dlc_tensor misaligned[1] = {{32, 0, 64}};
  const dlc_tensor empty_tensor[1] = {{0, 0, 0}};
  const dlc_tensor too_big[1] = {{0, 0, 4294967296LL}};
  check(dlc_quantize(F, F, 4096, 2, NULL, t, 1, U, F, F, 16u, W, 1 << 20, NULL) == DLC_ERR_INVALID_ARGUMENT,
        "unknown quantize flag");
  check(dlc_quantize(F, F, 4096, 2, NULL, t, 1, U, F, F, DLC_RANGE_GIVEN | DLC_DEBUG_CHECKS, W, 1 << 20, NULL) ==
            DLC_ERR_INVALID_ARGUMENT,
        "debug checks need the statistics stage");
  check(dlc_quantize(F, F, 256, 2, NULL, overlap, 2, U, F, F, 0, W, 1 << 20, NULL) == DLC_ERR_INVALID_ARGUMENT,
        "overlapping tensors rejected");
  check(dlc_quantize(F, F, 256, 2, NULL, misaligned, 1, U, F, F, 0, W, 1 << 20, NULL) == DLC_ERR_ALIGNMENT,
        "misaligned offset rejected");
  check(dlc_quantize(F, F, 256, 2, NULL, empty_tensor, 1, U, F, F, 0, W, 1 << 20, NULL) == DLC_ERR_INVALID_ARGUMENT,
        "empty tensor rejected");
  check(dlc_quantize(F, F, 4294967360LL, 2, NULL, too_big, 1, U, F, F, 0, W, 1 << 20, NULL) ==
            DLC_ERR_INVALID_ARGUMENT,
        "tensor of 2^32 elements rejected");
  check(dlc_quantize(F, F, 100, 2, NULL, misaligned, 1, U, F, F, 0, W, 1 << 20, NULL) == DLC_ERR_ALIGNMENT,
        "learner_stride not a multiple of 64 rejected");
  check(dlc_quantize(F, F, 4096, 65, NULL, t, 1, U, F, F, 0, W, 1 << 20, NULL) == DLC_ERR_INVALID_ARGUMENT,
        "65 learners rejected");
  check(dlc_quantize(F, F, 1 << 22, 2, NULL, t, 2, U, F, F, 0, W, 256, NULL) == DLC_ERR_WORKSPACE,
        "small workspace rejected");
  check(dlc_quantize(F, F, 1 << 22, 2, NULL, t, 2, U, F, F, 0, (void*)0x100008, (size_t)1 << 40, NULL) ==
            DLC_ERR_ALIGNMENT,
        "unaligned workspace rejected");
  const uint8_t nobody[2] = {0, 0};
  check(dlc_quantize_range(F, F, 1 << 22, 2, nobody, t, 2, F, W, 1 << 20, NULL) == DLC_ERR_NO_QUORUM,
        "no learner present");
  const float* bases[2] = {F, NULL};
  check(dlc_quantize_bases(bases, F, 4096, 2, NULL, t, 1, U, F, F, W, 1 << 20, NULL) == DLC_ERR_INVALID_ARGUMENT,
        "NULL base rejected");
  check(dlc_merge_outer_step(F, F, U, 4096, 2, F, ones, t, 1, 0.7, 0.9, 1u, NULL) == DLC_ERR_INVALID_ARGUMENT,
        "merge flags must be 0");
  const double negative[2] = {1.0, -1.0};
  check(dlc_merge_outer_step(F, F, U, 4096, 2, F, negative, t, 1, 0.7, 0.9, 0, NULL) == DLC_ERR_INVALID_ARGUMENT,
        "negative weight rejected");
  check(dlc_broadcast(F, (float*)0x100004, 4096, 2, NULL, t, 1, NULL) == DLC_ERR_ALIGNMENT,
        "unaligned broadcast rejected");
  const double cycle_w[8] = {1.0, 1.0, 0.0, 0.0, 1.0, 0.0, 1.0, 1.0};  /* fragment 1 has no quorum */
  const int32_t cycle_first[4] = {0, 2, 4, 5};
  check(dlc_outer_cycle(F, F, F, 1 << 20, 2, cycle_w, ragged, cycle_first, 3, U, F, F, 0.7, 0.9, 0, W,
                        (size_t)1 << 40, NULL, NULL) == DLC_ERR_NO_QUORUM,
        "a cycle with one fragment short of its quorum enqueues nothing");
  check(dlc_outer_cycle(F, F, F, 1 << 20, 2, ones, ragged, cycle_first, 3, U, F, F, 0.7, 0.9, 64u, W,
                        (size_t)1 << 40, NULL, NULL) == DLC_ERR_INVALID_ARGUMENT,
        "unknown cycle flag");
  void* streams[9] = {0};
  check(dlc_outer_cycle_lanes(F, F, F, 1 << 20, 2, ones, ragged, cycle_first, 3, U, F, F, 0.7, 0.9, 0, W,
                              (size_t)1 << 40, streams, 0) == DLC_ERR_INVALID_ARGUMENT,
        "zero lanes rejected");
  check(dlc_outer_cycle_lanes(F, F, F, 1 << 20, 2, ones, ragged, cycle_first, 3, U, F, F, 0.7, 0.9, 0, W,
                              (size_t)1 << 40, streams, 9) == DLC_ERR_INVALID_ARGUMENT,
        "nine lanes rejected");
  check(dlc_outer_cycle_rda(F, F, F, 1 << 20, 2, ones, ragged, cycle_first, 3, U, F, F, NULL, 0.7, 0.9, 0, W,
                            (size_t)1 << 40, streams, 1) == DLC_ERR_INVALID_ARGUMENT,
        "RDA cycle: NULL sq_norms rejected");
  check(dlc_outer_cycle_rda(F, F, F, 1 << 20, 2, cycle_w, ragged, cycle_first, 3, U, F, F, (double*)F, 0.7, 0.9, 0,
                            W, (size_t)1 << 40, streams, 2) == DLC_ERR_NO_QUORUM,
        "RDA cycle: a fragment short of its quorum enqueues nothing");
  check(dlc_outer_cycle_rda(F, F, F, 1 << 20, 2, ones, ragged, cycle_first, 3, U, F, F, (double*)F, 0.7, 0.9, 0, W,
                            512, streams, 2) == DLC_ERR_WORKSPACE,
        "RDA cycle: small lane shares rejected");
  check(dlc_outer_cycle_rda(F, F, F, 1 << 20, 2, ones, ragged, cycle_first, 3, U, F, F, (double*)F, 0.7, 0.9,
                            DLC_TWO_LANES, W, (size_t)1 << 40, streams, 2) == DLC_ERR_INVALID_ARGUMENT,
        "RDA cycle: unknown flag");
  check(dlc_ring_outer_step(F, F, F, 1 << 20, 7, ragged, 5, 0.7, 0.9, F, U, F, F, W, 256, NULL) ==
            DLC_ERR_WORKSPACE,
        "ring: small workspace rejected");
  check(dlc_ring_outer_step(F, F, F, 1 << 20, 7, ragged, 5, 1.0 / 0.0, 0.9, F, U, F, F, W, (size_t)1 << 40,
                            NULL) == DLC_ERR_INVALID_ARGUMENT,
        "ring: infinite lr rejected");
  const double zeros4[4] = {0.0, 0.0, 0.0, 0.0};
  check(dlc_rda_outer_step(F, F, F, NULL, 1 << 20, 4, ragged, 5, zeros4, 0.7, 0.9, U, F, F, (double*)F, W,
                           (size_t)1 << 40, NULL) == DLC_ERR_NO_QUORUM,
        "RDA: all-zero weights are a failed quorum");
  check(dlc_rda_outer_step(F, F, F, NULL, 1 << 20, 4, ragged, 5, ones, 0.7, 0.9, U, F, F, (double*)F, W, 256, NULL) ==
            DLC_ERR_WORKSPACE,
        "RDA: small workspace rejected");
  check(dlc_merge_weights(4, tokens, arrival, 4, 0.5, w, &when) == DLC_ERR_NO_QUORUM,
        "quorum of 4 with 3 arrivals fails");
  check(dlc_merge_weights(4, tokens, arrival, 2, -1.0, w, &when) == DLC_ERR_INVALID_ARGUMENT,
        "negative grace rejected");
  return failures == 0 ? 0 : 1;
}
