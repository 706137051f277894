/*
 * dlc.h -- C ABI of the DiLoCo outer-step merge on one gfx950 GPU.
 *
 * One outer step over one fragment of a model is two calls:
 *   dlc_quantize          learner side: pseudo-gradient, per-tensor statistics,
 *                         6-sigma clip, 256-bucket uint8 codes and a codebook of
 *                         per-bucket means, for every present learner;
 *   dlc_merge_outer_step  syncer side: dequantize every learner, take the weighted
 *                         mean in floating point, apply the Nesterov outer step.
 * dlc_quantize is also available as its two stages (dlc_quantize_range, then
 * dlc_quantize_encode) for callers that time or pin them separately, and
 * dlc_fragment_plan splits a model into balanced fragments.
 *
 * Sources:
 *   INTELLECT-1 reading notes ("Training a 10B Model Across 3 Continents"),
 *     section 3.2 (worked example, steps 4-7), section 4.1 (uniform quantization
 *     with clipping), section 4.2 (quantize for transport only; accumulate in
 *     floating point, since Q(a) + Q(b) != Q(a + b));
 *   Decoupled DiLoCo digest ("Resilient, Distributed AI Training at Scale"),
 *     section "architecture" item 4 (P = 24 fragments from greedy bin-packing of
 *     whole tensors) and "fault tolerance" items 1 and 3 (minimum quorum,
 *     weighted merge).
 *
 * Conventions shared by every call
 *   - Status: 0 = DLC_OK, negative = error.  The message of the last error on the
 *     calling thread is returned by dlc_last_error().  No exception crosses the ABI.
 *   - Ownership: every buffer is owned by the caller.  The library allocates and
 *     frees no memory, keeps no state between calls and never synchronizes the
 *     stream (except dlc_quantize with DLC_DEBUG_CHECKS).  Device pointers must be
 *     on the current HIP device.
 *   - Execution: work is enqueued on `hip_stream` (a hipStream_t; NULL = the null
 *     stream).  Argument errors are returned before anything is enqueued; a failed
 *     launch returns DLC_ERR_HIP.  Two calls in flight at once must not share any
 *     output buffer or workspace.
 *   - Layout: a call covers n_tensors tensors (a fragment).  Tensor t occupies
 *     elements [offset, offset + numel) of theta_global / momentum and elements
 *     [loffset, loffset + numel) of every learner row of theta_learners and codes
 *     (row i starts at i * learner_stride).  Per-(learner, tensor) outputs are
 *     indexed [learner][t] with the call's tensor index t in 0..n_tensors-1 and the
 *     learner's own index i in 0..n_learners-1.
 *   - Alignment: device base pointers 256-byte aligned; offset, loffset and
 *     learner_stride multiples of 64 elements; 1 <= numel <= 2^32 - 1 (any value
 *     in that range; tails are handled on the device); offsets below 2^38
 *     elements.  Tensor ranges must not overlap, in theta_global nor within a
 *     learner row.
 *   - Limits: 1 <= n_learners <= DLC_MAX_LEARNERS; n_tensors >= 1.
 */
#ifndef DLC_H
#define DLC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DLC_OK 0
#define DLC_ERR_INVALID_ARGUMENT (-1)
#define DLC_ERR_ALIGNMENT (-2)
#define DLC_ERR_NO_QUORUM (-3)
#define DLC_ERR_WORKSPACE (-4)
#define DLC_ERR_HIP (-5)
#define DLC_ERR_NON_FINITE (-6)

/* dlc_quantize flag: use the caller's `range` instead of computing it. */
#define DLC_RANGE_GIVEN 1u
/* dlc_outer_cycle flag: after each fragment's merge, copy its updated theta into
   every learner replica (dlc_broadcast). */
#define DLC_BROADCAST 2u
/* dlc_outer_cycle flag: the non-empty fragments alternate between the two streams
   (lanes); each fragment's quantize, merge and send back run on its lane, with its
   lane's half of the workspace, so consecutive fragments overlap entirely.  Needs
   twice dlc_cycle_workspace_bytes. */
#define DLC_TWO_LANES 4u
/* dlc_quantize flag: also check that every present learner's pseudo-gradient is
   finite (see dlc_quantize). */
#define DLC_DEBUG_CHECKS 8u

#define DLC_MAX_LEARNERS 64
#define DLC_MAX_LANES 8
#define DLC_N_BUCKETS 256
#define DLC_ALIGN_ELEMS 64
#define DLC_RANGE_FIELDS 4

typedef struct dlc_tensor {
    int64_t offset;   /* element offset into theta_global and momentum        */
    int64_t loffset;  /* element offset into each learner row (theta, codes)  */
    int64_t numel;    /* number of elements, >= 1                             */
} dlc_tensor;

/*
 * dlc_fragment_plan -- greedy bin-packing of whole tensors into balanced
 * fragments (Decoupled DiLoCo digest, "architecture" item 4, note 1; P = 24 there).
 *
 * Largest tensor first (ties: lower tensor index), each onto the fragment with the
 * smallest load so far (ties: lower fragment id).  Pure host code.
 *   numel          host [n_tensors], each >= 1
 *   n_fragments    >= 1 (fragments may stay empty when n_tensors < n_fragments)
 *   fragment_of    host out [n_tensors]: fragment id of each tensor
 *   fragment_numel host out [n_fragments]: elements per fragment (may be NULL)
 */
int32_t dlc_fragment_plan(const int64_t* numel, int32_t n_tensors, int32_t n_fragments,
                          int32_t* fragment_of, int64_t* fragment_numel);

/*
 * dlc_workspace_bytes -- device workspace that dlc_quantize / dlc_quantize_range /
 * dlc_quantize_encode need for these tensors and up to n_learners present learners
 * (per-block partial statistics and histograms).  Pure host code.
 */
int32_t dlc_workspace_bytes(int32_t n_learners, const dlc_tensor* tensors, int32_t n_tensors,
                            size_t* bytes);

/*
 * dlc_quantize_range -- stage A of quantization (INTELLECT-1 notes, section 3.2
 * step 4 and section 4.1 steps 1-3).  For every present learner i and tensor t:
 *   Delta = fl32(theta_global - theta_i)                       (never stored)
 *   mu, sigma = mean and population std of Delta, accumulated in fp64
 *   range[i][t] = { lo = fl32(mu - 6 sigma), hi = fl32(mu + 6 sigma),
 *                   wd = fl32(12 sigma / 256), fl32(mu) }
 *   theta_global    device fp32, read only
 *   theta_learners  device fp32 [n_learners][learner_stride], read only
 *   present         host uint8 [n_learners] (0 = absent: never read, outputs
 *                   untouched) or NULL = all present; at least one present
 *   range           device fp32 [n_learners][n_tensors][4], written
 *   workspace       device, >= dlc_workspace_bytes(n_learners, ...) bytes
 */
int32_t dlc_quantize_range(const float* theta_global, const float* theta_learners,
                           int64_t learner_stride, int32_t n_learners, const uint8_t* present,
                           const dlc_tensor* tensors, int32_t n_tensors, float* range,
                           void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * dlc_quantize_encode -- stage B of quantization (INTELLECT-1 notes, section 4.1
 * steps 2-4).  Given range[i][t] = {lo, hi, wd, mean} with lo <= hi:
 *   code  = clip(floor(fl32(fl32(Delta - lo) / wd)), 0, 255)   (IEEE fp32, RNE)
 *   x_c   = min(max(Delta, lo), hi)
 *   codebook[i][t][c] = fl32(mean of x_c over bucket c), or the midpoint
 *                       fl32(lo + (c + 1/2) wd) for an empty bucket.
 *   The bucket means come from exact integer sums of every element's position
 *   inside its bucket, each rounded to units of wd * 2^-26, so an entry is within
 *   wd * 2^-27 of the exact mean before its fp32 rounding (and independent of the
 *   order in which elements are accumulated).
 *   If wd is not a normal fp32 (zero variance), every code is 0 and every
 *   codebook entry is `mean`.  lo and hi must be finite (pseudo-gradients with
 *   |mu| + 6 sigma beyond the fp32 range are outside the contract).
 *   codes     device uint8 [n_learners][learner_stride], written at the tensors'
 *             ranges of present learners
 *   codebook  device fp32 [n_learners][n_tensors][256], written for present learners
 */
int32_t dlc_quantize_encode(const float* theta_global, const float* theta_learners,
                            int64_t learner_stride, int32_t n_learners, const uint8_t* present,
                            const dlc_tensor* tensors, int32_t n_tensors, const float* range,
                            uint8_t* codes, float* codebook, void* workspace,
                            size_t workspace_bytes, void* hip_stream);

/*
 * dlc_quantize -- dlc_quantize_range followed by dlc_quantize_encode.  With
 * DLC_RANGE_GIVEN in `flags`, `range` is an input (lo <= hi) and only the encode
 * stage runs.
 * With DLC_DEBUG_CHECKS in `flags` (not together with DLC_RANGE_GIVEN), the
 * statistics stage also records every (learner, tensor) whose pseudo-gradient
 * holds a NaN or an infinity (NaN and Inf inputs are outside the contract: the
 * kernels stay within their buffers, but codes, codebooks and ranges of such a
 * tensor are meaningless).  The call then waits for `hip_stream` before it
 * returns -- the one call mode that synchronizes, so it cannot be captured in a
 * graph -- and returns DLC_ERR_NON_FINITE naming the lowest such (learner,
 * tensor) pair; the outputs have been written all the same.
 */
int32_t dlc_quantize(const float* theta_global, const float* theta_learners,
                     int64_t learner_stride, int32_t n_learners, const uint8_t* present,
                     const dlc_tensor* tensors, int32_t n_tensors, uint8_t* codes,
                     float* codebook, float* range, uint32_t flags, void* workspace,
                     size_t workspace_bytes, void* hip_stream);

/*
 * dlc_quantize_static -- dlc_quantize for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same call, the same results bit for bit, with no
 * workspace argument.  Its workspace is the library's static scratch, a device
 * array of DLC_STATIC_SCRATCH_BYTES bytes that each device the library runs on
 * holds until the process ends; the call allocates nothing (no hipMalloc, no
 * hipFree, no allocating library routine).
 *   - A call whose workspace (dlc_workspace_bytes for its present learners)
 *     exceeds DLC_STATIC_SCRATCH_BYTES returns DLC_ERR_WORKSPACE before anything
 *     is enqueued: split it into smaller fragments, or use dlc_quantize.
 *   - The device is the stream's (the current device's for the null stream).
 *     Every call on one device shares that device's scratch, which keeps the last
 *     call's contents (no call needs it cleared).  Calls that overlap on one
 *     device -- on different streams or threads without ordering -- race on it:
 *     the caller orders them.
 *   - The first call on a device looks up that device's scratch address, making
 *     the device current for the lookup and restoring the caller's device after
 *     it; a failure there returns DLC_ERR_HIP.
 * Arguments, flags and errors otherwise as dlc_quantize.
 */
#define DLC_STATIC_SCRATCH_BYTES 67108864u /* 64 MiB */

int32_t dlc_quantize_static(const float* theta_global, const float* theta_learners, int64_t learner_stride,
                            int32_t n_learners, const uint8_t* present, const dlc_tensor* tensors,
                            int32_t n_tensors, uint8_t* codes, float* codebook, float* range, uint32_t flags,
                            void* hip_stream);

/*
 * dlc_quantize_bases -- dlc_quantize for learners that started from different
 * versions of the global parameters (Decoupled DiLoCo digest, "fault tolerance":
 * learners run asynchronously and may report against an older global fragment).
 * Learner i's pseudo-gradient is Delta_i = fl32(bases[i] - theta_i), every other
 * step as in dlc_quantize (range computed, never given).
 *   bases     host array [n_learners] of device pointers, each laid out like
 *             theta_global (tensor t at its offset); learners with the same
 *             pointer share one pass over that base.  Entries of absent learners
 *             are not read.
 * Learners are processed in groups of equal base, in order of first appearance,
 * one after another on the stream with the same workspace
 * (dlc_workspace_bytes(n_learners, ...) suffices).
 */
int32_t dlc_quantize_bases(const float* const* bases, const float* theta_learners, int64_t learner_stride,
                           int32_t n_learners, const uint8_t* present, const dlc_tensor* tensors,
                           int32_t n_tensors, uint8_t* codes, float* codebook, float* range, void* workspace,
                           size_t workspace_bytes, void* hip_stream);

/*
 * dlc_merge_outer_step -- dequantize, weighted mean, Nesterov (INTELLECT-1 notes,
 * section 3.2 steps 6-7 and section 4.2; Decoupled DiLoCo digest, "fault
 * tolerance" items 1 and 3).  Per element of every tensor:
 *   w_hat_i = w_i / sum_j w_j          (host, fp64, left-to-right sum)
 *   g       = sum_i w_hat_i * codebook[i][t][code_i]   (learners in index order,
 *             fp64 products and sums of the fp32 codebook values)
 *   v      <- beta * v + g
 *   theta  <- theta - lr * (g + beta * v)              (fp64, stored as fp32)
 * Dequantized values are never added in code space.
 *   theta_global, momentum  device fp32, updated in place at the tensors' ranges
 *   codes, codebook         as written by dlc_quantize (read only)
 *   weights                 host double [n_learners], finite and >= 0; 0 = absent
 *                           (its codes and codebook are never read).  A zero total
 *                           (no quorum) returns DLC_ERR_NO_QUORUM and changes nothing.
 *   lr, beta                outer learning rate and momentum (0.7 and 0.9 on the pages)
 *   flags                   reserved, must be 0
 */
int32_t dlc_merge_outer_step(float* theta_global, float* momentum, const uint8_t* codes,
                             int64_t learner_stride, int32_t n_learners, const float* codebook,
                             const double* weights, const dlc_tensor* tensors, int32_t n_tensors,
                             double lr, double beta, uint32_t flags, void* hip_stream);

/*
 * dlc_broadcast -- send the updated fragment back to the learners (INTELLECT-1
 * notes, section 3.2 step 8: every worker copies the updated weights before the
 * next outer step; Decoupled DiLoCo digest, "architecture": the syncer sends the
 * updated fragment back).  For every tensor and every learner i with rows[i] != 0
 * (rows NULL = all n_learners):
 *   theta_learners[i][loffset .. loffset + numel) = theta_global[offset .. offset + numel)
 * bit for bit.  theta_learners is written only there.  Same layout, alignment and
 * stream rules as the other calls.
 */
int32_t dlc_broadcast(const float* theta_global, float* theta_learners, int64_t learner_stride,
                      int32_t n_learners, const uint8_t* rows, const dlc_tensor* tensors, int32_t n_tensors,
                      void* hip_stream);

/*
 * dlc_outer_cycle -- one outer step over every fragment of a model, fragments in
 * id order (Decoupled DiLoCo digest, "architecture" item 4: P fragments merged one
 * at a time; the quantization of fragment p + 1 overlaps the merge of fragment p,
 * as the learners' and the syncer's work overlap with tau = 2 there).
 *   tensors         all tensors, grouped by fragment: fragment f owns
 *                   tensors[fragment_first[f] .. fragment_first[f + 1]) (may be empty)
 *   fragment_first  host int32 [n_fragments + 1], nondecreasing, fragment_first[0] = 0,
 *                   fragment_first[n_fragments] = number of tensors >= 1
 *   weights         host double [n_fragments][n_learners]: raw weights of each
 *                   fragment's merge; 0 = learner absent for that fragment (not
 *                   read, not quantized).  Every non-empty fragment needs a
 *                   positive total (else DLC_ERR_NO_QUORUM, nothing enqueued).
 *   codes           device uint8 [n_learners][learner_stride]
 *   codebook        device fp32 [n_learners][n_tensors][256], row = global tensor index
 *   range           device fp32 [n_learners][n_tensors][4], row = global tensor index
 *   flags           0, DLC_BROADCAST, DLC_TWO_LANES or both
 *   workspace       >= dlc_cycle_workspace_bytes(...) bytes (twice that with DLC_TWO_LANES)
 *   quantize_stream the quantize calls (dlc_quantize of each fragment);
 *   merge_stream    the merge (and broadcast) calls; each waits for its fragment's
 *                   quantization on the other stream through an event.  Both may
 *                   be the same stream.  At the end the quantize stream waits for
 *                   the merge stream, so synchronizing either completes the cycle.
 *                   With DLC_TWO_LANES the two streams are instead the two lanes:
 *                   the merge stream first waits for the work already enqueued on
 *                   the quantize stream, and each waits for the other at the end.
 * The call can be captured in a HIP graph on the quantize stream (the merge
 * stream joins the capture through the call's events).
 * Results are those of calling dlc_quantize, dlc_merge_outer_step (and
 * dlc_broadcast) fragment by fragment.  Per-call events are created and
 * destroyed inside the call.  All argument errors, including every fragment's
 * quorum and workspace size, are returned before anything is enqueued.
 */
int32_t dlc_cycle_workspace_bytes(int32_t n_learners, const dlc_tensor* tensors, const int32_t* fragment_first,
                                  int32_t n_fragments, size_t* bytes);

int32_t dlc_outer_cycle(float* theta_global, float* momentum, float* theta_learners, int64_t learner_stride,
                        int32_t n_learners, const double* weights, const dlc_tensor* tensors,
                        const int32_t* fragment_first, int32_t n_fragments, uint8_t* codes, float* codebook,
                        float* range, double lr, double beta, uint32_t flags, void* workspace,
                        size_t workspace_bytes, void* quantize_stream, void* merge_stream);

/*
 * dlc_outer_cycle_lanes -- the same cycle (same arguments, same results) with the
 * non-empty fragments taking n_lanes streams in turn: fragment j (counting
 * non-empty fragments only) runs its quantize, merge and send back on
 * streams[j % n_lanes], with that lane's share of the workspace.  Lanes pay off
 * when fragments are small (kernels of a few tens of microseconds): several
 * fragments in flight keep the device busy.  Lanes beyond the device's hardware
 * queues share queues and serialize.
 *   flags       0 or DLC_BROADCAST
 *   workspace   >= n_lanes * dlc_cycle_workspace_bytes(...) bytes, split into
 *               n_lanes equal shares (each rounded down to 256 bytes)
 *   streams     host [n_lanes] HIP streams (a stream may repeat)
 *   n_lanes     1..DLC_MAX_LANES; 1 runs everything on streams[0]
 * Lanes 1.. first wait for the work already enqueued on streams[0]; at the end
 * streams[0] waits for every lane and every lane for streams[0], so synchronizing
 * any one of them completes the cycle.  The call can be captured in a HIP graph
 * on streams[0] (the other lanes join the capture through the call's events).
 * DLC_TWO_LANES in dlc_outer_cycle is this call with the streams
 * {quantize_stream, merge_stream}.
 */
int32_t dlc_outer_cycle_lanes(float* theta_global, float* momentum, float* theta_learners, int64_t learner_stride,
                              int32_t n_learners, const double* weights, const dlc_tensor* tensors,
                              const int32_t* fragment_first, int32_t n_fragments, uint8_t* codes, float* codebook,
                              float* range, double lr, double beta, uint32_t flags, void* workspace,
                              size_t workspace_bytes, void* const* streams, int32_t n_lanes);

/*
 * dlc_outer_cycle_rda -- the cycle of dlc_outer_cycle_lanes with every fragment
 * merged by Radial-Directional Averaging (Decoupled DiLoCo digest,
 * "architecture": the syncer merges one fragment at a time, averaging the outer
 * gradients' directions and norms separately).  Fragment f's step is exactly
 * dlc_rda_outer_step over its tensors with weights[f]; the results equal those
 * calls made fragment by fragment on one stream, bit for bit.
 *   sq_norms    device fp64 [n_learners][n_tensors], written for every present
 *               (learner, tensor) pair: the squared norm of the dequantized
 *               pseudo-gradient, as dlc_rda_outer_step
 *   workspace   >= n_lanes * dlc_cycle_rda_workspace_bytes(...) bytes, split into
 *               n_lanes equal shares (each rounded down to 256 bytes)
 *   flags       0 or DLC_BROADCAST
 * Other arguments, streams, ordering and errors as dlc_outer_cycle_lanes.
 */
int32_t dlc_outer_cycle_rda(float* theta_global, float* momentum, float* theta_learners, int64_t learner_stride,
                            int32_t n_learners, const double* weights, const dlc_tensor* tensors,
                            const int32_t* fragment_first, int32_t n_fragments, uint8_t* codes, float* codebook,
                            float* range, double* sq_norms, double lr, double beta, uint32_t flags, void* workspace,
                            size_t workspace_bytes, void* const* streams, int32_t n_lanes);

/* Workspace bytes of one lane of dlc_outer_cycle_rda: the largest fragment's
 * quantize workspace, its direction sums and a coefficient table of
 * n_learners * n_tensors doubles. */
int32_t dlc_cycle_rda_workspace_bytes(int32_t n_learners, const dlc_tensor* tensors, const int32_t* fragment_first,
                                      int32_t n_fragments, size_t* bytes);

/*
 * dlc_merge_weights -- which learners a fragment's merge takes, and their weights
 * (Decoupled DiLoCo digest, "fault tolerance" items 1-3: merge once a minimum
 * quorum has arrived, wait a little longer while the window has slack, weight
 * learners by the tokens they processed).  Pure host code.
 *   tokens      host [n_learners]: tokens each learner processed since its base
 *   arrival     host [n_learners]: seconds after the fragment's window opened at
 *               which the learner's update arrived; +inf or NaN = not arrived
 *   quorum      minimum number of arrived learners, 1..n_learners
 *   grace       seconds the merge may wait after the quorum is met (the caller's
 *               remaining slack), finite and >= 0
 *   weights     host out [n_learners]: tokens_i for every learner that arrived
 *               by t_q + grace, 0 for the others, where t_q is the arrival of the
 *               quorum-th earliest learner (ties: lower index first)
 *   merge_time  host out (may be NULL): t_q + grace, or the last arrival if every
 *               learner arrived before that
 * DLC_ERR_NO_QUORUM when fewer than `quorum` learners arrived or the merged
 * learners report zero tokens in total (weights untouched then).
 */
int32_t dlc_merge_weights(int32_t n_learners, const double* tokens, const double* arrival, int32_t quorum,
                          double grace, double* weights, double* merge_time);

/*
 * dlc_ring_outer_step -- one outer step whose learners average their
 * pseudo-gradients through a ring that requantizes at every hop (INTELLECT-1
 * notes, section 3.2 step 6 and section 4.2: a message is quantized before it is
 * sent; the receiver dequantizes it and adds it to its own value in fp32), as K
 * virtual ranks on one device, all learners weighted equally.  Per tensor:
 *   chunks   K chunks of whole 64-element groups, chunk j = [64 floor(j m / K),
 *            64 floor((j + 1) m / K)) clipped to numel, m = ceil(numel / 64);
 *   reduce-scatter, hops s = 0 .. K - 2: rank r quantizes its running sum of
 *            chunk (r - s) mod K (statistics, clip, 256 buckets, codebook of
 *            bucket means, exactly as dlc_quantize on that chunk) and rank r + 1
 *            sets its sum to fl32(sum + deQ(message)); after the last hop each
 *            owner divides: mean = fl32(sum / K);
 *   gather:  each owner's mean is quantized once; every rank ends with
 *            g = deQ(message) for every chunk, and theta_global, momentum take
 *            the Nesterov step with that g (as dlc_merge_outer_step).
 * The start is Delta_r = fl32(theta_global - theta_r) for every row r < K.
 *   accum     device fp32 [n_learners][learner_stride] scratch: each rank's received running
 *             sums, kept negated (hop 0 quantizes the pseudo-gradients straight from
 *             theta_learners, so chunks a rank never receives are not written)
 *   codes     device uint8 [n_learners][learner_stride]: on return, the gather messages
 *   codebook  device fp32 [n_learners * n_tensors][256]: on return, the gather codebooks
 *             (one row per non-empty owned chunk, tensor by tensor, rank by rank)
 *   range     device fp32 [n_learners * n_tensors][4], likewise
 *   workspace >= dlc_ring_workspace_bytes(n_learners, tensors, n_tensors) bytes
 * Same layout, alignment and stream rules as the other calls; argument errors are
 * returned before anything is enqueued.
 */
int32_t dlc_ring_workspace_bytes(int32_t n_learners, const dlc_tensor* tensors, int32_t n_tensors, size_t* bytes);

int32_t dlc_ring_outer_step(float* theta_global, float* momentum, const float* theta_learners,
                            int64_t learner_stride, int32_t n_learners, const dlc_tensor* tensors, int32_t n_tensors,
                            double lr, double beta, float* accum, uint8_t* codes, float* codebook, float* range,
                            void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * dlc_rda_outer_step -- one outer step whose merge is Radial-Directional
 * Averaging (Decoupled DiLoCo digest, "architecture", the second engineering
 * detail, with "fault tolerance" item 3: the outer gradients' directions and
 * norms are averaged separately; the page gives no formula).  Per tensor, with
 * x_i the dequantized pseudo-gradient of learner i (quantized exactly as
 * dlc_quantize does) and w_hat_i = weights[i] / sum(weights) in fp64:
 *   ||x_i||^2 = sum over the tensor of x_i^2      (fp64, from the bucket counts)
 *   r = sum_i w_hat_i ||x_i||                      the averaged norm
 *   d = sum_i w_hat_i x_i / ||x_i||                the averaged direction
 *                                                  (a learner with x_i = 0 adds none)
 *   g = r d / ||d||                                (g = 0 when d = 0)
 * where d counts as zero when ||d|| <= 2^-40 W, W = sum of w_hat_i over the
 * learners with x_i != 0 (the largest ||d|| can be): directions that cancel in
 * real arithmetic leave only rounding noise in d;
 * then v <- beta v + g; theta <- theta - lr (g + beta v) as dlc_merge_outer_step.
 * Learners with weight 0 are absent: neither quantized nor read, and their rows
 * of every output are left untouched.  Results agree with the fp64 definition up
 * to the order of fp64 rounding (not bit for bit).
 *   bases     NULL: every pseudo-gradient is fl32(theta_global - theta_i); or a
 *             host array [n_learners] of device pointers, each laid out like
 *             theta_global: learner i's pseudo-gradient is fl32(bases[i] -
 *             theta_i), the version it started from (as dlc_quantize_bases; the
 *             Decoupled DiLoCo digest's asynchronous learners, merged by its
 *             syncer's rule); theta_global is still the state the step updates
 *   codes     device uint8 [n_learners][learner_stride], written (as dlc_quantize)
 *   codebook  device fp32 [n_learners][n_tensors][256], written
 *   range     device fp32 [n_learners][n_tensors][4], written
 *   sq_norms  device fp64 [n_learners][n_tensors]: ||x_i||^2 per tensor, written
 *   workspace >= dlc_rda_workspace_bytes(n_learners, tensors, n_tensors) bytes,
 *             256-byte aligned, no initial contents required
 * Errors: as dlc_quantize and dlc_merge_outer_step (DLC_ERR_NO_QUORUM when every
 * weight is zero), all returned before anything is enqueued.
 */
int32_t dlc_rda_workspace_bytes(int32_t n_learners, const dlc_tensor* tensors, int32_t n_tensors, size_t* bytes);

int32_t dlc_rda_outer_step(float* theta_global, float* momentum, const float* theta_learners,
                           const float* const* bases, int64_t learner_stride, int32_t n_learners,
                           const dlc_tensor* tensors, int32_t n_tensors,
                           const double* weights, double lr, double beta, uint8_t* codes, float* codebook,
                           float* range, double* sq_norms, void* workspace, size_t workspace_bytes,
                           void* hip_stream);

/* Message of the last error on the calling thread ("" if none). */
const char* dlc_last_error(void);

/* Library version string. */
const char* dlc_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DLC_H */
