// C ABI of the DiLoCo outer-step merge: argument checks, the fragment planner,
// the block partition of a call, and kernel launch orchestration.
//
// Nothing here allocates device memory, keeps state between calls or waits on the
// stream; argument errors are reported before anything is enqueued.
#include "dlc.h"
#include "dlc_internal.h"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <numeric>
#include <string>
#include <vector>

// Workspace of dlc_quantize_static, for callers that cannot allocate: one copy
// per device, held until the process ends, shared by every such call whose
// stream is on that device (calls that overlap on one device race on it).  No call needs it to
// start zeroed: every workspace slot is written before it is read.
static __device__ __align__(256) unsigned char scratch[DLC_STATIC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

int32_t fail(int32_t code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int32_t ok() {
  g_last_error.clear();
  return DLC_OK;
}

// Blocks per call that the statistics, encode and send-back passes aim for
// (several resident blocks per CU on 256 CUs).  Finer blocks shorten the tail at
// the end of a pass, coarser ones restart the load pipeline less often: measured
// in one process on identical inputs, the statistics pass does best with the
// fewest blocks.  The merge does best with the most: two tiles per block
// whatever the call's size (against 1, 3, 4, 7 and 13 tiles: 5% faster on the
// 1B set than 13, 10% on the 10B median fragment than 7, small calls unchanged).
constexpr int64_t kStatsBlocks = 4096;
constexpr int64_t kEncodeBlocks = 8192;
constexpr int64_t kMergeTilesPerBlock = 2;
// The direction pass of Radial-Directional Averaging reads only the codes, and
// each block first builds its K scaled codebook tables: it does best with
// coarser blocks than the merge.
constexpr int64_t kDirectionBlocks = 16384;
constexpr int64_t kBroadcastBlocks = 8192;
// At least one full group of 4 tiles per statistics or encode block: on a
// single 4096^2 tensor, 4-tile blocks ran the step 27% faster than 1-tile blocks
// (per-block setup, histogram flush and pipeline start amortized); large sets
// already get bigger blocks from the targets above.
constexpr int64_t kStatsMinTiles = 4;
constexpr int64_t kEncodeMinTiles = 4;

constexpr int64_t kMaxTensorNumel = (int64_t(1) << 32) - 1;
constexpr int64_t kMaxOffset = (int64_t(1) << 38) - DLC_ALIGN_ELEMS;

bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

struct Partition {
  std::vector<dlc::LaunchGeom> launches;
  int64_t n_slots = 0;
};

// Split the call's tensors into launches of at most kMaxTensorsPerLaunch tensors;
// each tensor gets ceil(tiles / tiles_per_block) blocks, tiles_per_block chosen
// from the whole call so that the call has about target_blocks blocks, at most
// max_tiles, at least min_tiles, and rounded up to a multiple of tile_multiple.
Partition make_partition(const dlc_tensor* t, int32_t n, int64_t max_tiles, int64_t target_blocks,
                         int64_t tile_multiple = 1, int64_t min_tiles = 1) {
  Partition p;
  int64_t total_tiles = 0;
  for (int32_t i = 0; i < n; ++i) total_tiles += (t[i].numel + dlc::kTile - 1) / dlc::kTile;
  int64_t tpb = std::max<int64_t>(min_tiles, (total_tiles + target_blocks - 1) / target_blocks);
  tpb = std::min(tpb, max_tiles);
  tpb = (tpb + tile_multiple - 1) / tile_multiple * tile_multiple;
  for (int32_t s = 0; s < n; s += dlc::kMaxTensorsPerLaunch) {
    dlc::LaunchGeom g;
    std::memset(&g, 0, sizeof(g));
    g.n_tensors = std::min<int32_t>(dlc::kMaxTensorsPerLaunch, n - s);
    g.t_base = s;
    g.n_tensors_call = n;
    g.tiles_per_block = (int32_t)tpb;
    g.slot_base = (int32_t)p.n_slots;
    int64_t blocks = 0;
    for (int32_t i = 0; i < g.n_tensors; ++i) {
      const dlc_tensor& d = t[s + i];
      g.t[i].off64 = (uint32_t)(d.offset / DLC_ALIGN_ELEMS);
      g.t[i].loff64 = (uint32_t)(d.loffset / DLC_ALIGN_ELEMS);
      g.t[i].count = (uint32_t)d.numel;
      g.t[i].block_first = (int32_t)blocks;
      const int64_t tiles = (d.numel + dlc::kTile - 1) / dlc::kTile;
      const int64_t nb = (tiles + tpb - 1) / tpb;
      blocks += nb;
      g.hist_slices = std::max<int32_t>(g.hist_slices, (int32_t)((nb + dlc::kHistSlice - 1) / dlc::kHistSlice));
    }
    g.n_blocks = (int32_t)blocks;
    p.n_slots += blocks;
    p.launches.push_back(g);
  }
  return p;
}

constexpr int64_t kUnlimitedTiles = int64_t(1) << 40;

// Range / codebook rows for a call that is one fragment of a cycle: its tensors
// are rows row_base.. of tables with rows_total rows per learner.
void set_rows(Partition& p, int32_t row_base, int32_t rows_total) {
  for (dlc::LaunchGeom& g : p.launches) {
    g.row_base = row_base;
    g.n_tensors_call = rows_total;
  }
}

// The block partition of each pass.  The workspace holds one statistics slot per
// statistics block and one histogram slot per encode block.
Partition stats_partition(const dlc_tensor* t, int32_t n) {
  return make_partition(t, n, kUnlimitedTiles, kStatsBlocks, 1, kStatsMinTiles);
}

Partition encode_partition(const dlc_tensor* t, int32_t n) {
  // whole groups per block: the blocks of a tensor take its groups in turn
  return make_partition(t, n, dlc::kMaxEncodeTiles, kEncodeBlocks, dlc::kEncodeGroupTiles, kEncodeMinTiles);
}

Partition broadcast_partition(const dlc_tensor* t, int32_t n) {
  return make_partition(t, n, kUnlimitedTiles, kBroadcastBlocks);
}

Partition direction_partition(const dlc_tensor* t, int32_t n) {
  return make_partition(t, n, kUnlimitedTiles, kDirectionBlocks / dlc::kMergeTiles, dlc::kMergeTiles);
}

// merge blocks work on kMergeTiles tiles side by side, kMergeTilesPerBlock in all
Partition merge_partition(const dlc_tensor* t, int32_t n) {
  // no block-count target: the tile count per block fixes the blocks
  return make_partition(t, n, kMergeTilesPerBlock, kUnlimitedTiles, dlc::kMergeTiles, kMergeTilesPerBlock);
}

struct WorkspaceLayout {
  size_t stats = 0, hist = 0, hist_sum = 0, status = 0, total = 0;
};

size_t round256(size_t v) { return (v + 255) & ~size_t(255); }

// Workspace: per-block statistics partials, per-block packed histograms, then
// the histogram slice entries (at most slots / kHistSlice + tensors + 2).
WorkspaceLayout workspace_layout(int64_t stats_slots, int64_t hist_slots, int32_t n_tensors, int32_t n_learners) {
  WorkspaceLayout w;
  w.stats = 0;
  w.hist = round256((size_t)stats_slots * (size_t)n_learners * sizeof(double) * 2);
  w.hist_sum = w.hist + round256((size_t)hist_slots * (size_t)n_learners * dlc::kBuckets * sizeof(uint64_t));
  const size_t entries = (size_t)(hist_slots / dlc::kHistSlice) + (size_t)n_tensors + 2;
  w.status = w.hist_sum + round256(entries * (size_t)n_learners * dlc::kBuckets * 2 * sizeof(uint64_t));
  w.total = w.status + 256;  // one status word (debug checks), padded
  return w;
}

int32_t check_tensors(const dlc_tensor* t, int32_t n, int64_t learner_stride, bool need_loffset) {
  if (t == nullptr) return fail(DLC_ERR_INVALID_ARGUMENT, "tensors is NULL");
  if (n < 1) return fail(DLC_ERR_INVALID_ARGUMENT, "n_tensors must be >= 1");
  if (need_loffset && (learner_stride < 1 || learner_stride % DLC_ALIGN_ELEMS != 0))
    return fail(DLC_ERR_ALIGNMENT, "learner_stride must be a positive multiple of 64 elements");
  for (int32_t i = 0; i < n; ++i) {
    const dlc_tensor& d = t[i];
    if (d.numel < 1 || d.numel > kMaxTensorNumel)
      return fail(DLC_ERR_INVALID_ARGUMENT, "tensor " + std::to_string(i) + ": numel must be in [1, 2^32 - 1]");
    if (d.offset > kMaxOffset || d.loffset > kMaxOffset)
      return fail(DLC_ERR_INVALID_ARGUMENT, "tensor " + std::to_string(i) + ": offset beyond 2^38 elements");
    if (d.offset < 0 || d.loffset < 0)
      return fail(DLC_ERR_INVALID_ARGUMENT, "tensor " + std::to_string(i) + ": negative offset");
    if (d.offset % DLC_ALIGN_ELEMS != 0 || d.loffset % DLC_ALIGN_ELEMS != 0)
      return fail(DLC_ERR_ALIGNMENT, "tensor " + std::to_string(i) + ": offset and loffset must be multiples of 64 elements");
    if (need_loffset && d.loffset + d.numel > learner_stride)
      return fail(DLC_ERR_INVALID_ARGUMENT, "tensor " + std::to_string(i) + ": loffset + numel exceeds learner_stride");
  }
  // No two tensors may overlap in theta_global, nor within a learner row.
  std::vector<int32_t> order(n);
  for (int pass = 0; pass < 2; ++pass) {
    std::iota(order.begin(), order.end(), 0);
    auto key = [&](int32_t i) { return pass == 0 ? t[i].offset : t[i].loffset; };
    std::sort(order.begin(), order.end(), [&](int32_t x, int32_t y) { return key(x) < key(y); });
    for (int32_t i = 1; i < n; ++i) {
      if (key(order[i - 1]) + t[order[i - 1]].numel > key(order[i]))
        return fail(DLC_ERR_INVALID_ARGUMENT, std::string("tensors ") + std::to_string(order[i - 1]) + " and " +
                                                  std::to_string(order[i]) + " overlap in " +
                                                  (pass == 0 ? "theta_global" : "the learner rows"));
    }
  }
  return DLC_OK;
}

struct Common {
  dlc::QuantArgs args;
  Partition part_stats;   // statistics pass (range stage)
  Partition part_enc;     // encode pass: blocks capped at kMaxEncodeTiles tiles
  hipStream_t stream;
  uint32_t* status;       // the workspace's status word (used only by debug checks)
};

// Shared checks and setup of the quantize stages.
int32_t setup_quant(Common& c, const float* theta_global, const float* theta_learners,
                    int64_t learner_stride, int32_t n_learners, const uint8_t* present,
                    const dlc_tensor* tensors, int32_t n_tensors, void* workspace,
                    size_t workspace_bytes, void* hip_stream, int32_t row_base = 0, int32_t rows_total = -1,
                    bool no_base = false) {
  if (n_learners < 1 || n_learners > DLC_MAX_LEARNERS)
    return fail(DLC_ERR_INVALID_ARGUMENT, "n_learners must be in [1, 64]");
  if ((!theta_global && !no_base) || !theta_learners) return fail(DLC_ERR_INVALID_ARGUMENT, "theta pointer is NULL");
  if ((theta_global && !aligned256(theta_global)) || !aligned256(theta_learners))
    return fail(DLC_ERR_ALIGNMENT, "theta pointers must be 256-byte aligned");
  int32_t rc = check_tensors(tensors, n_tensors, learner_stride, true);
  if (rc != DLC_OK) return rc;
  std::memset(&c.args, 0, sizeof(c.args));
  int32_t kp = 0;
  for (int32_t i = 0; i < n_learners; ++i) {
    if (present == nullptr || present[i] != 0) c.args.learner[kp++] = i;
  }
  if (kp == 0) return fail(DLC_ERR_NO_QUORUM, "no learner is present");
  c.part_stats = stats_partition(tensors, n_tensors);
  c.part_enc = encode_partition(tensors, n_tensors);
  if (rows_total >= 0) {
    set_rows(c.part_stats, row_base, rows_total);
    set_rows(c.part_enc, row_base, rows_total);
  }
  const WorkspaceLayout wl = workspace_layout(c.part_stats.n_slots, c.part_enc.n_slots, n_tensors, kp);
  if (workspace == nullptr || workspace_bytes < wl.total)
    return fail(DLC_ERR_WORKSPACE, "workspace too small: need " + std::to_string(wl.total) + " bytes");
  if (!aligned256(workspace)) return fail(DLC_ERR_ALIGNMENT, "workspace must be 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  c.args.theta_g = theta_global;
  c.args.theta_L = theta_learners;
  c.args.stride = learner_stride;
  c.args.n_present = kp;
  c.args.part_stats = reinterpret_cast<double2*>(ws + wl.stats);
  c.args.part_hist = reinterpret_cast<uint64_t*>(ws + wl.hist);
  c.args.hist_sum = reinterpret_cast<uint64_t*>(ws + wl.hist_sum);
  c.status = reinterpret_cast<uint32_t*>(ws + wl.status);
  c.stream = static_cast<hipStream_t>(hip_stream);
  return DLC_OK;
}

int32_t hip_fail(hipError_t e, const char* what) {
  return fail(DLC_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

int32_t run_range(Common& c) {
  for (const dlc::LaunchGeom& g : c.part_stats.launches) {
    // Learners in balanced chunks of at most kStatsChunk (e.g. 16 -> 8 + 8).
    const int32_t n_chunks = (c.args.n_present + dlc::kStatsChunk - 1) / dlc::kStatsChunk;
    for (int32_t ci = 0, k0 = 0; ci < n_chunks; ++ci) {
      const int32_t kc = (c.args.n_present - k0) / (n_chunks - ci);
      c.args.k_base = k0;
      c.args.k_count = kc;
      k0 += kc;
      hipError_t e = dlc::launch_stats(c.args, g, c.stream);
      if (e != hipSuccess) return hip_fail(e, "stats kernel launch");
    }
    hipError_t e = dlc::launch_range(c.args, g, c.stream);
    if (e != hipSuccess) return hip_fail(e, "range kernel launch");
  }
  return DLC_OK;
}

int32_t run_encode(Common& c) {
  for (const dlc::LaunchGeom& g : c.part_enc.launches) {
    for (int32_t k0 = 0; k0 < c.args.n_present; k0 += dlc::kLearnerChunk) {
      c.args.k_base = k0;
      c.args.k_count = std::min(dlc::kLearnerChunk, c.args.n_present - k0);
      hipError_t e = dlc::launch_encode(c.args, g, c.stream);
      if (e != hipSuccess) return hip_fail(e, "encode kernel launch");
    }
    hipError_t e = dlc::launch_codebook(c.args, g, c.stream);
    if (e != hipSuccess) return hip_fail(e, "codebook kernel launch");
  }
  return DLC_OK;
}

// Merge arguments: checks and fp64 weight normalization (left-to-right sum).
int32_t prepare_merge(dlc::MergeArgs& a, float* theta_global, float* momentum, const uint8_t* codes,
                      int64_t learner_stride, int32_t n_learners, const float* codebook, const double* weights,
                      double lr, double beta) {
  if (n_learners < 1 || n_learners > DLC_MAX_LEARNERS)
    return fail(DLC_ERR_INVALID_ARGUMENT, "n_learners must be in [1, 64]");
  if (!theta_global || !momentum || !codes || !codebook || !weights)
    return fail(DLC_ERR_INVALID_ARGUMENT, "theta_global, momentum, codes, codebook and weights must not be NULL");
  if (!aligned256(theta_global) || !aligned256(momentum) || !aligned256(codes) || !aligned256(codebook))
    return fail(DLC_ERR_ALIGNMENT, "device pointers must be 256-byte aligned");
  if (!std::isfinite(lr) || !std::isfinite(beta)) return fail(DLC_ERR_INVALID_ARGUMENT, "lr and beta must be finite");
  double total = 0.0;
  for (int32_t i = 0; i < n_learners; ++i) {
    if (!(weights[i] >= 0.0) || !std::isfinite(weights[i]))
      return fail(DLC_ERR_INVALID_ARGUMENT, "weights must be finite and >= 0");
    total += weights[i];
  }
  if (!(total > 0.0)) return fail(DLC_ERR_NO_QUORUM, "all learner weights are zero (no quorum)");
  std::memset(&a, 0, sizeof(a));
  int32_t kp = 0;
  for (int32_t i = 0; i < n_learners; ++i) {
    if (weights[i] > 0.0) {
      a.learner[kp] = i;
      a.w_hat[kp] = weights[i] / total;
      ++kp;
    }
  }
  a.theta_g = theta_global;
  a.momentum = momentum;
  a.codes = codes;
  a.codebook = codebook;
  a.stride = learner_stride;
  a.n_present = kp;
  a.lr = lr;
  a.beta = beta;
  return DLC_OK;
}

int32_t run_merge(const dlc::MergeArgs& a, const dlc_tensor* tensors, int32_t n_tensors, int32_t row_base,
                  int32_t rows_total, hipStream_t s) {
  Partition p = merge_partition(tensors, n_tensors);
  if (rows_total >= 0) set_rows(p, row_base, rows_total);
  for (const dlc::LaunchGeom& g : p.launches) {
    hipError_t e = dlc::launch_merge(a, g, s);
    if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
  }
  return DLC_OK;
}

int32_t run_broadcast(const float* theta_global, float* theta_learners, int64_t learner_stride, int32_t n_learners,
                      const uint8_t* rows, const dlc_tensor* tensors, int32_t n_tensors, hipStream_t s) {
  dlc::BroadcastArgs a;
  std::memset(&a, 0, sizeof(a));
  a.theta_g = theta_global;
  a.theta_L = theta_learners;
  a.stride = learner_stride;
  for (int32_t i = 0; i < n_learners; ++i) {
    if (rows == nullptr || rows[i] != 0) a.row[a.n_rows++] = i;
  }
  if (a.n_rows == 0) return DLC_OK;
  const Partition p = broadcast_partition(tensors, n_tensors);
  for (const dlc::LaunchGeom& g : p.launches) {
    hipError_t e = dlc::launch_broadcast(a, g, s);
    if (e != hipSuccess) return hip_fail(e, "broadcast kernel launch");
  }
  return DLC_OK;
}

// ---------------------------------------------------------------------------
// The ring: chunks of whole 64-element groups, the messages of every hop as
// segments of the flat [ranks][stride] accumulator and code buffers (one
// "learner" row of ranks * stride elements).
// ---------------------------------------------------------------------------
struct RingPlan {
  // stage s < k - 1: the messages of reduce-scatter hop s; stage k - 1: the
  // gather.  Segments (chunk offset in theta_global, the sender's offset in the
  // flat [ranks][stride] theta_learners / accum / codes, numel), by tensor, then
  // by sender.
  std::vector<std::vector<dlc_tensor>> stage;
  // add_row[s][j]: the stage-s message (its codebook row) that the sender of
  // stage s + 1's segment j received at hop s
  std::vector<std::vector<int32_t>> add_row;
  std::vector<dlc_tensor> merge;
};

std::pair<int64_t, int64_t> ring_chunk(int64_t n, int32_t k, int32_t j) {
  const int64_t m = (n + DLC_ALIGN_ELEMS - 1) / DLC_ALIGN_ELEMS;
  const int64_t a = std::min<int64_t>(n, DLC_ALIGN_ELEMS * ((j * m) / k));
  const int64_t b = std::min<int64_t>(n, DLC_ALIGN_ELEMS * (((j + 1) * m) / k));
  return {a, b};
}

// At hop s rank r sends chunk (r - s) mod k to rank r + 1: its own chunk first,
// then each chunk it has just received; after k - 1 hops it holds the whole sum
// of chunk r + 1, which the gather sends.  Stage 0 holds pseudo-gradients
// (quantized with theta_global as the base); every later message is a sum the
// previous hop's dequantize-add wrote, with its statistics partials.  A rank's
// chunk is untouched until the hop that delivers to it, so that add reads the
// receiver's pseudo-gradient from theta_global and theta_learners.
RingPlan ring_plan(const dlc_tensor* t, int32_t n, int32_t k, int64_t stride) {
  RingPlan p;
  p.stage.resize(k);
  std::vector<std::vector<int32_t>> index(k);  // [stage][tensor * k + chunk] -> segment
  for (int32_t s = 0; s < k; ++s) {
    index[s].assign((size_t)n * k, -1);
    for (int32_t i = 0; i < n; ++i) {
      for (int32_t r = 0; r < k; ++r) {
        const int32_t c = ((r - s) % k + k) % k;
        const auto ch = ring_chunk(t[i].numel, k, c);
        if (ch.second <= ch.first) continue;
        index[s][(size_t)i * k + c] = (int32_t)p.stage[s].size();
        p.stage[s].push_back({t[i].offset + ch.first, (int64_t)r * stride + t[i].loffset + ch.first,
                              ch.second - ch.first});
      }
    }
  }
  p.add_row.resize(k - 1);
  for (int32_t s = 0; s + 1 < k; ++s) {
    for (int32_t i = 0; i < n; ++i) {
      for (int32_t r = 0; r < k; ++r) {
        const int32_t c = ((r - s - 1) % k + k) % k;  // what r sends at stage s + 1, received at hop s
        if (index[s + 1][(size_t)i * k + c] < 0) continue;
        p.add_row[s].push_back(index[s][(size_t)i * k + c]);
      }
    }
  }
  p.merge = p.stage[k - 1];
  return p;
}

size_t ring_workspace(const RingPlan& p) {
  size_t most = 0;
  for (const auto& seg : p.stage) {
    const Partition ps = stats_partition(seg.data(), (int32_t)seg.size());
    const Partition pe = encode_partition(seg.data(), (int32_t)seg.size());
    most = std::max(most, workspace_layout(ps.n_slots, pe.n_slots, (int32_t)seg.size(), 1).total);
  }
  return most;
}

// fragment_first: n_fragments + 1 nondecreasing offsets from 0, at least one tensor.
// Radial-Directional Averaging: the quantize workspace, then one fp64 direction
// sum per merge block and one coefficient per (tensor, learner).
struct RdaWorkspace {
  size_t quant = 0, dir_part = 0, coef = 0, total = 0;
};

RdaWorkspace rda_workspace(int32_t n_learners, const dlc_tensor* tensors, int32_t n_tensors) {
  RdaWorkspace w;
  const Partition ps = stats_partition(tensors, n_tensors);
  const Partition pe = encode_partition(tensors, n_tensors);
  const Partition pm = direction_partition(tensors, n_tensors);
  w.quant = workspace_layout(ps.n_slots, pe.n_slots, n_tensors, n_learners).total;
  w.dir_part = w.quant;
  w.coef = w.dir_part + round256((size_t)pm.n_slots * sizeof(double));
  w.total = w.coef + round256((size_t)n_tensors * (size_t)n_learners * sizeof(double));
  return w;
}

// One fragment of a cycle merged by Radial-Directional Averaging, in its lane's
// share of the workspace: the quantize layout, one fp64 direction sum per
// direction block, then the coefficient table of every row of the cycle's tables
// ([rows_total][n_learners], the rows k_rda_coef and the merge index).
RdaWorkspace fragment_rda_workspace(int32_t n_learners, const dlc_tensor* tensors, int32_t n_tensors,
                                    int32_t rows_total) {
  RdaWorkspace w;
  const Partition ps = stats_partition(tensors, n_tensors);
  const Partition pe = encode_partition(tensors, n_tensors);
  const Partition pm = direction_partition(tensors, n_tensors);
  w.quant = workspace_layout(ps.n_slots, pe.n_slots, n_tensors, n_learners).total;
  w.dir_part = w.quant;
  w.coef = w.dir_part + round256((size_t)pm.n_slots * sizeof(double));
  w.total = w.coef + round256((size_t)rows_total * (size_t)n_learners * sizeof(double));
  return w;
}

int32_t check_fragments(const dlc_tensor* tensors, const int32_t* fragment_first, int32_t n_fragments) {
  if (!tensors || !fragment_first) return fail(DLC_ERR_INVALID_ARGUMENT, "tensors and fragment_first must not be NULL");
  if (n_fragments < 1) return fail(DLC_ERR_INVALID_ARGUMENT, "n_fragments must be >= 1");
  if (fragment_first[0] != 0) return fail(DLC_ERR_INVALID_ARGUMENT, "fragment_first[0] must be 0");
  for (int32_t f = 0; f < n_fragments; ++f) {
    if (fragment_first[f + 1] < fragment_first[f])
      return fail(DLC_ERR_INVALID_ARGUMENT, "fragment_first must be nondecreasing");
  }
  if (fragment_first[n_fragments] < 1) return fail(DLC_ERR_INVALID_ARGUMENT, "the fragments hold no tensor");
  return DLC_OK;
}

// One event recorded on `from` and waited on by `to`, created and destroyed here
// (a capture on `from` extends to `to` through it).  A stream is already ordered
// after itself: no event then (an event wait between two kernels of one stream
// delays the second by ~5 us).
hipError_t order_after(hipStream_t from, hipStream_t to) {
  if (from == to) return hipSuccess;
  hipEvent_t ev;
  hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventRecord(ev, from);
  if (e == hipSuccess) e = hipStreamWaitEvent(to, ev, 0);
  if (e == hipSuccess) e = hipEventDestroy(ev);
  return e;
}

// The fragment cycle.  n_lanes == 0: quantize calls on quantize_stream, merges
// (and broadcasts) on merge_stream, each merge after its fragment's quantization
// through an event.  n_lanes >= 1: the non-empty fragments take the lanes in turn,
// each lane with its own stream and its own equal share of the workspace, and a
// fragment's quantize, merge and broadcast all run on its lane.  sq_norms set:
// every fragment merges by Radial-Directional Averaging (its direction pass and
// coefficients on the merge's stream, before the merge), with the squared norms
// written to sq_norms [n_learners][rows].
int32_t outer_cycle(float* theta_global, float* momentum, float* theta_learners, int64_t learner_stride,
                    int32_t n_learners, const double* weights, const dlc_tensor* tensors,
                    const int32_t* fragment_first, int32_t n_fragments, uint8_t* codes, float* codebook,
                    float* range, double lr, double beta, bool broadcast, void* workspace, size_t workspace_bytes,
                    hipStream_t quantize_stream, hipStream_t merge_stream, const hipStream_t* lane_streams,
                    int32_t n_lanes, double* sq_norms = nullptr) {
  if (!range || !codes || !codebook) return fail(DLC_ERR_INVALID_ARGUMENT, "range, codes and codebook must not be NULL");
  if (!aligned256(range) || !aligned256(codes) || !aligned256(codebook) || (sq_norms && !aligned256(sq_norms)))
    return fail(DLC_ERR_ALIGNMENT, "range, codes, codebook and sq_norms must be 256-byte aligned");
  const bool rda = sq_norms != nullptr;
  int32_t rc = check_fragments(tensors, fragment_first, n_fragments);
  if (rc != DLC_OK) return rc;
  const int32_t n_tensors = fragment_first[n_fragments];
  rc = check_tensors(tensors, n_tensors, learner_stride, true);
  if (rc != DLC_OK) return rc;
  if (!weights) return fail(DLC_ERR_INVALID_ARGUMENT, "weights is NULL");
  const bool lanes = n_lanes > 0;
  const size_t share = lanes ? (workspace_bytes / (size_t)n_lanes) & ~size_t(255) : workspace_bytes;
  // Every check before anything is enqueued: per-fragment merge arguments and quorum,
  // quantize setup (workspace size) for every non-empty fragment.
  std::vector<dlc::MergeArgs> margs(n_fragments);
  std::vector<Common> qc(n_fragments);
  std::vector<RdaWorkspace> frw(n_fragments);
  std::vector<int32_t> lane(n_fragments, 0);
  std::vector<uint8_t> present(n_learners);
  int32_t busy = 0;
  for (int32_t f = 0; f < n_fragments; ++f) {
    const int32_t n = fragment_first[f + 1] - fragment_first[f];
    if (n == 0) continue;
    lane[f] = lanes ? busy++ % n_lanes : 0;
    const double* w = weights + (size_t)f * n_learners;
    rc = prepare_merge(margs[f], theta_global, momentum, codes, learner_stride, n_learners, codebook, w, lr, beta);
    if (rc != DLC_OK) return fail(rc, "fragment " + std::to_string(f) + ": " + g_last_error);
    for (int32_t i = 0; i < n_learners; ++i) present[i] = w[i] > 0.0 ? 1 : 0;
    void* lane_ws = workspace == nullptr ? nullptr : static_cast<char*>(workspace) + (size_t)lane[f] * share;
    size_t quant_bytes = share;
    if (rda) {
      frw[f] = fragment_rda_workspace(n_learners, tensors + fragment_first[f], n, n_tensors);
      if (lane_ws != nullptr && share < frw[f].total)
        return fail(DLC_ERR_WORKSPACE, "fragment " + std::to_string(f) + ": workspace too small: need " +
                                           std::to_string(frw[f].total) + " bytes per lane");
      quant_bytes = frw[f].quant;
    }
    rc = setup_quant(qc[f], theta_global, theta_learners, learner_stride, n_learners, present.data(),
                     tensors + fragment_first[f], n, lane_ws, quant_bytes,
                     lanes ? lane_streams[lane[f]] : quantize_stream, fragment_first[f], n_tensors);
    if (rc != DLC_OK) return fail(rc, "fragment " + std::to_string(f) + ": " + g_last_error);
    qc[f].args.range = reinterpret_cast<float4*>(range);
    qc[f].args.codes = codes;
    qc[f].args.codebook = codebook;
    qc[f].args.norm2 = sq_norms;
  }
  hipError_t e = hipSuccess;
  // the other lanes start after the work already on the first lane's stream (this
  // also joins them to a capture of that stream)
  for (int32_t l = 1; l < n_lanes && e == hipSuccess; ++l) e = order_after(lane_streams[0], lane_streams[l]);
  if (e != hipSuccess) return hip_fail(e, "cycle event");
  for (int32_t f = 0; f < n_fragments; ++f) {
    const int32_t n = fragment_first[f + 1] - fragment_first[f];
    if (n == 0) continue;
    rc = run_range(qc[f]);
    if (rc == DLC_OK) rc = run_encode(qc[f]);
    if (rc != DLC_OK) return rc;
    hipStream_t ms = merge_stream;
    if (lanes) {
      ms = lane_streams[lane[f]];
    } else {
      // merge of this fragment after its quantization; the next fragment's
      // quantization proceeds on the quantize stream meanwhile
      e = order_after(quantize_stream, merge_stream);
      if (e != hipSuccess) return hip_fail(e, "cycle event");
    }
    if (rda) {
      // direction norms, then the coefficients, then the merge with them (all on ms)
      char* ws = static_cast<char*>(workspace) + (size_t)lane[f] * share;
      dlc::MergeArgs ma = margs[f];
      ma.norm2 = sq_norms;
      ma.dir_part = reinterpret_cast<double*>(ws + frw[f].dir_part);
      Partition pm = direction_partition(tensors + fragment_first[f], n);
      set_rows(pm, fragment_first[f], n_tensors);
      for (const dlc::LaunchGeom& g : pm.launches) {
        e = dlc::launch_rda_direction(ma, g, ms);
        if (e != hipSuccess) return hip_fail(e, "direction kernel launch");
      }
      ma.coef = reinterpret_cast<double*>(ws + frw[f].coef);
      for (const dlc::LaunchGeom& g : pm.launches) {
        e = dlc::launch_rda_coef(ma, g, ms);
        if (e != hipSuccess) return hip_fail(e, "coefficient kernel launch");
      }
      ma.dir_part = nullptr;
      rc = run_merge(ma, tensors + fragment_first[f], n, fragment_first[f], n_tensors, ms);
    } else {
      rc = run_merge(margs[f], tensors + fragment_first[f], n, fragment_first[f], n_tensors, ms);
    }
    if (rc == DLC_OK && broadcast)
      rc = run_broadcast(theta_global, theta_learners, learner_stride, n_learners, nullptr,
                         tensors + fragment_first[f], n, ms);
    if (rc != DLC_OK) return rc;
  }
  // the streams join: any one of them completes the cycle
  if (lanes) {
    for (int32_t l = 1; l < n_lanes && e == hipSuccess; ++l) e = order_after(lane_streams[l], lane_streams[0]);
    for (int32_t l = 1; l < n_lanes && e == hipSuccess; ++l) e = order_after(lane_streams[0], lane_streams[l]);
  } else {
    e = order_after(merge_stream, quantize_stream);
  }
  if (e != hipSuccess) return hip_fail(e, "cycle event");
  return ok();
}

// dlc_quantize after its flag checks, on the given workspace.
int32_t quantize(const float* theta_global, const float* theta_learners, int64_t learner_stride,
                 int32_t n_learners, const uint8_t* present, const dlc_tensor* tensors, int32_t n_tensors,
                 uint8_t* codes, float* codebook, float* range, uint32_t flags, void* workspace,
                 size_t workspace_bytes, void* hip_stream) {
  const bool checks = (flags & DLC_DEBUG_CHECKS) != 0;
  Common c;
  int32_t rc = setup_quant(c, theta_global, theta_learners, learner_stride, n_learners, present, tensors,
                           n_tensors, workspace, workspace_bytes, hip_stream);
  if (rc != DLC_OK) return rc;
  if (!range || !codes || !codebook) return fail(DLC_ERR_INVALID_ARGUMENT, "range, codes and codebook must not be NULL");
  if (!aligned256(range) || !aligned256(codes) || !aligned256(codebook))
    return fail(DLC_ERR_ALIGNMENT, "range, codes and codebook must be 256-byte aligned");
  c.args.range = reinterpret_cast<float4*>(range);
  c.args.codes = codes;
  c.args.codebook = codebook;
  constexpr uint32_t kNone = 0xFFFFFFFFu;
  if (checks) {
    hipError_t e = dlc::launch_fill_u32(c.status, kNone, c.stream);
    if (e != hipSuccess) return hip_fail(e, "status word");
    c.args.status = c.status;
  }
  if ((flags & DLC_RANGE_GIVEN) == 0) {
    rc = run_range(c);
    if (rc != DLC_OK) return rc;
  }
  rc = run_encode(c);
  if (rc != DLC_OK) return rc;
  if (checks) {
    uint32_t first = kNone;
    hipError_t e = hipMemcpyAsync(&first, c.status, sizeof(first), hipMemcpyDeviceToHost, c.stream);
    if (e == hipSuccess) e = hipStreamSynchronize(c.stream);
    if (e != hipSuccess) return hip_fail(e, "debug checks");
    if (first != kNone)
      return fail(DLC_ERR_NON_FINITE, "learner " + std::to_string(first / (uint32_t)n_tensors) + ", tensor " +
                                          std::to_string(first % (uint32_t)n_tensors) +
                                          ": the pseudo-gradient holds NaN or Inf (the lowest such pair)");
  }
  return ok();
}

int32_t check_quantize_flags(uint32_t flags) {
  if ((flags & ~(DLC_RANGE_GIVEN | DLC_DEBUG_CHECKS)) != 0) return fail(DLC_ERR_INVALID_ARGUMENT, "unknown flag");
  if ((flags & DLC_DEBUG_CHECKS) != 0 && (flags & DLC_RANGE_GIVEN) != 0)
    return fail(DLC_ERR_INVALID_ARGUMENT, "DLC_DEBUG_CHECKS needs the statistics stage (not DLC_RANGE_GIVEN)");
  return DLC_OK;
}

// Workspace bytes of a quantize call with kp present learners (the layout setup_quant uses).
size_t quantize_workspace(const dlc_tensor* tensors, int32_t n_tensors, int32_t kp) {
  const Partition ps = stats_partition(tensors, n_tensors);
  const Partition pe = encode_partition(tensors, n_tensors);
  return workspace_layout(ps.n_slots, pe.n_slots, n_tensors, kp).total;
}

// Learners grouped by base (groups in order of first appearance), one quantize
// setup per group on the same workspace (the groups run one after another on the
// stream); every group checked before anything is enqueued.
int32_t setup_base_groups(std::vector<Common>& groups, const float* const* bases, const float* theta_learners,
                          int64_t learner_stride, int32_t n_learners, const uint8_t* present,
                          const dlc_tensor* tensors, int32_t n_tensors, void* workspace, size_t workspace_bytes,
                          void* hip_stream) {
  std::vector<const float*> order;
  for (int32_t i = 0; i < n_learners; ++i) {
    if (present != nullptr && present[i] == 0) continue;
    if (!bases[i]) return fail(DLC_ERR_INVALID_ARGUMENT, "bases[" + std::to_string(i) + "] is NULL");
    if (std::find(order.begin(), order.end(), bases[i]) == order.end()) order.push_back(bases[i]);
  }
  if (order.empty()) return fail(DLC_ERR_NO_QUORUM, "no learner is present");
  groups.assign(order.size(), Common());
  std::vector<uint8_t> member(n_learners);
  for (size_t gi = 0; gi < order.size(); ++gi) {
    for (int32_t i = 0; i < n_learners; ++i)
      member[i] = (present == nullptr || present[i] != 0) && bases[i] == order[gi] ? 1 : 0;
    const int32_t rc = setup_quant(groups[gi], order[gi], theta_learners, learner_stride, n_learners, member.data(),
                                   tensors, n_tensors, workspace, workspace_bytes, hip_stream);
    if (rc != DLC_OK) return rc;
  }
  return DLC_OK;
}

// The static scratch of dlc_quantize_static (the array is declared at the top of
// this file).  Host code never uses the array's name as an address: its address
// on each device comes from hipGetSymbolAddress, looked up once per device (the
// first call whose stream is on that device) with that device current, and kept.
constexpr size_t kStaticScratchBytes = DLC_STATIC_SCRATCH_BYTES;
static_assert(kStaticScratchBytes % 256 == 0, "whole 256-byte units");

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The device a call's work runs on: the stream's (the current device's for the
// null stream).
int32_t stream_device(hipStream_t s, int* dev) {
  const hipError_t e = s == nullptr ? hipGetDevice(dev) : hipStreamGetDevice(s, dev);
  return e == hipSuccess ? DLC_OK : hip_fail(e, "the stream's device");
}

// Device dev's address of the scratch array.  The lookup makes dev current and
// restores the caller's device afterwards.
int32_t static_scratch(int dev, void** ptr) {
  if (dev < 0 || dev >= kMaxDevices) return fail(DLC_ERR_HIP, "device index beyond the scratch table");
  std::call_once(g_scratch_once[dev], [dev] {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (e == hipSuccess) e = back;
    }
    g_scratch_err[dev] = e;
    g_scratch_ptr[dev] = e == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return hip_fail(g_scratch_err[dev], "static scratch address");
  if (g_scratch_ptr[dev] == nullptr || !aligned256(g_scratch_ptr[dev]))
    return fail(DLC_ERR_HIP, "static scratch address is not 256-byte aligned");
  *ptr = g_scratch_ptr[dev];
  return DLC_OK;
}

}  // namespace

extern "C" {

int32_t dlc_fragment_plan(const int64_t* numel, int32_t n_tensors, int32_t n_fragments,
                          int32_t* fragment_of, int64_t* fragment_numel) {
  if (!numel || !fragment_of) return fail(DLC_ERR_INVALID_ARGUMENT, "numel and fragment_of must not be NULL");
  if (n_tensors < 1) return fail(DLC_ERR_INVALID_ARGUMENT, "n_tensors must be >= 1");
  if (n_fragments < 1) return fail(DLC_ERR_INVALID_ARGUMENT, "n_fragments must be >= 1");
  for (int32_t i = 0; i < n_tensors; ++i)
    if (numel[i] < 1) return fail(DLC_ERR_INVALID_ARGUMENT, "numel must be >= 1");
  std::vector<int32_t> order(n_tensors);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return numel[a] > numel[b]; });
  std::vector<int64_t> load(n_fragments, 0);
  for (int32_t t : order) {
    int32_t best = 0;
    for (int32_t p = 1; p < n_fragments; ++p)
      if (load[p] < load[best]) best = p;
    fragment_of[t] = best;
    load[best] += numel[t];
  }
  if (fragment_numel) std::copy(load.begin(), load.end(), fragment_numel);
  return ok();
}

int32_t dlc_workspace_bytes(int32_t n_learners, const dlc_tensor* tensors, int32_t n_tensors,
                            size_t* bytes) {
  if (!bytes) return fail(DLC_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (n_learners < 1 || n_learners > DLC_MAX_LEARNERS)
    return fail(DLC_ERR_INVALID_ARGUMENT, "n_learners must be in [1, 64]");
  int32_t rc = check_tensors(tensors, n_tensors, 0, false);
  if (rc != DLC_OK) return rc;
  const Partition ps = stats_partition(tensors, n_tensors);
  const Partition pe = encode_partition(tensors, n_tensors);
  *bytes = workspace_layout(ps.n_slots, pe.n_slots, n_tensors, n_learners).total;
  return ok();
}

int32_t dlc_quantize_range(const float* theta_global, const float* theta_learners,
                           int64_t learner_stride, int32_t n_learners, const uint8_t* present,
                           const dlc_tensor* tensors, int32_t n_tensors, float* range,
                           void* workspace, size_t workspace_bytes, void* hip_stream) {
  Common c;
  int32_t rc = setup_quant(c, theta_global, theta_learners, learner_stride, n_learners, present, tensors,
                           n_tensors, workspace, workspace_bytes, hip_stream);
  if (rc != DLC_OK) return rc;
  if (!range) return fail(DLC_ERR_INVALID_ARGUMENT, "range is NULL");
  if (!aligned256(range)) return fail(DLC_ERR_ALIGNMENT, "range must be 256-byte aligned");
  c.args.range = reinterpret_cast<float4*>(range);
  rc = run_range(c);
  return rc == DLC_OK ? ok() : rc;
}

int32_t dlc_quantize_encode(const float* theta_global, const float* theta_learners,
                            int64_t learner_stride, int32_t n_learners, const uint8_t* present,
                            const dlc_tensor* tensors, int32_t n_tensors, const float* range,
                            uint8_t* codes, float* codebook, void* workspace,
                            size_t workspace_bytes, void* hip_stream) {
  Common c;
  int32_t rc = setup_quant(c, theta_global, theta_learners, learner_stride, n_learners, present, tensors,
                           n_tensors, workspace, workspace_bytes, hip_stream);
  if (rc != DLC_OK) return rc;
  if (!range || !codes || !codebook) return fail(DLC_ERR_INVALID_ARGUMENT, "range, codes and codebook must not be NULL");
  if (!aligned256(range) || !aligned256(codes) || !aligned256(codebook))
    return fail(DLC_ERR_ALIGNMENT, "range, codes and codebook must be 256-byte aligned");
  c.args.range = reinterpret_cast<float4*>(const_cast<float*>(range));
  c.args.codes = codes;
  c.args.codebook = codebook;
  rc = run_encode(c);
  return rc == DLC_OK ? ok() : rc;
}

int32_t dlc_quantize(const float* theta_global, const float* theta_learners,
                     int64_t learner_stride, int32_t n_learners, const uint8_t* present,
                     const dlc_tensor* tensors, int32_t n_tensors, uint8_t* codes,
                     float* codebook, float* range, uint32_t flags, void* workspace,
                     size_t workspace_bytes, void* hip_stream) {
  int32_t rc = check_quantize_flags(flags);
  if (rc != DLC_OK) return rc;
  return quantize(theta_global, theta_learners, learner_stride, n_learners, present, tensors, n_tensors, codes,
                  codebook, range, flags, workspace, workspace_bytes, hip_stream);
}

int32_t dlc_quantize_static(const float* theta_global, const float* theta_learners, int64_t learner_stride,
                            int32_t n_learners, const uint8_t* present, const dlc_tensor* tensors,
                            int32_t n_tensors, uint8_t* codes, float* codebook, float* range, uint32_t flags,
                            void* hip_stream) {
  int32_t rc = check_quantize_flags(flags);
  if (rc != DLC_OK) return rc;
  // the scratch this call needs, checked before any HIP call
  if (n_learners < 1 || n_learners > DLC_MAX_LEARNERS)
    return fail(DLC_ERR_INVALID_ARGUMENT, "n_learners must be in [1, 64]");
  rc = check_tensors(tensors, n_tensors, learner_stride, true);
  if (rc != DLC_OK) return rc;
  int32_t kp = 0;
  for (int32_t i = 0; i < n_learners; ++i) kp += present == nullptr || present[i] != 0 ? 1 : 0;
  if (kp == 0) return fail(DLC_ERR_NO_QUORUM, "no learner is present");
  const size_t need = quantize_workspace(tensors, n_tensors, kp);
  if (need > kStaticScratchBytes)
    return fail(DLC_ERR_WORKSPACE, "the call needs " + std::to_string(need) + " bytes of scratch, more than the " +
                                       std::to_string(kStaticScratchBytes) +
                                       " of the static scratch: split it into smaller fragments, or pass a "
                                       "workspace to dlc_quantize");
  int dev = -1;
  rc = stream_device(static_cast<hipStream_t>(hip_stream), &dev);
  if (rc != DLC_OK) return rc;
  void* ws = nullptr;
  rc = static_scratch(dev, &ws);
  if (rc != DLC_OK) return rc;
  return quantize(theta_global, theta_learners, learner_stride, n_learners, present, tensors, n_tensors, codes,
                  codebook, range, flags, ws, kStaticScratchBytes, hip_stream);
}

int32_t dlc_quantize_bases(const float* const* bases, const float* theta_learners, int64_t learner_stride,
                           int32_t n_learners, const uint8_t* present, const dlc_tensor* tensors,
                           int32_t n_tensors, uint8_t* codes, float* codebook, float* range, void* workspace,
                           size_t workspace_bytes, void* hip_stream) {
  if (!bases) return fail(DLC_ERR_INVALID_ARGUMENT, "bases is NULL");
  if (n_learners < 1 || n_learners > DLC_MAX_LEARNERS)
    return fail(DLC_ERR_INVALID_ARGUMENT, "n_learners must be in [1, 64]");
  if (!range || !codes || !codebook) return fail(DLC_ERR_INVALID_ARGUMENT, "range, codes and codebook must not be NULL");
  if (!aligned256(range) || !aligned256(codes) || !aligned256(codebook))
    return fail(DLC_ERR_ALIGNMENT, "range, codes and codebook must be 256-byte aligned");
  std::vector<Common> groups;
  int32_t rc = setup_base_groups(groups, bases, theta_learners, learner_stride, n_learners, present, tensors,
                                 n_tensors, workspace, workspace_bytes, hip_stream);
  if (rc != DLC_OK) return rc;
  for (Common& c : groups) {
    c.args.range = reinterpret_cast<float4*>(range);
    c.args.codes = codes;
    c.args.codebook = codebook;
  }
  // one workspace: the groups run one after another on the stream
  for (Common& c : groups) {
    int32_t rc = run_range(c);
    if (rc == DLC_OK) rc = run_encode(c);
    if (rc != DLC_OK) return rc;
  }
  return ok();
}

int32_t dlc_merge_outer_step(float* theta_global, float* momentum, const uint8_t* codes,
                             int64_t learner_stride, int32_t n_learners, const float* codebook,
                             const double* weights, const dlc_tensor* tensors, int32_t n_tensors,
                             double lr, double beta, uint32_t flags, void* hip_stream) {
  if (flags != 0) return fail(DLC_ERR_INVALID_ARGUMENT, "flags must be 0");
  dlc::MergeArgs a;
  int32_t rc = prepare_merge(a, theta_global, momentum, codes, learner_stride, n_learners, codebook, weights, lr, beta);
  if (rc != DLC_OK) return rc;
  rc = check_tensors(tensors, n_tensors, learner_stride, true);
  if (rc != DLC_OK) return rc;
  rc = run_merge(a, tensors, n_tensors, 0, -1, static_cast<hipStream_t>(hip_stream));
  return rc == DLC_OK ? ok() : rc;
}

int32_t dlc_broadcast(const float* theta_global, float* theta_learners, int64_t learner_stride,
                      int32_t n_learners, const uint8_t* rows, const dlc_tensor* tensors, int32_t n_tensors,
                      void* hip_stream) {
  if (n_learners < 1 || n_learners > DLC_MAX_LEARNERS)
    return fail(DLC_ERR_INVALID_ARGUMENT, "n_learners must be in [1, 64]");
  if (!theta_global || !theta_learners) return fail(DLC_ERR_INVALID_ARGUMENT, "theta pointer is NULL");
  if (!aligned256(theta_global) || !aligned256(theta_learners))
    return fail(DLC_ERR_ALIGNMENT, "theta pointers must be 256-byte aligned");
  int32_t rc = check_tensors(tensors, n_tensors, learner_stride, true);
  if (rc != DLC_OK) return rc;
  rc = run_broadcast(theta_global, theta_learners, learner_stride, n_learners, rows, tensors, n_tensors,
                     static_cast<hipStream_t>(hip_stream));
  return rc == DLC_OK ? ok() : rc;
}

int32_t dlc_cycle_workspace_bytes(int32_t n_learners, const dlc_tensor* tensors, const int32_t* fragment_first,
                                  int32_t n_fragments, size_t* bytes) {
  if (!bytes) return fail(DLC_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (n_learners < 1 || n_learners > DLC_MAX_LEARNERS)
    return fail(DLC_ERR_INVALID_ARGUMENT, "n_learners must be in [1, 64]");
  int32_t rc = check_fragments(tensors, fragment_first, n_fragments);
  if (rc != DLC_OK) return rc;
  size_t most = 0;
  for (int32_t f = 0; f < n_fragments; ++f) {
    const int32_t n = fragment_first[f + 1] - fragment_first[f];
    if (n == 0) continue;
    const dlc_tensor* t = tensors + fragment_first[f];
    rc = check_tensors(t, n, 0, false);
    if (rc != DLC_OK) return rc;
    const Partition ps = stats_partition(t, n);
    const Partition pe = encode_partition(t, n);
    most = std::max(most, workspace_layout(ps.n_slots, pe.n_slots, n, n_learners).total);
  }
  *bytes = most;
  return ok();
}

int32_t dlc_outer_cycle(float* theta_global, float* momentum, float* theta_learners, int64_t learner_stride,
                        int32_t n_learners, const double* weights, const dlc_tensor* tensors,
                        const int32_t* fragment_first, int32_t n_fragments, uint8_t* codes, float* codebook,
                        float* range, double lr, double beta, uint32_t flags, void* workspace,
                        size_t workspace_bytes, void* quantize_stream, void* merge_stream) {
  if ((flags & ~(DLC_BROADCAST | DLC_TWO_LANES)) != 0) return fail(DLC_ERR_INVALID_ARGUMENT, "unknown flag");
  const hipStream_t qs = static_cast<hipStream_t>(quantize_stream), ms = static_cast<hipStream_t>(merge_stream);
  const hipStream_t two[2] = {qs, ms};
  const bool lanes = (flags & DLC_TWO_LANES) != 0;
  return outer_cycle(theta_global, momentum, theta_learners, learner_stride, n_learners, weights, tensors,
                     fragment_first, n_fragments, codes, codebook, range, lr, beta, (flags & DLC_BROADCAST) != 0,
                     workspace, workspace_bytes, qs, ms, two, lanes ? 2 : 0);
}

int32_t dlc_outer_cycle_lanes(float* theta_global, float* momentum, float* theta_learners, int64_t learner_stride,
                              int32_t n_learners, const double* weights, const dlc_tensor* tensors,
                              const int32_t* fragment_first, int32_t n_fragments, uint8_t* codes, float* codebook,
                              float* range, double lr, double beta, uint32_t flags, void* workspace,
                              size_t workspace_bytes, void* const* streams, int32_t n_lanes) {
  if ((flags & ~DLC_BROADCAST) != 0) return fail(DLC_ERR_INVALID_ARGUMENT, "unknown flag");
  if (n_lanes < 1 || n_lanes > DLC_MAX_LANES) return fail(DLC_ERR_INVALID_ARGUMENT, "n_lanes must be in [1, 8]");
  if (!streams) return fail(DLC_ERR_INVALID_ARGUMENT, "streams is NULL");
  hipStream_t lane_streams[DLC_MAX_LANES];
  for (int32_t l = 0; l < n_lanes; ++l) lane_streams[l] = static_cast<hipStream_t>(streams[l]);
  return outer_cycle(theta_global, momentum, theta_learners, learner_stride, n_learners, weights, tensors,
                     fragment_first, n_fragments, codes, codebook, range, lr, beta, (flags & DLC_BROADCAST) != 0,
                     workspace, workspace_bytes, lane_streams[0], lane_streams[0], lane_streams, n_lanes);
}

int32_t dlc_cycle_rda_workspace_bytes(int32_t n_learners, const dlc_tensor* tensors, const int32_t* fragment_first,
                                      int32_t n_fragments, size_t* bytes) {
  if (!bytes) return fail(DLC_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (n_learners < 1 || n_learners > DLC_MAX_LEARNERS)
    return fail(DLC_ERR_INVALID_ARGUMENT, "n_learners must be in [1, 64]");
  int32_t rc = check_fragments(tensors, fragment_first, n_fragments);
  if (rc != DLC_OK) return rc;
  const int32_t rows = fragment_first[n_fragments];
  size_t most = 0;
  for (int32_t f = 0; f < n_fragments; ++f) {
    const int32_t n = fragment_first[f + 1] - fragment_first[f];
    if (n == 0) continue;
    const dlc_tensor* t = tensors + fragment_first[f];
    rc = check_tensors(t, n, 0, false);
    if (rc != DLC_OK) return rc;
    most = std::max(most, fragment_rda_workspace(n_learners, t, n, rows).total);
  }
  *bytes = most;
  return ok();
}

int32_t dlc_outer_cycle_rda(float* theta_global, float* momentum, float* theta_learners, int64_t learner_stride,
                            int32_t n_learners, const double* weights, const dlc_tensor* tensors,
                            const int32_t* fragment_first, int32_t n_fragments, uint8_t* codes, float* codebook,
                            float* range, double* sq_norms, double lr, double beta, uint32_t flags, void* workspace,
                            size_t workspace_bytes, void* const* streams, int32_t n_lanes) {
  if ((flags & ~DLC_BROADCAST) != 0) return fail(DLC_ERR_INVALID_ARGUMENT, "unknown flag");
  if (n_lanes < 1 || n_lanes > DLC_MAX_LANES) return fail(DLC_ERR_INVALID_ARGUMENT, "n_lanes must be in [1, 8]");
  if (!streams) return fail(DLC_ERR_INVALID_ARGUMENT, "streams is NULL");
  if (!sq_norms) return fail(DLC_ERR_INVALID_ARGUMENT, "sq_norms is NULL");
  hipStream_t lane_streams[DLC_MAX_LANES];
  for (int32_t l = 0; l < n_lanes; ++l) lane_streams[l] = static_cast<hipStream_t>(streams[l]);
  return outer_cycle(theta_global, momentum, theta_learners, learner_stride, n_learners, weights, tensors,
                     fragment_first, n_fragments, codes, codebook, range, lr, beta, (flags & DLC_BROADCAST) != 0,
                     workspace, workspace_bytes, lane_streams[0], lane_streams[0], lane_streams, n_lanes, sq_norms);
}

int32_t dlc_merge_weights(int32_t n_learners, const double* tokens, const double* arrival, int32_t quorum,
                          double grace, double* weights, double* merge_time) {
  if (n_learners < 1 || n_learners > DLC_MAX_LEARNERS)
    return fail(DLC_ERR_INVALID_ARGUMENT, "n_learners must be in [1, 64]");
  if (!tokens || !arrival || !weights) return fail(DLC_ERR_INVALID_ARGUMENT, "tokens, arrival and weights must not be NULL");
  if (quorum < 1 || quorum > n_learners) return fail(DLC_ERR_INVALID_ARGUMENT, "quorum must be in [1, n_learners]");
  if (!(grace >= 0.0) || std::isinf(grace)) return fail(DLC_ERR_INVALID_ARGUMENT, "grace must be finite and >= 0");
  std::vector<int32_t> arrived;
  for (int32_t i = 0; i < n_learners; ++i) {
    if (std::isfinite(arrival[i])) {
      if (arrival[i] < 0.0) return fail(DLC_ERR_INVALID_ARGUMENT, "arrival times must be >= 0");
      if (!(tokens[i] >= 0.0) || !std::isfinite(tokens[i]))
        return fail(DLC_ERR_INVALID_ARGUMENT, "tokens of an arrived learner must be finite and >= 0");
      arrived.push_back(i);
    }
  }
  if ((int32_t)arrived.size() < quorum) return fail(DLC_ERR_NO_QUORUM, "fewer learners arrived than the quorum");
  // the quorum is met when the quorum-th earliest learner arrives (ties: lower index first)
  std::stable_sort(arrived.begin(), arrived.end(), [&](int32_t a, int32_t b) { return arrival[a] < arrival[b]; });
  const double t_quorum = arrival[arrived[quorum - 1]];
  const double deadline = t_quorum + grace;
  double total = 0.0, last = t_quorum;
  std::vector<double> w(n_learners, 0.0);
  for (int32_t i : arrived) {
    if (arrival[i] <= deadline) {
      w[i] = tokens[i];
      total += tokens[i];
      last = std::max(last, arrival[i]);
    }
  }
  if (!(total > 0.0)) return fail(DLC_ERR_NO_QUORUM, "the merged learners report no tokens");
  std::copy(w.begin(), w.end(), weights);
  if (merge_time) *merge_time = (int32_t)arrived.size() == n_learners && last < deadline ? last : deadline;
  return ok();
}

int32_t dlc_ring_workspace_bytes(int32_t n_learners, const dlc_tensor* tensors, int32_t n_tensors, size_t* bytes) {
  if (!bytes) return fail(DLC_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (n_learners < 1 || n_learners > DLC_MAX_LEARNERS)
    return fail(DLC_ERR_INVALID_ARGUMENT, "n_learners must be in [1, 64]");
  int32_t rc = check_tensors(tensors, n_tensors, 0, false);
  if (rc != DLC_OK) return rc;
  // segment sizes do not depend on the row stride
  int64_t span = 0;
  for (int32_t i = 0; i < n_tensors; ++i) span = std::max(span, tensors[i].loffset + tensors[i].numel);
  const int64_t stride = (span + DLC_ALIGN_ELEMS - 1) / DLC_ALIGN_ELEMS * DLC_ALIGN_ELEMS;
  *bytes = ring_workspace(ring_plan(tensors, n_tensors, n_learners, stride));
  return ok();
}

int32_t dlc_ring_outer_step(float* theta_global, float* momentum, const float* theta_learners,
                            int64_t learner_stride, int32_t n_learners, const dlc_tensor* tensors, int32_t n_tensors,
                            double lr, double beta, float* accum, uint8_t* codes, float* codebook, float* range,
                            void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (n_learners < 1 || n_learners > DLC_MAX_LEARNERS)
    return fail(DLC_ERR_INVALID_ARGUMENT, "n_learners must be in [1, 64]");
  if (!theta_global || !momentum || !theta_learners || !accum || !codes || !codebook || !range)
    return fail(DLC_ERR_INVALID_ARGUMENT, "a buffer pointer is NULL");
  if (!aligned256(theta_global) || !aligned256(momentum) || !aligned256(theta_learners) || !aligned256(accum) ||
      !aligned256(codes) || !aligned256(codebook) || !aligned256(range))
    return fail(DLC_ERR_ALIGNMENT, "device pointers must be 256-byte aligned");
  if (!std::isfinite(lr) || !std::isfinite(beta)) return fail(DLC_ERR_INVALID_ARGUMENT, "lr and beta must be finite");
  int32_t rc = check_tensors(tensors, n_tensors, learner_stride, true);
  if (rc != DLC_OK) return rc;
  const int32_t k = n_learners;
  const int64_t flat = (int64_t)k * learner_stride;
  const RingPlan plan = ring_plan(tensors, n_tensors, k, learner_stride);
  if (workspace == nullptr || workspace_bytes < ring_workspace(plan))
    return fail(DLC_ERR_WORKSPACE, "workspace too small: need " + std::to_string(ring_workspace(plan)) + " bytes");
  // Every quantize call set up (and checked) before anything is enqueued.  The
  // range side of a stage reads theta_global and theta_learners (k_range's shift is
  // the sender's pseudo-gradient at the segment's first element, the shift the
  // dequantize-add used); stage 0 runs its statistics pass and encodes from them
  // too, later stages encode the negated sums in accum with no base.
  std::vector<Common> rng_c(k), enc_c(k);
  for (int32_t s = 0; s < k; ++s) {
    const std::vector<dlc_tensor>& seg = plan.stage[s];
    rc = setup_quant(rng_c[s], theta_global, theta_learners, flat, 1, nullptr, seg.data(), (int32_t)seg.size(),
                     workspace, workspace_bytes, hip_stream);
    if (rc == DLC_OK && s > 0)
      rc = setup_quant(enc_c[s], nullptr, accum, flat, 1, nullptr, seg.data(), (int32_t)seg.size(), workspace,
                       workspace_bytes, hip_stream, 0, -1, true);
    if (rc != DLC_OK) return rc;
    if (s == 0) enc_c[s] = rng_c[s];
    for (Common* c : {&rng_c[s], &enc_c[s]}) {
      c->args.range = reinterpret_cast<float4*>(range);
      c->args.codes = codes;
      c->args.codebook = codebook;
    }
  }
  dlc::MergeArgs ma;
  const double one = 1.0;
  rc = prepare_merge(ma, theta_global, momentum, codes, flat, 1, codebook, &one, lr, beta);
  if (rc != DLC_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  dlc::RingArgs ra;
  std::memset(&ra, 0, sizeof(ra));
  ra.theta_g = theta_global;
  ra.theta_L = theta_learners;
  ra.stride = learner_stride;
  ra.n_ranks = k;
  ra.accum = accum;
  ra.codes = codes;
  ra.codebook = codebook;
  for (int32_t s = 0; s < k; ++s) {
    // this stage's messages: range (stage 0 with its statistics pass), encode, codebook
    if (s == 0) {
      rc = run_range(rng_c[s]);
    } else {
      for (const dlc::LaunchGeom& g : rng_c[s].part_stats.launches) {
        hipError_t e = dlc::launch_range(rng_c[s].args, g, st);
        if (e != hipSuccess) return hip_fail(e, "range kernel launch");
      }
    }
    if (rc == DLC_OK) rc = run_encode(enc_c[s]);
    if (rc != DLC_OK) return rc;
    if (s + 1 == k) break;
    // hop s: the receivers add, in the statistics partition of stage s + 1, whose
    // partials they write; the last hop leaves the owners' means
    ra.divisor = s + 2 == k ? (float)k : 0.0f;
    ra.part_stats = rng_c[s + 1].args.part_stats;
    for (const dlc::LaunchGeom& g : rng_c[s + 1].part_stats.launches) {
      for (int32_t j = 0; j < g.n_tensors; ++j) ra.cb_row[j] = plan.add_row[s][g.t_base + j];
      hipError_t e = dlc::launch_dequant_add(ra, g, st);
      if (e != hipSuccess) return hip_fail(e, "dequantize-add kernel launch");
    }
  }
  // the gather's messages reach every rank unchanged, so the merge reads them directly
  rc = run_merge(ma, plan.merge.data(), (int32_t)plan.merge.size(), 0, -1, st);
  return rc == DLC_OK ? ok() : rc;
}

int32_t dlc_rda_workspace_bytes(int32_t n_learners, const dlc_tensor* tensors, int32_t n_tensors, size_t* bytes) {
  if (!bytes) return fail(DLC_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (n_learners < 1 || n_learners > DLC_MAX_LEARNERS)
    return fail(DLC_ERR_INVALID_ARGUMENT, "n_learners must be in [1, 64]");
  int32_t rc = check_tensors(tensors, n_tensors, 0, false);
  if (rc != DLC_OK) return rc;
  *bytes = rda_workspace(n_learners, tensors, n_tensors).total;
  return ok();
}

int32_t dlc_rda_outer_step(float* theta_global, float* momentum, const float* theta_learners,
                           const float* const* bases, int64_t learner_stride, int32_t n_learners,
                           const dlc_tensor* tensors, int32_t n_tensors,
                           const double* weights, double lr, double beta, uint8_t* codes, float* codebook,
                           float* range, double* sq_norms, void* workspace, size_t workspace_bytes,
                           void* hip_stream) {
  dlc::MergeArgs ma;
  int32_t rc = prepare_merge(ma, theta_global, momentum, codes, learner_stride, n_learners, codebook, weights, lr, beta);
  if (rc != DLC_OK) return rc;
  if (!range || !sq_norms) return fail(DLC_ERR_INVALID_ARGUMENT, "range and sq_norms must not be NULL");
  if (!aligned256(range) || !aligned256(sq_norms))
    return fail(DLC_ERR_ALIGNMENT, "range and sq_norms must be 256-byte aligned");
  rc = check_tensors(tensors, n_tensors, learner_stride, true);
  if (rc != DLC_OK) return rc;
  const RdaWorkspace rw = rda_workspace(n_learners, tensors, n_tensors);
  if (workspace == nullptr || workspace_bytes < rw.total)
    return fail(DLC_ERR_WORKSPACE, "workspace too small: need " + std::to_string(rw.total) + " bytes");
  // learners with a positive weight are quantized and merged, against theta_global
  // or, with bases, each against its own base (one quantize per distinct base)
  std::vector<uint8_t> present(n_learners);
  for (int32_t i = 0; i < n_learners; ++i) present[i] = weights[i] > 0.0 ? 1 : 0;
  std::vector<Common> groups;
  if (bases == nullptr) {
    groups.resize(1);
    rc = setup_quant(groups[0], theta_global, theta_learners, learner_stride, n_learners, present.data(), tensors,
                     n_tensors, workspace, rw.quant, hip_stream);
  } else {
    rc = setup_base_groups(groups, bases, theta_learners, learner_stride, n_learners, present.data(), tensors,
                           n_tensors, workspace, rw.quant, hip_stream);
  }
  if (rc != DLC_OK) return rc;
  for (Common& c : groups) {
    c.args.range = reinterpret_cast<float4*>(range);
    c.args.codes = codes;
    c.args.codebook = codebook;
    c.args.norm2 = sq_norms;
  }
  char* ws = static_cast<char*>(workspace);
  ma.norm2 = sq_norms;
  ma.dir_part = reinterpret_cast<double*>(ws + rw.dir_part);
  ma.coef = nullptr;
  double* coef = reinterpret_cast<double*>(ws + rw.coef);
  const Partition pm = direction_partition(tensors, n_tensors);
  for (Common& c : groups) {
    rc = run_range(c);
    if (rc == DLC_OK) rc = run_encode(c);
    if (rc != DLC_OK) return rc;
  }
  const hipStream_t st = groups[0].stream;
  for (const dlc::LaunchGeom& g : pm.launches) {
    hipError_t e = dlc::launch_rda_direction(ma, g, st);
    if (e != hipSuccess) return hip_fail(e, "direction kernel launch");
  }
  ma.coef = coef;
  for (const dlc::LaunchGeom& g : pm.launches) {
    hipError_t e = dlc::launch_rda_coef(ma, g, st);
    if (e != hipSuccess) return hip_fail(e, "coefficient kernel launch");
  }
  ma.dir_part = nullptr;
  rc = run_merge(ma, tensors, n_tensors, 0, -1, st);
  return rc == DLC_OK ? ok() : rc;
}

const char* dlc_last_error(void) { return g_last_error.c_str(); }

const char* dlc_version(void) { return "dlc 0.1.0 (gfx950)"; }

}  // extern "C"
