// Internal launch descriptors shared by the host orchestration and the gfx950 kernels.
//
// A call's tensors are processed in launches of at most kMaxTensorsPerLaunch
// tensors.  Every launch carries its tensor descriptors in the kernel arguments
// (no device-side tables, no host-to-device copies).  Within a launch each tensor
// owns a contiguous run of blocks; block j of tensor t covers tiles
// [j * tiles_per_block, (j + 1) * tiles_per_block) of that tensor only, so every
// block's partial statistics / histogram belong to exactly one tensor and sit in
// the workspace slot slot_base + blockIdx.x.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace dlc {

constexpr int kBuckets = 256;
constexpr int kMaxLearners = 64;
constexpr int kMaxTensorsPerLaunch = 160;
constexpr int kVec = 16;                  // elements per thread per tile (4 x float4)
constexpr int kBlock = 256;               // threads per block
constexpr int kTile = kBlock * kVec;      // elements per tile
constexpr int kLearnerChunk = 16;         // learners per encode launch
// Bucket histograms are packed 64-bit integers: bits 44..63 count elements, bits
// 0..43 sum each element's position inside its bucket in units of wd * 2^-s
// (s <= kHistFracBits), offset by a per-(learner, tensor) bias of at least kHistBias
// that keeps every position in [0, 2^27).  An encode block covers at most
// kMaxEncodeTiles full tiles of a tensor (whole groups of 4 tiles) plus, in the
// tensor's last block, its partial last tile: under 29 * 4096 < 2^17 elements per
// learner, so neither field can overflow: 2^17 * 2^27 <= 2^44 and 2^17 < 2^20.
constexpr int kMaxEncodeTiles = 28;
constexpr int kEncodeGroupTiles = 4;      // tiles per encode group
// The codebook stage sums a tensor's block histograms in slices of kHistSlice
// blocks (unpacked: 64 * 2^17 elements keep the count within 2^23 and the
// position sum within 2^50), then the slices.
constexpr int kHistSlice = 64;
constexpr int kHistFracBits = 26;
constexpr int kHistBias = 1 << 13;
constexpr int kHistCountShift = 44;
// Tiles a merge block works on side by side (kBlock threads each).  The kernel
// supports 1, 2 and 4; wider blocks measured slower on the 1B parameter set.
constexpr int kMergeTiles = 1;
constexpr int kStatsChunk = 14;           // learners per statistics launch (register accumulators)

// 16 bytes per tensor so that up to kMaxTensorsPerLaunch descriptors fit in the
// kernel arguments: offsets in units of 64 elements, numel below 2^32.
struct TensorDesc {
  uint32_t off64;       // offset into theta_global / momentum, in units of 64 elements
  uint32_t loff64;      // offset into each learner row, in units of 64 elements
  uint32_t count;       // number of elements
  int32_t block_first;  // first block of this tensor within the launch
  __host__ __device__ int64_t offset() const { return (int64_t)off64 * 64; }
  __host__ __device__ int64_t loffset() const { return (int64_t)loff64 * 64; }
  __host__ __device__ int64_t numel() const { return (int64_t)count; }
};

struct LaunchGeom {
  int32_t n_tensors;        // tensors in this launch
  int32_t t_base;           // call-level index of the launch's first tensor
  int32_t n_tensors_call;   // row length of range / codebook
  int32_t row_base;         // range / codebook row of the call's first tensor (0 unless part of a cycle)
  int32_t n_blocks;         // blocks in this launch
  int32_t tiles_per_block;
  int32_t slot_base;        // workspace slot of block 0
  int32_t hist_slices;      // most histogram slices of one tensor in this launch (encode partition)
  TensorDesc t[kMaxTensorsPerLaunch];
};

struct QuantArgs {
  const float* theta_g;
  const float* theta_L;
  int64_t stride;           // learner row length (elements)
  int32_t n_present;        // present learners in the call
  int32_t k_base;           // first present-learner position handled by this launch
  int32_t k_count;          // present learners handled by this launch (<= kLearnerChunk)
  int32_t learner[kMaxLearners];  // present position -> learner index
  float4* range;            // [n_learners][n_tensors_call] {lo, hi, wd, mean}
  uint8_t* codes;           // [n_learners][stride]
  float* codebook;          // [n_learners][n_tensors_call][256]
  double2* part_stats;      // [slot][n_present] {sum(d), sum(d^2)}, d = Delta - shift
  uint64_t* part_hist;      // [slot][n_present][256] packed (count, position sum)
  uint64_t* hist_sum;       // [slice entry][n_present][256][2] {position sum, count}, see hist_entry
  double* norm2;            // optional [n_learners][n_tensors_call]: sum over the tensor of the
                            // dequantized values squared, sum_c count_c * codebook_c^2 (fp64)
  uint32_t* status;         // optional: lowest learner * n_tensors_call + row whose statistics
                            // are not finite (k_range), 0xFFFFFFFF when none
};

struct MergeArgs {
  float* theta_g;
  float* momentum;
  const uint8_t* codes;
  const float* codebook;
  int64_t stride;
  int32_t n_present;
  int32_t learner[kMaxLearners];
  double w_hat[kMaxLearners];
  double lr;
  double beta;
  // Radial-Directional Averaging (all null for the weighted mean):
  const double* norm2;      // [n_learners][rows] squared norms of the dequantized pseudo-gradients
  double* dir_part;         // [slot] per-block sums of the squared averaged direction
  double* coef;             // [row][n_present] coefficient of each learner's codebook in g
};

struct BroadcastArgs {
  const float* theta_g;
  float* theta_L;
  int64_t stride;
  int32_t n_rows;                 // learner rows written
  int32_t row[kMaxLearners];      // their learner indices
};

// The ring with requantization at every hop: each rank's running sum of a chunk
// it received is kept negated (accum = -sum), so that quantizing with no base
// (Delta = fl32(0 - accum)) quantizes the sum itself.
struct RingArgs {
  const float* theta_g;
  const float* theta_L;
  int64_t stride;           // learner row length (elements); accum and codes rows likewise
  int32_t n_ranks;
  float* accum;             // [n_ranks][stride] negated running sums
  const uint8_t* codes;     // [n_ranks][stride] messages
  const float* codebook;    // [segment][256] message codebooks
  float divisor;            // 0: none; else the sum is divided by it after the add (fp32)
  double2* part_stats;      // [slot] {sum(d), sum(d^2)} of the new sums, d = sum - shift: the next
                            // message's statistics partials, in the statistics partition of the segments
  int32_t cb_row[kMaxTensorsPerLaunch];  // codebook row of the message each segment of the launch receives
};

// Kernel launchers (dlc_kernels.hip).  Each returns hipSuccess or the launch error.
hipError_t launch_stats(const QuantArgs& a, const LaunchGeom& g, hipStream_t s);
hipError_t launch_range(const QuantArgs& a, const LaunchGeom& g, hipStream_t s);
// *p = v, one device word written by a kernel (capturable, unlike a memset).
hipError_t launch_fill_u32(uint32_t* p, uint32_t v, hipStream_t s);
hipError_t launch_encode(const QuantArgs& a, const LaunchGeom& g, hipStream_t s);
// histogram slices, then the codebook (one kernel when every tensor has one slice)
hipError_t launch_codebook(const QuantArgs& a, const LaunchGeom& g, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, const LaunchGeom& g, hipStream_t s);
// Radial-Directional Averaging: the squared norm of the averaged direction per
// block, then each tensor's learner coefficients (which k_merge then uses)
hipError_t launch_rda_direction(const MergeArgs& a, const LaunchGeom& g, hipStream_t s);
hipError_t launch_rda_coef(const MergeArgs& a, const LaunchGeom& g, hipStream_t s);
hipError_t launch_broadcast(const BroadcastArgs& a, const LaunchGeom& g, hipStream_t s);
// segments: (offset of the chunk in theta_g, the receiver's offset in the flat theta_L / accum,
// numel); the sender's codes sit one rank row earlier, cyclically; the launch geometry must be the
// statistics partition of these segments (the partials land in its slots)
hipError_t launch_dequant_add(const RingArgs& a, const LaunchGeom& g, hipStream_t s);

}  // namespace dlc
