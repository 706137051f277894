// gfx950 kernels of the DiLoCo outer-step merge.
//
// Three streaming passes over HBM per outer step, plus two small finalizers:
//   k_stats     per-(learner, tensor) partial sum(d), sum(d^2) of d = Delta - shift, fp64
//   k_range     per-(learner, tensor) mu, sigma -> {lo, hi, wd, mean} (fp64 -> fp32)
//   k_encode    Delta -> clip -> bucket -> uint8 code (256-byte runs per wave store) + LDS histogram
//               of (count, fixed-point position sum) per bucket and learner
//   k_hist_reduce, k_codebook
//               per-(learner, tensor, bucket) mean of the clipped values -> fp32, from the
//               block histograms summed in slices (one kernel when a tensor has one slice)
//   k_merge     dequantize K learners through fp64 LDS tables w_hat_i * codebook_i,
//               sum, Nesterov update of theta and momentum, every byte read once
//
// and for the calls around that path:
//   k_broadcast     the updated theta copied into every learner row (sending back)
//   k_merge<NR, true>, k_rda_coef
//                   Radial-Directional Averaging: the squared norm of the averaged
//                   direction per block, then per-(tensor, learner) coefficients
//   k_dequant_add   one hop of the ring that requantizes at every hop: the receiver
//                   adds the dequantized message to its pseudo-gradient and forms the
//                   statistics partials of its next message
//
// The quantizer follows the INTELLECT-1 reading notes, section 4.1 (per-tensor mu
// and sigma, clip at 6 sigma, 256 equal buckets, codebook of bucket means); the
// merge follows section 3.2 steps 6-7 and section 4.2 (dequantize, accumulate in
// floating point, Nesterov with lr 0.7 / momentum 0.9); the ring, section 3.2 step
// 6 and section 4.2 (a quantized message before every send).  Sending back and
// Radial-Directional Averaging follow the Decoupled DiLoCo digest, "architecture".
//
// Memory layout of a tile: kTile = 4096 elements of one tensor; wave w of the block
// owns elements [1024 w, 1024 w + 1024) and each load instruction of a wave reads
// 1 KB of consecutive bytes.  Streaming reads and writes are non-temporal (each
// byte is touched once per pass and the working set is far larger than the caches).
// The next learner's tile is loaded while the current one is processed.
//
// Floating point contraction is off for this file: every operation that has to
// match the fp32/fp64 definition bit for bit is written as separate IEEE
// operations.  The only fused multiply-adds are explicit ones whose rounding is
// part of their argument: the sum(d^2) accumulation, the bucket index estimate
// (checked against the exact division near bucket edges) and the fixed-point
// histogram position.
#include "dlc_internal.h"

#include <cfloat>
#include <type_traits>

namespace dlc {
namespace {

typedef float vf4 __attribute__((ext_vector_type(4)));
typedef unsigned int vu4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = kBlock / 64;
constexpr int kHistBytes = kBuckets * 8;  // one copy of a learner's 256 packed 64-bit bucket accumulators

struct Span {
  int t;          // tensor index within the launch
  int64_t begin;  // first element of this block within the tensor
  int64_t end;    // one past the last element of this block
};

// Block -> (tensor, element span).  The launch geometry lives in the kernel
// arguments; the search index is uniform across the block (scalar loads).
__device__ __forceinline__ Span block_span(const LaunchGeom& g) {
  const int b = blockIdx.x;
  int lo = 0, hi = g.n_tensors - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (g.t[mid].block_first <= b) lo = mid; else hi = mid - 1;
  }
  Span s;
  s.t = lo;
  const int64_t per_block = (int64_t)g.tiles_per_block * kTile;
  s.begin = (int64_t)(b - g.t[lo].block_first) * per_block;
  const int64_t e = s.begin + per_block;
  s.end = e < g.t[lo].numel() ? e : g.t[lo].numel();
  return s;
}

__device__ __forceinline__ int tensor_block_end(const LaunchGeom& g, int t) {
  return t + 1 < g.n_tensors ? g.t[t + 1].block_first : g.n_blocks;
}

// Thread -> element mapping inside a tile: wave w owns the contiguous elements
// [1024 w, 1024 w + 1024); lane L of that wave holds float4 number 64 j + L of
// the chunk for j = 0..3.  Every load instruction of a wave reads 1 KB of
// consecutive bytes, and the wave's 1024 one-byte codes form one contiguous 1 KB
// block.
__device__ __forceinline__ int f4_index(int tid, int j) { return (tid & ~63) * 4 + j * 64 + (tid & 63); }

// 16 floats of a full tile through a buffer descriptor covering just that tile
// (non-temporal).  A descriptor with zero records makes every load return zeros
// without touching memory: a "null" request that still counts as a memory
// instruction, so ring slots without data keep the wait counts static.
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const float* p, bool valid) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), (short)0, valid ? kTile * 4 : 0, kBufferWord3);
}

__device__ __forceinline__ void load_tile_rsrc(__amdgpu_buffer_rsrc_t r, int tid, float (&v)[kVec]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const vf4 x = __builtin_bit_cast(vf4, __builtin_amdgcn_raw_buffer_load_b128(r, f4_index(tid, j) * 16, 0, 2));
    v[4 * j + 0] = x.x;
    v[4 * j + 1] = x.y;
    v[4 * j + 2] = x.z;
    v[4 * j + 3] = x.w;
  }
}

__device__ __forceinline__ int64_t elem_index(int tid, int j, int c) { return 4 * (int64_t)f4_index(tid, j) + c; }

__device__ __forceinline__ bool tail_valid(int tid, int j, int c, int64_t n) { return elem_index(tid, j, c) < n; }

// 16 floats of a tail tile: element e valid iff its index is below n.
__device__ __forceinline__ void load_tail(const float* __restrict__ p, int tid, int64_t n,
                                          float (&v)[kVec]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v[4 * j + c] = tail_valid(tid, j, c, n) ? p[elem_index(tid, j, c)] : 0.0f;
    }
  }
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ const float* learner_row(const QuantArgs& a, int k, const TensorDesc& td) {
  return a.theta_L + (int64_t)a.learner[a.k_base + k] * a.stride + td.loffset();
}

// ---------------------------------------------------------------------------
// k_stats: partial moments about a per-(learner, tensor) shift.
//
// shift = Delta at the tensor's first element, so sum(d) and sum(d^2) stay small
// and var = sum(d^2)/n - (sum(d)/n)^2 loses nothing in fp64.  Each block covers
// one tensor; its per-learner partial sums go to workspace slot slot_base + block.
// Accumulators live in registers (KC learners, unrolled).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void stats_accumulate(const float (&gv)[kVec], const float (&lv)[kVec],
                                                 double shift, double& s1, double& s2) {
#pragma unroll
  for (int e = 0; e < kVec; ++e) {
    const double d = (double)(gv[e] - lv[e]) - shift;
    s1 += d;
    s2 = __fma_rn(d, d, s2);
  }
}

// Tiles stream through a ring of kStatsRing register buffers.  A tile is KC + 1
// items: theta_g first, then learners 0..KC-1; item i + kStatsRing - 1 is
// requested while item i is accumulated.  KC + 1 is a multiple of the ring size,
// so ring slots are compile-time constants across tiles.  A learner item beyond
// k_count, and the look-ahead past the block's last tile, are null requests
// (zero-record buffer descriptor: no memory traffic); they are not accumulated.
// Every request is the same unconditional load through a selected descriptor, so
// the compiler's wait counts stay exact.
constexpr int kStatsRing = 3;

template <int KC>
__global__ __launch_bounds__(kBlock) void k_stats(const QuantArgs a, const LaunchGeom g) {
  static_assert((KC + 1) % kStatsRing == 0, "KC + 1 must be a multiple of the ring size");
  constexpr int kItems = KC + 1;
  const int tid = threadIdx.x;
  const Span sp = block_span(g);
  const TensorDesc td = g.t[sp.t];
  // No base (theta_g NULL): Delta = fl32(0 - theta_L); the base loads become null
  // requests that return zeros without memory traffic.
  const bool has_base = a.theta_g != nullptr;
  const float* __restrict__ tg = has_base ? a.theta_g + td.offset() : learner_row(a, 0, td);
  const int kc = a.k_count;

  float shift[KC];  // Delta at element 0: an fp32 value, widened where used
  double s1[KC], s2[KC];
  const float g0 = has_base ? tg[0] : 0.0f;
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    const float* row = learner_row(a, k < kc ? k : kc - 1, td);
    shift[k] = g0 - row[0];
    s1[k] = 0.0;
    s2[k] = 0.0;
  }

  const int64_t n_full = (sp.end - sp.begin) / kTile;
  if (n_full > 0) {
    const int64_t last = sp.begin + (n_full - 1) * kTile;
    auto request = [&](int item, int64_t base, float (&dst)[kVec], bool live = true) {
      const bool real = live && (item == 0 ? has_base : item <= kc);
      const float* src = (item == 0 || item > kc) ? tg : learner_row(a, item - 1, td);
      load_tile_rsrc(tile_rsrc(src + base, real), tid, dst);
    };
    float gv[kVec], ring[kStatsRing][kVec];
#pragma unroll
    for (int i = 0; i < kStatsRing - 1; ++i) request(i, sp.begin, ring[i]);
    for (int64_t base = sp.begin; base <= last; base += kTile) {
      const int64_t nbase = base < last ? base + kTile : last;
#pragma unroll
      for (int i = 0; i < kItems; ++i) {
        const int ip = i + kStatsRing - 1;
        if (ip < kItems) {
          request(ip, base, ring[ip % kStatsRing]);
        } else {
          request(ip - kItems, nbase, ring[ip % kStatsRing], base < last);
        }
        if (i == 0) {
#pragma unroll
          for (int e = 0; e < kVec; ++e) gv[e] = ring[0][e];
        } else if (i - 1 < kc) {
          stats_accumulate(gv, ring[i % kStatsRing], (double)shift[i - 1], s1[i - 1], s2[i - 1]);
        }
      }
    }
  }
  const int64_t full_end = sp.begin + n_full * kTile;
  if (full_end < sp.end) {
    const int64_t n = sp.end - full_end;
    float gv[kVec];
    load_tail(tg + full_end, tid, has_base ? n : 0, gv);
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      if (k < kc) {
        float lv[kVec];
        load_tail(learner_row(a, k, td) + full_end, tid, n, lv);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            if (tail_valid(tid, j, c, n)) {
              const int e = 4 * j + c;
              const double d = (double)(gv[e] - lv[e]) - (double)shift[k];
              s1[k] += d;
              s2[k] = __fma_rn(d, d, s2[k]);
            }
          }
        }
      }
    }
  }

  __shared__ double red[2][KC][kWaves];
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    const double r1 = wave_sum(s1[k]);
    const double r2 = wave_sum(s2[k]);
    if (lane == 0) {
      red[0][k][wave] = r1;
      red[1][k][wave] = r2;
    }
  }
  __syncthreads();
  if (tid < kc) {
    double r1 = 0.0, r2 = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      r1 += red[0][tid][w];
      r2 += red[1][tid][w];
    }
    const size_t slot = (size_t)(g.slot_base + blockIdx.x);
    a.part_stats[slot * a.n_present + a.k_base + tid] = make_double2(r1, r2);
  }
}

// ---------------------------------------------------------------------------
// k_range: one block per (present learner, tensor of the launch).  Thread j sums
// the tensor's block partials j, j + kRangeThreads, ... in that order, then a
// fixed pairwise tree combines the threads: deterministic for a given partition.
// ---------------------------------------------------------------------------
constexpr int kRangeThreads = 256;

__global__ __launch_bounds__(kRangeThreads) void k_range(const QuantArgs a, const LaunchGeom g) {
  __shared__ double r1[kRangeThreads], r2[kRangeThreads];
  const int k = blockIdx.x / g.n_tensors;
  const int t = blockIdx.x - k * g.n_tensors;
  const int j = threadIdx.x;
  const TensorDesc td = g.t[t];
  const int b0 = td.block_first, nb = tensor_block_end(g, t) - b0;
  const double2* p = a.part_stats + (size_t)(g.slot_base + b0) * a.n_present + k;
  double S1 = 0.0, S2 = 0.0;
  for (int b = j; b < nb; b += kRangeThreads) {
    const double2 v = p[(size_t)b * a.n_present];
    S1 += v.x;
    S2 += v.y;
  }
  r1[j] = S1;
  r2[j] = S2;
  __syncthreads();
#pragma unroll
  for (int h = kRangeThreads / 2; h > 0; h >>= 1) {
    if (j < h) {
      r1[j] += r1[j + h];
      r2[j] += r2[j + h];
    }
    __syncthreads();
  }
  if (j != 0) return;
  S1 = r1[0];
  S2 = r2[0];
  const int li = a.learner[k];
  // A NaN or an infinity among the pseudo-gradients makes a sum non-finite (finite
  // fp32 values cannot overflow an fp64 sum of squares of up to 2^32 terms).
  if (a.status != nullptr && !(__builtin_isfinite(S1) && __builtin_isfinite(S2)))
    atomicMin(a.status, (uint32_t)((size_t)li * g.n_tensors_call + g.row_base + g.t_base + t));
  const float g0 = a.theta_g != nullptr ? a.theta_g[td.offset()] : 0.0f;
  const float l0 = a.theta_L[(int64_t)li * a.stride + td.loffset()];
  const double shift = (double)(g0 - l0);
  const double n = (double)td.numel();
  const double m1 = S1 / n;
  const double mu = shift + m1;
  double var = S2 / n - m1 * m1;
  if (!(var > 0.0)) var = 0.0;
  const double sigma = sqrt(var);
  float4 r;
  r.x = (float)(mu - 6.0 * sigma);
  r.y = (float)(mu + 6.0 * sigma);
  r.z = (float)(12.0 * sigma / 256.0);
  r.w = (float)mu;
  a.range[(size_t)li * g.n_tensors_call + g.row_base + g.t_base + t] = r;
}

// ---------------------------------------------------------------------------
// k_encode: codes + per-block LDS histogram for up to kLearnerChunk learners.
//
// Bucket index.  The definition is c = clip(floor(fl32(fl32(x - lo) / wd)), 0, 255).
// With t = fl32(x - lo), r = fl32(1 / wd) and q' = fl32(t * r + 2^-14) (one fused
// multiply-add), both q' - 2^-14 and the correctly rounded quotient q = fl32(t / wd)
// lie within about 2^-24 |t / wd| of the exact t / wd, so |q' - 2^-14 - q| <=
// 3 * 2^-24 * |t / wd|, below 2^-14 wherever the result is not clamped (|t / wd| <
// 257).  Hence q lies in (q' - 2^-13, q'], and floor(q') = floor(q) whenever
// fract(q') >= 2^-13.  Only the elements with fract(q') < 2^-13 (about 1 in 8000)
// take the exact IEEE division; a wave redoes one element slot only when some lane
// needs it there.
//
// Histogram: one 64-bit LDS atomic per element adds the count unit and the
// element's position inside its bucket as a fixed-point integer, see
// EncodePar.  Integer sums make the histogram exact and independent of the order
// of the atomics.  Codes of a full tile are packed 4 per dword in the load layout
// and stored as they are: each of a wave's four dword store instructions writes 256
// consecutive bytes (whole cache lines), together the wave's 1 KB of codes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float uniform_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

__device__ __forceinline__ double uniform_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Fraction bits s and bias of the packed bucket-position sums for one (learner,
// tensor).  An element of bucket c contributes its position inside the bucket,
// q = round((x_c - lo) * 2^s / wd) - c * 2^s, plus the bias (see EncodePar).  In
// bucket widths, with e = (hi - lo) / wd - 255:
//   * an element in [lo, hi] that the fp32 index puts in bucket c < 255 sits in
//     [-2^-14, 1 + 2^-14] (the index misplaces x by at most 3 * 2^-24 * 257 widths);
//   * bucket 255 also holds the values clipped to hi: up to max(1, e);
//   * an element above hi is clipped to hi but coded from its own value, so it can
//     land in any bucket from floor((hi - lo) / wd) to 255.  Normally (hi - lo) / wd
//     is about 256 and that is bucket 255 at a position >= 0; but when lo and hi
//     round to fp32 steps coarser than wd (|mu| many orders above sigma, up to
//     lo == hi) it is a bucket above hi's, at a position down to e < 0.
// So q lies in [min(0, e) * 2^s - 2^12, max(1, e) * 2^s + 2^12] (plus 1 for the
// roundings).  The bias lifts the lowest position to >= 0:
//   bias = kHistBias + ceil(max(0, -e) * 2^s)
// and s is the largest value <= kHistFracBits that keeps the highest, q + bias,
// below 2^27: (max(1, e) + max(0, -e)) * 2^s + 2 * kHistBias < 2^27 (normally 26).
// Such an s exists for every tensor whose clip bounds are finite: a non-constant
// fp32 tensor of n <= 2^32 elements has sigma >= ulp(mu) / sqrt(n), so
// (hi - lo) / wd <= 256 + 21 * 2^-23 * |mu| / sigma + 1 < 1.5e6 (a constant tensor,
// or one whose wd underflows, takes the zero-variance path).  Infinite bounds
// (|mu| + 6 sigma beyond the fp32 range) are outside the contract, as for the
// statistics.
struct HistFormat {
  int s;
  double bias;  // an integer
};

__device__ __forceinline__ HistFormat hist_format(float lo, float hi, float wd) {
  const double ext = ((double)hi - (double)lo) / (double)wd - 255.0;
  const double top = ext > 1.0 ? ext : 1.0;
  const double neg = ext < 0.0 ? -ext : 0.0;
  int s = kHistFracBits;
  while (s > 0 && (top + neg) * (double)(1ll << s) + 2.0 * kHistBias >= (double)(1ll << 27)) --s;
  HistFormat f;
  f.s = s;
  f.bias = (double)kHistBias + __builtin_ceil(neg * (double)(1ll << s));
  return f;
}

// Fixed-point bucket positions without integer conversions.  With scale = 2^s / wd,
// B = -lo * scale and B_i = rint(B), the element's addend is the bit pattern of
//   y = fl64(fl64(x_c * scale + (2^52 + 2^44 + B_i + bias)) - c * 2^s)
// The first fused multiply-add rounds to an integer (the spacing of doubles in
// [2^52, 2^53) is 1), so y = 2^52 + 2^44 + v with v = rint(x_c * scale) + B_i -
// c * 2^s + bias in [0, 2^27) (HistFormat); the second is exact.  Its bits are
// kPosUnit * 2^44 + v: the low 44 bits carry v, the top 20 bits the odd constant
// kPosUnit, so a sum of N addends holds N * kPosUnit mod 2^20 on top (N < 2^20
// per block, recovered with the inverse kPosUnitInv) and the sum of v below.
// The exact position (x_c - lo) * scale - c * 2^s is v - bias + (B - B_i)
// within 1/2: the codebook subtracts the bias and adds the constant B - B_i back.
constexpr double kPosMagic = 0x1p52 + 0x1p44;
constexpr uint64_t kPosUnit = 0x43301;  // top 20 bits of every addend
constexpr uint64_t kPosUnitInv = 0x4cd01;  // kPosUnit * kPosUnitInv = 1 mod 2^20
static_assert((kPosUnit * kPosUnitInv & 0xFFFFF) == 1, "count unit inverse");
static_assert(kHistCountShift == 44, "addend layout");

// Per-learner encode parameters, staged in LDS once per block.
struct EncodePar {
  float lo, hi, wd, rcp;  // clip range, bucket width, fl32(1 / wd)
  double scale;           // 2^s / wd
  double magic;           // 2^52 + 2^44 + rint(-lo * scale) + bias
  double neg_two_s;       // -2^s
  double origin_frac;     // -lo * scale - rint(-lo * scale)
  double bias;            // HistFormat::bias
};

__device__ __forceinline__ EncodePar make_encode_par(float4 r) {
  EncodePar p;
  p.lo = r.x;
  p.hi = r.y;
  p.wd = r.z;
  p.rcp = 0.0f;
  p.scale = p.magic = p.neg_two_s = p.origin_frac = p.bias = 0.0;
  if (r.z >= FLT_MIN) {
    p.rcp = 1.0f / r.z;
    const HistFormat f = hist_format(r.x, r.y, r.z);
    const double two_s = (double)(1ll << f.s);
    p.scale = two_s / (double)r.z;
    const double b = -(double)r.x * p.scale;
    const double bi = __builtin_rint(b);
    p.magic = kPosMagic + (bi + f.bias);
    p.neg_two_s = -two_s;
    p.origin_frac = b - bi;
    p.bias = f.bias;
  }
  return p;
}

// Codes of one (learner, tile) item, packed 4 per dword in the load layout
// (dword j of a lane holds the codes of float4 number f4_index(tid, j)), and the
// item's histogram atomics.  FULL = every element of the tile is valid; otherwise
// element e is valid iff its index is below n.
template <bool FULL, int R>
__device__ __forceinline__ void encode_codes(uint64_t* __restrict__ hist, const float (&gv)[kVec],
                                             const float (&lv)[kVec], const EncodePar& par_lds, int tid,
                                             int64_t n, uint32_t (&packed)[4]) {
  static_assert((R & (R - 1)) == 0, "copies must be a power of two");
  // The parameters are the same for every lane: keep them in scalar registers.
  const float lo = uniform_f32(par_lds.lo), hi = uniform_f32(par_lds.hi), wd = uniform_f32(par_lds.wd);
  const float rcp = uniform_f32(par_lds.rcp);
  const double scale = uniform_f64(par_lds.scale), magic = uniform_f64(par_lds.magic);
  const double neg_two_s = uniform_f64(par_lds.neg_two_s);
#pragma unroll
  for (int j = 0; j < 4; ++j) packed[j] = 0u;
  if (!(wd >= FLT_MIN)) return;  // zero variance: every code is 0 and no histogram is needed
  constexpr float kShift = 0x1p-14f, kNearWin = 0x1p-13f;
  float x[kVec], qs[kVec];
  bool near_any = false;
#pragma unroll
  for (int e = 0; e < kVec; ++e) {
    x[e] = gv[e] - lv[e];
    qs[e] = __builtin_fmaf(x[e] - lo, rcp, kShift);
    near_any |= __builtin_amdgcn_fractf(qs[e]) < kNearWin;
  }
  // Rare: some lane holds an element within 2^-14 of a bucket edge.
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(near_any) != 0, 0)) {
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      const bool near = __builtin_amdgcn_fractf(qs[e]) < kNearWin;
      if (__builtin_amdgcn_ballot_w64(near) != 0) {
        const float exact = floorf((x[e] - lo) / wd);
        qs[e] = near ? exact : qs[e];
      }
    }
  }
  // this lane's copy of the histogram, as a byte address
  char* const hl = reinterpret_cast<char*>(hist) + 8 * (tid & (R - 1));
  constexpr int kShiftR = 3 + (R == 1 ? 0 : R == 2 ? 1 : R == 4 ? 2 : 3);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t w = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = 4 * j + c;
      const uint32_t code = (uint32_t)__builtin_amdgcn_fmed3f(qs[e], 0.0f, 255.0f);
      if (FULL || tail_valid(tid, j, c, n)) {
        const double xc = (double)__builtin_amdgcn_fmed3f(x[e], lo, hi);
        const double y = __fma_rn((double)code, neg_two_s, __fma_rn(xc, scale, magic));
        atomicAdd(reinterpret_cast<unsigned long long*>(hl + (code << kShiftR)),
                  __builtin_bit_cast(unsigned long long, y));
      }
      w |= code << (8 * c);
    }
    packed[j] = w;
  }
}

// Codes of a full tile through a buffer descriptor covering the tile's 4096 bytes
// (zero records when !valid: the stores are dropped).  Dword j of every lane of a
// wave covers 256 consecutive bytes, so each non-temporal store writes whole
// cache lines.
__device__ __forceinline__ void store_codes(uint8_t* cp, bool valid, int tid, const uint32_t (&packed)[4]) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(cp, (short)0, valid ? kTile : 0, kBufferWord3);
#pragma unroll
  for (int j = 0; j < 4; ++j) __builtin_amdgcn_raw_buffer_store_b32(packed[j], r, f4_index(tid, j) * 4, 0, 2);
}

// Order of work.  A tensor's full tiles form groups of kGroup consecutive tiles,
// dealt to the tensor's blocks in turn (block j of nb takes groups j, j + nb, ...),
// so blocks that run at the same time stream neighbouring parts of every buffer.
// For each group, theta_g's kGroup tiles are held in registers while every
// learner is encoded against them, one learner at a time; a learner's codes of the
// whole group (kGroup * 4 KB, contiguous) leave in one burst of stores once its
// last tile is done.  Long runs of consecutive bytes per block and learner keep
// the HBM write stream efficient next to the much larger read stream.
// Learner tiles stream through a ring of kGroup register buffers: the tile three
// items ahead is requested before a tile is encoded, across learner and group
// boundaries.  theta_g's tile u of the next group is requested into its own
// registers as soon as the group's last learner has encoded tile u.  A request for
// a tile beyond the tensor's full tiles (a partial last group) or past the block's
// last group is a null request: no memory traffic, and the tile is skipped.  The
// tensor's partial last tile, if any, is encoded by its last block.  Every load
// and store is unconditional, so the compiler's wait counts stay exact.
// Per-learner {lo, hi, wd, 1/wd, fixed-point constants} are staged in LDS once
// per block.
constexpr int kGroup = kEncodeGroupTiles;

template <int R>
__global__ __launch_bounds__(kBlock) void k_encode(const QuantArgs a, const LaunchGeom g) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int kc = a.k_count;
  uint64_t* hist = reinterpret_cast<uint64_t*>(smem);
  EncodePar* par = reinterpret_cast<EncodePar*>(smem + kc * R * kHistBytes);
  const int tid = threadIdx.x;

  // Block -> (tensor t, rank j among the tensor's nb blocks).  Block j encodes the
  // tensor's groups j, j + nb, j + 2 nb, ...: blocks that run at the same time
  // work on neighbouring groups.
  const Span sp = block_span(g);
  const int t = sp.t;
  const TensorDesc td = g.t[t];
  const int j = blockIdx.x - td.block_first;
  const int nb = tensor_block_end(g, t) - td.block_first;
  const size_t rrow = (size_t)g.row_base + g.t_base + t;
  for (int i = tid; i < kc * R * kBuckets; i += kBlock) hist[i] = 0;
  if (tid < kc) par[tid] = make_encode_par(a.range[(size_t)a.learner[a.k_base + tid] * g.n_tensors_call + rrow]);
  __syncthreads();

  const bool has_base = a.theta_g != nullptr;  // NULL: Delta = fl32(0 - theta_L), base tiles are zeros
  const float* __restrict__ tg = has_base ? a.theta_g + td.offset() : learner_row(a, 0, td);
  auto codes_of = [&](int k) {
    return a.codes + (int64_t)a.learner[a.k_base + k] * a.stride + td.loffset();
  };

  const int64_t n_full = td.numel() / kTile;  // full tiles of the tensor
  const int64_t groups_total = (n_full + kGroup - 1) / kGroup;
  const int64_t n_groups = groups_total > j ? (groups_total - j + nb - 1) / nb : 0;  // this block's groups
  if (n_groups > 0) {
    // tile u of this block's group gi of stream s (0 = theta_g, s >= 1 = learner s - 1)
    auto request = [&](float (&dst)[kVec], int64_t gi, int s, int u) {
      const int64_t tile = (j + gi * nb) * kGroup + u;
      const bool valid = gi < n_groups && tile < n_full && (s != 0 || has_base);
      const float* base = s == 0 ? tg : learner_row(a, s - 1, td);
      load_tile_rsrc(tile_rsrc(base + (valid ? tile : 0) * kTile, valid), tid, dst);
    };
    float gv[kGroup][kVec], ring[kGroup][kVec];
#pragma unroll
    for (int u = 0; u < kGroup; ++u) request(gv[u], 0, 0, u);
#pragma unroll
    for (int u = 0; u < kGroup - 1; ++u) request(ring[u], 0, 1, u);
    {
      const uint32_t zero[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int u = 0; u < kGroup; ++u) store_codes(codes_of(0), false, tid, zero);
    }
    __builtin_amdgcn_sched_barrier(0);
    for (int64_t gi = 0; gi < n_groups; ++gi) {
      const int64_t grp = j + gi * nb;
      const int64_t left = n_full - grp * kGroup;
      const int valid = left < kGroup ? (int)left : kGroup;
      auto pass = [&](int k, auto last_tag) {
        constexpr bool kLast = decltype(last_tag)::value;
        uint32_t cw[kGroup][4];
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
          if (u == 0) request(ring[kGroup - 1], gi, k + 1, kGroup - 1);
          else if (kLast) request(ring[u - 1], gi + 1, 1, u - 1);
          else request(ring[u - 1], gi, k + 2, u - 1);
          if (u < valid) {
            encode_codes<true, R>(hist + k * R * kBuckets, gv[u], ring[u], par[k], tid, kTile, cw[u]);
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) cw[u][q] = 0u;
          }
          if (kLast) request(gv[u], gi + 1, 0, u);
        }
        uint8_t* cp = codes_of(k) + grp * kGroup * kTile;
#pragma unroll
        for (int u = 0; u < kGroup; ++u) store_codes(cp + u * kTile, u < valid, tid, cw[u]);
      };
      for (int k = 0; k < kc - 1; ++k) pass(k, std::false_type{});
      pass(kc - 1, std::true_type{});
    }
  }
  // The partial last tile of the tensor, if any, belongs to the tensor's last block.
  const int64_t full_len = n_full * kTile;
  if (j == nb - 1 && full_len < td.numel()) {
    const int64_t n = td.numel() - full_len;
    float gv[kVec];
    load_tail(tg + full_len, tid, has_base ? n : 0, gv);
    for (int k = 0; k < kc; ++k) {
      float lv[kVec];
      load_tail(learner_row(a, k, td) + full_len, tid, n, lv);
      uint32_t cw[4];
      encode_codes<false, R>(hist + k * R * kBuckets, gv, lv, par[k], tid, n, cw);
      uint8_t* cp = codes_of(k) + full_len;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (tail_valid(tid, q, c, n)) cp[elem_index(tid, q, c)] = (uint8_t)(cw[q] >> (8 * c));
        }
      }
    }
  }

  __syncthreads();
  const size_t slot = (size_t)(g.slot_base + blockIdx.x);
  uint64_t* dst = a.part_hist + (slot * a.n_present + a.k_base) * kBuckets;
  for (int i = tid; i < kc * kBuckets; i += kBlock) {
    uint64_t v = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) v += hist[i * R + r];
    // count = (N * kPosUnit mod 2^20) * kPosUnitInv mod 2^20; positions stay below
    const uint64_t count = ((v >> kHistCountShift) * kPosUnitInv) & ((1ull << (64 - kHistCountShift)) - 1);
    dst[i] = (count << kHistCountShift) | (v & ((1ull << kHistCountShift) - 1));
  }
}

// ---------------------------------------------------------------------------
// The codebook stage, in two kernels.  k_hist_reduce: one block per (histogram
// slice, present learner, tensor): 4 groups of 256 threads (one per bucket) sum
// every fourth block histogram of the slice's kHistSlice blocks, unpacked to
// (position sum, count), combine in LDS and write one slice entry.  k_codebook:
// one block of 256 threads per (present learner, tensor) sums the tensor's slice
// entries and forms
//   cb[c] = fl32(lo + wd * (c + (Q / n + f) / 2^s))
// with n the bucket count, Q the sum of the element positions (bias removed) and
// f the origin fraction of EncodePar; an empty bucket holds its midpoint
// fl32(lo + (c + 1/2) wd).  Every sum is an integer sum, so the order does not
// matter.
// Slice entry of slice s of tensor t: floor(first global slot / kHistSlice) +
// global tensor index + s.  Distinct tensors never share an entry, and a call
// needs at most slots / kHistSlice + tensors + 2 entries.
// ---------------------------------------------------------------------------
constexpr int kCodebookGroups = 4;

__device__ __forceinline__ size_t hist_entry(const LaunchGeom& g, int t, int s) {
  return (size_t)((g.slot_base + g.t[t].block_first) / kHistSlice) + (size_t)(g.t_base + t) + (size_t)s;
}

__device__ __forceinline__ size_t codebook_row(const QuantArgs& a, const LaunchGeom& g, int k, int t) {
  return (size_t)a.learner[k] * g.n_tensors_call + g.row_base + g.t_base + t;
}

// Codebook entry c of (present learner k, tensor t) from its bucket totals.
// Returns bucket c's share of the squared norm of the dequantized tensor,
// count_c * entry_c^2 in fp64 (a zero-variance tensor codes every element as 0).
__device__ __forceinline__ double write_codebook(const QuantArgs& a, const LaunchGeom& g, int k, int t, int c,
                                                 uint64_t Qb, uint64_t N) {
  const size_t row = codebook_row(a, g, k, t);
  const float4 r = a.range[row];
  float out;
  if (!(r.z >= FLT_MIN)) {
    out = r.w;
    N = c == 0 ? (uint64_t)g.t[t].numel() : 0;
  } else if (N > 0) {
    const EncodePar par = make_encode_par(r);
    const int64_t Q = (int64_t)(Qb - N * (uint64_t)par.bias);
    const double frac = ((double)Q / (double)N + par.origin_frac) / -par.neg_two_s;
    out = (float)((double)r.x + (double)r.z * ((double)c + frac));
  } else {
    out = (float)((double)r.x + ((double)c + 0.5) * (double)r.z);
  }
  a.codebook[row * kBuckets + c] = out;
  return (double)N * ((double)out * (double)out);
}

// Sum of one value from each of the first kBuckets threads, in a fixed pairwise
// tree (the same order every run).  Every thread of the block calls it.
__device__ __forceinline__ double bucket_tree_sum(double v, double* s) {
  const int c = threadIdx.x;
  if (c < kBuckets) s[c] = v;
  __syncthreads();
  for (int w = kBuckets / 2; w > 0; w >>= 1) {
    if (c < w) s[c] += s[c + w];
    __syncthreads();
  }
  return s[0];
}

// FINAL: every tensor of the launch has a single slice; write the codebook
// directly instead of a slice entry.
template <bool FINAL>
__global__ __launch_bounds__(kBuckets * kCodebookGroups) void k_hist_reduce(const QuantArgs a, const LaunchGeom g) {
  __shared__ uint64_t sq[kCodebookGroups][kBuckets];
  __shared__ uint64_t sn[kCodebookGroups][kBuckets];
  const int sl = blockIdx.x;
  const int k = blockIdx.y / g.n_tensors;
  const int t = blockIdx.y - k * g.n_tensors;
  const int b0 = g.t[t].block_first, nb = tensor_block_end(g, t) - b0;
  const int first = sl * kHistSlice;
  if (first >= nb) return;
  const int count = nb - first < kHistSlice ? nb - first : kHistSlice;
  const int c = threadIdx.x & (kBuckets - 1);
  const int grp = threadIdx.x >> 8;
  const size_t step = (size_t)a.n_present * kBuckets;
  const uint64_t* p = a.part_hist + ((size_t)(g.slot_base + b0 + first) * a.n_present + k) * kBuckets + c;
  uint64_t Q = 0, N = 0;
  constexpr uint64_t kSumMask = (1ull << kHistCountShift) - 1;
  int b = grp;
  for (; b + 3 * kCodebookGroups < count; b += 4 * kCodebookGroups) {
    uint64_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = p[(size_t)(b + u * kCodebookGroups) * step];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      N += v[u] >> kHistCountShift;
      Q += v[u] & kSumMask;
    }
  }
  for (; b < count; b += kCodebookGroups) {
    const uint64_t v = p[(size_t)b * step];
    N += v >> kHistCountShift;
    Q += v & kSumMask;
  }
  sq[grp][c] = Q;
  sn[grp][c] = N;
  __syncthreads();
  double term = 0.0;
  if (grp == 0) {
    for (int u = 1; u < kCodebookGroups; ++u) {
      Q += sq[u][c];
      N += sn[u][c];
    }
    if (FINAL) {
      term = write_codebook(a, g, k, t, c, Q, N);
    } else {
      uint64_t* e = a.hist_sum + ((hist_entry(g, t, sl) * a.n_present + k) * kBuckets + c) * 2;
      e[0] = Q;
      e[1] = N;
    }
  }
  if (FINAL && a.norm2 != nullptr) {
    __shared__ double st[kBuckets];
    const double n2 = bucket_tree_sum(term, st);
    if (threadIdx.x == 0) a.norm2[codebook_row(a, g, k, t)] = n2;
  }
}

__global__ __launch_bounds__(kBuckets) void k_codebook(const QuantArgs a, const LaunchGeom g) {
  const int k = blockIdx.x / g.n_tensors;
  const int t = blockIdx.x - k * g.n_tensors;
  const int c = threadIdx.x;
  const int nb = tensor_block_end(g, t) - g.t[t].block_first;
  const int slices = (nb + kHistSlice - 1) / kHistSlice;
  uint64_t Qb = 0, N = 0;
  for (int sl = 0; sl < slices; ++sl) {
    const uint64_t* e = a.hist_sum + ((hist_entry(g, t, sl) * a.n_present + k) * kBuckets + c) * 2;
    Qb += e[0];
    N += e[1];
  }
  const double term = write_codebook(a, g, k, t, c, Qb, N);
  if (a.norm2 != nullptr) {
    __shared__ double st[kBuckets];
    const double n2 = bucket_tree_sum(term, st);
    if (threadIdx.x == 0) a.norm2[codebook_row(a, g, k, t)] = n2;
  }
}

// ---------------------------------------------------------------------------
// k_merge: g = sum_i tab_i[code_i] with tab_i[c] = w_hat_i * codebook_i[c] (fp64,
// in LDS), learners in index order; then the Nesterov step in fp64.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void nesterov16(float (&tv)[kVec], float (&vv)[kVec], const double (&acc)[kVec],
                                           double lr, double beta) {
#pragma unroll
  for (int e = 0; e < kVec; ++e) {
    const double gsum = acc[e];
    const double bv = beta * (double)vv[e];
    const double vn = bv + gsum;
    const double bvn = beta * vn;
    const double step = gsum + bvn;
    const double u = lr * step;
    const double tn = (double)tv[e] - u;
    tv[e] = (float)tn;
    vv[e] = (float)vn;
  }
}

// Code words of one (learner, tile) item: 4 dwords per lane through a buffer
// descriptor covering the tile's 4096 codes (zero records = null request).
__device__ __forceinline__ void load_codes_rsrc(const uint8_t* cp, bool valid, int tid, uint32_t (&cw)[4]) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(cp), (short)0, valid ? kTile : 0, kBufferWord3);
#pragma unroll
  for (int j = 0; j < 4; ++j) cw[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, f4_index(tid, j) * 4, 0, 2);
}

// theta or momentum of one tile through a buffer descriptor covering the tile's
// 16 KB (zero records when !valid: loads return zeros, stores are dropped).
__device__ __forceinline__ void store_tile_rsrc(__amdgpu_buffer_rsrc_t r, int tid, const float (&v)[kVec]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    vf4 x;
    x.x = v[4 * j + 0];
    x.y = v[4 * j + 1];
    x.z = v[4 * j + 2];
    x.w = v[4 * j + 3];
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(vu4, x), r, f4_index(tid, j) * 16, 0, 2);
  }
}

// A merge block is kMergeTiles groups of kBlock threads; group q works on tile
// kMergeTiles * s + q of the block's span in round s, so every learner's codes,
// theta and momentum move in runs of kMergeTiles * 4 KB (codes) and
// kMergeTiles * 16 KB per block.  Tiles past the block's full tiles are null
// requests and dropped stores (wave-uniform: a group is 4 whole waves).
// Code words of (learner, round) items stream through a ring of kMergeRing
// registers (item i + kMergeRing - 1 is requested while item i is looked up),
// items per round padded to a multiple of the ring with null requests, every
// request unconditional.
// theta and momentum of a round are requested when the round starts; they are
// needed only after every learner has been looked up.
// NR > 0: every round has exactly NR ring rounds of kMergeRing items (up to
// kMergeRing * NR learners), so the learner loop unrolls and every round issues the same
// sequence of memory operations; the prologue ends with a round's worth of (null)
// stores, so the static wait counts fit the first round as well as the others.
// NR = 0: any number of learners, ring rounds counted at run time.
//
// Radial-Directional Averaging reuses this kernel twice.  DIR = true: the table
// holds a_i * codebook_i[c] with a_i = w_hat_i / ||x_i|| (x_i the dequantized
// pseudo-gradient, ||x_i||^2 from the codebook stage), theta and momentum are
// neither read nor written, and each block writes the sum of the squared
// averaged direction over its elements.  With a.coef set (DIR = false): the table
// holds coef_i * codebook_i[c], coef_i = a_i * r / ||d|| from k_rda_coef.
// A ring of 3 (2 items ahead) measured faster than 2, 4 and 8 on the 1B set
// (5.7%) and the 10B median fragment (1.2%), and neutral on small calls.
constexpr int kMergeRing = 3;
constexpr int kMergeMaxRounds = 8;
constexpr int kMergeBlock = kBlock * kMergeTiles;

// a_i = w_hat_i / ||x_i|| (0 for a learner whose dequantized tensor is zero)
__device__ __forceinline__ double rda_unit_weight(const MergeArgs& a, const LaunchGeom& g, size_t trow, int k) {
  const double n2 = a.norm2[(size_t)a.learner[k] * g.n_tensors_call + trow];
  return n2 > 0.0 ? a.w_hat[k] / __builtin_sqrt(n2) : 0.0;
}

template <int NR, bool DIR = false>
__global__ __launch_bounds__(kMergeBlock) __attribute__((amdgpu_waves_per_eu(4))) void k_merge(
    const MergeArgs a, const LaunchGeom g) {
  extern __shared__ __align__(16) unsigned char smem[];
  double* tab = reinterpret_cast<double*>(smem);
  // tile slot of this thread's group (whole waves: keep it in a scalar register)
  const int q = __builtin_amdgcn_readfirstlane(threadIdx.x / kBlock);
  const int tid = threadIdx.x % kBlock;  // thread within the group
  const int kp = a.n_present;
  const Span sp = block_span(g);
  const TensorDesc td = g.t[sp.t];
  const size_t trow = (size_t)g.row_base + g.t_base + sp.t;

  for (int i = threadIdx.x; i < kp * kBuckets; i += kMergeBlock) {
    const int k = i >> 8, c = i & (kBuckets - 1);
    const float cb = a.codebook[((size_t)a.learner[k] * g.n_tensors_call + trow) * kBuckets + c];
    double w;
    if (DIR) w = rda_unit_weight(a, g, trow, k);
    else w = a.coef != nullptr ? a.coef[trow * kp + k] : a.w_hat[k];
    tab[i] = w * (double)cb;
  }
  __syncthreads();
  double dsum = 0.0;  // DIR: this thread's sum of squared direction values

  float* __restrict__ th = a.theta_g + td.offset();
  float* __restrict__ mv = a.momentum + td.offset();
  auto codes_of = [&](int k) { return a.codes + (int64_t)a.learner[k] * a.stride + td.loffset(); };
  const double lr = a.lr, beta = a.beta;

  const int64_t n_full = (sp.end - sp.begin) / kTile;
  if (n_full > 0) {
    const int items = NR > 0 ? NR * kMergeRing : (kp + kMergeRing - 1) / kMergeRing * kMergeRing;
    const int64_t n_rounds = (n_full + kMergeTiles - 1) / kMergeTiles;
    // this group's tile of round r (element offset in the tensor) and whether it is full
    auto tile_of = [&](int64_t r) { return r * kMergeTiles + q; };
    auto request = [&](uint32_t (&dst)[4], int64_t r, int i) {
      const int64_t tile = tile_of(r);
      const bool valid = i < kp && tile < n_full;
      load_codes_rsrc(codes_of(i < kp ? i : kp - 1) + sp.begin + (valid ? tile : 0) * kTile, valid, tid, dst);
    };
    uint32_t ring[kMergeRing][4];
#pragma unroll
    for (int i = 0; i < kMergeRing - 1; ++i) request(ring[i], 0, i);
    if (NR > 0 && !DIR) {
      const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(th, (short)0, 0, kBufferWord3);
      const float zero[kVec] = {};
      store_tile_rsrc(none, tid, zero);
      store_tile_rsrc(none, tid, zero);
    }
    __builtin_amdgcn_sched_barrier(0);
    for (int64_t r = 0; r < n_rounds; ++r) {
      const int64_t tile = tile_of(r);
      const bool valid = tile < n_full;
      const int64_t base = sp.begin + (valid ? tile : 0) * kTile;
      const __amdgpu_buffer_rsrc_t rt = tile_rsrc(th + base, valid && !DIR), rv = tile_rsrc(mv + base, valid && !DIR);
      float tv[kVec], vv[kVec];
      if (!DIR) {
        load_tile_rsrc(rt, tid, tv);
        load_tile_rsrc(rv, tid, vv);
      }
      double acc[kVec];
#pragma unroll
      for (int e = 0; e < kVec; ++e) acc[e] = 0.0;
      constexpr int kRoundsUnroll = NR > 0 ? NR : 1;
#pragma unroll kRoundsUnroll
      for (int i0 = 0; i0 < items; i0 += kMergeRing) {
#pragma unroll
        for (int u = 0; u < kMergeRing; ++u) {
          const int i = i0 + u;
          const int ip = i + kMergeRing - 1;
          if (ip < items) request(ring[(u + kMergeRing - 1) % kMergeRing], r, ip);
          else request(ring[(u + kMergeRing - 1) % kMergeRing], r + 1, ip - items);
          if (i < kp) {
            const double* tk = tab + i * kBuckets;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
#pragma unroll
              for (int c = 0; c < 4; ++c) acc[4 * j + c] += tk[(ring[u][j] >> (8 * c)) & 0xffu];
            }
          }
        }
      }
      if (DIR) {
        if (valid) {
#pragma unroll
          for (int e = 0; e < kVec; ++e) dsum += acc[e] * acc[e];
        }
      } else {
        nesterov16(tv, vv, acc, lr, beta);
        store_tile_rsrc(rt, tid, tv);
        store_tile_rsrc(rv, tid, vv);
      }
    }
  }
  const int64_t full_end = sp.begin + n_full * kTile;
  if (q == 0 && full_end < sp.end) {
    const int64_t n = sp.end - full_end;
    float tv[kVec], vv[kVec];
    if (!DIR) {
      load_tail(th + full_end, tid, n, tv);
      load_tail(mv + full_end, tid, n, vv);
    }
    double acc[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e) acc[e] = 0.0;
    for (int k = 0; k < kp; ++k) {
      const uint8_t* cp = codes_of(k) + full_end;
      const double* tk = tab + k * kBuckets;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (tail_valid(tid, j, c, n)) acc[4 * j + c] += tk[cp[elem_index(tid, j, c)]];
        }
      }
    }
    if (DIR) {
#pragma unroll
      for (int e = 0; e < kVec; ++e) dsum += acc[e] * acc[e];  // invalid elements hold 0
    } else {
      nesterov16(tv, vv, acc, lr, beta);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (tail_valid(tid, j, c, n)) {
            const int64_t e = full_end + elem_index(tid, j, c);
            th[e] = tv[4 * j + c];
            mv[e] = vv[4 * j + c];
          }
        }
      }
    }
  }
  if (DIR) {
    __shared__ double red[kMergeBlock / 64];
    const double w = wave_sum(dsum);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = w;
    __syncthreads();
    if (threadIdx.x == 0) {
      double total = 0.0;
      for (int i = 0; i < kMergeBlock / 64; ++i) total += red[i];
      a.dir_part[g.slot_base + blockIdx.x] = total;
    }
  }
}

// k_rda_coef: one block per tensor.  ||d||^2 = the tensor's block sums of the
// squared averaged direction (strided per thread, then a fixed tree);
// r = sum_i w_hat_i ||x_i|| in learner order; coef_i = a_i * r / ||d||, all 0
// (g = 0) when d counts as zero: ||d|| <= kRdaNullDirection * W, W = the summed
// w_hat_i of the learners with ||x_i|| > 0, the largest ||d|| can be.  Directions
// that cancel in real arithmetic leave only about K 2^-53 W of rounding noise in
// d, which points nowhere in particular.
constexpr double kRdaNullDirection = 0x1p-40;

__global__ __launch_bounds__(kBuckets) void k_rda_coef(const MergeArgs a, const LaunchGeom g) {
  __shared__ double st[kBuckets];
  __shared__ double scale;
  const int t = blockIdx.x;
  const int b1 = tensor_block_end(g, t);
  double v = 0.0;
  for (int b = g.t[t].block_first + threadIdx.x; b < b1; b += kBuckets) v += a.dir_part[g.slot_base + b];
  const double d2 = bucket_tree_sum(v, st);
  const size_t trow = (size_t)g.row_base + g.t_base + t;
  const int kp = a.n_present;
  if (threadIdx.x == 0) {
    double r = 0.0, moved = 0.0;
    for (int k = 0; k < kp; ++k) {
      const double n2 = a.norm2[(size_t)a.learner[k] * g.n_tensors_call + trow];
      r += a.w_hat[k] * __builtin_sqrt(n2);
      if (n2 > 0.0) moved += a.w_hat[k];
    }
    const double dn = __builtin_sqrt(d2);
    scale = dn > kRdaNullDirection * moved ? r / dn : 0.0;
  }
  __syncthreads();
  for (int k = threadIdx.x; k < kp; k += kBuckets) a.coef[trow * kp + k] = scale * rda_unit_weight(a, g, trow, k);
}

// ---------------------------------------------------------------------------
// k_broadcast: the updated theta_g of each tensor copied into every given learner
// row.  A full tile of theta_g is loaded once (the next one is requested before
// the current one is stored) and stored to each row as one 16 KB run of
// non-temporal stores; tiles past the block's full tiles, and rows past n_rows,
// are null requests and dropped stores.  NR > 0: rows padded to NR at compile
// time, so every tile issues the same sequence of memory operations (the
// prologue adds one tile's worth of null stores); NR = 0: any number of rows.
// The partial tail tile is copied element by element.
// ---------------------------------------------------------------------------
constexpr int kBroadcastMaxRows = 16;

template <int NR>
__global__ __launch_bounds__(kBlock) void k_broadcast(const BroadcastArgs a, const LaunchGeom g) {
  const int tid = threadIdx.x;
  const Span sp = block_span(g);
  const TensorDesc td = g.t[sp.t];
  const float* __restrict__ src = a.theta_g + td.offset() + sp.begin;
  const int64_t n_full = (sp.end - sp.begin) / kTile;
  auto row_of = [&](int r) { return a.theta_L + (int64_t)a.row[r] * a.stride + td.loffset() + sp.begin; };
  if (n_full > 0) {
    const int rows = NR > 0 ? NR : a.n_rows;
    auto request = [&](float (&dst)[kVec], int64_t tile) {
      const bool valid = tile < n_full;
      load_tile_rsrc(tile_rsrc(src + (valid ? tile : 0) * kTile, valid), tid, dst);
    };
    auto store_rows = [&](const float (&v)[kVec], int64_t tile) {
      constexpr int kUnroll = NR > 0 ? NR : 1;
#pragma unroll kUnroll
      for (int r = 0; r < rows; ++r) {
        const bool valid = tile < n_full && r < a.n_rows;
        float* dst = row_of(r < a.n_rows ? r : 0) + (valid ? tile : 0) * kTile;
        store_tile_rsrc(tile_rsrc(dst, valid), tid, v);
      }
    };
    float v0[kVec], v1[kVec];
    request(v0, 0);
    if (NR > 0) {
      const float zero[kVec] = {};
      store_rows(zero, n_full);  // null stores: the steady state's previous tile
    }
    __builtin_amdgcn_sched_barrier(0);
    for (int64_t i = 0; i < n_full; i += 2) {
      request(v1, i + 1);
      store_rows(v0, i);
      request(v0, i + 2);
      store_rows(v1, i + 1);
    }
  }
  const int64_t full_len = n_full * kTile;
  if (sp.begin + full_len < sp.end) {
    const int64_t n = sp.end - sp.begin - full_len;
    float v[kVec];
    load_tail(src + full_len, tid, n, v);
    for (int r = 0; r < a.n_rows; ++r) {
      float* dst = row_of(r) + full_len;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (tail_valid(tid, j, c, n)) dst[elem_index(tid, j, c)] = v[4 * j + c];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// The ring with requantization at every hop (INTELLECT-1 notes, section 3.2
// step 6 and section 4.2).
// k_dequant_add: for each message segment, the receiver's chunk (which it has
// never changed before: rank r receives chunk r - 1 - s at hop s and sends it at
// hop s + 1) becomes -fl32(Delta + deQ(message)), stored negated as
// fl32(fl32(theta_L - theta_g) - cb[code]) (fl32(theta_L - theta_g) = -Delta
// exactly), then optionally fl32(x / divisor) = -fl32(mean).  The segment's
// codebook row sits in LDS.  Segment descriptors: offset = the chunk in
// theta_g, loffset = the receiver's chunk in the flat [ranks][stride]
// theta_L / accum; the sender's codes sit one row earlier (cyclically).
// The new sum is the receiver's next message, so the kernel also forms that
// message's statistics partials exactly as k_stats would (the same partition,
// element order, shift and reductions): d = fl32(0 - x) - shift with shift =
// the receiver's pseudo-gradient at the segment's first element.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void k_dequant_add(const RingArgs a, const LaunchGeom g) {
  __shared__ float cb[kBuckets];
  const int tid = threadIdx.x;
  const Span sp = block_span(g);
  const TensorDesc td = g.t[sp.t];
  cb[tid] = a.codebook[(size_t)a.cb_row[sp.t] * kBuckets + tid];
  __syncthreads();
  const double shift = (double)(a.theta_g[td.offset()] - a.theta_L[td.loffset()]);
  double s1 = 0.0, s2 = 0.0;
  auto accumulate = [&](float x) {
    const double d = (double)(0.0f - x) - shift;
    s1 += d;
    s2 = __fma_rn(d, d, s2);
  };
  const int64_t dst0 = td.loffset();
  const int64_t src0 = dst0 >= a.stride ? dst0 - a.stride : dst0 + (int64_t)(a.n_ranks - 1) * a.stride;
  float* __restrict__ dst = a.accum + dst0 + sp.begin;
  const float* __restrict__ tl = a.theta_L + dst0 + sp.begin;
  const float* __restrict__ tg = a.theta_g + td.offset() + sp.begin;
  const uint8_t* __restrict__ src = a.codes + src0 + sp.begin;
  const float div = a.divisor;
  auto update = [&](float l, float g0, uint32_t code) {
    const float x = (l - g0) - cb[code];
    return div != 0.0f ? x / div : x;
  };
  const int64_t n_full = (sp.end - sp.begin) / kTile;
  // Two register slots: tile t + 1 is requested before tile t is updated and
  // stored; requests past the block's full tiles are null (zero-record
  // descriptors), so every iteration issues the same memory operations.
  float lv[2][kVec], gv[2][kVec];
  uint32_t cw[2][4];
  auto request = [&](int slot, int64_t tile) {
    const bool valid = tile < n_full;
    const int64_t o = (valid ? tile : 0) * kTile;
    load_tile_rsrc(tile_rsrc(tl + o, valid), tid, lv[slot]);
    load_tile_rsrc(tile_rsrc(tg + o, valid), tid, gv[slot]);
    load_codes_rsrc(src + o, valid, tid, cw[slot]);
  };
  auto finish = [&](int slot, int64_t tile) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int e = 4 * j + c;
        lv[slot][e] = update(lv[slot][e], gv[slot][e], (cw[slot][j] >> (8 * c)) & 0xffu);
      }
    }
    if (tile < n_full) {
#pragma unroll
      for (int e = 0; e < kVec; ++e) accumulate(lv[slot][e]);
    }
    store_tile_rsrc(tile_rsrc(dst + (tile < n_full ? tile : 0) * kTile, tile < n_full), tid, lv[slot]);
  };
  if (n_full > 0) {
    request(0, 0);
    // stand-ins for the stores that precede the loop head on the back edge, so
    // both paths into the loop carry the same memory operations (exact waits)
    const float zero[kVec] = {};
    store_tile_rsrc(tile_rsrc(dst, false), tid, zero);
    __builtin_amdgcn_sched_barrier(0);
    for (int64_t tile = 0; tile < n_full; tile += 2) {
      request(1, tile + 1);
      __builtin_amdgcn_sched_barrier(0);
      finish(0, tile);
      request(0, tile + 2);
      __builtin_amdgcn_sched_barrier(0);
      finish(1, tile + 1);
    }
  }
  const int64_t full_len = n_full * kTile;
  if (sp.begin + full_len < sp.end) {
    const int64_t n = sp.end - sp.begin - full_len;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (tail_valid(tid, j, c, n)) {
          const int64_t e = full_len + elem_index(tid, j, c);
          const float x = update(tl[e], tg[e], src[e]);
          dst[e] = x;
          accumulate(x);
        }
      }
    }
  }
  // the block's partials, reduced as k_stats reduces them
  __shared__ double red[2][kWaves];
  const int lane = tid & 63, wave = tid >> 6;
  const double r1 = wave_sum(s1), r2 = wave_sum(s2);
  if (lane == 0) {
    red[0][wave] = r1;
    red[1][wave] = r2;
  }
  __syncthreads();
  if (tid == 0) {
    double t1 = 0.0, t2 = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      t1 += red[0][w];
      t2 += red[1][w];
    }
    a.part_stats[g.slot_base + blockIdx.x] = make_double2(t1, t2);
  }
}

template <typename K>
hipError_t allow_lds(K kernel, size_t lds) {
  if (lds <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)lds);
}

// One device word, written by a kernel (a memset node may not replay correctly in a
// captured graph).
__global__ __launch_bounds__(64) void k_fill_u32(uint32_t* p, uint32_t v) {
  if (threadIdx.x == 0) *p = v;
}

}  // namespace

hipError_t launch_stats(const QuantArgs& a, const LaunchGeom& g, hipStream_t s) {
  const dim3 grid(g.n_blocks), block(kBlock);
  if (a.k_count <= 2) {
    hipLaunchKernelGGL(k_stats<2>, grid, block, 0, s, a, g);
  } else if (a.k_count <= 5) {
    hipLaunchKernelGGL(k_stats<5>, grid, block, 0, s, a, g);
  } else if (a.k_count <= 8) {
    hipLaunchKernelGGL(k_stats<8>, grid, block, 0, s, a, g);
  } else if (a.k_count <= 11) {
    hipLaunchKernelGGL(k_stats<11>, grid, block, 0, s, a, g);
  } else {
    hipLaunchKernelGGL(k_stats<14>, grid, block, 0, s, a, g);
  }
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, uint32_t v, hipStream_t s) {
  hipLaunchKernelGGL(k_fill_u32, dim3(1), dim3(64), 0, s, p, v);
  return hipGetLastError();
}

hipError_t launch_range(const QuantArgs& a, const LaunchGeom& g, hipStream_t s) {
  hipLaunchKernelGGL(k_range, dim3(a.n_present * g.n_tensors), dim3(kRangeThreads), 0, s, a, g);
  return hipGetLastError();
}

size_t encode_lds_bytes(int k_count, int copies) {
  return (size_t)k_count * copies * kHistBytes + (size_t)k_count * sizeof(EncodePar);
}

// Copies of each learner's histogram, interleaved per bucket and picked by lane:
// lanes that hit the same bucket in one instruction land on different words, so
// concentrated code distributions (for example pseudo-gradients that are exactly
// zero on untouched rows) do not serialize on one address.  Four copies up to 8
// learners per launch (64 KB of histogram), two above.
int encode_copies(int k_count) { return k_count <= 8 ? 4 : 2; }

template <int R>
hipError_t launch_encode_r(const QuantArgs& a, const LaunchGeom& g, hipStream_t s) {
  const size_t lds = encode_lds_bytes(a.k_count, R);
  hipError_t e = allow_lds(k_encode<R>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_encode<R>, dim3(g.n_blocks), dim3(kBlock), lds, s, a, g);
  return hipGetLastError();
}

hipError_t launch_encode(const QuantArgs& a, const LaunchGeom& g, hipStream_t s) {
  const int r = encode_copies(a.k_count);
  if (r == 4) return launch_encode_r<4>(a, g, s);
  if (r == 2) return launch_encode_r<2>(a, g, s);
  return launch_encode_r<1>(a, g, s);
}

hipError_t launch_codebook(const QuantArgs& a, const LaunchGeom& g, hipStream_t s) {
  const dim3 grid(g.hist_slices, a.n_present * g.n_tensors), block(kBuckets * kCodebookGroups);
  if (g.hist_slices == 1) {
    hipLaunchKernelGGL(k_hist_reduce<true>, grid, block, 0, s, a, g);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_hist_reduce<false>, grid, block, 0, s, a, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_codebook, dim3(a.n_present * g.n_tensors), dim3(kBuckets), 0, s, a, g);
  return hipGetLastError();
}

template <int NR>
hipError_t launch_merge_r(const MergeArgs& a, const LaunchGeom& g, hipStream_t s) {
  const size_t lds = (size_t)a.n_present * kBuckets * sizeof(double);
  hipError_t e = allow_lds(k_merge<NR>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_merge<NR>, dim3(g.n_blocks), dim3(kMergeBlock), lds, s, a, g);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, const LaunchGeom& g, hipStream_t s) {
  static_assert(kMergeMaxRounds == 8, "one instantiation per round count");
  switch ((a.n_present + kMergeRing - 1) / kMergeRing) {
    case 1: return launch_merge_r<1>(a, g, s);
    case 2: return launch_merge_r<2>(a, g, s);
    case 3: return launch_merge_r<3>(a, g, s);
    case 4: return launch_merge_r<4>(a, g, s);
    case 5: return launch_merge_r<5>(a, g, s);
    case 6: return launch_merge_r<6>(a, g, s);
    case 7: return launch_merge_r<7>(a, g, s);
    case 8: return launch_merge_r<8>(a, g, s);
    default: return launch_merge_r<0>(a, g, s);
  }
}

template <int NR>
hipError_t launch_rda_direction_r(const MergeArgs& a, const LaunchGeom& g, hipStream_t s) {
  const size_t lds = (size_t)a.n_present * kBuckets * sizeof(double);
  hipError_t e = allow_lds(k_merge<NR, true>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_merge<NR, true>), dim3(g.n_blocks), dim3(kMergeBlock), lds, s, a, g);
  return hipGetLastError();
}

hipError_t launch_rda_direction(const MergeArgs& a, const LaunchGeom& g, hipStream_t s) {
  switch ((a.n_present + kMergeRing - 1) / kMergeRing) {
    case 1: return launch_rda_direction_r<1>(a, g, s);
    case 2: return launch_rda_direction_r<2>(a, g, s);
    case 3: return launch_rda_direction_r<3>(a, g, s);
    case 4: return launch_rda_direction_r<4>(a, g, s);
    case 5: return launch_rda_direction_r<5>(a, g, s);
    case 6: return launch_rda_direction_r<6>(a, g, s);
    case 7: return launch_rda_direction_r<7>(a, g, s);
    case 8: return launch_rda_direction_r<8>(a, g, s);
    default: return launch_rda_direction_r<0>(a, g, s);
  }
}

hipError_t launch_rda_coef(const MergeArgs& a, const LaunchGeom& g, hipStream_t s) {
  hipLaunchKernelGGL(k_rda_coef, dim3(g.n_tensors), dim3(kBuckets), 0, s, a, g);
  return hipGetLastError();
}

hipError_t launch_broadcast(const BroadcastArgs& a, const LaunchGeom& g, hipStream_t s) {
  static_assert(kBroadcastMaxRows == 16, "one instantiation per padded row count");
  const dim3 grid(g.n_blocks), block(kBlock);
  switch ((a.n_rows + 3) / 4) {
    case 1: hipLaunchKernelGGL(k_broadcast<4>, grid, block, 0, s, a, g); break;
    case 2: hipLaunchKernelGGL(k_broadcast<8>, grid, block, 0, s, a, g); break;
    case 3: hipLaunchKernelGGL(k_broadcast<12>, grid, block, 0, s, a, g); break;
    case 4: hipLaunchKernelGGL(k_broadcast<16>, grid, block, 0, s, a, g); break;
    default: hipLaunchKernelGGL(k_broadcast<0>, grid, block, 0, s, a, g); break;
  }
  return hipGetLastError();
}

hipError_t launch_dequant_add(const RingArgs& a, const LaunchGeom& g, hipStream_t s) {
  hipLaunchKernelGGL(k_dequant_add, dim3(g.n_blocks), dim3(kBlock), 0, s, a, g);
  return hipGetLastError();
}

}  // namespace dlc
