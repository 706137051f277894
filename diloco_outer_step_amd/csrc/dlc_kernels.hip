// gfx950 kernels of the DiLoCo outer-step merge.
//
// Three streaming passes over HBM per outer step, plus two tiny finalizers:
//   k_stats     per-(learner, tensor) partial sum(d), sum(d^2) of d = Delta - shift, fp64
//   k_range     per-(learner, tensor) mu, sigma -> {lo, hi, wd, mean} (fp64 -> fp32)
//   k_encode    Delta -> clip -> bucket -> uint8 code (16-byte stores) + LDS histogram
//               of (sum of clipped values in fp64, count) per learner
//   k_codebook  per-(learner, tensor, bucket) mean of the clipped values -> fp32
//   k_merge     dequantize K learners through fp64 LDS tables w_hat_i * codebook_i,
//               sum, Nesterov update of theta and momentum, every byte read once
//
// The quantizer follows the INTELLECT-1 reading notes, section 4.1 (per-tensor mu
// and sigma, clip at 6 sigma, 256 equal buckets, codebook of bucket means); the
// merge follows section 3.2 steps 6-7 and section 4.2 (dequantize, accumulate in
// floating point, Nesterov with lr 0.7 / momentum 0.9).
//
// Every tile is kTile = 4096 elements of one tensor; thread tid owns the float4s
// q = j * kBlock + tid (j = 0..3), so each load instruction of a wave reads 1 KB
// of consecutive bytes.  Floating point contraction is off for this file: every
// operation that has to match the fp32/fp64 definition bit for bit is written as
// separate IEEE operations; the only fused multiply-add is the explicit one that
// accumulates sum(d^2).
#include "dlc_internal.h"

#include <cfloat>

namespace dlc {
namespace {

constexpr int kWaves = kBlock / 64;

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
  s.end = e < g.t[lo].numel ? e : g.t[lo].numel;
  return s;
}

__device__ __forceinline__ int tensor_block_end(const LaunchGeom& g, int t) {
  return t + 1 < g.n_tensors ? g.t[t + 1].block_first : g.n_blocks;
}

// 16 floats of a full tile (4 coalesced float4 loads).
__device__ __forceinline__ void load_full(const float* __restrict__ p, int tid, float (&v)[kVec]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float4 x = *reinterpret_cast<const float4*>(p + 4 * (j * kBlock + tid));
    v[4 * j + 0] = x.x;
    v[4 * j + 1] = x.y;
    v[4 * j + 2] = x.z;
    v[4 * j + 3] = x.w;
  }
}

// 16 floats of a tail tile: element e valid iff base_rel + e < n (n elements left).
__device__ __forceinline__ void load_tail(const float* __restrict__ p, int tid, int64_t n,
                                          float (&v)[kVec]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int64_t e = 4 * (j * kBlock + tid) + c;
      v[4 * j + c] = e < n ? p[e] : 0.0f;
    }
  }
}

__device__ __forceinline__ bool tail_valid(int tid, int j, int c, int64_t n) {
  return (int64_t)(4 * (j * kBlock + tid) + c) < n;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// ---------------------------------------------------------------------------
// k_stats: partial moments about a per-(learner, tensor) shift.
//
// shift = Delta at the tensor's first element, so sum(d) and sum(d^2) stay small
// and var = sum(d^2)/n - (sum(d)/n)^2 loses nothing in fp64.  Each block covers
// one tensor; its per-learner partial sums go to workspace slot slot_base + block.
// ---------------------------------------------------------------------------
template <int KC>
__global__ __launch_bounds__(kBlock) void k_stats(const QuantArgs a, const LaunchGeom g) {
  const int tid = threadIdx.x;
  const Span sp = block_span(g);
  const TensorDesc td = g.t[sp.t];
  const float* __restrict__ tg = a.theta_g + td.offset;
  const int kc = a.k_count;

  const float* tl[KC];
  double shift[KC], s1[KC], s2[KC];
  const float g0 = tg[0];
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    const int li = a.learner[a.k_base + (k < kc ? k : 0)];
    tl[k] = a.theta_L + (int64_t)li * a.stride + td.loffset;
    shift[k] = (double)(g0 - tl[k][0]);
    s1[k] = 0.0;
    s2[k] = 0.0;
  }

  for (int64_t base = sp.begin; base < sp.end; base += kTile) {
    const int64_t n = sp.end - base;
    float gv[kVec];
    if (n >= kTile) {
      load_full(tg + base, tid, gv);
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        if (k < kc) {
          float lv[kVec];
          load_full(tl[k] + base, tid, lv);
#pragma unroll
          for (int e = 0; e < kVec; ++e) {
            const double d = (double)(gv[e] - lv[e]) - shift[k];
            s1[k] += d;
            s2[k] = __fma_rn(d, d, s2[k]);
          }
        }
      }
    } else {
      load_tail(tg + base, tid, n, gv);
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        if (k < kc) {
          float lv[kVec];
          load_tail(tl[k] + base, tid, n, lv);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              if (tail_valid(tid, j, c, n)) {
                const int e = 4 * j + c;
                const double d = (double)(gv[e] - lv[e]) - shift[k];
                s1[k] += d;
                s2[k] = __fma_rn(d, d, s2[k]);
              }
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
// k_range: one thread per (present learner, tensor of the launch).
// Blocks of a tensor are summed in block order (deterministic).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_range(const QuantArgs a, const LaunchGeom g) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= a.n_present * g.n_tensors) return;
  const int k = idx / g.n_tensors;
  const int t = idx - k * g.n_tensors;
  const TensorDesc td = g.t[t];
  const int b0 = td.block_first, b1 = tensor_block_end(g, t);
  double S1 = 0.0, S2 = 0.0;
  for (int b = b0; b < b1; ++b) {
    const double2 p = a.part_stats[(size_t)(g.slot_base + b) * a.n_present + k];
    S1 += p.x;
    S2 += p.y;
  }
  const int li = a.learner[k];
  const float g0 = a.theta_g[td.offset];
  const float l0 = a.theta_L[(int64_t)li * a.stride + td.loffset];
  const double shift = (double)(g0 - l0);
  const double n = (double)td.numel;
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
  a.range[(size_t)li * g.n_tensors_call + g.t_base + t] = r;
}

// ---------------------------------------------------------------------------
// k_encode: codes + per-block LDS histogram for up to kLearnerChunk learners.
//
// Dynamic LDS: hsum[kc][256] (fp64), hcnt[kc][256] (u32), stage[kWaves][256] (u32).
// Codes of a full tile are packed 4 per dword in the load layout, transposed
// through a per-wave LDS stage, and written with 16-byte stores (16 lanes write
// 256 consecutive bytes).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t bucket_of(float x, float lo, float wd) {
  const float t = x - lo;
  const float q = t / wd;  // IEEE fp32 division (correctly rounded)
  const float c = fminf(fmaxf(floorf(q), 0.0f), 255.0f);
  return (uint32_t)c;
}

__global__ __launch_bounds__(kBlock) void k_encode(const QuantArgs a, const LaunchGeom g) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int kc = a.k_count;
  double* hsum = reinterpret_cast<double*>(smem);
  uint32_t* hcnt = reinterpret_cast<uint32_t*>(hsum + kc * kBuckets);
  uint32_t* stage = hcnt + kc * kBuckets;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  for (int i = tid; i < kc * kBuckets; i += kBlock) {
    hsum[i] = 0.0;
    hcnt[i] = 0u;
  }
  __syncthreads();

  const Span sp = block_span(g);
  const TensorDesc td = g.t[sp.t];
  const float* __restrict__ tg = a.theta_g + td.offset;
  const size_t rrow = (size_t)g.t_base + sp.t;
  uint32_t* st = stage + wave * 256;

  for (int64_t base = sp.begin; base < sp.end; base += kTile) {
    const int64_t n = sp.end - base;
    const bool full = n >= kTile;
    float gv[kVec];
    if (full) load_full(tg + base, tid, gv); else load_tail(tg + base, tid, n, gv);

    for (int k = 0; k < kc; ++k) {
      const int li = a.learner[a.k_base + k];
      const int64_t row = (int64_t)li * a.stride + td.loffset + base;
      const float4 r = a.range[(size_t)li * g.n_tensors_call + rrow];
      const float lo = r.x, hi = r.y, wd = r.z;
      const bool degenerate = !(wd >= FLT_MIN);
      double* hs = hsum + k * kBuckets;
      uint32_t* hc = hcnt + k * kBuckets;
      float lv[kVec];
      if (full) load_full(a.theta_L + row, tid, lv); else load_tail(a.theta_L + row, tid, n, lv);

      uint32_t packed[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t w = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int e = 4 * j + c;
          const float x = gv[e] - lv[e];
          uint32_t code = 0;
          if (!degenerate) {
            code = bucket_of(x, lo, wd);
            if (full || tail_valid(tid, j, c, n)) {
              const float xc = fminf(fmaxf(x, lo), hi);
              atomicAdd(&hs[code], (double)xc);
              atomicAdd(&hc[code], 1u);
            }
          }
          w |= code << (8 * c);
        }
        packed[j] = w;
      }

      uint8_t* cp = a.codes + row;
      if (full) {
#pragma unroll
        for (int j = 0; j < 4; ++j) st[j * 64 + lane] = packed[j];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int j = lane >> 4, r16 = lane & 15;
        const uint4 v = *reinterpret_cast<const uint4*>(st + j * 64 + 4 * r16);
        *reinterpret_cast<uint4*>(cp + 4 * (j * kBlock + 64 * wave + 4 * r16)) = v;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            if (tail_valid(tid, j, c, n)) cp[4 * (j * kBlock + tid) + c] = (uint8_t)(packed[j] >> (8 * c));
          }
        }
      }
    }
  }

  __syncthreads();
  const size_t slot = (size_t)(g.slot_base + blockIdx.x);
  for (int i = tid; i < kc * kBuckets; i += kBlock) {
    const int k = i >> 8, c = i & (kBuckets - 1);
    const size_t o = ((slot * a.n_present) + a.k_base + k) * kBuckets + c;
    a.part_sum[o] = hsum[i];
    a.part_cnt[o] = hcnt[i];
  }
}

// ---------------------------------------------------------------------------
// k_codebook: one block of 256 threads per (present learner, tensor); thread c
// sums bucket c over the tensor's blocks in block order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBuckets) void k_codebook(const QuantArgs a, const LaunchGeom g) {
  const int k = blockIdx.x / g.n_tensors;
  const int t = blockIdx.x - k * g.n_tensors;
  const int c = threadIdx.x;
  const int li = a.learner[k];
  const size_t row = (size_t)li * g.n_tensors_call + g.t_base + t;
  const float4 r = a.range[row];
  float out;
  if (!(r.z >= FLT_MIN)) {
    out = r.w;
  } else {
    const int b0 = g.t[t].block_first, b1 = tensor_block_end(g, t);
    double S = 0.0;
    uint64_t n = 0;
    for (int b = b0; b < b1; ++b) {
      const size_t o = ((size_t)(g.slot_base + b) * a.n_present + k) * kBuckets + c;
      S += a.part_sum[o];
      n += a.part_cnt[o];
    }
    if (n > 0) {
      out = (float)(S / (double)n);
    } else {
      out = (float)((double)r.x + ((double)c + 0.5) * (double)r.z);
    }
  }
  a.codebook[row * kBuckets + c] = out;
}

// ---------------------------------------------------------------------------
// k_merge: g = sum_i tab_i[code_i] with tab_i[c] = w_hat_i * codebook_i[c] (fp64,
// in LDS), learners in index order; then the Nesterov step in fp64.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void k_merge(const MergeArgs a, const LaunchGeom g) {
  extern __shared__ __align__(16) unsigned char smem[];
  double* tab = reinterpret_cast<double*>(smem);
  const int tid = threadIdx.x;
  const int kp = a.n_present;
  const Span sp = block_span(g);
  const TensorDesc td = g.t[sp.t];
  const size_t trow = (size_t)g.t_base + sp.t;

  for (int i = tid; i < kp * kBuckets; i += kBlock) {
    const int k = i >> 8, c = i & (kBuckets - 1);
    const float cb = a.codebook[((size_t)a.learner[k] * g.n_tensors_call + trow) * kBuckets + c];
    tab[i] = a.w_hat[k] * (double)cb;
  }
  __syncthreads();

  float* __restrict__ th = a.theta_g + td.offset;
  float* __restrict__ mv = a.momentum + td.offset;
  const double lr = a.lr, beta = a.beta;

  for (int64_t base = sp.begin; base < sp.end; base += kTile) {
    const int64_t n = sp.end - base;
    const bool full = n >= kTile;
    float tv[kVec], vv[kVec];
    if (full) {
      load_full(th + base, tid, tv);
      load_full(mv + base, tid, vv);
    } else {
      load_tail(th + base, tid, n, tv);
      load_tail(mv + base, tid, n, vv);
    }
    double acc[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e) acc[e] = 0.0;

    for (int k = 0; k < kp; ++k) {
      const uint8_t* cp = a.codes + (int64_t)a.learner[k] * a.stride + td.loffset + base;
      uint32_t cw[4];
      if (full) {
#pragma unroll
        for (int j = 0; j < 4; ++j) cw[j] = *reinterpret_cast<const uint32_t*>(cp + 4 * (j * kBlock + tid));
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t w = 0;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            if (tail_valid(tid, j, c, n)) w |= (uint32_t)cp[4 * (j * kBlock + tid) + c] << (8 * c);
          }
          cw[j] = w;
        }
      }
      const double* tk = tab + k * kBuckets;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[4 * j + c] += tk[(cw[j] >> (8 * c)) & 0xffu];
      }
    }

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

    if (full) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        *reinterpret_cast<float4*>(th + base + 4 * (j * kBlock + tid)) =
            make_float4(tv[4 * j], tv[4 * j + 1], tv[4 * j + 2], tv[4 * j + 3]);
        *reinterpret_cast<float4*>(mv + base + 4 * (j * kBlock + tid)) =
            make_float4(vv[4 * j], vv[4 * j + 1], vv[4 * j + 2], vv[4 * j + 3]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (tail_valid(tid, j, c, n)) {
            const int64_t e = base + 4 * (j * kBlock + tid) + c;
            th[e] = tv[4 * j + c];
            mv[e] = vv[4 * j + c];
          }
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_stats(const QuantArgs& a, const LaunchGeom& g, hipStream_t s) {
  if (a.k_count <= 4) {
    hipLaunchKernelGGL(k_stats<4>, dim3(g.n_blocks), dim3(kBlock), 0, s, a, g);
  } else if (a.k_count <= 8) {
    hipLaunchKernelGGL(k_stats<8>, dim3(g.n_blocks), dim3(kBlock), 0, s, a, g);
  } else {
    hipLaunchKernelGGL(k_stats<16>, dim3(g.n_blocks), dim3(kBlock), 0, s, a, g);
  }
  return hipGetLastError();
}

hipError_t launch_range(const QuantArgs& a, const LaunchGeom& g, hipStream_t s) {
  const int n = a.n_present * g.n_tensors;
  hipLaunchKernelGGL(k_range, dim3((n + 63) / 64), dim3(64), 0, s, a, g);
  return hipGetLastError();
}

hipError_t launch_encode(const QuantArgs& a, const LaunchGeom& g, hipStream_t s) {
  const size_t lds = (size_t)a.k_count * kBuckets * (sizeof(double) + sizeof(uint32_t)) +
                     (size_t)kWaves * 256 * sizeof(uint32_t);
  hipLaunchKernelGGL(k_encode, dim3(g.n_blocks), dim3(kBlock), lds, s, a, g);
  return hipGetLastError();
}

hipError_t launch_codebook(const QuantArgs& a, const LaunchGeom& g, hipStream_t s) {
  hipLaunchKernelGGL(k_codebook, dim3(a.n_present * g.n_tensors), dim3(kBuckets), 0, s, a, g);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, const LaunchGeom& g, hipStream_t s) {
  const size_t lds = (size_t)a.n_present * kBuckets * sizeof(double);
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_merge),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_merge, dim3(g.n_blocks), dim3(kBlock), lds, s, a, g);
  return hipGetLastError();
}

}  // namespace dlc
