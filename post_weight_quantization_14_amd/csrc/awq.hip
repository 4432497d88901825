// Activation-aware channel scaling (AWQ) in front of the linear quantizer.
//
// The page "大模型量化：GPTQ/AWQ/GGUF 原理对比…" (AWQ section) protects the
// input channels that carry large activations: importance = mean |x| over the
// calibration tokens; channels above the median are multiplied by a factor s
// (2 by default) before quantization, and the dequantized weight is divided
// by it again (at inference the activations are).  The quantizer is the
// pages' LinearQuantizer (rtn.hip), given the per-column factor.
//
//   awq_stats_kernel      Σ_t |x_t| per channel: one pass over X [T, n]; a
//                         workgroup owns 256·(16 B / element) channels of a
//                         token slice, 16-byte rows, fp64 accumulators; slices
//                         are summed in slice order (deterministic)
//   awq_scale_kernel      importance = Σ|x| / T (fp64), its lower median by a
//                         radix selection over order-preserving 64-bit keys
//                         (8 passes of 8 bits, histograms in LDS), and the
//                         factor s where importance > median, else 1
#include <algorithm>

#include "gptq_internal.hpp"

namespace gptq {
namespace {

constexpr int kAwqThreads = 256;

template <typename T>
__device__ __forceinline__ float awq_f32(T v);
template <>
__device__ __forceinline__ float awq_f32<uint16_t>(uint16_t v) {
  return __uint_as_float((uint32_t)v << 16);
}
template <>
__device__ __forceinline__ float awq_f32<float>(float v) {
  return v;
}

// Thread: CPT consecutive channels (one 16-byte vector per row when `vec`).
template <typename T, bool VEC>
__global__ __launch_bounds__(kAwqThreads) void awq_stats_kernel(const T* __restrict__ X, int64_t ldx,
                                                                int64_t tokens, int64_t n,
                                                                int64_t rows_per_slice,
                                                                double* __restrict__ part) {
  constexpr int CPT = 16 / (int)sizeof(T);
  const int64_t c0 = ((int64_t)blockIdx.x * kAwqThreads + threadIdx.x) * CPT;
  const int64_t s = blockIdx.y;
  const int64_t t0 = s * rows_per_slice, t1 = std::min<int64_t>(tokens, t0 + rows_per_slice);
  if (c0 >= n) return;
  double acc[CPT];
#pragma unroll
  for (int e = 0; e < CPT; ++e) acc[e] = 0.0;
  if (VEC && c0 + CPT <= n) {
    int64_t t = t0;
    for (; t + 4 <= t1; t += 4) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const uint4*>(X + (t + u) * ldx + c0);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const T* e8 = reinterpret_cast<const T*>(&v[u]);
#pragma unroll
        for (int e = 0; e < CPT; ++e) acc[e] += (double)fabsf(awq_f32<T>(e8[e]));
      }
    }
    for (; t < t1; ++t) {
      const uint4 v = *reinterpret_cast<const uint4*>(X + t * ldx + c0);
      const T* e8 = reinterpret_cast<const T*>(&v);
#pragma unroll
      for (int e = 0; e < CPT; ++e) acc[e] += (double)fabsf(awq_f32<T>(e8[e]));
    }
  } else {
    for (int64_t t = t0; t < t1; ++t)
#pragma unroll
      for (int e = 0; e < CPT; ++e)
        if (c0 + e < n) acc[e] += (double)fabsf(awq_f32<T>(X[t * ldx + c0 + e]));
  }
#pragma unroll
  for (int e = 0; e < CPT; ++e)
    if (c0 + e < n) part[s * n + c0 + e] = acc[e];
}

__global__ __launch_bounds__(kAwqThreads) void awq_stats_reduce_kernel(const double* __restrict__ part,
                                                                       int64_t slices, int64_t n,
                                                                       double* __restrict__ abs_sum) {
  const int64_t c = (int64_t)blockIdx.x * kAwqThreads + threadIdx.x;
  if (c >= n) return;
  double acc = abs_sum[c];
  for (int64_t s = 0; s < slices; ++s) acc += part[s * n + c];
  abs_sum[c] = acc;
}

__device__ __forceinline__ uint64_t d2u(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  return b ^ ((b >> 63) ? ~0ull : 0x8000000000000000ull);
}

// One workgroup of 1024.  Each radix pass counts the keys that match the
// selected prefix into 256 bins, each wave into a histogram of its own (the
// first passes see nearly every key in one bin: one shared histogram would
// serialise 11008 atomics on one address), and a wave whose matching keys
// all fall in one bin adds their count with one atomic; threads 0..255 (one
// bin each) sum the 16 histograms and take an inclusive scan (a 64-lane
// shuffle scan per wave, then the wave totals), and the one thread whose bin
// holds the remaining rank extends the prefix.  REG: the keys (n <= 1024·kAwqKeys) are computed once and held in
// registers, kAwqKeys per thread, for all eight passes; otherwise every
// pass recomputes them from abs_sum.
constexpr int kAwqKeys = 16;
template <bool REG>
__global__ __launch_bounds__(1024) void awq_scale_kernel(const double* __restrict__ abs_sum, int64_t n,
                                                         double tokens, float protect,
                                                         float* __restrict__ channel_scale, int* flag) {
  __shared__ uint32_t hist[16][256];   // per wave
  __shared__ uint32_t wtot[4];
  __shared__ uint64_t sel[2];   // prefix, remaining rank
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // this thread's keys j = tid + 1024·i (REG); past n they are ~0, which no
  // prefix of a finite key's matches before the last pass and which the
  // count skips by index
  uint64_t key[REG ? kAwqKeys : 1];
  bool bad = false;
  if constexpr (REG) {
    double v[kAwqKeys];
#pragma unroll
    for (int i = 0; i < kAwqKeys; ++i) v[i] = abs_sum[std::min<int64_t>(tid + 1024 * i, n - 1)];
#pragma unroll
    for (int i = 0; i < kAwqKeys; ++i) {
      bad |= !isfinite(v[i]);
      key[i] = d2u(v[i] / tokens);
    }
  } else {
    for (int64_t j = tid; j < n; j += 1024) bad |= !isfinite(abs_sum[j]);
  }
  // the call's flag word: this single workgroup is its only writer
  const int any_bad = __syncthreads_or(bad);
  if (tid == 0) *flag = any_bad;
  if (any_bad) return;
  if (tid == 0) {
    sel[0] = 0;
    sel[1] = (uint64_t)((n - 1) / 2);   // rank of the lower median
  }
  uint64_t mask = 0;
  for (int shift = 56; shift >= 0; shift -= 8) {
#pragma unroll
    for (int q = 0; q < 4; ++q) hist[q * 4 + (tid >> 8)][tid & 255] = 0;
    __syncthreads();
    const uint64_t prefix = sel[0], rem = sel[1];
    uint32_t* hw = hist[wave];
    // count key k if it matches the prefix (act); a wave whose active keys
    // share one bin adds their number at once
    auto count = [&](bool act, uint64_t k) {
      const uint32_t b = (uint32_t)(k >> shift) & 255u;
      const uint64_t am = __ballot(act);
      if (am == 0) return;
      const int first = __builtin_ctzll(am);
      const uint32_t bf = (uint32_t)__shfl((int)b, first, 64);
      if (__ballot(act && b != bf) == 0) {
        if (lane == first) atomicAdd(&hw[bf], (uint32_t)__popcll(am));
      } else if (act) {
        atomicAdd(&hw[b], 1u);
      }
    };
    if constexpr (REG) {
#pragma unroll
      for (int i = 0; i < kAwqKeys; ++i) count(tid + 1024 * i < n && (key[i] & mask) == prefix, key[i]);
    } else {
      for (int64_t j0 = 0; j0 < n; j0 += 1024) {
        const int64_t j = j0 + tid;
        const uint64_t k = j < n ? d2u(abs_sum[j] / tokens) : 0;
        count(j < n && (k & mask) == prefix, k);
      }
    }
    __syncthreads();
    uint32_t v = 0, x = 0;
    if (tid < 256) {
#pragma unroll
      for (int w = 0; w < 16; ++w) v += hist[w][tid];
      x = v;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
      }
      if (lane == 63) wtot[wave] = x;
    }
    __syncthreads();
    if (tid < 256) {
      uint32_t off = 0;
      for (int w = 0; w < wave; ++w) off += wtot[w];
      const uint64_t incl = (uint64_t)(x + off), excl = incl - v;
      if (excl <= rem && rem < incl) {   // exactly one bin (empty bins have excl == incl)
        sel[0] = prefix | ((uint64_t)tid << shift);
        sel[1] = rem - excl;
      }
    }
    mask |= 255ull << shift;
    __syncthreads();
  }
  const uint64_t med = sel[0];
  if constexpr (REG) {
#pragma unroll
    for (int i = 0; i < kAwqKeys; ++i)
      if (tid + 1024 * i < n) channel_scale[tid + 1024 * i] = key[i] > med ? protect : 1.f;
  } else {
    for (int64_t j = tid; j < n; j += 1024)
      channel_scale[j] = d2u(abs_sum[j] / tokens) > med ? protect : 1.f;
  }
}

}  // namespace

AwqStatsPlan plan_awq_stats(int64_t n, int64_t tokens) {
  AwqStatsPlan p;
  const int64_t colblocks = ceil_div(std::max<int64_t>(n, 1), kAwqThreads * 8);
  // ~1024 workgroups, at least 64 rows each
  p.slices = std::max<int64_t>(1, std::min<int64_t>(ceil_div(1024, colblocks), ceil_div(tokens, 64)));
  p.rows_per_slice = ceil_div(std::max<int64_t>(tokens, 1), p.slices);
  p.slices = ceil_div(std::max<int64_t>(tokens, 1), p.rows_per_slice);
  p.total = align256((size_t)(p.slices * n) * sizeof(double));
  return p;
}

gptq_status run_awq_stats(const void* X, int x_dtype, int64_t tokens, int64_t ldx, int64_t n,
                          double* abs_sum, void* ws, const AwqStatsPlan& p, hipStream_t stream) {
  double* part = static_cast<double*>(ws);
  const size_t esz = x_dtype == GPTQ_BF16 ? 2 : 4;
  const bool vec = ((uintptr_t)X % 16 == 0) && ((ldx * (int64_t)esz) % 16 == 0);
  const int cpt = (int)(16 / esz);
  const dim3 grid((unsigned)ceil_div(n, (int64_t)kAwqThreads * cpt), (unsigned)p.slices);
  if (x_dtype == GPTQ_BF16) {
    const uint16_t* x = static_cast<const uint16_t*>(X);
    if (vec)
      hipLaunchKernelGGL((awq_stats_kernel<uint16_t, true>), grid, dim3(kAwqThreads), 0, stream, x, ldx,
                         tokens, n, p.rows_per_slice, part);
    else
      hipLaunchKernelGGL((awq_stats_kernel<uint16_t, false>), grid, dim3(kAwqThreads), 0, stream, x, ldx,
                         tokens, n, p.rows_per_slice, part);
  } else {
    const float* x = static_cast<const float*>(X);
    if (vec)
      hipLaunchKernelGGL((awq_stats_kernel<float, true>), grid, dim3(kAwqThreads), 0, stream, x, ldx,
                         tokens, n, p.rows_per_slice, part);
    else
      hipLaunchKernelGGL((awq_stats_kernel<float, false>), grid, dim3(kAwqThreads), 0, stream, x, ldx,
                         tokens, n, p.rows_per_slice, part);
  }
  GPTQ_LAUNCH_CHECK();
  hipLaunchKernelGGL(awq_stats_reduce_kernel, dim3((unsigned)ceil_div(n, kAwqThreads)), dim3(kAwqThreads),
                     0, stream, (const double*)part, p.slices, n, abs_sum);
  GPTQ_LAUNCH_CHECK();
  return GPTQ_OK;
}

size_t awq_extra_bytes() { return 256; }

gptq_status run_awq_quantize(const void* W, int w_dtype, int64_t m, int64_t n, const double* abs_sum,
                             int64_t tokens, float protect, int bits, int sym, float clip,
                             uint32_t* qweight, float* scales, int32_t* zeros, float* channel_scale,
                             double* err, int32_t* status, void* ws, const RtnPlan& plan, hipStream_t stream) {
  int* flag = static_cast<int*>(ws);
  if (n <= 1024 * kAwqKeys)
    hipLaunchKernelGGL(awq_scale_kernel<true>, dim3(1), dim3(1024), 0, stream, abs_sum, n, (double)tokens,
                       protect, channel_scale, flag);
  else
    hipLaunchKernelGGL(awq_scale_kernel<false>, dim3(1), dim3(1024), 0, stream, abs_sum, n, (double)tokens,
                       protect, channel_scale, flag);
  GPTQ_LAUNCH_CHECK();
  return run_rtn(W, w_dtype, m, n, bits, sym, clip, qweight, scales, zeros, err, status,
                 static_cast<char*>(ws) + awq_extra_bytes(), plan, stream, channel_scale, flag);
}

}  // namespace gptq
