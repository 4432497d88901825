// The linear (round-to-nearest) quantizer: per-row or per-group affine grids
// with clip-ratio percentile clipping, no error feedback.
//
// Page "模型量化实战：从 INT8 PTQ 到 GPTQ 的精度保持与推理加速全解析" §2.1 (the
// affine formula) and §3.1 (the LinearQuantizer): symmetric scale =
// percentile(|w|, c) / (2^(b-1) - 1) and codes round(w/scale) in
// [-2^(b-1), 2^(b-1) - 1]; asymmetric scale = (hi - lo) / (2^b - 1) with lo, hi
// the (1-c)/2 and 1-(1-c)/2 percentiles, zero = -round(lo/scale), codes
// round(w/scale + zero) in [0, 2^b - 1]; scale floor 1e-8; the MSE and cosine
// similarity of the dequantized weights.  "Per channel" is one grid per
// output row; a group is g consecutive columns of a row.  Percentiles
// interpolate linearly between order statistics at position f·(N-1).
//
// One workgroup of 512 threads per output row:
//   1. the row's sort keys (|w| or w) go to LDS, each group padded to a power
//      of two P with +inf;
//   2. every P-segment is bitonic-sorted in place (the network only pairs
//      indices inside a segment, and the direction follows the index within
//      the segment, so all segments end ascending);
//   3. one thread per group reads its order statistics and forms the grid in
//      fp64 (the same operations, in the same order, as the float64
//      definition: no contraction into fused multiply-adds);
//   4. the row is read again, coded in fp64, packed (the GPTQ path's layout)
//      and its squared error, dot product and norms are summed in fp64.
// A second kernel reduces the per-row sums in a fixed order.
#include <algorithm>

#include "gptq_internal.hpp"

namespace gptq {
namespace {

constexpr int kRtnThreads = 512;
constexpr int kFlagNonFinite = 1;

template <typename T>
__device__ __forceinline__ float rtn_f32(T x);
template <>
__device__ __forceinline__ float rtn_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ float rtn_f32<uint16_t>(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

struct RtnArgs {
  const void* W;
  int64_t m, n;
  int bits, sym;
  int64_t g, G, P;   // group width, groups per row, padded segment length
  float clip;
  uint32_t* qweight;
  int64_t words;
  float* scales;
  int32_t* zeros;
  double* part;      // [m][4]: Σ(w-ŵ)², Σwŵ, Σw², Σŵ²
  int* flag;
};

#pragma clang fp contract(off)
// a[0..L-1] ascending; linear interpolation at position f·(L-1)
__device__ double rtn_percentile(const float* a, int64_t L, double f) {
  const double p = f * (double)(L - 1);
  const double fl = floor(p);
  const int64_t i = (int64_t)fl;
  if (i >= L - 1) return (double)a[L - 1];
  const double t = p - fl;
  const double lo = (double)a[i], hi = (double)a[i + 1];
  return lo + (hi - lo) * t;
}

__device__ void rtn_grid(const float* a, int64_t L, int bits, int sym, float clip, double& scale,
                         double& zp) {
  const double c = (double)clip;
  if (sym) {
    const double qmax = (double)((1 << (bits - 1)) - 1);
    const double amax = rtn_percentile(a, L, c < 1.0 ? c : 1.0);   // a = sorted |w|
    scale = fmax(amax / qmax, 1e-8);
    zp = 0.0;
  } else {
    const double qmax = (double)((1 << bits) - 1);
    double lo, hi;
    if (c < 1.0) {
      const double f = (1.0 - c) / 2.0;
      lo = rtn_percentile(a, L, f);
      hi = rtn_percentile(a, L, 1.0 - f);
    } else {
      lo = (double)a[0];
      hi = (double)a[L - 1];
    }
    scale = fmax((hi - lo) / qmax, 1e-8);
    zp = 0.0 - rint(lo / scale);
  }
}
#pragma clang fp contract(on)

template <typename T>
__global__ __launch_bounds__(kRtnThreads) void rtn_row_kernel(RtnArgs a) {
  extern __shared__ __attribute__((aligned(16))) float keys[];   // [G*P], then the grids
  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x;
  const T* w = static_cast<const T*>(a.W) + r * a.n;
  const int64_t total = a.G * a.P;
  double* gsc = reinterpret_cast<double*>(keys + ((total + 3) & ~int64_t(3)));   // [G] scale
  double* gzp = gsc + a.G;                                  // [G] zero point
  bool bad = false;

  for (int64_t i = tid; i < total; i += kRtnThreads) {
    const int64_t j = i / a.P, pos = i - j * a.P, c = j * a.g + pos;
    float key = __builtin_huge_valf();
    if (pos < a.g && c < a.n) {
      const float x = rtn_f32<T>(w[c]);
      bad |= !isfinite(x);
      key = a.sym ? fabsf(x) : x;
    }
    keys[i] = key;
  }
  __syncthreads();
  for (int64_t k = 2; k <= a.P; k <<= 1) {
    for (int64_t j = k >> 1; j > 0; j >>= 1) {
      for (int64_t i = tid; i < total; i += kRtnThreads) {
        const int64_t ixj = i ^ j;
        if (ixj > i) {
          const bool up = ((i & (a.P - 1)) & k) == 0;
          const float x = keys[i], y = keys[ixj];
          if ((x > y) == up) {
            keys[i] = y;
            keys[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int64_t j = tid; j < a.G; j += kRtnThreads) {
    const int64_t L = (a.n - j * a.g < a.g) ? a.n - j * a.g : a.g;
    double s, z;
    rtn_grid(keys + j * a.P, L, a.bits, a.sym, a.clip, s, z);
    gsc[j] = s;
    gzp[j] = z;
  }
  __syncthreads();

  const int off = a.sym ? (1 << (a.bits - 1)) : 0;
  const double qmin = a.sym ? -(double)(1 << (a.bits - 1)) : 0.0;
  const double qmax = a.sym ? (double)((1 << (a.bits - 1)) - 1) : (double)((1 << a.bits) - 1);
  double se = 0.0, dot = 0.0, ww = 0.0, dd = 0.0;
  uint32_t* qrow = a.qweight + r * a.words;
  for (int64_t c8 = tid; c8 * 8 < a.n; c8 += kRtnThreads) {
    uint32_t word0 = 0u, word1 = 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t c = c8 * 8 + e;
      if (c >= a.n) break;
      const double x = (double)rtn_f32<T>(w[c]);
      const int64_t j = c / a.g;
      const double s = gsc[j], z = gzp[j];
      double q = a.sym ? rint(x / s) : rint(x / s + z);
      q = fmin(fmax(q, qmin), qmax);
      const uint32_t code = (uint32_t)((int)q + off);
      const double dq = (q - z) * s;
      const double d = x - dq;
      se += d * d;
      dot += x * dq;
      ww += x * x;
      dd += dq * dq;
      if (a.bits <= 4) {
        word0 |= code << (4 * e);
      } else if (e < 4) {
        word0 |= code << (8 * e);
      } else {
        word1 |= code << (8 * (e - 4));
      }
    }
    if (a.bits <= 4) {
      qrow[c8] = word0;
    } else {
      qrow[2 * c8] = word0;
      if (2 * c8 + 1 < a.words) qrow[2 * c8 + 1] = word1;
    }
  }
  for (int64_t j = tid; j < a.G; j += kRtnThreads) {
    a.scales[r * a.G + j] = (float)gsc[j];
    a.zeros[r * a.G + j] = (int32_t)gzp[j] + off;
  }
  if (bad) atomicOr(a.flag, kFlagNonFinite);

  // row sums: wave butterflies, then the 8 waves in order
  __shared__ double red[4][kRtnThreads / 64];
  double v[4] = {se, dot, ww, dd};
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v[q] += __shfl_xor(v[q], d, 64);
  if ((tid & 63) == 0)
#pragma unroll
    for (int q = 0; q < 4; ++q) red[q][tid >> 6] = v[q];
  __syncthreads();
  if (tid < 4) {
    double s = 0.0;
    for (int wv = 0; wv < kRtnThreads / 64; ++wv) s += red[tid][wv];
    a.part[r * 4 + tid] = s;
  }
}

// err[0] = Σse / (m·n), err[1] = Σdot / (sqrt(Σww)·sqrt(Σdd) + 1e-8); rows in a
// fixed order (thread t sums rows t, t+1024, ...; then a fixed tree).
__global__ __launch_bounds__(1024) void rtn_reduce_kernel(const double* __restrict__ part, int64_t m,
                                                          int64_t count, double* __restrict__ err) {
  __shared__ double sh[4][1024];
  const int tid = threadIdx.x;
  double v[4] = {0.0, 0.0, 0.0, 0.0};
  for (int64_t r = tid; r < m; r += 1024)
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] += part[r * 4 + q];
#pragma unroll
  for (int q = 0; q < 4; ++q) sh[q][tid] = v[q];
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if (tid < s)
#pragma unroll
      for (int q = 0; q < 4; ++q) sh[q][tid] += sh[q][tid + s];
    __syncthreads();
  }
  if (tid == 0) {
    err[0] = sh[0][0] / (double)count;
    err[1] = sh[1][0] / (sqrt(sh[2][0]) * sqrt(sh[3][0]) + 1e-8);
  }
}

}  // namespace

RtnPlan plan_rtn(int64_t m, int64_t n, int32_t group_size) {
  RtnPlan p;
  p.g = (group_size == -1 || group_size >= n) ? std::max<int64_t>(n, 1) : group_size;
  p.G = ceil_div(std::max<int64_t>(n, 1), p.g);
  p.P = 1;
  while (p.P < p.g) p.P <<= 1;
  p.lds_bytes = (size_t)((p.G * p.P + 3) & ~int64_t(3)) * sizeof(float) + (size_t)p.G * 2 * sizeof(double);
  p.part_off = 0;
  p.flag_off = align256((size_t)std::max<int64_t>(m, 1) * 4 * sizeof(double));
  p.total = p.flag_off + 256;
  return p;
}

gptq_status run_rtn(const void* W, int w_dtype, int64_t m, int64_t n, int bits, int sym, float clip,
                    uint32_t* qweight, float* scales, int32_t* zeros, double* err, void* ws,
                    const RtnPlan& p, hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  RtnArgs a;
  a.W = W; a.m = m; a.n = n; a.bits = bits; a.sym = sym;
  a.g = p.g; a.G = p.G; a.P = p.P; a.clip = clip;
  a.qweight = qweight; a.words = gptq_qweight_words(n, bits);
  a.scales = scales; a.zeros = zeros;
  a.part = reinterpret_cast<double*>(w + p.part_off);
  a.flag = reinterpret_cast<int*>(w + p.flag_off);
  GPTQ_HIP_CHECK(hipMemsetAsync(a.flag, 0, sizeof(int), stream));
  const int lds = (int)p.lds_bytes;
  if (w_dtype == GPTQ_BF16) {
    if (lds > 65536)
      GPTQ_HIP_CHECK(hipFuncSetAttribute((const void*)rtn_row_kernel<uint16_t>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, lds));
    hipLaunchKernelGGL(rtn_row_kernel<uint16_t>, dim3((unsigned)m), dim3(kRtnThreads), lds, stream, a);
  } else {
    if (lds > 65536)
      GPTQ_HIP_CHECK(hipFuncSetAttribute((const void*)rtn_row_kernel<float>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, lds));
    hipLaunchKernelGGL(rtn_row_kernel<float>, dim3((unsigned)m), dim3(kRtnThreads), lds, stream, a);
  }
  GPTQ_LAUNCH_CHECK();
  hipLaunchKernelGGL(rtn_reduce_kernel, dim3(1), dim3(1024), 0, stream, (const double*)a.part, m, m * n,
                     err);
  GPTQ_LAUNCH_CHECK();
  int hflag = 0;
  GPTQ_HIP_CHECK(hipMemcpyAsync(&hflag, a.flag, sizeof(int), hipMemcpyDeviceToHost, stream));
  GPTQ_HIP_CHECK(hipStreamSynchronize(stream));
  if (hflag & kFlagNonFinite) {
    set_error("gptq_rtn_quantize: W holds a NaN or Inf");
    return GPTQ_ERR_NONFINITE;
  }
  return GPTQ_OK;
}

}  // namespace gptq
