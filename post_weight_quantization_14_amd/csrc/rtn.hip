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
//   1. the row's keys (|w| or w, as order-preserving uint32) go to LDS, each
//      group padded to a power of two P with the largest key;
//   2. the order statistics each percentile needs: for one group per row, the
//      extremes by a block reduction, or ranks floor(p) and floor(p)+1 by
//      four 8-bit radix-select passes; for groups, a bitonic sort of every
//      P-segment in place when clipping (the network only pairs indices
//      inside a segment and takes its direction from the index within the
//      segment, so all segments end ascending), else a scan per group;
//   3. the grid in fp64 from those values, with the same operations in the
//      same order as the float64 definition (no fused multiply-adds);
//   4. the row is read again, coded in fp64, packed (the GPTQ path's layout)
//      and its squared error, dot product and norms are summed in fp64.
// A second kernel reduces the per-row sums in a fixed order.
#include <algorithm>

#include "gptq_internal.hpp"

namespace gptq {
namespace {

constexpr int kRtnThreads = 512;

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
  int* badrow;       // [m]: 1 if the row holds a NaN or Inf (every row writes its own)
  const float* colscale;   // per input column, or null: quantize fl(w·colscale), errors against w
};

// Order-preserving map of a float to uint32 (and back): unsigned order of the
// codes is the numeric order (-0 just below +0).
__device__ __forceinline__ uint32_t f2u(float x) {
  const uint32_t b = __float_as_uint(x);
  return b ^ ((b & 0x80000000u) ? 0xffffffffu : 0x80000000u);
}
__device__ __forceinline__ float u2f(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u ^ 0x80000000u) : ~u);
}

#pragma clang fp contract(off)
// Linear interpolation between the order statistics v_i <= v_i1 (ranks i and
// i+1 of L values) at position p = f·(L-1), i = floor(p).
__device__ double rtn_lerp(float vi, float vi1, double p) {
  const double t = p - floor(p);
  const double lo = (double)vi, hi = (double)vi1;
  return lo + (hi - lo) * t;
}

__device__ void rtn_grid(double lo, double hi, int bits, int sym, double& scale, double& zp) {
  if (sym) {   // hi = the clipped max|w|
    scale = fmax(hi / (double)((1 << (bits - 1)) - 1), 1e-8);
    zp = 0.0;
  } else {
    scale = fmax((hi - lo) / (double)((1 << bits) - 1), 1e-8);
    zp = 0.0 - rint(lo / scale);
  }
}
#pragma clang fp contract(on)

// Positions of the percentiles of one group of L values: sym uses f = c on
// |w|; asym f = (1-c)/2 and 1-(1-c)/2 on w (c = 1: the extremes).
struct RtnRanks {
  double p[2];   // positions (lo, hi); sym: only p[1]
  int r[2];      // floor of each position
};
__device__ __forceinline__ RtnRanks rtn_ranks(int L, int sym, float clip) {
  RtnRanks k;
  const double c = (double)clip;
  const double f = (1.0 - c) / 2.0;
  const double flo = sym ? 0.0 : (c < 1.0 ? f : 0.0);
  const double fhi = sym ? (c < 1.0 ? c : 1.0) : (c < 1.0 ? 1.0 - f : 1.0);
  k.p[0] = flo * (double)(L - 1);
  k.p[1] = fhi * (double)(L - 1);
  k.r[0] = (int)floor(k.p[0]);
  k.r[1] = (int)floor(k.p[1]);
  return k;
}

constexpr int kWaves = kRtnThreads / 64;

// The k-th smallest (0-based) of L uint32 keys in LDS, by four 8-bit radix
// passes; each wave counts into its own 256-bin histogram (hist[8][256]) and
// wave 0 adds them while it scans.  The whole workgroup calls it.
__device__ uint32_t block_select(const uint32_t* keys, int L, int k, uint32_t* hist, int* bc) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t prefix = 0u, mask = 0u;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = tid; b < kWaves * 256; b += kRtnThreads) hist[b] = 0u;
    __syncthreads();
    uint32_t* hw = hist + wave * 256;
    for (int i = tid; i < L; i += kRtnThreads) {
      const uint32_t u = keys[i];
      if ((u & mask) == prefix) atomicAdd(&hw[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      uint32_t c[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int wv = 0; wv < kWaves; ++wv)
#pragma unroll
        for (int q = 0; q < 4; ++q) c[q] += hist[wv * 256 + 4 * lane + q];
      const uint32_t s = c[0] + c[1] + c[2] + c[3];
      uint32_t inc = s;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_up(inc, d, 64);
        if (lane >= d) inc += o;
      }
      const uint32_t before = inc - s, kk = (uint32_t)k;
      if (before <= kk && kk < inc) {
        uint32_t rem = kk - before, bin = 4 * lane;
        if (rem >= c[0]) { rem -= c[0]; ++bin;
          if (rem >= c[1]) { rem -= c[1]; ++bin;
            if (rem >= c[2]) { rem -= c[2]; ++bin; } } }
        bc[0] = (int)bin;
        bc[1] = (int)rem;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)bc[0] << shift;
    mask |= 0xffu << shift;
    k = bc[1];
    __syncthreads();   // bc and hist are rewritten by the next pass
  }
  return prefix;
}

// Given v = the key of rank r, the key of rank r+1 (r+1 < L): v itself when
// more than r+1 keys are <= v, else the smallest key above v.
__device__ uint32_t block_next(const uint32_t* keys, int L, int r, uint32_t v, uint32_t* red) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t cnt = 0u, mn = 0xffffffffu;
  for (int i = tid; i < L; i += kRtnThreads) {
    const uint32_t u = keys[i];
    if (u <= v) ++cnt;
    else mn = min(mn, u);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    cnt += (uint32_t)__shfl_xor(cnt, d, 64);
    mn = min(mn, (uint32_t)__shfl_xor(mn, d, 64));
  }
  if (lane == 0) { red[wave] = cnt; red[kWaves + wave] = mn; }
  __syncthreads();
  uint32_t c = 0u, m = 0xffffffffu;
  for (int wv = 0; wv < kWaves; ++wv) { c += red[wv]; m = min(m, red[kWaves + wv]); }
  __syncthreads();   // red is reused
  return c >= (uint32_t)(r + 2) ? v : m;
}

// Keys of ranks r and r+1 (0-based, r+1 clamped to L-1) of one group of L
// keys, by one wave: distinct values are peeled from the nearer end (the
// next minimum above, or maximum below, the last one, with its count) until
// both ranks are covered.
__device__ void wave_select2(const uint32_t* seg, int L, int r, uint32_t& va, uint32_t& vb);

// Wave-wide reductions of uint32
__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x = min(x, (uint32_t)__shfl_xor(x, d, 64));
  return x;
}
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x = max(x, (uint32_t)__shfl_xor(x, d, 64));
  return x;
}

__device__ void wave_select2(const uint32_t* seg, int L, int r, uint32_t& va, uint32_t& vb) {
  const int lane = threadIdx.x & 63;
  const int r1 = min(r + 1, L - 1);
  const bool top = r >= L / 2;
  bool ga = false, gb = false;
  uint32_t prev = 0u;
  int done = 0;   // keys already peeled (from the chosen end)
  for (int it = 0; it < L && !(ga && gb); ++it) {
    uint32_t m = top ? 0u : 0xffffffffu;
    for (int i = lane; i < L; i += 64) {
      const uint32_t u = seg[i];
      if (top) { if (it == 0 || u < prev) m = max(m, u); }
      else     { if (it == 0 || u > prev) m = min(m, u); }
    }
    m = top ? wave_max(m) : wave_min(m);
    int c = 0;
    for (int i = lane; i < L; i += 64) c += seg[i] == m;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) c += __shfl_xor(c, d, 64);
    // ranks held by m: [done, done + c) from the bottom, or from the top
    const int lo = top ? L - done - c : done, hi = top ? L - done : done + c;
    if (!ga && r >= lo && r < hi) { va = m; ga = true; }
    if (!gb && r1 >= lo && r1 < hi) { vb = m; gb = true; }
    done += c;
    prev = m;
  }
}

template <typename T>
__global__ __launch_bounds__(kRtnThreads) void rtn_row_kernel(RtnArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t keys[];   // [G*P], the grids, then hist
  __shared__ int bc[2];
  __shared__ uint32_t red_u[2][kRtnThreads / 64];
  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x;
  const int n = (int)a.n, g = (int)a.g, G = (int)a.G, P = (int)a.P;
  const int lgP = 31 - __builtin_clz(P);
  const T* w = static_cast<const T*>(a.W) + r * a.n;
  const int total = G * P;
  double* gsc = reinterpret_cast<double*>(keys + ((total + 3) & ~3));   // [G] scale
  double* gzp = gsc + G;                                                 // [G] zero point
  uint32_t* hist = reinterpret_cast<uint32_t*>(gzp + G);                 // [8][256], one group per row
  const bool clipped = a.clip < 1.f;
  bool bad = false;

  // 1. order-preserving keys of |w| (sym) or w (asym); padding sorts last
  uint32_t tmin = 0xffffffffu, tmax = 0u;
  for (int i = tid; i < total; i += kRtnThreads) {
    const int j = i >> lgP, pos = i & (P - 1), c = j * g + pos;
    uint32_t key = 0xffffffffu;
    if (pos < g && c < n) {
      float x = rtn_f32<T>(w[c]);
      if (a.colscale) x *= a.colscale[c];
      bad |= !isfinite(x);
      key = f2u(a.sym ? fabsf(x) : x);
      tmin = min(tmin, key);
      tmax = max(tmax, key);
    }
    keys[i] = key;
  }
  __syncthreads();

  if (G == 1) {
    // 2a. one group per row: the extremes by a block reduction, or each
    // needed order statistic by radix selection
    const RtnRanks rk = rtn_ranks(n, a.sym, a.clip);
    float lo0 = 0.f, lo1 = 0.f, hi0, hi1;   // values at ranks floor(p), floor(p)+1
    if (!clipped) {
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) {
        tmin = min(tmin, (uint32_t)__shfl_xor(tmin, d, 64));
        tmax = max(tmax, (uint32_t)__shfl_xor(tmax, d, 64));
      }
      if ((tid & 63) == 0) { red_u[0][tid >> 6] = tmin; red_u[1][tid >> 6] = tmax; }
      __syncthreads();
      uint32_t mn = red_u[0][0], mx = red_u[1][0];
      for (int wv = 1; wv < kRtnThreads / 64; ++wv) { mn = min(mn, red_u[0][wv]); mx = max(mx, red_u[1][wv]); }
      lo0 = lo1 = u2f(mn);
      hi0 = hi1 = u2f(mx);
    } else {
      if (!a.sym) {
        const uint32_t u = block_select(keys, n, rk.r[0], hist, bc);
        lo0 = u2f(u);
        lo1 = rk.r[0] + 1 < n ? u2f(block_next(keys, n, rk.r[0], u, &red_u[0][0])) : lo0;
      }
      const uint32_t u = block_select(keys, n, rk.r[1], hist, bc);
      hi0 = u2f(u);
      hi1 = rk.r[1] + 1 < n ? u2f(block_next(keys, n, rk.r[1], u, &red_u[0][0])) : hi0;
    }
    if (tid == 0) {
      // unclipped: the extremes themselves; clipped: interpolate unless the
      // position is the last rank
      const double lo = (!clipped || rk.r[0] >= n - 1) ? (double)lo0 : rtn_lerp(lo0, lo1, rk.p[0]);
      const double hi = (!clipped || rk.r[1] >= n - 1) ? (double)hi0 : rtn_lerp(hi0, hi1, rk.p[1]);
      double s_, z_;
      rtn_grid(lo, hi, a.bits, a.sym, s_, z_);
      gsc[0] = s_;
      gzp[0] = z_;
    }
  } else {
    // 2b. groups.  Up to 256 columns: one wave per group -- the extremes by
    // a wave reduction, or the needed ranks by counting (rank of an element =
    // keys below it, ties broken by position; every rank is held by exactly
    // one element) and a wave max over the element holding each rank.
    // Wider groups: bitonic sort of every P-segment, then one thread each.
    const int lane = tid & 63, wave = tid >> 6;
    if (P <= 256) {
      for (int j = wave; j < G; j += kWaves) {
        const int L = (n - j * g < g) ? n - j * g : g;
        const uint32_t* seg = keys + j * P;
        double lo, hi;
        if (!clipped) {
          uint32_t mn = 0xffffffffu, mx = 0u;
          for (int i = lane; i < L; i += 64) { mn = min(mn, seg[i]); mx = max(mx, seg[i]); }
          lo = (double)u2f(wave_min(mn));
          hi = (double)u2f(wave_max(mx));
        } else {
          const RtnRanks rk = rtn_ranks(L, a.sym, a.clip);
          uint32_t v0 = 0u, v1 = 0u, v2 = 0u, v3 = 0u;
          if (!a.sym) wave_select2(seg, L, rk.r[0], v0, v1);
          wave_select2(seg, L, rk.r[1], v2, v3);
          lo = (rk.r[0] >= L - 1) ? (double)u2f(v0) : rtn_lerp(u2f(v0), u2f(v1), rk.p[0]);
          hi = (rk.r[1] >= L - 1) ? (double)u2f(v2) : rtn_lerp(u2f(v2), u2f(v3), rk.p[1]);
        }
        if (lane == 0) {
          double s_, z_;
          rtn_grid(lo, hi, a.bits, a.sym, s_, z_);
          gsc[j] = s_;
          gzp[j] = z_;
        }
      }
    } else {
      if (clipped) {
        for (int k = 2; k <= P; k <<= 1) {
          for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < total; i += kRtnThreads) {
              const int ixj = i ^ j;
              if (ixj > i) {
                const bool up = ((i & (P - 1)) & k) == 0;
                const uint32_t x = keys[i], y = keys[ixj];
                if ((x > y) == up) {
                  keys[i] = y;
                  keys[ixj] = x;
                }
              }
            }
            __syncthreads();
          }
        }
      }
      for (int j = wave; j < G; j += kWaves) {
        const int L = (n - j * g < g) ? n - j * g : g;
        const uint32_t* seg = keys + j * P;
        double lo, hi;
        if (clipped) {
          const RtnRanks rk = rtn_ranks(L, a.sym, a.clip);
          lo = (rk.r[0] >= L - 1) ? (double)u2f(seg[L - 1]) : rtn_lerp(u2f(seg[rk.r[0]]), u2f(seg[rk.r[0] + 1]), rk.p[0]);
          hi = (rk.r[1] >= L - 1) ? (double)u2f(seg[L - 1]) : rtn_lerp(u2f(seg[rk.r[1]]), u2f(seg[rk.r[1] + 1]), rk.p[1]);
        } else {
          uint32_t mn = 0xffffffffu, mx = 0u;
          for (int i = lane; i < L; i += 64) { mn = min(mn, seg[i]); mx = max(mx, seg[i]); }
          lo = (double)u2f(wave_min(mn));
          hi = (double)u2f(wave_max(mx));
        }
        if (lane == 0) {
          double s_, z_;
          rtn_grid(lo, hi, a.bits, a.sym, s_, z_);
          gsc[j] = s_;
          gzp[j] = z_;
        }
      }
    }
  }
  __syncthreads();

  // 3. codes, packing and the row's error sums.  The code is rint(x/s) or
  // rint(x/s + z) of the fp64 quotient.  An fp32 quotient y (correctly
  // rounded division by the fp32-rounded scale, then + z) is within
  // 2e-7·(|x/s| + |y|) of it, so wherever y is farther than that from a
  // half-integer both round the same way; only the rest is recomputed in fp64.
  // The error sums keep Σd², Σx·d and Σx² (d = x - ŵ) in fp64; Σx·ŵ and Σŵ²
  // follow from them.
  const int off = a.sym ? (1 << (a.bits - 1)) : 0;
  const float qminf = a.sym ? -(float)(1 << (a.bits - 1)) : 0.f;
  const float qmaxf = a.sym ? (float)((1 << (a.bits - 1)) - 1) : (float)((1 << a.bits) - 1);
  double se = 0.0, xd = 0.0, ww = 0.0;
  uint32_t* qrow = a.qweight + r * a.words;
  for (int c8 = tid; c8 * 8 < n; c8 += kRtnThreads) {
    uint32_t word0 = 0u, word1 = 0u;
    int j = (c8 * 8) / g, jend = (j + 1) * g;
    double s = gsc[j], z = gzp[j];
    float sf = (float)s, zf = (float)z;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = c8 * 8 + e;
      if (c >= n) break;
      if (c >= jend) {
        while (c >= jend) { ++j; jend += g; }
        s = gsc[j];
        z = gzp[j];
        sf = (float)s;
        zf = (float)z;
      }
      const float x0 = rtn_f32<T>(w[c]);
      const float cs = a.colscale ? a.colscale[c] : 1.f;
      const float xf = a.colscale ? x0 * cs : x0;
      const float qf = xf / sf;
      const float y = a.sym ? qf : qf + zf;
      const float half = floorf(y) + 0.5f;
      const float tol = 2e-7f * (fabsf(qf) + fabsf(y)) + 1e-30f;
      float q;
      if (fabsf(y - half) > tol) {
        q = rintf(y);
      } else {
        const double xq = (double)xf / s;
        q = (float)(a.sym ? rint(xq) : rint(xq + z));
      }
      q = fminf(fmaxf(q, qminf), qmaxf);
      const uint32_t code = (uint32_t)((int)q + off);
      // with a column scale the error is taken in the original domain:
      // ŵ = (q - z)·s / colscale
      const double x = (double)x0;
      const double d = a.colscale ? x - ((double)q - z) * s / (double)cs : x - ((double)q - z) * s;
      se += d * d;
      xd += x * d;
      ww += x * x;
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
  for (int j = tid; j < G; j += kRtnThreads) {
    a.scales[r * a.G + j] = (float)gsc[j];
    a.zeros[r * a.G + j] = (int32_t)gzp[j] + off;
  }
  const int row_bad = __syncthreads_or(bad);
  if (tid == 0) a.badrow[r] = row_bad;

  // row sums: wave butterflies, then the 8 waves in order
  __shared__ double red[4][kRtnThreads / 64];
  // Σx·ŵ = Σx² - Σx·d, Σŵ² = Σx² - 2Σx·d + Σd²
  double v4[4] = {se, ww - xd, ww, ww - 2.0 * xd + se};
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v4[q] += __shfl_xor(v4[q], d, 64);
  if ((tid & 63) == 0)
#pragma unroll
    for (int q = 0; q < 4; ++q) red[q][tid >> 6] = v4[q];
  __syncthreads();
  if (tid < 4) {
    double sum = 0.0;
    for (int wv = 0; wv < kRtnThreads / 64; ++wv) sum += red[tid][wv];
    a.part[r * 4 + tid] = sum;
  }
}

// ---------------------------------------------------------------------------
// Streaming path for clip_ratio = 1, where every grid comes from its group's
// extremes and no order statistic is needed: one workgroup per output row,
// thread t holding the 8-column chunks t, t + NT, ... of the row in registers
// (one 16-byte load of bf16, two of fp32, per chunk); groups are whole chunks
// (g a multiple of 8, g/8 a power of two) or the whole row.  The grid is
// rtn_row_kernel's fp64 grid and every code the same rounding decision, so
// the two paths give identical codes, scales and zeros.
// ---------------------------------------------------------------------------
template <typename T> struct Chunk;
// hide() makes the held words opaque to the compiler (no instruction), so a
// second pass unpacks them again instead of keeping the first pass's floats
// alive in twice the registers.
template <> struct Chunk<uint16_t> {
  uint4 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void hide() { asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w)); }
  __device__ __forceinline__ void get(float (&x)[8]) const {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(u[i] << 16);
      x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  }
};
template <> struct Chunk<float> {
  f32x4_t a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const f32x4_t*>(p);
    b = *reinterpret_cast<const f32x4_t*>(p + 4);
  }
  __device__ __forceinline__ void hide() { asm volatile("" : "+v"(a), "+v"(b)); }
  __device__ __forceinline__ void get(float (&x)[8]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = a[i];
      x[i + 4] = b[i];
    }
  }
};

// The grid of one group (rtn_grid's fp64 values, so the scale and zero are
// those of the general kernel), plus what the code step needs in fp32.  The
// stored code is c = q + off (off = 2^(bits-1) for sym, else 0, so c lies in
// [0, 2^bits - 1] either way) and the fast path takes it as rint(y) with
// y = fl(x·fl(1/fl(s)) + fl(z + off)) (one fma).  Against the fp64
// x/s + z + off of the definition y errs by at most
// 2^-23·|x/s| + 2^-24·(|y| + |z + off|) (the scale's, the reciprocal's and
// the fma's roundings, z + off's own), below
// tol = 4e-7·(2·max|x|/s + |z + off|) for every x of the group; where
// |y - rint(y)| < half = fl(1/2 - tol) both round the same way, and the rest
// is recomputed as rint(x/s + z) + off in fp64, as the general kernel does.
// (fl(1/2 - tol) is within 2^-25 of 1/2 - tol; that slack only matters when
// max|x|/s < 0.05 and z + off = 0, where every |y| < 0.06 is far from a
// half-integer.)  A reciprocal below 2^-100 (scales near the fp32 limit)
// sends every code of the group to the fp64 route.
struct StreamGrid {
  double s, zo;    // scale, z + off
  float rf, zof;   // fl(1/fl(s)), fl(z + off)
  float half;      // fl(1/2 - tol)
  float pad;
};
static_assert(sizeof(StreamGrid) == 32, "StreamGrid is two 16-byte LDS words");

__device__ __forceinline__ StreamGrid stream_grid(float lo, float hi, int bits, int sym, float* scale_out,
                                                  int32_t* zero_out) {
  // sym: the grid is set by max|x| = max(-min x, max x)
  const float amax = fmaxf(-lo, hi);
  double s, z;
  rtn_grid((double)(sym ? 0.f : lo), (double)(sym ? amax : hi), bits, sym, s, z);
  const double off = sym ? (double)(1 << (bits - 1)) : 0.0;
  StreamGrid g;
  g.s = s;
  g.zo = z + off;
  g.pad = 0.f;
  const float sf = (float)s;
  g.rf = 1.f / sf;
  g.zof = (float)g.zo;
  const float tol = g.rf >= 0x1p-100f ? 4e-7f * (2.f * amax * g.rf + fabsf(g.zof)) : 1.f;
  g.half = 0.5f - tol;
  *scale_out = sf;
  *zero_out = (int32_t)g.zo;
  return g;
}
template <bool CS>
__device__ __forceinline__ void chunk_colscale(const float* colscale, int c8, float (&cs)[8]) {
  if constexpr (CS) {
    const f32x4_t c0 = *reinterpret_cast<const f32x4_t*>(colscale + 8 * c8);
    const f32x4_t c1 = *reinterpret_cast<const f32x4_t*>(colscale + 8 * c8 + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { cs[i] = c0[i]; cs[i + 4] = c1[i]; }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) cs[i] = 1.f;
  }
}

// min and max of one chunk's x·colscale, and a non-finite detector: nf stays
// 0 unless some value is NaN or ±Inf (then value·0 is NaN).
template <typename T, bool CS>
__device__ __forceinline__ void chunk_extremes(const float* colscale, const Chunk<T>& raw, int c8, float& lo,
                                               float& hi, float& nf) {
  float x[8], cs[8];
  raw.get(x);
  chunk_colscale<CS>(colscale, c8, cs);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float v = CS ? x[e] * cs[e] : x[e];
    nf = fmaf(v, 0.f, nf);
    lo = fminf(lo, v);
    hi = fmaxf(hi, v);
  }
}

// Codes, packing and the error sums of one 8-column chunk on grid g.  The
// error is taken in the original domain: d = x - (q - z)·s / colscale, with
// q - z = c - (z + off) exact in fp64; the division is a multiplication by
// 1/colscale from v_rcp_f64 and one Newton step (within an ulp or two of the
// quotient, far below the sums' tolerance of relative 1e-12).
template <typename T, bool CS>
__device__ __forceinline__ void stream_chunk(const RtnArgs& a, const Chunk<T>& raw, int c8, const StreamGrid& g,
                                             float cmax, float offf, uint32_t* qrow, double& se, double& xd,
                                             double& ww) {
  float x[8], cs[8];
  raw.get(x);
  chunk_colscale<CS>(a.colscale, c8, cs);
  float c[8];
  float dist = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float xf = CS ? x[e] * cs[e] : x[e];
    const float y = fmaf(xf, g.rf, g.zof);
    c[e] = rintf(y);
    dist = fmaxf(dist, fabsf(y - c[e]));
  }
  if (dist >= g.half) {   // some code near a half-integer: decide those in fp64
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float xf = CS ? x[e] * cs[e] : x[e];
      const float y = fmaf(xf, g.rf, g.zof);
      if (fabsf(y - c[e]) >= g.half) c[e] = (float)(rint((double)xf / g.s + (g.zo - (double)offf)) + (double)offf);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    c[e] = __builtin_amdgcn_fmed3f(c[e], 0.f, cmax);
    const double xv = (double)x[e];
    const double qz = (double)c[e] - g.zo;
    double d;
    if constexpr (CS) {
      const double c = (double)cs[e];
      double r = __builtin_amdgcn_rcp(c);
      r = fma(r, fma(-c, r, 1.0), r);
      d = xv - (qz * g.s) * r;
    } else {
      d = fma(-qz, g.s, xv);
    }
    se = fma(d, d, se);
    xd = fma(xv, d, xd);
    ww = fma(xv, xv, ww);
  }
  // codes are exact integers in [0, 255]: convert and place them a byte at a
  // time (4-bit: two codes per byte, c0 + 16·c1)
  if (a.bits <= 4) {
    uint32_t w = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) w = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(c[2 * i + 1], 16.f, c[2 * i]), i, w);
    qrow[c8] = w;
  } else {
    uint32_t w0 = 0u, w1 = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w0 = __builtin_amdgcn_cvt_pk_u8_f32(c[i], i, w0);
      w1 = __builtin_amdgcn_cvt_pk_u8_f32(c[i + 4], i, w1);
    }
    qrow[2 * c8] = w0;
    qrow[2 * c8 + 1] = w1;
  }
}

// LDS of the streaming kernel: the row's grids, then (groups of chunks) every
// chunk's extremes, and the cross-wave reduction slots.
template <int NT>
struct StreamLds {
  StreamGrid* grid;   // [G]
  float2* ext;        // [nc] chunk (min, max)
  float* red_lo;      // [NT/64]
  float* red_hi;      // [NT/64]
  double* red;        // [4][NT/64]
};

// The row's KR chunks of this thread (chunk t + NT·k), every load issued
// (chunks past the row's end re-read its last chunk), so that the number of
// loads in flight is the same on every path.
template <typename T, int NT, int KR>
__device__ __forceinline__ void stream_load(Chunk<T> (&buf)[KR], const T* wrow, int nc) {
#pragma unroll
  for (int k = 0; k < KR; ++k) buf[k].load(wrow + 8 * min((int)threadIdx.x + NT * k, nc - 1));
}

// One row: pass 1 writes every chunk's extremes to LDS, the first G threads
// reduce them to their group's (one group per row, lgl < 0: a block
// reduction instead) and turn them into grids (writing the scales and
// zeros), and pass 2 takes the codes and the error sums from the same
// registers.  Ends with the row's four sums in part[4r..4r+3] and its
// non-finite flag.
template <typename T, int NT, int KR, bool CS>
__device__ __forceinline__ void stream_row(const RtnArgs& a, int lgl, int64_t r, Chunk<T> (&raw)[KR],
                                           const StreamLds<NT>& L) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nc = (int)(a.n >> 3);
  const int kc = (nc + NT - 1) / NT;   // chunks of the row per thread (uniform, <= KR)
  uint32_t* qrow = a.qweight + r * a.words;
  const int G = (int)a.G;
  const bool rowgroup = lgl < 0;

  // pass 1: extremes
  float nf = 0.f, rlo = INFINITY, rhi = -INFINITY;
#pragma unroll
  for (int k = 0; k < KR; ++k) {
    const int c8 = tid + NT * k;
    if (k < kc && c8 < nc) {
      float lo = INFINITY, hi = -INFINITY;
      chunk_extremes<T, CS>(a.colscale, raw[k], c8, lo, hi, nf);
      if (rowgroup) {
        rlo = fminf(rlo, lo);
        rhi = fmaxf(rhi, hi);
      } else {
        L.ext[c8] = make_float2(lo, hi);
      }
    }
  }
  if (rowgroup) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      rlo = fminf(rlo, __shfl_xor(rlo, d, 64));
      rhi = fmaxf(rhi, __shfl_xor(rhi, d, 64));
    }
    if (lane == 0) { L.red_lo[wave] = rlo; L.red_hi[wave] = rhi; }
  }
  if constexpr (CS) {
    // x·colscale can overflow where x cannot: flag it here (nf != 0, NaN
    // compares unequal); without a column scale the row's Σx² flags it
    const int row_bad = __syncthreads_or(nf != 0.f);
    if (tid == 0) a.badrow[r] = row_bad;
  } else {
    __syncthreads();
  }
  for (int j = tid; j < G; j += NT) {
    float lo = INFINITY, hi = -INFINITY;
    if (rowgroup) {
#pragma unroll
      for (int wv = 0; wv < NW; ++wv) { lo = fminf(lo, L.red_lo[wv]); hi = fmaxf(hi, L.red_hi[wv]); }
    } else {
      const int c0 = j << lgl, c1 = min(c0 + (1 << lgl), nc);
      for (int c = c0; c < c1; ++c) {
        const float2 e = L.ext[c];
        lo = fminf(lo, e.x);
        hi = fmaxf(hi, e.y);
      }
    }
    L.grid[j] = stream_grid(lo, hi, a.bits, a.sym, a.scales + r * G + j, a.zeros + r * G + j);
  }
  __syncthreads();

  // pass 2: codes and error sums
#pragma unroll
  for (int k = 0; k < KR; ++k) raw[k].hide();
  const float cmax = (float)((1 << a.bits) - 1);
  const float offf = a.sym ? (float)(1 << (a.bits - 1)) : 0.f;
  const int gsh = rowgroup ? 31 : lgl;   // chunk -> group: c8 >> gsh (0 for one group per row)
  double se = 0.0, xd = 0.0, ww = 0.0;
#pragma unroll
  for (int k = 0; k < KR; ++k) {
    const int c8 = tid + NT * k;
    if (k < kc && c8 < nc) stream_chunk<T, CS>(a, raw[k], c8, L.grid[c8 >> gsh], cmax, offf, qrow, se, xd, ww);
  }
  double v4[4] = {se, ww - xd, ww, ww - 2.0 * xd + se};
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v4[q] += __shfl_xor(v4[q], d, 64);
  if (lane == 0)
#pragma unroll
    for (int q = 0; q < 4; ++q) L.red[q * NW + wave] = v4[q];
  __syncthreads();
  if (tid < 4) {
    double sum = 0.0;
    for (int wv = 0; wv < NW; ++wv) sum += L.red[tid * NW + wv];
    a.part[r * 4 + tid] = sum;
    // Σx² is finite exactly when every x is (x² <= 2^256 in fp64)
    if (!CS && tid == 2) a.badrow[r] = !isfinite(sum);
  }
}

// One workgroup per row.
template <typename T, int NT, int KR, bool CS>
__global__ __launch_bounds__(NT) void rtn_stream_kernel(RtnArgs a, int lgl) {
  extern __shared__ __attribute__((aligned(16))) unsigned char stream_smem[];
  constexpr int NW = NT / 64;
  __shared__ float red_lo[NW], red_hi[NW];
  __shared__ double red[4 * NW];
  StreamLds<NT> L;
  L.grid = reinterpret_cast<StreamGrid*>(stream_smem);
  L.ext = reinterpret_cast<float2*>(L.grid + a.G);
  L.red_lo = red_lo;
  L.red_hi = red_hi;
  L.red = red;
  const int64_t r = blockIdx.x;
  Chunk<T> raw[KR];
  stream_load<T, NT, KR>(raw, static_cast<const T*>(a.W) + r * a.n, (int)(a.n >> 3));
  stream_row<T, NT, KR, CS>(a, lgl, r, raw, L);
}

// err[0] = Σse / (m·n), err[1] = Σdot / (sqrt(Σww)·sqrt(Σdd) + 1e-8); rows in a
// fixed order (thread t sums rows t, t+1024, ...; then a fixed tree).  The
// status word: GPTQ_ERR_NONFINITE if a row (or, for AWQ, the channel
// statistics: extra_flag) held a NaN or Inf, else GPTQ_OK.
__global__ __launch_bounds__(1024) void rtn_reduce_kernel(const double* __restrict__ part, int64_t m,
                                                          int64_t count, double* __restrict__ err,
                                                          const int* __restrict__ badrow,
                                                          const int* extra_flag, int32_t* status) {
  __shared__ double sh[4][1024];
  const int tid = threadIdx.x;
  double v[4] = {0.0, 0.0, 0.0, 0.0};
  int bad = 0;
  for (int64_t r = tid; r < m; r += 1024) {
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] += part[r * 4 + q];
    bad |= badrow[r];
  }
  bad = __syncthreads_or(bad);
  if (tid == 0 && status)
    *status = (bad || (extra_flag && *extra_flag)) ? (int32_t)GPTQ_ERR_NONFINITE : (int32_t)GPTQ_OK;
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
  if (p.G == 1) p.lds_bytes += 8 * 256 * sizeof(uint32_t);   // radix-select histograms
  p.part_off = 0;
  p.flag_off = align256((size_t)std::max<int64_t>(m, 1) * 4 * sizeof(double));   // per-row flags
  p.total = p.flag_off + align256((size_t)std::max<int64_t>(m, 1) * sizeof(int));
  return p;
}

namespace {
// log2(chunks per group) for the streaming kernel (-1: one group per row), or
// -2 when the layer needs the general kernel: clipping, unaligned rows, a
// group width that is not 8 times a power of two, a row longer than the
// registers of one workgroup hold, or more LDS than a workgroup has.
constexpr size_t kStreamMaxLds = 160 * 1024;

// Workgroup shapes (threads, chunks per thread) by the row's chunk count: the
// fewest chunks per thread that hold the row, since registers a row does not
// need only lower the number of rows in flight per CU.
struct StreamShape { int nt, kr; };
StreamShape stream_shape(int64_t nc, int w_dtype) {
  if (nc <= 256 * 2) return {256, 2};
  if (nc <= 256 * 4) return {256, 4};
  if (nc <= 256 * 6) return {256, 6};
  if (nc <= 256 * 8) return {256, 8};
  if (w_dtype == GPTQ_BF16) {
    if (nc <= 256 * 16) return {256, 16};
    if (nc <= 512 * 16) return {512, 16};
  } else if (nc <= 512 * 8) {
    return {512, 8};
  }
  return {0, 0};
}

size_t stream_lds_bytes(int64_t nc, const RtnPlan& p) {
  return (size_t)p.G * sizeof(StreamGrid) + (p.G > 1 ? (size_t)nc * sizeof(float2) : 0);
}

int rtn_stream_lgl(const void* W, int w_dtype, const float* colscale, int64_t n, float clip, const RtnPlan& p) {
  if (!(clip >= 1.f) || n % 8 != 0 || stream_shape(n / 8, w_dtype).nt == 0) return -2;
  if (stream_lds_bytes(n / 8, p) > kStreamMaxLds) return -2;
  if ((reinterpret_cast<uintptr_t>(W) & 15) != 0 || (reinterpret_cast<uintptr_t>(colscale) & 15) != 0) return -2;
  if (p.G == 1) return -1;
  if (p.g % 8 != 0) return -2;
  const int64_t gl = p.g / 8;
  if ((gl & (gl - 1)) != 0) return -2;
  return __builtin_ctzll((unsigned long long)gl);
}

template <typename T, int NT, int KR, bool CS>
gptq_status launch_stream_kernel(int lgl, const RtnArgs& a, size_t lds, hipStream_t stream) {
  const void* fn = reinterpret_cast<const void*>(&rtn_stream_kernel<T, NT, KR, CS>);
  if (lds > 65536) GPTQ_HIP_CHECK(hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
  hipLaunchKernelGGL((rtn_stream_kernel<T, NT, KR, CS>), dim3((unsigned)a.m), dim3(NT), lds, stream, a, lgl);
  return GPTQ_OK;
}

template <typename T, int NT, int KR>
gptq_status launch_stream_shape(int lgl, const RtnArgs& a, size_t lds, hipStream_t stream) {
  if (a.colscale) return launch_stream_kernel<T, NT, KR, true>(lgl, a, lds, stream);
  return launch_stream_kernel<T, NT, KR, false>(lgl, a, lds, stream);
}

template <typename T>
gptq_status launch_stream(int lgl, int w_dtype, const RtnArgs& a, const RtnPlan& p, hipStream_t stream) {
  const StreamShape sh = stream_shape(a.n / 8, w_dtype);
  const size_t lds = stream_lds_bytes(a.n / 8, p);
  if (sh.nt == 256 && sh.kr == 2) return launch_stream_shape<T, 256, 2>(lgl, a, lds, stream);
  if (sh.nt == 256 && sh.kr == 4) return launch_stream_shape<T, 256, 4>(lgl, a, lds, stream);
  if (sh.nt == 256 && sh.kr == 6) return launch_stream_shape<T, 256, 6>(lgl, a, lds, stream);
  if (sh.nt == 256 && sh.kr == 8) return launch_stream_shape<T, 256, 8>(lgl, a, lds, stream);
  if constexpr (sizeof(T) == 2) {   // bf16: up to 16 chunks (64 registers) per thread
    if (sh.nt == 256) return launch_stream_shape<T, 256, 16>(lgl, a, lds, stream);
    return launch_stream_shape<T, 512, 16>(lgl, a, lds, stream);
  } else {                          // fp32: up to 8 chunks per thread
    return launch_stream_shape<T, 512, 8>(lgl, a, lds, stream);
  }
}
}  // namespace

gptq_status run_rtn(const void* W, int w_dtype, int64_t m, int64_t n, int bits, int sym, float clip,
                    uint32_t* qweight, float* scales, int32_t* zeros, double* err, int32_t* status, void* ws,
                    const RtnPlan& p, hipStream_t stream, const float* colscale, const int* extra_flag) {
  char* w = static_cast<char*>(ws);
  RtnArgs a;
  a.W = W; a.m = m; a.n = n; a.bits = bits; a.sym = sym;
  a.g = p.g; a.G = p.G; a.P = p.P; a.clip = clip;
  a.qweight = qweight; a.words = gptq_qweight_words(n, bits);
  a.scales = scales; a.zeros = zeros;
  a.part = reinterpret_cast<double*>(w + p.part_off);
  a.badrow = reinterpret_cast<int*>(w + p.flag_off);
  a.colscale = colscale;
  const int lgl = rtn_stream_lgl(W, w_dtype, colscale, n, clip, p);
  if (lgl >= -1) {
    const gptq_status st = w_dtype == GPTQ_BF16 ? launch_stream<uint16_t>(lgl, w_dtype, a, p, stream)
                                                : launch_stream<float>(lgl, w_dtype, a, p, stream);
    if (st != GPTQ_OK) return st;
  } else {
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
  }
  GPTQ_LAUNCH_CHECK();
  hipLaunchKernelGGL(rtn_reduce_kernel, dim3(1), dim3(1024), 0, stream, (const double*)a.part, m, m * n,
                     err, (const int*)a.badrow, extra_flag, status);
  GPTQ_LAUNCH_CHECK();
  return GPTQ_OK;
}

}  // namespace gptq
