// Stage 1: H += alpha * XᵀX and key += alpha * Σ_t x_t² (fp64) over a token tile.
//
// The Hessian of the layer objective is the (scaled) Gram matrix of the
// calibration activations (page "模型量化实战：从 INT8 PTQ 到 GPTQ…" §3.2,
// accumulate_hessian: H grows by 2·XᵀX per batch).  It is a symmetric rank-T
// update, so only lower-triangle tiles are computed and each result is
// mirrored to the upper triangle.
//
// bf16 path: v_mfma_f32_32x32x16_bf16.  X is token-major, so the reduction
// axis (tokens) is the strided one; each thread loads an 8-token x 8-channel
// block with eight 16-byte reads, transposes it in registers (v_perm), and
// stores eight channel rows of 8 tokens into LDS.  The LDS layout is
// [token octet][256 channels] x 16 bytes with the channel slot swizzled by
// ch ^ ((ch >> 4) & 7), which keeps both the transposing stores and the MFMA
// operand reads free of bank conflicts.
//
// Tiles are 256 x 256 (4 waves, 128 x 128 each).  Long token ranges are cut
// into `splits` slices (split-K) so the grid fills 256 CUs and every fp32
// register chain stays <= 32768 tokens long; with splits a multiple of 8 all
// workgroups of one XCD share a token slice.  Slices meet in a partial buffer
// and the last workgroup of a tile to finish (an atomic ticket) sums the
// partials in slice order, so the result is deterministic.
#include <algorithm>

#include "gptq_internal.hpp"

namespace gptq {
namespace {

struct SyrkArgs {
  const uint16_t* X;
  int64_t ldx, T;
  int64_t n;
  int64_t tiles, splits, slice_tokens;
  float* H;
  double* key;
  float alpha;
  float* partials;
  double* keyparts;
  int* counters;
};

constexpr int kOcts = kSyrkStage / 8;   // token octets per stage

__device__ __forceinline__ int swz(int ch) { return ch ^ ((ch >> 4) & 7); }

__device__ __forceinline__ void tri_decode(int64_t t, int64_t& ti, int64_t& tj) {
  int64_t r = (int64_t)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
  while (r * (r + 1) / 2 > t) --r;
  while ((r + 1) * (r + 2) / 2 <= t) ++r;
  ti = r;
  tj = t - r * (r + 1) / 2;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 8 tokens (rows) x 8 channels starting at (t0, c0); zero outside [.., t_end) x [.., n).
template <bool VEC>
__device__ __forceinline__ void load_block(const uint16_t* __restrict__ X, int64_t ldx, int64_t t0,
                                           int64_t t_end, int64_t c0, int64_t n, uint4 (&v)[8]) {
  if (VEC && t0 + 8 <= t_end && c0 + 8 <= n) {
    const uint16_t* p = X + t0 * ldx + c0;
#pragma unroll
    for (int r = 0; r < 8; ++r) v[r] = *reinterpret_cast<const uint4*>(p + r * ldx);
    return;
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int64_t t = t0 + r;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (t < t_end && c0 < n) {
      const uint16_t* p = X + t * ldx + c0;
      if (VEC && c0 + 8 <= n) {
        x = *reinterpret_cast<const uint4*>(p);
      } else {
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = (c0 + e < n) ? (uint32_t)p[e] : 0u;
        x.x = h[0] | (h[1] << 16);
        x.y = h[2] | (h[3] << 16);
        x.z = h[4] | (h[5] << 16);
        x.w = h[6] | (h[7] << 16);
      }
    }
    v[r] = x;
  }
}

__device__ __forceinline__ uint32_t dw(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Transpose the 8x8 block (rows = tokens) into 8 channel vectors of 8 tokens and
// store them at LDS [oct][swz(ch)].  With KEY, add each channel's Σx² (fp64).
template <bool KEY>
__device__ __forceinline__ void transpose_store(const uint4 (&v)[8], uint4* __restrict__ panel,
                                                int oct, int ch0, double (&keyacc)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint4 o;
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t a = dw(v[2 * k], e >> 1), b = dw(v[2 * k + 1], e >> 1);
      w[k] = (e & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
    o.x = w[0]; o.y = w[1]; o.z = w[2]; o.w = w[3];
    panel[oct * 256 + swz(ch0 + e)] = o;
    if (KEY) {
      double s = 0.0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float lo = bf16_lo(w[k]), hi = bf16_hi(w[k]);
        s += (double)(lo * lo);   // a bf16 square is exact in fp32
        s += (double)(hi * hi);
      }
      keyacc[e] += s;
    }
  }
}

template <bool VEC>
__global__ __launch_bounds__(256, 1) void syrk_bf16_kernel(SyrkArgs a) {
  // [buffer][panel I/J][token octet * 256 + channel slot]: 2 x 2 x 4 x 256 x 16 B = 64 KB
  __shared__ uint4 lds[2][2][kOcts * 256];
  __shared__ double red[kOcts][256];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;

  // workgroup -> (tile, slice); without slices-per-XCD, spread contiguous
  // logical ranges over the 8 XCDs (dispatch is round-robin over XCDs).
  const int64_t total = a.tiles * a.splits;
  int64_t b = blockIdx.x;
  if (a.splits % 8 != 0) {
    const int64_t per = (total + 7) / 8;
    b = (b % 8) * per + b / 8;
    if (b >= total) return;
  }
  const int64_t tile = b / a.splits, s = b % a.splits;
  int64_t ti, tj;
  tri_decode(tile, ti, tj);
  const bool diag = (ti == tj);
  const bool idle_wave = diag && wr == 0 && wc == 1;   // strictly upper quarter

  const int64_t t_begin = s * a.slice_tokens;
  const int64_t t_end = (t_begin + a.slice_tokens < a.T) ? t_begin + a.slice_tokens : a.T;
  const int64_t nst = (t_end > t_begin) ? (t_end - t_begin + kSyrkStage - 1) / kSyrkStage : 0;

  // staging role: one 8-token x 8-channel block of panel I (threads 0-127) or J
  const int panel = tid >> 7;
  const int ch_oct = tid & 31, tok_oct = (tid >> 5) & 3;
  const bool stager = !(diag && panel == 1);
  const bool keyer = diag && panel == 0;
  const int64_t cbase = (panel == 0 ? ti : tj) * kSyrkTile + ch_oct * 8;

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  double keyacc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) keyacc[e] = 0.0;

  uint4 vb[8];
  if (nst > 0 && stager) {
    load_block<VEC>(a.X, a.ldx, t_begin + tok_oct * 8, t_end, cbase, a.n, vb);
    if (keyer) transpose_store<true>(vb, lds[0][0], tok_oct, ch_oct * 8, keyacc);
    else transpose_store<false>(vb, lds[0][panel], tok_oct, ch_oct * 8, keyacc);
  }
  __syncthreads();

  for (int64_t st = 0; st < nst; ++st) {
    const int cur = (int)(st & 1);
    const bool more = st + 1 < nst;
    if (more && stager)
      load_block<VEC>(a.X, a.ldx, t_begin + (st + 1) * kSyrkStage + tok_oct * 8, t_end, cbase, a.n, vb);
    if (!idle_wave) {
      const uint4* pI = lds[cur][0];
      const uint4* pJ = diag ? lds[cur][0] : lds[cur][1];
#pragma unroll
      for (int kk = 0; kk < kSyrkStage / 16; ++kk) {
        const int oct = 2 * kk + (lane >> 5);
        bf16x8_t af[4], bfm[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          af[i] = __builtin_bit_cast(bf16x8_t, pI[oct * 256 + swz(wr * 128 + i * 32 + (lane & 31))]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bfm[j] = __builtin_bit_cast(bf16x8_t, pJ[oct * 256 + swz(wc * 128 + j * 32 + (lane & 31))]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfm[j], acc[i][j], 0, 0, 0);
      }
    }
    if (more && stager) {
      if (keyer) transpose_store<true>(vb, lds[cur ^ 1][0], tok_oct, ch_oct * 8, keyacc);
      else transpose_store<false>(vb, lds[cur ^ 1][panel], tok_oct, ch_oct * 8, keyacc);
    }
    __syncthreads();
  }

  // ---- per-channel key of a diagonal tile: reduce the token-octet partials
  double ksum = 0.0;
  if (diag) {
    if (keyer) {
#pragma unroll
      for (int e = 0; e < 8; ++e) red[tok_oct][ch_oct * 8 + e] = keyacc[e];
    }
    __syncthreads();
#pragma unroll
    for (int o = 0; o < kOcts; ++o) ksum += red[o][tid];
  }

  const int64_t n = a.n;
  const int64_t gi0 = ti * kSyrkTile + wr * 128 + 4 * (lane >> 5);
  const int64_t gj0 = tj * kSyrkTile + wc * 128 + (lane & 31);

  if (a.splits > 1) {
    // ---- split-K: publish the partial, take a ticket; the last workgroup of
    // the tile re-reads all slices (its own included) and sums them in slice
    // order, so the result does not depend on which one finishes last.
    float* mine = a.partials + ((tile * a.splits + s) * 256) * 256;
    if (!idle_wave) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) mine[((i * 4 + j) * 16 + v) * 256 + tid] = acc[i][j][v];
    }
    if (diag) {
      const int64_t c = ti * kSyrkTile + tid;
      if (c < n) a.keyparts[s * n + c] = ksum;
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const int old = __hip_atomic_fetch_add(&a.counters[tile], 1, __ATOMIC_ACQ_REL,
                                             __HIP_MEMORY_SCOPE_AGENT);
      s_last = (old == (int)a.splits - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    if (!idle_wave) {
      const float* base = a.partials + (tile * a.splits) * 256 * 256;
      for (int64_t q = 0; q < a.splits; ++q) {
        const float* pq = base + q * 256 * 256;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const float x = pq[((i * 4 + j) * 16 + v) * 256 + tid];
              acc[i][j][v] = (q == 0) ? x : acc[i][j][v] + x;
            }
      }
    }
    if (diag) {
      const int64_t c = ti * kSyrkTile + tid;
      double sum = 0.0;
      if (c < n)
        for (int64_t q = 0; q < a.splits; ++q) sum += a.keyparts[q * n + c];
      ksum = sum;
    }
  }

  // ---- H (lower tile, mirrored) and key
  if (!idle_wave) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t gi = gi0 + i * 32 + 8 * (v >> 2) + (v & 3);
          const int64_t gj = gj0 + j * 32;
          if (gi < n && gj < n && (!diag || gi >= gj)) {
            const float val = a.H[gi * n + gj] + a.alpha * acc[i][j][v];
            a.H[gi * n + gj] = val;
            if (gi != gj) a.H[gj * n + gi] = val;
          }
        }
  }
  if (diag && a.key) {
    const int64_t c = ti * kSyrkTile + tid;
    if (c < n) a.key[c] += (double)a.alpha * ksum;
  }
}

__global__ void fill_i32_kernel(int* p, int64_t count, int val) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = val;
}

// ---------------------------------------------------------------------------
// fp32 activations: v_mfma_f32_32x32x2f32 on 128 x 128 tiles, no split.  The
// X tile is kept token-major in LDS ([32 tokens][128 channels], pitch 160) --
// an fp32 MFMA operand is one element per lane, so no transpose is needed.
// ---------------------------------------------------------------------------
constexpr int FT = 128, FK = 32, FP = FT + 32;

template <bool VEC>
__global__ __launch_bounds__(256) void syrk_f32_kernel(const float* __restrict__ X, int64_t ldx,
                                                       int64_t T, int64_t n, float* H, double* key,
                                                       float alpha) {
  __shared__ float xs[2][FK * FP];
  __shared__ double red[8][FT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1, li = lane & 31, lk = lane >> 5;
  int64_t ti, tj;
  tri_decode(blockIdx.x, ti, tj);
  const bool diag = ti == tj;
  const int64_t cI = ti * FT, cJ = tj * FT;

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  double kacc[4] = {0.0, 0.0, 0.0, 0.0};

  const int c4 = tid & 31;   // this thread's 4 channels (same for every u)
  for (int64_t t0 = 0; t0 < T; t0 += FK) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      if (p == 1 && diag) break;
      const int64_t cb = p == 0 ? cI : cJ;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int f = tid + 256 * u;
        const int tr = f >> 5;
        const int64_t t = t0 + tr, c = cb + 4 * c4;
        f32x4_t v = {0.f, 0.f, 0.f, 0.f};
        if (t < T && c < n) {
          const float* src = X + t * ldx + c;
          if (VEC && c + 4 <= n) v = *reinterpret_cast<const f32x4_t*>(src);
          else
            for (int e = 0; e < 4; ++e)
              if (c + e < n) v[e] = src[e];
        }
        *reinterpret_cast<f32x4_t*>(&xs[p][tr * FP + 4 * c4]) = v;
        if (p == 0 && diag)
#pragma unroll
          for (int e = 0; e < 4; ++e) kacc[e] += (double)v[e] * (double)v[e];
      }
    }
    __syncthreads();
    const float* sI = xs[0];
    const float* sJ = diag ? xs[0] : xs[1];
    if (!(diag && wr == 0 && wc == 1)) {
#pragma unroll
      for (int kk = 0; kk < FK / 2; ++kk) {
        const int k = 2 * kk + lk;
        float af[2], bf[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) af[i] = sI[k * FP + wr * 64 + i * 32 + li];
#pragma unroll
        for (int j = 0; j < 2; ++j) bf[j] = sJ[k * FP + wc * 64 + j * 32 + li];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  if (!(diag && wr == 0 && wc == 1)) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t gi = cI + wr * 64 + i * 32 + 8 * (v >> 2) + 4 * lk + (v & 3);
          const int64_t gj = cJ + wc * 64 + j * 32 + li;
          if (gi < n && gj < n && (!diag || gi >= gj)) {
            const float val = H[gi * n + gj] + alpha * acc[i][j][v];
            H[gi * n + gj] = val;
            if (gi != gj) H[gj * n + gi] = val;
          }
        }
  }
  if (diag && key) {
#pragma unroll
    for (int e = 0; e < 4; ++e) red[tid >> 5][4 * c4 + e] = kacc[e];
    __syncthreads();
    if (tid < FT) {
      double s = 0.0;
#pragma unroll
      for (int o = 0; o < 8; ++o) s += red[o][tid];
      if (cI + tid < n) key[cI + tid] += (double)alpha * s;
    }
  }
}

}  // namespace

SyrkPlan plan_syrk_bf16(int64_t n, int64_t tokens) {
  SyrkPlan p;
  p.panels = ceil_div(n, kSyrkTile);
  p.tiles = p.panels * (p.panels + 1) / 2;
  const int64_t smin = tokens > 0 ? ceil_div(tokens, kSyrkMaxSliceTokens) : 1;
  // Pick the slice count that minimises a simple time model: rounds of 256
  // resident workgroups times the per-slice MFMA time, plus the partial-tile
  // traffic of split-K.
  const double per_tok = (double)kSyrkTile * kSyrkTile * 2.0 / 9.8e12;   // one CU at peak
  double best = 1e300;
  int64_t best_s = smin;
  const int64_t cands[] = {1, 2, 4, 8, 16, 24, 32, 40, 48, 56, 64};
  for (int64_t c : cands) {
    if (c < smin) continue;
    const int64_t slice = round_up(ceil_div(std::max<int64_t>(tokens, 1), c), kSyrkStage);
    const double rounds = (double)ceil_div(p.tiles * c, 256);
    double t = rounds * (double)slice * per_tok;
    if (c > 1) t += 2.0 * (double)c * (double)p.tiles * 256.0 * 1024.0 / 4e12;
    if (t < best * 0.999) { best = t; best_s = c; }
  }
  if (best_s < smin) best_s = smin;
  p.splits = best_s;
  p.slice_tokens = round_up(ceil_div(std::max<int64_t>(tokens, 1), p.splits), kSyrkStage);
  if (p.splits > 1) {
    p.partial_bytes = align256((size_t)p.splits * p.tiles * 256 * 256 * sizeof(float));
    p.keypart_bytes = align256((size_t)p.splits * n * sizeof(double));
    p.counter_bytes = align256((size_t)p.tiles * sizeof(int));
  }
  p.total_bytes = p.partial_bytes + p.keypart_bytes + p.counter_bytes;
  return p;
}

gptq_status launch_hessian_bf16(float* H, double* key, int64_t n, const uint16_t* X, int64_t tokens,
                                int64_t ldx, float alpha, void* ws, const SyrkPlan& plan,
                                hipStream_t stream) {
  SyrkArgs a;
  a.X = X; a.ldx = ldx; a.T = tokens; a.n = n;
  a.tiles = plan.tiles; a.splits = plan.splits; a.slice_tokens = plan.slice_tokens;
  a.H = H; a.key = key; a.alpha = alpha;
  char* w = static_cast<char*>(ws);
  a.partials = plan.splits > 1 ? reinterpret_cast<float*>(w) : nullptr;
  a.keyparts = plan.splits > 1 ? reinterpret_cast<double*>(w + plan.partial_bytes) : nullptr;
  a.counters = plan.splits > 1 ? reinterpret_cast<int*>(w + plan.partial_bytes + plan.keypart_bytes)
                               : nullptr;
  if (plan.splits > 1) {
    hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)std::min<int64_t>(ceil_div(plan.tiles, 256), 1024)),
                       dim3(256), 0, stream, a.counters, plan.tiles, 0);
    GPTQ_LAUNCH_CHECK();
  }
  int64_t grid = plan.tiles * plan.splits;
  if (plan.splits % 8 != 0) grid = round_up(grid, 8);
  const bool vec = (ldx % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0);
  if (vec) hipLaunchKernelGGL(syrk_bf16_kernel<true>, dim3((unsigned)grid), dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(syrk_bf16_kernel<false>, dim3((unsigned)grid), dim3(256), 0, stream, a);
  GPTQ_LAUNCH_CHECK();
  return GPTQ_OK;
}

gptq_status launch_hessian_f32(float* H, double* key, int64_t n, const float* X, int64_t tokens,
                               int64_t ldx, float alpha, hipStream_t stream) {
  const int64_t p = ceil_div(n, FT);
  const unsigned grid = (unsigned)(p * (p + 1) / 2);
  const bool vec = (ldx % 4 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0);
  if (vec) hipLaunchKernelGGL(syrk_f32_kernel<true>, dim3(grid), dim3(256), 0, stream, X, ldx, tokens, n, H, key, alpha);
  else hipLaunchKernelGGL(syrk_f32_kernel<false>, dim3(grid), dim3(256), 0, stream, X, ldx, tokens, n, H, key, alpha);
  GPTQ_LAUNCH_CHECK();
  return GPTQ_OK;
}

}  // namespace gptq
