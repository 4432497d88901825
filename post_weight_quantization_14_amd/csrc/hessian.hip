// Stage 1: H += alpha * XᵀX and key += alpha * Σ_t x_t² (fp64) over a token tile.
//
// The Hessian of the layer objective is the (scaled) Gram matrix of the
// calibration activations (page "模型量化实战：从 INT8 PTQ 到 GPTQ…" §3.2,
// accumulate_hessian: H grows by 2·XᵀX per batch).  It is a symmetric rank-T
// update, so only lower-triangle tiles are computed and each result is
// mirrored to the upper triangle.
//
// bf16 path: v_mfma_f32_32x32x16_bf16.  X is token-major, so the reduction
// axis (tokens) is the strided one.  Each 32-token stage of the two 256-channel
// panels is copied into LDS as is (16-byte loads, token-major rows, octet slot
// swizzled), and the MFMA operands -- 8 consecutive tokens of one channel per
// lane -- come out of LDS through gfx950's transposing ds_read_b64_tr_b16.
// The fp64 diagonal key of a diagonal tile is summed from the staged panel.
//
// Tiles are 256 x 256 with 8 waves (two per SIMD), each 64 x 128 = 2 x 4
// MFMA blocks (128 accumulator registers), so a second wave hides each
// wave's LDS and barrier latency.
// Long token ranges are cut into `splits` slices (split-K) so the grid fills
// 256 CUs and every fp32 register chain stays <= 32768 tokens long; with
// splits a multiple of 8 all workgroups of one XCD share a token slice.
// Slices meet in a partial buffer and the last workgroup of a tile to finish
// (an atomic ticket) sums the partials in slice order, so the result is
// deterministic.
#include <algorithm>

#include "gptq_internal.hpp"

namespace gptq {
namespace {

struct SyrkArgs {
  const uint16_t* X;
  int64_t ldx, T;
  int64_t n;
  int64_t panels, tiles, splits, slice_tokens;
  float* H;
  double* key;
  float alpha;
  float* partials;
  double* keyparts;
  int* counters;
};

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

constexpr int kRowBytes = 512;                       // one token of a 256-channel panel
constexpr int kPanelBytes = kSyrkStage * kRowBytes;  // 32 KB per panel per stage

// Byte offset of (token t, channel octet o) in a panel stage: token-major rows
// of 32 octets, octet slot swizzled by 4·(t mod 4).  The transposing reads
// below touch 4 consecutive tokens x 2 octets per 16-lane group; the swizzle
// spreads them over 8 distinct bank quads, and the paired group (16 channels
// further) over the other 8, so a 32-lane half reads all 64 banks once.
__device__ __forceinline__ int lds_off(int t, int o) { return t * kRowBytes + ((o ^ ((t & 3) << 2)) << 4); }

__device__ __forceinline__ void tri_decode(int64_t t, int64_t& ti, int64_t& tj) {
  int64_t r = (int64_t)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
  while (r * (r + 1) / 2 > t) --r;
  while ((r + 1) * (r + 2) / 2 <= t) ++r;
  ti = r;
  tj = t - r * (r + 1) / 2;
}

// Lower-triangle tile number t -> (ti, tj) in a grouped order: super-blocks of
// 8 x 8 tiles, super-blocks row by row, tiles row by row inside each.  The 32
// workgroups an XCD runs at once then cover about 4 x 8 tiles (12 panels of X)
// instead of a long tile row, so more of their panel reads hit the XCD's L2.
constexpr int kGroup = 8;
__device__ __forceinline__ void tile_decode_grouped(int64_t t, int64_t panels, int64_t& ti,
                                                    int64_t& tj) {
  const int64_t nr = (panels + kGroup - 1) / kGroup;
  int64_t rem = t;
  for (int64_t R = 0; R < nr; ++R) {
    const int64_t r0 = R * kGroup, r1 = (r0 + kGroup < panels) ? r0 + kGroup : panels;
    for (int64_t C = 0; C <= R; ++C) {
      const int64_t c0 = C * kGroup, c1 = (c0 + kGroup < panels) ? c0 + kGroup : panels;
      const int64_t w = c1 - c0, h = r1 - r0;
      const int64_t cnt = (C < R) ? h * w : h * (h + 1) / 2;
      if (rem < cnt) {
        if (C < R) {
          ti = r0 + rem / w;
          tj = c0 + rem % w;
        } else {
          int64_t li, lj;
          tri_decode(rem, li, lj);
          ti = r0 + li;
          tj = c0 + lj;
        }
        return;
      }
      rem -= cnt;
    }
  }
  ti = tj = 0;   // not reached for t < tiles
}

// 16 bytes = channels [c, c+8) of token t; zero where t >= t_lim or c + e >= n.
__device__ __forceinline__ uint4 load16(const uint16_t* __restrict__ X, int64_t ldx, int64_t t,
                                        int64_t t_lim, int64_t c, int64_t n) {
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = (t < t_lim && c + e < n) ? (uint32_t)X[t * ldx + c + e] : 0u;
  return make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
}

// MFMA operand of 32 channels [c0, c0+32) for the 16-token step at token k0:
// lane l gets channel c0 + l%32 at tokens k0 + 8·(l/32) + e, e = 0..7, via two
// ds_read_b64_tr_b16 (each 16-lane group points at 4 tokens x 16 channels).
__device__ __forceinline__ bf16x8_t tr_frag(const uint8_t* panel, int k0, int c0, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int c = c0 + ((g & 1) << 4) + ((s & 3) << 2);
  const int t = k0 + ((g >> 1) << 3) + (s >> 2);
  const uint8_t* p0 = panel + lds_off(t, c >> 3) + ((c & 7) << 1);
  const uint8_t* p1 = panel + lds_off(t + 4, c >> 3) + ((c & 7) << 1);
  const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(p0));
  const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(p1));
  const auto v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

template <bool VEC>
__global__ __launch_bounds__(512, 1) void syrk_bf16_kernel(SyrkArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kPanelBytes];   // [buffer][panel]: 128 KB
  __shared__ double kred[256];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;   // wave tile: rows wr*64 (+64), cols wc*128 (+128)

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
  tile_decode_grouped(tile, a.panels, ti, tj);
  const bool diag = (ti == tj);
  const bool idle_wave = diag && wc == 1 && wr < 2;   // strictly above the diagonal
  const int64_t n = a.n;

  const int64_t t_begin = s * a.slice_tokens;
  const int64_t t_end = (t_begin + a.slice_tokens < a.T) ? t_begin + a.slice_tokens : a.T;
  const int64_t nst = (t_end > t_begin) ? (t_end - t_begin + kSyrkStage - 1) / kSyrkStage : 0;

  // staging: thread loads octet o of tokens tr + 16u (u = 0..3) of both panels
  const int o = tid & 31, tr = tid >> 5;
  const int64_t cI = ti * kSyrkTile + 8 * o, cJ = tj * kSyrkTile + 8 * o;
  const bool okI = cI < n, okJ = cJ < n;   // (VEC: n % 8 == 0, so cI < n covers the octet)

  f32x16_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  double ksum = 0.0;   // diagonal tiles: Σx² of channel tid % 256 over half of each stage

  // VEC: buffer loads off a per-stage scalar base, one 32-bit lane offset per
  // panel and the 16-token row step in an SGPR.  The descriptor's size ends at
  // the slice's last token, so rows past it read as zeros; channel octets past
  // n read a valid octet and are zeroed in put().  Every stage issues the same
  // 8 loads, so the loop needs no per-path wait bookkeeping.
  constexpr int kU = kSyrkStage / 16;   // loads per panel per thread and stage
  uint4 vI[kU], vJ[kU];
  const int32_t rowb = (int32_t)(a.ldx * 2);
  const int32_t vofsI = tr * rowb + (int32_t)((okI ? cI : n - 8) * 2);
  const int32_t vofsJ = tr * rowb + (int32_t)((okJ ? cJ : n - 8) * 2);
  auto load = [&](int64_t t0) {
    if (VEC) {
      const int64_t bytes = (t_end - t0) * a.ldx * 2;
      const int32_t nrec = bytes > 0x7fffffff ? 0x7fffffff : (int32_t)bytes;
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.X + t0 * a.ldx), 0, nrec, 0x00020000);
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        vI[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, vofsI, 16 * u * rowb, 0));
        vJ[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, vofsJ, 16 * u * rowb, 0));
      }
    } else {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        vI[u] = load16(a.X, a.ldx, t0 + tr + 16 * u, t_end, cI, n);
        vJ[u] = load16(a.X, a.ldx, t0 + tr + 16 * u, t_end, cJ, n);
      }
    }
  };
  auto put = [&](int buf) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int off = lds_off(tr + 16 * u, o);
      *reinterpret_cast<uint4*>(&lds[buf][0][off]) = okI ? vI[u] : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(&lds[buf][1][off]) = okJ ? vJ[u] : make_uint4(0, 0, 0, 0);
    }
  };
  auto mma = [&](int buf) {
    if (!idle_wave) {
      const uint8_t* pI = lds[buf][0];
      const uint8_t* pJ = lds[buf][1];
#pragma unroll
      for (int kk = 0; kk < kSyrkStage / 16; ++kk) {
        bf16x8_t af[2], bfm[4];
#pragma unroll
        for (int i = 0; i < 2; ++i) af[i] = tr_frag(pI, 16 * kk, wr * 64 + i * 32, lane);
#pragma unroll
        for (int j = 0; j < 4; ++j) bfm[j] = tr_frag(pJ, 16 * kk, wc * 128 + j * 32, lane);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfm[j], acc[i][j], 0, 0, 0);
      }
    }
    if (diag) {   // fp64 key: channel tid % 256, one half of the stage's tokens
      const uint8_t* pI = lds[buf][0];
      const int c = tid & 255, t0 = (tid >> 8) * (kSyrkStage / 2);
#pragma unroll
      for (int t = 0; t < kSyrkStage / 2; ++t) {
        const uint16_t hv = *reinterpret_cast<const uint16_t*>(pI + lds_off(t0 + t, c >> 3) + ((c & 7) << 1));
        const float x = __uint_as_float((uint32_t)hv << 16);
        ksum += (double)(x * x);   // a bf16 square is exact in fp32
      }
    }
  };

  if (nst > 0) {
    load(t_begin);
    put(0);
    __syncthreads();
    // stage st sits in lds[st & 1]; the loads of stage st + 1 are in flight
    // while its MFMAs run (the last iteration re-reads the last stage)
    for (int64_t st = 0; st < nst; ++st) {
      const int64_t nx = (st + 1 < nst) ? st + 1 : st;
      load(t_begin + nx * kSyrkStage);
      mma((int)(st & 1));
      if (st + 1 < nst) put((int)((st + 1) & 1));
      __syncthreads();
    }
  }
  if (diag) {   // combine the two token halves of each channel
    if (tid >= 256) kred[tid - 256] = ksum;
    __syncthreads();
    if (tid < 256) ksum += kred[tid];
  }

  const int64_t gi0 = ti * kSyrkTile + wr * 64 + 4 * (lane >> 5);
  const int64_t gj0 = tj * kSyrkTile + wc * 128 + (lane & 31);
  constexpr int kRegs = 2 * 4 * 16;   // accumulator registers per lane

  if (a.splits > 1) {
    // ---- split-K: publish the partial, take a ticket; the last workgroup of
    // the tile re-reads all slices (its own included) and sums them in slice
    // order, so the result does not depend on which one finishes last.
    float* mine = a.partials + (tile * a.splits + s) * (int64_t)(kRegs * 512);
    if (!idle_wave) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) mine[((i * 4 + j) * 16 + v) * 512 + tid] = acc[i][j][v];
    }
    if (diag && tid < 256) {
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
      const float* base = a.partials + (tile * a.splits) * (int64_t)(kRegs * 512);
      for (int64_t q = 0; q < a.splits; ++q) {
        const float* pq = base + q * (int64_t)(kRegs * 512);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const float x = pq[((i * 4 + j) * 16 + v) * 512 + tid];
              acc[i][j][v] = (q == 0) ? x : acc[i][j][v] + x;
            }
      }
    }
    if (diag && tid < 256) {
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
    for (int i = 0; i < 2; ++i)
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
  if (diag && a.key && tid < 256) {
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
  a.panels = plan.panels; a.tiles = plan.tiles; a.splits = plan.splits;
  a.slice_tokens = plan.slice_tokens;
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
  // the vector path needs 16-byte rows and whole channel octets
  const bool vec = (ldx % 8 == 0) && (n % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0);
  if (vec) hipLaunchKernelGGL(syrk_bf16_kernel<true>, dim3((unsigned)grid), dim3(512), 0, stream, a);
  else hipLaunchKernelGGL(syrk_bf16_kernel<false>, dim3((unsigned)grid), dim3(512), 0, stream, a);
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
