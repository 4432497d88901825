// Product of bf16 activations with the quantizer's low-bit weights (W4A16).
//
// The page "模型量化实战：从 INT8 PTQ 到 GPTQ…" §4.3 notes that 4-bit weights
// have no native matrix product: they are dequantized to a 16-bit type and
// multiplied, and the gain is the 4x smaller weight stream.  §2.1 gives the
// dequantization x̂ = (q - z)·s.  Here the 16-bit type is bf16 and the scale
// is applied per group after the product, which keeps every weight exact:
//   Y[t][r] = Σ_g s_g · ( Σ_{k∈g} x_k·(128 + q_k) - (128 + z_g)·Σ_{k∈g} x_k ).
// 128 + q (q < 16) is exactly the bf16 with bits 0x4300 | q, so a 4-bit code
// becomes an MFMA operand with one AND-OR: bf16 × bf16 products are exact in
// the fp32 accumulator, and only the group sums round.
//
// Packed weight (gptq_w4a16_pack, once per weight):
//   order  int32 [n128]            processing position -> input column (-1: pad);
//                                  groups contiguous, derived from g_idx
//   params float2 [mt][Gp][16]     (s, 128 + z) per row and group
//   codes  u32x4 [mt][kc][64]      the B operand of v_mfma_f32_16x16x32_bf16 in
//                                  lane order: lane l, word j of 128-chunk C of
//                                  row tile T holds the 8 codes of row 16T + l%16,
//                                  positions 128C + 32j + 8(l/16) + e, e = 0..7,
//                                  e in nibble (e%2)·4 + e/2, so that
//                                  ((w >> 4v) & 0x000F000F) | 0x43004300 is the
//                                  bf16 pair (e = 2v, 2v + 1)
// with mt = ceil(m/16), kc = ceil(n/128), n128 = 128·kc, Gp = ceil(n128/g).
//
// Product (gptq_w4a16_matmul), per call of up to 64 tokens:
//   gather : X' [Mp][n128] bf16 in processing order and its 32-position sums
//   gemm   : split-K over 128-chunks; a workgroup of 4 waves holds 8 row tiles
//            (128 rows) x one slice; each wave streams its codes straight from
//            HBM into registers (16 B per lane per chunk), the slice of X' and
//            the slice's scales sit in LDS; per group the accumulator is
//            scaled and folded into the result
//   reduce : Y = Σ over slices in slice order (deterministic)
#include <algorithm>
#include <mutex>
#include <vector>

#include "gptq_internal.hpp"

namespace gptq {
namespace {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kW4Rows = 16;          // rows per tile (MFMA N)
constexpr int kW4Chunk = 128;        // positions per chunk (4 MFMA k-steps of 32)
constexpr int kW4TilesPerWave = 2;
constexpr int kW4Waves = 4;
constexpr int kW4TilesPerWg = kW4TilesPerWave * kW4Waves;
constexpr int kW4MaxChunks = 4;      // chunks per slice
constexpr int kW4MaxGroups = kW4MaxChunks * 4 + 1;   // groups one slice can touch (g >= 32)
constexpr int kW4TokTile = 16;
constexpr int kW4MaxTokTiles = 4;    // tokens per launch <= 64
constexpr int kW4Pad = 8;            // bf16 padding per LDS row of X'
constexpr int kW4GemvMaxTokens = 16; // the whole-K path: X' of every position in LDS

// ---------------------------------------------------------------- pack
// One workgroup per group slot: the columns with g_idx == grp, ascending, go
// to positions grp·g ...; a count other than the group's size flags the call.
__global__ __launch_bounds__(256) void w4_order_kernel(const int32_t* __restrict__ g_idx, int64_t n,
                                                       int64_t g, int64_t G, int64_t n128,
                                                       int32_t* __restrict__ order, int* flag) {
  __shared__ int wcnt[4];
  const int64_t grp = blockIdx.x;
  const int64_t base = grp * g;
  const int64_t want = grp < G ? std::min<int64_t>(g, n - base) : 0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int64_t cnt = 0;
  for (int64_t c0 = 0; c0 < n; c0 += 256) {
    const int64_t j = c0 + threadIdx.x;
    const bool hit = j < n && (int64_t)g_idx[j] == grp;
    const uint64_t b = __ballot(hit);
    const int before = __popcll(b & ((1ull << lane) - 1ull));
    if (lane == 0) wcnt[wave] = __popcll(b);
    __syncthreads();
    int off = 0, tot = 0;
    for (int w = 0; w < 4; ++w) {
      off += w < wave ? wcnt[w] : 0;
      tot += wcnt[w];
    }
    if (hit) {
      const int64_t pos = cnt + off + before;
      if (pos < want) order[base + pos] = (int32_t)j;
    }
    cnt += tot;
    __syncthreads();
  }
  if (threadIdx.x == 0 && cnt != want) atomicOr(flag, 1);
  const int64_t end = std::min<int64_t>(base + g, n128);
  for (int64_t p = base + std::min<int64_t>(cnt, want) + threadIdx.x; p < end; p += 256)
    order[p] = -1;
}

__global__ __launch_bounds__(256) void w4_params_kernel(const float* __restrict__ scales,
                                                        const int32_t* __restrict__ zeros, int64_t m,
                                                        int64_t G, int64_t mt, int64_t Gp,
                                                        float2* __restrict__ params) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= mt * Gp * kW4Rows) return;
  const int64_t r = (i / (Gp * kW4Rows)) * kW4Rows + (i % kW4Rows);
  const int64_t grp = (i / kW4Rows) % Gp;
  float2 v = make_float2(0.f, 0.f);
  if (r < m && grp < G) v = make_float2(scales[r * G + grp], 128.f + (float)zeros[r * G + grp]);
  params[i] = v;
}

__global__ __launch_bounds__(256) void w4_codes_kernel(const uint32_t* __restrict__ qweight,
                                                       int64_t words, int64_t m, int64_t n,
                                                       int64_t kc, int64_t total,
                                                       const int32_t* __restrict__ order,
                                                       uint32_t* __restrict__ codes) {
  const int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (w >= total) return;
  const int j = (int)(w & 3), l = (int)((w >> 2) & 63);
  const int64_t tc = w >> 8;              // T·kc + C
  const int64_t T = tc / kc, C = tc % kc;
  const int64_t r = T * kW4Rows + (l & 15);
  const int64_t kb = C * kW4Chunk + 32 * j + 8 * (l >> 4);
  uint32_t word = 0;
  if (r < m) {
    for (int e = 0; e < 8; ++e) {
      const int64_t p = kb + e;
      if (p >= n) break;
      const int32_t col = order[p];
      if (col < 0) continue;
      const uint32_t q = (qweight[r * words + (col >> 3)] >> (4 * (col & 7))) & 15u;
      word |= q << (4 * ((e & 1) * 4 + (e >> 1)));
    }
  }
  codes[w] = word;
}

// ---------------------------------------------------------------- product
// X' = X[:, order] and the sum of every 32 positions, for the real tokens.
// Thread: 4 consecutive positions; 8 threads make one 32-position sum.
__global__ __launch_bounds__(256) void w4_gather_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                        const int32_t* __restrict__ order,
                                                        int64_t n128, uint16_t* __restrict__ Xp,
                                                        float* __restrict__ xs) {
  const int64_t t = blockIdx.y;
  const int64_t p0 = (int64_t)blockIdx.x * 1024 + 4 * threadIdx.x;
  if (p0 >= n128) return;   // n128 is a multiple of 128: whole 8-thread groups leave together
  uint16_t v[4];
  float s = 0.f;
  const int4 o = *reinterpret_cast<const int4*>(order + p0);
  const int oi[4] = {o.x, o.y, o.z, o.w};
  // unconditional loads (padding positions, order < 0, read column 0 and
  // drop it): all four in flight at once instead of a branch and wait each
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint16_t x = X[t * ldx + (oi[e] >= 0 ? oi[e] : 0)];
    v[e] = oi[e] >= 0 ? x : (uint16_t)0;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) s += __builtin_bit_cast(float, (uint32_t)v[e] << 16);
  uint2 pk;
  pk.x = (uint32_t)v[0] | ((uint32_t)v[1] << 16);
  pk.y = (uint32_t)v[2] | ((uint32_t)v[3] << 16);
  *reinterpret_cast<uint2*>(Xp + t * n128 + p0) = pk;
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  s += __shfl_xor(s, 4);
  if ((threadIdx.x & 7) == 0) xs[t * (n128 / 32) + (p0 >> 5)] = s;
}

struct W4GemmArgs {
  const uint16_t* Xp;      // [tokens][n128], processing order
  const float* xs;         // [tokens][n128 / 32]
  const float2* params;    // [mt][Gp][16]
  const u32x4_t* codes;    // [mt][kc][64]
  float* part;             // [splits][tokens][m16]
  int64_t tokens, m16, mt, kc, n128, Gp;
  int chunks;              // 128-chunks per slice (<= kW4MaxChunks)
};

// The empty asm keeps the unpacking at its use: hoisted out of the token-tile
// loop, the unpacked operands of every chunk would stay live (4x the VGPRs).
__device__ __forceinline__ bf16x8_t w4_unpack(uint32_t w) {
  asm volatile("" : "+v"(w));
  u32x4_t r;
  r[0] = (w & 0x000F000Fu) | 0x43004300u;
  r[1] = ((w >> 4) & 0x000F000Fu) | 0x43004300u;
  r[2] = ((w >> 8) & 0x000F000Fu) | 0x43004300u;
  r[3] = ((w >> 12) & 0x000F000Fu) | 0x43004300u;
  return __builtin_bit_cast(bf16x8_t, r);
}

// GS = 32-position steps per group (1, 2, 4 for groups of 32, 64, 128), or 0
// for one group per row.  Slices are whole 128-chunks, so with GS > 0 every
// slice starts on a group boundary and holds steps / GS whole groups.
template <int GS>
__global__ __launch_bounds__(256) void w4_gemm_kernel(W4GemmArgs a) {
  constexpr int RS = kW4MaxChunks * kW4Chunk + kW4Pad;   // LDS row of X' (bf16)
  constexpr int SS = kW4MaxChunks * 4;                   // 32-sums per LDS row
  constexpr int NG = GS > 0 ? SS / GS : 1;               // groups per slice (max)
  constexpr int PI = (kW4TilesPerWg * NG * kW4Rows + 255) / 256;   // param items per thread
  __shared__ __attribute__((aligned(16))) uint16_t xsh[kW4TokTile * RS];
  __shared__ float ssh[kW4TokTile * SS];
  __shared__ float2 psh[kW4TilesPerWg * NG * kW4Rows];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t s = blockIdx.y;
  const int64_t C0 = s * a.chunks;
  const int nch = (int)std::min<int64_t>(a.chunks, a.kc - C0);
  const int steps = 4 * nch;
  const int ng = GS > 0 ? steps / GS : 1;
  const int64_t T0 = (int64_t)blockIdx.x * kW4TilesPerWg;
  const int64_t g0 = GS > 0 ? C0 * 4 / GS : 0;

  // Every global load of the prologue is issued before the first store.  All
  // loads and LDS stores are unconditional, at indices clamped into range (a
  // load under a condition compiles to a branch and a wait of its own):
  // clamped items reload and rewrite an in-range item with its own value, and
  // tiles past the last row tile (never computed) hold the last tile's data.
  u32x4_t cw[kW4TilesPerWave][kW4MaxChunks];
#pragma unroll
  for (int r = 0; r < kW4TilesPerWave; ++r) {
    const int64_t T = std::min<int64_t>(T0 + wave * kW4TilesPerWave + r, a.mt - 1);
#pragma unroll
    for (int c = 0; c < kW4MaxChunks; ++c)
      cw[r][c] = a.codes[(T * a.kc + C0 + std::min(c, nch - 1)) * 64 + lane];
  }
  const int npar = kW4TilesPerWg * ng * kW4Rows;
  float2 pv[PI];
#pragma unroll
  for (int u = 0; u < PI; ++u) {
    const int i = std::min(tid + 256 * u, npar - 1);
    const int tl = i / (ng * kW4Rows), gi = (i / kW4Rows) % ng, rr = i % kW4Rows;
    const int64_t T = std::min<int64_t>(T0 + tl, a.mt - 1);
    pv[u] = a.params[(T * a.Gp + g0 + gi) * kW4Rows + rr];
  }
  // (their LDS stores go with the first X' tile's, so the code loads are not
  // held back behind a wait for these)

  const int row = lane & 15, quad = lane >> 4;
  const int vec_per_row = nch * (kW4Chunk / 8);   // 16-byte pieces of a row of the slice
  const int ntt = (int)((a.tokens + kW4TokTile - 1) / kW4TokTile);
  for (int tt = 0; tt < ntt; ++tt) {
    const int64_t t0 = (int64_t)tt * kW4TokTile;
    // X' tile: 16 rows x the slice.  Rows past the last token repeat the last
    // token (their outputs are never written); loads and stores at clamped
    // indices, unconditional, as above.
    const int nxv = kW4TokTile * vec_per_row, nsv = kW4TokTile * steps;
    // four named loads (an array here stays in scratch memory)
    auto xidx = [&](int u) { return std::min(tid + 256 * u, nxv - 1); };
    auto xload = [&](int u) {
      const int i = xidx(u);
      const int64_t t = std::min<int64_t>(t0 + i / vec_per_row, a.tokens - 1);
      return *reinterpret_cast<const uint4*>(a.Xp + t * a.n128 + C0 * kW4Chunk + 8 * (i % vec_per_row));
    };
    auto xstore = [&](int u, const uint4& v) {
      const int i = xidx(u);
      *reinterpret_cast<uint4*>(xsh + (i / vec_per_row) * RS + 8 * (i % vec_per_row)) = v;
    };
    const uint4 x0 = xload(0), x1 = xload(1), x2 = xload(2), x3 = xload(3);
    const int si = std::min(tid, nsv - 1);
    const float sv = a.xs[std::min<int64_t>(t0 + si / steps, a.tokens - 1) * (a.n128 / 32) + C0 * 4 + si % steps];
    if (tt > 0) __syncthreads();   // the previous tile is consumed
    if (tt == 0) {
#pragma unroll
      for (int u = 0; u < PI; ++u) psh[std::min(tid + 256 * u, npar - 1)] = pv[u];
    }
    xstore(0, x0);
    xstore(1, x1);
    xstore(2, x2);
    xstore(3, x3);
    ssh[(si / steps) * SS + si % steps] = sv;
    __syncthreads();

#pragma unroll
    for (int r = 0; r < kW4TilesPerWave; ++r) {
      const int tl = wave * kW4TilesPerWave + r;
      const int64_t T = T0 + tl;
      if (T >= a.mt) break;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < kW4MaxChunks; ++c) {
        if (c >= nch) break;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int ls = 4 * c + j;
          const uint4 av = *reinterpret_cast<const uint4*>(
              xsh + row * RS + c * kW4Chunk + 32 * j + 8 * quad);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                        w4_unpack(cw[r][c][j]), acc, 0, 0, 0);
          const bool close = GS > 0 ? (ls + 1) % GS == 0 : (c == nch - 1 && j == 3);
          if (close) {
            const int gi = GS > 0 ? ls / GS : 0;
            const int fs = GS > 0 ? ls + 1 - GS : 0;
            const float2 p = psh[(tl * ng + gi) * kW4Rows + row];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float* sp = ssh + (4 * quad + v) * SS;
              float sx = 0.f;
              if (GS > 0) {
#pragma unroll
                for (int q = 0; q < (GS > 0 ? GS : 1); ++q) sx += sp[fs + q];
              } else {
                for (int q = 0; q < steps; ++q) sx += sp[q];
              }
              y[v] = fmaf(p.x, fmaf(-p.y, sx, acc[v]), y[v]);
            }
            acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
          }
        }
      }
      // D[4·quad + v][row]: token t0 + 4·quad + v, weight row 16T + row
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t t = t0 + 4 * quad + v;
        if (t < a.tokens) a.part[(s * a.tokens + t) * a.m16 + T * kW4Rows + row] = y[v];
      }
    }
  }
}

// Few tokens (up to 16, while X' fits in LDS and all workgroups are resident
// at once): one workgroup of 8 waves per 16-row tile covers the
// whole K range, wave w a contiguous eighth of the chunks, so no partial sums
// leave the workgroup.  X' (every position, the real tokens only), its
// 32-sums and the tile's (s, 128 + z) of every group sit in LDS; each wave
// streams its codes in batches of 8 chunks, the next batch in flight while
// one computes; the 8 waves' results are added in wave order in LDS.
struct W4GemvArgs {
  const uint16_t* Xp;      // [tokens][n128]
  const float* xs;         // [tokens][n128 / 32]
  const float2* params;    // [mt][Gp][16]
  const u32x4_t* codes;    // [mt][kc][64]
  float* Y;                // [tokens][ldy]
  int64_t ldy, m, mt, kc, n128, Gp;
  int tokens;              // 1 .. kW4GemvMaxTokens
};

template <int GS>
__global__ __launch_bounds__(512) void w4_gemv_kernel(W4GemvArgs a) {
  constexpr int B = 8;                       // chunks per batch
  extern __shared__ __attribute__((aligned(16))) uint8_t w4_lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t T = blockIdx.x;
  const int xrow = (int)a.n128 + kW4Pad;     // bf16 per LDS row of X'
  const int srow = (int)(a.n128 / 32);
  uint16_t* xsh = reinterpret_cast<uint16_t*>(w4_lds);
  float* ssh = reinterpret_cast<float*>(w4_lds + (size_t)a.tokens * xrow * 2);
  float2* psh = reinterpret_cast<float2*>(ssh + a.tokens * srow + ((a.tokens * srow) & 1));
  float* red = reinterpret_cast<float*>(psh + a.Gp * kW4Rows);   // [8][64][4]

  const int cpw = (int)((a.kc + 7) / 8);
  const int c0 = wave * cpw, c1 = (int)std::min<int64_t>(a.kc, (int64_t)c0 + cpw);
  const u32x4_t* cbase = a.codes + T * a.kc * 64 + lane;

  // the first batch of codes (HBM) goes out first, so that its latency and
  // the LDS fills' below overlap; chunk indices are clamped into this wave's
  // range (an empty range loads some other chunk and never uses it)
  u32x4_t cw[B];
#pragma unroll
  for (int b = 0; b < B; ++b) cw[b] = cbase[(int64_t)std::max(0, std::min(c0 + b, c1 - 1)) * 64];
  // LDS fills: per round, twelve loads in flight per thread (X', sums,
  // params) before their stores.  Loads and stores are unconditional, at an
  // index clamped into range (past the end a thread rewrites the last element
  // with its own value): under a condition each load compiles to a branch and
  // a wait of its own.
  {
    const int vrow = (int)(a.n128 / 8);
    const int nv = a.tokens * vrow;            // 16-byte pieces of X'
    const int ns = a.tokens * srow;            // 32-sums
    const int np = (int)(a.Gp * kW4Rows);      // (s, 128 + z) pairs of the tile
    const float2* pb = a.params + T * a.Gp * kW4Rows;
    const int rounds = (std::max(nv, std::max(ns, np)) + 4 * 512 - 1) / (4 * 512);
    for (int rd = 0; rd < rounds; ++rd) {
      const int i0 = rd * 4 * 512;
      uint4 xv[4];
      float sv[4];
      float2 pv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int ix = std::min(i0 + u * 512 + tid, nv - 1);
        xv[u] = *reinterpret_cast<const uint4*>(a.Xp + (int64_t)(ix / vrow) * a.n128 + 8 * (ix % vrow));
        sv[u] = a.xs[std::min(i0 + u * 512 + tid, ns - 1)];
        pv[u] = pb[std::min(i0 + u * 512 + tid, np - 1)];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int ix = std::min(i0 + u * 512 + tid, nv - 1);
        *reinterpret_cast<uint4*>(xsh + (ix / vrow) * xrow + 8 * (ix % vrow)) = xv[u];
        ssh[std::min(i0 + u * 512 + tid, ns - 1)] = sv[u];
        psh[std::min(i0 + u * 512 + tid, np - 1)] = pv[u];
      }
    }
  }
  __syncthreads();

  const int row = lane & 15, quad = lane >> 4;
  const bool arow = row < a.tokens;           // A-operand rows past the last token are zero
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
  int fs = 4 * c0;                            // first global 32-step of the open group
  for (int cb = c0; cb < c1; cb += B) {
    u32x4_t nx[B];   // the next batch (clamped: chunks past the range are loaded, not used)
#pragma unroll
    for (int b = 0; b < B; ++b) nx[b] = cbase[(int64_t)std::min(cb + B + b, c1 - 1) * 64];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int c = cb + b;
      if (c < c1) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int st = 4 * c + j;
        uint4 av = make_uint4(0u, 0u, 0u, 0u);
        if (arow) av = *reinterpret_cast<const uint4*>(xsh + row * xrow + 32 * st + 8 * quad);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                      w4_unpack(cw[b][j]), acc, 0, 0, 0);
        const bool close = GS > 0 ? (st + 1) % GS == 0 : (c == c1 - 1 && j == 3);
        if (close) {
          const int grp = GS > 0 ? st / GS : 0;
          const float2 p = psh[grp * kW4Rows + row];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int t = 4 * quad + v;
            float sx = 0.f;
            if (t < a.tokens) {
              const float* sp = ssh + t * srow;
              if (GS > 0) {
#pragma unroll
                for (int q = 0; q < (GS > 0 ? GS : 1); ++q) sx += sp[st + 1 - GS + q];
              } else {
                for (int q = fs; q <= st; ++q) sx += sp[q];
              }
            }
            y[v] = fmaf(p.x, fmaf(-p.y, sx, acc[v]), y[v]);
          }
          acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
          fs = st + 1;
        }
      }
      }
    }
#pragma unroll
    for (int b = 0; b < B; ++b) cw[b] = nx[b];
  }

  // D[4·quad + v][row]: token 4·quad + v; the waves' sums in wave order
#pragma unroll
  for (int v = 0; v < 4; ++v) red[(wave * 64 + lane) * 4 + v] = y[v];
  __syncthreads();
  if (tid < 64) {
    const int t0 = 4 * (tid >> 4);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int t = t0 + v;
      const int64_t r = T * kW4Rows + (tid & 15);
      if (t < a.tokens && r < a.m) {
        float sum = 0.f;
        for (int w = 0; w < 8; ++w) sum += red[(w * 64 + tid) * 4 + v];
        a.Y[t * a.ldy + r] = sum;
      }
    }
  }
}

// Y = Σ over slices in slice order; eight loads in flight per thread.
__global__ __launch_bounds__(256) void w4_reduce_kernel(const float* __restrict__ part, int64_t splits,
                                                        int64_t tokens, int64_t m16, int64_t m,
                                                        float* __restrict__ Y, int64_t ldy) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t t = blockIdx.y;
  if (r >= m) return;
  const int64_t stride = tokens * m16;
  const float* p = part + t * m16 + r;
  float acc = 0.f;
  int64_t s = 0;
  for (; s + 8 <= splits; s += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[(s + u) * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  for (; s < splits; ++s) acc += p[s * stride];
  Y[t * ldy + r] = acc;
}

}  // namespace

constexpr size_t kW4GemvMaxLds = 150 * 1024;

size_t w4_gemv_lds(int64_t tokens, const W4Layout& L) {
  const size_t x = (size_t)tokens * (size_t)(L.n128 + kW4Pad) * 2;
  const size_t sc = (size_t)tokens * (size_t)(L.n128 / 32);
  return x + (sc + (sc & 1)) * 4 + (size_t)L.Gp * kW4Rows * sizeof(float2) + 8 * 64 * 4 * sizeof(float);
}

W4Layout plan_w4a16(int64_t m, int64_t n, int32_t group_size) {
  W4Layout L;
  L.m = m;
  L.n = n;
  L.mt = ceil_div(m, kW4Rows);
  L.kc = ceil_div(n, kW4Chunk);
  L.n128 = L.kc * kW4Chunk;
  L.g = group_size == -1 ? L.n128 : group_size;
  L.G = group_size == -1 ? 1 : ceil_div(n, group_size);
  L.Gp = ceil_div(L.n128, L.g);
  L.flag_off = 0;
  L.order_off = 256;
  L.param_off = L.order_off + align256((size_t)L.n128 * sizeof(int32_t));
  L.code_off = L.param_off + align256((size_t)(L.mt * L.Gp * kW4Rows) * sizeof(float2));
  L.total = L.code_off + (size_t)(L.mt * L.kc) * 64 * sizeof(u32x4_t);
  return L;
}

W4GemmPlan plan_w4a16_gemm(int64_t tokens, int64_t m, int64_t n, int64_t max_chunk_tokens) {
  W4GemmPlan p;
  p.chunk_tokens = std::min<int64_t>(std::max<int64_t>(tokens, 1),
                                     std::min<int64_t>(max_chunk_tokens, (int64_t)kW4TokTile * kW4MaxTokTiles));
  p.mp = p.chunk_tokens;
  const int64_t mt = ceil_div(m, kW4Rows), kc = ceil_div(n, kW4Chunk);
  const int64_t wgs_rows = ceil_div(mt, kW4TilesPerWg);
  // chunks per slice: the largest (<= 4) that still gives >= 512 workgroups
  p.chunks = kW4MaxChunks;
  while (p.chunks > 1 && wgs_rows * ceil_div(kc, p.chunks) < 512) p.chunks /= 2;
  p.splits = ceil_div(kc, p.chunks);
  const int64_t n128 = kc * kW4Chunk, m16 = mt * kW4Rows;
  p.xp_off = 0;
  p.xs_off = align256((size_t)(p.mp * n128) * sizeof(uint16_t));
  p.part_off = p.xs_off + align256((size_t)(p.mp * (n128 / 32)) * sizeof(float));
  p.total = p.part_off + (size_t)(p.splits * p.chunk_tokens * m16) * sizeof(float);
  return p;
}

gptq_status run_w4a16_pack(const uint32_t* qweight, const float* scales, const int32_t* zeros,
                           const int32_t* g_idx, int bits, const W4Layout& L, void* packed,
                           hipStream_t stream) {
  (void)bits;
  char* base = static_cast<char*>(packed);
  int* flag = reinterpret_cast<int*>(base + L.flag_off);
  int32_t* order = reinterpret_cast<int32_t*>(base + L.order_off);
  GPTQ_HIP_CHECK(hipMemsetAsync(flag, 0, sizeof(int), stream));
  hipLaunchKernelGGL(w4_order_kernel, dim3((unsigned)L.Gp), dim3(256), 0, stream, g_idx, L.n, L.g,
                     L.G, L.n128, order, flag);
  GPTQ_LAUNCH_CHECK();
  const int64_t np = L.mt * L.Gp * kW4Rows;
  hipLaunchKernelGGL(w4_params_kernel, dim3((unsigned)ceil_div(np, 256)), dim3(256), 0, stream,
                     scales, zeros, L.m, L.G, L.mt, L.Gp,
                     reinterpret_cast<float2*>(base + L.param_off));
  GPTQ_LAUNCH_CHECK();
  const int64_t nw = L.mt * L.kc * 256;
  hipLaunchKernelGGL(w4_codes_kernel, dim3((unsigned)ceil_div(nw, 256)), dim3(256), 0, stream,
                     qweight, ceil_div(L.n, 8), L.m, L.n, L.kc, nw, (const int32_t*)order,
                     reinterpret_cast<uint32_t*>(base + L.code_off));
  GPTQ_LAUNCH_CHECK();
  int hflag = 0;
  GPTQ_HIP_CHECK(hipMemcpyAsync(&hflag, flag, sizeof(int), hipMemcpyDeviceToHost, stream));
  GPTQ_HIP_CHECK(hipStreamSynchronize(stream));
  if (hflag) {
    set_error("gptq_w4a16_pack: g_idx does not split the columns into groups of the group size "
              "(group p must hold min(g, n - p·g) columns)");
    return GPTQ_ERR_INVALID_ARG;
  }
  return GPTQ_OK;
}

gptq_status run_w4a16_matmul(const uint16_t* X, int64_t tokens, int64_t ldx, const void* packed,
                             const W4Layout& L, float* Y, int64_t ldy, void* ws,
                             const W4GemmPlan& p, hipStream_t stream) {
  const char* base = static_cast<const char*>(packed);
  char* w = static_cast<char*>(ws);
  uint16_t* Xp = reinterpret_cast<uint16_t*>(w + p.xp_off);
  float* xs = reinterpret_cast<float*>(w + p.xs_off);
  float* part = reinterpret_cast<float*>(w + p.part_off);
  W4GemmArgs a;
  a.Xp = Xp;
  a.xs = xs;
  a.params = reinterpret_cast<const float2*>(base + L.param_off);
  a.codes = reinterpret_cast<const u32x4_t*>(base + L.code_off);
  a.part = part;
  a.m16 = L.mt * kW4Rows;
  a.mt = L.mt;
  a.kc = L.kc;
  a.n128 = L.n128;
  a.Gp = L.Gp;
  a.chunks = (int)p.chunks;
  const int32_t* order = reinterpret_cast<const int32_t*>(base + L.order_off);
  const int gsteps = L.g >= L.n128 ? 0 : (int)(L.g / 32);
  // few tokens: gather, then one product kernel over the whole K range
  const size_t gemv_lds = w4_gemv_lds(tokens, L);
  // while its X' fits in LDS and every workgroup is resident at once
  const int64_t resident = 256 * std::max<int64_t>(1, (int64_t)(160 * 1024 / std::max<size_t>(gemv_lds, 1)));
  if (tokens <= kW4GemvMaxTokens && gemv_lds <= kW4GemvMaxLds && L.mt <= resident) {
    hipLaunchKernelGGL(w4_gather_kernel, dim3((unsigned)ceil_div(L.n128, 1024), (unsigned)tokens),
                       dim3(256), 0, stream, X, ldx, order, L.n128, Xp, xs);
    GPTQ_LAUNCH_CHECK();
    W4GemvArgs g;
    g.Xp = Xp; g.xs = xs; g.params = a.params; g.codes = a.codes; g.Y = Y; g.ldy = ldy;
    g.m = L.m; g.mt = L.mt; g.kc = L.kc; g.n128 = L.n128; g.Gp = L.Gp; g.tokens = (int)tokens;
    const void* fn = nullptr;
    switch (gsteps) {
      case 1: fn = (const void*)w4_gemv_kernel<1>; break;
      case 2: fn = (const void*)w4_gemv_kernel<2>; break;
      case 4: fn = (const void*)w4_gemv_kernel<4>; break;
      case 0: fn = (const void*)w4_gemv_kernel<0>; break;
      default:
        set_error("group width %lld not built", (long long)L.g);
        return GPTQ_ERR_UNSUPPORTED;
    }
    if (gemv_lds > 65536)
      GPTQ_HIP_CHECK(hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)gemv_lds));
    switch (gsteps) {
      case 1: hipLaunchKernelGGL(w4_gemv_kernel<1>, dim3((unsigned)L.mt), dim3(512), gemv_lds, stream, g); break;
      case 2: hipLaunchKernelGGL(w4_gemv_kernel<2>, dim3((unsigned)L.mt), dim3(512), gemv_lds, stream, g); break;
      case 4: hipLaunchKernelGGL(w4_gemv_kernel<4>, dim3((unsigned)L.mt), dim3(512), gemv_lds, stream, g); break;
      default: hipLaunchKernelGGL(w4_gemv_kernel<0>, dim3((unsigned)L.mt), dim3(512), gemv_lds, stream, g); break;
    }
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
  }
  for (int64_t t0 = 0; t0 < tokens; t0 += p.chunk_tokens) {
    const int64_t tk = std::min<int64_t>(p.chunk_tokens, tokens - t0);
    hipLaunchKernelGGL(w4_gather_kernel, dim3((unsigned)ceil_div(L.n128, 1024), (unsigned)tk),
                       dim3(256), 0, stream, X + t0 * ldx, ldx, order, L.n128, Xp, xs);
    GPTQ_LAUNCH_CHECK();
    a.tokens = tk;
    const dim3 grid((unsigned)ceil_div(L.mt, kW4TilesPerWg), (unsigned)p.splits);
    switch (gsteps) {
      case 1: hipLaunchKernelGGL(w4_gemm_kernel<1>, grid, dim3(256), 0, stream, a); break;
      case 2: hipLaunchKernelGGL(w4_gemm_kernel<2>, grid, dim3(256), 0, stream, a); break;
      case 4: hipLaunchKernelGGL(w4_gemm_kernel<4>, grid, dim3(256), 0, stream, a); break;
      case 0: hipLaunchKernelGGL(w4_gemm_kernel<0>, grid, dim3(256), 0, stream, a); break;
      default:
        set_error("group width %lld not built", (long long)L.g);
        return GPTQ_ERR_UNSUPPORTED;
    }
    GPTQ_LAUNCH_CHECK();
    hipLaunchKernelGGL(w4_reduce_kernel, dim3((unsigned)ceil_div(L.m, 256), (unsigned)tk), dim3(256),
                       0, stream, (const float*)part, p.splits, tk, a.m16, L.m, Y + t0 * ldy, ldy);
    GPTQ_LAUNCH_CHECK();
  }
  return GPTQ_OK;
}

// ---------------------------------------------------------------------------
// The product without caller workspace (gptq_w4a16_matmul_noalloc), for
// callers that cannot allocate device memory: its gather, partial sums and
// per-32-position sums live in this file-scope array, one copy per GPU, held
// until the process ends.  Host code never passes the array's name to a
// kernel (in host code it is only a stand-in for the symbol): each device's
// address comes from hipGetSymbolAddress, taken once per device with that
// device current, and every launch gets that address.  Nothing in the array
// needs to start at zero (every byte a call reads it wrote first), and calls
// that overlap on one GPU race on it.
// ---------------------------------------------------------------------------
constexpr size_t kW4NoAllocScratchBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kW4NoAllocScratchBytes];

namespace {
gptq_status noalloc_scratch(void** out) {
  static std::mutex mu;
  static std::vector<void*> per_device;
  int dev = 0;
  GPTQ_HIP_CHECK(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lock(mu);
  if ((int)per_device.size() <= dev) per_device.resize(dev + 1, nullptr);
  if (per_device[dev] == nullptr) {
    void* ptr = nullptr;
    GPTQ_HIP_CHECK(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    per_device[dev] = ptr;
  }
  *out = per_device[dev];
  return GPTQ_OK;
}
}  // namespace

size_t w4a16_noalloc_scratch_bytes() { return kW4NoAllocScratchBytes; }

W4GemmPlan plan_w4a16_noalloc(int64_t tokens, int64_t m, int64_t n) {
  // fewer tokens per launch sequence when 64 would not fit the array
  W4GemmPlan p = plan_w4a16_gemm(tokens, m, n);
  for (int64_t chunk = p.chunk_tokens / 2; p.total > kW4NoAllocScratchBytes && chunk >= kW4TokTile; chunk /= 2)
    p = plan_w4a16_gemm(tokens, m, n, chunk);
  return p;
}

gptq_status run_w4a16_matmul_noalloc(const uint16_t* X, int64_t tokens, int64_t ldx, const void* packed,
                                     const W4Layout& L, float* Y, int64_t ldy, hipStream_t stream) {
  const W4GemmPlan p = plan_w4a16_noalloc(tokens, L.m, L.n);
  if (p.total > kW4NoAllocScratchBytes) {
    set_error("gptq_w4a16_matmul_noalloc: a %lld x %lld weight needs %zu bytes of scratch at 16 tokens "
              "per launch; the library holds %zu (use gptq_w4a16_matmul with a workspace)",
              (long long)L.m, (long long)L.n, p.total, kW4NoAllocScratchBytes);
    return GPTQ_ERR_UNSUPPORTED;
  }
  void* ws = nullptr;
  GPTQ_TRY(noalloc_scratch(&ws));
  return run_w4a16_matmul(X, tokens, ldx, packed, L, Y, ldy, ws, p, stream);
}

}  // namespace gptq
