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
//            (128 rows) x one slice x every token; X', its sums, the codes and
//            the scales of each chunk are copied straight into an LDS ring;
//            per group the accumulator is scaled and folded into the result;
//            partial results leave in the MFMA's own lane layout
//   reduce : Y = Σ over slices in slice order (deterministic)
#include <algorithm>
#include <mutex>
#include <vector>

#include "gptq_internal.hpp"

namespace gptq {
namespace {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kW4Rows = 16;          // rows per tile (MFMA N)
constexpr int kW4Chunk = 128;        // positions per chunk (4 MFMA k-steps of 32)
constexpr int kW4Waves = 4;           // waves per workgroup that split the rows (x2 when the tokens split too)
constexpr int kW4TilesPerWave = 2;
constexpr int kW4TilesPerWg = kW4Waves * kW4TilesPerWave;   // 128 rows per workgroup
constexpr int kW4Ring = 4;           // LDS ring slots of the split-K product (chunks in flight + 1)
constexpr int kW4TargetWgs = 256;    // split-K: slices so that about this many workgroups run
constexpr int kW4TokTile = 16;
constexpr int kW4MaxTokTiles = 4;    // tokens per launch <= 64
constexpr int kW4Pad = 8;            // bf16 padding per LDS row of X'
constexpr int kW4XRow = kW4Chunk + kW4Pad;   // bf16 per LDS row of one X' chunk
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
// Workgroup L covers positions 1024·part ... of token t, with the
// workgroups of one token on one XCD (dispatch goes round-robin over the 8
// XCDs, L % 8): its row of X (read in scattered 2-byte pieces) then comes
// from memory once, into that XCD's L2, instead of once per XCD.
// wpt = workgroups per token; the grid is 8·ceil(tokens/8)·wpt.
__global__ __launch_bounds__(256) void w4_gather_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                        const int32_t* __restrict__ order,
                                                        int64_t n128, uint16_t* __restrict__ Xp,
                                                        float* __restrict__ xs, float* __restrict__ xs4,
                                                        int64_t tokens, int wpt) {
  const int64_t L = blockIdx.x, q = L >> 3;
  const int64_t t = (L & 7) + 8 * (q / wpt);
  if (t >= tokens) return;
  const int64_t p0 = (q % wpt) * 1024 + 4 * threadIdx.x;
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
  // the 128-position sum ((s0 + s1) + s2) + s3 of the four 32-sums, for
  // groups of 128 (32 threads; n128 is a multiple of 128, so whole 32-thread
  // blocks leave together above)
  const float s1 = __shfl_down(s, 8), s2 = __shfl_down(s, 16), s3 = __shfl_down(s, 24);
  if ((threadIdx.x & 31) == 0) xs4[t * (n128 / 128) + (p0 >> 7)] = ((s + s1) + s2) + s3;
}

struct W4GemmArgs {
  const uint16_t* Xp;      // [tokens][n128], processing order
  const float* xs;         // [tokens][n128 / 32]
  const float* xs4;        // [tokens][n128 / 128]
  const float2* params;    // [mt][Gp][16]
  const u32x4_t* codes;    // [mt][kc][64]
  float* part;             // [splits][mt][TT][64 lanes][4]: the D fragments of every 16 x 16 tile
  int64_t tokens, mt, kc, n128, Gp;
  int64_t nrb, splits;     // 128-row blocks, K-slices (nrb·splits workgroups)
  int chunks;              // 128-chunks per slice
};

// Workgroup -> (row block, slice).  Dispatch deals workgroups round-robin
// to the 8 XCDs (workgroup i runs on XCD i mod 8); when the slice count is a
// multiple of 8, every workgroup of slice s runs on XCD s mod 8, so each
// XCD's L2 holds the X' columns of its own slices only (one miss per line
// per XCD instead of one per line on every XCD).  Both are wave-uniform
// (scalar registers), so the buffer descriptors built from them are too.
__device__ __forceinline__ void w4_block_coords(const W4GemmArgs& a, int64_t& rb, int64_t& s) {
  const uint32_t i = blockIdx.x, nrb = (uint32_t)a.nrb;
  uint32_t r, t;
  if ((a.splits & 7) == 0) {
    const uint32_t q = i >> 3;
    t = (i & 7) + 8 * (q / nrb);
    r = q % nrb;
  } else {
    r = i % nrb;
    t = i / nrb;
  }
  rb = __builtin_amdgcn_readfirstlane(r);
  s = __builtin_amdgcn_readfirstlane(t);
}

// The empty asm keeps the unpacking at its use: hoisted out of the token-tile
// loop, the unpacked operands of every chunk would stay live (4x the VGPRs).
// Each word is (shifted codes & 0x000F000F) | 0x43004300, one v_and_or_b32:
// gfx9 VOP3 takes no literal, so both constants must sit in registers, and
// with them visible as constants the compiler folds them and emits an AND and
// an OR.  W4Consts hides them (an empty asm that claims to change them, no
// instruction) once per kernel, outside every loop.
struct W4Consts {
  uint32_t m, c;
  __device__ __forceinline__ W4Consts() : m(0x000F000Fu), c(0x43004300u) {
    asm volatile("" : "+v"(m), "+v"(c));
  }
};
__device__ __forceinline__ bf16x8_t w4_unpack(uint32_t w, const W4Consts& k) {
  asm volatile("" : "+v"(w));
  const uint32_t m = k.m, c = k.c;
  u32x4_t r;
  r[0] = (w & m) | c;
  r[1] = ((w >> 4) & m) | c;
  r[2] = ((w >> 8) & m) | c;
  r[3] = ((w >> 12) & m) | c;
  return __builtin_bit_cast(bf16x8_t, r);
}

// s_waitcnt vmcnt(n) with the other counters left free
__device__ __forceinline__ constexpr int w4_vmcnt(int n) {
  return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

// One ring slot of the split-K product: the chunk's X' (TT·16 token rows of
// 16 pieces of 16 B; row t's piece p sits in slot p ^ (t mod 16), so the
// A-operand reads of 16 consecutive rows hit distinct banks), its 32-sums
// (64 tokens x 4), the codes of every row tile (1 KB each) and the group
// parameters of every row tile (4 groups x 16 rows x (s, 128 + z), 512 B).
// TS: the workgroup's waves split the tokens TS ways (4·TS waves, each with
// TT/TS token tiles of its row pair); the copies are spread over all of them.
template <int GS, int TT, int TS>
struct W4Slot {
  static constexpr int kX = TT * 16 * 256;
  static constexpr int kS = kX;
  static constexpr int kC = kS + 64 * 4 * 4;
  static constexpr int kP = kC + kW4TilesPerWg * 1024;
  static constexpr int kBytes = kP + kW4TilesPerWg * 512;
  // 256-byte copies of one row tile's parameters per chunk: the chunk's
  // groups (4 for g = 32, else 1 or 2) are 128 bytes each
  static constexpr int kPCopies = GS == 1 ? 2 : 1;
  static constexpr int kWaves = 4 * TS;
  static constexpr int kTilesPerWave = TT / TS;                  // token tiles each wave multiplies
  static constexpr int kCopyTiles = kW4TilesPerWg / kWaves;      // row tiles each wave copies
  static_assert(TT % TS == 0, "token tiles split evenly");
  // copies per wave per chunk: X', sums, and codes and params per copied row tile
  static constexpr int kCopies = kTilesPerWave + 1 + (1 + kPCopies) * kCopyTiles;
};

// Split-K product for up to 64 tokens.  Workgroup (rb, s): rows 128·rb ..
// 128·rb + 127 (wave w: row tiles 8·rb + 2w, + 1) x slice s (chunks
// [s·chunks, ...)),
// every token of the launch at once (TT tiles of 16).  Every operand a chunk
// needs -- X', its 32-position sums, the codes and the group parameters --
// is copied from memory straight into LDS (buffer loads with an LDS
// destination) through a ring of kW4Ring slots, kW4Ring - 1 chunks in flight
// while one is multiplied; no register waits for a load, so nothing but the
// explicit vmcnt below orders them.  Tokens past the last read as zero (the
// X' and sum descriptors end at the last token).  Every code is
// read once and every X' byte once per 128 rows; each A fragment feeds both
// of a wave's row tiles.
// GS = 32-position steps per group (1, 2, 4 for groups of 32, 64, 128), or 0
// for one group per row.  A group of GS > 0 lies inside one chunk (chunks are
// 128 positions, group starts are multiples of g), so a chunk closes 4/GS
// groups; GS = 0 closes its one group at the end of the slice (the per-group
// formula is linear, so each slice applies s and 128 + z to its own part).
template <int GS, int TT, int TS>
__device__ __forceinline__ void w4_ring_stream(const W4GemmArgs& a, int64_t rb, int64_t sl,
                                               f32x4_t (&y)[kW4TilesPerWave][TT / TS],
                                               uint8_t* __restrict__ s0, uint8_t* __restrict__ s1,
                                               uint8_t* __restrict__ s2, uint8_t* __restrict__ s3) {
  using Sl = W4Slot<GS, TT, TS>;
  constexpr int K = Sl::kCopies;
  constexpr int RT = kW4TilesPerWave;
  constexpr int TW = Sl::kTilesPerWave;
  constexpr int CT = Sl::kCopyTiles;
  constexpr int NP = GS > 0 ? 4 / GS : 1;   // groups closed per chunk
  const int lane = threadIdx.x & 63;
  // wave-uniform (a scalar register): the buffer descriptors below are then
  // uniform and each copy is one instruction
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  // the wave multiplies row tiles RT·rg .. RT·rg + RT - 1 of the workgroup
  // by token tiles TW·th .. TW·th + TW - 1
  const int rg = wave & 3, th = wave >> 2;
  const int row = lane & 15, quad = lane >> 4;
  const int64_t C0 = sl * a.chunks;
  const int nch = (int)std::min<int64_t>(a.chunks, a.kc - C0);
  const int64_t spr = a.n128 / 32;   // 32-sums per token
  auto clamp32 = [](int64_t b) { return (int32_t)std::min<int64_t>(b, 0x7fffffff); };
  // descriptors, once: tokens past the last read as zero (descriptor bounds)
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.Xp + C0 * kW4Chunk), 0, clamp32(a.tokens * a.n128 * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rs =
      GS == 4 ? __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.xs4 + C0), 0,
                                                  clamp32(a.tokens * (a.n128 / 128) * 4), 0x00020000)
              : __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.xs + C0 * 4), 0,
                                                  clamp32(a.tokens * spr * 4), 0x00020000);
  // the row tiles this wave copies: CT·wave .. CT·wave + CT - 1
  __amdgpu_buffer_rsrc_t rc[CT], rp[CT];
#pragma unroll
  for (int r = 0; r < CT; ++r) {
    // row tiles past the last compute on it and store nothing
    const int64_t T = std::min<int64_t>(rb * kW4TilesPerWg + wave * CT + r, a.mt - 1);
    rc[r] = __builtin_amdgcn_make_buffer_rsrc(const_cast<u32x4_t*>(a.codes + (T * a.kc + C0) * 64), 0,
                                              nch * 1024, 0x00020000);
    rp[r] = __builtin_amdgcn_make_buffer_rsrc(const_cast<float2*>(a.params + T * a.Gp * kW4Rows), 0,
                                              clamp32(a.Gp * kW4Rows * 8), 0x00020000);
  }
  // this lane's pieces of the X' copies: piece q = (w·TW + u)·64 + lane is row
  // q / 16, LDS slot q % 16, which holds X' piece (q % 16) ^ (row % 16)
  int32_t xoff[TW];
#pragma unroll
  for (int u = 0; u < TW; ++u) {
    const int q = (wave * TW + u) * 64 + lane, t = q >> 4, pc = (q & 15) ^ (t & 15);
    xoff[u] = clamp32((int64_t)t * a.n128 * 2 + pc * 16);
  }
  // this lane's sum: GS = 4, the 128-sum of token `lane` (every wave writes
  // the same 64 to one place); else the 32-sum of token sf / 4, step sf % 4
  // (waves 4.. write the same quarters as waves 0..3)
  const int sf = (wave & 3) * 64 + lane;
  const int32_t soff = GS == 4 ? clamp32((int64_t)lane * (a.n128 / 128) * 4)
                               : clamp32(((int64_t)(sf >> 2) * spr + (sf & 3)) * 4);

  // chunk c of the slice -> slot; steps past the slice re-read its last
  // chunk (nobody uses it).  Always K copies, so the vmcnt bookkeeping is the
  // same on every step.
  auto issue = [&](int c, uint8_t* slot) {
    const int cl = std::min(c, nch - 1);
#pragma unroll
    for (int u = 0; u < TW; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t*)(slot + (wave * TW + u) * 1024), 16,
                                              xoff[u] + cl * kW4Chunk * 2, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(slot + Sl::kS + (GS == 4 ? 0 : (wave & 3) * 256)), 4,
                                            soff + cl * (GS == 4 ? 4 : 16), 0, 0, 0);
    const int64_t g0 = GS > 0 ? (C0 + cl) * 4 / GS : 0;
#pragma unroll
    for (int r = 0; r < CT; ++r) {
      const int tl = wave * CT + r;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rc[r], (lds_void_t*)(slot + Sl::kC + tl * 1024), 16,
                                              (cl * 64 + lane) * 16, 0, 0, 0);
#pragma unroll
      for (int k = 0; k < Sl::kPCopies; ++k)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rp[r], (lds_void_t*)(slot + Sl::kP + tl * 512 + k * 256), 4,
                                                clamp32(g0 * kW4Rows * 8 + (k * 64 + lane) * 4), 0, 0, 0);
    }
  };

  const W4Consts kc;
  f32x4_t acc[RT][TW], sxa[TW];
#pragma unroll
  for (int tt = 0; tt < TW; ++tt) {
    sxa[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < RT; ++r) acc[r][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  float2 p0[RT];   // GS = 0: each row tile's (s, 128 + z)
#pragma unroll
  for (int r = 0; r < RT; ++r) p0[r] = make_float2(0.f, 0.f);
  auto compute = [&](const uint8_t* cur) {
    // every operand of the chunk from LDS first (one wait), then the MFMAs
    u32x4_t cw[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r)
      cw[r] = *reinterpret_cast<const u32x4_t*>(cur + Sl::kC + (rg * RT + r) * 1024 + lane * 16);
    // token tile tt of this wave is tile TW·th + tt of the chunk
    uint4 av[4][TW];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int tt = 0; tt < TW; ++tt)
        av[j][tt] = *reinterpret_cast<const uint4*>(
            cur + ((16 * (TW * th + tt) + row) * 16 + ((4 * j + quad) ^ row)) * 16);
    // GS = 4: s4[tt][v] = the 128-sum of token 16·tt' + 4·quad + v; else
    // sm[tt][v] = its 4 step sums
    f32x4_t sm[TW][4], s4[TW];
#pragma unroll
    for (int tt = 0; tt < TW; ++tt) {
      const int tg = TW * th + tt;
      if (GS == 4) {
        s4[tt] = *reinterpret_cast<const f32x4_t*>(cur + Sl::kS + (16 * tg + 4 * quad) * 4);
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          sm[tt][v] = *reinterpret_cast<const f32x4_t*>(cur + Sl::kS + (16 * tg + 4 * quad + v) * 16);
      }
    }
    float2 pp[RT][NP];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int q = 0; q < NP; ++q)
        pp[r][q] = reinterpret_cast<const float2*>(cur + Sl::kP + (rg * RT + r) * 512)[q * kW4Rows + row];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const bf16x8_t bw = w4_unpack(cw[r][j], kc);
#pragma unroll
        for (int tt = 0; tt < TW; ++tt)
          acc[r][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[j][tt]), bw,
                                                               acc[r][tt], 0, 0, 0);
      }
      if (GS > 0 && (j + 1) % (GS > 0 ? GS : 1) == 0) {
#pragma unroll
        for (int tt = 0; tt < TW; ++tt)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            float sx;
            if (GS == 4) {
              sx = s4[tt][v];
            } else {
              sx = sm[tt][v][j + 1 - (GS > 0 ? GS : 1)];
#pragma unroll
              for (int q = 1; q < (GS > 0 ? GS : 1); ++q) sx += sm[tt][v][j + 1 - GS + q];
            }
#pragma unroll
            for (int r = 0; r < RT; ++r) {
              const float2 p = pp[r][GS > 0 ? j / GS : 0];
              y[r][tt][v] = fmaf(p.x, fmaf(-p.y, sx, acc[r][tt][v]), y[r][tt][v]);
            }
          }
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
          for (int tt = 0; tt < TW; ++tt) acc[r][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
    if (GS == 0) {   // one group per row: the slice's running 32-sums
#pragma unroll
      for (int tt = 0; tt < TW; ++tt)
#pragma unroll
        for (int v = 0; v < 4; ++v) sxa[tt][v] += ((sm[tt][v][0] + sm[tt][v][1]) + sm[tt][v][2]) + sm[tt][v][3];
#pragma unroll
      for (int r = 0; r < RT; ++r) p0[r] = pp[r][0];
    }
  };
  // One step: this wave's copies of chunk c are the oldest K of the 3K in
  // flight; after the barrier every wave's are in LDS and every wave has
  // finished reading the slot of chunk c - 1, which chunk c + 3 now refills.
  auto step = [&](int c, const uint8_t* cur, uint8_t* refill) {
    __builtin_amdgcn_s_waitcnt(w4_vmcnt(K * (kW4Ring - 2)));
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    issue(c + kW4Ring - 1, refill);
    if (c < nch) compute(cur);
  };
  issue(0, s0);
  issue(1, s1);
  issue(2, s2);
  // the chunk count is rounded up to whole turns of the ring: steps past the
  // slice only wait, meet and refill
  for (int c = 0; c < nch; c += kW4Ring) {
    step(c, s0, s3);
    step(c + 1, s1, s0);
    step(c + 2, s2, s1);
    step(c + 3, s3, s2);
  }
  __builtin_amdgcn_s_waitcnt(w4_vmcnt(0));   // no copy may land after the workgroup ends
  if (GS == 0) {
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int tt = 0; tt < TW; ++tt)
#pragma unroll
        for (int v = 0; v < 4; ++v) y[r][tt][v] = p0[r].x * fmaf(-p0[r].y, sxa[tt][v], acc[r][tt][v]);
  }
}

template <int GS, int TT, int TS>
__global__ __launch_bounds__(256 * TS) void w4_gemm_kernel(W4GemmArgs a) {
  using Sl = W4Slot<GS, TT, TS>;
  constexpr int TW = Sl::kTilesPerWave;
  __shared__ __attribute__((aligned(16))) uint8_t s0[Sl::kBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s1[Sl::kBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s2[Sl::kBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s3[Sl::kBytes];
  f32x4_t y[kW4TilesPerWave][TW];
#pragma unroll
  for (int r = 0; r < kW4TilesPerWave; ++r)
#pragma unroll
    for (int tt = 0; tt < TW; ++tt) y[r][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  int64_t rb, sl;
  w4_block_coords(a, rb, sl);
  w4_ring_stream<GS, TT, TS>(a, rb, sl, y, s0, s1, s2, s3);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rg = wave & 3, th = wave >> 2;
  // lane l's D fragment of tile (T, tt): tokens 16·tt + 4·(l/16) + v, v = 0..3,
  // of weight row 16T + l % 16; one 16-byte store each (tokens past the last
  // hold zeros and are never read)
#pragma unroll
  for (int r = 0; r < kW4TilesPerWave; ++r) {
    const int64_t T = rb * kW4TilesPerWg + rg * kW4TilesPerWave + r;
    if (T < a.mt) {
#pragma unroll
      for (int tt = 0; tt < TW; ++tt)
        *reinterpret_cast<f32x4_t*>(a.part + (((sl * a.mt + T) * TT + TW * th + tt) * 64 + lane) * 4) = y[r][tt];
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
  const W4Consts kc;
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
                                                      w4_unpack(cw[b][j], kc), acc, 0, 0, 0);
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

// Y = Σ over slices in slice order.  Thread (r, q): weight row r, tokens
// 4q .. 4q + 3, one 16-byte fragment per slice (lane 16·(q % 4) + r % 16 of
// tile (r / 16, q / 4)); eight loads in flight.
__global__ __launch_bounds__(256) void w4_reduce_kernel(const float* __restrict__ part, int64_t splits,
                                                        int64_t mt, int tt_count, int64_t tokens, int64_t m,
                                                        float* __restrict__ Y, int64_t ldy) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t q = blockIdx.y;
  if (r >= m) return;
  const int64_t stride = mt * tt_count * 64;   // fragments per slice
  const f32x4_t* p = reinterpret_cast<const f32x4_t*>(part) +
                     ((r >> 4) * tt_count + (q >> 2)) * 64 + (q & 3) * 16 + (r & 15);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  int64_t s = 0;
  for (; s + 8 <= splits; s += 8) {
    f32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[(s + u) * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  for (; s < splits; ++s) acc += p[s * stride];
#pragma unroll
  for (int v = 0; v < 4; ++v)
    if (4 * q + v < tokens) Y[(4 * q + v) * ldy + r] = acc[v];
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
  // slices: about kW4TargetWgs workgroups in all, whole chunks per slice
  const int64_t want = std::max<int64_t>(1, std::min<int64_t>(kc, ceil_div(kW4TargetWgs, wgs_rows)));
  p.chunks = ceil_div(kc, want);
  p.splits = ceil_div(kc, p.chunks);
  const int64_t n128 = kc * kW4Chunk, m16 = mt * kW4Rows;
  p.xp_off = 0;
  p.xs_off = align256((size_t)(p.mp * n128) * sizeof(uint16_t));
  // 32-position sums, then 128-position sums
  p.part_off = p.xs_off + align256((size_t)(p.mp * (n128 / 32 + n128 / 128)) * sizeof(float));
  // partial results: whole 16-token tiles
  p.total = p.part_off + (size_t)(p.splits * kW4TokTile * ceil_div(p.chunk_tokens, kW4TokTile) * m16) * sizeof(float);
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

gptq_status launch_w4_gather(const uint16_t* X, int64_t ldx, const int32_t* order, int64_t n128, uint16_t* Xp,
                             float* xs, float* xs4, int64_t tokens, hipStream_t stream) {
  const int64_t wpt = ceil_div(n128, 1024);
  const int64_t grid = 8 * ceil_div(tokens, 8) * wpt;
  hipLaunchKernelGGL(w4_gather_kernel, dim3((unsigned)grid), dim3(256), 0, stream, X, ldx, order, n128, Xp, xs,
                     xs4, tokens, (int)wpt);
  GPTQ_LAUNCH_CHECK();
  return GPTQ_OK;
}

// Two or four token tiles: eight waves, each pair sharing a row pair and
// splitting the tokens (two waves per SIMD, so one's VALU work runs beside
// the other's matrix and LDS work); one or three: four waves.
template <int GS>
gptq_status launch_w4_gemm_gs(int tt, dim3 grid, const W4GemmArgs& a, hipStream_t stream) {
  switch (tt) {
    case 1: hipLaunchKernelGGL((w4_gemm_kernel<GS, 1, 1>), grid, dim3(256), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((w4_gemm_kernel<GS, 2, 2>), grid, dim3(512), 0, stream, a); break;
    case 3: hipLaunchKernelGGL((w4_gemm_kernel<GS, 3, 1>), grid, dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL((w4_gemm_kernel<GS, 4, 2>), grid, dim3(512), 0, stream, a); break;
  }
  GPTQ_LAUNCH_CHECK();
  return GPTQ_OK;
}

gptq_status launch_w4_gemm(int gsteps, int tt, dim3 grid, const W4GemmArgs& a, hipStream_t stream) {
  switch (gsteps) {
    case 1: return launch_w4_gemm_gs<1>(tt, grid, a, stream);
    case 2: return launch_w4_gemm_gs<2>(tt, grid, a, stream);
    case 4: return launch_w4_gemm_gs<4>(tt, grid, a, stream);
    case 0: return launch_w4_gemm_gs<0>(tt, grid, a, stream);
    default:
      set_error("group width not built (32, 64, 128 or one group per row)");
      return GPTQ_ERR_UNSUPPORTED;
  }
}

gptq_status run_w4a16_matmul(const uint16_t* X, int64_t tokens, int64_t ldx, const void* packed,
                             const W4Layout& L, float* Y, int64_t ldy, void* ws,
                             const W4GemmPlan& p, hipStream_t stream) {
  const char* base = static_cast<const char*>(packed);
  char* w = static_cast<char*>(ws);
  uint16_t* Xp = reinterpret_cast<uint16_t*>(w + p.xp_off);
  float* xs = reinterpret_cast<float*>(w + p.xs_off);
  float* xs4 = xs + p.mp * (L.n128 / 32);
  float* part = reinterpret_cast<float*>(w + p.part_off);
  W4GemmArgs a;
  a.Xp = Xp;
  a.xs = xs;
  a.xs4 = xs4;
  a.params = reinterpret_cast<const float2*>(base + L.param_off);
  a.codes = reinterpret_cast<const u32x4_t*>(base + L.code_off);
  a.part = part;
  a.mt = L.mt;
  a.nrb = ceil_div(L.mt, kW4TilesPerWg);
  a.splits = p.splits;
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
    GPTQ_TRY(launch_w4_gather(X, ldx, order, L.n128, Xp, xs, xs4, tokens, stream));
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
    GPTQ_TRY(launch_w4_gather(X + t0 * ldx, ldx, order, L.n128, Xp, xs, xs4, tk, stream));
    a.tokens = tk;
    const dim3 grid((unsigned)(a.nrb * p.splits));
    const int tt = (int)ceil_div(tk, kW4TokTile);
    GPTQ_TRY(launch_w4_gemm(gsteps, tt, grid, a, stream));
    hipLaunchKernelGGL(w4_reduce_kernel, dim3((unsigned)ceil_div(L.m, 256), (unsigned)ceil_div(tk, 4)),
                       dim3(256), 0, stream, (const float*)part, p.splits, L.mt, tt, tk, L.m, Y + t0 * ldy,
                       ldy);
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
