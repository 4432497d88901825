// Stage 1: H += alpha * XᵀX and key += alpha * Σ_t x_t² (fp64) over a token tile.
//
// The Hessian of the layer objective is the (scaled) Gram matrix of the
// calibration activations (page "模型量化实战：从 INT8 PTQ 到 GPTQ…" §3.2,
// accumulate_hessian: H grows by 2·XᵀX per batch).  It is a symmetric rank-T
// update, so only lower-triangle tiles are computed and each result is
// mirrored to the upper triangle.
//
// bf16 path: v_mfma_f32_32x32x16_bf16 on 256 x 256 tiles, 8 waves (two per
// SIMD) of 64 x 128 each, so one wave's LDS waits hide behind the other's
// MFMAs.  X is token-major, so the reduction axis (tokens) is the strided one:
// each 32-token stage of the tile's two 256-channel panels is copied into LDS
// as is (token-major rows, octet slot swizzled) and the MFMA operands -- 8
// consecutive tokens of one channel per lane -- come out through gfx950's
// transposing ds_read_b64_tr_b16.
//
// Aligned X (the usual case) is streamed with buffer loads that write LDS
// directly, into a ring of kRing stage slots: kRing - 1 stages are in flight
// while one is multiplied, enough bytes to cover HBM latency at MFMA rate
// without holding any of them in registers.  The ring is driven by explicit
// vmcnt waits and a bare s_barrier (a __syncthreads would drain every load in
// flight).  Rows past the token range and channels past n lie outside the
// buffer descriptor and land in LDS as zeros.
//
// Long token ranges are cut into `splits` slices (split-K) so the grid fills
// 256 CUs and every fp32 register chain stays <= 32768 tokens long.  Each
// workgroup writes its fp32 tile to a partial buffer and a second kernel sums
// the slices in slice order (deterministic), adds the result into H's lower
// triangle and writes the mirror, coalesced through an LDS transpose.  No
// cross-workgroup synchronisation is needed: on gfx950 that would take an L2
// write-back and invalidate per workgroup.
#include <algorithm>

#include "gptq_internal.hpp"

namespace gptq {
namespace {

struct SyrkArgs {
  const uint16_t* X;
  int64_t ldx, T;
  int64_t n;
  int64_t panels, tiles, splits, slice_tokens;
  float* partials;    // [splits][tiles][256][256] fp32, row-major tiles
  double* keyparts;   // [splits][n]
};

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kRowBytes = 512;                        // one token of a 256-channel panel
constexpr int kPanelBytes = kSyrkStage * kRowBytes;   // 16 KB: one panel, one stage
constexpr int kSlotBytes = 2 * kPanelBytes;           // 32 KB: both panels
constexpr int kRing = 4;                              // ring slots (128 KB)
constexpr int kTilePartial = kSyrkTile * kSyrkTile;   // floats per partial tile

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

// Workgroup -> (tile, slice, tile coordinates).  Jobs run in rounds of 256
// workgroups (one per CU) that stream the same token slice: chunks of 256
// tiles, and within a chunk one slice after the other.  Dispatch is
// round-robin over the 8 XCDs, so inside a round XCD x gets the 32
// consecutive tiles 32x .. 32x + 31 of the chunk (in the grouped order about a
// 4 x 8 block, 12 panels), which share panel reads in that XCD's L2; the
// other XCDs read other panels of the same tokens, which the shared memory-side
// cache can serve.  Returns false for padding workgroups.
struct TileJob {
  int64_t tile, s, ti, tj, t_begin, t_end;
};
__device__ __forceinline__ bool decode_job(const SyrkArgs& a, TileJob& j) {
  const int64_t L = blockIdx.x;
  if (L >= a.tiles * a.splits) return false;
  const int64_t per_chunk = 256 * a.splits;
  const int64_t c = L / per_chunk, cb = c * 256;
  const int64_t csz = (a.tiles - cb < 256) ? a.tiles - cb : 256;
  const int64_t rem = L - c * per_chunk;
  j.s = rem / csz;
  const int64_t q = rem % csz;
  // with csz % 8 == 0 the round starts on an XCD boundary: position q runs on
  // XCD q % 8 and takes tile (q % 8)·csz/8 + q/8 of the chunk
  j.tile = cb + ((csz % 8 == 0) ? (q % 8) * (csz / 8) + q / 8 : q);
  tile_decode_grouped(j.tile, a.panels, j.ti, j.tj);
  j.t_begin = j.s * a.slice_tokens;
  j.t_end = (j.t_begin + a.slice_tokens < a.T) ? j.t_begin + a.slice_tokens : a.T;
  if (j.t_end < j.t_begin) j.t_end = j.t_begin;
  return true;
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

// The per-wave tile work shared by both bf16 kernels.
struct WaveTile {
  f32x16_t acc[2][4];
  double ksum;   // diagonal tiles: Σx² of channel tid % 256 over half of each stage
};

__device__ __forceinline__ void wave_tile_init(WaveTile& w) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) w.acc[i][j][v] = 0.f;
  w.ksum = 0.0;
}

// k-steps [KB, KE) of a 32-token stage (16 tokens each): 2 x 4 MFMAs per wave.
template <int KB, int KE>
__device__ __forceinline__ void stage_kk(WaveTile& w, const uint8_t* pI, const uint8_t* pJ, bool active,
                                         int wr, int wc, int lane) {
  if (active) {
#pragma unroll
    for (int kk = KB; kk < KE; ++kk) {
      bf16x8_t af[2], bfm[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = tr_frag(pI, 16 * kk, wr * 64 + i * 32, lane);
#pragma unroll
      for (int j = 0; j < 4; ++j) bfm[j] = tr_frag(pJ, 16 * kk, wc * 128 + j * 32, lane);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          w.acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfm[j], w.acc[i][j], 0, 0, 0);
    }
  }
}

// Diagonal tiles: the stage's squares into the fp64 key (half of the stage's
// tokens per thread, channel tid % 256).
__device__ __forceinline__ void stage_key(WaveTile& w, const uint8_t* pI, bool diag, int tid) {
  if (diag) {
    const int c = tid & 255, t0 = (tid >> 8) * (kSyrkStage / 2);
#pragma unroll
    for (int t = 0; t < kSyrkStage / 2; ++t) {
      const uint16_t hv = *reinterpret_cast<const uint16_t*>(pI + lds_off(t0 + t, c >> 3) + ((c & 7) << 1));
      const float x = __uint_as_float((uint32_t)hv << 16);
      w.ksum += (double)(x * x);   // a bf16 square is exact in fp32
    }
  }
}

// One whole 32-token stage (the register-staged kernel).
__device__ __forceinline__ void stage_mma(WaveTile& w, const uint8_t* pI, const uint8_t* pJ, bool active,
                                          bool diag, int wr, int wc, int lane, int tid) {
  stage_kk<0, kSyrkStage / 16>(w, pI, pJ, active, wr, wc, lane);
  stage_key(w, pI, diag, tid);
}

// Partial tile (row-major 256 x 256 fp32) and key part of one slice.  `kred`
// is 256 doubles of LDS that no wave reads or writes any more.
__device__ __forceinline__ void store_partial(const SyrkArgs& a, const TileJob& jb, WaveTile& w,
                                              bool active, bool diag, int wr, int wc, int lane,
                                              int tid, double* kred) {
  if (diag) {   // combine the two token halves of each channel
    if (tid >= 256) kred[tid - 256] = w.ksum;
    __syncthreads();
    if (tid < 256) {
      const int64_t c = jb.ti * kSyrkTile + tid;
      if (c < a.n) a.keyparts[jb.s * a.n + c] = w.ksum + kred[tid];
    }
  }
  if (!active) return;
  float* P = a.partials + (jb.s * a.tiles + jb.tile) * (int64_t)kTilePartial;
  const int r0 = wr * 64 + 4 * (lane >> 5), c0 = wc * 128 + (lane & 31);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        P[(r0 + i * 32 + 8 * (v >> 2) + (v & 3)) * kSyrkTile + c0 + j * 32] = w.acc[i][j][v];
}

__device__ __forceinline__ constexpr int vmcnt_only(int n) {   // s_waitcnt vmcnt(n), other counters free
  return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

// ---------------------------------------------------------------------------
// Aligned X: direct-to-LDS ring.  Needs ldx % 8 == 0, n % 8 == 0 and a
// 16-byte aligned X (every 16-byte chunk is 8 whole channels of one token).
// ---------------------------------------------------------------------------
// The streaming loop over one slice.  The four slots come in as distinct
// __restrict__ pointers, so every LDS access below carries no-alias scopes
// that tell the compiler a read of one slot cannot see a copy into another:
// it then waits only for the copies the explicit vmcnt below names.
__device__ __forceinline__ void ring_stream(const SyrkArgs& a, const TileJob& jb, WaveTile& w,
                                            bool active, bool diag, uint8_t* __restrict__ s0,
                                            uint8_t* __restrict__ s1, uint8_t* __restrict__ s2,
                                            uint8_t* __restrict__ s3) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int64_t n = a.n;
  const int64_t nst = (jb.t_end - jb.t_begin + kSyrkStage - 1) / kSyrkStage;

  // Direct-to-LDS copy: instruction (panel p, half h) of wave w writes 1 KB at
  // slot + p·16K + h·8K + w·1K, lane l at +16·l: token row 16h + 2w + l/32,
  // slot position l % 32, which holds channel octet o = (l%32) ^ 4·(row%4).
  const int row0 = 2 * wave + (lane >> 5);
  const int oct = (lane & 31) ^ ((row0 & 3) << 2);   // (row0 + 16) % 4 == row0 % 4
  const int32_t rowb = (int32_t)(a.ldx * 2);
  constexpr int32_t kOut = 0x7ffffff0;   // beyond any descriptor size: reads as zero
  const int64_t cI = jb.ti * kSyrkTile + 8 * oct, cJ = jb.tj * kSyrkTile + 8 * oct;
  const int32_t vI0 = cI < n ? row0 * rowb + (int32_t)(cI * 2) : kOut;
  const int32_t vJ0 = cJ < n ? row0 * rowb + (int32_t)(cJ * 2) : kOut;
  const int32_t vI1 = cI < n ? vI0 + 16 * rowb : kOut;
  const int32_t vJ1 = cJ < n ? vJ0 + 16 * rowb : kOut;

  // Stage st (possibly past the end: then the descriptor is empty and the slot
  // fills with zeros nobody reads) -> `slot`.  Always 4 loads, so the vmcnt
  // bookkeeping below is the same on every step.
  auto issue = [&](int64_t st, uint8_t* slot) {
    const int64_t t0 = jb.t_begin + st * kSyrkStage;
    const int64_t bytes = (jb.t_end - t0) * (int64_t)rowb;
    const int32_t nrec = bytes <= 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : (int32_t)bytes);
    const uint16_t* base = a.X + (bytes <= 0 ? 0 : t0 * a.ldx);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, nrec, 0x00020000);
    uint8_t* d = slot + wave * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(d), 16, vI0, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(d + 8192), 16, vI1, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(d + kPanelBytes), 16, vJ0, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(d + kPanelBytes + 8192), 16, vJ1, 0, 0, 0);
  };
  // One step: this wave's loads of stage st are the oldest 4 of the 12 in
  // flight; after the barrier every wave's are in LDS and every wave has
  // finished reading the slot of stage st - 1, which stage st + 3 now refills.
  // The refill is issued after the stage's first k-step: issued right after the
  // barrier, all eight waves would stall on a full vector-memory queue at once
  // and leave the matrix cores idle (7% slower, measured).
  auto step = [&](int64_t st, const uint8_t* cur, uint8_t* refill) {
    __builtin_amdgcn_s_waitcnt(vmcnt_only(4 * (kRing - 2)));
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    stage_kk<0, 1>(w, cur, cur + kPanelBytes, active, wr, wc, lane);
    issue(st + kRing - 1, refill);
    stage_kk<1, kSyrkStage / 16>(w, cur, cur + kPanelBytes, active, wr, wc, lane);
    stage_key(w, cur, diag, tid);
  };
  issue(0, s0);
  issue(1, s1);
  issue(2, s2);
  // the stage count is rounded up to whole turns of the ring: stages past the
  // slice read zero-filled slots and add nothing
  for (int64_t st = 0; st < nst; st += 4) {
    step(st, s0, s3);
    step(st + 1, s1, s0);
    step(st + 2, s2, s1);
    step(st + 3, s3, s2);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));   // no copy may land after the workgroup ends
}

__global__ __launch_bounds__(512, 1) void syrk_bf16_ring_kernel(SyrkArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t slot0[kSlotBytes], slot1[kSlotBytes],
      slot2[kSlotBytes], slot3[kSlotBytes];
  __shared__ double kred[256];
  static_assert(kRing == 4, "the stream loop is unrolled over four slot arrays");

  TileJob jb;
  if (!decode_job(a, jb)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;   // wave tile: rows wr*64 (+64), cols wc*128 (+128)
  const bool diag = jb.ti == jb.tj;
  const bool active = !(diag && wc == 1 && wr < 2);   // idle waves sit strictly above the diagonal
  WaveTile w;
  wave_tile_init(w);
  ring_stream(a, jb, w, active, diag, slot0, slot1, slot2, slot3);
  __syncthreads();
  store_partial(a, jb, w, active, diag, wr, wc, lane, tid, kred);
}

// ---------------------------------------------------------------------------
// Any X (unaligned rows or n % 8 != 0): element loads into registers, zero
// outside [t_begin, t_end) x [0, n), double-buffered LDS stages.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(512, 1) void syrk_bf16_any_kernel(SyrkArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][kSlotBytes];
  __shared__ double kred[256];

  TileJob jb;
  if (!decode_job(a, jb)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const bool diag = jb.ti == jb.tj;
  const bool active = !(diag && wc == 1 && wr < 2);
  const int64_t n = a.n;
  const int64_t nst = (jb.t_end - jb.t_begin + kSyrkStage - 1) / kSyrkStage;

  // thread loads octet o of tokens tr + 16u (u = 0, 1) of both panels
  const int o = tid & 31, tr = tid >> 5;
  const int64_t cI = jb.ti * kSyrkTile + 8 * o, cJ = jb.tj * kSyrkTile + 8 * o;
  uint4 vI[2], vJ[2];
  auto load = [&](int64_t t0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      vI[u] = load16(a.X, a.ldx, t0 + tr + 16 * u, jb.t_end, cI, n);
      vJ[u] = load16(a.X, a.ldx, t0 + tr + 16 * u, jb.t_end, cJ, n);
    }
  };
  auto put = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int off = lds_off(tr + 16 * u, o);
      *reinterpret_cast<uint4*>(&lds[buf][off]) = vI[u];
      *reinterpret_cast<uint4*>(&lds[buf][kPanelBytes + off]) = vJ[u];
    }
  };

  WaveTile w;
  wave_tile_init(w);
  if (nst > 0) {
    load(jb.t_begin);
    put(0);
    __syncthreads();
    for (int64_t st = 0; st < nst; ++st) {
      const bool more = st + 1 < nst;
      if (more) load(jb.t_begin + (st + 1) * kSyrkStage);
      stage_mma(w, lds[st & 1], lds[st & 1] + kPanelBytes, active, diag, wr, wc, lane, tid);
      if (more) put((int)((st + 1) & 1));
      __syncthreads();
    }
  }
  store_partial(a, jb, w, active, diag, wr, wc, lane, tid, kred);
}

// ---------------------------------------------------------------------------
// Slice reduction: one workgroup per 64 x 64 block of a lower tile.  Sums the
// slices in order, H[gi][gj] += alpha·sum for gi >= gj, then writes the mirror
// H[gj][gi] (gi > gj) from an LDS transpose so both writes are row segments.
// Diagonal blocks of diagonal tiles also reduce the key of their 64 channels.
// ---------------------------------------------------------------------------
struct ReduceArgs {
  const float* partials;
  const double* keyparts;
  int64_t n, panels, tiles, splits;
  float* H;
  double* key;
  float alpha;
};

__global__ __launch_bounds__(256) void syrk_reduce_kernel(ReduceArgs r) {
  __shared__ float tb[64][65];
  const int64_t tile = blockIdx.x >> 4;
  const int bi = (blockIdx.x >> 2) & 3, bj = blockIdx.x & 3;
  int64_t ti, tj;
  tile_decode_grouped(tile, r.panels, ti, tj);
  const bool diag = ti == tj;
  if (diag && bj > bi) return;
  const int tid = threadIdx.x, c = tid & 63, rq = tid >> 6;
  const int64_t n = r.n;
  const int64_t row0 = ti * kSyrkTile + bi * 64, col0 = tj * kSyrkTile + bj * 64;
  const int64_t gj = col0 + c;

  float sum[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) sum[k] = 0.f;
  const float* P = r.partials + tile * (int64_t)kTilePartial + (bi * 64) * kSyrkTile + bj * 64 + c;
  for (int64_t s = 0; s < r.splits; ++s) {
    const float* Ps = P + s * r.tiles * (int64_t)kTilePartial;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float x = Ps[(rq + 4 * k) * kSyrkTile];
      sum[k] = (s == 0) ? x : sum[k] + x;
    }
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int lr = rq + 4 * k;
    const int64_t gi = row0 + lr;
    float val = 0.f;
    if (gi < n && gj < n && (!diag || gi >= gj)) {
      val = r.H[gi * n + gj] + r.alpha * sum[k];
      r.H[gi * n + gj] = val;
    }
    tb[lr][c] = val;
  }
  __syncthreads();
  // mirror block: row gj' = col0 + lr, column gi' = row0 + c holds H[gi'][gj']
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int lr = rq + 4 * k;
    const int64_t mrow = col0 + lr, mcol = row0 + c;   // (gj, gi) of the source element
    if (mrow < n && mcol < n && mcol > mrow) r.H[mrow * n + mcol] = tb[c][lr];
  }
  if (diag && bi == bj && r.key && tid < 64) {
    const int64_t ch = row0 + tid;
    if (ch < n) {
      double s = 0.0;
      for (int64_t q = 0; q < r.splits; ++q) s += r.keyparts[q * n + ch];
      r.key[ch] += (double)r.alpha * s;
    }
  }
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
  // traffic of the slice reduction.
  const double per_tok = (double)kSyrkTile * kSyrkTile * 2.0 / 8.4e12;   // one CU near peak
  double best = 1e300;
  int64_t best_s = smin;
  const int64_t cands[] = {1, 2, 4, 8, 16, 24, 32, 40, 48, 56, 64};
  for (int64_t c : cands) {
    if (c < smin) continue;
    const int64_t slice = round_up(ceil_div(std::max<int64_t>(tokens, 1), c), kSyrkStage);
    const double rounds = (double)ceil_div(p.tiles * c, 256);
    double t = rounds * (double)slice * per_tok;
    t += 2.0 * (double)c * (double)p.tiles * 256.0 * 1024.0 / 4e12;
    if (t < best * 0.999) { best = t; best_s = c; }
  }
  if (best_s < smin) best_s = smin;
  p.splits = best_s;
  p.slice_tokens = round_up(ceil_div(std::max<int64_t>(tokens, 1), p.splits), kSyrkStage);
  p.partial_bytes = align256((size_t)p.splits * p.tiles * kTilePartial * sizeof(float));
  p.keypart_bytes = align256((size_t)p.splits * n * sizeof(double));
  p.total_bytes = p.partial_bytes + p.keypart_bytes;
  return p;
}

gptq_status launch_hessian_bf16(float* H, double* key, int64_t n, const uint16_t* X, int64_t tokens,
                                int64_t ldx, float alpha, void* ws, const SyrkPlan& plan,
                                hipStream_t stream) {
  SyrkArgs a;
  a.X = X; a.ldx = ldx; a.T = tokens; a.n = n;
  a.panels = plan.panels; a.tiles = plan.tiles; a.splits = plan.splits;
  a.slice_tokens = plan.slice_tokens;
  char* w = static_cast<char*>(ws);
  a.partials = reinterpret_cast<float*>(w);
  a.keyparts = reinterpret_cast<double*>(w + plan.partial_bytes);
  const int64_t grid = plan.tiles * plan.splits;
  // the ring path copies whole 16-byte channel octets with 32-bit offsets
  const bool ring = (ldx % 8 == 0) && (n % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0) &&
                    ldx <= (int64_t(1) << 24);
  if (ring) hipLaunchKernelGGL(syrk_bf16_ring_kernel, dim3((unsigned)grid), dim3(512), 0, stream, a);
  else hipLaunchKernelGGL(syrk_bf16_any_kernel, dim3((unsigned)grid), dim3(512), 0, stream, a);
  GPTQ_LAUNCH_CHECK();
  ReduceArgs r;
  r.partials = a.partials; r.keyparts = a.keyparts;
  r.n = n; r.panels = plan.panels; r.tiles = plan.tiles; r.splits = plan.splits;
  r.H = H; r.key = key; r.alpha = alpha;
  hipLaunchKernelGGL(syrk_reduce_kernel, dim3((unsigned)(plan.tiles * 16)), dim3(256), 0, stream, r);
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
