// Column quantizer for one block of 128 columns; included once per group
// width by block_quant_g*.hip (the unrolled column loop takes a while to
// compile, so each width is its own translation unit).
//
// GPTQ's in-block step (page "模型量化实战：从 INT8 PTQ 到 GPTQ…" §3.2,
// quantize_block; page "大模型量化：GPTQ/AWQ/GGUF 原理对比…", section on
// Hessian-based error compensation, for the column-by-column flow): per
// column c, the group grid at the group's first column (from the current,
// already compensated weights), the code, e = (w - x̂)/U[c][c], and
// w_k -= e·U[c][k] for the rest of the block.
//
// Layout: 16 lanes per output row, lane j of a row holding columns 8j..8j+7
// of the row's 128-column slab in VGPRs; a 256-thread workgroup covers 16
// rows, so an m-row layer runs m/16 workgroups (one wave per SIMD at
// m = 4096).  U's 128 x 128 diagonal block is staged in LDS with its strict
// lower triangle zeroed, so every lane updates all eight of its columns with
// no mask: columns already quantized see U[c][k] = 0 (k < c) or are never read
// again (k = c).  The weight of column c is broadcast from its owner lane by
// DPP row_newbcast, the group min/max is a 16-lane butterfly.  Codes, the
// error block and ½Σe² are written out; the workgroup then applies the
// block's errors to its own rows of the superblock's remaining columns, and
// the columns after the superblock are updated by the trailing GEMM.
#include <utility>

#include "quant_common.hpp"

#ifndef GPTQ_BQ_GW
#error "define GPTQ_BQ_GW"
#endif

namespace gptq {
namespace {

constexpr int kBqRows = 16;   // rows per workgroup: 4 waves x 4 rows

// value of lane K of this lane's 16-lane row
template <int K>
__device__ __forceinline__ float row_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + K, 0xf, 0xf, false));
}

struct BqCtx {
  float w[8];      // columns 8j .. 8j+7 of this lane's row
  float e8[8];     // errors of the owned columns (lane j owns columns 8j..8j+7)
  uint32_t c8[2];  // codes of the owned columns, one per byte
  // U[c][8j .. 8j+7] and 1/U[c][c] of column c in slot c % 3: each row is
  // read two columns ahead into its own slot (no register moves, so no wait
  // on the read until the column that uses it)
  f32x4_t ua[3], ub[3];
  float rd[3];
  float s, rs, z, lacc;   // the group's scale, its reciprocal and zero point
  // branch-free code: clamp(rint(w·(1/s) + zpre), qlo, qhi) + post, with
  // zpre = z, post = 0 (asym) or zpre = 0, post = z (sym): no branch on sym
  // and no division in the column chain
  float zpre, post, qlo, qhi;
  int bits, sym, bw, j;
  bool act;
  float* srow;
  int32_t* zrow;
  int64_t g_base;
  const float* us;   // LDS U block [128][128]
  const float* rdg;  // LDS reciprocals of U's diagonal [128]
};

// FULL: a whole 128-column block (no per-column bound check, so the column
// chain is one straight basic block)
template <int GW, bool FULL, int C>
__device__ __forceinline__ void bq_col(BqCtx& x) {
  if constexpr (!FULL) {
    if (C >= x.bw) return;   // uniform: ragged last block
  }
  constexpr int J = C >> 3, P = C & 7;
  if constexpr (GW > 0 && C % GW == 0) {
    // group = columns [C, C + GW) ∩ [0, bw), spread over lanes C/8 ..
    float lo = __builtin_huge_valf(), hi = -__builtin_huge_valf(), am = 0.f;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int col = 8 * x.j + p;
      if (col >= C && col < C + GW && col < x.bw) {
        lo = fminf(lo, x.w[p]);
        hi = fmaxf(hi, x.w[p]);
        am = fmaxf(am, fabsf(x.w[p]));
      }
    }
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      lo = fminf(lo, __shfl_xor(lo, d, 16));
      hi = fmaxf(hi, __shfl_xor(hi, d, 16));
      am = fmaxf(am, __shfl_xor(am, d, 16));
    }
    grid_params(lo, hi, am, x.bits, x.sym, x.s, x.z);
    x.rs = 1.f / x.s;
    x.zpre = x.sym ? 0.f : x.z;
    x.post = x.sym ? x.z : 0.f;
    if (x.act && x.j == 0) {
      const int64_t g = (x.g_base + C) / GW;
      x.srow[g] = x.s;
      x.zrow[g] = (int32_t)x.z;
    }
  }
  // U of the column after next, in flight while this one and the next are
  // quantized.  The scheduling barrier keeps these reads here: left to
  // itself the scheduler sinks them to their use, two columns on, and the
  // chain then waits for them.
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (C + 2 < QB) {
    constexpr int CN = C + 2, SN = CN % 3;
    x.ua[SN] = *reinterpret_cast<const f32x4_t*>(x.us + CN * QB + 8 * x.j);
    x.ub[SN] = *reinterpret_cast<const f32x4_t*>(x.us + CN * QB + 8 * x.j + 4);
    x.rd[SN] = x.rdg[CN];
  }
  constexpr int SC = C % 3;
  const float v = row_bcast<J>(x.w[P]);
  // the code from w·(1/s) (within one ulp of w/s: only a grid position that
  // close to a half-integer can round the other way) and e·(1/U[c][c])
  const float code = fminf(fmaxf(rintf(v * x.rs + x.zpre), x.qlo), x.qhi) + x.post;
  const float e = (v - (code - x.z) * x.s) * x.rd[SC];
  if (x.j == J) {
    x.e8[P] = e;
    x.c8[P >> 2] |= ((uint32_t)code) << (8 * (P & 3));
    x.lacc += e * e;
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    x.w[p] -= e * x.ua[SC][p];
    x.w[p + 4] -= e * x.ub[SC][p];
  }
}

template <int GW, bool FULL, int... Cs>
__device__ __forceinline__ void bq_cols(std::integer_sequence<int, Cs...>, BqCtx& x) {
  (bq_col<GW, FULL, Cs>(x), ...);
}

// The lazy update of the rest of the superblock from this block's errors,
// W[rows, i2:i2+ncols] -= E[rows, 0:128] · U[i1:i1+128, i2:i2+ncols], done by
// each workgroup for its own 16 rows (rows are independent, so no other
// workgroup touches them) with v_mfma_f32_16x16x4f32.  Columns go in blocks
// of 32, wave w taking blocks w, w+4, ...; in a block, lane l owns the two
// adjacent columns 2 (l % 16) and 2 (l % 16) + 1, which feed MFMA 0 and MFMA 1
// as their column l % 16, so U and W move as 8-byte loads (U row 4 kk + l/16
// per k-step).  A = E from LDS, held in registers for all blocks.  Two blocks'
// loads (U and the W values they update) are in flight at once, and the
// first block's are issued before the column loop.
constexpr int kPushK = QB / 4;    // MFMA k-steps per block
constexpr int kEsPitch = QB + 4;  // row pitch of the error block in LDS
constexpr int kPushCols = 32;     // columns per push block

struct PushBlk {
  float2 b[kPushK];   // U[4 kk + l/16][2 (l%16) + e], e = .x / .y
  float2 w[4];        // W[4 (l/16) + v][2 (l%16) + e]
};

// pair: both columns in range and 8-byte aligned rows (even ld, even column)
__device__ __forceinline__ float2 ld_pair(const float* __restrict__ p, bool ok0, bool ok1, bool vec) {
  if (vec && ok1) return *reinterpret_cast<const float2*>(p);
  return make_float2(ok0 ? p[0] : 0.f, ok1 ? p[1] : 0.f);
}

__device__ __forceinline__ void push_load(PushBlk& t, const float* __restrict__ up, int64_t ldu,
                                          const float* __restrict__ wp, int64_t ldw, int64_t rows_left,
                                          int blk, int ncols, bool vec, int lane) {
  const int col = kPushCols * blk + 2 * (lane & 15);
  const bool ok0 = col < ncols, ok1 = col + 1 < ncols;
  const int c = ok0 ? col : 0;
  const float* src = up + (int64_t)(lane >> 4) * ldu + c;
#pragma unroll
  for (int kk = 0; kk < kPushK; ++kk) t.b[kk] = ld_pair(src + (int64_t)(4 * kk) * ldu, ok0, ok1, vec);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int row = 4 * (lane >> 4) + v;
    const bool rok = row < rows_left;
    t.w[v] = ld_pair(wp + (int64_t)(rok ? row : 0) * ldw + c, ok0 && rok, ok1 && rok, vec);
  }
}

// GW > 0: group width (a power of two dividing 128); GW == 0: one group per
// row, its grid already in scales/zeros.  FULL: bw == 128.
template <int GW, bool FULL>
__global__ __launch_bounds__(256) void block_quant_kernel(QArgs q, const float* __restrict__ ublk,
                                                         int64_t ldu, int64_t i1, int bw,
                                                         const float* __restrict__ upush, int ncols) {
  __shared__ __attribute__((aligned(16))) float us[QB * QB];
  __shared__ float rdg[QB];
  __shared__ __attribute__((aligned(16))) float es[kBqRows * kEsPitch];
  const int tid = threadIdx.x;
  // the push's operands (its first block's loads go out below)
  const int64_t prow0 = (int64_t)blockIdx.x * kBqRows;
  const int64_t rows_left = q.m - prow0;
  float* wpush = q.Wp + prow0 * q.ldw + i1 + bw;   // processed column i2 = i1 + bw
  const bool pvec = ((ldu | q.ldw | (i1 + bw)) & 1) == 0 &&
                    ((reinterpret_cast<uintptr_t>(upush) | reinterpret_cast<uintptr_t>(q.Wp)) & 7) == 0;
  PushBlk pb[2];
  // U block: rows and columns < bw, upper triangle only (the rest zero), and
  // the reciprocals of its diagonal.  Every load is unconditional (indices
  // clamped into the block) and a thread's loads are in flight together
  // before its first LDS store: under a condition each load compiles to a
  // branch and a wait of its own, 64 round trips to L2 per thread.  Loads
  // complete in issue order, so the block's loads go out first, then the
  // row's weights, then the push's first operands: each wait then covers
  // only what its use needs.
  const bool uvec = FULL && (ldu & 3) == 0 && (reinterpret_cast<uintptr_t>(ublk) & 15) == 0;
  constexpr int kV = QB * QB / 4 / 256;   // 16-byte pieces per thread
  f32x4_t uv[kV];
  if (uvec) {
#pragma unroll
    for (int k = 0; k < kV; ++k) {
      const int i4 = tid + 256 * k, ur = i4 >> 5, uc = (i4 & 31) << 2;
      uv[k] = *reinterpret_cast<const f32x4_t*>(ublk + (int64_t)ur * ldu + uc);
    }
  }
  const int lane = tid & 63, wave = tid >> 6;
  BqCtx x;
  x.j = lane & 15;
  const int64_t r = (int64_t)blockIdx.x * kBqRows + wave * 4 + (lane >> 4);
  x.act = r < q.m;
  const int64_t rr = x.act ? r : 0;
  {
    const float* src = q.Wp + rr * q.ldw + i1 + 8 * x.j;
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(src);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(src + 4);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      x.w[p] = a[p];
      x.w[p + 4] = b[p];
    }
  }
  if ((tid >> 6) * kPushCols < ncols)
    push_load(pb[0], upush, ldu, wpush, q.ldw, rows_left, tid >> 6, ncols, pvec, tid & 63);
  if (uvec) {
#pragma unroll
    for (int k = 0; k < kV; ++k) {
      const int i4 = tid + 256 * k, ur = i4 >> 5, uc = (i4 & 31) << 2;
      f32x4_t o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = uc + e >= ur ? uv[k][e] : 0.f;
      *reinterpret_cast<f32x4_t*>(us + ur * QB + uc) = o;
      if (uc <= ur && ur < uc + 4) rdg[ur] = 1.f / uv[k][ur - uc];
    }
  } else {
    constexpr int kS = 16;   // loads in flight per round
    for (int k0 = 0; k0 < QB * QB / 256; k0 += kS) {
      float v[kS];
#pragma unroll
      for (int u = 0; u < kS; ++u) {
        const int idx = tid + 256 * (k0 + u), ur = idx >> 7, uc = idx & (QB - 1);
        v[u] = ublk[(int64_t)std::min(ur, bw - 1) * ldu + std::min(uc, bw - 1)];
      }
#pragma unroll
      for (int u = 0; u < kS; ++u) {
        const int idx = tid + 256 * (k0 + u), ur = idx >> 7, uc = idx & (QB - 1);
        us[idx] = (ur < bw && uc < bw && uc >= ur) ? v[u] : 0.f;
        if (ur == uc) rdg[ur] = ur < bw ? 1.f / v[u] : 1.f;
      }
    }
  }

#pragma unroll
  for (int p = 0; p < 8; ++p) x.e8[p] = 0.f;
  x.c8[0] = x.c8[1] = 0u;
  x.bits = q.bits; x.sym = q.sym; x.bw = bw;
  x.s = 1.f; x.z = 0.f;
  if (GW == 0) {
    x.s = q.scales[rr * q.G];
    x.z = (float)q.zeros[rr * q.G];
  }
  x.rs = 1.f / x.s;
  x.qlo = q.sym ? -(float)((1 << (q.bits - 1)) - 1) : 0.f;
  x.qhi = q.sym ? (float)((1 << (q.bits - 1)) - 1) : (float)((1 << q.bits) - 1);
  x.zpre = q.sym ? 0.f : x.z;
  x.post = q.sym ? x.z : 0.f;
  x.lacc = 0.f;
  x.srow = q.scales + rr * q.G;
  x.zrow = q.zeros + rr * q.G;
  x.g_base = i1;
  x.us = us;
  x.rdg = rdg;
  __syncthreads();
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    x.ua[c] = *reinterpret_cast<const f32x4_t*>(us + c * QB + 8 * x.j);
    x.ub[c] = *reinterpret_cast<const f32x4_t*>(us + c * QB + 8 * x.j + 4);
    x.rd[c] = rdg[c];
  }
  bq_cols<GW, FULL>(std::make_integer_sequence<int, QB>{}, x);

  float lacc = x.lacc;
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) lacc += __shfl_xor(lacc, d, 16);
  if (x.act) {
    // columns >= bw carry code 0 and error 0
    *reinterpret_cast<uint2*>(q.codes + r * q.ldw + i1 + 8 * x.j) = make_uint2(x.c8[0], x.c8[1]);
    // the errors straight into the superblock's x6 planes: columns 8j..8j+7
    // are 16 contiguous bytes of k-step j/2 in each plane
    uint16_t hv[8], mv[8], lv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x6_split(x.e8[e], hv[e], mv[e], lv[e]);
    uint16_t* ep = q.eplane + (x.j >> 1) * q.esst + 16 * r + 8 * (x.j & 1);
    auto pack8 = [](const uint16_t (&v)[8]) {
      return make_uint4(v[0] | ((uint32_t)v[1] << 16), v[2] | ((uint32_t)v[3] << 16), v[4] | ((uint32_t)v[5] << 16),
                        v[6] | ((uint32_t)v[7] << 16));
    };
    *reinterpret_cast<uint4*>(ep) = pack8(hv);
    *reinterpret_cast<uint4*>(ep + q.epstride) = pack8(mv);
    *reinterpret_cast<uint4*>(ep + 2 * q.epstride) = pack8(lv);
    if (x.j == 0) q.loss_rows[r] += 0.5 * (double)lacc;
  }
  if (ncols <= 0) return;   // uniform: last block of its superblock

  // ---- push this block's errors into the rest of the superblock (own rows)
  {
    float* erow = es + (wave * 4 + (lane >> 4)) * kEsPitch + 8 * x.j;
    *reinterpret_cast<f32x4_t*>(erow) = f32x4_t{x.e8[0], x.e8[1], x.e8[2], x.e8[3]};
    *reinterpret_cast<f32x4_t*>(erow + 4) = f32x4_t{x.e8[4], x.e8[5], x.e8[6], x.e8[7]};
  }
  __syncthreads();
  // A operand: lane l supplies E[l % 16][4 kk + l / 16]
  float ea[kPushK];
#pragma unroll
  for (int kk = 0; kk < kPushK; ++kk) ea[kk] = es[(lane & 15) * kEsPitch + 4 * kk + (lane >> 4)];
  const int nblk = (ncols + kPushCols - 1) / kPushCols;
  auto apply = [&](const PushBlk& t, int blk) {
    f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < kPushK; ++kk) {
      acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(ea[kk], t.b[kk].x, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(ea[kk], t.b[kk].y, acc1, 0, 0, 0);
    }
    // D[4 (l / 16) + v][l % 16] of MFMA e: row 4 (l / 16) + v, column 2 (l % 16) + e
    const int col = kPushCols * blk + 2 * (lane & 15);
    const bool ok0 = col < ncols, ok1 = col + 1 < ncols;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = 4 * (lane >> 4) + v;
      if (row >= rows_left || !ok0) continue;
      float* dst = wpush + (int64_t)row * q.ldw + col;
      const float2 nv = make_float2(t.w[v].x - acc0[v], t.w[v].y - acc1[v]);
      if (pvec && ok1) {
        *reinterpret_cast<float2*>(dst) = nv;
      } else {
        dst[0] = nv.x;
        if (ok1) dst[1] = nv.y;
      }
    }
  };
  // blocks wave, wave + 4, ... alternate between pb[0] and pb[1]
#pragma unroll 1
  for (int blk = wave; blk < nblk; blk += 8) {
    if (blk + 4 < nblk) push_load(pb[1], upush, ldu, wpush, q.ldw, rows_left, blk + 4, ncols, pvec, lane);
    apply(pb[0], blk);
    if (blk + 4 >= nblk) break;
    if (blk + 8 < nblk) push_load(pb[0], upush, ldu, wpush, q.ldw, rows_left, blk + 8, ncols, pvec, lane);
    apply(pb[1], blk + 4);
  }
}

}  // namespace

template <>
void launch_block_quant<GPTQ_BQ_GW>(const QArgs& a, const float* ublk, int64_t ldu, int64_t i1,
                                    int bw, int ncols, hipStream_t stream) {
  if (bw == QB)
    hipLaunchKernelGGL((block_quant_kernel<GPTQ_BQ_GW, true>), dim3((unsigned)ceil_div(a.m, kBqRows)), dim3(256),
                       0, stream, a, ublk, ldu, i1, bw, ublk + bw, ncols);
  else
    hipLaunchKernelGGL((block_quant_kernel<GPTQ_BQ_GW, false>), dim3((unsigned)ceil_div(a.m, kBqRows)), dim3(256),
                       0, stream, a, ublk, ldu, i1, bw, ublk + bw, ncols);
}

}  // namespace gptq
