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
// error block and ½Σe² are written out; the columns after the block are
// updated by the trailing GEMM.
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
  f32x4_t u0, u1;  // U[c][8j .. 8j+7] of the current column c (prefetched one step ahead)
  float ud;        // U[c][c]
  float s, z, lacc;
  int bits, sym, bw, j;
  bool act;
  float* srow;
  int32_t* zrow;
  int64_t g_base;
  const float* us;   // LDS U block [128][128]
};

template <int GW, int C>
__device__ __forceinline__ void bq_col(BqCtx& x) {
  if (C >= x.bw) return;   // uniform: ragged last block
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
    if (x.act && x.j == 0) {
      const int64_t g = (x.g_base + C) / GW;
      x.srow[g] = x.s;
      x.zrow[g] = (int32_t)x.z;
    }
  }
  // U of the next column, in flight while this one is quantized
  constexpr int CN = (C + 1 < QB) ? C + 1 : C;
  const f32x4_t n0 = *reinterpret_cast<const f32x4_t*>(x.us + CN * QB + 8 * x.j);
  const f32x4_t n1 = *reinterpret_cast<const f32x4_t*>(x.us + CN * QB + 8 * x.j + 4);
  const float nd = x.us[CN * QB + CN];
  const float v = row_bcast<J>(x.w[P]);
  const float code = quant_code(v, x.s, x.z, x.bits, x.sym);
  const float e = (v - (code - x.z) * x.s) / x.ud;
  if (x.j == J) {
    x.e8[P] = e;
    x.c8[P >> 2] |= ((uint32_t)code) << (8 * (P & 3));
    x.lacc += e * e;
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    x.w[p] -= e * x.u0[p];
    x.w[p + 4] -= e * x.u1[p];
  }
  x.u0 = n0;
  x.u1 = n1;
  x.ud = nd;
}

template <int GW, int... Cs>
__device__ __forceinline__ void bq_cols(std::integer_sequence<int, Cs...>, BqCtx& x) {
  (bq_col<GW, Cs>(x), ...);
}

// GW > 0: group width (a power of two dividing 128); GW == 0: one group per
// row, its grid already in scales/zeros.
template <int GW>
__global__ __launch_bounds__(256) void block_quant_kernel(QArgs q, const float* __restrict__ ublk,
                                                         int64_t ldu, int64_t i1, int bw) {
  __shared__ __attribute__((aligned(16))) float us[QB * QB];
  const int tid = threadIdx.x;
  // U block: rows and columns < bw, upper triangle only (the rest zero)
  for (int idx = tid; idx < QB * QB; idx += 256) {
    const int r = idx >> 7, c = idx & (QB - 1);
    us[idx] = (r < bw && c < bw && c >= r) ? ublk[r * ldu + c] : 0.f;
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
#pragma unroll
  for (int p = 0; p < 8; ++p) x.e8[p] = 0.f;
  x.c8[0] = x.c8[1] = 0u;
  x.bits = q.bits; x.sym = q.sym; x.bw = bw;
  x.s = 1.f; x.z = 0.f;
  if (GW == 0) {
    x.s = q.scales[rr * q.G];
    x.z = (float)q.zeros[rr * q.G];
  }
  x.lacc = 0.f;
  x.srow = q.scales + rr * q.G;
  x.zrow = q.zeros + rr * q.G;
  x.g_base = i1;
  x.us = us;
  __syncthreads();
  x.u0 = *reinterpret_cast<const f32x4_t*>(us + 8 * x.j);
  x.u1 = *reinterpret_cast<const f32x4_t*>(us + 8 * x.j + 4);
  x.ud = us[0];
  bq_cols<GW>(std::make_integer_sequence<int, QB>{}, x);

  float lacc = x.lacc;
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) lacc += __shfl_xor(lacc, d, 16);
  if (x.act) {
    // columns >= bw carry code 0 and error 0
    *reinterpret_cast<uint2*>(q.codes + r * q.ldw + i1 + 8 * x.j) = make_uint2(x.c8[0], x.c8[1]);
    float* erow = q.err + r * q.lde + 8 * x.j;
    *reinterpret_cast<f32x4_t*>(erow) = f32x4_t{x.e8[0], x.e8[1], x.e8[2], x.e8[3]};
    *reinterpret_cast<f32x4_t*>(erow + 4) = f32x4_t{x.e8[4], x.e8[5], x.e8[6], x.e8[7]};
    if (x.j == 0) q.loss_rows[r] += 0.5 * (double)lacc;
  }
}

}  // namespace

template <>
void launch_block_quant<GPTQ_BQ_GW>(const QArgs& a, const float* ublk, int64_t ldu, int64_t i1,
                                    int bw, hipStream_t stream) {
  hipLaunchKernelGGL(block_quant_kernel<GPTQ_BQ_GW>, dim3((unsigned)ceil_div(a.m, kBqRows)), dim3(256), 0,
                     stream, a, ublk, ldu, i1, bw);
}

}  // namespace gptq
