// Shared by the column quantizer translation units: the argument block, the
// grid of one group, and the code of one weight on it.
#pragma once

#include "gptq_internal.hpp"

namespace gptq {

constexpr int QB = kQBlock;
// Columns per superblock of the two-level lazy update: inside a superblock a
// block's errors update only the superblock's later columns; the columns after
// it are updated once, from all of its errors (K = 512).
constexpr int kQSuper = 4 * QB;

struct QArgs {
  float* Wp;          // [m][ldw] working weights, processing order
  int64_t ldw, m, n;
  const float* U;     // [n][n]
  int64_t ldu;
  int bits, sym;
  float* scales;      // [m][G]
  int32_t* zeros;     // [m][G]
  int64_t G;
  // the superblock's errors as x6 planes (k-step-major, see X6Planes): this
  // block's first k-step of plane 0 at eplane, planes epstride apart, k-steps
  // esst apart
  uint16_t* eplane;
  int64_t epstride, esst;
  uint8_t* codes;     // [m][ldw], processing order
  double* loss_rows;  // [m]
};

// Grid of one group (page "模型量化实战：从 INT8 PTQ 到 GPTQ…" §2.1/§3.1):
// asym -> range [min(w,0), max(w,0)] in 2^b - 1 steps, zero point = rounded
// position of 0; sym -> scale max|w| / (2^(b-1) - 1), zero = storage offset
// 2^(b-1).  Scales are floored at 1e-8.
// The zero point is the round-half-to-even of -lo / step on the exact step
// (hi - lo)/(2^b - 1), not on the rounded scale: in fp64, -lo·(2^b - 1) and
// hi - lo of fp32 operands are exact (hi >= 0 >= lo), so the quotient is
// correctly rounded and a range with max = -min lands exactly on the
// half-integer (2^b - 1)/2 and goes to the even neighbour.  (When hi - lo
// needs more than 53 bits, -lo is below 2^-29 of the range and the zero
// point is 0 either way.)  It is taken once per group.
__device__ __forceinline__ void grid_params(float lo, float hi, float amax, int bits, int sym,
                                            float& s, float& z) {
  if (sym) {
    s = fmaxf(amax / (float)((1 << (bits - 1)) - 1), 1e-8f);
    z = (float)(1 << (bits - 1));
  } else {
    lo = fminf(lo, 0.f);
    hi = fmaxf(hi, 0.f);
    const int qmax = (1 << bits) - 1;
    s = fmaxf((hi - lo) / (float)qmax, 1e-8f);
    const double span = (double)hi - (double)lo;
    const double pos = span >= (double)qmax * 1e-8 ? -(double)lo * (double)qmax / span : -(double)lo / 1e-8;
    z = (float)rint(pos);
  }
}

__device__ __forceinline__ float quant_code(float w, float s, float z, int bits, int sym) {
  if (sym) {
    const float qs = (float)((1 << (bits - 1)) - 1);
    return fminf(fmaxf(rintf(w / s), -qs), qs) + z;
  }
  return fminf(fmaxf(rintf(w / s + z), 0.f), (float)((1 << bits) - 1));
}


// One block of bw <= 128 columns starting at processed column i1, all rows;
// GW = group width or 0 for one group per row.  ublk points at U[i1][i1] with
// row stride ldu; rows and columns < bw of the diagonal block are read, and,
// with ncols > 0 (then bw = 128), the block's errors are pushed into the
// ncols working-weight columns after it through U rows i1 .. i1+127, columns
// i1+128 .. i1+128+ncols-1.
// Instantiated in block_quant_g*.hip.
template <int GW>
void launch_block_quant(const QArgs& a, const float* ublk, int64_t ldu, int64_t i1, int bw,
                        int ncols, hipStream_t stream);
template <> void launch_block_quant<0>(const QArgs&, const float*, int64_t, int64_t, int, int, hipStream_t);
template <> void launch_block_quant<8>(const QArgs&, const float*, int64_t, int64_t, int, int, hipStream_t);
template <> void launch_block_quant<16>(const QArgs&, const float*, int64_t, int64_t, int, int, hipStream_t);
template <> void launch_block_quant<32>(const QArgs&, const float*, int64_t, int64_t, int, int, hipStream_t);
template <> void launch_block_quant<64>(const QArgs&, const float*, int64_t, int64_t, int, int, hipStream_t);
template <> void launch_block_quant<128>(const QArgs&, const float*, int64_t, int64_t, int, int, hipStream_t);

}  // namespace gptq
