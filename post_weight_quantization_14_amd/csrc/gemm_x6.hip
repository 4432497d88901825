// fp32-accurate GEMM on bf16 MFMA: C = alpha·A·Bᵀ + beta·C from operands
// split exactly into three bf16 planes.
//
// An fp32 value x is hi + mid + lo exactly, each a bf16 (hi = x truncated to
// bf16, mid = (x - hi) truncated, lo = the rest, which fits: 24 significand
// bits in three 8-bit pieces).  The product a·b keeps the six cross terms
// whose weight is at least 2⁻¹⁶ of hi·hi (lo·lo, lo·mid, mid·lo dropped, below
// fp32's own rounding), each an exact bf16 × bf16 product accumulated in fp32
// by v_mfma_f32_32x32x16_bf16.  At the bf16 MFMA rate that is 1.4x faster
// than v_mfma_f32_32x32x2f32 on the same GEMM, with a result within fp32
// rounding of it (relative Frobenius difference ~5e-8).
//
// Planes are three bf16 arrays stored k-step-major ([kp/16][rows][16], kp a
// multiple of 16, zero padded), so that one k-step of a tile's rows is one
// contiguous block and every direct-to-LDS copy reads 1 KB in one piece (with
// rows of kp contiguous positions a copy gathered 32 bytes from each of 32
// rows kp·2 bytes apart, and the copies took 70% of the GEMM's time); the split
// kernels write them from fp32 rows (A, or B stored with k contiguous) or from
// fp32 columns (B stored k-major, transposed on the way).
//
// GEMM: tiles of 128 x 128 per workgroup of 4 waves (64 x 64 each); per
// 16-position k-step the six operand planes (2 x 3 x 4 KB) stream into a
// three-slot LDS ring by direct-to-LDS buffer loads, rows past the operand's
// end read as zero; the lower variant computes only element row >= column of
// the output (a triangle of tiles over a rectangle of full tiles).
#include "gptq_internal.hpp"

namespace gptq {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
constexpr int X6T = 128;             // tile edge
constexpr int X6KS = 16;             // k per stage (one MFMA k-step)
static_assert(X6KS == kX6Step, "a stage is one contiguous k-step piece of the planes");
constexpr int X6ROWB = X6KS * 2;     // 32 bytes per row per plane
constexpr int X6PLANEB = X6T * X6ROWB;
constexpr int X6OPB = 3 * X6PLANEB;  // 12 KB per operand
constexpr int X6SLOTB = 2 * X6OPB;   // 24 KB per stage
constexpr int X6RING = 3;
constexpr int kX6Band = 16;         // tile rows per band of the tile order
// 73728 B static + this > 80 KB (one workgroup per CU), and <= 160 KB - 77312 B
// (the Cholesky leaf's LDS, the largest workgroup meant to run beside it)
constexpr size_t kX6PolitePad = 12288;
static_assert(3 * X6SLOTB + kX6PolitePad > 81920 && 3 * X6SLOTB + kX6PolitePad + 77312 <= 163840,
              "polite footprint: one per CU, a 75.5 KB workgroup beside it");

__device__ __forceinline__ constexpr int x6_vmcnt(int n) {
  return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}


// planes of X[r][k] (k < K), zero for K <= k < kp, and with `lower` zero for
// k > r as well (X's strictly upper part is not read).  Element i of the sweep
// is k-step i / (16 rows), row (i / 16) % rows, position i % 16: the writes
// are contiguous, the reads 64-byte row pieces.
__global__ __launch_bounds__(256) void x6_split_rows_kernel(const float* __restrict__ X, int64_t ldx,
                                                            int64_t rows, int64_t K, int64_t kp,
                                                            uint16_t* __restrict__ out, int64_t pstride,
                                                            int64_t sst, int lower) {
  const int64_t total = rows * kp;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t ks = i / (rows * kX6Step), r = (i / kX6Step) % rows, kk = i % kX6Step;
    const int64_t k = ks * kX6Step + kk;
    const float x = (k < K && (!lower || k <= r)) ? X[r * ldx + k] : 0.f;
    uint16_t h, m, l;
    x6_split(x, h, m, l);
    const int64_t o = ks * sst + r * kX6Step + kk;
    out[o] = h;
    out[pstride + o] = m;
    out[2 * pstride + o] = l;
  }
}

// planes of row c = X[k][c] over k (k < K, c < cols), zero for K <= k < kp,
// and with `lower` zero for k < c as well (X's strictly upper part is not
// used): 64 x 64 tiles through LDS, read along c; written as 4 k-steps of 64
// rows, 256 contiguous elements per pass of the workgroup
__global__ __launch_bounds__(256) void x6_split_cols_kernel(const float* __restrict__ X, int64_t ldx,
                                                            int64_t K, int64_t cols, int64_t kp,
                                                            uint16_t* __restrict__ out, int64_t pstride,
                                                            int64_t sst, int lower) {
  __shared__ float t[64][65];
  const int64_t c0 = (int64_t)blockIdx.x * 64, k0 = (int64_t)blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  // all sixteen loads in flight: unconditional at clamped indices (a
  // conditional load compiles to a branch and a wait of its own)
  float v[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int64_t k = k0 + ty + 4 * u, c = c0 + tx;
    v[u] = X[std::min<int64_t>(k, K - 1) * ldx + std::min<int64_t>(c, cols - 1)];
  }
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int r = ty + 4 * u;
    t[r][tx] = (k0 + r < K && c0 + tx < cols && (!lower || k0 + r >= c0 + tx)) ? v[u] : 0.f;
  }
  __syncthreads();
#pragma unroll 1
  for (int j = 0; j < 16; ++j) {
    const int e = 256 * j + (int)threadIdx.x;
    const int ks = e >> 10, cl = (e >> 4) & 63, kk = e & 15;
    const int64_t c = c0 + cl, k = k0 + 16 * ks + kk;
    if (c < cols && k < kp) {
      uint16_t h, m, l;
      x6_split(t[16 * ks + kk][cl], h, m, l);
      const int64_t o = (k / kX6Step) * sst + c * kX6Step + kk;
      out[o] = h;
      out[pstride + o] = m;
      out[2 * pstride + o] = l;
    }
  }
}

// Tile order.  Workgroup b runs on XCD b mod 8 (each XCD has its own L2), so
// XCD x is given a contiguous chunk of the order below and its resident
// workgroups work on neighbouring tiles.  The order sweeps bands of GM tile
// rows column by column (the band's A panels stay in L2 while B panels are
// read by GM tiles each); for the lower part the bands cover the triangle of
// tiles (band rows f..f+GM-1, columns up to each row's diagonal) and then the
// full rows below it.
template <bool LOWER, int GM, int TM = X6T>
__host__ __device__ inline void x6_tile(int64_t b, int64_t T, int64_t M, int64_t N, int64_t& ti, int64_t& tj) {
  const int64_t x = b % 8, q = T / 8, rr = T % 8;
  int64_t t = x * q + (x < rr ? x : rr) + b / 8;
  const int64_t mt = (M + TM - 1) / TM, nt = (N + X6T - 1) / X6T;
  int64_t f = 0;   // first row of the current band
  if (LOWER) {
    // bands of the triangle: rows f..f+g-1 hold g·f + g(g+1)/2 tiles
    for (;;) {
      const int64_t g = nt - f < GM ? nt - f : GM;
      if (g <= 0) break;
      const int64_t cnt = g * f + g * (g + 1) / 2;
      if (t < cnt) {
        if (t < (f + 1) * g) {   // columns 0..f: all g rows
          ti = f + t % g;
          tj = t / g;
          return;
        }
        int64_t r = t - (f + 1) * g;   // column f + c holds rows f + c..f + g - 1
        for (int64_t c = 1;; ++c) {
          if (r < g - c) {
            ti = f + c + r;
            tj = f + c;
            return;
          }
          r -= g - c;
        }
      }
      t -= cnt;
      f += g;
    }
    // rows below the triangle: a rectangle of mt - nt full rows
  }
  const int64_t rows = mt - f, per = GM * nt, g0 = t / per, f1 = g0 * GM;
  const int64_t g = rows - f1 < GM ? rows - f1 : GM, r = t % per;
  ti = f + f1 + r % g;
  tj = r / g;
}

// TM: rows of C per tile, 128 or (full product only) 64 for products of few
// tiles; the waves then hold one 32-row block each instead of two.
// krange: the k-steps a tile multiplies, for an A that is triangular
// (X6KRange): all, from the tile's first row on, or up to its last row.
template <bool LOWER, int GM, int TM>
__global__ __launch_bounds__(256, 2) void x6_gemm_kernel(X6Planes A, X6Planes B, float* __restrict__ C,
                                                        int64_t ldc, int64_t M, int64_t N, float alpha,
                                                        float beta, int krange) {
  __shared__ __attribute__((aligned(16))) uint8_t s0[X6SLOTB], s1[X6SLOTB], s2[X6SLOTB];
  // the wave index in a scalar register: every buffer descriptor and LDS
  // destination below derives from it, and only wave-uniform ones give one
  // instruction per copy (from a vector register the compiler wraps each
  // copy in a loop over the distinct values, a dozen instructions a copy)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  int64_t ti, tj;
  static_assert(TM == X6T || (TM == 64 && !LOWER), "64-row tiles for the full product only");
  constexpr int BI = TM / 64;   // 32-row blocks per wave
  x6_tile<LOWER, GM, TM>(blockIdx.x, gridDim.x, M, N, ti, tj);
  const int64_t i0 = ti * TM, j0 = tj * X6T;
  const int64_t kp = A.kp;
  const int64_t nst = kp / X6KS;
  // stages [st0, st1) of the tile; the ring below runs from st0
  const int64_t st0 = krange == kX6FromRow ? (i0 / X6KS < nst ? i0 / X6KS : nst) : 0;
  const int64_t st1 = krange == kX6ToRow ? ((i0 + TM) / X6KS < nst ? (i0 + TM) / X6KS : nst) : nst;
  // 24 copy instructions per stage = (operand, plane, row quarter); wave w
  // issues 6 of them.  Lane i of one covers row 32q + i/2, 16 bytes, into LDS
  // chunk i%2 holding source chunk (i%2) ^ ((row >> 3) & 1) (bank spread); the
  // source of one instruction is the 1 KB k-step piece of its 32 rows.
  constexpr int32_t kOut = 0x7ffffff0;
  int32_t voff[6];
  const uint16_t* obase[6];
  int64_t ostep[6];
  int32_t obytes[6];
  int ldso[6];
#pragma unroll
  for (int u = 0; u < 6; ++u) {
    const int idx = wave * 6 + u;
    const int op = idx / 12, plane = (idx / 4) % 3, q = idx % 4;
    const int row = 32 * q + (lane >> 1);
    const int cs = (lane & 1) ^ ((row >> 3) & 1);
    const X6Planes& P = op == 0 ? A : B;
    const int64_t grow = (op == 0 ? i0 : j0) + row;
    obase[u] = P.p + (int64_t)plane * P.pstride;
    ostep[u] = P.sst;
    obytes[u] = (int32_t)(P.rows * kX6Step * 2);
    // A rows past the tile (TM = 64) read as zero like rows past the operand
    voff[u] = (grow < P.rows && (op != 0 || row < TM)) ? (int32_t)(grow * kX6Step * 2 + cs * 16) : kOut;
    ldso[u] = op * X6OPB + plane * X6PLANEB + q * 1024;
  }
  auto issue = [&](int64_t st, uint8_t* slot) {
#pragma unroll
    for (int u = 0; u < 6; ++u) {
      const bool live = st < st1;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(obase[u]) + (live ? st * ostep[u] : 0), 0, live ? obytes[u] : 0, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(slot + ldso[u]), 16, voff[u], 0, 0, 0);
    }
  };
  f32x16 acc[BI][2];
#pragma unroll
  for (int i = 0; i < BI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  auto frag = [&](const uint8_t* slot, int op, int plane, int r0) {
    const int row = r0 + (lane & 31);
    const int c = (lane >> 5) ^ ((row >> 3) & 1);
    return *reinterpret_cast<const bf16x8_t*>(slot + op * X6OPB + plane * X6PLANEB + row * X6ROWB + c * 16);
  };
  auto compute = [&](const uint8_t* slot, int64_t st, uint8_t* refill) {
    bf16x8_t fa[BI][3], fb[2][3];
#pragma unroll
    for (int p = 0; p < 3; ++p) {
#pragma unroll
      for (int i = 0; i < BI; ++i) fa[i][p] = frag(slot, 0, p, wr * (TM / 2) + i * 32);
#pragma unroll
      for (int i = 0; i < 2; ++i) fb[i][p] = frag(slot, 1, p, wc * 64 + i * 32);
    }
#pragma unroll
    for (int i = 0; i < BI; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        // smallest terms first: lo·hi, hi·lo, mid·mid, mid·hi, hi·mid, hi·hi
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i][2], fb[j][0], acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i][0], fb[j][2], acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i][1], fb[j][1], acc[i][j], 0, 0, 0);
        if (i == 0 && j == 0) issue(st + X6RING - 1, refill);
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i][1], fb[j][0], acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i][0], fb[j][1], acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i][0], fb[j][0], acc[i][j], 0, 0, 0);
      }
  };
  // stage st is in slot (st - st0) % 3; before computing it, every wave's
  // copies of it are done (its own by vmcnt, the others' by the barrier) and
  // every wave has finished stage st - 1, whose slot the refill of stage
  // st + 2 reuses
  auto step = [&](int64_t st, const uint8_t* cur, uint8_t* refill) {
    __builtin_amdgcn_s_waitcnt(x6_vmcnt(6 * (X6RING - 2)));
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    compute(cur, st, refill);
  };
  issue(st0, s0);
  issue(st0 + 1, s1);
  for (int64_t st = st0; st < st1; st += 3) {
    step(st, s0, s2);
    step(st + 1, s1, s0);
    step(st + 2, s2, s1);
  }
  __builtin_amdgcn_s_waitcnt(x6_vmcnt(0));
  // C tile: element (i, j) of a 32 x 32 block in lane j%32 + 32((i/4)%2),
  // register (i%4) + 4(i/8).  Reads of C are unconditional loads from an
  // address inside the tile (elements outside the result read the tile's
  // first element and drop it), so all of them are in flight together; a
  // conditional load would be compiled as a branch with a wait of its own.
  const int li = lane & 31, lk = lane >> 5;
  const int64_t rows = M - i0 < TM ? M - i0 : TM, cols = N - j0 < X6T ? N - j0 : X6T;
  float* const ct = C + i0 * ldc + j0;
  const bool diag = LOWER && ti == tj;   // a diagonal tile of the lower part: row >= column only
  float old[BI][2][16];
  if (beta != 0.f) {
#pragma unroll
    for (int bi = 0; bi < BI; ++bi)
#pragma unroll
      for (int bj = 0; bj < 2; ++bj) {
        const int j = wc * 64 + bj * 32 + li;
        const int ib = wr * (TM / 2) + bi * 32 + 4 * lk;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int i = ib + 8 * (v >> 2) + (v & 3);
          const bool in = i < rows && j < cols && (!diag || i >= j);
          const float x = ct[in ? (int64_t)i * ldc + j : 0];
          old[bi][bj][v] = in ? x : 0.f;
        }
      }
  } else {
#pragma unroll
    for (int bi = 0; bi < BI; ++bi)
#pragma unroll
      for (int bj = 0; bj < 2; ++bj)
#pragma unroll
        for (int v = 0; v < 16; ++v) old[bi][bj][v] = 0.f;
  }
#pragma unroll
  for (int bi = 0; bi < BI; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) {
      const int j = wc * 64 + bj * 32 + li;
      const int ib = wr * (TM / 2) + bi * 32 + 4 * lk;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = ib + 8 * (v >> 2) + (v & 3);
        const bool in = i < rows && j < cols && (!diag || i >= j);
        if (in) ct[(int64_t)i * ldc + j] = alpha * acc[bi][bj][v] + beta * old[bi][bj][v];
      }
    }
}

}  // namespace

gptq_status launch_x6_split_rows(const float* X, int64_t ldx, int64_t rows, int64_t K, int64_t kp,
                                 uint16_t* out, int64_t pstride, int64_t sst, hipStream_t stream, bool lower) {
  if (rows <= 0) return GPTQ_OK;
  if (kp % kX6Step != 0 || sst < rows * kX6Step) {
    set_error("launch_x6_split_rows: kp %lld, step stride %lld for %lld rows", (long long)kp, (long long)sst,
              (long long)rows);
    return GPTQ_ERR_INVALID_ARG;
  }
  const int64_t total = rows * kp;
  hipLaunchKernelGGL(x6_split_rows_kernel, dim3((unsigned)std::min<int64_t>(ceil_div(total, 256), 4096)),
                     dim3(256), 0, stream, X, ldx, rows, K, kp, out, pstride, sst, (int)lower);
  GPTQ_LAUNCH_CHECK();
  return GPTQ_OK;
}

gptq_status launch_x6_split_cols(const float* X, int64_t ldx, int64_t K, int64_t cols, int64_t kp,
                                 uint16_t* out, int64_t pstride, int64_t sst, hipStream_t stream, bool lower) {
  if (cols <= 0) return GPTQ_OK;
  if (kp % 64 != 0 || sst < cols * kX6Step) {   // the kernel writes whole 64-position tiles of k
    set_error("launch_x6_split_cols: kp %lld, step stride %lld for %lld columns", (long long)kp, (long long)sst,
              (long long)cols);
    return GPTQ_ERR_INVALID_ARG;
  }
  if (K <= 0 || K > kp) {   // the kernel reads rows up to min(k, K - 1)
    set_error("launch_x6_split_cols: K = %lld (1 .. %lld)", (long long)K, (long long)kp);
    return GPTQ_ERR_INVALID_ARG;
  }
  hipLaunchKernelGGL(x6_split_cols_kernel, dim3((unsigned)ceil_div(cols, 64), (unsigned)ceil_div(kp, 64)),
                     dim3(256), 0, stream, X, ldx, K, cols, kp, out, pstride, sst, (int)lower);
  GPTQ_LAUNCH_CHECK();
  return GPTQ_OK;
}

gptq_status launch_x6_gemm(const X6Planes& A, const X6Planes& B, float* C, int64_t ldc, int64_t M,
                           int64_t N, float alpha, float beta, bool lower, hipStream_t stream, bool polite,
                           int tile_rows, int krange) {
  if (M <= 0 || N <= 0) return GPTQ_OK;
  if (A.kp != B.kp || A.kp % X6KS != 0 || A.sst < A.rows * kX6Step || B.sst < B.rows * kX6Step ||
      A.rows * kX6Step * 2 > INT32_MAX || B.rows * kX6Step * 2 > INT32_MAX) {
    set_error("launch_x6_gemm: plane widths %lld / %lld", (long long)A.kp, (long long)B.kp);
    return GPTQ_ERR_INVALID_ARG;
  }
  const int64_t mt = ceil_div(M, X6T), nt = ceil_div(N, X6T);
  // polite: dynamic LDS padding to more than half a CU's LDS, so one workgroup
  // per CU and room beside it for a 74 KB workgroup of another kernel
  const size_t pad = polite ? kX6PolitePad : 0;
  if (krange != kX6All && (lower || tile_rows != X6T || krange < kX6All || krange > kX6ToRow)) {
    set_error("launch_x6_gemm: k range %d (full products of 128-row tiles)", krange);
    return GPTQ_ERR_INVALID_ARG;
  }
  if (tile_rows != X6T && (tile_rows != 64 || lower)) {
    set_error("launch_x6_gemm: tile_rows %d (128, or 64 for a full product)", tile_rows);
    return GPTQ_ERR_INVALID_ARG;
  }
  if (lower) {
    if (M < N) {
      set_error("launch_x6_gemm: lower part needs M (%lld) >= N (%lld)", (long long)M, (long long)N);
      return GPTQ_ERR_INVALID_ARG;
    }
    hipLaunchKernelGGL((x6_gemm_kernel<true, kX6Band, X6T>), dim3((unsigned)(nt * (nt + 1) / 2 + (mt - nt) * nt)),
                       dim3(256), pad, stream, A, B, C, ldc, M, N, alpha, beta, krange);
  } else if (tile_rows == 64) {
    hipLaunchKernelGGL((x6_gemm_kernel<false, kX6Band, 64>), dim3((unsigned)(ceil_div(M, 64) * nt)), dim3(256), pad,
                       stream, A, B, C, ldc, M, N, alpha, beta, krange);
  } else {
    hipLaunchKernelGGL((x6_gemm_kernel<false, kX6Band, X6T>), dim3((unsigned)(mt * nt)), dim3(256), pad, stream, A,
                       B, C, ldc, M, N, alpha, beta, krange);
  }
  GPTQ_LAUNCH_CHECK();
  return GPTQ_OK;
}

}  // namespace gptq
