// fp32 MFMA GEMM tiles for gfx950: C = alpha * A * B + beta * C.
//
// Used by the blocked Cholesky (panel solve and trailing update), the blocked
// triangular inverse and the lazy trailing update of the column quantizer.
// All three are dense fp32 contractions, so they run on v_mfma_f32_32x32x2f32.
//
// Tile: 128 x 128 outputs per workgroup of 256 threads (4 waves in 2 x 2);
// each wave owns 64 x 64 = 2 x 2 MFMA blocks of 32 x 32.  K is staged through
// LDS 32 at a time, double buffered, with the next stage's global loads in
// flight while the current one feeds the MFMAs.
//
// LDS layouts (floats):
//   A (row-major source)      [128 rows][34]  -> lane reads (row, k): bank
//                              34*row + k covers 64 distinct banks per wave.
//   B row-major source        [32 k][160]     -> bank 32*k + col: distinct.
//   B column-major source     [128 cols][34]  -> same as A.
#include "gptq_internal.hpp"

namespace gptq {
namespace {

constexpr int GT = 128;
constexpr int GK = 32;
constexpr int PA = GK + 2;   // row-major tile pitch
constexpr int PB = GT + 32;  // k-major tile pitch
constexpr int SA = GT * PA;
constexpr int SB = (GT * PA > GK * PB) ? GT * PA : GK * PB;

struct GemmSmem {
  float a[2][SA];
  float b[2][SB];
};

// Sixteen zero bytes: the source of every out-of-range 16-byte piece.
__device__ __attribute__((aligned(16))) float gemm_zero4[4];

// base[row * ld + col + e] for e < 4, zero outside row < row_lim, col + e < col_lim.
// Every load is unconditional and its value is used as loaded: a load under
// a condition, or a select on its value, makes the compiler wait for it at
// once, so the loads of a stage would go out one memory latency apart
// instead of together.  VEC (16-byte aligned rows, col and col_lim multiples
// of 4, so a piece is wholly in range or wholly out): one 16-byte load, of
// gemm_zero4 for a piece out of range.  Otherwise every element is loaded
// from a clamped address inside the operand and selected.
template <bool VEC>
__device__ __forceinline__ f32x4_t load4(const float* __restrict__ base, int64_t row, int64_t ld,
                                         int64_t col, int64_t row_lim, int64_t col_lim) {
  const bool rok = row < row_lim;
  const float* prow = base + (rok ? row : 0) * ld;
  if (VEC) return *reinterpret_cast<const f32x4_t*>(rok && col < col_lim ? prow + col : gemm_zero4);
  f32x4_t v;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bool ok = rok && col + e < col_lim;
    const float y = prow[ok ? col + e : 0];
    v[e] = ok ? y : 0.f;
  }
  return v;
}

// Accumulate one 128 x 128 tile over k in [k_begin, k_end).
//   A: tile row 0, k = 0 of a row-major [rows x K] operand (lda); rows < a_rows valid.
//   B: row-major -> points at k = 0, tile column 0 (ldb); column-major -> points at
//      tile column 0, k = 0 with B[k][j] = B[j * ldb + k].  Columns < b_cols valid.
// TM = rows of the tile: 128, or 64 (each wave then holds one 32-row block;
// A rows 64..127 load as zero and are never multiplied).
template <bool BCOL, bool VEC, int TM = GT>
__device__ __forceinline__ void gemm_tile_acc(const float* __restrict__ A, int64_t lda,
                                              int64_t a_rows, const float* __restrict__ B,
                                              int64_t ldb, int64_t b_cols, int64_t k_begin,
                                              int64_t k_end, GemmSmem& sm, f32x16_t (&acc)[TM / 64][2]) {
  constexpr int BI = TM / 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int li = lane & 31, lk = lane >> 5;

#pragma unroll
  for (int bi = 0; bi < BI; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[bi][bj][v] = 0.f;

  if (k_end <= k_begin) return;
  const int64_t nst = (k_end - k_begin + GK - 1) / GK;

  f32x4_t ra[4], rb[4];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int f = tid + 256 * u;
      ra[u] = load4<VEC>(A, f >> 3, lda, k0 + 4 * (f & 7), a_rows, k_end);
      if (BCOL)
        rb[u] = load4<VEC>(B, f >> 3, ldb, k0 + 4 * (f & 7), b_cols, k_end);
      else
        rb[u] = load4<VEC>(B, k0 + (f >> 5), ldb, 4 * (f & 31), k_end, b_cols);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int f = tid + 256 * u;
      float* pa = &sm.a[buf][(f >> 3) * PA + 4 * (f & 7)];
      pa[0] = ra[u][0]; pa[1] = ra[u][1]; pa[2] = ra[u][2]; pa[3] = ra[u][3];
      if (BCOL) {
        float* pb = &sm.b[buf][(f >> 3) * PA + 4 * (f & 7)];
        pb[0] = rb[u][0]; pb[1] = rb[u][1]; pb[2] = rb[u][2]; pb[3] = rb[u][3];
      } else {
        *reinterpret_cast<f32x4_t*>(&sm.b[buf][(f >> 5) * PB + 4 * (f & 31)]) = rb[u];
      }
    }
  };

  gload(k_begin);
  sstore(0);
  __syncthreads();
  for (int64_t st = 0; st < nst; ++st) {
    const int cur = (int)(st & 1);
    if (st + 1 < nst) gload(k_begin + (st + 1) * GK);
    const float* sa = sm.a[cur];
    const float* sb = sm.b[cur];
#pragma unroll
    for (int kk = 0; kk < GK / 2; ++kk) {
      const int k = 2 * kk + lk;
      float af[BI], bf[2];
#pragma unroll
      for (int bi = 0; bi < BI; ++bi) af[bi] = sa[(wr * (TM / 2) + bi * 32 + li) * PA + k];
#pragma unroll
      for (int bj = 0; bj < 2; ++bj)
        bf[bj] = BCOL ? sb[(wc * 64 + bj * 32 + li) * PA + k] : sb[k * PB + wc * 64 + bj * 32 + li];
#pragma unroll
      for (int bi = 0; bi < BI; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
          acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[bi], bf[bj], acc[bi][bj], 0, 0, 0);
    }
    if (st + 1 < nst) sstore(cur ^ 1);
    __syncthreads();
  }
}

// C tile update.  Element (i, j) of the tile sits in lane j % 32 + 32 * ((i / 4) % 2),
// register (i % 4) + 4 * (i / 8) of the 32 x 32 block (the MFMA output layout).
// All 64 reads of C are issued before the first write, as unconditional loads
// from an address inside the tile (an element outside the result reads the
// tile's first element, C[0], and drops it): a conditional load compiles to a
// branch with a wait of its own, one memory latency per element.
template <bool LOWER, int TM = GT>
__device__ __forceinline__ void gemm_tile_store(float* __restrict__ C, int64_t ldc, int64_t c_rows,
                                                int64_t c_cols, int64_t diag_off, float alpha,
                                                float beta, const f32x16_t (&acc)[TM / 64][2]) {
  constexpr int BI = TM / 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int li = lane & 31, lk = lane >> 5;
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
          const bool in = i < c_rows && j < c_cols && (!LOWER || i + diag_off >= j);
          const float x = C[in ? (int64_t)i * ldc + j : 0];
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
        const bool in = i < c_rows && j < c_cols && (!LOWER || i + diag_off >= j);
        if (in) C[(int64_t)i * ldc + j] = alpha * acc[bi][bj][v] + beta * old[bi][bj][v];
      }
    }
}

template <bool BCOL, bool VEC, int TM = GT>
__global__ __launch_bounds__(256) void gemm_rect_kernel(GemmArgs g) {
  __shared__ GemmSmem sm;
  const int64_t i0 = (int64_t)blockIdx.y * TM, j0 = (int64_t)blockIdx.x * GT;
  const float* A = g.A + i0 * g.lda;
  const float* B = BCOL ? g.B + j0 * g.ldb : g.B + j0;
  f32x16_t acc[TM / 64][2];
  const int64_t rows = g.M - i0 < TM ? g.M - i0 : TM;
  const int64_t cols = g.N - j0 < GT ? g.N - j0 : GT;
  gemm_tile_acc<BCOL, VEC, TM>(A, g.lda, rows, B, g.ldb, cols, g.k_begin, g.k_end, sm, acc);
  gemm_tile_store<false, TM>(g.C + i0 * g.ldc + j0, g.ldc, rows, cols, 0, g.alpha, g.beta, acc);
  if (g.pl != nullptr && i0 + TM > g.pl_row0) {   // uniform: the tile reaches the plane rows
    // the tile through LDS (free after the main loop's last barrier), then
    // eight consecutive columns of one row per thread: 16 contiguous bytes of
    // one k-step in each plane
    constexpr int BI = TM / 64;
    constexpr int TP = GT + 4;   // row pitch of the staged tile (floats)
    static_assert(TM * TP * sizeof(float) <= sizeof(GemmSmem), "the staged tile fits the GEMM's LDS");
    float* st = reinterpret_cast<float*>(&sm);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1, li = lane & 31, lk = lane >> 5;
#pragma unroll
    for (int bi = 0; bi < BI; ++bi)
#pragma unroll
      for (int bj = 0; bj < 2; ++bj) {
        const int j = wc * 64 + bj * 32 + li;
        const int ib = wr * (TM / 2) + bi * 32 + 4 * lk;
#pragma unroll
        for (int v = 0; v < 16; ++v) st[(ib + 8 * (v >> 2) + (v & 3)) * TP + j] = g.alpha * acc[bi][bj][v];
      }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < TM * GT / 8 / 256; ++u) {
      const int e = tid + 256 * u;
      const int i = e / (GT / 8), j = 8 * (e % (GT / 8));
      const int64_t pr = i0 + i - g.pl_row0;
      if (i < rows && j < cols && pr >= 0) {
        const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(st + i * TP + j);
        const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(st + i * TP + j + 4);
        uint32_t hw[4], mw[4], lw[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint16_t h0, m0, l0, h1, m1, l1;
          x6_split(q < 2 ? x0[2 * q] : x1[2 * q - 4], h0, m0, l0);
          x6_split(q < 2 ? x0[2 * q + 1] : x1[2 * q - 3], h1, m1, l1);
          hw[q] = h0 | ((uint32_t)h1 << 16);
          mw[q] = m0 | ((uint32_t)m1 << 16);
          lw[q] = l0 | ((uint32_t)l1 << 16);
        }
        const int64_t kc = g.pl_col0 + j0 + j;   // a multiple of 8
        uint16_t* o = g.pl + (kc / kX6Step) * g.pl_sst + pr * kX6Step + kc % kX6Step;
        *reinterpret_cast<uint4*>(o) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        *reinterpret_cast<uint4*>(o + g.pl_pstride) = make_uint4(mw[0], mw[1], mw[2], mw[3]);
        *reinterpret_cast<uint4*>(o + 2 * g.pl_pstride) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      }
    }
  }
}

__device__ __forceinline__ void tri_decode(int64_t t, int64_t& ti, int64_t& tj) {
  int64_t r = (int64_t)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
  while (r * (r + 1) / 2 > t) --r;
  while ((r + 1) * (r + 2) / 2 <= t) ++r;
  ti = r;
  tj = t - r * (r + 1) / 2;
}

// Lower part (i >= j) of an M x N result with M >= N: first the triangle of
// tiles over the top N rows, then the full tiles of the rows below.
template <bool BCOL, bool VEC>
__global__ __launch_bounds__(256) void gemm_lower_kernel(GemmArgs g) {
  __shared__ GemmSmem sm;
  const int64_t nt = (g.N + GT - 1) / GT;
  const int64_t tri = nt * (nt + 1) / 2;
  int64_t ti, tj;
  if ((int64_t)blockIdx.x < tri) {
    tri_decode(blockIdx.x, ti, tj);
  } else {
    const int64_t r = (int64_t)blockIdx.x - tri;
    ti = nt + r / nt;
    tj = r % nt;
  }
  const int64_t i0 = ti * GT, j0 = tj * GT;
  const float* A = g.A + i0 * g.lda;
  const float* B = BCOL ? g.B + j0 * g.ldb : g.B + j0;
  f32x16_t acc[2][2];
  const int64_t rows = g.M - i0 < GT ? g.M - i0 : GT;
  const int64_t cols = g.N - j0 < GT ? g.N - j0 : GT;
  gemm_tile_acc<BCOL, VEC>(A, g.lda, rows, B, g.ldb, cols, g.k_begin, g.k_end, sm, acc);
  gemm_tile_store<true>(g.C + i0 * g.ldc + j0, g.ldc, rows, cols, i0 - j0, g.alpha, g.beta, acc);
}

// ---------------------------------------------------------------------------
// Triangular inverse, one level of the bottom-up doubling.
// M = L^{-1} for a lower-triangular L of nblk x nblk blocks of 128.  At the
// level with `half` blocks per side, node p joins the inverses of blocks
// [l0, l0+half) and [l0+half, r1) (r1 = min(l0 + 2 half, nblk)):
//   step 1: T  = L21 * M11           (K restricted to M11's lower triangle)
//   step 2: M21 = -M22 * T           (K restricted to M22's lower triangle)
// T is parked, transposed, in the strictly upper block triangle of the
// Cholesky buffer, which the factorisation never reads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void trtri_step1_kernel(float* Amat, const float* Mmat,
                                                          int64_t lda, int64_t nblk, int64_t half,
                                                          int64_t p0) {
  __shared__ GemmSmem sm;
  const int64_t p = p0 + blockIdx.y;
  const int64_t l0 = p * 2 * half, r0 = l0 + half;
  const int64_t r1 = (l0 + 2 * half < nblk) ? l0 + 2 * half : nblk;
  const int64_t ti = blockIdx.x / half, tj = blockIdx.x % half;
  if (r0 + ti >= r1) return;
  const float* A = Amat + (r0 + ti) * GT * lda + l0 * GT;           // L21 block row
  const float* B = Mmat + l0 * GT * lda + l0 * GT + tj * GT;         // M11 column block
  f32x16_t acc[2][2];
  gemm_tile_acc<false, true>(A, lda, GT, B, lda, GT, tj * GT, half * GT, sm, acc);
  // store T^T at rows (l0+tj) block, columns (r0+ti) block
  float* Tt = Amat + (l0 + tj) * GT * lda + (r0 + ti) * GT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1, li = lane & 31, lk = lane >> 5;
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // registers 4q..4q+3 hold rows i..i+3 of column j: one 16-byte store
        const int i = wr * 64 + bi * 32 + 8 * q + 4 * lk;
        const int j = wc * 64 + bj * 32 + li;
        f32x4_t v = {acc[bi][bj][4 * q], acc[bi][bj][4 * q + 1], acc[bi][bj][4 * q + 2],
                     acc[bi][bj][4 * q + 3]};
        *reinterpret_cast<f32x4_t*>(Tt + (int64_t)j * lda + i) = v;
      }
}

__global__ __launch_bounds__(256) void trtri_step2_kernel(const float* Amat, float* Mmat,
                                                          int64_t lda, int64_t nblk, int64_t half,
                                                          int64_t p0) {
  __shared__ GemmSmem sm;
  const int64_t p = p0 + blockIdx.y;
  const int64_t l0 = p * 2 * half, r0 = l0 + half;
  const int64_t r1 = (l0 + 2 * half < nblk) ? l0 + 2 * half : nblk;
  const int64_t ti = blockIdx.x / half, tj = blockIdx.x % half;
  if (r0 + ti >= r1) return;
  const float* A = Mmat + (r0 + ti) * GT * lda + r0 * GT;                 // M22 block row
  const float* Bt = Amat + (l0 + tj) * GT * lda + r0 * GT;                // T^T (column-major T)
  f32x16_t acc[2][2];
  gemm_tile_acc<true, true>(A, lda, GT, Bt, lda, GT, 0, (ti + 1) * GT, sm, acc);
  gemm_tile_store<false>(Mmat + (r0 + ti) * GT * lda + l0 * GT + tj * GT, lda, GT, GT, 0, -1.f,
                         0.f, acc);
}

// The 16-byte loads: aligned operand rows, and every 4-element piece wholly
// inside or wholly outside the k range and (row-major B) the columns.
bool vec_ok(const GemmArgs& g, bool bcol) {
  auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  return al(g.A) && al(g.B) && (g.lda % 4 == 0) && (g.ldb % 4 == 0) && (g.k_begin % 4 == 0) &&
         (g.k_end % 4 == 0) && (bcol || g.N % 4 == 0);
}

}  // namespace

gptq_status launch_gemm_rect(const GemmArgs& g, bool b_colmajor, hipStream_t stream, int tile_rows) {
  if (g.M <= 0 || g.N <= 0) return GPTQ_OK;
  if (g.pl != nullptr && (g.beta != 0.f || g.N % 8 != 0 || g.pl_col0 % 8 != 0 ||
                          (reinterpret_cast<uintptr_t>(g.pl) & 15) != 0 || g.pl_sst % 8 != 0 || g.pl_pstride % 8 != 0)) {
    set_error("launch_gemm_rect: plane output needs beta = 0 and 16-byte pieces of 8 columns");
    return GPTQ_ERR_INVALID_ARG;
  }
  if (tile_rows != GT && (tile_rows != 64 || !b_colmajor)) {
    set_error("launch_gemm_rect: tile_rows %d (128, or 64 with a column-major B)", tile_rows);
    return GPTQ_ERR_INVALID_ARG;
  }
  const bool v = vec_ok(g, b_colmajor);
  if (tile_rows == 64) {
    dim3 grid64((unsigned)ceil_div(g.N, GT), (unsigned)ceil_div(g.M, 64));
    if (v) hipLaunchKernelGGL((gemm_rect_kernel<true, true, 64>), grid64, dim3(256), 0, stream, g);
    else hipLaunchKernelGGL((gemm_rect_kernel<true, false, 64>), grid64, dim3(256), 0, stream, g);
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
  }
  dim3 grid((unsigned)ceil_div(g.N, GT), (unsigned)ceil_div(g.M, GT));
  if (b_colmajor) {
    if (v) hipLaunchKernelGGL((gemm_rect_kernel<true, true>), grid, dim3(256), 0, stream, g);
    else hipLaunchKernelGGL((gemm_rect_kernel<true, false>), grid, dim3(256), 0, stream, g);
  } else {
    if (v) hipLaunchKernelGGL((gemm_rect_kernel<false, true>), grid, dim3(256), 0, stream, g);
    else hipLaunchKernelGGL((gemm_rect_kernel<false, false>), grid, dim3(256), 0, stream, g);
  }
  GPTQ_LAUNCH_CHECK();
  return GPTQ_OK;
}

gptq_status launch_gemm_lower(const GemmArgs& g, bool b_colmajor, hipStream_t stream) {
  if (g.M <= 0 || g.N <= 0) return GPTQ_OK;
  if (g.M < g.N) {
    set_error("launch_gemm_lower: M (%lld) < N (%lld)", (long long)g.M, (long long)g.N);
    return GPTQ_ERR_INVALID_ARG;
  }
  const int64_t mt = ceil_div(g.M, GT), nt = ceil_div(g.N, GT);
  dim3 grid((unsigned)(nt * (nt + 1) / 2 + (mt - nt) * nt));
  const bool v = vec_ok(g, b_colmajor);
  if (b_colmajor) {
    if (v) hipLaunchKernelGGL((gemm_lower_kernel<true, true>), grid, dim3(256), 0, stream, g);
    else hipLaunchKernelGGL((gemm_lower_kernel<true, false>), grid, dim3(256), 0, stream, g);
  } else {
    if (v) hipLaunchKernelGGL((gemm_lower_kernel<false, true>), grid, dim3(256), 0, stream, g);
    else hipLaunchKernelGGL((gemm_lower_kernel<false, false>), grid, dim3(256), 0, stream, g);
  }
  GPTQ_LAUNCH_CHECK();
  return GPTQ_OK;
}

gptq_status launch_trtri_nodes(float* Amat, float* Mmat, int64_t lda, int64_t nblk, int64_t half,
                               int64_t p0, int64_t count, int step, hipStream_t stream) {
  if (count <= 0) return GPTQ_OK;
  dim3 grid((unsigned)(half * half), (unsigned)count);
  if (step == 1)
    hipLaunchKernelGGL(trtri_step1_kernel, grid, dim3(256), 0, stream, Amat, (const float*)Mmat, lda,
                       nblk, half, p0);
  else
    hipLaunchKernelGGL(trtri_step2_kernel, grid, dim3(256), 0, stream, (const float*)Amat, Mmat, lda,
                       nblk, half, p0);
  GPTQ_LAUNCH_CHECK();
  return GPTQ_OK;
}

}  // namespace gptq
