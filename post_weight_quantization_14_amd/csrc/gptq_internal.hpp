// Internal declarations shared by the HIP translation units of libgptq_mi355x.
// Device code targets gfx950 (CDNA4) only: wave64, MFMA, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "gptq_mi355x.h"

namespace gptq {

// ---------------------------------------------------------------- vectors
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// ---------------------------------------------------------------- errors
void set_error(const char* fmt, ...);
void clear_error();

#define GPTQ_HIP_CHECK(expr)                                                         \
  do {                                                                               \
    hipError_t _e = (expr);                                                          \
    if (_e != hipSuccess) {                                                          \
      ::gptq::set_error("%s failed: %s (%s:%d)", #expr, hipGetErrorString(_e),       \
                        __FILE__, __LINE__);                                         \
      return GPTQ_ERR_HIP;                                                           \
    }                                                                                \
  } while (0)

#define GPTQ_LAUNCH_CHECK()                                                          \
  do {                                                                               \
    hipError_t _e = hipGetLastError();                                               \
    if (_e != hipSuccess) {                                                          \
      ::gptq::set_error("kernel launch failed: %s (%s:%d)", hipGetErrorString(_e),   \
                        __FILE__, __LINE__);                                         \
      return GPTQ_ERR_HIP;                                                           \
    }                                                                                \
  } while (0)

#define GPTQ_TRY(expr)                 \
  do {                                 \
    gptq_status _st = (expr);          \
    if (_st != GPTQ_OK) return _st;    \
  } while (0)

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ---------------------------------------------------------------- side stream
// Lookahead: work the caller's stream does not need until later runs on
// other streams of the same device, ordered by events.  kSideStreams side
// streams with four events each per host thread and device, created on first
// use (default priority) and kept until the process ends, so concurrent calls
// from different host threads never share them.
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t ready = nullptr;   // recorded on the caller's stream, waited on by the side stream
  hipEvent_t done = nullptr;    // recorded on the side stream, waited on by the caller's stream
  hipEvent_t aux[2] = {nullptr, nullptr};   // two more side-stream points, used alternately
};
constexpr int kSideStreams = 3;
gptq_status get_side_stream(SideStream& out, int which = 0);   // 0 <= which < kSideStreams

// Joins side streams back into the caller's stream when a launcher returns
// early (a failed launch or runtime call after side work was issued): the
// caller's stream, and so the caller's allocator, must not run ahead of
// kernels still reading or writing its buffers.  The normal path joins
// explicitly and then calls release().
class SideJoin {
 public:
  explicit SideJoin(hipStream_t caller) : caller_(caller) {}
  SideJoin(const SideJoin&) = delete;
  SideJoin& operator=(const SideJoin&) = delete;
  void add(const SideStream& s) {
    if (count_ < kSideStreams) sides_[count_++] = s;
  }
  void release() { count_ = 0; }
  ~SideJoin() {
    for (int i = 0; i < count_; ++i) {
      if (hipEventRecord(sides_[i].done, sides_[i].stream) == hipSuccess)
        (void)hipStreamWaitEvent(caller_, sides_[i].done, 0);
    }
  }

 private:
  hipStream_t caller_;
  SideStream sides_[kSideStreams];
  int count_ = 0;
};

// ---------------------------------------------------------------- Hessian (stage 1)
constexpr int kSyrkTile = 256;      // output tile edge of the bf16 SYRK
constexpr int kSyrkStage = 32;      // tokens per LDS ring slot
constexpr int kSyrkMaxSliceTokens = 32768;  // fp32 register chains stay this short

struct SyrkPlan {
  int64_t panels = 0;   // ceil(n / 256)
  int64_t tiles = 0;    // lower-triangle tiles
  int64_t splits = 1;   // token slices (split-K)
  int64_t slice_tokens = 0;
  size_t partial_bytes = 0, keypart_bytes = 0;
  size_t total_bytes = 0;
};
SyrkPlan plan_syrk_bf16(int64_t n, int64_t tokens);

gptq_status launch_hessian_bf16(float* H, double* key, int64_t n, const uint16_t* X, int64_t tokens,
                                int64_t ldx, float alpha, void* ws, const SyrkPlan& plan,
                                hipStream_t stream);
gptq_status launch_hessian_f32(float* H, double* key, int64_t n, const float* X, int64_t tokens,
                               int64_t ldx, float alpha, hipStream_t stream);

// ---------------------------------------------------------------- prepare (stages 2-3)
constexpr int kNb = 128;            // panel / tile edge of the fp32 factorisations
constexpr int64_t kPrepareMaxN = 40960;  // one row of H must fit in LDS (160 KB)

struct PreparePlan {
  int64_t n = 0, n_pad = 0, nblk = 0;
  size_t a_off = 0, m_off = 0, lam_off = 0, flag_off = 0, x6_off = 0, tx6_off = 0, total = 0;
};
PreparePlan plan_prepare(int64_t n);
gptq_status run_prepare(float* H, const double* key, int64_t n, double damp, int desc_act,
                        int32_t* perm, void* ws, const PreparePlan& plan, double* damp_out,
                        hipStream_t stream);

// ---------------------------------------------------------------- quantize (stages 4-5)
constexpr int kQBlock = 128;

struct QuantPlan {
  int64_t m = 0, n = 0, ldw = 0, groups = 0, words = 0;
  size_t wp_off = 0, part_off = 0, codes_off = 0, loss_off = 0, inv_off = 0,
         flag_off = 0, x6a_off = 0, x6b_off = 0, total = 0;
};
QuantPlan plan_quantize(int64_t m, int64_t n, const gptq_config& cfg);
gptq_status run_quantize(const void* W, int w_dtype, int64_t m, int64_t n, const float* U,
                         const int32_t* perm, const gptq_config& cfg, uint32_t* qweight,
                         float* scales, int32_t* zeros, int32_t* g_idx, double* loss,
                         int32_t* status, void* ws, const QuantPlan& plan, hipStream_t stream);

// ---------------------------------------------------------------- linear (RTN) quantizer
// One workgroup per output row sorts each group's keys in LDS: G·P floats plus
// two doubles per group must fit in kRtnMaxLds.
constexpr size_t kRtnMaxLds = 150 * 1024;
struct RtnPlan {
  int64_t g = 1, G = 1, P = 1;   // group width, groups per row, padded segment length
  size_t lds_bytes = 0;
  size_t part_off = 0, flag_off = 0, total = 0;
};
RtnPlan plan_rtn(int64_t m, int64_t n, int32_t group_size);
// colscale (optional, per input column): quantize fl(w·colscale) and take the
// errors against w with ŵ = (q - z)·s / colscale.  extra_flag (optional):
// a device flag set by an earlier kernel of the same call, read at the end.
// status (device, optional): receives GPTQ_OK or GPTQ_ERR_NONFINITE in stream
// order; nothing synchronises.
gptq_status run_rtn(const void* W, int w_dtype, int64_t m, int64_t n, int bits, int sym, float clip,
                    uint32_t* qweight, float* scales, int32_t* zeros, double* err, int32_t* status, void* ws,
                    const RtnPlan& plan, hipStream_t stream, const float* colscale = nullptr,
                    const int* extra_flag = nullptr);

// ---------------------------------------------------------------- AWQ channel scaling
struct AwqStatsPlan {
  int64_t slices = 1, rows_per_slice = 0;
  size_t total = 0;   // partial sums [slices][n] fp64
};
AwqStatsPlan plan_awq_stats(int64_t n, int64_t tokens);
gptq_status run_awq_stats(const void* X, int x_dtype, int64_t tokens, int64_t ldx, int64_t n,
                          double* abs_sum, void* ws, const AwqStatsPlan& plan, hipStream_t stream);
size_t awq_extra_bytes();   // workspace of the scale step, before the quantizer's
gptq_status run_awq_quantize(const void* W, int w_dtype, int64_t m, int64_t n, const double* abs_sum,
                             int64_t tokens, float protect, int bits, int sym, float clip,
                             uint32_t* qweight, float* scales, int32_t* zeros, float* channel_scale,
                             double* err, int32_t* status, void* ws, const RtnPlan& plan, hipStream_t stream);

// ---------------------------------------------------------------- W4A16 product
struct W4Layout {
  int64_t m = 0, n = 0, mt = 0, kc = 0, n128 = 0, g = 0, G = 0, Gp = 0;
  size_t flag_off = 0, order_off = 0, param_off = 0, code_off = 0, total = 0;
};
W4Layout plan_w4a16(int64_t m, int64_t n, int32_t group_size);
struct W4GemmPlan {
  int64_t chunk_tokens = 0, mp = 0, chunks = 0, splits = 0;
  size_t xp_off = 0, xs_off = 0, part_off = 0, total = 0;
};
// max_chunk_tokens: tokens per gather / product / reduce sequence, at most 64
W4GemmPlan plan_w4a16_gemm(int64_t tokens, int64_t m, int64_t n, int64_t max_chunk_tokens = 64);
gptq_status run_w4a16_pack(const uint32_t* qweight, const float* scales, const int32_t* zeros,
                           const int32_t* g_idx, int bits, const W4Layout& L, void* packed,
                           hipStream_t stream);
gptq_status run_w4a16_matmul(const uint16_t* X, int64_t tokens, int64_t ldx, const void* packed,
                             const W4Layout& L, float* Y, int64_t ldy, void* ws,
                             const W4GemmPlan& p, hipStream_t stream);
// The same product on the library's own per-device scratch array (no workspace
// argument, no allocation); GPTQ_ERR_UNSUPPORTED when even 16 tokens per launch
// need more than it holds.
size_t w4a16_noalloc_scratch_bytes();
W4GemmPlan plan_w4a16_noalloc(int64_t tokens, int64_t m, int64_t n);
gptq_status run_w4a16_matmul_noalloc(const uint16_t* X, int64_t tokens, int64_t ldx, const void* packed,
                                     const W4Layout& L, float* Y, int64_t ldy, hipStream_t stream);

// ---------------------------------------------------------------- fp32-accurate GEMM on bf16 MFMA
// Operands as three exact bf16 planes, each stored k-step-major: element
// (r, k) of plane q at p + q·pstride + (k / 16)·sst + 16·r + k % 16, so the 16
// k positions of one MFMA step are 32 contiguous bytes per row and a step of
// consecutive rows is one contiguous block (sst = 16 × the rows allocated; a
// view of rows r0.. of a plane is p + 16·r0 with the same sst).
// C = alpha·A·Bᵀ + beta·C, or only its lower part (row >= column).
struct X6Planes {
  const uint16_t* p;
  int64_t rows, kp, pstride, sst;
};
constexpr int64_t kX6K = 512;   // k extent of the trailing updates that use it
// x = h + m + l exactly, each a bf16 (bit pattern): h = x truncated to bf16,
// m = (x - h) truncated, l = the rest (24 significand bits in three pieces)
__device__ __forceinline__ void x6_split(float x, uint16_t& h, uint16_t& m, uint16_t& l) {
  const uint32_t hb = __float_as_uint(x) & 0xffff0000u;
  const float r1 = x - __uint_as_float(hb);
  const uint32_t mb = __float_as_uint(r1) & 0xffff0000u;
  const float r2 = r1 - __uint_as_float(mb);
  const uint32_t lb = __float_as_uint(r2) & 0xffff0000u;
  h = (uint16_t)(hb >> 16);
  m = (uint16_t)(mb >> 16);
  l = (uint16_t)(lb >> 16);
}
constexpr int64_t kX6Step = 16;  // k positions per contiguous row piece
// planes of X[r][k] (r < rows, k < K; zero for K <= k < kp) at out, rows
// 0..rows-1; lower: X is lower triangular, its entries k > r taken as zero
gptq_status launch_x6_split_rows(const float* X, int64_t ldx, int64_t rows, int64_t K, int64_t kp,
                                 uint16_t* out, int64_t pstride, int64_t sst, hipStream_t stream,
                                 bool lower = false);
// planes of the transpose of X[k][c] (k < K, c < cols): plane row c holds
// column c; lower: X is lower triangular, its entries k < c taken as zero
gptq_status launch_x6_split_cols(const float* X, int64_t ldx, int64_t K, int64_t cols, int64_t kp,
                                 uint16_t* out, int64_t pstride, int64_t sst, hipStream_t stream,
                                 bool lower = false);
// k range of a full product whose A is triangular (128-row tiles): every
// k-step; from the tile's first row on (A upper triangular: A[i][k] = 0 for
// k < i); up to the tile's last row (A lower triangular: A[i][k] = 0 for k > i)
enum X6KRange { kX6All = 0, kX6FromRow = 1, kX6ToRow = 2 };
// polite: at most one workgroup per CU, leaving LDS for a latency-bound
// kernel of another stream (the leaf or the block quantizer) beside it.
// tile_rows: 128, or 64 (full product only) for products of few tiles.
gptq_status launch_x6_gemm(const X6Planes& A, const X6Planes& B, float* C, int64_t ldc, int64_t M,
                           int64_t N, float alpha, float beta, bool lower, hipStream_t stream,
                           bool polite = false, int tile_rows = 128, int krange = kX6All);

// ---------------------------------------------------------------- fp32 MFMA GEMM (shared)
// C[M,N] = alpha * A[M,K] * B[K,N] + beta * C, A row-major; B row-major or, with
// b_colmajor, stored as B[k][j] = Bp[j * ldb + k].  Tiles of 128 x 128.
struct GemmArgs {
  const float* A; int64_t lda;
  const float* B; int64_t ldb;
  float* C; int64_t ldc;
  int64_t M, N;
  int64_t k_begin, k_end;
  float alpha, beta;
  // optional (launch_gemm_rect, beta = 0): rows >= pl_row0 of the result also
  // go to x6 planes, result (i, j) as plane row i - pl_row0, position
  // pl_col0 + j (layout of X6Planes: planes pl_pstride apart, k-steps pl_sst)
  uint16_t* pl = nullptr;
  int64_t pl_pstride = 0, pl_sst = 0, pl_row0 = 0, pl_col0 = 0;
};
// tile_rows: 128, or 64 (column-major B only) for products of few row tiles.
gptq_status launch_gemm_rect(const GemmArgs& g, bool b_colmajor, hipStream_t stream, int tile_rows = 128);
// Lower part only (element row >= column) of an M x N result, M >= N: the
// trailing updates of the blocked Cholesky (a triangle, or a triangle over a
// rectangle of full tiles).
gptq_status launch_gemm_lower(const GemmArgs& g, bool b_colmajor, hipStream_t stream);
// Step 1 (T = L21·M11) or step 2 (M21 = -M22·T) of nodes p0 .. p0+count-1 of
// one level (`half` blocks per side) of the blocked triangular inverse's
// bottom-up doubling (see prepare.hip).
gptq_status launch_trtri_nodes(float* Amat, float* Mmat, int64_t lda, int64_t nblk, int64_t half,
                               int64_t p0, int64_t count, int step, hipStream_t stream);

// Export to the checkpoint tensor layout (checkpoint.hip): qweight
// [ceil(n·bits/32)][m], qzeros [G][ceil(m·bits/32)] int32 bit streams,
// scales [G][m] fp16.  Arguments checked by the caller.
gptq_status run_checkpoint_export(const uint32_t* qweight, const float* scales, const int32_t* zeros, int64_t m,
                                  int64_t n, int bits, int64_t G, int zero_offset, int32_t* ck_qweight,
                                  int32_t* ck_qzeros, uint16_t* ck_scales, hipStream_t stream);

}  // namespace gptq
