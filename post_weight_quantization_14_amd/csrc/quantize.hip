// Stages 4-5: block-wise column quantization with error feedback, then packing.
//
// Column c (processing order) of every output row is rounded to the row's
// grid and its rounding error is pushed onto the columns not yet quantized
// through row c of U, the upper Cholesky factor of H⁻¹ (page "大模型量化：
// GPTQ/AWQ/GGUF 原理对比", GPTQ section and its column-by-column flow; page
// "模型量化实战：从 INT8 PTQ 到 GPTQ…" §3.2 quantize_block, §2.1/§3.1 grid):
//     e = (w_c - x̂_c) / U[c][c];   w_k -= e · U[c][k]  (k > c)
// Rows are independent given U.  Columns go in blocks of 128:
//   block_quant : one lane = one output row.  The row's 128-column slab lives
//                 in VGPRs (fully unrolled, static indices); the rows of U's
//                 128 x 128 diagonal block arrive by scalar loads.  Group
//                 min/max at each group start, codes, Err block, ½Σe² per row;
//                 then each workgroup pushes its rows' errors into the rest of
//                 the 512-column superblock (fp32 MFMA, U streamed from HBM).
//   trailing    : W[:, s2:] -= Err · U[s1:s2, s2:] per superblock, as an fp32
//                 MFMA GEMM.
//   finalize    : g_idx / inverse permutation, nibble packing in original
//                 column order, ‖W − Ŵ‖² from the packed outputs, fixed-order
//                 fp64 reductions.
#include <algorithm>

#include "quant_common.hpp"

namespace gptq {
namespace {

constexpr int kFlagNonFinite = 2;


// W_p[r][p] = W[r][perm[p]] (fp32), zero padding up to ldw; flags non-finite W.
template <typename T>
__device__ __forceinline__ float to_f32(T x);
template <>
__device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

template <typename T>
__global__ __launch_bounds__(256) void qprep_kernel(const T* __restrict__ W, int64_t n,
                                                    const int32_t* __restrict__ perm,
                                                    float* __restrict__ Wp, int64_t ldw, int* flag) {
  extern __shared__ float row[];
  __shared__ int bad;
  const int64_t r = blockIdx.x;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  // four loads per thread in flight (unconditional, at clamped indices; a
  // conditional load compiles to a branch and a wait of its own)
  int b = 0;
  for (int64_t j0 = threadIdx.x; j0 < n; j0 += 4 * 256) {
    float x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = to_f32<T>(W[r * n + std::min<int64_t>(j0 + 256 * u, n - 1)]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (!isfinite(x[u])) b = 1;
      row[std::min<int64_t>(j0 + 256 * u, n - 1)] = x[u];
    }
  }
  if (b) atomicOr(&bad, 1);
  __syncthreads();
  if (threadIdx.x == 0 && bad) atomicOr(flag, kFlagNonFinite);
  for (int64_t p0 = threadIdx.x; p0 < ldw; p0 += 4 * 256) {
    int32_t pi[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) pi[u] = perm[std::min<int64_t>(p0 + 256 * u, n - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t p = p0 + 256 * u;
      if (p < ldw) Wp[r * ldw + p] = (p < n) ? row[pi[u]] : 0.f;
    }
  }
}

// One group per row (group_size = -1): grid from the whole original row.
__global__ __launch_bounds__(256) void row_params_kernel(const float* __restrict__ Wp, int64_t ldw,
                                                         int64_t n, int bits, int sym,
                                                         float* scales, int32_t* zeros) {
  __shared__ float rlo[256], rhi[256], ram[256];
  const int64_t r = blockIdx.x;
  float lo = INFINITY, hi = -INFINITY, am = 0.f;
  for (int64_t j = threadIdx.x; j < n; j += 256) {
    const float x = Wp[r * ldw + j];
    lo = fminf(lo, x);
    hi = fmaxf(hi, x);
    am = fmaxf(am, fabsf(x));
  }
  rlo[threadIdx.x] = lo; rhi[threadIdx.x] = hi; ram[threadIdx.x] = am;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      rlo[threadIdx.x] = fminf(rlo[threadIdx.x], rlo[threadIdx.x + w]);
      rhi[threadIdx.x] = fmaxf(rhi[threadIdx.x], rhi[threadIdx.x + w]);
      ram[threadIdx.x] = fmaxf(ram[threadIdx.x], ram[threadIdx.x + w]);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    float s, z;
    grid_params(rlo[0], rhi[0], ram[0], bits, sym, s, z);
    scales[r] = s;
    zeros[r] = (int32_t)z;
  }
}

__global__ __launch_bounds__(256) void gidx_kernel(const int32_t* __restrict__ perm, int64_t n,
                                                   int64_t gw, int32_t* g_idx, int32_t* invperm) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= n) return;
  const int32_t j = perm[p];
  invperm[j] = (int32_t)p;
  g_idx[j] = gw > 0 ? (int32_t)(p / gw) : 0;
}

// qweight word (r, wd) in original column order, and this word's share of
// ‖W − Ŵ‖² (Ŵ rebuilt from the stored code, scale and zero), reduced per
// workgroup into part[].
template <typename T>
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ codes, int64_t ldw,
                                                   const int32_t* __restrict__ invperm,
                                                   const int32_t* __restrict__ g_idx,
                                                   const float* __restrict__ scales,
                                                   const int32_t* __restrict__ zeros, int64_t G,
                                                   const T* __restrict__ W, int64_t m, int64_t n,
                                                   int bits, int64_t words, int64_t bpr,
                                                   uint32_t* __restrict__ qweight, double* part) {
  __shared__ double red[256];
  const int64_t r = blockIdx.x / bpr;
  const int64_t wd = (blockIdx.x % bpr) * 256 + threadIdx.x;
  const int per = bits <= 4 ? 8 : 4, width = bits <= 4 ? 4 : 8;
  double acc = 0.0;
  if (wd < words) {
    uint32_t word = 0;
    float dacc = 0.f;
    for (int i = 0; i < per; ++i) {
      const int64_t j = wd * per + i;
      if (j < n) {
        const uint32_t c = codes[r * ldw + invperm[j]];
        word |= c << (width * i);
        const int64_t g = g_idx[j];
        const float s = scales[r * G + g];
        const float zz = (float)zeros[r * G + g];
        const float d = to_f32<T>(W[r * n + j]) - ((float)c - zz) * s;
        dacc += d * d;
      }
    }
    qweight[r * words + wd] = word;
    acc = dacc;
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

// loss[0] = Σ_rows ½Σe², loss[1] = Σ parts; one workgroup, fixed order.
__global__ __launch_bounds__(1024) void loss_reduce_kernel(const double* loss_rows, int64_t m,
                                                           const double* part, int64_t nparts,
                                                           double* loss) {
  __shared__ double r0[1024], r1[1024];
  double a = 0.0, b = 0.0;
  for (int64_t i = threadIdx.x; i < m; i += 1024) a += loss_rows[i];
  for (int64_t i = threadIdx.x; i < nparts; i += 1024) b += part[i];
  r0[threadIdx.x] = a;
  r1[threadIdx.x] = b;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      r0[threadIdx.x] += r0[threadIdx.x + w];
      r1[threadIdx.x] += r1[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    loss[0] = r0[0];
    loss[1] = r1[0];
  }
}

__global__ void zero_f64_kernel(double* p, int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.0;
}


}  // namespace

static_assert(kQSuper <= kX6K, "a superblock's errors must fit the plane width");
// far updates narrower than this run one workgroup per CU (measured crossover
// between the block quantizer's chain and the far GEMM as the bottleneck)
constexpr int64_t kQPoliteFar = 6500;

QuantPlan plan_quantize(int64_t m, int64_t n, const gptq_config& cfg) {
  QuantPlan p;
  p.m = m;
  p.n = n;
  p.ldw = round_up(std::max<int64_t>(n, 1), QB);
  p.groups = gptq_num_groups(n, cfg.group_size);
  p.words = gptq_qweight_words(n, cfg.bits);
  const int64_t bpr = ceil_div(std::max<int64_t>(p.words, 1), 256);
  size_t off = 0;
  p.wp_off = off; off += align256((size_t)m * p.ldw * sizeof(float));
  p.part_off = off;  // pack partials: one double per (row, word-block)
  off += align256((size_t)m * bpr * sizeof(double));
  p.codes_off = off; off += align256((size_t)m * p.ldw);
  p.err_off = off; off += align256((size_t)2 * m * kQSuper * sizeof(float));   // two superblocks
  p.loss_off = off; off += align256((size_t)m * sizeof(double));
  p.inv_off = off; off += align256((size_t)n * sizeof(int32_t));
  p.flag_off = off; off += 256;
  // bf16 planes of the superblock errors and of U's rows for the trailing
  // updates, double-buffered like the errors
  p.x6a_off = off; off += align256((size_t)2 * 3 * m * kX6K * sizeof(uint16_t));
  p.x6b_off = off; off += align256((size_t)2 * 3 * n * kX6K * sizeof(uint16_t));
  p.total = off;
  return p;
}

gptq_status run_quantize(const void* W, int w_dtype, int64_t m, int64_t n, const float* U,
                         const int32_t* perm, const gptq_config& cfg, uint32_t* qweight,
                         float* scales, int32_t* zeros, int32_t* g_idx, double* loss, void* ws,
                         const QuantPlan& p, hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  float* Wp = reinterpret_cast<float*>(w + p.wp_off);
  double* part = reinterpret_cast<double*>(w + p.part_off);
  uint8_t* codes = reinterpret_cast<uint8_t*>(w + p.codes_off);
  float* err = reinterpret_cast<float*>(w + p.err_off);
  double* loss_rows = reinterpret_cast<double*>(w + p.loss_off);
  int32_t* invperm = reinterpret_cast<int32_t*>(w + p.inv_off);
  int* flag = reinterpret_cast<int*>(w + p.flag_off);

  GPTQ_HIP_CHECK(hipMemsetAsync(flag, 0, sizeof(int), stream));
  hipLaunchKernelGGL(zero_f64_kernel, dim3((unsigned)std::min<int64_t>(ceil_div(m, 256), 1024)),
                     dim3(256), 0, stream, loss_rows, m);
  GPTQ_LAUNCH_CHECK();

  const size_t row_bytes = (size_t)n * sizeof(float);
  if (w_dtype == GPTQ_BF16) {
    if (row_bytes > 65536)
      GPTQ_HIP_CHECK(hipFuncSetAttribute((const void*)qprep_kernel<uint16_t>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)row_bytes));
    hipLaunchKernelGGL(qprep_kernel<uint16_t>, dim3((unsigned)m), dim3(256), row_bytes, stream,
                       static_cast<const uint16_t*>(W), n, perm, Wp, p.ldw, flag);
  } else {
    if (row_bytes > 65536)
      GPTQ_HIP_CHECK(hipFuncSetAttribute((const void*)qprep_kernel<float>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)row_bytes));
    hipLaunchKernelGGL(qprep_kernel<float>, dim3((unsigned)m), dim3(256), row_bytes, stream,
                       static_cast<const float*>(W), n, perm, Wp, p.ldw, flag);
  }
  GPTQ_LAUNCH_CHECK();

  const int gw = cfg.group_size;
  if (gw == -1) {
    hipLaunchKernelGGL(row_params_kernel, dim3((unsigned)m), dim3(256), 0, stream,
                       (const float*)Wp, p.ldw, n, cfg.bits, cfg.sym, scales, zeros);
    GPTQ_LAUNCH_CHECK();
  }

  QArgs a;
  a.Wp = Wp; a.ldw = p.ldw; a.m = m; a.n = n; a.U = U; a.ldu = n;
  a.bits = cfg.bits; a.sym = cfg.sym; a.scales = scales; a.zeros = zeros; a.G = p.groups;
  a.err = err; a.lde = kQSuper; a.codes = codes; a.loss_rows = loss_rows;

  // Two-level lazy update (exact: the same rank-1 corrections, grouped).  A
  // block's errors update the rest of its 512-column superblock at once
  // (K = 128, inside the block's own kernel); the columns after the
  // superblock are updated once per superblock from all of its errors
  // (K = 512), so the working weights are read and written a quarter as often
  // as with per-block updates.
  // Lookahead: of that superblock update, the next superblock's columns run on
  // the caller's stream and the columns after them on the side stream, while
  // the next superblock's column loop (its own columns only) runs here.  The
  // error block alternates between two buffers, so the side stream's reads of
  // one superblock's errors never meet the next superblock's writes.
  SideStream side;
  GPTQ_TRY(get_side_stream(side));
  bool side_pending = false;
  for (int64_t s1 = 0; s1 < n; s1 += kQSuper) {
    const int64_t s2 = std::min<int64_t>(s1 + kQSuper, n);
    float* errs = err + ((s1 / kQSuper) & 1) * m * kQSuper;
    for (int64_t i1 = s1; i1 < s2; i1 += QB) {
      const int bw = (int)std::min<int64_t>(QB, s2 - i1);
      // the quantizer reads only rows and columns < bw of U's diagonal block
      const float* ublk = U + i1 * n + i1;
      const int64_t ldub = n;
      a.err = errs + (i1 - s1);
      // W_p[rows, i1+bw : s2] -= Err_block · U[i1:i1+bw, i1+bw:s2], in the kernel
      const int ncols = (int)(s2 - i1 - bw);
      switch (gw) {
        case -1: launch_block_quant<0>(a, ublk, ldub, i1, bw, ncols, stream); break;
        case 8: launch_block_quant<8>(a, ublk, ldub, i1, bw, ncols, stream); break;
        case 16: launch_block_quant<16>(a, ublk, ldub, i1, bw, ncols, stream); break;
        case 32: launch_block_quant<32>(a, ublk, ldub, i1, bw, ncols, stream); break;
        case 64: launch_block_quant<64>(a, ublk, ldub, i1, bw, ncols, stream); break;
        case 128: launch_block_quant<128>(a, ublk, ldub, i1, bw, ncols, stream); break;
        default:
          set_error("group_size %d not built", gw);
          return GPTQ_ERR_UNSUPPORTED;
      }
      GPTQ_LAUNCH_CHECK();
    }
    if (s2 < n) {   // W_p[:, s2:] -= Err_super · U[s1:s2, s2:]
      const int64_t near = std::min<int64_t>(kQSuper, n - s2), far = n - s2 - near;
      // both operands as exact bf16 planes (fp32-accurate on bf16 MFMA): the
      // errors [m][512] as rows, U[s1:s2, s2:] transposed to [n - s2][512]
      const int par = (int)((s1 / kQSuper) & 1);
      uint16_t* pa = reinterpret_cast<uint16_t*>(w + p.x6a_off) + (size_t)par * 3 * m * kX6K;
      uint16_t* pb = reinterpret_cast<uint16_t*>(w + p.x6b_off) + (size_t)par * 3 * n * kX6K;
      const int64_t K = s2 - s1;
      GPTQ_TRY(launch_x6_split_rows(errs, kQSuper, m, K, kX6K, pa, m * kX6K, stream));
      GPTQ_TRY(launch_x6_split_cols(U + s1 * n + s2, n, K, n - s2, kX6K, pb, n * kX6K, stream));
      const X6Planes PA{pa, m, kX6K, m * kX6K};
      if (side_pending) GPTQ_HIP_CHECK(hipStreamWaitEvent(stream, side.done, 0));
      side_pending = false;
      if (far > 0) {
        GPTQ_HIP_CHECK(hipEventRecord(side.ready, stream));
        GPTQ_HIP_CHECK(hipStreamWaitEvent(side.stream, side.ready, 0));
        const X6Planes PF{pb + near * kX6K, far, kX6K, n * kX6K};
        // a small far update leaves CU room for the next superblock's blocks;
        // a large one is the stage's bottleneck and takes the whole chip
        const bool polite = far < kQPoliteFar;
        GPTQ_TRY(launch_x6_gemm(PA, PF, Wp + s2 + near, p.ldw, m, far, -1.f, 1.f, false, side.stream, polite));
        GPTQ_HIP_CHECK(hipEventRecord(side.done, side.stream));
        side_pending = true;
      }
      const X6Planes PN{pb, near, kX6K, n * kX6K};
      // on the chain: with fewer 128-row tiles than CUs, 64-row tiles
      const int near_rows = ceil_div(m, 128) * ceil_div(near, 128) < 256 ? 64 : 128;
      GPTQ_TRY(launch_x6_gemm(PA, PN, Wp + s2, p.ldw, m, near, -1.f, 1.f, false, stream, false, near_rows));
    }
  }
  if (side_pending) GPTQ_HIP_CHECK(hipStreamWaitEvent(stream, side.done, 0));

  hipLaunchKernelGGL(gidx_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, stream, perm, n,
                     (int64_t)(gw > 0 ? gw : 0), g_idx, invperm);
  GPTQ_LAUNCH_CHECK();
  const int64_t bpr = ceil_div(std::max<int64_t>(p.words, 1), 256);
  const unsigned pgrid = (unsigned)(m * bpr);
  if (w_dtype == GPTQ_BF16)
    hipLaunchKernelGGL(pack_kernel<uint16_t>, dim3(pgrid), dim3(256), 0, stream, (const uint8_t*)codes,
                       p.ldw, (const int32_t*)invperm, (const int32_t*)g_idx, (const float*)scales,
                       (const int32_t*)zeros, p.groups, static_cast<const uint16_t*>(W), m, n,
                       cfg.bits, p.words, bpr, qweight, part);
  else
    hipLaunchKernelGGL(pack_kernel<float>, dim3(pgrid), dim3(256), 0, stream, (const uint8_t*)codes,
                       p.ldw, (const int32_t*)invperm, (const int32_t*)g_idx, (const float*)scales,
                       (const int32_t*)zeros, p.groups, static_cast<const float*>(W), m, n,
                       cfg.bits, p.words, bpr, qweight, part);
  GPTQ_LAUNCH_CHECK();
  hipLaunchKernelGGL(loss_reduce_kernel, dim3(1), dim3(1024), 0, stream, (const double*)loss_rows, m,
                     (const double*)part, (int64_t)(m * bpr), loss);
  GPTQ_LAUNCH_CHECK();

  int hflag = 0;
  GPTQ_HIP_CHECK(hipMemcpyAsync(&hflag, flag, sizeof(int), hipMemcpyDeviceToHost, stream));
  GPTQ_HIP_CHECK(hipStreamSynchronize(stream));
  if (hflag & kFlagNonFinite) {
    set_error("gptq_quantize_layer: W holds a NaN or Inf");
    return GPTQ_ERR_NONFINITE;
  }
  return GPTQ_OK;
}

}  // namespace gptq
