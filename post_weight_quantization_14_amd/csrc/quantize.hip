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

// VEC: rows of 16-byte pieces (n a multiple of 16 / sizeof(T), W 16-byte
// aligned), staged with one 16-byte load per piece.  Loads are unconditional
// at clamped indices, eight (staging) and sixteen (gather) in flight per
// thread: a conditional load compiles to a branch and a wait of its own.
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void qprep_kernel(const T* __restrict__ W, int64_t n,
                                                    const int32_t* __restrict__ perm,
                                                    float* __restrict__ Wp, int64_t ldw, int* flag) {
  extern __shared__ __attribute__((aligned(16))) float row[];
  __shared__ int bad;
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid == 0) bad = 0;
  __syncthreads();
  int b = 0;
  if constexpr (VEC) {
    constexpr int E = 16 / sizeof(T);   // elements per piece
    const int64_t nq = n / E;
    const uint4* src = reinterpret_cast<const uint4*>(W + r * n);
    for (int64_t q0 = tid; q0 < nq; q0 += 8 * 256) {
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = src[std::min<int64_t>(q0 + 256 * u, nq - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t q = q0 + 256 * u;
        if (q < nq) {
          const uint32_t wd[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
          float x[E];
          if constexpr (E == 8) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              x[2 * e] = __uint_as_float(wd[e] << 16);
              x[2 * e + 1] = __uint_as_float(wd[e] & 0xffff0000u);
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(wd[e]);
          }
#pragma unroll
          for (int e = 0; e < E; ++e)
            if (!isfinite(x[e])) b = 1;
#pragma unroll
          for (int e = 0; e < E; e += 4)
            *reinterpret_cast<f32x4_t*>(row + q * E + e) = f32x4_t{x[e], x[e + 1], x[e + 2], x[e + 3]};
        }
      }
    }
  } else {
    for (int64_t j0 = tid; j0 < n; j0 += 8 * 256) {
      float x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = to_f32<T>(W[r * n + std::min<int64_t>(j0 + 256 * u, n - 1)]);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (!isfinite(x[u])) b = 1;
        row[std::min<int64_t>(j0 + 256 * u, n - 1)] = x[u];
      }
    }
  }
  if (b) atomicOr(&bad, 1);
  __syncthreads();
  if (tid == 0 && bad) atomicOr(flag, kFlagNonFinite);
  for (int64_t p0 = tid; p0 < ldw; p0 += 16 * 256) {
    int32_t pi[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) pi[u] = perm[std::min<int64_t>(p0 + 256 * u, n - 1)];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
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
  if (p >= n) {   // invperm is padded to whole 8-entry pieces: positions n.. read as 0
    if (p < (n + 7) / 8 * 8) invperm[p] = 0;
    return;
  }
  const int32_t j = perm[p];
  invperm[j] = (int32_t)p;
  g_idx[j] = gw > 0 ? (int32_t)(p / gw) : 0;
}

// qweight word (r, wd) in original column order, and this word's share of
// ‖W − Ŵ‖² (Ŵ rebuilt from the stored code, scale and zero), reduced per
// workgroup into part[].
template <typename T, int PER>
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ codes, int64_t ldw,
                                                   const int32_t* __restrict__ invperm, int64_t gw,
                                                   const float* __restrict__ scales,
                                                   const int32_t* __restrict__ zeros, int64_t G,
                                                   const T* __restrict__ W, int64_t n, int64_t words,
                                                   uint32_t* __restrict__ qweight, double* part) {
  constexpr int kWidth = 32 / PER;   // bits per code slot: 4 (2-4 bit codes) or 8
  // the row's codes (in processing order) and group parameters go to LDS
  // first: read in original order they are a gather, one cache line per
  // byte, which bound the kernel on the address units
  extern __shared__ __attribute__((aligned(16))) uint8_t psm[];
  uint8_t* cs = psm;
  float* ss = reinterpret_cast<float*>(psm + ldw);
  float* zs = ss + G;
  __shared__ double red[256];
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x;
  for (int64_t o = 16 * tid; o < ldw; o += 16 * 256)   // ldw is a multiple of 128
    *reinterpret_cast<uint4*>(cs + o) = *reinterpret_cast<const uint4*>(codes + r * ldw + o);
  for (int64_t g = tid; g < G; g += 256) {
    ss[g] = scales[r * G + g];
    zs[g] = (float)zeros[r * G + g];
  }
  __syncthreads();
  float dacc = 0.f;
  for (int64_t wd = tid; wd < words; wd += 256) {
    // unconditional loads at clamped positions, all in flight together (a
    // conditional load compiles to a branch and a wait of its own)
    // the word's processing positions: 16-byte loads (invperm is padded to
    // whole pieces of 8); its group is the position's 128-column block of
    // groups, position / gw (gw = 0: one group)
    int32_t ip[PER];
    float wv[PER];
#pragma unroll
    for (int h = 0; h < PER / 4; ++h) {
      const int4 q = *reinterpret_cast<const int4*>(invperm + wd * PER + 4 * h);
      ip[4 * h] = q.x; ip[4 * h + 1] = q.y; ip[4 * h + 2] = q.z; ip[4 * h + 3] = q.w;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) wv[i] = to_f32<T>(W[r * n + std::min<int64_t>(wd * PER + i, n - 1)]);
    int32_t gi[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) gi[i] = gw > 0 ? ip[i] / (int32_t)gw : 0;
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (wd * PER + i < n) {
        const uint32_t c = cs[ip[i]];
        word |= c << (kWidth * i);
        const float d = wv[i] - ((float)c - zs[gi[i]]) * ss[gi[i]];
        dacc += d * d;
      }
    }
    qweight[r * words + wd] = word;
  }
  red[tid] = dacc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (tid == 0) part[r] = red[0];
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

// Clears the per-row loss accumulators and the call's flag word (a kernel,
// not a memset, so the call can be captured in a graph).
__global__ void zero_f64_kernel(double* p, int64_t count, int* flag) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *flag = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.0;
}

// The call's status word for the caller: 0, or GPTQ_ERR_NONFINITE.
__global__ void status_kernel(const int* flag, int32_t* status) {
  *status = (*flag & kFlagNonFinite) ? (int32_t)GPTQ_ERR_NONFINITE : (int32_t)GPTQ_OK;
}


}  // namespace

static_assert(kQSuper <= kX6K, "a superblock's errors must fit the plane width");
// far updates narrower than this run one workgroup per CU (measured crossover
// between the block quantizer's chain and the far GEMM as the bottleneck)
constexpr int64_t kQPoliteFar = 6500;

// Plane rows of U's trailing-update operands for the superblocks before s1
// (all of them for s1 = n): superblock [t, t + 512) contributes n - t - 512
// rows when t + 512 < n.
int64_t uplane_rows(int64_t n, int64_t s1) {
  int64_t rows = 0;
  for (int64_t t = 0; t < s1 && t + kQSuper < n; t += kQSuper) rows += n - t - kQSuper;
  return rows;
}

QuantPlan plan_quantize(int64_t m, int64_t n, const gptq_config& cfg) {
  QuantPlan p;
  p.m = m;
  p.n = n;
  p.ldw = round_up(std::max<int64_t>(n, 1), QB);
  p.groups = gptq_num_groups(n, cfg.group_size);
  p.words = gptq_qweight_words(n, cfg.bits);
  size_t off = 0;
  p.wp_off = off; off += align256((size_t)m * p.ldw * sizeof(float));
  p.part_off = off;  // pack partials: one double per row
  off += align256((size_t)m * sizeof(double));
  p.codes_off = off; off += align256((size_t)m * p.ldw);
  p.loss_off = off; off += align256((size_t)m * sizeof(double));
  p.inv_off = off; off += align256((size_t)round_up(n, int64_t(8)) * sizeof(int32_t));   // padded to 8
  p.flag_off = off; off += 256;
  // bf16 planes of the superblock errors (double-buffered by superblock
  // parity) and of U[s1:s2, s2:] for every superblock with a trailing update,
  // back to back (superblock s: n - s2 plane rows)
  p.x6a_off = off; off += align256((size_t)2 * 3 * m * kX6K * sizeof(uint16_t));
  p.x6b_off = off; off += align256((size_t)3 * kX6K * sizeof(uint16_t) * (size_t)uplane_rows(n, n));
  p.total = off;
  return p;
}

gptq_status run_quantize(const void* W, int w_dtype, int64_t m, int64_t n, const float* U,
                         const int32_t* perm, const gptq_config& cfg, uint32_t* qweight,
                         float* scales, int32_t* zeros, int32_t* g_idx, double* loss,
                         int32_t* status, void* ws, const QuantPlan& p, hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  float* Wp = reinterpret_cast<float*>(w + p.wp_off);
  double* part = reinterpret_cast<double*>(w + p.part_off);
  uint8_t* codes = reinterpret_cast<uint8_t*>(w + p.codes_off);
  double* loss_rows = reinterpret_cast<double*>(w + p.loss_off);
  int32_t* invperm = reinterpret_cast<int32_t*>(w + p.inv_off);
  int* flag = reinterpret_cast<int*>(w + p.flag_off);

  hipLaunchKernelGGL(zero_f64_kernel, dim3((unsigned)std::min<int64_t>(ceil_div(m, 256), 1024)),
                     dim3(256), 0, stream, loss_rows, m, flag);
  GPTQ_LAUNCH_CHECK();

  const size_t row_bytes = (size_t)n * sizeof(float);
  auto qprep = [&](auto kern, const auto* Wt) -> gptq_status {
    if (row_bytes > 65536)
      GPTQ_HIP_CHECK(hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)row_bytes));
    hipLaunchKernelGGL(kern, dim3((unsigned)m), dim3(256), row_bytes, stream, Wt, n, perm, Wp, p.ldw, flag);
    return GPTQ_OK;
  };
  const bool w16 = (reinterpret_cast<uintptr_t>(W) & 15) == 0;
  if (w_dtype == GPTQ_BF16) {
    const uint16_t* Wb = static_cast<const uint16_t*>(W);
    if (w16 && n % 8 == 0) GPTQ_TRY(qprep(qprep_kernel<uint16_t, true>, Wb));
    else GPTQ_TRY(qprep(qprep_kernel<uint16_t, false>, Wb));
  } else {
    const float* Wf = static_cast<const float*>(W);
    if (w16 && n % 4 == 0) GPTQ_TRY(qprep(qprep_kernel<float, true>, Wf));
    else GPTQ_TRY(qprep(qprep_kernel<float, false>, Wf));
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
  a.eplane = nullptr; a.epstride = m * kX6K; a.esst = m * kX6Step; a.codes = codes; a.loss_rows = loss_rows;

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
  SideStream usplit;
  GPTQ_TRY(get_side_stream(usplit, 2));
  SideJoin join(stream);
  join.add(side);
  join.add(usplit);
  bool side_pending = false;
  // U is fixed for the whole call: the planes of U[s1:s2, s2:] for every
  // superblock after the first are split up front on side stream 2, beside
  // the first superblock's blocks; the first superblock's own split stays on
  // this stream, and the second's update waits for the rest once
  uint16_t* const ub = reinterpret_cast<uint16_t*>(w + p.x6b_off);
  auto uplanes = [&](int64_t s1) {
    const int64_t s2 = s1 + kQSuper, rows = n - s2;
    return X6Planes{ub + 3 * kX6K * uplane_rows(n, s1), rows, kX6K, rows * kX6K, rows * kX6Step};
  };
  auto split_u = [&](int64_t s1, hipStream_t st) -> gptq_status {
    const X6Planes P = uplanes(s1);
    const int64_t s2 = s1 + kQSuper;
    return launch_x6_split_cols(U + s1 * n + s2, n, kQSuper, n - s2, kX6K, const_cast<uint16_t*>(P.p), P.pstride,
                                P.sst, st);
  };
  bool usplit_pending = false;
  if (kQSuper < n) {
    GPTQ_TRY(split_u(0, stream));
    if (2 * kQSuper < n) {
      GPTQ_HIP_CHECK(hipEventRecord(usplit.ready, stream));
      GPTQ_HIP_CHECK(hipStreamWaitEvent(usplit.stream, usplit.ready, 0));
      for (int64_t s1 = kQSuper; s1 + kQSuper < n; s1 += kQSuper) GPTQ_TRY(split_u(s1, usplit.stream));
      GPTQ_HIP_CHECK(hipEventRecord(usplit.done, usplit.stream));
      usplit_pending = true;
    }
  }
  for (int64_t s1 = 0; s1 < n; s1 += kQSuper) {
    const int64_t s2 = std::min<int64_t>(s1 + kQSuper, n);
    // the superblock's errors go straight into its x6 planes (double-buffered
    // by parity: the far update of superblock s reads them while the blocks
    // of s + 1 write the other buffer, and s + 2 starts after that update)
    const int par = (int)((s1 / kQSuper) & 1);
    uint16_t* pa = reinterpret_cast<uint16_t*>(w + p.x6a_off) + (size_t)par * 3 * m * kX6K;
    for (int64_t i1 = s1; i1 < s2; i1 += QB) {
      const int bw = (int)std::min<int64_t>(QB, s2 - i1);
      // the quantizer reads only rows and columns < bw of U's diagonal block
      const float* ublk = U + i1 * n + i1;
      const int64_t ldub = n;
      a.eplane = pa + ((i1 - s1) / kX6Step) * a.esst;
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
      const X6Planes PU = uplanes(s1);
      if (usplit_pending && s1 > 0) {   // superblock 0's planes were split on this stream
        GPTQ_HIP_CHECK(hipStreamWaitEvent(stream, usplit.done, 0));
        usplit_pending = false;
      }
      const X6Planes PA{pa, m, kX6K, m * kX6K, m * kX6Step};
      if (side_pending) GPTQ_HIP_CHECK(hipStreamWaitEvent(stream, side.done, 0));
      side_pending = false;
      if (far > 0) {
        GPTQ_HIP_CHECK(hipEventRecord(side.ready, stream));
        GPTQ_HIP_CHECK(hipStreamWaitEvent(side.stream, side.ready, 0));
        const X6Planes PF{PU.p + near * kX6Step, far, kX6K, PU.pstride, PU.sst};
        // a small far update leaves CU room for the next superblock's blocks;
        // a large one is the stage's bottleneck and takes the whole chip
        const bool polite = far < kQPoliteFar;
        GPTQ_TRY(launch_x6_gemm(PA, PF, Wp + s2 + near, p.ldw, m, far, -1.f, 1.f, false, side.stream, polite));
        GPTQ_HIP_CHECK(hipEventRecord(side.done, side.stream));
        side_pending = true;
      }
      const X6Planes PN{PU.p, near, kX6K, PU.pstride, PU.sst};
      // on the chain: with fewer 128-row tiles than CUs, 64-row tiles
      const int near_rows = ceil_div(m, 128) * ceil_div(near, 128) < 256 ? 64 : 128;
      GPTQ_TRY(launch_x6_gemm(PA, PN, Wp + s2, p.ldw, m, near, -1.f, 1.f, false, stream, false, near_rows));
    }
  }
  if (side_pending) GPTQ_HIP_CHECK(hipStreamWaitEvent(stream, side.done, 0));
  if (usplit_pending) GPTQ_HIP_CHECK(hipStreamWaitEvent(stream, usplit.done, 0));
  join.release();

  hipLaunchKernelGGL(gidx_kernel, dim3((unsigned)ceil_div(round_up(n, int64_t(8)), 256)), dim3(256), 0, stream, perm, n,
                     (int64_t)(gw > 0 ? gw : 0), g_idx, invperm);
  GPTQ_LAUNCH_CHECK();
  // one workgroup per row; its codes and group parameters staged in LDS
  const unsigned pgrid = (unsigned)m;
  const size_t pack_lds = (size_t)p.ldw + 8 * (size_t)p.groups;
  const bool bf = w_dtype == GPTQ_BF16, nib = cfg.bits <= 4;   // 8 codes per word, else 4
  const int32_t* ip = (const int32_t*)invperm;
  const float* sc = (const float*)scales;
  const int32_t* zp = (const int32_t*)zeros;
  const uint8_t* cd = (const uint8_t*)codes;
  auto pack = [&](auto kern, const auto* Wt) -> gptq_status {
    if (pack_lds > 64 * 1024)
      GPTQ_HIP_CHECK(hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)pack_lds));
    hipLaunchKernelGGL(kern, dim3(pgrid), dim3(256), pack_lds, stream, cd, p.ldw, ip, (int64_t)(gw > 0 ? gw : 0), sc, zp, p.groups, Wt, n,
                       p.words, qweight, part);
    return GPTQ_OK;
  };
  const uint16_t* Wb = static_cast<const uint16_t*>(W);
  const float* Wf = static_cast<const float*>(W);
  if (bf && nib) GPTQ_TRY(pack(pack_kernel<uint16_t, 8>, Wb));
  else if (bf) GPTQ_TRY(pack(pack_kernel<uint16_t, 4>, Wb));
  else if (nib) GPTQ_TRY(pack(pack_kernel<float, 8>, Wf));
  else GPTQ_TRY(pack(pack_kernel<float, 4>, Wf));
  GPTQ_LAUNCH_CHECK();
  hipLaunchKernelGGL(loss_reduce_kernel, dim3(1), dim3(1024), 0, stream, (const double*)loss_rows, m,
                     (const double*)part, m, loss);
  GPTQ_LAUNCH_CHECK();

  if (status) {
    hipLaunchKernelGGL(status_kernel, dim3(1), dim3(1), 0, stream, (const int*)flag, status);
    GPTQ_LAUNCH_CHECK();
  }
  return GPTQ_OK;
}

}  // namespace gptq
