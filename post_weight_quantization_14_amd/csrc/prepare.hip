// Stages 2-3: damping, act-order and the inverse factor U (UᵀU = H_p⁻¹).
//
// The page "模型量化实战：从 INT8 PTQ 到 GPTQ…" §3.2 (prepare) damps H by
// 1% of its mean diagonal, factors it, inverts it and takes the upper
// Cholesky factor of the inverse.  Here the same U is reached with half the
// work: let J be the exchange matrix and H_f = J H_p J (the permuted matrix
// read back to front).  With H_f = L Lᵀ (ordinary lower Cholesky) and
// M = L⁻¹, H_p⁻¹ = (J M J)ᵀ (J M J), and J M J is upper triangular with a
// positive diagonal, so it is the unique upper Cholesky factor of H_p⁻¹:
//     U[i][j] = M[n-1-i][n-1-j].
// Cost: n³/3 (Cholesky) + n³/3 (triangular inverse), both on fp32 MFMA.
//
// Data flow (all fp32, row-major, n_pad = n rounded up to 128):
//   stats     : λ = p · mean(diag H) in fp64, non-finite check
//   rank      : perm = stable descending order of the key (O(n²) ranks)
//   permute   : A[a][b] = H[perm[n-1-a]][perm[n-1-b]] + λ δ_ab, identity pad
//   cholesky  : per 128-column panel: leaf (factor + invert the diagonal
//               block in LDS), panel solve as a GEMM with the leaf inverse,
//               trailing update on lower tiles (all MFMA)
//   trtri     : bottom-up doubling on the leaf inverses (2 GEMMs per level)
//   flip      : U = J M J written over H, lower triangle zeroed
#include <algorithm>

#include "gptq_internal.hpp"

namespace gptq {
namespace {

constexpr int NB = kNb;

// flag bits
constexpr int kFlagNotPD = 1;
constexpr int kFlagNonFinite = 2;

__device__ __forceinline__ double key_of(const double* key, const float* H, int64_t n, int64_t j) {
  return key ? key[j] : (double)H[j * n + j];
}

// λ = damp * mean(diag); one workgroup, fixed reduction order.
__global__ __launch_bounds__(1024) void stats_kernel(const double* key, const float* H, int64_t n,
                                                     double damp, double* lam_out, int* flag) {
  __shared__ double red[1024];
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  double s = 0.0;
  int b = 0;
  for (int64_t j = threadIdx.x; j < n; j += 1024) {
    const double k = key_of(key, H, n, j);
    if (!isfinite(k)) b = 1;
    s += k;
  }
  red[threadIdx.x] = s;
  if (b) atomicOr(&bad, 1);
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double mean = red[0] / (double)n;
    *lam_out = damp * mean;
    // the first kernel of the call: it sets the flag word (later kernels OR into it)
    *flag = (bad || !isfinite(mean)) ? kFlagNonFinite : 0;
  }
}

// perm[rank(j)] = j, rank = #{i: k_i > k_j} + #{i < j: k_i == k_j}.  NaN keys
// sort as -inf, so the result is always a permutation.  Two kernels: block
// (jb, ic) counts, for the 256 columns j of block jb, the columns i of chunk
// ic that precede j (part[ic][j]); then rank(j) = Σ_ic part[ic][j], summed in
// chunk order, and perm[rank(j)] = j.  Counts are integers: the order of the
// sums cannot change them.
__device__ __forceinline__ double rank_key(const double* key, const float* H, int64_t n, int64_t j) {
  const double k = key_of(key, H, n, j);
  return isnan(k) ? -INFINITY : k;
}

__global__ __launch_bounds__(256) void rank_part_kernel(const double* key, const float* H, int64_t n,
                                                        int32_t* __restrict__ part) {
  __shared__ double ks[256];
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t i0 = (int64_t)blockIdx.y * 256;
  const int64_t li = i0 + threadIdx.x;
  ks[threadIdx.x] = li < n ? rank_key(key, H, n, li) : -INFINITY;
  __syncthreads();
  if (j >= n) return;
  const double kj = rank_key(key, H, n, j);
  const int lim = (int)std::min<int64_t>(256, n - i0);
  int cnt = 0;
  for (int t = 0; t < lim; ++t) {
    const double ki = ks[t];
    cnt += (ki > kj) || (ki == kj && i0 + t < j);
  }
  part[blockIdx.y * n + j] = cnt;
}

__global__ __launch_bounds__(256) void rank_perm_kernel(const int32_t* __restrict__ part, int64_t chunks,
                                                        int64_t n, int desc_act, int32_t* perm) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= n) return;
  if (!desc_act) {
    perm[j] = (int32_t)j;
    return;
  }
  int64_t rank = 0;
  for (int64_t c = 0; c < chunks; ++c) rank += part[c * n + j];
  perm[rank] = (int32_t)j;
}

// One output row a of A = J P (H + λI) Pᵀ J, padded with the identity.
template <bool VEC>
__global__ __launch_bounds__(256) void permute_kernel(const float* __restrict__ H, int64_t n,
                                                      const int32_t* __restrict__ perm,
                                                      const double* lam, float* __restrict__ A,
                                                      int64_t lda) {
  extern __shared__ __attribute__((aligned(16))) float row[];
  const int64_t a = blockIdx.x;
  float* out = A + a * lda;
  if (a >= n) {
    for (int64_t b = threadIdx.x; b < lda; b += 256) out[b] = (a == b) ? 1.f : 0.f;
    return;
  }
  const int64_t src = perm[n - 1 - a];
  const float* h = H + src * n;
  // loads unconditional at clamped indices, eight (row) and sixteen (gather)
  // in flight per thread: a conditional load compiles to a branch and a wait
  // of its own.  VEC (n a multiple of 4, H 16-byte aligned): 16-byte pieces.
  if constexpr (VEC) {
    const int64_t nq = n / 4;
    const f32x4_t* hq = reinterpret_cast<const f32x4_t*>(h);
    for (int64_t q0 = threadIdx.x; q0 < nq; q0 += 8 * 256) {
      f32x4_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = hq[std::min<int64_t>(q0 + 256 * u, nq - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        reinterpret_cast<f32x4_t*>(row)[std::min<int64_t>(q0 + 256 * u, nq - 1)] = v[u];
    }
  } else {
    for (int64_t b0 = threadIdx.x; b0 < n; b0 += 8 * 256) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = h[std::min<int64_t>(b0 + 256 * u, n - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u) row[std::min<int64_t>(b0 + 256 * u, n - 1)] = v[u];
    }
  }
  __syncthreads();
  const float l = (float)*lam;
  for (int64_t b0 = threadIdx.x; b0 < lda; b0 += 16 * 256) {
    int32_t pi[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) pi[u] = perm[n - 1 - std::min<int64_t>(b0 + 256 * u, n - 1)];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int64_t b = b0 + 256 * u;
      if (b >= lda) break;
      float v = 0.f;
      if (b < n) {
        v = row[pi[u]];
        if (b == a) v += l;
      }
      out[b] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Leaf: Cholesky of the 128 x 128 diagonal block at (k0, k0), then its inverse.
// The block is cut into 8 x 8 sub-blocks of 16 x 16; threads 16t .. 16t+15
// (t < 36) serve the t-th lower sub-block (bi, bj), thread 16t + r holding its
// row r (Cholesky) or column r (inverse) in registers.  The 16 threads of a
// sub-block are one 16-lane row of a wave.  Both phases run 8 block steps with
// operands through LDS (row pitch 20 floats: 16-byte aligned rows, and the 16
// rows of a sub-block on distinct bank quads):
//   Cholesky, step jb: the lanes of (jb, jb) factor it column by column,
//     broadcasting within their row by DPP row_newbcast (pivots through
//     v_rsq_f32; the solves multiply by the kept 1/L[c][c]); owners of (bi, jb)
//     solve X · L_jbᵀ = A_bi,jb along their row; owners of (bi, bj),
//     jb < bj <= bi, subtract L_bi,jb · L_bj,jbᵀ.
//   Inverse by doubling: the owners of the eight diagonal sub-blocks invert
//     them at once (forward substitution down their column); then three
//     levels join neighbouring lower-triangular blocks of 1, 2 and 4
//     sub-blocks, [M11 0; M21 M22] with M21 = -M22 · (L21 · M11), as
//     v_mfma_f32_16x16x4f32 products of 16 x 16 sub-blocks spread over the
//     nine waves (two barriers per level instead of two per 16-row step).
// Writes L back into A (lower triangle of the block) and D = L⁻¹ into the same
// block of Mmat (strict upper part of that block set to 0).
// ---------------------------------------------------------------------------
constexpr int LE = 16;                  // sub-block edge
constexpr int LN = NB / LE;             // sub-blocks per side
constexpr int LT = LN * (LN + 1) / 2;   // lower sub-blocks
constexpr int LP = 20;                  // LDS row pitch (floats)
constexpr int LSZ = LE * LP;            // floats per stored sub-block
constexpr int kLeafThreads = LT * LE;   // 576

__device__ __forceinline__ void sub_decode(int t, int& bi, int& bj) {
  int r = 0;
  while ((r + 1) * (r + 2) / 2 <= t) ++r;
  bi = r;
  bj = t - r * (r + 1) / 2;
}
__device__ __forceinline__ int lblk(int bi, int bj) { return (bi * (bi + 1) / 2 + bj) * LSZ; }

// value of lane K of this lane's 16-lane row
template <int K>
__device__ __forceinline__ float row_bcast16(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + K, 0xf, 0xf, false));
}

template <int J>
__device__ __forceinline__ void diag_update(float (&a)[LE], float lc) {
  if constexpr (J < LE) {
    a[J] -= lc * row_bcast16<J>(lc);   // a[r][J] -= L[r][C] · L[J][C]
    diag_update<J + 1>(a, lc);
  }
}

// Column C of the 16 x 16 diagonal Cholesky; lane r holds row r.  The pivot's
// reciprocal square root (v_rsq_f32, within 1 ulp) scales the column, and lane
// C keeps it as 1/L[C][C] for the solves.
template <int C>
__device__ __forceinline__ void diag_factor(float (&a)[LE], int r, bool& bad, float& dinv) {
  if constexpr (C < LE) {
    float d = row_bcast16<C>(a[C]);
    if (!(d > 0.f) || !isfinite(d)) {
      bad = true;
      d = 1.f;
    }
    const float rs = __builtin_amdgcn_rsqf(d);
    const float lc = (r > C) ? a[C] * rs : (r == C ? d * rs : 0.f);
    if (r == C) dinv = rs;
    a[C] = lc;
    diag_update<C + 1>(a, lc);
    diag_factor<C + 1>(a, r, bad, dinv);
  }
}

// pre != 0: the block first takes the trailing update from the panel just
// before it, A_kk -= P·Pᵀ with P = A[k0:k0+128, k0-128:k0] (that panel's
// solved rows for this block), by v_mfma_f32_16x16x4f32: wave w computes the
// 16 x 16 sub-blocks 4w .. 4w+3 and parks them in Ls, where their owners pick
// them up.  P is staged in LDS 32 columns at a time (row pitch 36: the
// operand reads of a wave hit 64 distinct banks), which keeps the kernel's LDS
// small enough to share a CU with a trailing-update GEMM workgroup.
constexpr int kPk = 32;          // columns of P per staged pass
constexpr int kPp = kPk + 4;     // row pitch of the staged pass
// Ps holds a pass of P, or the 16 sub-blocks of T at the last inverse level
constexpr int kPsFloats = (NB * kPp > 16 * LSZ) ? NB * kPp : 16 * LSZ;

// C += A · B for 16 x 16 sub-blocks stored row-major in LDS (pitch LP), by
// four v_mfma_f32_16x16x4f32: lane l supplies A[l % 16][4kk + l / 16] and
// B[4kk + l / 16][l % 16]; C[4 (l / 16) + v][l % 16] is element v of the result.
__device__ __forceinline__ f32x4_t sub_mma(const float* A, const float* B, f32x4_t c, int lane) {
  const float* pa = A + (lane & 15) * LP + (lane >> 4);
  const float* pb = B + (lane >> 4) * LP + (lane & 15);
#pragma unroll
  for (int kk = 0; kk < LE / 4; ++kk) c = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[4 * kk], pb[4 * kk * LP], c, 0, 0, 0);
  return c;
}
__device__ __forceinline__ void sub_store(float* dst, f32x4_t c, float sign, int lane) {
  float* p = dst + 4 * (lane >> 4) * LP + (lane & 15);
#pragma unroll
  for (int v = 0; v < 4; ++v) p[v * LP] = sign * c[v];
}

__global__ __launch_bounds__(kLeafThreads) void chol_leaf_kernel(float* A, float* Mm, int64_t lda,
                                                                 int64_t k0, int pre, int* flag) {
  __shared__ __attribute__((aligned(16))) float Ls[LT * LSZ];   // L by lower sub-block
  __shared__ __attribute__((aligned(16))) float Ms[LN * LSZ];   // M row block of the step
  __shared__ float Ldi[NB];                                     // 1 / L[c][c]
  // one pass of P (pre-update), later T = L21 · M11 of one inverse level
  __shared__ __attribute__((aligned(16))) float Ps[kPsFloats];
  const int tid = threadIdx.x;
  const int t = tid >> 4, r = tid & (LE - 1);
  int bi, bj;
  sub_decode(t, bi, bj);
  float* Ab = A + k0 * lda + k0;
  float* Mb = Mm + k0 * lda + k0;

  // P for all passes is loaded up front with the block itself (one memory
  // latency): thread tid holds float4 number tid and tid + 576 of each pass
  // (a pass is 128 rows x 8 float4).
  constexpr int kPq = NB * kPk / 4;   // float4 per pass
  f32x4_t pv[NB / kPk][2];
  if (pre) {
    const float* P = Ab - NB;
#pragma unroll
    for (int ps = 0; ps < NB / kPk; ++ps)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int idx = tid + kLeafThreads * u;
        if (idx < kPq)
          pv[ps][u] = *reinterpret_cast<const f32x4_t*>(P + (int64_t)(idx >> 3) * lda + ps * kPk +
                                                        4 * (idx & 7));
      }
  }

  float a[LE];
#pragma unroll
  for (int c = 0; c < LE; ++c) a[c] = Ab[(int64_t)(LE * bi + r) * lda + LE * bj + c];

  if (pre) {
    const int lane = tid & 63, wave = tid >> 6;
    f32x4_t d[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) d[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ps = 0; ps < NB / kPk; ++ps) {
      if (ps > 0) __syncthreads();   // the previous pass is consumed
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int idx = tid + kLeafThreads * u;
        if (idx < kPq) *reinterpret_cast<f32x4_t*>(Ps + (idx >> 3) * kPp + 4 * (idx & 7)) = pv[ps][u];
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        int ci, cj;
        sub_decode(4 * wave + q, ci, cj);
        // A = P rows of sub-block row ci, B = Pᵀ columns of sub-block column
        // cj: lane l supplies P[16 ci + l % 16][4 kk + l / 16], same for cj
        const float* pa = Ps + (LE * ci + (lane & 15)) * kPp + (lane >> 4);
        const float* pb = Ps + (LE * cj + (lane & 15)) * kPp + (lane >> 4);
#pragma unroll
        for (int kk = 0; kk < kPk / 4; ++kk)
          d[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[4 * kk], pb[4 * kk], d[q], 0, 0, 0);
      }
    }
    // D[4 (l / 16) + v][l % 16]
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int ci, cj;
      sub_decode(4 * wave + q, ci, cj);
      float* dst = Ls + lblk(ci, cj) + (4 * (lane >> 4)) * LP + (lane & 15);
#pragma unroll
      for (int v = 0; v < 4; ++v) dst[v * LP] = d[q][v];
    }
    __syncthreads();
    const float* src = Ls + lblk(bi, bj) + r * LP;
#pragma unroll
    for (int c = 0; c < LE; ++c) a[c] -= src[c];
    // Ls(0, 0) is rewritten below only by the lanes that read it, in order;
    // every other sub-block is rewritten after the step's first barrier
  }

  // ---- Cholesky by 16-column block steps; thread = row r of (bi, bj)
  bool bad = false;
#pragma unroll 1
  for (int jb = 0; jb < LN; ++jb) {
    if (bi == jb && bj == jb) {
      float dinv = 1.f;
      diag_factor<0>(a, r, bad, dinv);
      Ldi[LE * jb + r] = dinv;
      float* dst = Ls + lblk(jb, jb) + r * LP;
#pragma unroll
      for (int c = 0; c < LE; ++c) {
        if (c > r) a[c] = 0.f;
        dst[c] = a[c];
      }
    }
    __syncthreads();
    if (bj == jb && bi > jb) {
      // X · Lᵀ = A along the row: x[c] = (a[c] - Σ_{k<c} x[k] L[c][k]) / L[c][c]
      const float* L = Ls + lblk(jb, jb);
#pragma unroll
      for (int c = 0; c < LE; ++c) {
        float v = a[c];
#pragma unroll
        for (int k = 0; k < c; ++k) v -= a[k] * L[c * LP + k];
        a[c] = v * Ldi[LE * jb + c];
      }
      float* dst = Ls + lblk(bi, jb) + r * LP;
#pragma unroll
      for (int c = 0; c < LE; ++c) dst[c] = a[c];
    }
    __syncthreads();
    if (bj > jb && bi >= bj) {
      const float* X = Ls + lblk(bi, jb) + r * LP;
      const float* Y = Ls + lblk(bj, jb);
      float x[LE];
#pragma unroll
      for (int k = 0; k < LE; ++k) x[k] = X[k];
#pragma unroll
      for (int c = 0; c < LE; ++c) {
        float acc = a[c];
#pragma unroll
        for (int k = 0; k < LE; ++k) acc -= x[k] * Y[c * LP + k];
        a[c] = acc;
      }
    }
    // the next step's diagonal factor uses only its own registers, and its
    // writes go to a sub-block no thread reads in this step
  }
  if (bad) atomicOr(flag, kFlagNotPD);

  // ---- L to A (lower triangle of the block)
#pragma unroll
  for (int c = 0; c < LE; ++c)
    if (bi != bj || c <= r) Ab[(int64_t)(LE * bi + r) * lda + LE * bj + c] = a[c];

  // ---- D = L⁻¹.  Diagonal sub-blocks of D go to Ms, an off-diagonal one
  // replaces the sub-block of L at its place in Ls: every L sub-block below
  // the diagonal belongs to exactly one join and is last read by that join's
  // first product, before the barrier after which its D block is written.
  // (The Cholesky's last reads of Ls ended at its final barrier.)
  auto dblk = [&](int i, int j) -> float* { return i == j ? Ms + i * LSZ : Ls + lblk(i, j); };
  if (bi == bj) {
    // column r of L_ii⁻¹: m[i] = (δ_ir - Σ_{k<i} L[i][k] m[k]) / L[i][i]
    const float* L = Ls + lblk(bi, bi);
    float m[LE];
#pragma unroll
    for (int i = 0; i < LE; ++i) {
      float v = (i == r) ? 1.f : 0.f;
#pragma unroll
      for (int k = 0; k < i; ++k) v -= L[i * LP + k] * m[k];
      m[i] = v * Ldi[LE * bi + i];
    }
    float* dst = Ms + bi * LSZ + r;
#pragma unroll
    for (int i = 0; i < LE; ++i) dst[i * LP] = m[i];
  }
  __syncthreads();
  {
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    constexpr int kWaves = kLeafThreads / 64;
    const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int h = 1; h < LN; h *= 2) {   // join pairs of lower-triangular blocks of h sub-blocks
      const int jobs = (LN / (2 * h)) * h * h;   // 16 x 16 outputs per product phase
      // T(i, j) = Σ_{k=j}^{h-1} L21(i, k) · M11(k, j)
#pragma unroll 1
      for (int job = wave; job < jobs; job += kWaves) {
        const int q = job / (h * h), i = (job / h) % h, j = job % h;
        const int c1 = 2 * q * h, r2 = c1 + h;
        f32x4_t c = zero;
#pragma unroll 1
        for (int k = j; k < h; ++k) c = sub_mma(Ls + lblk(r2 + i, c1 + k), dblk(c1 + k, c1 + j), c, lane);
        sub_store(Ps + job * LSZ, c, 1.f, lane);
      }
      __syncthreads();
      // M21(i, j) = -Σ_{k=0}^{i} M22(i, k) · T(k, j), written over L21(i, j)
#pragma unroll 1
      for (int job = wave; job < jobs; job += kWaves) {
        const int q = job / (h * h), i = (job / h) % h, j = job % h;
        const int c1 = 2 * q * h, r2 = c1 + h;
        f32x4_t c = zero;
#pragma unroll 1
        for (int k = 0; k <= i; ++k) c = sub_mma(dblk(r2 + i, r2 + k), Ps + (q * h * h + k * h + j) * LSZ, c, lane);
        sub_store(Ls + lblk(r2 + i, c1 + j), c, -1.f, lane);
      }
      __syncthreads();
    }
  }

  // ---- D to Mmat: thread r of (bi, bj) writes column r; owners of (bi, bj),
  // bi > bj, also zero (bj, bi)
  {
    const float* src = dblk(bi, bj) + r;
#pragma unroll
    for (int i = 0; i < LE; ++i) Mb[(int64_t)(LE * bi + i) * lda + LE * bj + r] = src[i * LP];
  }
  if (bi > bj) {
#pragma unroll
    for (int i = 0; i < LE; ++i) Mb[(int64_t)(LE * bj + i) * lda + LE * bi + r] = 0.f;
  }
}

// U[a][b] = M[n-1-a][n-1-b] for a <= b, 0 below the diagonal.  Four
// consecutive b per thread: with vec (n % 4 == 0 and 16-byte aligned U and M;
// M's rows are padded to 128) one 16-byte load of M's row n-1-a read back to
// front and one 16-byte store; a piece wholly below the diagonal stores
// zeros without reading M.
__global__ __launch_bounds__(256) void flip_kernel(const float* __restrict__ Mm, int64_t lda,
                                                   int64_t n, float* __restrict__ U, int vec) {
  const int64_t a = blockIdx.y;
  const int64_t b0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (b0 >= n) return;
  const float* mrow = Mm + (n - 1 - a) * lda;
  if (vec) {
    f32x4_t out = {0.f, 0.f, 0.f, 0.f};
    if (b0 + 3 >= a) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(mrow + (n - 4 - b0));
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = (b0 + e >= a) ? v[3 - e] : 0.f;
    }
    *reinterpret_cast<f32x4_t*>(U + a * n + b0) = out;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t b = b0 + e;
      if (b < n) U[a * n + b] = (a <= b) ? mrow[n - 1 - b] : 0.f;
    }
  }
}

}  // namespace

// Triangular-inverse nodes whose halves span at least this many 128-blocks
// run on bf16 MFMA from exact three-plane splits of their operands (the
// fp32-accurate product of the trailing updates); the joins of single and
// paired blocks stay on fp32 MFMA (one launch each instead of three).
constexpr int64_t kTriX6Half = 4;

// Bytes of the planes of one such node: step 1 splits M11ᵀ (h x h blocks) and
// L21 (r x h), step 2 M22 (r x r) and Tᵀ (h x r), with r <= h.
size_t tri_x6_bytes(int64_t h, int64_t r) {
  const int64_t H = h * NB, R = r * NB;
  return align256((size_t)3 * H * H * sizeof(uint16_t)) + align256((size_t)3 * R * H * sizeof(uint16_t));
}

PreparePlan plan_prepare(int64_t n) {
  PreparePlan p;
  p.n = n;
  p.n_pad = round_up(std::max<int64_t>(n, 1), NB);
  p.nblk = p.n_pad / NB;
  const size_t mat = align256((size_t)p.n_pad * p.n_pad * sizeof(float));
  p.a_off = 0;
  p.m_off = mat;
  p.lam_off = 2 * mat;
  p.flag_off = p.lam_off + 256;
  // bf16 planes of an outer block's panel rows for its trailing update,
  // double-buffered (the far part of one block runs beside the next block)
  p.x6_off = p.flag_off + 256;
  p.tx6_off = p.x6_off + align256((size_t)2 * 3 * p.n_pad * kX6K * sizeof(uint16_t));
  // planes of the largest triangular-inverse node on the bf16 path (the
  // nodes run one after another on one stream and reuse them)
  size_t tx6 = 0;
  for (int64_t half = kTriX6Half; half < p.nblk; half *= 2)
    for (int64_t r0 = half; r0 < p.nblk; r0 += 2 * half)
      tx6 = std::max(tx6, tri_x6_bytes(half, std::min<int64_t>(r0 + half, p.nblk) - r0));
  p.total = p.tx6_off + tx6;
  return p;
}

gptq_status run_prepare(float* H, const double* key, int64_t n, double damp, int desc_act,
                        int32_t* perm, void* ws, const PreparePlan& p, double* damp_out,
                        hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  float* A = reinterpret_cast<float*>(w + p.a_off);
  float* Mm = reinterpret_cast<float*>(w + p.m_off);
  double* lam = reinterpret_cast<double*>(w + p.lam_off);
  int* flag = reinterpret_cast<int*>(w + p.flag_off);
  const int64_t lda = p.n_pad;

  hipLaunchKernelGGL(stats_kernel, dim3(1), dim3(1024), 0, stream, key, (const float*)H, n, damp,
                     lam, flag);
  GPTQ_LAUNCH_CHECK();
  // the ranks' partial counts borrow M, which the factorisation writes later
  const int64_t chunks = ceil_div(n, 256);
  if (desc_act) {
    hipLaunchKernelGGL(rank_part_kernel, dim3((unsigned)chunks, (unsigned)chunks), dim3(256), 0, stream, key,
                       (const float*)H, n, reinterpret_cast<int32_t*>(Mm));
    GPTQ_LAUNCH_CHECK();
  }
  hipLaunchKernelGGL(rank_perm_kernel, dim3((unsigned)chunks), dim3(256), 0, stream,
                     (const int32_t*)reinterpret_cast<int32_t*>(Mm), chunks, n, desc_act, perm);
  GPTQ_LAUNCH_CHECK();
  const size_t row_bytes = (size_t)n * sizeof(float);
  const bool vec = n % 4 == 0 && (reinterpret_cast<uintptr_t>(H) & 15) == 0;
  const void* pk = vec ? (const void*)permute_kernel<true> : (const void*)permute_kernel<false>;
  if (row_bytes > 65536)
    GPTQ_HIP_CHECK(hipFuncSetAttribute(pk, hipFuncAttributeMaxDynamicSharedMemorySize, (int)row_bytes));
  if (vec)
    hipLaunchKernelGGL(permute_kernel<true>, dim3((unsigned)p.n_pad), dim3(256), row_bytes, stream,
                       (const float*)H, n, (const int32_t*)perm, (const double*)lam, A, lda);
  else
    hipLaunchKernelGGL(permute_kernel<false>, dim3((unsigned)p.n_pad), dim3(256), row_bytes, stream,
                       (const float*)H, n, (const int32_t*)perm, (const double*)lam, A, lda);
  GPTQ_LAUNCH_CHECK();

  // Blocked right-looking Cholesky of A (lower), leaf inverses into Mm, with
  // two levels of trailing update (exact: the same products, grouped).  A
  // 128-panel updates only the rest of its 512-column outer block (all rows
  // below, K = 128); the columns after the outer block are updated once per
  // outer block from its four panels (K = 512), so the trailing matrix is read
  // and written a quarter as often.
  constexpr int64_t OB = 4 * NB;
  static_assert(OB <= kX6K, "an outer block's panel must fit the plane width");
  // far outer updates of fewer columns run one workgroup per CU (measured
  // crossover between the leaf chain and the far GEMM as the bottleneck)
  constexpr int64_t kPolitePrepFar = 11000;
  SideStream side, tri, inr;
  GPTQ_TRY(get_side_stream(side, 0));
  GPTQ_TRY(get_side_stream(tri, 1));
  GPTQ_TRY(get_side_stream(inr, 2));
  SideJoin join(stream);
  join.add(side);
  join.add(tri);
  join.add(inr);
  bool side_pending = false, tri_pending = false, inr_pending = false;
  // Triangular inverse, overlapped with the factorisation.  A node of the
  // bottom-up doubling joins blocks [l0, r0) and [r0, r1): its step 1
  // (T = L21·M11) needs L rows [r0, r1) of columns [l0, r0), final once panel
  // r0 - 1 is solved, and M11 (the child node, issued before it); its step 2
  // (M21 = -M22·T) also needs M22, complete once panel r1 - 1 is.  Steps run in
  // that order on their own stream (smaller levels first, so children precede
  // parents).  Their writes (T parked in A's strict upper block triangle, M's
  // off-diagonal blocks) touch nothing the factorisation still uses.
  // `solved` is recorded on the caller's stream once panel kb is solved.
  // A large node as two x6 products from planes split on the same stream:
  //   step 1: Tᵀ = M11ᵀ · L21ᵀ; row j of M11ᵀ (column j of M11) is zero before
  //           position j, so a tile of rows from j0 on starts at k = j0;
  //   step 2: M21 = -M22 · (Tᵀ)ᵀ; row i of M22 ends at position i.
  // The planes of a node are dead once its product has run, so every node
  // reuses the same region.
  uint16_t* const tx6 = reinterpret_cast<uint16_t*>(w + p.tx6_off);
  auto trtri_x6 = [&](int64_t half, int64_t q, int step) -> gptq_status {
    const int64_t l0 = q * 2 * half, r0 = l0 + half, r1 = std::min<int64_t>(r0 + half, p.nblk);
    const int64_t H = half * NB, R = (r1 - r0) * NB;
    float* const Tt = A + l0 * NB * lda + r0 * NB;   // Tᵀ, H x R, in A's strict upper block triangle
    if (step == 1) {
      uint16_t* const pb = tx6 + align256((size_t)3 * H * H * sizeof(uint16_t)) / sizeof(uint16_t);
      GPTQ_TRY(launch_x6_split_cols(Mm + l0 * NB * lda + l0 * NB, lda, H, H, H, tx6, H * H, H * kX6Step,
                                    tri.stream, /*lower=*/true));
      GPTQ_TRY(launch_x6_split_rows(A + r0 * NB * lda + l0 * NB, lda, R, H, H, pb, R * H, R * kX6Step,
                                    tri.stream));
      const X6Planes PA{tx6, H, H, H * H, H * kX6Step}, PB{pb, R, H, R * H, R * kX6Step};
      return launch_x6_gemm(PA, PB, Tt, lda, H, R, 1.f, 0.f, false, tri.stream, false, NB, kX6FromRow);
    }
    uint16_t* const pb = tx6 + align256((size_t)3 * R * R * sizeof(uint16_t)) / sizeof(uint16_t);
    GPTQ_TRY(launch_x6_split_rows(Mm + r0 * NB * lda + r0 * NB, lda, R, R, R, tx6, R * R, R * kX6Step,
                                  tri.stream, /*lower=*/true));
    GPTQ_TRY(launch_x6_split_rows(Tt, lda, H, R, R, pb, H * R, H * kX6Step, tri.stream));
    const X6Planes PA{tx6, R, R, R * R, R * kX6Step}, PB{pb, H, R, H * R, H * kX6Step};
    return launch_x6_gemm(PA, PB, Mm + r0 * NB * lda + l0 * NB, lda, R, H, -1.f, 0.f, false, tri.stream, false,
                          NB, kX6ToRow);
  };
  auto issue_trtri = [&](int64_t kb, hipEvent_t solved) -> gptq_status {
    bool waited = false;
    for (int64_t half = 1; half < p.nblk; half *= 2) {
      for (int64_t q = 0; q * 2 * half + half < p.nblk; ++q) {
        const int64_t r0 = q * 2 * half + half;
        const int64_t r1 = std::min<int64_t>(r0 + half, p.nblk);
        for (int step = 1; step <= 2; ++step) {
          if ((step == 1 ? r0 : r1) != kb + 1) continue;
          if (!waited) {
            GPTQ_HIP_CHECK(hipStreamWaitEvent(tri.stream, solved, 0));
            waited = true;
          }
          if (half >= kTriX6Half) {
            GPTQ_TRY(trtri_x6(half, q, step));
          } else {
            GPTQ_TRY(launch_trtri_nodes(A, Mm, lda, p.nblk, half, q, 1, step, tri.stream));
          }
          tri_pending = true;
        }
      }
    }
    return GPTQ_OK;
  };
  // Inside an outer block, panel k's update of the block's later columns is
  // split three ways: the next panel's 128 x 128 diagonal block is updated by
  // the next leaf itself, which follows the panel solve at once; the rest of
  // the next panel's columns ("rect") and the block's columns after it
  // ("lower") run on the inner side stream beside that leaf.  The next panel
  // solve waits for both (rect rewrites its rows; lower covers the diagonal
  // block of panel k + 2, whose leaf comes after that solve on this stream),
  // one event for the two.  Concurrent kernels always touch disjoint parts of A.
  for (int64_t K0 = 0; K0 < p.n_pad; K0 += OB) {
    const int64_t K1 = std::min<int64_t>(K0 + OB, p.n_pad);
    // the panel rows L[K1:, K0:K1] as exact bf16 planes for the outer update,
    // written by the panel solves (double-buffered by block parity: the far
    // update of the previous block reads the other buffer, and the one of the
    // block before that was awaited before that previous far update began)
    const int par = (int)((K0 / OB) & 1);
    uint16_t* const pl = reinterpret_cast<uint16_t*>(w + p.x6_off) + (size_t)par * 3 * p.n_pad * kX6K;
    const int64_t pst = p.n_pad * kX6K, sst = p.n_pad * kX6Step;
    for (int64_t k0 = K0; k0 < K1; k0 += NB) {
      // inside an outer block, the leaf applies the previous panel's update to
      // its own diagonal block (the rows below get it on the inner stream)
      hipLaunchKernelGGL(chol_leaf_kernel, dim3(1), dim3(kLeafThreads), 0, stream, A, Mm, lda, k0,
                         (int)(k0 > K0), flag);
      GPTQ_LAUNCH_CHECK();
      const int64_t rows = p.n_pad - k0 - NB;
      if (rows <= 0) {
        GPTQ_HIP_CHECK(hipEventRecord(inr.ready, stream));
        GPTQ_TRY(issue_trtri(k0 / NB, inr.ready));
        break;
      }
      if (inr_pending) GPTQ_HIP_CHECK(hipStreamWaitEvent(stream, inr.done, 0));
      inr_pending = false;
      // panel solve: P = A_panel · D_kᵀ  (D_kᵀ read column-major from D_k)
      GemmArgs g;
      g.A = A + (k0 + NB) * lda + k0; g.lda = lda;
      g.B = Mm + k0 * lda + k0; g.ldb = lda;
      g.C = A + (k0 + NB) * lda + k0; g.ldc = lda;
      g.M = rows; g.N = NB; g.k_begin = 0; g.k_end = NB; g.alpha = 1.f; g.beta = 0.f;
      if (K1 < p.n_pad) {   // rows K1.. of this panel also go to the outer update's planes
        g.pl = pl; g.pl_pstride = pst; g.pl_sst = sst;
        g.pl_row0 = K1 - (k0 + NB); g.pl_col0 = k0 - K0;
      }
      // on the chain: with fewer than 128 row tiles of 128, tiles of 64 rows
      GPTQ_TRY(launch_gemm_rect(g, /*b_colmajor=*/true, stream, ceil_div(rows, NB) < 128 ? 64 : NB));
      GPTQ_HIP_CHECK(hipEventRecord(inr.ready, stream));
      GPTQ_TRY(issue_trtri(k0 / NB, inr.ready));
      // inner update: A[k0+NB:, k0+NB:K1] -= P · P[k0+NB:K1]ᵀ (lower part); its
      // first 128 x 128 diagonal block is left to the next leaf.  Here: the
      // rows below that block, on the inner stream: the rest of the next
      // panel's columns, then the lower part of the outer block's columns
      // after it.
      const int64_t cols = K1 - k0 - NB;
      if (cols > 0 && rows > NB) {
        const float* P = A + (k0 + 2 * NB) * lda + k0;   // solved rows k0+2NB .. n_pad
        const float* Pc = A + (k0 + NB) * lda + k0;      // solved rows k0+NB .. K1
        GPTQ_HIP_CHECK(hipStreamWaitEvent(inr.stream, inr.ready, 0));
        GemmArgs r;
        r.A = P; r.lda = lda;
        r.B = Pc; r.ldb = lda;
        r.C = A + (k0 + 2 * NB) * lda + k0 + NB; r.ldc = lda;
        r.M = rows - NB; r.N = NB; r.k_begin = 0; r.k_end = NB; r.alpha = -1.f; r.beta = 1.f;
        GPTQ_TRY(launch_gemm_rect(r, /*b_colmajor=*/true, inr.stream, ceil_div(r.M, NB) < 128 ? 64 : NB));
        if (cols > NB) {
          r.B = P;
          r.C = A + (k0 + 2 * NB) * lda + k0 + 2 * NB;
          r.N = cols - NB;
          GPTQ_TRY(launch_gemm_lower(r, /*b_colmajor=*/true, inr.stream));
        }
        // one event for both: the next panel solve waits for it, and the leaf
        // of panel k + 2 (which needs lower) follows that solve here
        GPTQ_HIP_CHECK(hipEventRecord(inr.done, inr.stream));
        inr_pending = true;
      }
    }
    // outer update: A[K1:, K1:] -= L[K1:, K0:K1] · L[K1:, K0:K1]ᵀ (lower part),
    // split with lookahead: the next outer block's columns [K1, K1+OB) on the
    // caller's stream, the columns after them on the side stream, where they
    // run while the next outer block's leaf chain (which touches only its own
    // columns) runs here.  The near part writes columns the previous far part
    // wrote, so it waits for that first.
    const int64_t rest = p.n_pad - K1;
    if (rest > 0) {
      const int64_t near = std::min<int64_t>(OB, rest), far = rest - near;
      // the panel rows L[K1:, K0:K1] (A and B operand alike) are in the
      // planes: the block's panel solves wrote them
      if (side_pending) GPTQ_HIP_CHECK(hipStreamWaitEvent(stream, side.done, 0));
      side_pending = false;
      if (far > 0) {
        GPTQ_HIP_CHECK(hipEventRecord(side.ready, stream));
        GPTQ_HIP_CHECK(hipStreamWaitEvent(side.stream, side.ready, 0));
        const X6Planes PF{pl + near * kX6Step, far, kX6K, pst, sst};
        // a small far update leaves CU room for the next outer block's
        // leaves; a large one is the bottleneck and takes the whole chip
        const bool polite = far < kPolitePrepFar;
        GPTQ_TRY(launch_x6_gemm(PF, PF, A + (K1 + near) * lda + K1 + near, lda, far, far, -1.f, 1.f, true,
                                side.stream, polite));
        GPTQ_HIP_CHECK(hipEventRecord(side.done, side.stream));
        side_pending = true;
      }
      const X6Planes PR{pl, rest, kX6K, pst, sst}, PN{pl, near, kX6K, pst, sst};
      GPTQ_TRY(launch_x6_gemm(PR, PN, A + K1 * lda + K1, lda, rest, near, -1.f, 1.f, true, stream));
    }
  }
  if (side_pending) GPTQ_HIP_CHECK(hipStreamWaitEvent(stream, side.done, 0));
  if (inr_pending) GPTQ_HIP_CHECK(hipStreamWaitEvent(stream, inr.done, 0));
  if (tri_pending) {
    GPTQ_HIP_CHECK(hipEventRecord(tri.done, tri.stream));
    GPTQ_HIP_CHECK(hipStreamWaitEvent(stream, tri.done, 0));
  }
  join.release();
  const int flip_vec = (n % 4 == 0) && (reinterpret_cast<uintptr_t>(H) % 16 == 0) &&
                       (reinterpret_cast<uintptr_t>(Mm) % 16 == 0) && (lda % 4 == 0);
  hipLaunchKernelGGL(flip_kernel, dim3((unsigned)ceil_div(n, 1024), (unsigned)n), dim3(256), 0,
                     stream, (const float*)Mm, lda, n, H, flip_vec);
  GPTQ_LAUNCH_CHECK();

  int hflag = 0;
  double hlam = 0.0;
  GPTQ_HIP_CHECK(hipMemcpyAsync(&hflag, flag, sizeof(int), hipMemcpyDeviceToHost, stream));
  GPTQ_HIP_CHECK(hipMemcpyAsync(&hlam, lam, sizeof(double), hipMemcpyDeviceToHost, stream));
  GPTQ_HIP_CHECK(hipStreamSynchronize(stream));
  if (damp_out) *damp_out = hlam;
  if (hflag & kFlagNonFinite) {
    set_error("gptq_prepare_hinv: non-finite value on the Hessian diagonal");
    return GPTQ_ERR_NONFINITE;
  }
  if (hflag & kFlagNotPD) {
    set_error("gptq_prepare_hinv: damped Hessian is not positive definite");
    return GPTQ_ERR_NOT_PD;
  }
  return GPTQ_OK;
}

}  // namespace gptq
