// Export of a quantized layer into the tensor layout GPTQ checkpoints use.
//
// The page "模型量化实战：从 INT8 PTQ 到 GPTQ…" §3.3 saves the quantized
// model as a GPTQ checkpoint (about 4.1 GB for a 7B model) without defining
// its tensors.  The layout written here is the one such checkpoints commonly
// carry, stated as a bit-stream definition:
//   qweight [ceil(n·b/32)][m] int32: column i (one output row of W) is the
//           little-endian bit stream of its n codes in input order, code k
//           in bits [k·b, k·b + b); word w of the stream is qweight[w][i];
//   qzeros  [G][ceil(m·b/32)] int32: row g is the bit stream of the m zero
//           points of group g, each stored as (zero - zero_offset) mod 2^b
//           (zero_offset 1 is the older checkpoints' convention);
//   scales  [G][m] fp16, the fp32 scale rounded to nearest even.
// Padding bits past the last code are zero.  g_idx is the quantizer's own.
//
// Input is the quantizer's layout: qweight [m][words] uint32 with eight 4-bit
// fields per word for bits <= 4 (column 8w + j in bits [4j, 4j + 4)) or four
// bytes for bits = 8; only the low b bits of each field are taken.
//
// qweight kernel: a 64-row x 32-word tile of the input goes to LDS with
// coalesced row reads; each thread then assembles output words of one column
// (consecutive threads: consecutive columns, so the stores are coalesced).
// The tile starts at code 256·x (b <= 4) or 128·x (b = 8), a multiple of 32
// codes, so it maps to whole output words; for 4- and 8-bit codes the input
// words are the output words and the kernel is a transpose.  params kernel:
// 32 rows x 32 groups per workgroup through LDS (coalesced reads of each
// row's run of groups): fp16 scales, and the zeros' bit streams.
#include "gptq_internal.hpp"

namespace gptq {
namespace {

constexpr int kCkRows = 64;    // input rows (output columns) per qweight tile
constexpr int kCkWords = 32;   // input words per qweight tile
constexpr int kCkThreads = 256;
constexpr int kPrRows = 32;    // rows per params tile (32·b bits: b whole qzeros words)
constexpr int kPrGroups = 32;  // groups per params tile (m/32 x G/32 workgroups)

// Bits [32·ow, 32·ow + 32) of a stream whose code c is field(c).
template <int B, typename F>
__device__ __forceinline__ uint32_t stream_word(int ow, F field) {
  const int c0 = (32 * ow) / B, c1 = (32 * ow + 31) / B;
  uint32_t acc = 0u;
  for (int c = c0; c <= c1; ++c) {
    const uint32_t v = field(c);
    const int s = c * B - 32 * ow;
    acc |= s >= 0 ? (v << s) : (v >> -s);
  }
  return acc;
}

template <int B>
__global__ __launch_bounds__(kCkThreads) void ck_qweight_kernel(const uint32_t* __restrict__ qw, int64_t m,
                                                                int64_t n, int64_t words,
                                                                uint32_t* __restrict__ out, int64_t rows_out) {
  constexpr int kPer = B <= 4 ? 8 : 4, kWidth = B <= 4 ? 4 : 8;
  constexpr uint32_t kMask = (1u << B) - 1u;
  constexpr int kOws = kCkWords * kPer * B / 32;   // output words of the tile
  __shared__ uint32_t tile[kCkRows][kCkWords + 1];
  const int tid = threadIdx.x;
  const int64_t w0 = (int64_t)blockIdx.x * kCkWords;
  const int64_t i0 = (int64_t)blockIdx.y * kCkRows;
#pragma unroll
  for (int e = 0; e < kCkRows * kCkWords / kCkThreads; ++e) {
    const int idx = tid + kCkThreads * e;
    const int r = idx / kCkWords, c = idx % kCkWords;
    const int64_t i = i0 + r, w = w0 + c;
    tile[r][c] = (i < m && w < words) ? qw[i * words + w] : 0u;
  }
  __syncthreads();
  const int64_t code0 = w0 * kPer;   // first code of the tile
  const int64_t ow0 = code0 * B / 32;
  const int il = tid % kCkRows;
  const int64_t i = i0 + il;
  if (i >= m) return;
#pragma unroll
  for (int ow = tid / kCkRows; ow < kOws; ow += kCkThreads / kCkRows) {
    if (ow0 + ow >= rows_out) break;
    uint32_t v;
    if constexpr (B == kWidth) {
      // the field is the code and a word holds whole codes: the words move
      // as they are, the last one of a row cut at code n
      v = tile[il][ow];
      const int64_t keep = n - (code0 + (int64_t)ow * kPer);
      if (keep < kPer) v = keep <= 0 ? 0u : v & ((1u << (keep * kWidth)) - 1u);
    } else {
      v = stream_word<B>(ow, [&](int c) -> uint32_t {
        if (code0 + c >= n) return 0u;
        return (tile[il][c / kPer] >> (kWidth * (c % kPer))) & kMask;
      });
    }
    out[(ow0 + ow) * m + i] = v;
  }
}

// One workgroup per 32 rows x 32 groups: the rows' scales and zero points
// (contiguous runs of each row) through LDS, then fp16 scales [g][i] and the
// zero points' b words per group.
template <int B>
__global__ __launch_bounds__(kCkThreads) void ck_params_kernel(const float* __restrict__ scales,
                                                               const int32_t* __restrict__ zeros, int64_t m,
                                                               int64_t G, int zero_offset,
                                                               uint32_t* __restrict__ qzeros, int64_t zwords,
                                                               _Float16* __restrict__ sc_out) {
  constexpr uint32_t kMask = (1u << B) - 1u;
  __shared__ float s[kPrRows][kPrGroups + 1];
  __shared__ uint32_t z[kPrRows][kPrGroups + 1];
  const int tid = threadIdx.x;
  const int64_t i0 = (int64_t)blockIdx.x * kPrRows;
  const int64_t g0 = (int64_t)blockIdx.y * kPrGroups;
#pragma unroll 4
  for (int e = tid; e < kPrRows * kPrGroups; e += kCkThreads) {
    const int r = e / kPrGroups, gl = e % kPrGroups;
    const int64_t i = i0 + r, g = g0 + gl;
    const bool in = i < m && g < G;
    s[r][gl] = in ? scales[i * G + g] : 0.f;
    z[r][gl] = in ? (uint32_t)(zeros[i * G + g] - zero_offset) & kMask : 0u;
  }
  __syncthreads();
#pragma unroll 4
  for (int e = tid; e < kPrRows * kPrGroups; e += kCkThreads) {
    const int gl = e / kPrRows, r = e % kPrRows;
    const int64_t i = i0 + r, g = g0 + gl;
    if (i < m && g < G) sc_out[g * m + i] = (_Float16)s[r][gl];
  }
  // rows i0 .. i0 + 31 are bits [i0·b, i0·b + 32·b) of each group's stream
  const int64_t ow0 = i0 * B / 32;
  for (int e = tid; e < kPrGroups * B; e += kCkThreads) {
    const int gl = e / B, w = e % B;
    const int64_t g = g0 + gl;
    if (g < G && ow0 + w < zwords)
      qzeros[g * zwords + ow0 + w] = stream_word<B>(w, [&](int c) -> uint32_t { return z[c][gl]; });
  }
}

template <int B>
gptq_status launch_export(const uint32_t* qweight, const float* scales, const int32_t* zeros, int64_t m,
                          int64_t n, int64_t G, int zero_offset, uint32_t* ck_qweight, uint32_t* ck_qzeros,
                          _Float16* ck_scales, hipStream_t stream) {
  const int64_t words = B <= 4 ? ceil_div(n, 8) : ceil_div(n, 4);
  const int64_t rows_out = ceil_div(n * B, 32);
  const int64_t zwords = ceil_div(m * B, 32);
  hipLaunchKernelGGL(ck_qweight_kernel<B>, dim3((unsigned)ceil_div(words, kCkWords), (unsigned)ceil_div(m, kCkRows)),
                     dim3(kCkThreads), 0, stream, qweight, m, n, words, ck_qweight, rows_out);
  GPTQ_LAUNCH_CHECK();
  hipLaunchKernelGGL(ck_params_kernel<B>, dim3((unsigned)ceil_div(m, kPrRows), (unsigned)ceil_div(G, kPrGroups)),
                     dim3(kCkThreads), 0, stream, scales, zeros, m, G, zero_offset, ck_qzeros, zwords, ck_scales);
  GPTQ_LAUNCH_CHECK();
  return GPTQ_OK;
}

}  // namespace

gptq_status run_checkpoint_export(const uint32_t* qweight, const float* scales, const int32_t* zeros, int64_t m,
                                  int64_t n, int bits, int64_t G, int zero_offset, int32_t* ck_qweight,
                                  int32_t* ck_qzeros, uint16_t* ck_scales, hipStream_t stream) {
  uint32_t* const qo = reinterpret_cast<uint32_t*>(ck_qweight);
  uint32_t* const zo = reinterpret_cast<uint32_t*>(ck_qzeros);
  _Float16* const so = reinterpret_cast<_Float16*>(ck_scales);
  switch (bits) {
    case 2: return launch_export<2>(qweight, scales, zeros, m, n, G, zero_offset, qo, zo, so, stream);
    case 3: return launch_export<3>(qweight, scales, zeros, m, n, G, zero_offset, qo, zo, so, stream);
    case 4: return launch_export<4>(qweight, scales, zeros, m, n, G, zero_offset, qo, zo, so, stream);
    case 8: return launch_export<8>(qweight, scales, zeros, m, n, G, zero_offset, qo, zo, so, stream);
    default: break;
  }
  set_error("gptq_export_checkpoint: bits=%d", bits);
  return GPTQ_ERR_UNSUPPORTED;
}

}  // namespace gptq
