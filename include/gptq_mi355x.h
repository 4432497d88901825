/*
 * gptq_mi355x.h -- C ABI of the MI355X (gfx950) GPTQ layer-quantization path.
 *
 * The path has the three calls of the GPTQ quantizer sketched on the page
 * "模型量化实战：从 INT8 PTQ 到 GPTQ 的精度保持与推理加速全解析" (qwbw.cn), §3.2
 * (accumulate_hessian -> prepare -> quantize), with the quantize_config fields
 * {bits, group_size, damp_percent, desc_act} of the page "Llama-2 GPTQ
 * quantization in practice" (mjmagnets.cn), §3.3, and sym of the page
 * "GPTQ量化损失深度解析" (bmjup.com).
 *
 * Conventions shared by every call:
 *   - All tensor pointers are DEVICE memory owned by the caller (allocated
 *     through PyTorch or hipMalloc).  The library allocates no device memory;
 *     its only state is a thread-local error message and, for
 *     gptq_prepare_hinv and gptq_quantize_layer, up to three extra HIP
 *     streams (default priority) with their events per host thread and
 *     device, created on first use and kept until the process ends.  They
 *     carry no data between calls: they are execution resources, like a BLAS
 *     handle's internal streams, that let the latency-bound chain of a call
 *     run beside its bulk updates.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *     on it in order; calls return after enqueueing, except where a call says
 *     it synchronises.  Work a call puts on its extra streams is ordered
 *     after what `stream` held at the call and before anything enqueued on
 *     `stream` after it (events), so to the caller it is one stream-ordered
 *     operation; this holds for a call that fails after launching, too.
 *     Concurrent calls from one host thread on different streams share those
 *     extra streams and are serialised by them.
 *   - Argument errors are detected on the host and returned before anything
 *     is launched.  A failed HIP launch or copy returns GPTQ_ERR_HIP.
 *   - Matrices are row-major.  n = in_features (columns of W, size of H),
 *     m = out_features (rows of W), tokens = calibration rows of X.
 *   - gptq_last_error() returns a message for the last non-OK status of the
 *     calling thread (empty string if none).
 */
#ifndef GPTQ_MI355X_H
#define GPTQ_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GPTQ_OK = 0,
  GPTQ_ERR_INVALID_ARG = -1, /* null pointer, negative size, bad stride      */
  GPTQ_ERR_UNSUPPORTED = -2, /* bits/group/block/dtype outside what is built */
  GPTQ_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required   */
  GPTQ_ERR_NOT_PD = -4,      /* damped Hessian not positive definite         */
  GPTQ_ERR_NONFINITE = -5,   /* NaN/Inf in the Hessian diagonal or in W      */
  GPTQ_ERR_HIP = -6          /* a HIP runtime call failed                    */
} gptq_status;

typedef enum { GPTQ_BF16 = 0, GPTQ_FP32 = 1 } gptq_dtype;

/* Quantizer settings (the quantize_config of the pages, plus sym).
 *   bits         2, 3, 4 or 8.
 *   group_size   a power of two dividing block_size (1..128), or -1 for one
 *                group per output row.  Groups are runs of group_size
 *                consecutive columns in PROCESSING order (after desc_act).
 *   sym          0: asymmetric grid with a zero point; 1: symmetric grid.
 *   desc_act     1: process columns by descending Hessian diagonal.
 *   block_size   columns per lazy-update block; must be 128.
 *   damp_percent read by gptq_prepare_hinv only (lambda = damp_percent *
 *                mean(diag H)); ignored here.                              */
typedef struct {
  int32_t bits;
  int32_t group_size;
  int32_t sym;
  int32_t desc_act;
  int32_t block_size;
  double damp_percent;
} gptq_config;

/* ------------------------------------------------------------------------
 * Stage 1 -- Hessian accumulation.
 * Defines: H = 2·XᵀX summed over calibration tokens (page "模型量化实战…"
 * §3.2, accumulate_hessian; the page "Llama-2 GPTQ quantization in practice"
 * §2.2.1 writes the same matrix as the expectation of x⊗x).
 *
 *   H          [n, n] fp32, in/out.  ACCUMULATED: the caller zeroes H (and
 *              diag_key) once, then calls once per token tile.  On return
 *              both triangles hold H + alpha·XᵀX (H stays symmetric); the
 *              kernels read only the lower triangle of the incoming H.
 *   diag_key   [n] fp64, in/out, accumulated like H: key += alpha·Σ_t x_t²,
 *              summed in fp64 so that the act-order sort is exact enough.
 *              May be NULL.
 *   X          [tokens, ldx] of x_dtype (GPTQ_BF16 or GPTQ_FP32), token-
 *              major (row t = one token's n activations).  ldx >= n.
 *              tokens == 0 is a no-op.
 *   alpha      scale of the product (2.0 gives H = 2·XᵀX).
 *   workspace  device scratch of at least gptq_hessian_workspace_bytes(n,
 *              tokens, x_dtype) bytes (split-K partial tiles and counters);
 *              may be NULL when that size is 0.  Its contents are not kept.
 * Deterministic: the same inputs give bitwise the same H.
 * ---------------------------------------------------------------------- */
size_t gptq_hessian_workspace_bytes(int64_t n, int64_t tokens, int32_t x_dtype);
gptq_status gptq_hessian_accumulate(float* H, double* diag_key, int64_t n, const void* X,
                                    int32_t x_dtype, int64_t tokens, int64_t ldx, float alpha,
                                    void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Stages 2-3 -- damping, act-order and the inverse factor.
 * Defines: H += damp·mean(diag H)·I, then the upper Cholesky factor of the
 * inverse (page "模型量化实战…" §3.2, prepare: damping, Cholesky, inverse,
 * upper Cholesky -- the factorisation is taken once); desc_act orders the
 * columns by the Hessian diagonal (page "GPTQ量化损失深度解析", tuning
 * section; page "Qwen2.5模型GPTQ量化精度损失实测" on act-order reordering).
 *
 *   H_inout    [n, n] fp32.  In: the symmetric H from stage 1 (un-permuted).
 *              Out: U, upper triangular with positive diagonal and
 *              UᵀU = (P (H + λI) Pᵀ)⁻¹ in PROCESSING order; the strictly
 *              lower triangle is set to 0.
 *   diag_key   [n] fp64 sort key and damping mean (stage 1's diag_key), or
 *              NULL to use diag(H) in fp32.
 *   desc_act   1: perm = stable descending sort of the key (ties keep the
 *              lower original index first); 0: identity.
 *   perm_out   [n] int32, out: perm_out[p] = original column processed at
 *              position p.
 *   workspace  at least gptq_prepare_workspace_bytes(n) bytes.
 *   damp_out   HOST pointer, may be NULL: receives λ (fp64).
 * Synchronises `stream` once at the end, to return GPTQ_ERR_NONFINITE (a NaN
 * or Inf on the Hessian diagonal) or GPTQ_ERR_NOT_PD (a non-positive pivot);
 * H_inout then holds no usable factor.  n == 0 is a no-op.
 * ---------------------------------------------------------------------- */
size_t gptq_prepare_workspace_bytes(int64_t n);
gptq_status gptq_prepare_hinv(float* H_inout, const double* diag_key, int64_t n,
                              double damp_percent, int32_t desc_act, int32_t* perm_out,
                              void* workspace, size_t ws_bytes, double* damp_out, void* stream);

/* ------------------------------------------------------------------------
 * Stage 4-5 -- block-wise column quantization with error feedback, then
 * packing.  Defines: column by column in processing order, each output row's
 * weight is rounded to the row's group grid and the rounding error is pushed
 * onto the not-yet-quantized columns through the inverse factor (page
 * "大模型量化：GPTQ/AWQ/GGUF 原理对比", GPTQ section and its column-flow
 * description; page "模型量化实战…" §3.2 quantize_block); the grid is the
 * affine x_q = round(x/scale + zero) of that page's §2.1/§3.1.
 *
 *   W        [m, n] of w_dtype, row-major (nn.Linear layout), read only.
 *   U, perm  outputs of gptq_prepare_hinv for this layer's H.
 *   cfg      see gptq_config (block_size must be 128).
 * Outputs, all in ORIGINAL column order where columns appear:
 *   qweight  [m, gptq_qweight_words(n, bits)] uint32.  bits <= 4: eight
 *            codes per word, column 8w+i in bits [4i, 4i+4); bits == 8: four
 *            codes per word, column 4w+i in bits [8i, 8i+8).  Last word of a
 *            row zero-padded.
 *   scales   [m, G] fp32, G = gptq_num_groups(n, group_size), group order.
 *   zeros    [m, G] int32.  Dequantization is always (q - zero)·scale; a
 *            symmetric grid stores codes offset by 2^(bits-1) and zero =
 *            2^(bits-1).
 *   g_idx    [n] int32: group of each original column (p // group_size for
 *            the column processed at position p; 0 when group_size == -1).
 *   loss     [2] fp64 device: loss[0] = ½·Σ e² over all columns, which
 *            equals ½·tr(ΔW (H+λI) ΔWᵀ); loss[1] = ‖W − Ŵ‖²_F.  The
 *            reconstruction loss ‖ΔW Xᵀ‖²_F = loss[0] − (λ/2)·loss[1].
 *   status_out  [1] int32 DEVICE word, may be NULL: receives GPTQ_OK, or
 *            GPTQ_ERR_NONFINITE if W holds a NaN or Inf (the other outputs
 *            are then meaningless).  Written in stream order as the call's
 *            last step; the caller reads it when it chooses to synchronise.
 *   workspace at least gptq_quantize_workspace_bytes(m, n, cfg) bytes.
 * Stream-ordered: the call returns after enqueueing and never synchronises
 * the host (a layer sweep issues no host sync per quantization).  The return
 * value covers argument checks and launch failures only.  m == 0 or n == 0
 * is a no-op (status_out is left unchanged).
 * ---------------------------------------------------------------------- */
size_t gptq_quantize_workspace_bytes(int64_t m, int64_t n, const gptq_config* cfg);
gptq_status gptq_quantize_layer(const void* W, int32_t w_dtype, int64_t m, int64_t n,
                                const float* U, const int32_t* perm, const gptq_config* cfg,
                                uint32_t* qweight, float* scales, int32_t* zeros, int32_t* g_idx,
                                double* loss, int32_t* status_out, void* workspace, size_t ws_bytes,
                                void* stream);

/* ------------------------------------------------------------------------
 * The linear round-to-nearest quantizer (no Hessian, no error feedback).
 * Defines: the LinearQuantizer of page "模型量化实战：从 INT8 PTQ 到 GPTQ…"
 * §3.1 with the affine formula of its §2.1: per output row ("per channel")
 * or per group of group_size consecutive columns of a row,
 *   symmetric:  scale = percentile(|w|, clip) / (2^(b-1) - 1),
 *               q = round(w / scale) clamped to [-2^(b-1), 2^(b-1) - 1];
 *   asymmetric: lo, hi = percentile(w, (1-clip)/2), percentile(w, 1-(1-clip)/2),
 *               scale = (hi - lo) / (2^b - 1), zero = -round(lo / scale),
 *               q = round(w / scale + zero) clamped to [0, 2^b - 1];
 * scale floored at 1e-8; round = half to even; percentile(v, f) interpolates
 * linearly between the sorted values at position f·(N-1) (clip = 1: the
 * maximum, or the minimum and maximum); the range is NOT widened to include
 * 0, so an asymmetric zero may lie outside [0, 2^b - 1].  The grid and the
 * codes are computed in fp64.
 *
 *   W        [m, n] of w_dtype (GPTQ_BF16 or GPTQ_FP32), row-major, read only.
 *   cfg      bits 2, 3, 4 or 8; group_size -1 (one group per row) or >= 1;
 *            sym 0/1; clip_ratio in (0, 1].
 * Outputs (original column order; layouts as in gptq_quantize_layer):
 *   qweight  [m, gptq_qweight_words(n, bits)] uint32.
 *   scales   [m, G] fp32 (the fp64 scale rounded), G = gptq_num_groups(n, g).
 *   zeros    [m, G] int32; dequantization is (q - zero)·scale, symmetric codes
 *            stored offset by 2^(bits-1) with zero = 2^(bits-1).
 *   err      [2] fp64 device: err[0] = mean over the m·n weights of
 *            (w - ŵ)², err[1] = Σ w·ŵ / (‖w‖·‖ŵ‖ + 1e-8) (the page's
 *            quantization_error), ŵ from the fp64 scale.
 *   status_out  [1] int32 DEVICE word, may be NULL: receives GPTQ_OK, or
 *            GPTQ_ERR_NONFINITE if W holds a NaN or Inf, in stream order.
 *   workspace at least gptq_rtn_workspace_bytes(m, n, cfg) bytes.
 * Returns GPTQ_ERR_UNSUPPORTED when one row's groups do not fit the on-chip
 * sort (n <= 32768 for one group per row; for groups of g columns,
 * ceil(n/g)·(4·P + 16) <= 150 KiB with P = g rounded up to a power of two).
 * With clip_ratio = 1 (no order statistics), 16-byte aligned rows
 * (n % 8 == 0), n <= 32768 and a group of 8·d columns with d dividing 64 (or
 * one group per row), the rows are streamed in one pass; the outputs are the
 * same.  Stream-ordered, no synchronisation.  m == 0 or n == 0 is a no-op.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t bits;
  int32_t group_size;
  int32_t sym;
  float clip_ratio;
} gptq_rtn_config;

size_t gptq_rtn_workspace_bytes(int64_t m, int64_t n, const gptq_rtn_config* cfg);
gptq_status gptq_rtn_quantize(const void* W, int32_t w_dtype, int64_t m, int64_t n,
                              const gptq_rtn_config* cfg, uint32_t* qweight, float* scales,
                              int32_t* zeros, double* err, int32_t* status_out, void* workspace,
                              size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Activation-aware channel scaling (AWQ) in front of the linear quantizer
 *
 * Page "大模型量化：GPTQ/AWQ/GGUF 原理对比，4-bit 量化对推理精度的影响", AWQ
 * section: the importance of input channel j is mean_t |x_t[j]| over the
 * calibration tokens; channels whose importance is strictly above its median
 * (torch.median: the lower middle value for an even count) are multiplied by
 * a protection factor s (2.0 in the page), the others by 1; the scaled weight
 * is quantized, and dequantization divides by the channel factor again (at
 * inference the activations are divided by it).
 *
 * gptq_awq_channel_stats ACCUMULATES abs_sum[j] += Σ_t |X[t][j]| (fp64) over
 * X [tokens][ldx] (bf16 or fp32, unit column stride): the caller zeroes
 * abs_sum once and may call once per token tile.  Stream-ordered; the
 * summation order is fixed (reproducible).  workspace: at least
 * gptq_awq_stats_workspace_bytes(n, tokens) bytes, 256-byte aligned.
 *
 * gptq_awq_quantize computes the channel factors from abs_sum and the token
 * count (tokens > 0), writes them to channel_scale (fp32 [n], s or 1), and
 * quantizes fl32(W·channel_scale) with the linear quantizer of
 * gptq_rtn_quantize (same cfg, same qweight / scales / zeros layout).  err[0],
 * err[1] are the MSE and cosine between W and the dequantized weight divided
 * by the channel factor.  protect > 0 and finite.  workspace: at least
 * gptq_awq_workspace_bytes(m, n, cfg) bytes.  status_out (device int32,
 * may be NULL) receives GPTQ_ERR_NONFINITE if W or abs_sum holds a NaN or
 * Inf, else GPTQ_OK, in stream order; the call does not synchronise.  The
 * same limits as gptq_rtn_quantize apply (GPTQ_ERR_UNSUPPORTED).
 * ---------------------------------------------------------------------- */
size_t gptq_awq_stats_workspace_bytes(int64_t n, int64_t tokens);
gptq_status gptq_awq_channel_stats(const void* X, int32_t x_dtype, int64_t tokens, int64_t ldx,
                                   int64_t n, double* abs_sum, void* workspace, size_t ws_bytes,
                                   void* stream);
size_t gptq_awq_workspace_bytes(int64_t m, int64_t n, const gptq_rtn_config* cfg);
gptq_status gptq_awq_quantize(const void* W, int32_t w_dtype, int64_t m, int64_t n,
                              const double* abs_sum, int64_t tokens, float protect,
                              const gptq_rtn_config* cfg, uint32_t* qweight, float* scales,
                              int32_t* zeros, float* channel_scale, double* err, int32_t* status_out,
                              void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Product of bf16 activations with the quantized weights (W4A16)
 *
 * Page "模型量化实战：从 INT8 PTQ 到 GPTQ 的精度保持与推理加速全解析" §4.3:
 * 4-bit weights have no native matrix product; they are dequantized to a
 * 16-bit type (§2.1: x̂ = (q - z)·s) and multiplied, and the gain is the 4x
 * smaller weight stream.  Y[t][r] = Σ_k X[t][k]·(q[r][k] - z[r][g_idx[k]])·
 * s[r][g_idx[k]] with bf16 X, fp32 Y.  The codes enter the bf16 products
 * exactly (as 128 + q) and each group's scale is applied to its fp32 partial
 * sum, so the only roundings are those of the fp32 sums.
 *
 * gptq_w4a16_pack converts gptq_quantize_layer's output (qweight, scales,
 * zeros, g_idx of an m x n weight, bits 2, 3 or 4, group_size 32, 64, 128 or
 * -1) once into the product's layout, `packed` (device memory of at least
 * gptq_w4a16_packed_bytes(m, n, group_size) bytes, 256-byte aligned, owned by
 * the caller, read-only afterwards): the column order is derived from g_idx
 * (group p's columns in ascending order), so act-order weights need no
 * separate permutation.  Synchronises `stream` once and returns
 * GPTQ_ERR_INVALID_ARG if g_idx does not assign exactly min(g, n - p·g)
 * columns to every group p (exactly n to group 0 when group_size = -1).
 *
 * gptq_w4a16_matmul computes Y = X·Ŵᵀ for X bf16 [tokens][ldx] (unit column
 * stride, ldx >= n), Y fp32 [tokens][ldy] (ldy >= m), with workspace of at
 * least gptq_w4a16_workspace_bytes(tokens, m, n) bytes (256-byte aligned).
 * Stream-ordered, no synchronisation; tokens are processed 64 per launch
 * sequence (gather, product, reduce); the summation order is fixed, so the
 * result is reproducible bit for bit.  tokens == 0 is a no-op.
 * ---------------------------------------------------------------------- */
size_t gptq_w4a16_packed_bytes(int64_t m, int64_t n, int32_t group_size);
gptq_status gptq_w4a16_pack(const uint32_t* qweight, const float* scales, const int32_t* zeros,
                            const int32_t* g_idx, int64_t m, int64_t n, int32_t bits,
                            int32_t group_size, void* packed, size_t packed_bytes, void* stream);
size_t gptq_w4a16_workspace_bytes(int64_t tokens, int64_t m, int64_t n);
gptq_status gptq_w4a16_matmul(const void* X, int64_t tokens, int64_t ldx, const void* packed,
                              int64_t m, int64_t n, int32_t group_size, float* Y, int64_t ldy,
                              void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * gptq_w4a16_matmul without a workspace: for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, result and rules as
 * gptq_w4a16_matmul minus the workspace: the gather, partial sums and
 * position sums live in a static device array the library holds on every GPU
 * it runs on until the process ends (gptq_w4a16_noalloc_scratch_bytes()
 * bytes, 32 MiB).  The call allocates nothing; when 64 tokens per launch
 * sequence would not fit it takes fewer, and it returns GPTQ_ERR_UNSUPPORTED
 * (before launching anything) when even 16 tokens per launch do not fit the
 * array.  Calls that overlap on one GPU race on the array: serialise them
 * (one stream, or events).  The result is bit-identical to gptq_w4a16_matmul.
 * ---------------------------------------------------------------------- */
size_t gptq_w4a16_noalloc_scratch_bytes(void);
gptq_status gptq_w4a16_matmul_noalloc(const void* X, int64_t tokens, int64_t ldx, const void* packed,
                                      int64_t m, int64_t n, int32_t group_size, float* Y, int64_t ldy,
                                      void* stream);

/* ------------------------------------------------------------------------
 * Export of a quantized layer to the tensor layout of GPTQ checkpoints.
 * Page "模型量化实战：从 INT8 PTQ 到 GPTQ…" §3.3 saves the quantized model as
 * a GPTQ checkpoint (about 4.1 GB for 7B) but does not define its tensors;
 * the layout here is the one such checkpoints commonly carry, defined as bit
 * streams (b = bits; "the bit stream" of a list of codes puts code k in bits
 * [k·b, k·b + b) of consecutive little-endian 32-bit words, padding bits 0):
 *
 *   qweight, scales, zeros  gptq_quantize_layer's (or gptq_rtn_quantize's)
 *            outputs for an m x n weight with this bits and group_size;
 *            only the low b bits of each code field are read.
 *   zero_offset  0: zero points stored as they are; 1: stored as zero - 1
 *            (the older checkpoints' convention).  Values are kept mod 2^b.
 * Outputs (device, caller-owned, all fully written):
 *   ck_qweight [gptq_checkpoint_qweight_rows(n, bits)][m] int32: column i is
 *            the bit stream of output row i's n codes in input order.
 *   ck_qzeros  [G][gptq_checkpoint_qzeros_words(m, bits)] int32: row g is the
 *            bit stream of (zeros[i][g] - zero_offset) mod 2^b over i.
 *   ck_scales  [G][m] IEEE fp16 (uint16 bits): scales[i][g] rounded to
 *            nearest even (overflow to infinity, subnormals kept).
 * g_idx is the quantizer's own, unchanged.  G = gptq_num_groups(n,
 * group_size).  Stream-ordered, no synchronisation, no workspace.  m == 0 or
 * n == 0 is a no-op.  Returns GPTQ_ERR_UNSUPPORTED for bits outside
 * {2, 3, 4, 8} or more than 65535 groups or 4194240 rows.
 * ---------------------------------------------------------------------- */
int64_t gptq_checkpoint_qweight_rows(int64_t n, int32_t bits);
int64_t gptq_checkpoint_qzeros_words(int64_t m, int32_t bits);
gptq_status gptq_export_checkpoint(const uint32_t* qweight, const float* scales, const int32_t* zeros,
                                   int64_t m, int64_t n, int32_t bits, int32_t group_size, int32_t zero_offset,
                                   int32_t* ck_qweight, int32_t* ck_qzeros, uint16_t* ck_scales, void* stream);

/* Sizes of the outputs above (host-only helpers, no GPU work). */
int64_t gptq_qweight_words(int64_t n, int32_t bits);
int64_t gptq_num_groups(int64_t n, int32_t group_size);

/* Message of the calling thread's last non-OK status. */
const char* gptq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GPTQ_MI355X_H */
