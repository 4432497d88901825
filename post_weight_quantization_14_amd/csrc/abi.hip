// extern "C" entry points of libgptq_mi355x: argument validation on the host,
// workspace layout, then the stage launchers (hessian.hip, prepare.hip,
// quantize.hip).  Every check here runs before any HIP call, so a rejected
// call touches no GPU state.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <vector>

#include "gptq_internal.hpp"

namespace gptq {
namespace {
thread_local char g_err[512] = {0};
}

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

void clear_error() { g_err[0] = 0; }

namespace {
constexpr int64_t kMaxN = 131072;

gptq_status fail(gptq_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

bool bad_ptr(const void* p, size_t align) {
  return p == nullptr || (reinterpret_cast<uintptr_t>(p) % align) != 0;
}

gptq_status check_config(const gptq_config* cfg) {
  if (!cfg) return fail(GPTQ_ERR_INVALID_ARG, "cfg is NULL");
  if (!(cfg->bits == 2 || cfg->bits == 3 || cfg->bits == 4 || cfg->bits == 8))
    return fail(GPTQ_ERR_UNSUPPORTED, "bits=%d (built: 2, 3, 4, 8)", cfg->bits);
  if (cfg->block_size != kQBlock)
    return fail(GPTQ_ERR_UNSUPPORTED, "block_size=%d (built: 128)", cfg->block_size);
  const int g = cfg->group_size;
  if (!(g == -1 || g == 8 || g == 16 || g == 32 || g == 64 || g == 128))
    return fail(GPTQ_ERR_UNSUPPORTED, "group_size=%d (built: -1, 8, 16, 32, 64, 128)", g);
  if (cfg->sym != 0 && cfg->sym != 1) return fail(GPTQ_ERR_INVALID_ARG, "sym=%d", cfg->sym);
  if (cfg->desc_act != 0 && cfg->desc_act != 1)
    return fail(GPTQ_ERR_INVALID_ARG, "desc_act=%d", cfg->desc_act);
  return GPTQ_OK;
}
}  // namespace
}  // namespace gptq

using namespace gptq;

namespace gptq {

gptq_status get_side_stream(SideStream& out, int which) {
  thread_local std::vector<SideStream> per_device;   // [device][which]
  if (which < 0 || which >= kSideStreams) {
    set_error("side stream %d out of range", which);
    return GPTQ_ERR_INVALID_ARG;
  }
  int dev = 0;
  GPTQ_HIP_CHECK(hipGetDevice(&dev));
  if ((int)per_device.size() < kSideStreams * (dev + 1)) per_device.resize(kSideStreams * (dev + 1));
  SideStream& s = per_device[kSideStreams * dev + which];
  if (s.stream == nullptr) {
    GPTQ_HIP_CHECK(hipStreamCreateWithFlags(&s.stream, hipStreamNonBlocking));
    // only streams of this device wait on them: a device-scope release suffices
    GPTQ_HIP_CHECK(hipEventCreateWithFlags(&s.ready, hipEventDisableTiming | hipEventReleaseToDevice));
    GPTQ_HIP_CHECK(hipEventCreateWithFlags(&s.done, hipEventDisableTiming | hipEventReleaseToDevice));
    for (hipEvent_t& e : s.aux)
      GPTQ_HIP_CHECK(hipEventCreateWithFlags(&e, hipEventDisableTiming | hipEventReleaseToDevice));
  }
  out = s;
  return GPTQ_OK;
}

}  // namespace gptq

extern "C" {

const char* gptq_last_error(void) { return g_err; }

int64_t gptq_qweight_words(int64_t n, int32_t bits) {
  if (n < 0) return -1;
  if (bits == 2 || bits == 3 || bits == 4) return ceil_div(n, 8);
  if (bits == 8) return ceil_div(n, 4);
  return -1;
}

int64_t gptq_num_groups(int64_t n, int32_t group_size) {
  if (n < 0) return -1;
  if (group_size == -1) return n > 0 ? 1 : 0;
  if (group_size <= 0) return -1;
  return ceil_div(n, group_size);
}

size_t gptq_hessian_workspace_bytes(int64_t n, int64_t tokens, int32_t x_dtype) {
  if (n <= 0 || n > kMaxN || tokens < 0) return 0;
  if (x_dtype != GPTQ_BF16) return 0;
  return plan_syrk_bf16(n, tokens).total_bytes;
}

gptq_status gptq_hessian_accumulate(float* H, double* diag_key, int64_t n, const void* X,
                                    int32_t x_dtype, int64_t tokens, int64_t ldx, float alpha,
                                    void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  if (n <= 0) return fail(GPTQ_ERR_INVALID_ARG, "n=%lld must be positive", (long long)n);
  if (n > kMaxN) return fail(GPTQ_ERR_UNSUPPORTED, "n=%lld above %lld", (long long)n, (long long)kMaxN);
  if (tokens < 0) return fail(GPTQ_ERR_INVALID_ARG, "tokens=%lld", (long long)tokens);
  if (x_dtype != GPTQ_BF16 && x_dtype != GPTQ_FP32)
    return fail(GPTQ_ERR_UNSUPPORTED, "x_dtype=%d", x_dtype);
  if (bad_ptr(H, 4)) return fail(GPTQ_ERR_INVALID_ARG, "H is NULL or misaligned");
  if (diag_key && bad_ptr(diag_key, 8)) return fail(GPTQ_ERR_INVALID_ARG, "diag_key misaligned");
  if (!std::isfinite(alpha)) return fail(GPTQ_ERR_INVALID_ARG, "alpha not finite");
  if (tokens == 0) return GPTQ_OK;
  if (ldx < n) return fail(GPTQ_ERR_INVALID_ARG, "ldx=%lld < n=%lld", (long long)ldx, (long long)n);
  if (bad_ptr(X, x_dtype == GPTQ_BF16 ? 2 : 4)) return fail(GPTQ_ERR_INVALID_ARG, "X is NULL or misaligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (x_dtype == GPTQ_FP32)
    return launch_hessian_f32(H, diag_key, n, static_cast<const float*>(X), tokens, ldx, alpha, s);
  const SyrkPlan plan = plan_syrk_bf16(n, tokens);
  if (plan.total_bytes > 0 && (workspace == nullptr || ws_bytes < plan.total_bytes || bad_ptr(workspace, 256)))
    return fail(GPTQ_ERR_WORKSPACE, "workspace %zu bytes, need %zu (256-byte aligned)", ws_bytes,
                plan.total_bytes);
  return launch_hessian_bf16(H, diag_key, n, static_cast<const uint16_t*>(X), tokens, ldx, alpha,
                             workspace, plan, s);
}

size_t gptq_prepare_workspace_bytes(int64_t n) {
  if (n <= 0 || n > kPrepareMaxN) return 0;
  return plan_prepare(n).total;
}

gptq_status gptq_prepare_hinv(float* H_inout, const double* diag_key, int64_t n,
                              double damp_percent, int32_t desc_act, int32_t* perm_out,
                              void* workspace, size_t ws_bytes, double* damp_out, void* stream) {
  clear_error();
  if (n < 0) return fail(GPTQ_ERR_INVALID_ARG, "n=%lld", (long long)n);
  if (n == 0) return GPTQ_OK;
  if (n > kPrepareMaxN)
    return fail(GPTQ_ERR_UNSUPPORTED, "n=%lld above %lld", (long long)n, (long long)kPrepareMaxN);
  if (bad_ptr(H_inout, 4)) return fail(GPTQ_ERR_INVALID_ARG, "H_inout is NULL or misaligned");
  if (diag_key && bad_ptr(diag_key, 8)) return fail(GPTQ_ERR_INVALID_ARG, "diag_key misaligned");
  if (bad_ptr(perm_out, 4)) return fail(GPTQ_ERR_INVALID_ARG, "perm_out is NULL or misaligned");
  if (desc_act != 0 && desc_act != 1) return fail(GPTQ_ERR_INVALID_ARG, "desc_act=%d", desc_act);
  if (!std::isfinite(damp_percent) || damp_percent < 0.0)
    return fail(GPTQ_ERR_INVALID_ARG, "damp_percent=%g", (double)damp_percent);
  const PreparePlan plan = plan_prepare(n);
  if (workspace == nullptr || ws_bytes < plan.total || bad_ptr(workspace, 256))
    return fail(GPTQ_ERR_WORKSPACE, "workspace %zu bytes, need %zu (256-byte aligned)", ws_bytes,
                plan.total);
  return run_prepare(H_inout, diag_key, n, damp_percent, desc_act, perm_out, workspace, plan,
                     damp_out, static_cast<hipStream_t>(stream));
}

size_t gptq_quantize_workspace_bytes(int64_t m, int64_t n, const gptq_config* cfg) {
  if (m <= 0 || n <= 0 || n > kPrepareMaxN || check_config(cfg) != GPTQ_OK) {
    clear_error();
    return 0;
  }
  return plan_quantize(m, n, *cfg).total;
}

gptq_status gptq_quantize_layer(const void* W, int32_t w_dtype, int64_t m, int64_t n,
                                const float* U, const int32_t* perm, const gptq_config* cfg,
                                uint32_t* qweight, float* scales, int32_t* zeros, int32_t* g_idx,
                                double* loss, int32_t* status_out, void* workspace, size_t ws_bytes,
                                void* stream) {
  clear_error();
  if (m < 0 || n < 0) return fail(GPTQ_ERR_INVALID_ARG, "m=%lld n=%lld", (long long)m, (long long)n);
  gptq_status st = check_config(cfg);
  if (st != GPTQ_OK) return st;
  if (w_dtype != GPTQ_BF16 && w_dtype != GPTQ_FP32)
    return fail(GPTQ_ERR_UNSUPPORTED, "w_dtype=%d", w_dtype);
  if (m == 0 || n == 0) return GPTQ_OK;
  if (n > kPrepareMaxN)
    return fail(GPTQ_ERR_UNSUPPORTED, "n=%lld above %lld", (long long)n, (long long)kPrepareMaxN);
  if (m > (int64_t)1 << 24) return fail(GPTQ_ERR_UNSUPPORTED, "m=%lld too large", (long long)m);
  if (bad_ptr(W, w_dtype == GPTQ_BF16 ? 2 : 4)) return fail(GPTQ_ERR_INVALID_ARG, "W is NULL or misaligned");
  if (bad_ptr(U, 4)) return fail(GPTQ_ERR_INVALID_ARG, "U is NULL or misaligned");
  if (bad_ptr(perm, 4)) return fail(GPTQ_ERR_INVALID_ARG, "perm is NULL or misaligned");
  if (bad_ptr(qweight, 4) || bad_ptr(scales, 4) || bad_ptr(zeros, 4) || bad_ptr(g_idx, 4))
    return fail(GPTQ_ERR_INVALID_ARG, "an output pointer is NULL or misaligned");
  if (bad_ptr(loss, 8)) return fail(GPTQ_ERR_INVALID_ARG, "loss is NULL or misaligned");
  if (status_out && bad_ptr(status_out, 4)) return fail(GPTQ_ERR_INVALID_ARG, "status_out misaligned");
  const QuantPlan plan = plan_quantize(m, n, *cfg);
  if (workspace == nullptr || ws_bytes < plan.total || bad_ptr(workspace, 256))
    return fail(GPTQ_ERR_WORKSPACE, "workspace %zu bytes, need %zu (256-byte aligned)", ws_bytes,
                plan.total);
  return run_quantize(W, w_dtype, m, n, U, perm, *cfg, qweight, scales, zeros, g_idx, loss,
                      status_out, workspace, plan, static_cast<hipStream_t>(stream));
}

static gptq_status check_rtn_config(const gptq_rtn_config* cfg) {
  if (cfg == nullptr) return fail(GPTQ_ERR_INVALID_ARG, "cfg is NULL");
  if (cfg->bits != 2 && cfg->bits != 3 && cfg->bits != 4 && cfg->bits != 8)
    return fail(GPTQ_ERR_UNSUPPORTED, "bits=%d", cfg->bits);
  if (cfg->group_size != -1 && cfg->group_size < 1)
    return fail(GPTQ_ERR_INVALID_ARG, "group_size=%d", cfg->group_size);
  if (cfg->sym != 0 && cfg->sym != 1) return fail(GPTQ_ERR_INVALID_ARG, "sym=%d", cfg->sym);
  if (!(cfg->clip_ratio > 0.f && cfg->clip_ratio <= 1.f))
    return fail(GPTQ_ERR_INVALID_ARG, "clip_ratio=%g outside (0, 1]", (double)cfg->clip_ratio);
  return GPTQ_OK;
}

size_t gptq_rtn_workspace_bytes(int64_t m, int64_t n, const gptq_rtn_config* cfg) {
  if (m < 0 || n < 0 || cfg == nullptr) return 0;
  return plan_rtn(m, n, cfg->group_size).total;
}

gptq_status gptq_rtn_quantize(const void* W, int32_t w_dtype, int64_t m, int64_t n,
                              const gptq_rtn_config* cfg, uint32_t* qweight, float* scales,
                              int32_t* zeros, double* err, int32_t* status_out, void* workspace,
                              size_t ws_bytes, void* stream) {
  clear_error();
  if (m < 0 || n < 0) return fail(GPTQ_ERR_INVALID_ARG, "m=%lld n=%lld", (long long)m, (long long)n);
  gptq_status st = check_rtn_config(cfg);
  if (st != GPTQ_OK) return st;
  if (w_dtype != GPTQ_BF16 && w_dtype != GPTQ_FP32)
    return fail(GPTQ_ERR_UNSUPPORTED, "w_dtype=%d", w_dtype);
  if (m == 0 || n == 0) return GPTQ_OK;
  if (m > ((int64_t)1 << 31) - 1) return fail(GPTQ_ERR_UNSUPPORTED, "m=%lld too large", (long long)m);
  const RtnPlan plan = plan_rtn(m, n, cfg->group_size);
  if (plan.lds_bytes > kRtnMaxLds)
    return fail(GPTQ_ERR_UNSUPPORTED, "n=%lld with group_size %d needs %zu bytes of LDS per row (max %zu)",
                (long long)n, cfg->group_size, plan.lds_bytes, kRtnMaxLds);
  if (bad_ptr(W, w_dtype == GPTQ_BF16 ? 2 : 4)) return fail(GPTQ_ERR_INVALID_ARG, "W is NULL or misaligned");
  if (bad_ptr(qweight, 4) || bad_ptr(scales, 4) || bad_ptr(zeros, 4))
    return fail(GPTQ_ERR_INVALID_ARG, "an output pointer is NULL or misaligned");
  if (bad_ptr(err, 8)) return fail(GPTQ_ERR_INVALID_ARG, "err is NULL or misaligned");
  if (status_out && bad_ptr(status_out, 4)) return fail(GPTQ_ERR_INVALID_ARG, "status_out misaligned");
  if (workspace == nullptr || ws_bytes < plan.total || bad_ptr(workspace, 256))
    return fail(GPTQ_ERR_WORKSPACE, "workspace %zu bytes, need %zu (256-byte aligned)", ws_bytes,
                plan.total);
  return run_rtn(W, w_dtype, m, n, cfg->bits, cfg->sym, cfg->clip_ratio, qweight, scales, zeros, err,
                 status_out, workspace, plan, static_cast<hipStream_t>(stream));
}

size_t gptq_awq_stats_workspace_bytes(int64_t n, int64_t tokens) {
  if (n < 0 || tokens < 0) return 0;
  return plan_awq_stats(n, tokens).total;
}

gptq_status gptq_awq_channel_stats(const void* X, int32_t x_dtype, int64_t tokens, int64_t ldx,
                                   int64_t n, double* abs_sum, void* workspace, size_t ws_bytes,
                                   void* stream) {
  clear_error();
  if (tokens < 0 || n < 0) return fail(GPTQ_ERR_INVALID_ARG, "tokens=%lld n=%lld", (long long)tokens, (long long)n);
  if (x_dtype != GPTQ_BF16 && x_dtype != GPTQ_FP32) return fail(GPTQ_ERR_UNSUPPORTED, "x_dtype=%d", x_dtype);
  if (tokens == 0 || n == 0) return GPTQ_OK;
  if (ldx < n) return fail(GPTQ_ERR_INVALID_ARG, "ldx=%lld < n=%lld", (long long)ldx, (long long)n);
  if (bad_ptr(X, x_dtype == GPTQ_BF16 ? 2 : 4)) return fail(GPTQ_ERR_INVALID_ARG, "X is NULL or misaligned");
  if (bad_ptr(abs_sum, 8)) return fail(GPTQ_ERR_INVALID_ARG, "abs_sum is NULL or misaligned");
  const AwqStatsPlan p = plan_awq_stats(n, tokens);
  if (workspace == nullptr || ws_bytes < p.total || bad_ptr(workspace, 256))
    return fail(GPTQ_ERR_WORKSPACE, "workspace %zu bytes, need %zu (256-byte aligned)", ws_bytes, p.total);
  return run_awq_stats(X, x_dtype, tokens, ldx, n, abs_sum, workspace, p, static_cast<hipStream_t>(stream));
}

size_t gptq_awq_workspace_bytes(int64_t m, int64_t n, const gptq_rtn_config* cfg) {
  if (m < 0 || n < 0 || cfg == nullptr) return 0;
  return awq_extra_bytes() + plan_rtn(m, n, cfg->group_size).total;
}

gptq_status gptq_awq_quantize(const void* W, int32_t w_dtype, int64_t m, int64_t n,
                              const double* abs_sum, int64_t tokens, float protect,
                              const gptq_rtn_config* cfg, uint32_t* qweight, float* scales,
                              int32_t* zeros, float* channel_scale, double* err, int32_t* status_out,
                              void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  if (m < 0 || n < 0) return fail(GPTQ_ERR_INVALID_ARG, "m=%lld n=%lld", (long long)m, (long long)n);
  gptq_status st = check_rtn_config(cfg);
  if (st != GPTQ_OK) return st;
  if (w_dtype != GPTQ_BF16 && w_dtype != GPTQ_FP32) return fail(GPTQ_ERR_UNSUPPORTED, "w_dtype=%d", w_dtype);
  if (tokens <= 0) return fail(GPTQ_ERR_INVALID_ARG, "tokens=%lld: importance is a mean over tokens", (long long)tokens);
  if (!(protect > 0.f) || !std::isfinite(protect))
    return fail(GPTQ_ERR_INVALID_ARG, "protect=%g must be positive and finite", (double)protect);
  if (m == 0 || n == 0) return GPTQ_OK;
  if (m > ((int64_t)1 << 31) - 1) return fail(GPTQ_ERR_UNSUPPORTED, "m=%lld too large", (long long)m);
  const RtnPlan plan = plan_rtn(m, n, cfg->group_size);
  if (plan.lds_bytes > kRtnMaxLds)
    return fail(GPTQ_ERR_UNSUPPORTED, "n=%lld with group_size %d needs %zu bytes of LDS per row (max %zu)",
                (long long)n, cfg->group_size, plan.lds_bytes, kRtnMaxLds);
  if (bad_ptr(W, w_dtype == GPTQ_BF16 ? 2 : 4)) return fail(GPTQ_ERR_INVALID_ARG, "W is NULL or misaligned");
  if (bad_ptr(abs_sum, 8)) return fail(GPTQ_ERR_INVALID_ARG, "abs_sum is NULL or misaligned");
  if (bad_ptr(qweight, 4) || bad_ptr(scales, 4) || bad_ptr(zeros, 4) || bad_ptr(channel_scale, 4))
    return fail(GPTQ_ERR_INVALID_ARG, "an output pointer is NULL or misaligned");
  if (bad_ptr(err, 8)) return fail(GPTQ_ERR_INVALID_ARG, "err is NULL or misaligned");
  if (status_out && bad_ptr(status_out, 4)) return fail(GPTQ_ERR_INVALID_ARG, "status_out misaligned");
  const size_t need = awq_extra_bytes() + plan.total;
  if (workspace == nullptr || ws_bytes < need || bad_ptr(workspace, 256))
    return fail(GPTQ_ERR_WORKSPACE, "workspace %zu bytes, need %zu (256-byte aligned)", ws_bytes, need);
  return run_awq_quantize(W, w_dtype, m, n, abs_sum, tokens, protect, cfg->bits, cfg->sym, cfg->clip_ratio,
                          qweight, scales, zeros, channel_scale, err, status_out, workspace, plan,
                          static_cast<hipStream_t>(stream));
}

static bool w4_group_ok(int32_t g) { return g == -1 || g == 32 || g == 64 || g == 128; }

size_t gptq_w4a16_packed_bytes(int64_t m, int64_t n, int32_t group_size) {
  if (m < 0 || n < 0 || !w4_group_ok(group_size)) return 0;
  return plan_w4a16(m, n, group_size).total;
}

gptq_status gptq_w4a16_pack(const uint32_t* qweight, const float* scales, const int32_t* zeros,
                            const int32_t* g_idx, int64_t m, int64_t n, int32_t bits,
                            int32_t group_size, void* packed, size_t packed_bytes, void* stream) {
  clear_error();
  if (m < 0 || n < 0) return fail(GPTQ_ERR_INVALID_ARG, "m=%lld n=%lld", (long long)m, (long long)n);
  if (bits != 2 && bits != 3 && bits != 4)
    return fail(GPTQ_ERR_UNSUPPORTED, "bits=%d (the W4A16 product takes 2-, 3- and 4-bit codes)", bits);
  if (!w4_group_ok(group_size))
    return fail(GPTQ_ERR_UNSUPPORTED, "group_size=%d (32, 64, 128 or -1)", group_size);
  if (m == 0 || n == 0) return GPTQ_OK;
  if (m > ((int64_t)1 << 30) || n > ((int64_t)1 << 30))
    return fail(GPTQ_ERR_UNSUPPORTED, "m=%lld n=%lld too large", (long long)m, (long long)n);
  if (bad_ptr(qweight, 4) || bad_ptr(scales, 4) || bad_ptr(zeros, 4) || bad_ptr(g_idx, 4))
    return fail(GPTQ_ERR_INVALID_ARG, "an input pointer is NULL or misaligned");
  const W4Layout L = plan_w4a16(m, n, group_size);
  if (packed == nullptr || packed_bytes < L.total || bad_ptr(packed, 256))
    return fail(GPTQ_ERR_WORKSPACE, "packed buffer %zu bytes, need %zu (256-byte aligned)",
                packed_bytes, L.total);
  return run_w4a16_pack(qweight, scales, zeros, g_idx, bits, L, packed,
                        static_cast<hipStream_t>(stream));
}

int64_t gptq_checkpoint_qweight_rows(int64_t n, int32_t bits) {
  if (n < 0 || !(bits == 2 || bits == 3 || bits == 4 || bits == 8)) return -1;
  return ceil_div(n * bits, 32);
}

int64_t gptq_checkpoint_qzeros_words(int64_t m, int32_t bits) {
  if (m < 0 || !(bits == 2 || bits == 3 || bits == 4 || bits == 8)) return -1;
  return ceil_div(m * bits, 32);
}

gptq_status gptq_export_checkpoint(const uint32_t* qweight, const float* scales, const int32_t* zeros,
                                   int64_t m, int64_t n, int32_t bits, int32_t group_size, int32_t zero_offset,
                                   int32_t* ck_qweight, int32_t* ck_qzeros, uint16_t* ck_scales, void* stream) {
  clear_error();
  if (m < 0 || n < 0) return fail(GPTQ_ERR_INVALID_ARG, "m=%lld n=%lld", (long long)m, (long long)n);
  if (!(bits == 2 || bits == 3 || bits == 4 || bits == 8))
    return fail(GPTQ_ERR_UNSUPPORTED, "bits=%d (2, 3, 4 or 8)", bits);
  if (zero_offset != 0 && zero_offset != 1) return fail(GPTQ_ERR_INVALID_ARG, "zero_offset=%d (0 or 1)", zero_offset);
  const int64_t G = gptq_num_groups(n, group_size);
  if (G < 0) return fail(GPTQ_ERR_INVALID_ARG, "group_size=%d", group_size);
  if (m == 0 || n == 0) return GPTQ_OK;
  if (m > 65535LL * 64 || G > 65535 || n > ((int64_t)1 << 40))
    return fail(GPTQ_ERR_UNSUPPORTED, "m=%lld n=%lld (%lld groups) too large", (long long)m, (long long)n,
                (long long)G);
  if (bad_ptr(qweight, 4) || bad_ptr(scales, 4) || bad_ptr(zeros, 4))
    return fail(GPTQ_ERR_INVALID_ARG, "an input pointer is NULL or misaligned");
  if (bad_ptr(ck_qweight, 4) || bad_ptr(ck_qzeros, 4) || bad_ptr(ck_scales, 2))
    return fail(GPTQ_ERR_INVALID_ARG, "an output pointer is NULL or misaligned");
  return run_checkpoint_export(qweight, scales, zeros, m, n, bits, G, zero_offset, ck_qweight, ck_qzeros,
                               ck_scales, static_cast<hipStream_t>(stream));
}

size_t gptq_w4a16_workspace_bytes(int64_t tokens, int64_t m, int64_t n) {
  if (tokens < 0 || m < 0 || n < 0) return 0;
  return plan_w4a16_gemm(tokens, m, n).total;
}

gptq_status gptq_w4a16_matmul(const void* X, int64_t tokens, int64_t ldx, const void* packed,
                              int64_t m, int64_t n, int32_t group_size, float* Y, int64_t ldy,
                              void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  if (tokens < 0 || m < 0 || n < 0)
    return fail(GPTQ_ERR_INVALID_ARG, "tokens=%lld m=%lld n=%lld", (long long)tokens, (long long)m,
                (long long)n);
  if (!w4_group_ok(group_size))
    return fail(GPTQ_ERR_UNSUPPORTED, "group_size=%d (32, 64, 128 or -1)", group_size);
  if (tokens == 0 || m == 0 || n == 0) return GPTQ_OK;
  if (m > ((int64_t)1 << 30) || n > ((int64_t)1 << 30))
    return fail(GPTQ_ERR_UNSUPPORTED, "m=%lld n=%lld too large", (long long)m, (long long)n);
  if (ldx < n || ldy < m)
    return fail(GPTQ_ERR_INVALID_ARG, "ldx=%lld < n or ldy=%lld < m", (long long)ldx, (long long)ldy);
  if (bad_ptr(X, 2) || bad_ptr(Y, 4)) return fail(GPTQ_ERR_INVALID_ARG, "X or Y is NULL or misaligned");
  if (bad_ptr(packed, 256)) return fail(GPTQ_ERR_INVALID_ARG, "packed is NULL or not 256-byte aligned");
  const W4GemmPlan p = plan_w4a16_gemm(tokens, m, n);
  if (workspace == nullptr || ws_bytes < p.total || bad_ptr(workspace, 256))
    return fail(GPTQ_ERR_WORKSPACE, "workspace %zu bytes, need %zu (256-byte aligned)", ws_bytes, p.total);
  return run_w4a16_matmul(static_cast<const uint16_t*>(X), tokens, ldx, packed,
                          plan_w4a16(m, n, group_size), Y, ldy, workspace, p,
                          static_cast<hipStream_t>(stream));
}

size_t gptq_w4a16_noalloc_scratch_bytes(void) { return w4a16_noalloc_scratch_bytes(); }

gptq_status gptq_w4a16_matmul_noalloc(const void* X, int64_t tokens, int64_t ldx, const void* packed,
                                      int64_t m, int64_t n, int32_t group_size, float* Y, int64_t ldy,
                                      void* stream) {
  clear_error();
  if (tokens < 0 || m < 0 || n < 0)
    return fail(GPTQ_ERR_INVALID_ARG, "tokens=%lld m=%lld n=%lld", (long long)tokens, (long long)m,
                (long long)n);
  if (!w4_group_ok(group_size))
    return fail(GPTQ_ERR_UNSUPPORTED, "group_size=%d (32, 64, 128 or -1)", group_size);
  if (tokens == 0 || m == 0 || n == 0) return GPTQ_OK;
  if (m > ((int64_t)1 << 30) || n > ((int64_t)1 << 30))
    return fail(GPTQ_ERR_UNSUPPORTED, "m=%lld n=%lld too large", (long long)m, (long long)n);
  if (ldx < n || ldy < m)
    return fail(GPTQ_ERR_INVALID_ARG, "ldx=%lld < n or ldy=%lld < m", (long long)ldx, (long long)ldy);
  if (bad_ptr(X, 2) || bad_ptr(Y, 4)) return fail(GPTQ_ERR_INVALID_ARG, "X or Y is NULL or misaligned");
  if (bad_ptr(packed, 256)) return fail(GPTQ_ERR_INVALID_ARG, "packed is NULL or not 256-byte aligned");
  return run_w4a16_matmul_noalloc(static_cast<const uint16_t*>(X), tokens, ldx, packed,
                                  plan_w4a16(m, n, group_size), Y, ldy, static_cast<hipStream_t>(stream));
}

}  // extern "C"
