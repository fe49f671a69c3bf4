// C-ABI entry points of libqsa: argument validation (before anything is
// enqueued), workspace sizing and kernel dispatch.  The operations and their
// sources are documented in include/qsa.h.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <cmath>
#include <mutex>

#include "qsa_common.h"

// Step workspace of qsa_decode_step_noalloc: one copy per device, held
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory; the device address comes from hipGetSymbolAddress.
static constexpr size_t kNoAllocScratchBytes = size_t{32} << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

thread_local char g_err[512] = "";

qsa_status fail(qsa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

qsa_status ok() {
  g_err[0] = '\0';
  return QSA_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool aligned16(const void* p) { return aligned(p, 16); }

// Required pointer with its alignment: 16 for tensors read with 16-byte
// vector loads, 8 or 4 for the rest.
#define QSA_REQUIRE_PTR(p, a)                                                            \
  do {                                                                                   \
    if (!(p)) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: %s must not be NULL", fn, #p); \
    if (!aligned((p), (a)))                                                              \
      return fail(QSA_ERR_INVALID_ARGUMENT, "%s: %s must be %d-byte aligned", fn, #p,   \
                  (int)(a));                                                             \
  } while (0)

// Validates the configuration and fills the kernel-side dimensions.
qsa_status check_config(const char* fn, const qsa_config* cfg, qsa::Dims* d) {
  if (!cfg) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: cfg must not be NULL", fn);
  if (cfg->block_size <= 0 || cfg->token_budget <= 0 || cfg->idx_heads <= 0 ||
      cfg->idx_dim <= 0 || cfg->rope_dims < 0 || cfg->q_heads <= 0 || cfg->kv_heads <= 0 ||
      cfg->head_dim <= 0)
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: sizes in cfg must be positive", fn);
  if (cfg->dtype != QSA_F32 && cfg->dtype != QSA_BF16)
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: unknown dtype %d", fn, cfg->dtype);
  if (cfg->q_heads % cfg->kv_heads != 0)
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: q_heads (%d) must be a multiple of kv_heads (%d)",
                fn, cfg->q_heads, cfg->kv_heads);
  if (!(cfg->rope_base > 0.0) || !std::isfinite(cfg->rope_base))
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: rope_base must be positive", fn);
  if (!(cfg->rms_eps >= 0.0f))
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: rms_eps must be >= 0", fn);
  if (cfg->block_size > 128 || (cfg->block_size & (cfg->block_size - 1)))
    return fail(QSA_ERR_UNSUPPORTED, "%s: block_size %d (a power of two from 1 to 128)", fn,
                cfg->block_size);
  if (cfg->idx_dim != 128)
    return fail(QSA_ERR_UNSUPPORTED, "%s: idx_dim %d (only 128 is built)", fn, cfg->idx_dim);
  if (cfg->idx_heads > 16)
    return fail(QSA_ERR_UNSUPPORTED, "%s: idx_heads %d (at most 16)", fn, cfg->idx_heads);
  if (cfg->rope_dims % 4 != 0 || cfg->rope_dims > cfg->idx_dim)
    return fail(QSA_ERR_UNSUPPORTED, "%s: rope_dims %d (a multiple of 4 up to idx_dim)", fn,
                cfg->rope_dims);
  if (cfg->head_dim != 64 && cfg->head_dim != 128)
    return fail(QSA_ERR_UNSUPPORTED, "%s: head_dim %d (64 or 128)", fn, cfg->head_dim);
  if (cfg->q_heads > 64)
    return fail(QSA_ERR_UNSUPPORTED, "%s: q_heads %d (at most 64)", fn, cfg->q_heads);
  const int kB = (cfg->token_budget + cfg->block_size - 1) / cfg->block_size;
  if (kB > 512 && cfg->block_size >= 4)
    return fail(QSA_ERR_UNSUPPORTED, "%s: k_B = ceil(K/r) = %d (at most 512 for r >= 4)", fn,
                kB);
  if ((int64_t)kB * cfg->block_size > 2048)
    return fail(QSA_ERR_UNSUPPORTED, "%s: k_B * r = %lld selected tokens (at most 2048)", fn,
                (long long)kB * cfg->block_size);
  d->r = cfg->block_size;
  d->lr = __builtin_ctz((unsigned)cfg->block_size);
  d->kB = kB;
  d->idx_heads = cfg->idx_heads;
  d->idx_dim = cfg->idx_dim;
  d->rope_dims = cfg->rope_dims;
  d->q_heads = cfg->q_heads;
  d->kv_heads = cfg->kv_heads;
  d->head_dim = cfg->head_dim;
  d->bf16 = cfg->dtype == QSA_BF16;
  d->eps = cfg->rms_eps;
  d->scale = cfg->softmax_scale > 0.0f ? cfg->softmax_scale
                                       : (float)(1.0 / std::sqrt((double)cfg->head_dim));
  d->base = cfg->rope_base;
  return QSA_OK;
}

qsa_status check_sizes(const char* fn, int32_t batch, int32_t n_q, int64_t cap_tokens,
                       int32_t max_pos_end) {
  if (batch <= 0) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: batch must be > 0", fn);
  if (n_q <= 0) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: n_q must be > 0", fn);
  if (cap_tokens < 4)
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: cap_tokens must be >= block_size", fn);
  if (max_pos_end <= 0 || (int64_t)max_pos_end > cap_tokens)
    return fail(QSA_ERR_INVALID_ARGUMENT,
                "%s: max_pos_end %d must be in [1, cap_tokens=%lld]", fn, max_pos_end,
                (long long)cap_tokens);
  if ((int64_t)batch * n_q > (int64_t)INT32_MAX / 16)
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: batch * n_q too large", fn);
  return QSA_OK;
}

size_t select_ws(const qsa::Dims& d, int32_t batch, int32_t n_q, int32_t max_pos_end) {
  return qsa::select_plan(d, batch, n_q, max_pos_end).bytes;
}

qsa_status launched(const char* fn, hipError_t e) {
  if (e != hipSuccess)
    return fail(QSA_ERR_DEVICE, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of scratch, per device
bool g_scratch_cleared[kMaxDevices];

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// The current device's scratch address; *first is true on the first call
// for that device (the caller then clears the control area).
qsa_status scratch_for_current_device(const char* fn, void** ptr, bool* first) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return fail(QSA_ERR_DEVICE, "%s: no usable current device", fn);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(QSA_ERR_DEVICE, "%s: hipGetSymbolAddress(scratch) failed: %s", fn,
                  hipGetErrorString(e));
    }
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  *first = !g_scratch_cleared[dev];
  g_scratch_cleared[dev] = true;
  return QSA_OK;
}

}  // namespace

extern "C" {

int32_t qsa_abi_version(void) { return 2; }

const char* qsa_last_error(void) { return g_err; }

const char* qsa_status_string(qsa_status st) {
  switch (st) {
    case QSA_OK: return "QSA_OK";
    case QSA_ERR_INVALID_ARGUMENT: return "QSA_ERR_INVALID_ARGUMENT";
    case QSA_ERR_UNSUPPORTED: return "QSA_ERR_UNSUPPORTED";
    case QSA_ERR_WORKSPACE: return "QSA_ERR_WORKSPACE";
    case QSA_ERR_DEVICE: return "QSA_ERR_DEVICE";
  }
  return "QSA_UNKNOWN_STATUS";
}

qsa_status qsa_workspace_size(const qsa_config* cfg, int32_t op, int32_t batch, int32_t n_q,
                              int32_t max_pos_end, size_t* bytes) {
  const char* fn = "qsa_workspace_size";
  qsa::Dims d;
  qsa_status st = check_config(fn, cfg, &d);
  if (st != QSA_OK) return st;
  if (!bytes) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: bytes must not be NULL", fn);
  if (batch <= 0 || n_q <= 0 || max_pos_end <= 0)
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: batch, n_q and max_pos_end must be > 0", fn);
  if (d.r < 4 && (op == QSA_OP_BACKWARD || op == QSA_OP_DISTILL || op == QSA_OP_DECODE_STEP))
    return fail(QSA_ERR_UNSUPPORTED, "%s: op %d needs block_size >= 4", fn, op);
  switch (op) {
    case QSA_OP_INDEX_BUILD: *bytes = 0; break;
    case QSA_OP_SELECT: *bytes = select_ws(d, batch, n_q, max_pos_end); break;
    case QSA_OP_PREFILL: *bytes = qsa::attn_workspace_bytes(d, batch, n_q, false); break;
    case QSA_OP_DECODE: *bytes = qsa::attn_workspace_bytes(d, batch, 1, true); break;
    case QSA_OP_DECODE_STEP: *bytes = qsa::step_plan(d, batch, max_pos_end).bytes; break;
    case QSA_OP_BACKWARD: *bytes = qsa::bwd_workspace_bytes(d, batch, n_q, max_pos_end); break;
    case QSA_OP_DISTILL: *bytes = qsa::distill_workspace_bytes(d, batch, n_q, max_pos_end); break;
    default: return fail(QSA_ERR_INVALID_ARGUMENT, "%s: unknown op %d", fn, op);
  }
  return ok();
}

qsa_status qsa_index_build(const qsa_config* cfg, int32_t batch, const void* k_idx,
                           int64_t cap_tokens, const int32_t* len_before,
                           const int32_t* len_after, int32_t max_new_blocks,
                           const float* rms_gain, void* k_cmp, hipStream_t stream) {
  const char* fn = "qsa_index_build";
  qsa::Dims d;
  qsa_status st = check_config(fn, cfg, &d);
  if (st != QSA_OK) return st;
  if (batch <= 0) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: batch must be > 0", fn);
  if (cap_tokens < 4)
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: cap_tokens must be >= block_size", fn);
  if (max_new_blocks < 0)
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: max_new_blocks must be >= 0", fn);
  QSA_REQUIRE_PTR(k_idx, 8);
  QSA_REQUIRE_PTR(len_before, 4);
  QSA_REQUIRE_PTR(len_after, 4);
  QSA_REQUIRE_PTR(k_cmp, 8);
  if (rms_gain && !aligned(rms_gain, 8))
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: rms_gain must be 8-byte aligned", fn);
  return launched(fn, qsa::launch_compress(d, batch, k_idx, cap_tokens, len_before, len_after,
                                           max_new_blocks, rms_gain, k_cmp, stream));
}

qsa_status qsa_index_build_backward(const qsa_config* cfg, int32_t batch, const void* k_idx,
                                    int64_t cap_tokens, const int32_t* len_before,
                                    const int32_t* len_after, int32_t max_new_blocks,
                                    const float* rms_gain, const float* dk_cmp, float* dk_idx,
                                    hipStream_t stream) {
  const char* fn = "qsa_index_build_backward";
  qsa::Dims d;
  qsa_status st = check_config(fn, cfg, &d);
  if (st != QSA_OK) return st;
  if (batch <= 0 || batch > 65535)
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: batch must be in [1, 65535]", fn);
  if (cap_tokens < d.r)
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: cap_tokens must be >= block_size", fn);
  if (max_new_blocks < 0)
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: max_new_blocks must be >= 0", fn);
  QSA_REQUIRE_PTR(k_idx, 8);
  QSA_REQUIRE_PTR(len_before, 4);
  QSA_REQUIRE_PTR(len_after, 4);
  QSA_REQUIRE_PTR(dk_cmp, 8);
  QSA_REQUIRE_PTR(dk_idx, 8);
  if (rms_gain && !aligned(rms_gain, 8))
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: rms_gain must be 8-byte aligned", fn);
  return launched(fn, qsa::launch_compress_backward(d, batch, k_idx, cap_tokens, len_before,
                                                    len_after, max_new_blocks, rms_gain, dk_cmp,
                                                    dk_idx, stream));
}

qsa_status qsa_select_topk(const qsa_config* cfg, int32_t batch, int32_t n_q,
                           const void* q_idx, const int32_t* q_pos0, int32_t max_pos_end,
                           const void* k_cmp, int64_t cap_tokens, int32_t* sel_blocks,
                           int32_t* sel_count, float* sel_scores, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "qsa_select_topk";
  qsa::Dims d;
  qsa_status st = check_config(fn, cfg, &d);
  if (st != QSA_OK) return st;
  st = check_sizes(fn, batch, n_q, cap_tokens, max_pos_end);
  if (st != QSA_OK) return st;
  QSA_REQUIRE_PTR(q_idx, 16);
  QSA_REQUIRE_PTR(q_pos0, 4);
  QSA_REQUIRE_PTR(k_cmp, 16);
  QSA_REQUIRE_PTR(sel_blocks, 4);
  QSA_REQUIRE_PTR(sel_count, 4);
  if (sel_scores && !aligned(sel_scores, 4))
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: sel_scores must be 4-byte aligned", fn);
  const size_t need = select_ws(d, batch, n_q, max_pos_end);
  if (!workspace || workspace_bytes < need)
    return fail(QSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace))
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: workspace must be 16-byte aligned", fn);
  const qsa::SelectPlan pl = qsa::select_plan(d, batch, n_q, max_pos_end);
  if (pl.kernel == 1 && pl.W >= (int64_t{1} << 26))  // 32-bit offsets within a 64-row tile
    return fail(QSA_ERR_UNSUPPORTED, "%s: max_pos_end %d is beyond the scoring kernel's range", fn,
                max_pos_end);
  hipError_t e = qsa::launch_score(d, pl, batch, n_q, q_idx, q_pos0, k_cmp, cap_tokens,
                                   workspace, stream);
  if (e == hipSuccess)
    e = qsa::launch_select(d, pl, batch, n_q, q_pos0, cap_tokens, workspace, sel_blocks,
                           sel_count, sel_scores, q_idx, k_cmp, stream);
  return launched(fn, e);
}

static qsa_status attn_common(const char* fn, const qsa_config* cfg, int32_t batch, int32_t n_q,
                              const void* q, const void* k_cache, const void* v_cache,
                              int64_t cap_tokens, const int32_t* q_pos0, int32_t max_pos_end,
                              const int32_t* sel_blocks, const int32_t* sel_count, void* out,
                              float* lse, void* workspace, size_t workspace_bytes, bool decode,
                              hipStream_t stream) {
  qsa::Dims d;
  qsa_status st = check_config(fn, cfg, &d);
  if (st != QSA_OK) return st;
  st = check_sizes(fn, batch, n_q, cap_tokens, max_pos_end);
  if (st != QSA_OK) return st;
  QSA_REQUIRE_PTR(q, 16);
  QSA_REQUIRE_PTR(k_cache, 16);
  QSA_REQUIRE_PTR(v_cache, 16);
  QSA_REQUIRE_PTR(q_pos0, 4);
  QSA_REQUIRE_PTR(sel_blocks, 4);
  QSA_REQUIRE_PTR(sel_count, 4);
  QSA_REQUIRE_PTR(out, 4);
  if (lse && !aligned(lse, 4))
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: lse must be 4-byte aligned", fn);
  const size_t need = qsa::attn_workspace_bytes(d, batch, n_q, decode);
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(QSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace))
      return fail(QSA_ERR_INVALID_ARGUMENT, "%s: workspace must be 16-byte aligned", fn);
  }
  return launched(fn, qsa::launch_attn(d, batch, n_q, q, k_cache, v_cache, cap_tokens, q_pos0,
                                       sel_blocks, sel_count, out, lse, workspace, decode,
                                       stream));
}

qsa_status qsa_sparse_attn_prefill(const qsa_config* cfg, int32_t batch, int32_t n_q,
                                   const void* q, const void* k_cache, const void* v_cache,
                                   int64_t cap_tokens, const int32_t* q_pos0,
                                   int32_t max_pos_end, const int32_t* sel_blocks,
                                   const int32_t* sel_count, void* out, float* lse,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return attn_common("qsa_sparse_attn_prefill", cfg, batch, n_q, q, k_cache, v_cache, cap_tokens,
                     q_pos0, max_pos_end, sel_blocks, sel_count, out, lse, workspace,
                     workspace_bytes, false, stream);
}

qsa_status qsa_sparse_attn_decode(const qsa_config* cfg, int32_t batch, const void* q,
                                  const void* k_cache, const void* v_cache, int64_t cap_tokens,
                                  const int32_t* q_pos, int32_t max_pos_end,
                                  const int32_t* sel_blocks, const int32_t* sel_count,
                                  void* out, float* lse, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  return attn_common("qsa_sparse_attn_decode", cfg, batch, 1, q, k_cache, v_cache, cap_tokens,
                     q_pos, max_pos_end, sel_blocks, sel_count, out, lse, workspace,
                     workspace_bytes, true, stream);
}

qsa_status qsa_sparse_attn_backward(const qsa_config* cfg, int32_t batch, int32_t n_q,
                                    const void* q, const void* k_cache, const void* v_cache,
                                    int64_t cap_tokens, const int32_t* q_pos0,
                                    int32_t max_pos_end, const int32_t* sel_blocks,
                                    const int32_t* sel_count, const void* out, const float* lse,
                                    const void* dout, void* dq, float* dk, float* dv,
                                    void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  const char* fn = "qsa_sparse_attn_backward";
  qsa::Dims d;
  qsa_status st = check_config(fn, cfg, &d);
  if (st != QSA_OK) return st;
  st = check_sizes(fn, batch, n_q, cap_tokens, max_pos_end);
  if (st != QSA_OK) return st;
  if (d.kv_heads > 2)
    return fail(QSA_ERR_UNSUPPORTED, "%s: kv_heads %d (at most 2)", fn, d.kv_heads);
  if (d.r < 4)
    return fail(QSA_ERR_UNSUPPORTED, "%s: block_size %d (the key side works on 4-token units: "
                "r >= 4)", fn, d.r);
  QSA_REQUIRE_PTR(q, 16);
  QSA_REQUIRE_PTR(k_cache, 16);
  QSA_REQUIRE_PTR(v_cache, 16);
  QSA_REQUIRE_PTR(q_pos0, 4);
  QSA_REQUIRE_PTR(sel_blocks, 4);
  QSA_REQUIRE_PTR(sel_count, 4);
  QSA_REQUIRE_PTR(out, 4);
  QSA_REQUIRE_PTR(lse, 4);
  QSA_REQUIRE_PTR(dout, 4);
  QSA_REQUIRE_PTR(dq, 4);
  QSA_REQUIRE_PTR(dk, 4);
  QSA_REQUIRE_PTR(dv, 4);
  const size_t need = qsa::bwd_workspace_bytes(d, batch, n_q, max_pos_end);
  if (!workspace || workspace_bytes < need)
    return fail(QSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace))
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: workspace must be 16-byte aligned", fn);
  return launched(fn, qsa::launch_attn_backward(d, batch, n_q, q, k_cache, v_cache, cap_tokens,
                                                q_pos0, max_pos_end, sel_blocks, sel_count, out,
                                                lse, dout, dq, dk, dv, workspace, stream));
}

// Validation shared by qsa_decode_step and qsa_decode_step_noalloc: every
// argument but the workspace.  Fills the kernel dimensions and the plan.
static qsa_status step_validate(const char* fn, const qsa_config* cfg, int32_t batch,
                                const void* q_idx, const void* q, const void* k_idx,
                                const void* k_cmp, const float* rms_gain, const void* k_cache,
                                const void* v_cache, int64_t cap_tokens, const int32_t* q_pos,
                                int32_t max_pos_end, const int32_t* sel_blocks,
                                const int32_t* sel_count, const float* sel_scores,
                                const void* out, const float* lse, qsa::Dims* dp,
                                qsa::StepPlan* plan) {
  qsa::Dims& d = *dp;
  qsa_status st = check_config(fn, cfg, &d);
  if (st != QSA_OK) return st;
  st = check_sizes(fn, batch, 1, cap_tokens, max_pos_end);
  if (st != QSA_OK) return st;
  if (!qsa::decode_step_layout_ok(d))
    return fail(QSA_ERR_UNSUPPORTED,
                "%s: needs bf16, block_size 4, idx_heads 4 and 16 query heads with (kv_heads, "
                "head_dim) in {(2,128), (2,64), (1,128)}",
                fn);
  if (batch > qsa::kStepMaxBatch)
    return fail(QSA_ERR_UNSUPPORTED, "%s: batch %d (at most %d)", fn, batch, qsa::kStepMaxBatch);
  if ((int64_t)(max_pos_end - 1) / d.r > qsa::kStepMaxBlocks)
    return fail(QSA_ERR_UNSUPPORTED, "%s: max_pos_end %d (at most %lld candidate blocks)", fn,
                max_pos_end, (long long)qsa::kStepMaxBlocks);
  QSA_REQUIRE_PTR(q_idx, 16);
  QSA_REQUIRE_PTR(q, 16);
  QSA_REQUIRE_PTR(k_idx, 8);
  QSA_REQUIRE_PTR(k_cmp, 16);
  QSA_REQUIRE_PTR(k_cache, 16);
  QSA_REQUIRE_PTR(v_cache, 16);
  QSA_REQUIRE_PTR(q_pos, 4);
  QSA_REQUIRE_PTR(sel_blocks, 4);
  QSA_REQUIRE_PTR(sel_count, 4);
  QSA_REQUIRE_PTR(out, 4);
  if (rms_gain && !aligned(rms_gain, 8))
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: rms_gain must be 8-byte aligned", fn);
  if (sel_scores && !aligned(sel_scores, 4))
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: sel_scores must be 4-byte aligned", fn);
  if (lse && !aligned(lse, 4))
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: lse must be 4-byte aligned", fn);
  *plan = qsa::step_plan(d, batch, max_pos_end);
  return QSA_OK;
}

qsa_status qsa_decode_step(const qsa_config* cfg, int32_t batch, const void* q_idx,
                           const void* q, const void* k_idx, void* k_cmp,
                           const float* rms_gain, const void* k_cache, const void* v_cache,
                           int64_t cap_tokens, const int32_t* q_pos, int32_t max_pos_end,
                           int32_t* sel_blocks, int32_t* sel_count, float* sel_scores,
                           void* out, float* lse, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  const char* fn = "qsa_decode_step";
  qsa::Dims d;
  qsa::StepPlan pl;
  qsa_status st = step_validate(fn, cfg, batch, q_idx, q, k_idx, k_cmp, rms_gain, k_cache,
                                v_cache, cap_tokens, q_pos, max_pos_end, sel_blocks, sel_count,
                                sel_scores, out, lse, &d, &pl);
  if (st != QSA_OK) return st;
  if (!workspace || workspace_bytes < pl.bytes)
    return fail(QSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, pl.bytes,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace))
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: workspace must be 16-byte aligned", fn);
  return launched(fn, qsa::launch_decode_step(d, pl, batch, q_idx, q, k_idx, k_cmp, rms_gain,
                                              k_cache, v_cache, cap_tokens, q_pos, sel_blocks,
                                              sel_count, sel_scores, out, lse, workspace,
                                              stream));
}

qsa_status qsa_indexer_distill(const qsa_config* cfg, int32_t batch, int32_t n_q, const void* q,
                               const void* k_cache, int64_t cap_tokens, const int32_t* q_pos0,
                               int32_t max_pos_end, const void* q_idx, const void* k_cmp,
                               float* loss, float* dq_idx, float* dk_cmp, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "qsa_indexer_distill";
  qsa::Dims d;
  qsa_status st = check_config(fn, cfg, &d);
  if (st != QSA_OK) return st;
  st = check_sizes(fn, batch, n_q, cap_tokens, max_pos_end);
  if (st != QSA_OK) return st;
  if (d.kv_heads > 2 || d.q_heads > 16 || d.head_dim > 128 || d.head_dim % 8 != 0)
    return fail(QSA_ERR_UNSUPPORTED,
                "%s: q_heads <= 16, kv_heads <= 2 and head_dim a multiple of 8 up to 128 are "
                "built (got %d, %d, %d)", fn, d.q_heads, d.kv_heads, d.head_dim);
  if (d.idx_heads > 8)
    return fail(QSA_ERR_UNSUPPORTED, "%s: idx_heads %d (at most 8)", fn, d.idx_heads);
  if (d.r < 4)
    return fail(QSA_ERR_UNSUPPORTED, "%s: block_size %d (the teacher's maximum is kept per "
                "4-token unit: r >= 4)", fn, d.r);
  QSA_REQUIRE_PTR(q, 16);
  QSA_REQUIRE_PTR(k_cache, 16);
  QSA_REQUIRE_PTR(q_pos0, 4);
  QSA_REQUIRE_PTR(q_idx, 16);
  QSA_REQUIRE_PTR(k_cmp, 16);
  QSA_REQUIRE_PTR(loss, 4);
  QSA_REQUIRE_PTR(dq_idx, 8);
  QSA_REQUIRE_PTR(dk_cmp, 8);
  const size_t need = qsa::distill_workspace_bytes(d, batch, n_q, max_pos_end);
  if (!workspace || workspace_bytes < need)
    return fail(QSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace_bytes);
  if (!aligned16(workspace))
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: workspace must be 16-byte aligned", fn);
  return launched(fn, qsa::launch_distill(d, batch, n_q, q, k_cache, cap_tokens, q_pos0,
                                          max_pos_end, q_idx, k_cmp, loss, dq_idx, dk_cmp,
                                          workspace, stream));
}

qsa_status qsa_offload_stage(const qsa_config* cfg, int32_t batch, const int32_t* q_pos,
                             const int32_t* sel_blocks, const int32_t* sel_count,
                             const void* k_host, const void* v_host, int64_t cap_tokens,
                             void* hot_k, void* hot_v, int32_t* hot_tag, int32_t hot_units,
                             void* stage_k, void* stage_v, int64_t stage_tokens,
                             int32_t* stage_sel, int32_t* stage_cnt, int32_t* stage_pos,
                             int32_t* stats, hipStream_t stream) {
  const char* fn = "qsa_offload_stage";
  qsa::Dims d;
  qsa_status st = check_config(fn, cfg, &d);
  if (st != QSA_OK) return st;
  if (!d.bf16) return fail(QSA_ERR_UNSUPPORTED, "%s: bf16 caches only", fn);
  if (d.r < 4)
    return fail(QSA_ERR_UNSUPPORTED, "%s: block_size %d (4-token units: r >= 4)", fn, d.r);
  if (batch <= 0 || batch > 65535)
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: batch must be in [1, 65535]", fn);
  if (cap_tokens < d.r || cap_tokens > INT32_MAX)
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: cap_tokens must be in [block_size, 2^31)", fn);
  if (hot_units <= 0) return fail(QSA_ERR_INVALID_ARGUMENT, "%s: hot_units must be > 0", fn);
  if (stage_tokens < (int64_t)(d.kB + 1) * d.r)
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: stage_tokens %lld < (k_B + 1) * block_size = %lld",
                fn, (long long)stage_tokens, (long long)(d.kB + 1) * d.r);
  if ((d.kv_heads * d.head_dim) % 8 != 0)
    return fail(QSA_ERR_UNSUPPORTED, "%s: kv_heads * head_dim must be a multiple of 8", fn);
  QSA_REQUIRE_PTR(q_pos, 4);
  QSA_REQUIRE_PTR(sel_blocks, 4);
  QSA_REQUIRE_PTR(sel_count, 4);
  QSA_REQUIRE_PTR(k_host, 16);
  QSA_REQUIRE_PTR(v_host, 16);
  QSA_REQUIRE_PTR(hot_k, 16);
  QSA_REQUIRE_PTR(hot_v, 16);
  QSA_REQUIRE_PTR(hot_tag, 4);
  QSA_REQUIRE_PTR(stage_k, 16);
  QSA_REQUIRE_PTR(stage_v, 16);
  QSA_REQUIRE_PTR(stage_sel, 4);
  QSA_REQUIRE_PTR(stage_cnt, 4);
  QSA_REQUIRE_PTR(stage_pos, 4);
  QSA_REQUIRE_PTR(stats, 4);
  // the host caches must be pinned, device-mapped host memory
  void* kd = nullptr;
  void* vd = nullptr;
  if (hipHostGetDevicePointer(&kd, const_cast<void*>(k_host), 0) != hipSuccess || !kd ||
      hipHostGetDevicePointer(&vd, const_cast<void*>(v_host), 0) != hipSuccess || !vd) {
    (void)hipGetLastError();
    return fail(QSA_ERR_INVALID_ARGUMENT,
                "%s: k_host / v_host must be pinned host memory (hipHostMalloc)", fn);
  }
  return launched(fn, qsa::launch_offload_stage(d, batch, q_pos, sel_blocks, sel_count, kd, vd,
                                                cap_tokens, hot_k, hot_v, hot_tag, hot_units,
                                                stage_k, stage_v, stage_tokens, stage_sel,
                                                stage_cnt, stage_pos, stats, stream));
}

// qsa_decode_step_noalloc: qsa_decode_step with its workspace in the
// library's own device memory, for callers that cannot allocate.  The
// workspace is `scratch`, a file-scope device array; its device address is
// looked up once per device (hipGetSymbolAddress with that device current)
// and only that address is handed to kernels.  The first call on a device
// also enqueues, on its stream, a clear of the control area the fused step
// expects to find zero before its first call; later calls keep their state
// there.
qsa_status qsa_decode_step_noalloc(const qsa_config* cfg, int32_t batch, const void* q_idx,
                                   const void* q, const void* k_idx, void* k_cmp,
                                   const float* rms_gain, const void* k_cache,
                                   const void* v_cache, int64_t cap_tokens, const int32_t* q_pos,
                                   int32_t max_pos_end, int32_t* sel_blocks, int32_t* sel_count,
                                   float* sel_scores, void* out, float* lse, hipStream_t stream) {
  const char* fn = "qsa_decode_step_noalloc";
  qsa::Dims d;
  qsa::StepPlan pl;
  qsa_status st = step_validate(fn, cfg, batch, q_idx, q, k_idx, k_cmp, rms_gain, k_cache,
                                v_cache, cap_tokens, q_pos, max_pos_end, sel_blocks, sel_count,
                                sel_scores, out, lse, &d, &pl);
  if (st != QSA_OK) return st;
  if (pl.bytes > kNoAllocScratchBytes)
    return fail(QSA_ERR_UNSUPPORTED,
                "%s: these sizes need %zu bytes of step workspace, beyond the library's "
                "%zu-byte scratch (use qsa_decode_step with a workspace)",
                fn, pl.bytes, kNoAllocScratchBytes);
  void* ws = nullptr;
  bool first = false;
  st = scratch_for_current_device(fn, &ws, &first);
  if (st != QSA_OK) return st;
  if (first) {
    hipLaunchKernelGGL(zero_words_kernel, dim3(256), dim3(256), 0, stream,
                       static_cast<uint32_t*>(ws), qsa::kStepCtlBytes / 4);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return launched(fn, e);
  }
  return launched(fn, qsa::launch_decode_step(d, pl, batch, q_idx, q, k_idx, k_cmp, rms_gain,
                                              k_cache, v_cache, cap_tokens, q_pos, sel_blocks,
                                              sel_count, sel_scores, out, lse, ws, stream));
}

}  // extern "C"
