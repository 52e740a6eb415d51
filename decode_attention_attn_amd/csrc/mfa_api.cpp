// C ABI of libmfa: argument validation, workspace sizing and dispatch to the
// HIP kernels. Every check that can be made on the host runs before the first
// HIP call, so invalid calls fail the same way on a machine without a GPU.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <atomic>

#include "../../include/mfa.h"
#include "mfa_internal.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned_n(const void* p, uintptr_t n) { return ((uintptr_t)p & (n - 1)) == 0; }

thread_local int g_last_hip_error = 0;

// HIP failures map to MFA_ERR_HIP; the HIP code is kept for mfa_last_hip_error()
// and printed when MFA_DEBUG is set.
int hip_status(hipError_t e) {
  if (e == hipSuccess) return MFA_OK;
  g_last_hip_error = (int)e;
  if (getenv("MFA_DEBUG")) fprintf(stderr, "libmfa: HIP error %d: %s\n", (int)e, hipGetErrorString(e));
  return MFA_ERR_HIP;
}

// Compute units of the current device (cached per device).
int current_cu_count(int* status) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) {
    *status = hip_status(e != hipSuccess ? e : hipErrorInvalidDevice);
    return 0;
  }
  if (dev < kMaxDevices) {
    const int c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess || cus <= 0) {
    *status = hip_status(e != hipSuccess ? e : hipErrorInvalidDevice);
    return 0;
  }
  if (dev < kMaxDevices) g_cu_count[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

bool act_dtype_ok(mfa_dtype dt) { return dt == MFA_F32 || dt == MFA_BF16; }

// Compute units a call's projection plans are made for: the device's, at
// most mfa::kPlanCus. Workspace sizes need no device: they reserve the
// partial-sum bytes that bound the plan of every CU count up to kPlanCus
// (mfa::gemm_partial_bound), and each call checks its own plan against that.
int plan_cus(int* status) {
  const int c = current_cu_count(status);
  return c < mfa::kPlanCus ? c : mfa::kPlanCus;
}


}  // namespace

extern "C" {

int mfa_version(void) { return 10000 * 1 + 100 * 0 + 0; }

int mfa_last_hip_error(void) { return g_last_hip_error; }

const char* mfa_status_string(int status) {
  switch (status) {
    case MFA_OK: return "MFA_OK";
    case MFA_ERR_INVALID_ARG: return "MFA_ERR_INVALID_ARG: null pointer or size out of range";
    case MFA_ERR_UNSUPPORTED: return "MFA_ERR_UNSUPPORTED: dtype combination not provided";
    case MFA_ERR_ALIGNMENT: return "MFA_ERR_ALIGNMENT: pointer not suitably aligned";
    case MFA_ERR_WORKSPACE: return "MFA_ERR_WORKSPACE: workspace missing or too small";
    case MFA_ERR_HIP: return "MFA_ERR_HIP: HIP runtime call or kernel launch failed";
    default: return "unknown libmfa status";
  }
}

// ------------------------------------------------------------------ q path
// Workspace: partial sums (those of the down-projection, later reused by the
// up-projection's), then the normalized latent c_hat (mfa::qproj_layout).
size_t mfa_qproj_workspace_size(int B, mfa_dtype dt) {
  if (B < 1 || B > MFA_MAX_BATCH || !act_dtype_ok(dt)) return 0;
  return mfa::qproj_layout(B, dt == MFA_BF16).total;
}

// The device's plans of the q path, checked against the reserved region
// (a failed check would be a planning bug: it is reported, never run).
static int qproj_plans(int B, bool bf, bool w8, mfa::GemmPlan* dn, mfa::GemmPlan* up, mfa::QprojLayout* l) {
  int st = MFA_OK;
  const int cus = plan_cus(&st);
  if (st != MFA_OK) return st;
  *dn = mfa::plan_gemm(bf, B, MFA_RANK, MFA_HIDDEN, MFA_RANK, cus, w8);
  *up = mfa::plan_gemm(bf, B, MFA_QDIM, MFA_RANK, MFA_QDIM, cus, w8);
  *l = mfa::qproj_layout(B, bf);
  return mfa::qproj_part_need(B, bf, *dn, *up) <= l->part_bytes ? MFA_OK : MFA_ERR_WORKSPACE;
}

static int qproj_run(const void* x, const void* w_dq, const float* s_dq, const float* gamma, float eps,
                     const void* w_uq, const float* s_uq, void* q_out, void* ws, int B, bool bf, hipStream_t s) {
  mfa::GemmPlan plan, up;
  mfa::QprojLayout l;
  const int st = qproj_plans(B, bf, s_dq != nullptr, &plan, &up, &l);
  if (st != MFA_OK) return st;
  float* part = (float*)ws;
  void* chat = (char*)ws + l.chat_offset;
  hipError_t e = mfa::launch_gemm(bf, plan, x, w_dq, w_dq, part, mfa::GemmOut::Partial, s, s_dq, s_dq);
  if (e != hipSuccess) return hip_status(e);
  e = mfa::launch_rmsnorm_reduce(bf, part, bf ? plan.splits : 1, B, MFA_RANK, gamma, eps, chat, s);
  if (e != hipSuccess) return hip_status(e);
  if (bf && up.splits > 1) {
    // the down-projection's partials were consumed by the reduce above
    e = mfa::launch_gemm(true, up, chat, w_uq, w_uq, part, mfa::GemmOut::Partial, s, s_uq, s_uq);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(mfa::launch_sum_reduce(true, part, up.splits, B, MFA_QDIM, q_out, s, up.tile_n));
  }
  return hip_status(mfa::launch_gemm(bf, up, chat, w_uq, w_uq, q_out, mfa::GemmOut::Direct, s, s_uq, s_uq));
}

int mfa_qproj(const void* x, const void* w_dq, const float* gamma, float eps, const void* w_uq, void* q_out, void* ws,
              size_t ws_bytes, int B, mfa_dtype dt, void* stream) {
  if (!x || !w_dq || !w_uq || !q_out || B < 1 || B > MFA_MAX_BATCH || !(eps >= 0.f) || !isfinite(eps))
    return MFA_ERR_INVALID_ARG;
  if (!act_dtype_ok(dt)) return MFA_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(w_dq) || !aligned16(w_uq) || !aligned16(q_out) || !aligned16(ws) ||
      (gamma && !aligned_n(gamma, 4)))
    return MFA_ERR_ALIGNMENT;
  if (!ws || ws_bytes < mfa_qproj_workspace_size(B, dt)) return MFA_ERR_WORKSPACE;
  return qproj_run(x, w_dq, nullptr, gamma, eps, w_uq, nullptr, q_out, ws, B, dt == MFA_BF16, (hipStream_t)stream);
}

// Block-fp8 weights: the bf16 q path with e4m3 weight bytes and their
// 128 x 128 block scales (the same plans, so the same workspace).
int mfa_qproj_w8(const void* x, const void* w_dq, const float* s_dq, const float* gamma, float eps, const void* w_uq,
                 const float* s_uq, void* q_out, void* ws, size_t ws_bytes, int B, void* stream) {
  if (!x || !w_dq || !s_dq || !w_uq || !s_uq || !q_out || B < 1 || B > MFA_MAX_BATCH || !(eps >= 0.f) ||
      !isfinite(eps))
    return MFA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_dq) || !aligned16(w_uq) || !aligned16(q_out) || !aligned16(ws) ||
      !aligned_n(s_dq, 4) || !aligned_n(s_uq, 4) || (gamma && !aligned_n(gamma, 4)))
    return MFA_ERR_ALIGNMENT;
  if (!ws || ws_bytes < mfa_qproj_workspace_size(B, MFA_BF16)) return MFA_ERR_WORKSPACE;
  return qproj_run(x, w_dq, s_dq, gamma, eps, w_uq, s_uq, q_out, ws, B, true, (hipStream_t)stream);
}

// ------------------------------------------------------------------ q path and K/V append in one
size_t mfa_qproj_kv_append_workspace_size(int B) {
  if (B < 1 || B > MFA_MAX_BATCH) return 0;
  return mfa::qkv_layout(B).total;
}

// The stacked product and its epilogue, then the q up-projection; s_* are the
// block scales of block-fp8 weights (all null for bf16 weights).
static int qkv_run(const void* x, const void* w_dq, const float* s_dq, const float* gamma, float eps, const void* w_uq,
                   const float* s_uq, const void* w_k, const float* s_k, const void* w_v, const float* s_v,
                   void* q_out, void* k_cache, void* v_cache, const int64_t* seq_off, const int32_t* seq_len,
                   int32_t* seq_len_out, float k_scale, float v_scale, void* ws, size_t ws_bytes, int B,
                   mfa_dtype cache_dt, hipStream_t s) {
  if (cache_dt != MFA_BF16 && cache_dt != MFA_FP8_E4M3) return MFA_ERR_UNSUPPORTED;
  const bool fp8 = cache_dt == MFA_FP8_E4M3;
  float inv_k = 1.f, inv_v = 1.f;
  if (fp8) {
    // the stored byte is e4m3(x * (1 / scale)): the reciprocal must be finite and non-zero
    inv_k = 1.f / k_scale;
    inv_v = 1.f / v_scale;
    if (!(k_scale > 0.f) || !(v_scale > 0.f) || !isfinite(k_scale) || !isfinite(v_scale) || !isfinite(inv_k) ||
        !isfinite(inv_v) || !(inv_k > 0.f) || !(inv_v > 0.f))
      return MFA_ERR_INVALID_ARG;
  }
  if (!aligned16(x) || !aligned16(w_dq) || !aligned16(w_uq) || !aligned16(w_k) || !aligned16(w_v) ||
      !aligned16(q_out) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(ws) || !aligned_n(seq_off, 8) ||
      !aligned_n(seq_len, 4) || !aligned_n(seq_len_out, 4) || (gamma && !aligned_n(gamma, 4)) ||
      (s_dq && (!aligned_n(s_dq, 4) || !aligned_n(s_uq, 4) || !aligned_n(s_k, 4) || !aligned_n(s_v, 4))))
    return MFA_ERR_ALIGNMENT;
  if (!ws || ws_bytes < mfa_qproj_kv_append_workspace_size(B)) return MFA_ERR_WORKSPACE;
  int st = MFA_OK;
  const int cus = plan_cus(&st);
  if (st != MFA_OK) return st;
  const bool w8 = s_dq != nullptr;
  const mfa::GemmPlan dn = mfa::plan_gemm(true, B, mfa::kPlanQkv, MFA_HIDDEN, MFA_RANK, cus, w8);
  const mfa::GemmPlan up = mfa::plan_gemm(true, B, MFA_QDIM, MFA_RANK, MFA_QDIM, cus, w8);
  const mfa::QprojLayout l = mfa::qkv_layout(B);
  if (mfa::qproj_part_need(B, true, dn, up) > l.part_bytes) return MFA_ERR_WORKSPACE;  // a planning bug, never run
  float* part = (float*)ws;
  void* chat = (char*)ws + l.chat_offset;
  // rows 0..2047 of the product from W_dq, 2048..2303 from W_k, 2304..2559 from W_v
  hipError_t e = mfa::launch_gemm(true, dn, x, w_dq, w_k, part, mfa::GemmOut::Partial, s, s_dq, s_k, w_v,
                                  MFA_RANK + MFA_HEAD_DIM, s_v);
  if (e != hipSuccess) return hip_status(e);
  e = mfa::launch_qkv_epilogue(part, dn.splits, B, gamma, eps, chat, k_cache, v_cache, seq_off, seq_len, fp8, inv_k,
                               inv_v, seq_len_out, s);
  if (e != hipSuccess) return hip_status(e);
  if (up.splits > 1) {
    // the first product's partials were consumed by the epilogue above
    e = mfa::launch_gemm(true, up, chat, w_uq, w_uq, part, mfa::GemmOut::Partial, s, s_uq, s_uq);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(mfa::launch_sum_reduce(true, part, up.splits, B, MFA_QDIM, q_out, s, up.tile_n));
  }
  return hip_status(mfa::launch_gemm(true, up, chat, w_uq, w_uq, q_out, mfa::GemmOut::Direct, s, s_uq, s_uq));
}

int mfa_qproj_kv_append(const void* x, const void* w_dq, const float* gamma, float eps, const void* w_uq,
                        const void* w_k, const void* w_v, void* q_out, void* k_cache, void* v_cache,
                        const int64_t* seq_off, const int32_t* seq_len, int32_t* seq_len_out, float k_scale,
                        float v_scale, void* ws, size_t ws_bytes, int B, mfa_dtype cache_dt, void* stream) {
  if (!x || !w_dq || !w_uq || !w_k || !w_v || !q_out || !k_cache || !v_cache || !seq_off || !seq_len || B < 1 ||
      B > MFA_MAX_BATCH || !(eps >= 0.f) || !isfinite(eps))
    return MFA_ERR_INVALID_ARG;
  return qkv_run(x, w_dq, nullptr, gamma, eps, w_uq, nullptr, w_k, nullptr, w_v, nullptr, q_out, k_cache, v_cache,
                 seq_off, seq_len, seq_len_out, k_scale, v_scale, ws, ws_bytes, B, cache_dt, (hipStream_t)stream);
}

int mfa_qproj_kv_append_w8(const void* x, const void* w_dq, const float* s_dq, const float* gamma, float eps,
                           const void* w_uq, const float* s_uq, const void* w_k, const float* s_k, const void* w_v,
                           const float* s_v, void* q_out, void* k_cache, void* v_cache, const int64_t* seq_off,
                           const int32_t* seq_len, int32_t* seq_len_out, float k_scale, float v_scale, void* ws,
                           size_t ws_bytes, int B, mfa_dtype cache_dt, void* stream) {
  if (!x || !w_dq || !s_dq || !w_uq || !s_uq || !w_k || !s_k || !w_v || !s_v || !q_out || !k_cache || !v_cache ||
      !seq_off || !seq_len || B < 1 || B > MFA_MAX_BATCH || !(eps >= 0.f) || !isfinite(eps))
    return MFA_ERR_INVALID_ARG;
  return qkv_run(x, w_dq, s_dq, gamma, eps, w_uq, s_uq, w_k, s_k, w_v, s_v, q_out, k_cache, v_cache, seq_off,
                 seq_len, seq_len_out, k_scale, v_scale, ws, ws_bytes, B, cache_dt, (hipStream_t)stream);
}

// ------------------------------------------------------------------ K/V append
size_t mfa_kv_append_workspace_size(int B, mfa_dtype act_dt) {
  if (B < 1 || B > MFA_MAX_BATCH || !act_dtype_ok(act_dt)) return 0;
  return mfa::kv_ws_bytes(B, act_dt == MFA_BF16);
}

// The device's plan of the [W_k; W_v] product, checked against the reserved region.
static int kv_plan(int B, bool bf, bool w8, mfa::GemmPlan* p) {
  int st = MFA_OK;
  const int cus = plan_cus(&st);
  if (st != MFA_OK) return st;
  *p = mfa::plan_gemm(bf, B, 2 * MFA_HEAD_DIM, MFA_HIDDEN, MFA_HEAD_DIM, cus, w8);
  return mfa::kv_part_need(B, bf, *p) <= mfa::kv_ws_bytes(B, bf) ? MFA_OK : MFA_ERR_WORKSPACE;
}

int mfa_kv_append(const void* x, const void* w_k, const void* w_v, void* k_cache, void* v_cache,
                  const int64_t* seq_off, const int32_t* seq_len, int32_t* seq_len_out, void* ws, size_t ws_bytes, int B,
                  mfa_dtype act_dt,
                  mfa_dtype cache_dt, void* stream) {
  if (!x || !w_k || !w_v || !k_cache || !v_cache || !seq_off || !seq_len || B < 1 || B > MFA_MAX_BATCH)
    return MFA_ERR_INVALID_ARG;
  if (!act_dtype_ok(act_dt) || cache_dt != act_dt) return MFA_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(w_k) || !aligned16(w_v) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(ws) || !aligned_n(seq_off, 8) || !aligned_n(seq_len, 4) ||
      !aligned_n(seq_len_out, 4))
    return MFA_ERR_ALIGNMENT;
  if (!ws || ws_bytes < mfa_kv_append_workspace_size(B, act_dt)) return MFA_ERR_WORKSPACE;
  const bool bf = act_dt == MFA_BF16;
  mfa::GemmPlan plan;
  const int st = kv_plan(B, bf, false, &plan);
  if (st != MFA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = mfa::launch_gemm(bf, plan, x, w_k, w_v, ws, mfa::GemmOut::Partial, s);
  if (e != hipSuccess) return hip_status(e);
  e = mfa::launch_kv_scatter(bf, (const float*)ws, bf ? plan.splits : 1, B, k_cache, v_cache, seq_off, seq_len,
                             seq_len_out, s);
  return hip_status(e);
}

int mfa_kv_append_fp8(const void* x, const void* w_k, const void* w_v, void* k_cache, void* v_cache,
                      const int64_t* seq_off, const int32_t* seq_len, int32_t* seq_len_out, float k_scale,
                      float v_scale, void* ws,
                      size_t ws_bytes, int B, mfa_dtype act_dt, void* stream) {
  if (!x || !w_k || !w_v || !k_cache || !v_cache || !seq_off || !seq_len || B < 1 || B > MFA_MAX_BATCH)
    return MFA_ERR_INVALID_ARG;
  // the stored byte is e4m3(x * (1 / scale)): the reciprocal must be finite and non-zero
  const float inv_k = 1.f / k_scale, inv_v = 1.f / v_scale;
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || !isfinite(k_scale) || !isfinite(v_scale) || !isfinite(inv_k) ||
      !isfinite(inv_v) || !(inv_k > 0.f) || !(inv_v > 0.f))
    return MFA_ERR_INVALID_ARG;
  if (!act_dtype_ok(act_dt)) return MFA_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(w_k) || !aligned16(w_v) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(ws) || !aligned_n(seq_off, 8) || !aligned_n(seq_len, 4) ||
      !aligned_n(seq_len_out, 4))
    return MFA_ERR_ALIGNMENT;
  if (!ws || ws_bytes < mfa_kv_append_workspace_size(B, act_dt)) return MFA_ERR_WORKSPACE;
  const bool bf = act_dt == MFA_BF16;
  mfa::GemmPlan plan;
  const int st = kv_plan(B, bf, false, &plan);
  if (st != MFA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = mfa::launch_gemm(bf, plan, x, w_k, w_v, ws, mfa::GemmOut::Partial, s);
  if (e != hipSuccess) return hip_status(e);
  e = mfa::launch_kv_scatter_fp8((const float*)ws, bf ? plan.splits : 1, B, k_cache, v_cache, seq_off, seq_len,
                                 inv_k, inv_v, seq_len_out, s);
  return hip_status(e);
}

int mfa_kv_append_w8(const void* x, const void* w_k, const float* s_k, const void* w_v, const float* s_v,
                     void* k_cache, void* v_cache, const int64_t* seq_off, const int32_t* seq_len,
                     int32_t* seq_len_out, mfa_dtype cache_dt,
                     float k_scale, float v_scale, void* ws, size_t ws_bytes, int B, void* stream) {
  if (!x || !w_k || !s_k || !w_v || !s_v || !k_cache || !v_cache || !seq_off || !seq_len || B < 1 ||
      B > MFA_MAX_BATCH)
    return MFA_ERR_INVALID_ARG;
  const bool fp8 = cache_dt == MFA_FP8_E4M3;
  if (cache_dt != MFA_BF16 && !fp8) return MFA_ERR_UNSUPPORTED;
  const float inv_k = 1.f / k_scale, inv_v = 1.f / v_scale;
  if (fp8 && (!(k_scale > 0.f) || !(v_scale > 0.f) || !isfinite(k_scale) || !isfinite(v_scale) ||
              !isfinite(inv_k) || !isfinite(inv_v) || !(inv_k > 0.f) || !(inv_v > 0.f)))
    return MFA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_k) || !aligned16(w_v) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(ws) || !aligned_n(s_k, 4) || !aligned_n(s_v, 4) || !aligned_n(seq_off, 8) || !aligned_n(seq_len, 4) ||
      !aligned_n(seq_len_out, 4))
    return MFA_ERR_ALIGNMENT;
  if (!ws || ws_bytes < mfa_kv_append_workspace_size(B, MFA_BF16)) return MFA_ERR_WORKSPACE;
  mfa::GemmPlan plan;
  const int st = kv_plan(B, true, true, &plan);
  if (st != MFA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = mfa::launch_gemm(true, plan, x, w_k, w_v, ws, mfa::GemmOut::Partial, s, s_k, s_v);
  if (e != hipSuccess) return hip_status(e);
  e = fp8 ? mfa::launch_kv_scatter_fp8((const float*)ws, plan.splits, B, k_cache, v_cache, seq_off, seq_len, inv_k,
                                       inv_v, seq_len_out, s)
          : mfa::launch_kv_scatter(true, (const float*)ws, plan.splits, B, k_cache, v_cache, seq_off, seq_len,
                                   seq_len_out, s);
  return hip_status(e);
}

// ------------------------------------------------------------------ attention
size_t mfa_decode_attn_workspace_size(int B, int num_workgroups) {
  if (B < 1 || B > MFA_MAX_BATCH || num_workgroups < 0 || num_workgroups > 65536) return 0;
  int G = num_workgroups;
  if (G == 0) {
    int st = MFA_OK;
    G = current_cu_count(&st);
    if (st != MFA_OK) return 0;
  }
  return mfa::attn_ws_bytes(B, G);
}

// Shared by the contiguous and the paged entry points (table == null: contiguous).
// use_scratch: the library's own static scratch replaces ws / ws_bytes.
static int decode_attn_impl(const void* q, const void* k_cache, const void* v_cache, const int64_t* seq_off,
                            const int32_t* block_table, int max_blocks, int page_rows, const int32_t* seq_len,
                            int n_tokens, float softmax_scale, float k_scale, float v_scale, void* out, float* lse,
                            void* ws, size_t ws_bytes, int B, int num_workgroups, mfa_dtype q_dt, mfa_dtype kv_dt,
                            void* stream, bool use_scratch = false) {
  const bool paged = block_table != nullptr;
  if (!q || !k_cache || !v_cache || (!paged && !seq_off) || !seq_len || !out || B < 1 || B > MFA_MAX_BATCH ||
      num_workgroups < 0 || num_workgroups > 65536 || !isfinite(softmax_scale) || !isfinite(k_scale) ||
      !isfinite(v_scale) || n_tokens < 1 || n_tokens > MFA_MAX_TOKENS)
    return MFA_ERR_INVALID_ARG;
  int page_shift = 0;
  if (paged) {
    if (max_blocks < 1 || page_rows < 64 || page_rows > (1 << 20) || (page_rows & (page_rows - 1)) != 0)
      return MFA_ERR_INVALID_ARG;
    while ((1 << page_shift) < page_rows) ++page_shift;
  }
  mfa::AttnKind kind;
  if (q_dt == MFA_F32 && kv_dt == MFA_F32 && !paged && n_tokens == 1)
    kind = mfa::AttnKind::F32;
  else if (q_dt == MFA_BF16 && kv_dt == MFA_BF16)
    kind = mfa::AttnKind::BF16;
  else if (q_dt == MFA_BF16 && kv_dt == MFA_FP8_E4M3)
    kind = mfa::AttnKind::BF16_FP8KV;
  else
    return MFA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      (!use_scratch && !aligned16(ws)) || (!paged && !aligned_n(seq_off, 8)) ||
      (paged && !aligned_n(block_table, 4)) || !aligned_n(seq_len, 4) || (lse && !aligned_n(lse, 4)))
    return MFA_ERR_ALIGNMENT;
  if (use_scratch) {
    ws = nullptr;
    ws_bytes = mfa::kAttnScratchBytes;
  } else if (!ws) {
    return MFA_ERR_WORKSPACE;
  }
  int G = num_workgroups;
  if (G == 0) {
    int st = MFA_OK;
    G = current_cu_count(&st);
    if (st != MFA_OK) return st;
  }
  if (ws_bytes < mfa::attn_ws_bytes(B, G, n_tokens)) return MFA_ERR_WORKSPACE;
  if (use_scratch) {
    const hipError_t e = mfa::attn_scratch(&ws);
    if (e != hipSuccess) return hip_status(e);
  }
  mfa::AttnLaunch p;
  p.kind = kind;
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.seq_off = seq_off;
  p.seq_len = seq_len;
  p.out = out;
  p.lse = lse;
  p.ws = ws;
  p.B = B;
  p.G = G;
  p.softmax_scale = softmax_scale;
  p.k_scale = kind == mfa::AttnKind::BF16_FP8KV ? k_scale : 1.f;
  p.v_scale = kind == mfa::AttnKind::BF16_FP8KV ? v_scale : 1.f;
  p.table = block_table;
  p.max_blocks = paged ? max_blocks : 0;
  p.page_shift = page_shift;
  p.nt = n_tokens;
  return hip_status(mfa::launch_decode_attn(p, (hipStream_t)stream));
}

int mfa_decode_attn(const void* q, const void* k_cache, const void* v_cache, const int64_t* seq_off,
                    const int32_t* seq_len, float softmax_scale, float k_scale, float v_scale, void* out, float* lse,
                    void* ws, size_t ws_bytes, int B, int num_workgroups, mfa_dtype q_dt, mfa_dtype kv_dt,
                    void* stream) {
  if (!seq_off) return MFA_ERR_INVALID_ARG;
  return decode_attn_impl(q, k_cache, v_cache, seq_off, nullptr, 0, 0, seq_len, 1, softmax_scale, k_scale, v_scale,
                          out, lse, ws, ws_bytes, B, num_workgroups, q_dt, kv_dt, stream);
}

static_assert(MFA_NOALLOC_SCRATCH_BYTES == mfa::kAttnScratchBytes, "scratch size in the header");

int mfa_decode_attn_noalloc(const void* q, const void* k_cache, const void* v_cache, const int64_t* seq_off,
                            const int32_t* seq_len, float softmax_scale, float k_scale, float v_scale, void* out,
                            float* lse, int B, int num_workgroups, mfa_dtype q_dt, mfa_dtype kv_dt, void* stream) {
  if (!seq_off) return MFA_ERR_INVALID_ARG;
  return decode_attn_impl(q, k_cache, v_cache, seq_off, nullptr, 0, 0, seq_len, 1, softmax_scale, k_scale, v_scale,
                          out, lse, nullptr, 0, B, num_workgroups, q_dt, kv_dt, stream, true);
}

size_t mfa_decode_attn_mt_workspace_size(int B, int n_tokens, int num_workgroups) {
  if (n_tokens < 1 || n_tokens > MFA_MAX_TOKENS) return 0;
  const size_t one = mfa_decode_attn_workspace_size(B, num_workgroups);
  if (one == 0) return 0;
  int G = num_workgroups;
  if (G == 0) {
    int st = MFA_OK;
    G = current_cu_count(&st);
    if (st != MFA_OK) return 0;
  }
  return mfa::attn_ws_bytes(B, G, n_tokens);
}

int mfa_decode_attn_mt(const void* q, const void* k_cache, const void* v_cache, const int64_t* seq_off,
                       const int32_t* seq_len, int n_tokens, float softmax_scale, float k_scale, float v_scale,
                       void* out, float* lse, void* ws, size_t ws_bytes, int B, int num_workgroups, mfa_dtype q_dt,
                       mfa_dtype kv_dt, void* stream) {
  if (!seq_off) return MFA_ERR_INVALID_ARG;
  return decode_attn_impl(q, k_cache, v_cache, seq_off, nullptr, 0, 0, seq_len, n_tokens, softmax_scale, k_scale,
                          v_scale, out, lse, ws, ws_bytes, B, num_workgroups, q_dt, kv_dt, stream);
}

int mfa_decode_attn_paged(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                          int max_blocks, int page_rows, const int32_t* seq_len, float softmax_scale, float k_scale,
                          float v_scale, void* out, float* lse, void* ws, size_t ws_bytes, int B,
                          int num_workgroups, mfa_dtype q_dt, mfa_dtype kv_dt, void* stream) {
  if (!block_table) return MFA_ERR_INVALID_ARG;
  return decode_attn_impl(q, k_pages, v_pages, nullptr, block_table, max_blocks, page_rows, seq_len, 1,
                          softmax_scale, k_scale, v_scale, out, lse, ws, ws_bytes, B, num_workgroups, q_dt, kv_dt,
                          stream);
}

int mfa_decode_attn_paged_mt(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                             int max_blocks, int page_rows, const int32_t* seq_len, int n_tokens, float softmax_scale,
                             float k_scale, float v_scale, void* out, float* lse, void* ws, size_t ws_bytes, int B,
                             int num_workgroups, mfa_dtype q_dt, mfa_dtype kv_dt, void* stream) {
  if (!block_table) return MFA_ERR_INVALID_ARG;
  return decode_attn_impl(q, k_pages, v_pages, nullptr, block_table, max_blocks, page_rows, seq_len, n_tokens,
                          softmax_scale, k_scale, v_scale, out, lse, ws, ws_bytes, B, num_workgroups, q_dt, kv_dt,
                          stream);
}

// ------------------------------------------------------------------ out-projection
size_t mfa_oproj_workspace_size(int B, mfa_dtype dt) {
  if (B < 1 || B > MFA_MAX_BATCH || !act_dtype_ok(dt)) return 0;
  return mfa::oproj_ws_bytes(B, dt == MFA_BF16);
}

static int oproj_run(const void* attn, const void* w_o, const float* s_o, void* y, void* ws, size_t ws_bytes, int B,
                     bool bf, hipStream_t s) {
  int st = MFA_OK;
  const int cus = plan_cus(&st);
  if (st != MFA_OK) return st;
  const mfa::GemmPlan plan = mfa::plan_gemm(bf, B, MFA_HIDDEN, MFA_QDIM, MFA_HIDDEN, cus, s_o != nullptr);
  if (mfa::oproj_part_need(bf, plan) > ws_bytes) return MFA_ERR_WORKSPACE;  // within the documented size
  if (bf && plan.splits > 1) {
    hipError_t e = mfa::launch_gemm(true, plan, attn, w_o, w_o, ws, mfa::GemmOut::Partial, s, s_o, s_o);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(mfa::launch_sum_reduce(true, (const float*)ws, plan.splits, B, MFA_HIDDEN, y, s,
                                             plan.tile_n));
  }
  return hip_status(mfa::launch_gemm(bf, plan, attn, w_o, w_o, y, mfa::GemmOut::Direct, s, s_o, s_o));
}

int mfa_oproj(const void* attn, const void* w_o, void* y, void* ws, size_t ws_bytes, int B, mfa_dtype dt,
              void* stream) {
  if (!attn || !w_o || !y || B < 1 || B > MFA_MAX_BATCH) return MFA_ERR_INVALID_ARG;
  if (!act_dtype_ok(dt)) return MFA_ERR_UNSUPPORTED;
  if (!aligned16(attn) || !aligned16(w_o) || !aligned16(y) || !aligned16(ws)) return MFA_ERR_ALIGNMENT;
  const size_t need = mfa_oproj_workspace_size(B, dt);
  if (need > 0 && (!ws || ws_bytes < need)) return MFA_ERR_WORKSPACE;
  return oproj_run(attn, w_o, nullptr, y, ws, ws ? ws_bytes : 0, B, dt == MFA_BF16, (hipStream_t)stream);
}

int mfa_oproj_w8(const void* attn, const void* w_o, const float* s_o, void* y, void* ws, size_t ws_bytes, int B,
                 void* stream) {
  if (!attn || !w_o || !s_o || !y || B < 1 || B > MFA_MAX_BATCH) return MFA_ERR_INVALID_ARG;
  if (!aligned16(attn) || !aligned16(w_o) || !aligned16(y) || !aligned16(ws) || !aligned_n(s_o, 4))
    return MFA_ERR_ALIGNMENT;
  const size_t need = mfa_oproj_workspace_size(B, MFA_BF16);
  if (need > 0 && (!ws || ws_bytes < need)) return MFA_ERR_WORKSPACE;
  return oproj_run(attn, w_o, s_o, y, ws, ws ? ws_bytes : 0, B, true, (hipStream_t)stream);
}

// ------------------------------------------------------------------ bandwidth probe
int mfa_bw_probe(const void* buf, size_t bytes, uint32_t* sink, int num_workgroups, void* stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 != 0 || num_workgroups < 0 || num_workgroups > 65536)
    return MFA_ERR_INVALID_ARG;
  if (!aligned16(buf) || !aligned_n(sink, 4)) return MFA_ERR_ALIGNMENT;
  int G = num_workgroups;
  if (G == 0) {
    int st = MFA_OK;
    G = current_cu_count(&st);
    if (st != MFA_OK) return st;
  }
  return hip_status(mfa::launch_bw_probe(buf, bytes, sink, G, (hipStream_t)stream));
}

}  // extern "C"
