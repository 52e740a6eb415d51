// Host-side interface between the C ABI (mfa_api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>
#include <utility>

#include "plan.h"

namespace mfa {

// Launch and return this launch's own status (not a stale error of earlier
// work). Arguments are converted to the kernel's parameter types first.
template <typename... Params, size_t... I>
inline hipError_t launch_impl(void (*kernel)(Params...), dim3 grid, dim3 block, hipStream_t stream,
                              std::tuple<Params...>& vals, std::index_sequence<I...>) {
  void* ptrs[] = {(void*)&std::get<I>(vals)...};
  return hipLaunchKernel((const void*)kernel, grid, block, ptrs, 0, stream);
}
template <typename... Params, typename... Args>
inline hipError_t launch(void (*kernel)(Params...), dim3 grid, dim3 block, hipStream_t stream, Args... args) {
  static_assert(sizeof...(Params) == sizeof...(Args), "kernel arity");
  std::tuple<Params...> vals(static_cast<Params>(args)...);
  return launch_impl(kernel, grid, block, stream, vals, std::index_sequence_for<Params...>{});
}

// ------------------------------------------------------------------ attention
enum class AttnKind { F32, BF16, BF16_FP8KV };

struct AttnLaunch {
  AttnKind kind;
  const void* q;
  const void* k;
  const void* v;
  const int64_t* seq_off;
  const int32_t* seq_len;
  void* out;
  float* lse;
  void* ws;
  int B;
  int G;  // workgroups of the main kernel
  float softmax_scale, k_scale, v_scale;
  // paged cache (MFMA kinds only): null table = contiguous rows at seq_off
  const int32_t* table = nullptr;
  int max_blocks = 0;
  int page_shift = 0;
  int nt = 1;  // query tokens per sequence (2: multi-token decode, contiguous cache)
};

// Workspace: partial outputs [(G + B) nt][64][256] (fp32-sized; bf16 partials
// use half), partial lse [(G + B) nt][64] fp32, then per-sequence combine
// metadata [B] x {first slot, piece count}; nt = query tokens per sequence.
inline size_t attn_part_o_bytes(int B, int G, int nt = 1) {
  return (size_t)(G + B) * nt * 64 * 256 * sizeof(float);
}
inline size_t attn_meta_offset(int B, int G, int nt = 1) {
  return attn_part_o_bytes(B, G, nt) + (size_t)(G + B) * nt * 64 * sizeof(float);
}
inline size_t attn_ws_bytes(int B, int G, int nt = 1) { return attn_meta_offset(B, G, nt) + (size_t)B * 2 * sizeof(int); }

hipError_t launch_decode_attn(const AttnLaunch& p, hipStream_t stream);

// Library-owned device scratch of the allocation-free attention call (one
// copy per GPU, held until the process ends): its size, and its device
// address on the current device (looked up once per device).
constexpr size_t kAttnScratchBytes = (size_t)40 << 20;
hipError_t attn_scratch(void** ptr);

// Streaming-read probe: G workgroups XOR bytes / 16 16-byte words of buf,
// one 32-bit checksum per workgroup into sink[G].
hipError_t launch_bw_probe(const void* buf, size_t bytes, unsigned* sink, int G, hipStream_t stream);

// ------------------------------------------------------------------ projections
// Y[M, N] = X[M, K] * W^T where W = [W0 (N0 rows); W1 (N - N0 rows)], each [rows, K].
enum class GemmOut {
  Partial,  // fp32 partial sums [S][M][N] (S = split count) into the workspace
  Direct    // final values [M][N] in the activation dtype
};

// S0 / S1 non-null: W0 / W1 are block-fp8 (e4m3 bytes, fp32 scales per 128 x 128 block, [rows/128][K/128])
// W2 non-null (MFMA path): rows N0 <= n < N1 from W1, n >= N1 from W2; for block-fp8 weights S2 holds W2's
// scales and N0, N1 are multiples of 128.
hipError_t launch_gemm(bool bf16, const GemmPlan& p, const void* X, const void* W0, const void* W1, void* Y,
                       GemmOut mode, hipStream_t stream, const float* S0 = nullptr, const float* S1 = nullptr,
                       const void* W2 = nullptr, int N1 = 0, const float* S2 = nullptr);

// c_hat[M, N] = rmsnorm(sum_s part[s]) * gamma, in the activation dtype.
hipError_t launch_rmsnorm_reduce(bool bf16, const float* part, int S, int M, int N, const float* gamma,
                                 float eps, void* out, hipStream_t stream);
// out[M, N] = sum_s part[s], in the activation dtype. tile_n: the column tile of
// the MFMA product that wrote the parts (its sum is then placed by tile where the
// tile count is a multiple of 8 and the width 64 or 128), or 0.
hipError_t launch_sum_reduce(bool bf16, const float* part, int S, int M, int N, void* out, hipStream_t stream,
                             int tile_n = 0);
// rows m: k = sum_s part[s][m][0:256], v = sum_s part[s][m][256:512] written at cache row off[m] + len[m].
hipError_t launch_kv_scatter(bool bf16, const float* part, int S, int M, void* k_cache, void* v_cache,
                             const int64_t* seq_off, const int32_t* seq_len, int32_t* len_out, hipStream_t stream);
// The [W_dq; W_k; W_v] product's partials [S][M][2560] (bf16 activations): c_hat[M, 2048] =
// rmsnorm(columns 0..2047) * gamma, and the K/V rows (columns 2048..2559) written as the two scatters do.
hipError_t launch_qkv_epilogue(const float* part, int S, int M, const float* gamma, float eps, void* chat,
                               void* k_cache, void* v_cache, const int64_t* seq_off, const int32_t* seq_len,
                               bool fp8_cache, float inv_k, float inv_v, int32_t* len_out, hipStream_t stream);
// rows into e4m3 caches: byte = e4m3(clamp(x * inv, +-448)), round to nearest even
hipError_t launch_kv_scatter_fp8(const float* part, int S, int M, void* k_cache, void* v_cache,
                                 const int64_t* seq_off, const int32_t* seq_len, float inv_k, float inv_v,
                                 int32_t* len_out, hipStream_t stream);

}  // namespace mfa
