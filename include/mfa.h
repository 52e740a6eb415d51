/*
 * libmfa — decode-time Multi-Matrix Factorization Attention (MFA) on AMD
 * Instinct MI355X (gfx950). C ABI.
 *
 * What is computed (Step-3 paper, "Step-3 is Large yet Affordable: Model-system
 * Co-design for Cost-effective Decoding"; summary page on bud-325.pages.dev,
 * sections "Key claims" and "Method"; redeep.blog Step3 post, architecture
 * table): per new token the hidden state (7168) is down-projected to a 2048-wide
 * latent, normalized, and up-projected to 64 query heads of width 256; all 64
 * heads attend over ONE shared K head and ONE shared V head of width 256 held
 * in a per-sequence cache (one K row and one V row per token); the 64 head
 * outputs are projected back to 7168.
 *
 * Choices where the pages are silent: the normalization is RMSNorm
 * (x * rsqrt(mean(x^2) + eps) * gamma); the softmax scale is a parameter
 * (1/sqrt(256) = 0.0625 for this model); no rotary/positional term; no biases;
 * weights are row-major [out, in] (y = x W^T); query column n is head n / 256,
 * channel n % 256, and the attention output is flattened the same way.
 *
 * Conventions for every call:
 *  - All tensor pointers are DEVICE pointers the caller allocated; the library
 *    never allocates, frees or keeps them. Scalars and sizes are host values.
 *  - Tensors are dense row-major. Each pointer must be 16-byte aligned.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    is asynchronous: no call synchronizes. Results are valid once the stream
 *    reaches them.
 *  - Calls return MFA_OK or a negative status and never abort. Argument
 *    checks (null pointers, sizes, dtype combinations, alignment, workspace
 *    size) run on the host before any HIP call. A failed launch returns
 *    MFA_ERR_HIP. Device-side preconditions (documented per call) are not
 *    checked.
 *  - Calls on different streams or threads are independent, except calls of
 *    mfa_decode_attn_noalloc on one GPU, which share that GPU's library-owned
 *    scratch buffer; the library keeps no other state than a cached
 *    per-device property table and that buffer's per-device address.
 */
#ifndef MFA_H_
#define MFA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Model dimensions (fixed by the architecture). */
#define MFA_HIDDEN 7168
#define MFA_RANK 2048
#define MFA_HEADS 64
#define MFA_HEAD_DIM 256
#define MFA_QDIM (MFA_HEADS * MFA_HEAD_DIM) /* 16384 */

/* Storage types. MFA_BF16 is bfloat16; MFA_FP8_E4M3 is the OCP 8-bit E4M3
 * ("fn": max 448, no infinity) with one fp32 scale per tensor (value = byte
 * value * scale). mfa_dtype is a plain int, so that every value a caller may
 * pass is well defined on both sides of the ABI (an enum type would give C++
 * code undefined behaviour for values outside its enumerators); values other
 * than these three are rejected with MFA_ERR_UNSUPPORTED. */
enum { MFA_F32 = 0, MFA_BF16 = 1, MFA_FP8_E4M3 = 2 };
typedef int mfa_dtype;

enum {
  MFA_OK = 0,
  MFA_ERR_INVALID_ARG = -1, /* null pointer, size out of range */
  MFA_ERR_UNSUPPORTED = -2, /* dtype combination not provided */
  MFA_ERR_ALIGNMENT = -3,   /* a pointer is not 16-byte aligned */
  MFA_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required */
  MFA_ERR_HIP = -5          /* a HIP runtime call or launch failed */
};

/* Largest batch any call accepts. */
#define MFA_MAX_BATCH 65536
/* Most new query tokens per sequence the multi-token attention calls accept. */
#define MFA_MAX_TOKENS 4

int mfa_version(void);                       /* 10000 * major + 100 * minor + patch */
const char* mfa_status_string(int status);   /* static string, never NULL */
int mfa_last_hip_error(void);                /* hipError_t behind this thread's last MFA_ERR_HIP (0 if none) */

/* ------------------------------------------------------------------ q path
 * Low-rank query (Step-3 summary, "Method": 7168 -> 2048, normalized, -> 64 x 256).
 *   c     = x W_dq^T                      x [B, 7168], W_dq [2048, 7168]
 *   c_hat = c * rsqrt(mean(c^2) + eps) * gamma   (gamma [2048] fp32, NULL = ones)
 *   q     = c_hat W_uq^T as [B, 64, 256]  W_uq [16384, 2048]
 * dt = MFA_F32 (all fp32) or MFA_BF16 (x, weights, q in bf16; fp32
 * accumulation; c_hat is rounded to bf16 before the up-projection).
 * ws: device scratch of at least mfa_qproj_workspace_size(B, dt) bytes
 * (contents undefined on return). 1 <= B <= MFA_MAX_BATCH.
 */
size_t mfa_qproj_workspace_size(int B, mfa_dtype dt);
int mfa_qproj(const void* x, const void* w_dq, const float* gamma, float eps, const void* w_uq,
              void* q_out, void* ws, size_t ws_bytes, int B, mfa_dtype dt, void* stream);

/* ------------------------------------------------------------------ K/V append
 * The new token's shared K and V rows (Step-3 summary, "Method": one K and one
 * V per token): k = x W_k^T, v = x W_v^T (W_k, W_v [256, 7168]), written to
 * rows seq_off[b] + seq_len[b] of k_cache / v_cache ([rows, 256], cache_dt).
 * seq_off (int64) and seq_len (int32) are device arrays of length B.
 * seq_len_out: NULL, or a device int32 array of length B (4-byte aligned)
 * that receives seq_len[b] + 1, the length including the appended row, for
 * the attention call that follows; it may be seq_len itself (an in-place
 * increment, done after the row is written). Note: the call then mutates
 * the lengths, which a plain append leaves to the caller; with seq_len_out
 * NULL (or a separate array) seq_len is never written. Supported:
 * act_dt = cache_dt = MFA_F32, or act_dt = cache_dt = MFA_BF16.
 * Device-side precondition: the target rows exist and are distinct.
 * ws: at least mfa_kv_append_workspace_size(B, act_dt) bytes.
 */
size_t mfa_kv_append_workspace_size(int B, mfa_dtype act_dt);
int mfa_kv_append(const void* x, const void* w_k, const void* w_v, void* k_cache, void* v_cache,
                  const int64_t* seq_off, const int32_t* seq_len, int32_t* seq_len_out, void* ws, size_t ws_bytes,
                  int B, mfa_dtype act_dt, mfa_dtype cache_dt, void* stream);

/* ------------------------------------------------------------------ q path and K/V append in one call
 * mfa_qproj followed by mfa_kv_append (bf16 activations and weights) with
 * the down-projection and the K/V projections, which all multiply x, done as
 * one product over the stacked [W_dq; W_k; W_v] (2560 output columns) and
 * one epilogue (RMSNorm of c, the K/V rows written at seq_off[b] +
 * seq_len[b]); the q up-projection then follows as in mfa_qproj. The results
 * are those of the two calls up to the order of fp32 additions (the K split
 * of the stacked product is planned for its own shape). cache_dt = MFA_BF16
 * (bf16 caches) or MFA_FP8_E4M3 (rows quantized as mfa_kv_append_fp8 does,
 * with the host scales k_scale and v_scale; ignored for bf16). q_out, gamma,
 * eps as for mfa_qproj; caches, seq_off, seq_len, seq_len_out and the
 * device-side precondition as for mfa_kv_append. ws: at least
 * mfa_qproj_kv_append_workspace_size(B) bytes (contents undefined on return).
 * Other cache dtypes: MFA_ERR_UNSUPPORTED.
 */
size_t mfa_qproj_kv_append_workspace_size(int B);
int mfa_qproj_kv_append(const void* x, const void* w_dq, const float* gamma, float eps, const void* w_uq,
                        const void* w_k, const void* w_v, void* q_out, void* k_cache, void* v_cache,
                        const int64_t* seq_off, const int32_t* seq_len, int32_t* seq_len_out, float k_scale,
                        float v_scale, void* ws, size_t ws_bytes, int B, mfa_dtype cache_dt, void* stream);

/* ------------------------------------------------------------------ K/V append, e4m3 cache
 * As mfa_kv_append, but the rows are stored quantized into e4m3 caches (the
 * model runs in FP8, attention included: Step-3 summary, "Key claims"), the
 * cache format mfa_decode_attn reads with kv_dt = MFA_FP8_E4M3 and the same
 * per-tensor scales. Byte j of the new row is e4m3(x_j / scale) (OCP E4M3,
 * "fn" variant: no infinity), rounded to nearest with ties to even, the
 * quotient computed in fp32 as x_j * (1 / scale) with the reciprocal rounded
 * to fp32, and clamped to +-448, the largest finite magnitude. k_scale and
 * v_scale are host values, finite, > 0, with finite reciprocals (else
 * MFA_ERR_INVALID_ARG). act_dt = MFA_F32 or MFA_BF16. Caches [rows, 256]
 * bytes, 16-byte aligned. ws: at least mfa_kv_append_workspace_size(B, act_dt)
 * bytes. seq_off, seq_len, seq_len_out and the device-side precondition as
 * for mfa_kv_append.
 */
int mfa_kv_append_fp8(const void* x, const void* w_k, const void* w_v, void* k_cache, void* v_cache,
                      const int64_t* seq_off, const int32_t* seq_len, int32_t* seq_len_out, float k_scale,
                      float v_scale, void* ws, size_t ws_bytes, int B, mfa_dtype act_dt, void* stream);

/* ------------------------------------------------------------------ attention
 * Shared-KV decode attention (Step-3 summary, "Key claims"/"Method": 64 query
 * heads attend over one shared K and one shared V head of width 256). For each
 * sequence b and head h, over cache rows j in [seq_off[b], seq_off[b]+seq_len[b]):
 *   s_j = (q[b,h,:] . K_j) * softmax_scale * k_scale
 *   out[b,h,:] = sum_j softmax(s)_j * V_j * v_scale
 *   lse[b,h]   = ln sum_j exp(s_j)           (natural log; optional output)
 * A sequence with seq_len 0 yields out = 0 and lse = -inf.
 * Supported (q_dt, kv_dt): (F32, F32) -> fp32 out; (BF16, BF16) -> bf16 out;
 * (BF16, FP8_E4M3) -> bf16 out. k_scale / v_scale are used for FP8_E4M3 only
 * (pass 1 otherwise). q [B, 64, 256]; caches [rows, 256]; out [B, 64, 256];
 * lse [B, 64] fp32 or NULL. seq_off/seq_len as for mfa_kv_append.
 * The key range of all sequences is cut into equal contiguous pieces, one per
 * workgroup; sequences cut into several pieces are merged by log-sum-exp.
 * num_workgroups: 0 = one per compute unit (the default), > 0 forces that many
 * (tests use 1 to disable all splitting). ws: at least
 * mfa_decode_attn_workspace_size(B, num_workgroups) bytes; with
 * num_workgroups = 0 this queries the current device.
 */
size_t mfa_decode_attn_workspace_size(int B, int num_workgroups);
int mfa_decode_attn(const void* q, const void* k_cache, const void* v_cache, const int64_t* seq_off,
                    const int32_t* seq_len, float softmax_scale, float k_scale, float v_scale,
                    void* out, float* lse, void* ws, size_t ws_bytes, int B, int num_workgroups,
                    mfa_dtype q_dt, mfa_dtype kv_dt, void* stream);

/* ------------------------------------------------------------------ attention, no allocation
 * For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation. Computes exactly what mfa_decode_attn computes, with the same
 * kernels and arguments, but its partial outputs and merge records go to a
 * static device buffer the library owns, MFA_NOALLOC_SCRATCH_BYTES on every
 * GPU it runs on (held until the process ends). Neither the call nor the
 * kernels allocate or free anything. A call whose
 * mfa_decode_attn_workspace_size(B, num_workgroups) exceeds the buffer
 * returns MFA_ERR_WORKSPACE before any launch (with num_workgroups = 0, one
 * per CU, up to about 380 sequences on 256 CUs). All calls on one GPU share
 * its buffer, which keeps the last call's contents (nothing in it needs to
 * start zeroed): calls that overlap on one GPU (other streams or threads)
 * race, so the caller orders them. The buffer's device address is looked up
 * on the first call on each device.
 */
#define MFA_NOALLOC_SCRATCH_BYTES ((size_t)40 << 20)
int mfa_decode_attn_noalloc(const void* q, const void* k_cache, const void* v_cache, const int64_t* seq_off,
                            const int32_t* seq_len, float softmax_scale, float k_scale, float v_scale, void* out,
                            float* lse, int B, int num_workgroups, mfa_dtype q_dt, mfa_dtype kv_dt, void* stream);

/* ------------------------------------------------------------------ attention, several new tokens
 * Multi-token decode (speculative or multi-token-prediction verification;
 * the pages' throughput figures exclude multi-token prediction, Step-3
 * summary, "Key claims"): each sequence brings n_tokens new query tokens
 * whose K/V rows are already the last n_tokens rows of its cache (seq_len
 * counts them). Token t (0-based) of sequence b attends causally, over rows
 * [seq_off[b], seq_off[b] + seq_len[b] - (n_tokens - 1 - t)); otherwise as
 * mfa_decode_attn. q [B, n_tokens, 64, 256]; out [B, n_tokens, 64, 256];
 * lse [B, n_tokens, 64] or NULL. A token that sees no row gets out = 0 and
 * lse = -inf. n_tokens: 1 .. MFA_MAX_TOKENS (else MFA_ERR_INVALID_ARG); 1
 * is exactly mfa_decode_attn. Supported (q_dt, kv_dt): (BF16, BF16),
 * (BF16, FP8_E4M3) for n_tokens >= 2. Each key is fetched from memory once
 * for tokens 0 and 1 and once more for tokens 2 .. n_tokens - 1. ws: at least mfa_decode_attn_mt_workspace_size(B, n_tokens,
 * num_workgroups) bytes (0 for invalid arguments).
 */
size_t mfa_decode_attn_mt_workspace_size(int B, int n_tokens, int num_workgroups);
int mfa_decode_attn_mt(const void* q, const void* k_cache, const void* v_cache, const int64_t* seq_off,
                       const int32_t* seq_len, int n_tokens, float softmax_scale, float k_scale,
                       float v_scale, void* out, float* lse, void* ws, size_t ws_bytes, int B,
                       int num_workgroups, mfa_dtype q_dt, mfa_dtype kv_dt, void* stream);

/* ------------------------------------------------------------------ attention, paged cache
 * mfa_decode_attn over a paged cache: sequence b's rows live in fixed-size
 * pages of page_rows rows, its j-th block of page_rows keys (rows
 * j*page_rows .. j*page_rows + page_rows - 1 of the sequence) in page
 * block_table[b * max_blocks + j], which occupies rows
 * page*page_rows .. page*page_rows + page_rows - 1 of k_pages / v_pages
 * ([n_pages * page_rows, 256], kv_dt). Everything else (the computation,
 * scales, outputs, lse, num_workgroups, workspace size) is as for
 * mfa_decode_attn; the same workspace size applies. Supported (q_dt, kv_dt):
 * (BF16, BF16), (BF16, FP8_E4M3). page_rows: a power of two, 64 <= page_rows
 * <= 2^20; max_blocks >= 1 (else MFA_ERR_INVALID_ARG); block_table int32,
 * 4-byte aligned. Device-side precondition: seq_len[b] <= max_blocks *
 * page_rows and the first ceil(seq_len[b] / page_rows) entries of row b are
 * valid pages (rows past seq_len[b] are never used as keys).
 */
int mfa_decode_attn_paged(const void* q, const void* k_pages, const void* v_pages,
                          const int32_t* block_table, int max_blocks, int page_rows,
                          const int32_t* seq_len, float softmax_scale, float k_scale, float v_scale,
                          void* out, float* lse, void* ws, size_t ws_bytes, int B, int num_workgroups,
                          mfa_dtype q_dt, mfa_dtype kv_dt, void* stream);

/* ------------------------------------------------------------------ attention, paged cache, several new tokens
 * Multi-token decode over a paged cache: the causal multi-token computation of
 * mfa_decode_attn_mt, with sequence b's keys located through its block table
 * as in mfa_decode_attn_paged (token t sees the first seq_len[b] -
 * (n_tokens - 1 - t) keys of the sequence). Shapes, outputs, n_tokens
 * (1 .. MFA_MAX_TOKENS), supported dtypes and the workspace size
 * (mfa_decode_attn_mt_workspace_size) are those of mfa_decode_attn_mt; the
 * page arguments and their preconditions are those of mfa_decode_attn_paged.
 * block_table NULL: MFA_ERR_INVALID_ARG.
 */
int mfa_decode_attn_paged_mt(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                             int max_blocks, int page_rows, const int32_t* seq_len, int n_tokens,
                             float softmax_scale, float k_scale, float v_scale, void* out, float* lse, void* ws,
                             size_t ws_bytes, int B, int num_workgroups, mfa_dtype q_dt, mfa_dtype kv_dt,
                             void* stream);

/* ------------------------------------------------------------------ out-projection
 * y = O_flat W_o^T: attn [B, 16384] (the [B, 64, 256] attention output),
 * W_o [7168, 16384], y [B, 7168]. dt = MFA_F32 or MFA_BF16 (fp32 accumulation).
 * ws: at least mfa_oproj_workspace_size(B, dt) bytes.
 */
size_t mfa_oproj_workspace_size(int B, mfa_dtype dt);
int mfa_oproj(const void* attn, const void* w_o, void* y, void* ws, size_t ws_bytes, int B,
              mfa_dtype dt, void* stream);

/* ------------------------------------------------------------------ block-fp8 weights
 * The projections with block-fp8 weights (the model's checkpoints come in
 * bf16 and in block-fp8, and it runs in FP8: step3-fp8 model card, precision
 * notes; Step-3 summary, "Key claims"). A weight W [out, in] is given as e4m3
 * bytes W8 [out, in] (OCP E4M3 "fn") and fp32 scales S [out/128][in/128], one
 * per 128 x 128 block, row-major: W[n][k] = W8[n][k] * S[n/128][k/128]. Each
 * call computes what its bf16 counterpart computes with that W (bf16
 * activations and outputs, fp32 accumulation; the bytes are widened exactly
 * and each 64-wide slice of a block is scaled in fp32). Workspace sizes are
 * those of the bf16 calls (mfa_qproj_workspace_size(B, MFA_BF16), ...).
 * mfa_kv_append_w8 writes a bf16 cache (cache_dt = MFA_BF16, scales unused)
 * or an e4m3 cache as mfa_kv_append_fp8 does (cache_dt = MFA_FP8_E4M3);
 * seq_len_out as for mfa_kv_append. mfa_qproj_kv_append_w8 is
 * mfa_qproj_kv_append with these weights (one product over the stacked
 * [W_dq; W_k; W_v] bytes, each matrix with its own scales; the same
 * workspace, mfa_qproj_kv_append_workspace_size(B), and cache_dt choices).
 * Scale arrays: device fp32, 4-byte aligned.
 */
int mfa_qproj_w8(const void* x, const void* w_dq, const float* s_dq, const float* gamma, float eps,
                 const void* w_uq, const float* s_uq, void* q_out, void* ws, size_t ws_bytes, int B,
                 void* stream);
int mfa_kv_append_w8(const void* x, const void* w_k, const float* s_k, const void* w_v, const float* s_v,
                     void* k_cache, void* v_cache, const int64_t* seq_off, const int32_t* seq_len,
                     int32_t* seq_len_out, mfa_dtype cache_dt, float k_scale, float v_scale, void* ws,
                     size_t ws_bytes, int B, void* stream);
int mfa_oproj_w8(const void* attn, const void* w_o, const float* s_o, void* y, void* ws, size_t ws_bytes,
                 int B, void* stream);
int mfa_qproj_kv_append_w8(const void* x, const void* w_dq, const float* s_dq, const float* gamma, float eps,
                           const void* w_uq, const float* s_uq, const void* w_k, const float* s_k, const void* w_v,
                           const float* s_v, void* q_out, void* k_cache, void* v_cache, const int64_t* seq_off,
                           const int32_t* seq_len, int32_t* seq_len_out, float k_scale, float v_scale, void* ws,
                           size_t ws_bytes, int B, mfa_dtype cache_dt, void* stream);

/* ------------------------------------------------------------------ bandwidth probe
 * Measures the achievable HBM read rate that the attention kernels' KV rate
 * is compared with: num_workgroups workgroups (0: one per CU) read the
 * bytes of buf (device, 16-byte aligned, bytes a non-zero multiple of 16)
 * with 16-byte loads, and workgroup i writes the XOR of the 32-bit words it
 * read to sink[i] (device uint32 array with num_workgroups entries, or one
 * per CU when num_workgroups is 0). The XOR of all sink entries is the XOR
 * of every 32-bit word of buf. Errors: MFA_ERR_INVALID_ARG (null pointer,
 * bad size or count), MFA_ERR_ALIGNMENT.
 */
int mfa_bw_probe(const void* buf, size_t bytes, uint32_t* sink, int num_workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MFA_H_ */
