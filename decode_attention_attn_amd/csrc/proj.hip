// Projection kernels of the MFA decode layer on gfx950: the low-rank query
// path (7168 -> 2048 -> RMSNorm -> 16384), the shared K/V projections
// (7168 -> 256 each, appended to the cache) and the out-projection
// (16384 -> 7168). Step-3 paper summary, "Method": the decode cost model
// counts these as the "linear projections" term.
//
// At decode time M = batch is small (2..128) and every weight byte is used M
// times, so these products are bound by streaming the weights from HBM. The
// bf16 kernel therefore tiles 128 weight rows x 128 batch rows per workgroup,
// stages both operands through a 4-deep LDS ring filled by direct-to-LDS DMA
// (weights read exactly once, as 128 B runs), and multiplies with
// v_mfma_f32_16x16x32_bf16. The weight tile is the MFMA A operand, so each
// lane ends up with four consecutive output columns of one batch row (one
// 16-byte store). When the output tile count alone cannot fill the GPU, the
// K dimension is split and fp32 partial sums go to the workspace; a small
// epilogue kernel adds them and applies what follows the product (RMSNorm of
// the latent, the cache-row scatter of K/V, or the cast of y).
// The fp32 path (used for exact-ish parity at tiny batch) is a VALU GEMV.
#include "mfa_common.h"
#include "mfa_internal.h"

namespace mfa {

constexpr int kGN = 128;    // output columns (weight rows) per workgroup (narrow tile)
constexpr int kGM = 128;    // batch rows per workgroup
constexpr int kGK = 64;     // K per stage

// Tile shapes. Every wave owns 32 batch rows x 128 output columns. The wide
// tile (8 waves, 256 columns) reads each activation chunk once per 256
// weight rows instead of 128, which halves the activation share of the bytes
// a workgroup streams; it is used for the wide products (the out-projection).
// W8: block-fp8 weights (e4m3 bytes, 64-byte rows per chunk), widened to bf16
// in registers; the ring then holds 4 stages of 24 KB or 32 KB.
template <int NW, bool W8 = false>
struct GTile {
  static constexpr int kN = NW;                      // output columns per workgroup
  static constexpr int kWaves = NW / 32;             // 4 or 8
  static constexpr int kStages = (NW == 128 || W8) ? 4 : 3;
  static constexpr int kWRow = W8 ? kGK : kGK * 2;   // bytes of one weight row per chunk
  static constexpr int kWBytes = NW * kWRow;         // weight tile
  static constexpr int kXBytes = kGM * kGK * 2;      // activation tile (16 KB)
  static constexpr int kStageBytes = kWBytes + kXBytes;
  static constexpr int kDmaPerWave = (kStageBytes / 1024) / kWaves;  // 8 or 6
  static constexpr int kSteadyVm = (kStages - 2) * kDmaPerWave;
};

struct GemmArgs {
  const bf16* X;
  const bf16* W0;  // (e4m3 bytes for block-fp8 weights)
  const bf16* W1;
  void* Y;
  int M, N, K, N0, S;
  const float* S0;  // block-fp8: [rows / 128][K / 128] scales of W0 / W1
  const float* S1;
};

// 16-byte chunk swizzle for the 64-byte rows of a block-fp8 weight chunk:
// the 16 rows one MFMA fragment reads at a time land on distinct banks.
__device__ __forceinline__ int gswz8(int r) { return (r >> 2) & 3; }

// 16-byte chunk swizzle for 128-byte rows: ds_read_b128 of 16 consecutive rows
// at one logical chunk runs without bank conflicts on gfx950 (measured with
// SQ_LDS_BANK_CONFLICT; (r & 7) ^ ((r >> 3) & 1) costs about four conflict
// cycles per read).
__device__ __forceinline__ int gswz(int r) { return r & 7; }

// One K chunk of the weight tile (T::kN rows) and the activation tile (128
// rows) into a ring stage: 1 KB blocks of 8 rows x 128 B, dealt evenly to
// the waves (weight blocks first).
template <int NW, bool W8>
__device__ __forceinline__ void gemm_issue(const GemmArgs& a, int n0, int m0, int kc, char* stage, int w, int lane) {
  using T = GTile<NW, W8>;
  const int r_in = lane >> 3;  // 8 rows of 128 B per 1 KB block
  const int pc = lane & 7;
  const int k0 = kc * kGK;
  constexpr int kWBlocks = T::kWBytes / 1024;
  // Weight rows of the wide bf16 tile (the out-projection) stream with the
  // nontemporal cache policy: 71 -> 66.5 us for it on MI355X; the same policy
  // made the narrower and block-fp8 tiles slower (q path 44 -> 48 us), so they
  // keep the default.
  constexpr int kWCpol = (NW == 256 && !W8) ? 2 : 0;
#pragma unroll
  for (int jj = 0; jj < T::kDmaPerWave; ++jj) {
    const int blk = T::kDmaPerWave * w + jj;
    if (W8 && blk < kWBlocks) {
      // 16 rows of 64 B per 1 KB block
      const int r = 16 * blk + (lane >> 2);
      const int c = (lane & 3) ^ gswz8(r);
      const int n = n0 + r;
      const unsigned char* wrow = n < a.N0 ? (const unsigned char*)a.W0 + (long long)n * a.K
                                            : (const unsigned char*)a.W1 + (long long)(n - a.N0) * a.K;
      __builtin_amdgcn_global_load_lds((const void*)(wrow + k0 + c * 16), (MFA_LDS void*)(stage + blk * 1024), 16,
                                       0, 0);
    } else if (blk < kWBlocks) {
      const int r = 8 * blk + r_in;
      const int c = pc ^ gswz(r);
      const int n = n0 + r;
      const bf16* wrow = n < a.N0 ? a.W0 + (long long)n * a.K : a.W1 + (long long)(n - a.N0) * a.K;
      __builtin_amdgcn_global_load_lds((const void*)(wrow + k0 + c * 8), (MFA_LDS void*)(stage + blk * 1024), 16, 0,
                                       kWCpol);
    } else {
      const int r = 8 * (blk - kWBlocks) + r_in;
      const int c = pc ^ gswz(r);
      int m = m0 + r;
      m = m < a.M ? m : a.M - 1;
      const bf16* xrow = a.X + (long long)m * a.K;
      __builtin_amdgcn_global_load_lds((const void*)(xrow + k0 + c * 8), (MFA_LDS void*)(stage + blk * 1024), 16, 0,
                                       0);
    }
  }
}

template <GemmOut MODE, int NW, bool W8 = false>
__global__ __launch_bounds__(NW * 2, 1) void gemm_bf16_kernel(GemmArgs a) {
  using T = GTile<NW, W8>;
  constexpr int kGStages = T::kStages;
  constexpr int kGStageBytes = T::kStageBytes;
  constexpr int kGSteadyVm = T::kSteadyVm;
  __shared__ __attribute__((aligned(1024))) char ring[kGStages * kGStageBytes];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int w = wave & 3;            // batch rows 32w..32w+31 of the tile
  const int wn = (wave >> 2) * 128;  // this wave's 128 output columns within the tile
  const int i16 = lane & 15;
  const int g = lane >> 4;
  const int n0 = blockIdx.x * T::kN;
  const int split = blockIdx.y;
  const int m0 = blockIdx.z * kGM;
  const int nch = a.K / kGK;
  const int c_begin = (int)((long long)split * nch / a.S);
  const int c_end = (int)((long long)(split + 1) * nch / a.S);
  const int nloc = c_end - c_begin;

  f32x4 acc[2][8];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) acc[mi][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Block-fp8 weights: this wave's 128 weight rows form one row of scale
  // blocks, so a 64-wide K chunk has one scale (blocks are 128 x 128). The
  // row index is wave-uniform, so the scale reads are scalar loads, which do
  // not touch the vector-memory counter the DMA ring waits on; each chunk's
  // scale is read one chunk ahead.
  const float* srow = nullptr;
  float sc_next = 0.f;
  if constexpr (W8) {
    const int nrow = n0 + __builtin_amdgcn_readfirstlane(wn);
    srow = nrow < a.N0 ? a.S0 + (long long)(nrow >> 7) * (a.K >> 7)
                       : a.S1 + (long long)((nrow - a.N0) >> 7) * (a.K >> 7);
    if (nloc > 0) sc_next = load_scalar(srow, c_begin >> 1);
  }

  int issued = 0;
#pragma unroll
  for (int s = 0; s < kGStages - 1; ++s)
    if (issued < nloc) {
      gemm_issue<NW, W8>(a, n0, m0, c_begin + issued, ring + s * kGStageBytes, wave, lane);
      ++issued;
    }

  for (int t = 0; t < nloc; ++t) {
    if (issued - t - 1 >= kGStages - 2)
      wait_vmcnt<kGSteadyVm>();
    else
      wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (issued < nloc) {
      gemm_issue<NW, W8>(a, n0, m0, c_begin + issued, ring + ((t + kGStages - 1) % kGStages) * kGStageBytes, wave,
                         lane);
      ++issued;
    }
    const char* xs = ring + (t % kGStages) * kGStageBytes + T::kWBytes;
    if constexpr (W8) {
      // The chunk's product is formed from the exact bf16 widening of the
      // bytes, then scaled into the accumulator in fp32.
      const float sc = sc_next;
      sc_next = load_scalar(srow, (c_begin + (t + 1 < nloc ? t + 1 : t)) >> 1);
      const char* ws8 = ring + (t % kGStages) * kGStageBytes + wn * T::kWRow;
      f32x4 tmp[2][8];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = 4 * j + g;  // 8-element chunk of the 64: bytes 8c..8c+7 of the row
        bf16x8 wa[8], xb[2];
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          const int r = 16 * nb + i16;
          const u32x2 raw = *(const MFA_LDS u32x2*)(ws8 + r * 64 + ((((c >> 1) ^ gswz8(r))) << 4) + ((c & 1) << 3));
          fp8x4_to_bf16(raw[0], wa[nb], 0);
          fp8x4_to_bf16(raw[1], wa[nb], 4);
        }
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
          const int r = 16 * (2 * w + mi) + i16;
          xb[mi] = *(const MFA_LDS bf16x8*)(xs + r * 128 + ((c ^ gswz(r)) << 4));
        }
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int nb = 0; nb < 8; ++nb)
            tmp[mi][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                wa[nb], xb[mi], j == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : tmp[mi][nb], 0, 0, 0);
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) acc[mi][nb] += tmp[mi][nb] * sc;
      continue;
    }
    const char* ws = ring + (t % kGStages) * kGStageBytes + wn * 128;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = 4 * j + g;
      bf16x8 wa[8], xb[2];
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const int r = 16 * nb + i16;
        wa[nb] = *(const MFA_LDS bf16x8*)(ws + r * 128 + ((c ^ gswz(r)) << 4));
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int r = 16 * (2 * w + mi) + i16;
        xb[mi] = *(const MFA_LDS bf16x8*)(xs + r * 128 + ((c ^ gswz(r)) << 4));
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
          acc[mi][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[nb], xb[mi], acc[mi][nb], 0, 0, 0);
    }
  }

  // lane (i16, g), register i of acc[mi][nb] = Y[m0 + 16(2w+mi) + i16][n0 + 16nb + 4g + i]
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    const int m = m0 + 16 * (2 * w + mi) + i16;
    if (m >= a.M) continue;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const int n = n0 + wn + 16 * nb + 4 * g;
      if constexpr (MODE == GemmOut::Partial) {
        float* dst = (float*)a.Y + ((long long)split * a.M + m) * a.N + n;
        *(f32x4*)dst = acc[mi][nb];
      } else {
        bf16* dst = (bf16*)a.Y + (long long)m * a.N + n;
        const bf16x4 o = {(bf16)acc[mi][nb][0], (bf16)acc[mi][nb][1], (bf16)acc[mi][nb][2], (bf16)acc[mi][nb][3]};
        *(bf16x4*)dst = o;
      }
    }
  }
}

// fp32 GEMV-style product: one wave per output column, rows of X in groups of 4.
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* X, const float* W0, const float* W1, float* Y,
                                                       int M, int N, int K, int N0) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const float* wrow = n < N0 ? W0 + (long long)n * K : W1 + (long long)(n - N0) * K;
  for (int mb = 0; mb < M; mb += 4) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int k = 4 * lane; k < K; k += 256) {
      const f32x4 wv = *(const f32x4*)(wrow + k);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        if (mb + mi < M) {
          const f32x4 xv = *(const f32x4*)(X + (long long)(mb + mi) * K + k);
          acc[mi] = fmaf(wv[0], xv[0], acc[mi]);
          acc[mi] = fmaf(wv[1], xv[1], acc[mi]);
          acc[mi] = fmaf(wv[2], xv[2], acc[mi]);
          acc[mi] = fmaf(wv[3], xv[3], acc[mi]);
        }
      }
    }
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      float v = acc[mi];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
      if (lane == 0 && mb + mi < M) Y[(long long)(mb + mi) * N + n] = v;
    }
  }
}

// ------------------------------------------------------------------ epilogues
// The epilogues are latency-bound (a few MB in total): every thread keeps
// several independent 16-byte partial loads in flight instead of summing the
// splits one dependent load at a time.

// sum over s < S of the f32x4 at p + s * stride, 16 loads in flight.
__device__ __forceinline__ f32x4 sum_splits(const float* p, long long stride, int S) {
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += 16) {
    f32x4 t[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) t[k] = s0 + k < S ? *(const f32x4*)(p + (s0 + k) * stride) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 16; ++k) v += t[k];
  }
  return v;
}

template <typename OutT>
__global__ __launch_bounds__(512) void rmsnorm_reduce_kernel(const float* part, int S, int M, int N,
                                                             const float* gamma, float eps, OutT* out) {
  // one block per row; N <= 8192 and N % 2048 == 0: thread t owns columns
  // 4t + 2048i .. +3
  const int m = blockIdx.x;
  const int t = threadIdx.x;
  f32x4 c[4];
  float ss = 0.f;
  const int per = N / 2048;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < per) {
      c[i] = sum_splits(part + (long long)m * N + 4 * t + 2048 * i, (long long)M * N, S);
      ss += c[i][0] * c[i][0] + c[i][1] * c[i][1] + c[i][2] * c[i][2] + c[i][3] * c[i][3];
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
  __shared__ float red[8];
  if ((t & 63) == 0) red[t >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3] + red[4] + red[5] + red[6] + red[7];
  const float r = rsqrtf(tot / (float)N + eps);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < per) {
      const int col = 4 * t + 2048 * i;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float v = c[i][e] * r;
        if (gamma != nullptr) v *= gamma[col + e];
        out[(long long)m * N + col + e] = (OutT)v;
      }
    }
  }
}

template <typename OutT>
__global__ __launch_bounds__(256) void sum_reduce_kernel(const float* part, int S, int M, int N, OutT* out) {
  const long long i4 = (long long)blockIdx.x * 256 + threadIdx.x;  // index of 4 outputs
  const long long total4 = (long long)M * N / 4;
  if (i4 >= total4) return;
  const f32x4 v = sum_splits(part + 4 * i4, (long long)M * N, S);
  OutT* dst = out + 4 * i4;
  dst[0] = (OutT)v[0];
  dst[1] = (OutT)v[1];
  dst[2] = (OutT)v[2];
  dst[3] = (OutT)v[3];
}

// The length including the appended row, for the attention call that
// follows: written once every thread of the row's workgroup has read the old
// length (len_out may be seq_len itself: an in-place increment).
__device__ __forceinline__ void write_len_out(int32_t* len_out, int m, int32_t len) {
  if (len_out != nullptr) {
    __syncthreads();
    if (threadIdx.x == 0) len_out[m] = len + 1;
  }
}

template <typename OutT>
__global__ __launch_bounds__(128) void kv_scatter_kernel(const float* part, int S, int M, OutT* kc, OutT* vc,
                                                         const int64_t* seq_off, const int32_t* seq_len,
                                                         int32_t* len_out) {
  const int m = blockIdx.x;
  const int col = 4 * threadIdx.x;  // 0..508 of the [k | v] row
  const f32x4 v = sum_splits(part + (long long)m * 512 + col, (long long)M * 512, S);
  const int32_t len = seq_len[m];
  const long long row = seq_off[m] + (long long)len;
  OutT* dst = (col < 256 ? kc : vc) + row * 256 + (col & 255);
  dst[0] = (OutT)v[0];
  dst[1] = (OutT)v[1];
  dst[2] = (OutT)v[2];
  dst[3] = (OutT)v[3];
  write_len_out(len_out, m, len);
}

// The same rows into an e4m3 cache: stored byte = e4m3(x / scale) with round to
// nearest even, the quotient taken as x * inv (inv = 1 / scale rounded to fp32
// on the host) and clamped to the largest finite magnitude, 448 (NaN stays NaN).
__global__ __launch_bounds__(128) void kv_scatter_fp8_kernel(const float* part, int S, int M, unsigned char* kc,
                                                             unsigned char* vc, const int64_t* seq_off,
                                                             const int32_t* seq_len, float inv_k, float inv_v,
                                                             int32_t* len_out) {
  const int m = blockIdx.x;
  const int col = 4 * threadIdx.x;  // 0..508 of the [k | v] row
  const f32x4 v = sum_splits(part + (long long)m * 512 + col, (long long)M * 512, S);
  const float inv = col < 256 ? inv_k : inv_v;
  float x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float t = v[i] * inv;
    x[i] = t > 448.f ? 448.f : (t < -448.f ? -448.f : t);
  }
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);  // bytes 0, 1
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], w, true);       // bytes 2, 3
  const int32_t len = seq_len[m];
  const long long row = seq_off[m] + (long long)len;
  *(int*)((col < 256 ? kc : vc) + row * 256 + (col & 255)) = w;
  write_len_out(len_out, m, len);
}

// ------------------------------------------------------------------ host side
GemmPlan plan_gemm(bool bf16_path, int M, int N, int K, int N0, int cus) {
  GemmPlan p{M, N, K, N0, 1, 1, kGN};
  if (!bf16_path) return p;
  p.mchunks = (M + kGM - 1) / kGM;
  const int nch = K / kGK;
  // For each tile width, split K so that the workgroups fill the compute
  // units once (one per CU; a second partial wave would only lengthen the
  // tail), then pick the width with the smaller estimated time: each CU
  // streams (tile_n + 128) * K / S * 2 bytes of weights and activations, and
  // the partial sums add 2 * S * M * N * 4 bytes across the chip.
  double best = 0.0;
  for (int tn = 128; tn <= 256; tn *= 2) {
    if (N % tn != 0) continue;
    const int tiles = (N / tn) * p.mchunks;
    int s = cus / tiles;
    // at least 4 K chunks per split: below that a workgroup is all start-up
    // latency and the partial sums outgrow the weights
    const int smax = nch / 4 > 0 ? nch / 4 : 1;
    if (s > smax) s = smax;
    if (s < 1) s = 1;
    const int waves = (tiles * s + cus - 1) / cus;
    const double per_cu = (double)(tn + kGM) * K / s * 2.0 * waves;  // bytes, ~30 GB/s per CU
    const double partial = s > 1 ? 2.0 * s * M * (double)N * 4.0 : 0.0;  // bytes, ~5 TB/s chip-wide
    const double t = per_cu / 30e9 + partial / 5e12;
    if (best == 0.0 || t < best) {
      best = t;
      p.tile_n = tn;
      p.splits = s;
    }
  }
  return p;
}

size_t gemm_partial_bytes(const GemmPlan& p) { return (size_t)p.splits * p.M * p.N * sizeof(float); }

hipError_t launch_gemm(bool bf16_path, const GemmPlan& p, const void* X, const void* W0, const void* W1, void* Y,
                       GemmOut mode, hipStream_t stream, const float* S0, const float* S1) {
  if (!bf16_path) {
    return launch(gemm_f32_kernel, dim3((p.N + 3) / 4), dim3(256), stream, (const float*)X, (const float*)W0,
                       (const float*)W1, (float*)Y, p.M, p.N, p.K, p.N0);
  }
  GemmArgs a{(const bf16*)X, (const bf16*)W0, (const bf16*)W1, Y, p.M, p.N, p.K, p.N0, p.splits, S0, S1};
  const dim3 grid(p.N / p.tile_n, p.splits, p.mchunks);
  if (S0 != nullptr) {  // block-fp8 weights
    if (p.tile_n == 256)
      return mode == GemmOut::Partial
                 ? launch(gemm_bf16_kernel<GemmOut::Partial, 256, true>, grid, dim3(512), stream, a)
                 : launch(gemm_bf16_kernel<GemmOut::Direct, 256, true>, grid, dim3(512), stream, a);
    return mode == GemmOut::Partial ? launch(gemm_bf16_kernel<GemmOut::Partial, 128, true>, grid, dim3(256), stream, a)
                                    : launch(gemm_bf16_kernel<GemmOut::Direct, 128, true>, grid, dim3(256), stream, a);
  }
  if (p.tile_n == 256) {
    if (mode == GemmOut::Partial) return launch(gemm_bf16_kernel<GemmOut::Partial, 256>, grid, dim3(512), stream, a);
    return launch(gemm_bf16_kernel<GemmOut::Direct, 256>, grid, dim3(512), stream, a);
  }
  if (mode == GemmOut::Partial) return launch(gemm_bf16_kernel<GemmOut::Partial, 128>, grid, dim3(256), stream, a);
  return launch(gemm_bf16_kernel<GemmOut::Direct, 128>, grid, dim3(256), stream, a);
}

hipError_t launch_rmsnorm_reduce(bool bf16_path, const float* part, int S, int M, int N, const float* gamma, float eps,
                                 void* out, hipStream_t stream) {
  if (bf16_path)
    return launch(rmsnorm_reduce_kernel<bf16>, dim3(M), dim3(512), stream, part, S, M, N, gamma, eps,
                       (bf16*)out);
  else
    return launch(rmsnorm_reduce_kernel<float>, dim3(M), dim3(512), stream, part, S, M, N, gamma, eps,
                       (float*)out);
}

hipError_t launch_sum_reduce(bool bf16_path, const float* part, int S, int M, int N, void* out, hipStream_t stream) {
  const long long total4 = (long long)M * N / 4;
  const dim3 grid((unsigned)((total4 + 255) / 256));
  if (bf16_path)
    return launch(sum_reduce_kernel<bf16>, grid, dim3(256), stream, part, S, M, N, (bf16*)out);
  else
    return launch(sum_reduce_kernel<float>, grid, dim3(256), stream, part, S, M, N, (float*)out);
}

hipError_t launch_kv_scatter(bool bf16_path, const float* part, int S, int M, void* k_cache, void* v_cache,
                             const int64_t* seq_off, const int32_t* seq_len, int32_t* len_out, hipStream_t stream) {
  if (bf16_path)
    return launch(kv_scatter_kernel<bf16>, dim3(M), dim3(128), stream, part, S, M, (bf16*)k_cache,
                       (bf16*)v_cache, seq_off, seq_len, len_out);
  else
    return launch(kv_scatter_kernel<float>, dim3(M), dim3(128), stream, part, S, M, (float*)k_cache,
                       (float*)v_cache, seq_off, seq_len, len_out);
}

hipError_t launch_kv_scatter_fp8(const float* part, int S, int M, void* k_cache, void* v_cache,
                                 const int64_t* seq_off, const int32_t* seq_len, float inv_k, float inv_v,
                                 int32_t* len_out, hipStream_t stream) {
  return launch(kv_scatter_fp8_kernel, dim3(M), dim3(128), stream, part, S, M, (unsigned char*)k_cache,
                (unsigned char*)v_cache, seq_off, seq_len, inv_k, inv_v, len_out);
}

}  // namespace mfa
