// Projection kernels of the MFA decode layer on gfx950: the low-rank query
// path (7168 -> 2048 -> RMSNorm -> 16384), the shared K/V projections
// (7168 -> 256 each, appended to the cache) and the out-projection
// (16384 -> 7168). Step-3 paper summary, "Method": the decode cost model
// counts these as the "linear projections" term.
//
// At decode time M = batch is small (2..128) and every weight byte is used M
// times, so these products are bound by streaming the weights from HBM. The
// MFMA kernel therefore tiles 64..256 weight rows x 128 batch rows per
// workgroup, stages both operands through a 4-deep LDS ring filled by
// direct-to-LDS DMA (weights read exactly once), and multiplies with
// v_mfma_f32_16x16x32_bf16 (block-fp8 weights are widened to bf16 in
// registers and scaled per 128-wide K block). The weight tile is the MFMA A
// operand, so each lane ends up with four consecutive output columns of one
// batch row (one 16-byte store). When the output tile count alone cannot fill the GPU, the
// K dimension is split and fp32 partial sums go to the workspace; a small
// epilogue kernel adds them and applies what follows the product (RMSNorm of
// the latent, the cache-row scatter of K/V, or the cast of y).
// The fp32 path (used for exact-ish parity at tiny batch) is a VALU GEMV.
#include "mfa_common.h"
#include "mfa_internal.h"

namespace mfa {

constexpr int kGM = kGemmTileM;  // batch rows per workgroup
constexpr int kGK = kGemmChunkK; // K per stage

// Weight rows n < N0 come from W0, N0 <= n < N1 from W1, n >= N1 from W2
// (N1 = N: two matrices), block-fp8 scales from S0, S1, S2 alike.
struct GemmArgs {
  const bf16* X;
  const bf16* W0;  // (e4m3 bytes for block-fp8 weights)
  const bf16* W1;
  void* Y;
  int M, N, K, N0, S;
  const float* S0;  // block-fp8: [rows / 128][K / 128] scales of W0 / W1 / W2
  const float* S1;
  const bf16* W2;
  int N1;
  const float* S2;
};

// 16-byte chunk swizzle for the 64-byte rows of a block-fp8 weight chunk: a
// fragment read takes one whole 16-byte chunk (16 k values) of 16 rows, and
// the 8 lanes the LDS serves per clock (rows r..r+7 at one logical chunk) hit
// 8 distinct 16-byte bank groups of the 128 bytes: rows two apart share a
// 128-byte bank line, so the chunk position cycles with r >> 1.
__device__ __forceinline__ int gswz8(int r) { return (r >> 1) & 3; }

// 16-byte LDS read of raw bytes; the __restrict__ parameter keeps the compiler
// from waiting for the in-flight LDS DMAs before it (as for lds_read_b128).
__device__ __forceinline__ u32x4 lds_read_u128(const MFA_LDS u32x4* __restrict__ p) { return *p; }

// 16-byte chunk swizzle for 128-byte rows: ds_read_b128 of 16 consecutive rows
// at one logical chunk runs without bank conflicts on gfx950 (measured with
// SQ_LDS_BANK_CONFLICT; (r & 7) ^ ((r >> 3) & 1) costs about four conflict
// cycles per read).
__device__ __forceinline__ int gswz(int r) { return r & 7; }

// Activation chunks under block-fp8 weights. There k-block j of a lane in
// k-slot group g takes 16-byte chunk 2g + j of the activation row (the order
// of the weight bytes), where bf16 weights take chunk 4j + g; read at the
// same swizzle, that order cost 4 conflict cycles per read (measured). So
// chunk c is stored where bf16 keeps chunk ((c & 1) << 2) | (c >> 1) (its
// three bits rotated, 2g + j -> 4j + g), and the block-fp8 activation reads
// use the very addresses of the bf16 ones. act8_chunk is the inverse
// rotation: LDS chunk slot p of a row (before the swizzle) holds activation
// chunk act8_chunk(p).
__device__ __forceinline__ int act8_chunk(int p) { return ((p & 3) << 1) | (p >> 2); }

// ------------------------------------------------------------------ MFMA product
// The product for bf16 and block-fp8 weights. A workgroup of eight waves (two per SIMD)
// owns TN weight rows x 128 batch rows and one K range; each 64-wide K chunk
// of both operands goes HBM -> LDS by direct-to-LDS DMA into a ring, every
// wave issuing its share, one barrier per chunk. Wave w owns 16 WN weight rows
// x 16 WM batch rows. Measured on MI355X: LDS reads (about 128 B per clock
// per CU) and MFMAs (16 clocks per 16x16x32 per SIMD) of one wave barely
// overlap, and together they take about as long per chunk as the chunk's
// weight bytes take to arrive, so the wave tile keeps LDS reads down
// (each fragment feeds WM or WN MFMAs), two waves per SIMD fill each other's
// gaps, and the second k-block's fragments are read while the first
// k-block's MFMAs run. bf16 weights: TN = 64 for products whose activations
// stay in L2, 128 (weights read nontemporal) for the out-projection.
// Block-fp8 weights (W8, 64-byte rows per chunk): TN = 128, or 256 for the
// out-projection, so a chunk stage holds about as many bytes as for bf16.
template <int TN, int WN, int WM, bool W8 = false>
struct PTile {
  static constexpr int kWaves = 8;
  static constexpr int kWavesN = TN / (16 * WN);
  static constexpr int kWavesM = 8 / WM;
  static_assert(kWavesN * kWavesM == kWaves, "wave grid");
  static constexpr int kWRow = W8 ? 64 : 128;              // bytes of a weight row per chunk (64 e4m3 / bf16)
  static constexpr int kWBytes = TN * kWRow;
  static constexpr int kXBytes = kGM * 128;                // activation rows x 64 bf16
  static constexpr int kStageBytes = kWBytes + kXBytes;
  // three chunks in flight (measured on MI355X: five in flight for either width,
  // or six stages of the 64-column tile, no faster; 64 columns 0.3-1.3 us slower)
  static constexpr int kStages = 4;
  static_assert(kStages * kStageBytes <= 160 * 1024, "LDS");
  static constexpr int kDpw = kStageBytes / 1024 / kWaves;  // 1 KB DMAs per wave per chunk
  static_assert(kDpw * kWaves * 1024 == kStageBytes, "DMA blocks dealt evenly");
  static_assert((kStages - 1) * kDpw < 64, "DMAs in flight exceed the wait counter");
};

// lgkmcnt(0) only: this wave's LDS reads have completed.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

template <int TN, int WN, int WM, bool W8>
__device__ __forceinline__ void pipe_issue(const GemmArgs& a, int n0, int m0, int kc, char* stage, int w, int lane) {
  using T = PTile<TN, WN, WM, W8>;
  const int r_in = lane >> 3;  // 8 rows of 128 B per 1 KB block
  const int pc = lane & 7;
  const int k0 = kc * kGK;
  constexpr int kWBlocks = T::kWBytes / 1024;
#pragma unroll
  for (int jj = 0; jj < T::kDpw; ++jj) {
    const int blk = T::kDpw * w + jj;  // weight blocks first, then activation blocks
    if (W8 && blk < kWBlocks) {
      // 16 rows of 64 weight bytes per 1 KB block, chunks swizzled by gswz8
      const int r = 16 * blk + (lane >> 2);
      const int n = n0 + r;
      const unsigned char* wrow = n < a.N0   ? (const unsigned char*)a.W0 + (long long)n * a.K
                                  : n < a.N1 ? (const unsigned char*)a.W1 + (long long)(n - a.N0) * a.K
                                             : (const unsigned char*)a.W2 + (long long)(n - a.N1) * a.K;
      __builtin_amdgcn_global_load_lds((const void*)(wrow + k0 + ((lane & 3) ^ gswz8(r)) * 16),
                                       (MFA_LDS void*)(stage + blk * 1024), 16, 0, 0);
    } else if (blk < kWBlocks) {
      const int r = 8 * blk + r_in;
      const int n = n0 + r;
      const bf16* wrow = n < a.N0   ? a.W0 + (long long)n * a.K
                         : n < a.N1 ? a.W1 + (long long)(n - a.N0) * a.K
                                    : a.W2 + (long long)(n - a.N1) * a.K;
      // (the 128-column tile streams its weights nontemporal)
      __builtin_amdgcn_global_load_lds((const void*)(wrow + k0 + (pc ^ gswz(r)) * 8),
                                       (MFA_LDS void*)(stage + blk * 1024), 16, 0, TN == 128 ? 2 : 0);
    } else {
      const int r = 8 * (blk - kWBlocks) + r_in;
      int m = m0 + r;
      m = m < a.M ? m : a.M - 1;
      const int c = W8 ? act8_chunk(pc ^ gswz(r)) : pc ^ gswz(r);  // the chunk LDS slot pc of row r holds
      __builtin_amdgcn_global_load_lds((const void*)(a.X + (long long)m * a.K + k0 + c * 8),
                                       (MFA_LDS void*)(stage + blk * 1024), 16, 0, 0);
    }
  }
}

// W8: block-fp8 weights (e4m3 bytes, one fp32 scale per 128 x 128 block). A
// lane reads one whole 16-byte chunk of its weight row (16 k values) and feeds
// its halves to the chunk's two MFMAs, the activation fragments taking the
// same contraction order (16-byte chunk 2g + j of the activation row for MFMA
// j); the bytes are widened to bf16 exactly, each chunk's product goes to a
// zeroed fp32 tile and is added to the accumulators times the chunk's block
// scale (a wave's weight rows lie in one block row, a 64-wide chunk in one
// block column).
template <GemmOut MODE, int TN, int WN, int WM, bool W8 = false>
__global__ __launch_bounds__(512, 1) void gemm_pipe_kernel(GemmArgs a) {
  using T = PTile<TN, WN, WM, W8>;
  __shared__ __attribute__((aligned(1024))) char ring[T::kStages * T::kStageBytes];
  const int lane = threadIdx.x & 63;
  const int wave = uniform((int)(threadIdx.x >> 6));
  const int wn = (wave % T::kWavesN) * 16 * WN;  // this wave's weight rows within the tile
  const int wm = (wave / T::kWavesN) * 16 * WM;  // and batch rows
  const int i16 = lane & 15;
  const int g = lane >> 4;
  const int n0 = blockIdx.x * TN;
  const int split = blockIdx.y;
  const int m0 = blockIdx.z * kGM;
  const int nch = a.K / kGK;
  const int c_begin = (int)((long long)split * nch / a.S);
  const int c_end = (int)((long long)(split + 1) * nch / a.S);
  const int nloc = c_end - c_begin;

  f32x4 acc[WN][WM];
#pragma unroll
  for (int nb = 0; nb < WN; ++nb)
#pragma unroll
    for (int mb = 0; mb < WM; ++mb) acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 tmp[W8 ? WN : 1][W8 ? WM : 1];  // W8: one chunk's product before its scale
  u32x4 raw8[W8 ? WN : 1];              // W8: the weight bytes of the chunk being multiplied
  const float* srow = nullptr;          // W8: this wave's row of block scales
  if constexpr (W8) {
    const int nrow = n0 + wn;
    srow = nrow < a.N0   ? a.S0 + (long long)(nrow >> 7) * (a.K >> 7)
           : nrow < a.N1 ? a.S1 + (long long)((nrow - a.N0) >> 7) * (a.K >> 7)
                         : a.S2 + (long long)((nrow - a.N1) >> 7) * (a.K >> 7);
  }

  // fragments of k-block j (32 of the chunk's 64) of chunk t: lane (i16, g)
  // holds elements 32j + 8g .. +7 (W8: 16g + 8j .. +7) of weight row
  // 16nb + i16 and of batch row 16mb + i16. W8: frags reads the batch rows
  // only; the chunk's weight bytes are read once by read_w8 and widened to
  // bf16 per k-block by widen, away from the reads, so that the LDS latency
  // hides behind MFMAs.
  auto frags = [&](int t, int j, bf16x8 (&wa)[WN], bf16x8 (&xb)[WM]) {
    const char* st = ring + (t % T::kStages) * T::kStageBytes;
    const char* ws = st + wn * T::kWRow;
    const char* xs = st + T::kWBytes + wm * 128;
    // (W8: activation chunk 2g + j, which the DMA stored in slot 4j + g)
    const int off = ((4 * j + g) ^ gswz(i16)) << 4;
    if constexpr (!W8) {
#pragma unroll
      for (int nb = 0; nb < WN; ++nb) wa[nb] = lds_read_b128((const MFA_LDS bf16x8*)(ws + (16 * nb + i16) * 128 + off));
    }
#pragma unroll
    for (int mb = 0; mb < WM; ++mb) xb[mb] = lds_read_b128((const MFA_LDS bf16x8*)(xs + (16 * mb + i16) * 128 + off));
  };
  auto read_w8 = [&](int t) {
    const char* ws = ring + (t % T::kStages) * T::kStageBytes + wn * T::kWRow;
#pragma unroll
    for (int nb = 0; nb < WN; ++nb) {
      const int r = 16 * nb + i16;
      raw8[nb] = lds_read_u128((const MFA_LDS u32x4*)(ws + r * 64 + ((g ^ gswz8(r)) << 4)));
    }
  };
  auto widen = [&](int j, bf16x8 (&wa)[WN]) {
#pragma unroll
    for (int nb = 0; nb < WN; ++nb) {
      fp8x4_to_bf16(raw8[nb][2 * j], wa[nb], 0);
      fp8x4_to_bf16(raw8[nb][2 * j + 1], wa[nb], 4);
    }
  };
  // j = 0 / 1: the chunk's first / second k-block (W8: into tmp, then scaled
  // in by sc, the chunk's block scale)
  auto mfmas = [&](float sc, int j, const bf16x8 (&wa)[WN], const bf16x8 (&xb)[WM]) {
    if constexpr (W8) {
#pragma unroll
      for (int nb = 0; nb < WN; ++nb)
#pragma unroll
        for (int mb = 0; mb < WM; ++mb)
          tmp[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[nb], xb[mb], j == 0 ? f32x4{0.f, 0.f, 0.f, 0.f}
                                                                                  : tmp[nb][mb], 0, 0, 0);
      if (j == 1) {
#pragma unroll
        for (int nb = 0; nb < WN; ++nb)
#pragma unroll
          for (int mb = 0; mb < WM; ++mb) acc[nb][mb] += tmp[nb][mb] * sc;
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < WN; ++nb)
#pragma unroll
        for (int mb = 0; mb < WM; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[nb], xb[mb], acc[nb][mb], 0, 0, 0);
    }
  };

  // Every stage starts filled; afterwards chunk t + kStages goes into the
  // stage of chunk t once all waves are past reading it.
  int issued = 0;
#pragma unroll
  for (int s = 0; s < T::kStages; ++s)
    if (issued < nloc) {
      pipe_issue<TN, WN, WM, W8>(a, n0, m0, c_begin + issued, ring + s * T::kStageBytes, wave, lane);
      ++issued;
    }
  bf16x8 wa0[WN], xb0[WM], wa1[WN], xb1[WM];
  if (nloc > 0) {
    if (issued == T::kStages)
      wait_vmcnt<(T::kStages - 1) * T::kDpw>();
    else
      wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if constexpr (W8) read_w8(0);
    frags(0, 0, wa0, xb0);
    if constexpr (W8) {
      wait_lds();
      widen(0, wa0);
    }
  }
  // Explicit LDS waits at the loop head and tail keep the compiler's own
  // wait analysis exact across the back edge (otherwise it waits for every
  // read, including those meant to overlap the MFMAs).
  wait_lds();
  for (int t = 0; t + 1 < nloc; ++t) {
    // W8: the scale's load is covered by the LDS wait after the first MFMAs
    const float sc = W8 ? load_scalar(srow, (c_begin + t) >> 1) : 0.f;
    frags(t, 1, wa1, xb1);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (W8) widen(1, wa1);
    mfmas(sc, 0, wa0, xb0);
    __builtin_amdgcn_sched_barrier(0);
    wait_lds();  // done reading chunk t
    // chunk t + 1 has landed once at most the chunks after it are in flight
    if (issued - (t + 2) >= T::kStages - 2)
      wait_vmcnt<(T::kStages - 2) * T::kDpw>();
    else
      wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (issued < nloc) {
      pipe_issue<TN, WN, WM, W8>(a, n0, m0, c_begin + issued, ring + (issued % T::kStages) * T::kStageBytes, wave,
                                 lane);
      ++issued;
    }
    if constexpr (W8) read_w8(t + 1);
    frags(t + 1, 0, wa0, xb0);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(sc, 1, wa1, xb1);
    __builtin_amdgcn_sched_barrier(0);
    wait_lds();
    if constexpr (W8) widen(0, wa0);
  }
  if (nloc > 0) {
    const float sc = W8 ? load_scalar(srow, (c_begin + nloc - 1) >> 1) : 0.f;
    frags(nloc - 1, 1, wa1, xb1);
    if constexpr (W8) widen(1, wa1);
    mfmas(sc, 0, wa0, xb0);
    mfmas(sc, 1, wa1, xb1);
  }

  // lane (i16, g), register i of acc[nb][mb] = Y[m0 + wm + 16mb + i16][n0 + wn + 16nb + 4g + i]
#pragma unroll
  for (int mb = 0; mb < WM; ++mb) {
    const int m = m0 + wm + 16 * mb + i16;
    if (m >= a.M) continue;
#pragma unroll
    for (int nb = 0; nb < WN; ++nb) {
      const int n = n0 + wn + 16 * nb + 4 * g;
      if constexpr (MODE == GemmOut::Partial) {
        float* dst = (float*)a.Y + ((long long)split * a.M + m) * a.N + n;
        *(f32x4*)dst = acc[nb][mb];
      } else {
        bf16* dst = (bf16*)a.Y + (long long)m * a.N + n;
        const bf16x4 o = {(bf16)acc[nb][mb][0], (bf16)acc[nb][mb][1], (bf16)acc[nb][mb][2], (bf16)acc[nb][mb][3]};
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

// The same sum for a split product with bf16 weights, one workgroup per
// tile_n columns x (1024 / tile_n) rows. The product's workgroup (x, split, m
// chunk) ran on XCD x % 8 when the column-tile count is a multiple of 8
// (workgroups are dealt round-robin to the 8 XCDs in launch order), so the
// sum of tile x is placed on that XCD, which wrote all of the tile's parts
// (measured on MI355X: layer step about 1 us faster). Placement only affects
// speed.
template <typename OutT, int TN>
__global__ __launch_bounds__(256) void sum_reduce_tiles_kernel(const float* part, int S, int M, int N, OutT* out) {
  constexpr int kRows = 1024 / TN;
  const int rblocks = (M + kRows - 1) / kRows;
  const int tiles = N / TN;  // a multiple of 8
  const int i = blockIdx.x;
  const int x = i & 7, j = i >> 3;
  const int tile = x + 8 * (j / rblocks);
  const int m = (j % rblocks) * kRows + threadIdx.x / (TN / 4);
  if (m >= M || tile >= tiles) return;
  const int n = tile * TN + 4 * (threadIdx.x % (TN / 4));
  const f32x4 v = sum_splits(part + (long long)m * N + n, (long long)M * N, S);
  OutT* dst = out + (long long)m * N + n;
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

// The down-projection and K/V products of one step from one GEMM over
// [W_dq; W_k; W_v] (2048 + 256 + 256 columns): row m of the summed partials
// gives c (columns 0..2047, RMS-normalized into c_hat as
// rmsnorm_reduce_kernel does) and the new K and V rows (columns 2048..2559,
// written as kv_scatter_kernel / kv_scatter_fp8_kernel do). One block of 512
// threads per row; threads 0..127 also take 4 of the 512 K/V columns each.
template <typename OutT, bool FP8KV>
__global__ __launch_bounds__(512) void qkv_epilogue_kernel(const float* part, int S, int M, const float* gamma,
                                                           float eps, OutT* chat, void* kc, void* vc,
                                                           const int64_t* seq_off, const int32_t* seq_len,
                                                           float inv_k, float inv_v, int32_t* len_out) {
  constexpr int kN = 2560, kR = 2048;
  const int m = blockIdx.x;
  const int t = threadIdx.x;
  const float* prow = part + (long long)m * kN;
  const long long stride = (long long)M * kN;
  // K/V columns first, so their loads are in flight with the latent's
  f32x4 kv = {0.f, 0.f, 0.f, 0.f};
  if (t < 128) kv = sum_splits(prow + kR + 4 * t, stride, S);
  const f32x4 c = sum_splits(prow + 4 * t, stride, S);
  float ss = c[0] * c[0] + c[1] * c[1] + c[2] * c[2] + c[3] * c[3];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
  __shared__ float red[8];
  if ((t & 63) == 0) red[t >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3] + red[4] + red[5] + red[6] + red[7];
  const float r = rsqrtf(tot / (float)kR + eps);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float v = c[e] * r;
    if (gamma != nullptr) v *= gamma[4 * t + e];
    chat[(long long)m * kR + 4 * t + e] = (OutT)v;
  }
  const int32_t len = seq_len[m];
  if (t < 128) {
    const int col = 4 * t;  // 0..508 of the [k | v] row
    const long long row = seq_off[m] + (long long)len;
    if constexpr (FP8KV) {
      const float inv = col < 256 ? inv_k : inv_v;
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float q = kv[i] * inv;
        x[i] = q > 448.f ? 448.f : (q < -448.f ? -448.f : q);
      }
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], w, true);
      *(int*)((unsigned char*)(col < 256 ? kc : vc) + row * 256 + (col & 255)) = w;
    } else {
      OutT* dst = (OutT*)(col < 256 ? kc : vc) + row * 256 + (col & 255);
      dst[0] = (OutT)kv[0];
      dst[1] = (OutT)kv[1];
      dst[2] = (OutT)kv[2];
      dst[3] = (OutT)kv[3];
    }
  }
  write_len_out(len_out, m, len);
}

// ------------------------------------------------------------------ host side
hipError_t launch_gemm(bool bf16_path, const GemmPlan& p, const void* X, const void* W0, const void* W1, void* Y,
                       GemmOut mode, hipStream_t stream, const float* S0, const float* S1, const void* W2, int N1,
                       const float* S2) {
  if (W2 == nullptr) {
    W2 = W1;
    S2 = S1;
    N1 = p.N;
  } else if (!bf16_path || (S0 != nullptr) != (S2 != nullptr) || N1 < p.N0 || N1 > p.N ||
             (S0 != nullptr && (p.N0 % 128 != 0 || N1 % 128 != 0))) {
    // a third matrix only on the MFMA path; for block-fp8 weights with its
    // scales, every matrix starting on a 128-row scale block
    return hipErrorInvalidValue;
  }
  if (!bf16_path) {
    return launch(gemm_f32_kernel, dim3((p.N + 3) / 4), dim3(256), stream, (const float*)X, (const float*)W0,
                       (const float*)W1, (float*)Y, p.M, p.N, p.K, p.N0);
  }
  // a plan is made for one weight format: block-fp8 plans use 128/256-column
  // tiles, bf16 plans 64/128-column tiles of the pipelined kernel
  if ((S0 != nullptr) != p.w8 || p.N % p.tile_n != 0) return hipErrorInvalidValue;
  GemmArgs a{(const bf16*)X, (const bf16*)W0, (const bf16*)W1, Y, p.M, p.N, p.K, p.N0, p.splits, S0, S1,
             (const bf16*)W2, N1, S2};
  const dim3 grid(p.N / p.tile_n, p.splits, p.mchunks);
  const bool part = mode == GemmOut::Partial;
  if (p.w8) {
    if (p.tile_n == 256)
      return part ? launch(gemm_pipe_kernel<GemmOut::Partial, 256, 4, 4, true>, grid, dim3(512), stream, a)
                  : launch(gemm_pipe_kernel<GemmOut::Direct, 256, 4, 4, true>, grid, dim3(512), stream, a);
    if (p.tile_n == 128)
      return part ? launch(gemm_pipe_kernel<GemmOut::Partial, 128, 4, 2, true>, grid, dim3(512), stream, a)
                  : launch(gemm_pipe_kernel<GemmOut::Direct, 128, 4, 2, true>, grid, dim3(512), stream, a);
    return hipErrorInvalidValue;
  }
  if (p.tile_n == 64)
    return part ? launch(gemm_pipe_kernel<GemmOut::Partial, 64, 2, 2>, grid, dim3(512), stream, a)
                : launch(gemm_pipe_kernel<GemmOut::Direct, 64, 2, 2>, grid, dim3(512), stream, a);
  if (p.tile_n == 128)
    return part ? launch(gemm_pipe_kernel<GemmOut::Partial, 128, 4, 2>, grid, dim3(512), stream, a)
                : launch(gemm_pipe_kernel<GemmOut::Direct, 128, 4, 2>, grid, dim3(512), stream, a);
  return hipErrorInvalidValue;
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

hipError_t launch_sum_reduce(bool bf16_path, const float* part, int S, int M, int N, void* out, hipStream_t stream,
                             int tile_n) {
  if (bf16_path && (tile_n == 64 || tile_n == 128) && N % (8 * tile_n) == 0) {
    const int rblocks = (M + 1024 / tile_n - 1) / (1024 / tile_n);
    const dim3 grid((unsigned)((N / tile_n) * rblocks));
    return tile_n == 64 ? launch(sum_reduce_tiles_kernel<bf16, 64>, grid, dim3(256), stream, part, S, M, N, (bf16*)out)
                        : launch(sum_reduce_tiles_kernel<bf16, 128>, grid, dim3(256), stream, part, S, M, N, (bf16*)out);
  }
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

hipError_t launch_qkv_epilogue(const float* part, int S, int M, const float* gamma, float eps, void* chat,
                               void* k_cache, void* v_cache, const int64_t* seq_off, const int32_t* seq_len,
                               bool fp8_cache, float inv_k, float inv_v, int32_t* len_out, hipStream_t stream) {
  if (fp8_cache)
    return launch(qkv_epilogue_kernel<bf16, true>, dim3(M), dim3(512), stream, part, S, M, gamma, eps, (bf16*)chat,
                  k_cache, v_cache, seq_off, seq_len, inv_k, inv_v, len_out);
  return launch(qkv_epilogue_kernel<bf16, false>, dim3(M), dim3(512), stream, part, S, M, gamma, eps, (bf16*)chat,
                k_cache, v_cache, seq_off, seq_len, inv_k, inv_v, len_out);
}

hipError_t launch_kv_scatter_fp8(const float* part, int S, int M, void* k_cache, void* v_cache,
                                 const int64_t* seq_off, const int32_t* seq_len, float inv_k, float inv_v,
                                 int32_t* len_out, hipStream_t stream) {
  return launch(kv_scatter_fp8_kernel, dim3(M), dim3(128), stream, part, S, M, (unsigned char*)k_cache,
                (unsigned char*)v_cache, seq_off, seq_len, inv_k, inv_v, len_out);
}

}  // namespace mfa
