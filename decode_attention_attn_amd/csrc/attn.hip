// Shared-KV decode attention for MFA on gfx950.
//
// What is computed (Step-3 paper summary, "Key claims" and "Method"): every
// one of the 64 query heads of a decoding sequence attends, with one softmax,
// over the single shared K head and single shared V head (width 256) that the
// sequence's cache holds, one row per past token. The decode cost model on the
// same page prices this step as max(attention compute, KV memory access): at
// 65,536 FLOP per 1 KB (bf16) or 512 B (fp8) cache row it sits well below the
// MI355X ridge point, so the kernel is built to stream the cache at HBM rate.
//
// Design (MI355X-first):
//  * Work split. The key ranges of all sequences are laid end to end and cut
//    into G equal pieces (G = one workgroup per CU), each a multiple of the
//    32-row tile. A workgroup walks its piece, which may cover the tail of one
//    sequence and the head of the next. Ragged lengths therefore never leave
//    CUs idle. A sequence cut into several pieces is merged afterwards by a
//    log-sum-exp combine; a sequence inside one piece is written directly.
//  * Data path. K/V tiles (32 rows) go HBM -> LDS by direct-to-LDS DMA
//    (global_load_lds_dwordx4: each lane moves 16 B, a wave moves 1 KB = 2
//    bf16 rows) into a 4-stage (bf16) or 8-stage (fp8) ring, three or seven
//    tiles ahead of the compute, one barrier per tile. Rows are XOR-swizzled
//    in 16-byte chunks at DMA time so that the MFMA operand reads below are
//    bank-conflict free; every row is still read as whole 512 B (256 B) runs.
//  * Math. The 64 heads are the dense M dimension. Wave w owns heads
//    16w..16w+15. Scores are computed transposed, S^T = K Q^T with
//    v_mfma_f32_16x16x32_bf16 (K from LDS with ds_read_b128, Q^T resident in
//    registers), so each lane ends up holding 8 scores of ONE head: the
//    online-softmax statistics stay per lane, and the exponentiated scores
//    are already laid out as the B operand of the second product
//    O^T = V^T P^T. V^T is read from LDS with the gfx950 transposing reads
//    ds_read_b64_tr_b16 (bf16) / ds_read_b64_tr_b8 (fp8), so no transpose
//    pass exists. fp8 cache bytes are widened to bf16 in registers
//    (v_cvt_scalef32_pk_bf16_fp8, exact); the per-tensor scales are folded
//    into the score multiplier (K) and the final normalisation (V).
//  * Softmax in base 2: scores are multiplied by scale*log2(e) once, the
//    running max/sum live in registers, the O accumulator is rescaled when the
//    max moves, and the row sums are reduced across the 4 lanes of a head only
//    at the end of a piece.
#include "mfa_common.h"
#include "mfa_internal.h"

namespace mfa {

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const int64_t* seq_off;
  const int32_t* seq_len;
  void* out;
  float* lse;
  float* part_o;    // [G + B][64][256] fp32, normalized partial outputs
  float* part_lse;  // [G + B][64] fp32, base-2 log-sum-exp of each partial
  int B;
  int G;
  float score_mul;  // softmax_scale * k_scale * log2(e)
  float v_mul;      // v_scale
};

constexpr int kTile = 32;  // cache rows per tile (all kernels use the same piece granularity)

// ---------------------------------------------------------------------------
// Work split shared by the attention kernels and the combine kernel. Every
// wave computes it redundantly from seq_len (B small), so no inter-wave sync.
__device__ __forceinline__ long long total_len(const int32_t* len, int B, int lane) {
  long long s = 0;
  for (int i = lane; i < B; i += 64) s += len[i];
  return wave_sum_ll(s);
}

__device__ __forceinline__ long long piece_len(long long total, int G) {
  long long per = (total + G - 1) / G;
  return (per + kTile - 1) / kTile * kTile;
}

// First sequence whose key range contains global position r0 and that
// sequence's start. Requires 0 <= r0 < total.
__device__ __forceinline__ void find_seq(const int32_t* len, int B, long long r0, int lane, int& b_out,
                                         long long& start_out) {
  long long base = 0;
  b_out = B - 1;
  start_out = 0;
  for (int c0 = 0; c0 < B; c0 += 64) {
    const int idx = c0 + lane;
    const long long v = idx < B ? (long long)len[idx] : 0;
    long long incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      long long t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    const unsigned long long hit = __ballot(idx < B && base + incl > r0);
    if (hit) {
      const int first = __ffsll((long long)hit) - 1;
      const long long incl_f = __shfl(incl, first);
      const long long v_f = __shfl(v, first);
      b_out = c0 + first;
      start_out = base + incl_f - v_f;
      return;
    }
    base += __shfl(incl, 63);
  }
}

// Exclusive prefix of len[0..b).
__device__ __forceinline__ long long seq_start_of(const int32_t* len, int b, int lane) {
  long long s = 0;
  for (int i = lane; i < b; i += 64) s += len[i];
  return wave_sum_ll(s);
}

// Walks one workgroup's piece tile by tile (wave-uniform state).
struct Cursor {
  long long gpos, r1;              // next global position, end of the workgroup's piece
  long long seq_start, seq_end;    // global range of the current sequence
  long long off;                   // cache row of the sequence's first key
  int b;

  __device__ __forceinline__ bool valid() const { return gpos < r1; }
  __device__ __forceinline__ long long part_end() const { return seq_end < r1 ? seq_end : r1; }
  // Rows [lo, hi) of the current tile, relative to the sequence start.
  __device__ __forceinline__ void tile(long long& lo, long long& hi) const {
    lo = gpos - seq_start;
    long long e = gpos + kTile;
    const long long pe = part_end();
    hi = (e < pe ? e : pe) - seq_start;
  }
  __device__ __forceinline__ void advance(const int32_t* len, const int64_t* offs) {
    const long long pe = part_end();
    long long e = gpos + kTile;
    gpos = e < pe ? e : pe;
    if (gpos == seq_end && gpos < r1) {
      do {
        ++b;
        seq_start = seq_end;
        seq_end = seq_start + load_scalar(len, b);
      } while (seq_end == seq_start);
      off = load_scalar(offs, b);
    }
  }
};

__device__ __forceinline__ bool init_cursor(const AttnArgs& a, int wg, int lane, Cursor& c) {
  const long long total = uniform(total_len(a.seq_len, a.B, lane));
  const long long per = piece_len(total, a.G);
  const long long r0 = (long long)wg * per;
  if (r0 >= total) return false;
  c.r1 = r0 + per < total ? r0 + per : total;
  c.gpos = r0;
  int b;
  long long start;
  find_seq(a.seq_len, a.B, r0, lane, b, start);
  c.b = uniform(b);
  c.seq_start = uniform(start);
  c.seq_end = c.seq_start + load_scalar(a.seq_len, c.b);
  c.off = load_scalar(a.seq_off, c.b);
  return true;
}

// ---------------------------------------------------------------------------
// MFMA kernel (bf16 q; bf16 or fp8 cache).
template <bool FP8>
struct Cfg {
  static constexpr int kRowBytes = FP8 ? 256 : 512;
  static constexpr int kTileBytes = kTile * kRowBytes;            // one of K or V
  static constexpr int kStageBytes = 2 * kTileBytes;              // K then V
  static constexpr int kStages = FP8 ? 8 : 4;
  static constexpr int kBlocks = kTileBytes / 1024;               // 1 KB DMA blocks per K (or V) tile
  static constexpr int kRowsPerBlock = 1024 / kRowBytes;          // 2 (bf16) / 4 (fp8)
  static constexpr int kDmaPerWave = 2 * kBlocks / 4;             // DMA instructions per wave per tile
  static constexpr int kSteadyVm = (kStages - 2) * kDmaPerWave;   // DMAs allowed in flight after a tile landed
};

// XOR swizzles of 16-byte chunks within a tile row (row r = 0..31 of the tile).
__device__ __forceinline__ int swz_k(int r) { return r & 15; }
__device__ __forceinline__ int swz_v16(int r) { return (r & 7) << 1; }
__device__ __forceinline__ int swz_v8(int r) { return (r & 3) | (((r >> 4) & 1) << 2) | (((r >> 2) & 1) << 3); }

template <bool FP8>
__device__ __forceinline__ void issue_tile(const AttnArgs& a, const Cursor& c, char* stage, int w, int lane) {
  using C = Cfg<FP8>;
  long long lo, hi;
  c.tile(lo, hi);
  const char* kb = (const char*)a.k + (c.off + lo) * C::kRowBytes;
  const char* vb = (const char*)a.v + (c.off + lo) * C::kRowBytes;
  const int nvalid = (int)(hi - lo);
  constexpr int kChunks = C::kRowBytes / 16;
  const int r_in = FP8 ? (lane >> 4) : (lane >> 5);
  const int pc = lane & (kChunks - 1);
#pragma unroll
  for (int jj = 0; jj < C::kBlocks / 4; ++jj) {
    const int blk = w * (C::kBlocks / 4) + jj;
    const int r = blk * C::kRowsPerBlock + r_in;
    const int rr = r < nvalid ? r : nvalid - 1;  // clamp: masked rows re-read a valid row
    const int ck = pc ^ swz_k(r);
    const int cv = pc ^ (FP8 ? swz_v8(r) : swz_v16(r));
    __builtin_amdgcn_global_load_lds((const void*)(kb + (long long)rr * C::kRowBytes + ck * 16),
                                     (MFA_LDS void*)(stage + blk * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)(vb + (long long)rr * C::kRowBytes + cv * 16),
                                     (MFA_LDS void*)(stage + C::kTileBytes + blk * 1024), 16, 0, 0);
  }
}

template <bool FP8>
__device__ __forceinline__ void load_q(const AttnArgs& a, int b, int w, int n, int g, bf16x8 (&qf)[8]) {
  const bf16* qrow = (const bf16*)a.q + ((long long)b * kHeads + 16 * w + n) * kHeadDim;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    // k-slot group g of step j <-> the same 8 channels the K operand reads
    const int d0 = FP8 ? (64 * (j >> 1) + 16 * g + 8 * (j & 1)) : (32 * j + 8 * g);
    qf[j] = *(const bf16x8*)(qrow + d0);
  }
}

// K operand (A of S^T = K Q^T) for the 32 rows of a tile: kf[pb][j] holds the
// 8 channels of k-slot group g at step j for row 16pb + n.
template <bool FP8>
__device__ __forceinline__ void read_k(const char* ks, int n, int g, bf16x8 (&kf)[2][8]) {
  if constexpr (!FP8) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int pc = ((4 * j + g) ^ n) << 4;
      kf[0][j] = *(const MFA_LDS bf16x8*)(ks + n * 512 + pc);
      kf[1][j] = *(const MFA_LDS bf16x8*)(ks + (16 + n) * 512 + pc);
    }
  } else {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int pc = ((4 * jj + g) ^ n) << 4;
#pragma unroll
      for (int pb = 0; pb < 2; ++pb) {
        const u32x4 r = *(const MFA_LDS u32x4*)(ks + (16 * pb + n) * 256 + pc);
        fp8x4_to_bf16(r[0], kf[pb][2 * jj], 0);
        fp8x4_to_bf16(r[1], kf[pb][2 * jj], 4);
        fp8x4_to_bf16(r[2], kf[pb][2 * jj + 1], 0);
        fp8x4_to_bf16(r[3], kf[pb][2 * jj + 1], 4);
      }
    }
  }
}

// V^T operand (A of O^T = V^T P^T): vf[db] holds, for channel 16db + n, the
// cache rows of k-slots 8g..8g+7, i.e. rows 16b + 4g + i (b = 0,1; i = 0..3).
template <bool FP8>
__device__ __forceinline__ void read_v(const char* vs, int n, int g, bf16x8 (&vf)[16]) {
  if constexpr (!FP8) {
    // tr16: lane i of a 16-lane group supplies row 4g + i/4 (+16), channels 4(i%4)..+3
    const int rq = n >> 2;
    const int half = (n & 1) << 3;
    const int lc_lo = (n & 3) >> 1;
    const int r0 = 4 * g + rq, r1 = 16 + 4 * g + rq;
    const int base0 = r0 * 512 + half, base1 = r1 * 512 + half;
    const int sw0 = swz_v16(r0), sw1 = swz_v16(r1);
#pragma unroll
    for (int db = 0; db < 16; ++db) {
      const int lc = 2 * db + lc_lo;
      const bf16x4 lo = lds_read_tr16((const MFA_LDS bf16x4*)(vs + base0 + ((lc ^ sw0) << 4)));
      const bf16x4 hi = lds_read_tr16((const MFA_LDS bf16x4*)(vs + base1 + ((lc ^ sw1) << 4)));
      vf[db] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  } else {
    // tr8: lane i of a 16-lane group supplies k-slot row r' = i/2, byte half i&1
    const int rp = n >> 1;
    const int r = 16 * (rp >> 2) + 4 * g + (rp & 3);
    const int base = r * 256 + ((n & 1) << 3);
    const int sw = swz_v8(r);
#pragma unroll
    for (int db = 0; db < 16; ++db) {
      const i32x2 raw = lds_read_tr8((const MFA_LDS i32x2*)(vs + base + ((db ^ sw) << 4)));
      fp8x4_to_bf16((unsigned)raw[0], vf[db], 0);
      fp8x4_to_bf16((unsigned)raw[1], vf[db], 4);
    }
  }
}

template <bool FP8>
__global__ __launch_bounds__(256, 1) void attn_mfma_kernel(AttnArgs a) {
  using C = Cfg<FP8>;
  __shared__ __attribute__((aligned(1024))) char ring[C::kStages * C::kStageBytes];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int wg = blockIdx.x;

  Cursor prod;
  if (!init_cursor(a, wg, lane, prod)) return;
  Cursor cons = prod;

  int issued = 0;
#pragma unroll
  for (int s = 0; s < C::kStages - 1; ++s) {
    if (prod.valid()) {
      issue_tile<FP8>(a, prod, ring + s * C::kStageBytes, w, lane);
      prod.advance(a.seq_len, a.seq_off);
      ++issued;
    }
  }

  bf16x8 qf[8];
  f32x4 acc[16];
  float m_run = -INFINITY, l_run = 0.f;
  long long piece_lo = 0;
  bool fresh = true;
  bool drained = false;  // stores issued since the last wait: next wait drains fully

  for (int t = 0; cons.valid(); ++t) {
    if (fresh) {
      // Wait for this Q right away (a full drain at each piece start): a
      // pending Q load would otherwise make every later wait drain the ring.
      load_q<FP8>(a, cons.b, w, n, g, qf);
      wait_vmcnt<0>();
#pragma unroll
      for (int db = 0; db < 16; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
      m_run = -INFINITY;
      l_run = 0.f;
      piece_lo = cons.gpos - cons.seq_start;
      fresh = false;
    }
    if (!drained && issued - t - 1 >= C::kStages - 2)
      wait_vmcnt<C::kSteadyVm>();
    else
      wait_vmcnt<0>();
    drained = false;
    __builtin_amdgcn_s_barrier();
    if (prod.valid()) {
      issue_tile<FP8>(a, prod, ring + ((t + C::kStages - 1) % C::kStages) * C::kStageBytes, w, lane);
      prod.advance(a.seq_len, a.seq_off);
      ++issued;
    }

    long long lo, hi;
    cons.tile(lo, hi);
    const int nvalid = (int)(hi - lo);
    const char* ks = ring + (t % C::kStages) * C::kStageBytes;

    bf16x8 kf[2][8];
    read_k<FP8>(ks, n, g, kf);
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][j], qf[j], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][j], qf[j], s1, 0, 0, 0);
    }
    // V reads do not depend on the scores: issue them before the softmax.
    bf16x8 vf[16];
    read_v<FP8>(ks + C::kTileBytes, n, g, vf);

    float sc[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[i] = (4 * g + i < nvalid) ? s0[i] * a.score_mul : -INFINITY;
      sc[4 + i] = (16 + 4 * g + i < nvalid) ? s1[i] * a.score_mul : -INFINITY;
    }
    float mx = sc[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sc[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    float p[8];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = fast_exp2(sc[i] - m_new);
      psum += p[i];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__ballot(alpha != 1.f)) {  // the running max moved for some head of this wave
#pragma unroll
      for (int db = 0; db < 16; ++db) acc[db] *= alpha;
    }
    const bf16x8 pf = {(bf16)p[0], (bf16)p[1], (bf16)p[2], (bf16)p[3],
                       (bf16)p[4], (bf16)p[5], (bf16)p[6], (bf16)p[7]};
#pragma unroll
    for (int db = 0; db < 16; ++db) acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db], pf, acc[db], 0, 0, 0);

    const long long pe = cons.part_end() - cons.seq_start;
    if (hi == pe) {
      // finalize this piece of sequence cons.b
      float lt = l_run + __shfl_xor(l_run, 16);
      lt += __shfl_xor(lt, 32);
      const float inv = a.v_mul / lt;
      const float lse2 = m_run + fast_log2(lt);
      const int h = 16 * w + n;
      const long long L = cons.seq_end - cons.seq_start;
      if (piece_lo == 0 && hi == L) {
        bf16* orow = (bf16*)a.out + ((long long)cons.b * kHeads + h) * kHeadDim + 4 * g;
#pragma unroll
        for (int db = 0; db < 16; ++db) {
          const bf16x4 o = {(bf16)(acc[db][0] * inv), (bf16)(acc[db][1] * inv), (bf16)(acc[db][2] * inv),
                            (bf16)(acc[db][3] * inv)};
          *(bf16x4*)(orow + 16 * db) = o;
        }
        if (a.lse != nullptr && g == 0) a.lse[(long long)cons.b * kHeads + h] = lse2 * kLn2;
      } else {
        const long long slot = (long long)wg + cons.b;
        float* prow = a.part_o + (slot * kHeads + h) * kHeadDim + 4 * g;
#pragma unroll
        for (int db = 0; db < 16; ++db) *(f32x4*)(prow + 16 * db) = acc[db] * inv;
        if (g == 0) a.part_lse[slot * kHeads + h] = lse2;
      }
      fresh = true;
      drained = true;
    }
    cons.advance(a.seq_len, a.seq_off);
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel (fp32 q and cache): plain VALU dot products, same work split and
// partial format. Lane (n, g) of wave w owns head 16w+n and channels 64g..64g+63.
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int wg = blockIdx.x;
  Cursor cons;
  if (!init_cursor(a, wg, lane, cons)) return;
  const int h = 16 * w + n;

  float qr[64], acc[64];
  float m_run = -INFINITY, l_run = 0.f;
  long long piece_lo = 0;
  bool fresh = true;
  while (cons.valid()) {
    if (fresh) {
      const float* qrow = (const float*)a.q + ((long long)cons.b * kHeads + h) * kHeadDim + 64 * g;
#pragma unroll
      for (int d = 0; d < 64; d += 4) {
        const f32x4 v = *(const f32x4*)(qrow + d);
        qr[d] = v[0]; qr[d + 1] = v[1]; qr[d + 2] = v[2]; qr[d + 3] = v[3];
      }
#pragma unroll
      for (int d = 0; d < 64; ++d) acc[d] = 0.f;
      m_run = -INFINITY;
      l_run = 0.f;
      piece_lo = cons.gpos - cons.seq_start;
      fresh = false;
    }
    long long lo, hi;
    cons.tile(lo, hi);
    const int nvalid = (int)(hi - lo);
    const float* kb = (const float*)a.k + (cons.off + lo) * kHeadDim + 64 * g;
    const float* vb = (const float*)a.v + (cons.off + lo) * kHeadDim + 64 * g;
    float s[kTile];
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
      s[j] = -INFINITY;
      if (j < nvalid) {
        float part = 0.f;
#pragma unroll
        for (int d = 0; d < 64; d += 4) {
          const f32x4 kv = *(const f32x4*)(kb + (long long)j * kHeadDim + d);
          part = fmaf(qr[d], kv[0], part);
          part = fmaf(qr[d + 1], kv[1], part);
          part = fmaf(qr[d + 2], kv[2], part);
          part = fmaf(qr[d + 3], kv[3], part);
        }
        part += __shfl_xor(part, 16);
        part += __shfl_xor(part, 32);
        s[j] = part * a.score_mul;
      }
    }
    float mx = s[0];
#pragma unroll
    for (int j = 1; j < kTile; ++j) mx = fmaxf(mx, s[j]);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < 64; ++d) acc[d] *= alpha;
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
      if (j < nvalid) {
        const float pj = fast_exp2(s[j] - m_new);
        l_run += pj;
#pragma unroll
        for (int d = 0; d < 64; d += 4) {
          const f32x4 vv = *(const f32x4*)(vb + (long long)j * kHeadDim + d);
          acc[d] = fmaf(pj, vv[0], acc[d]);
          acc[d + 1] = fmaf(pj, vv[1], acc[d + 1]);
          acc[d + 2] = fmaf(pj, vv[2], acc[d + 2]);
          acc[d + 3] = fmaf(pj, vv[3], acc[d + 3]);
        }
      }
    }
    m_run = m_new;

    const long long pe = cons.part_end() - cons.seq_start;
    if (hi == pe) {
      // every lane of head h holds the full row sum (scores were all-reduced)
      const float inv = a.v_mul / l_run;
      const float lse2 = m_run + fast_log2(l_run);
      const long long L = cons.seq_end - cons.seq_start;
      float* dst;
      if (piece_lo == 0 && hi == L) {
        dst = (float*)a.out + ((long long)cons.b * kHeads + h) * kHeadDim + 64 * g;
        if (a.lse != nullptr && g == 0) a.lse[(long long)cons.b * kHeads + h] = lse2 * kLn2;
      } else {
        const long long slot = (long long)wg + cons.b;
        dst = a.part_o + (slot * kHeads + h) * kHeadDim + 64 * g;
        if (g == 0) a.part_lse[slot * kHeads + h] = lse2;
      }
#pragma unroll
      for (int d = 0; d < 64; d += 4)
        *(f32x4*)(dst + d) = f32x4{acc[d] * inv, acc[d + 1] * inv, acc[d + 2] * inv, acc[d + 3] * inv};
      fresh = true;
    }
    cons.advance(a.seq_len, a.seq_off);
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the pieces of each split sequence. Grid (B, 4): block
// (b, hg) merges heads 16hg..16hg+15; thread t owns head 16hg + t/16 and
// channels 16*(t%16)..+15. Sequences inside one piece were written by the
// attention kernel and are skipped; empty sequences get out = 0, lse = -inf.
template <typename OutT>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int h = 16 * blockIdx.y + (threadIdx.x >> 4);
  const int d0 = 16 * (threadIdx.x & 15);
  const long long L = a.seq_len[b];
  OutT* orow = (OutT*)a.out + ((long long)b * kHeads + h) * kHeadDim + d0;
  if (L == 0) {
#pragma unroll
    for (int d = 0; d < 16; ++d) orow[d] = (OutT)0.f;
    if (a.lse != nullptr && (threadIdx.x & 15) == 0) a.lse[(long long)b * kHeads + h] = -INFINITY;
    return;
  }
  const long long total = total_len(a.seq_len, a.B, lane);
  const long long per = piece_len(total, a.G);
  const long long start = seq_start_of(a.seq_len, b, lane);
  const long long w0 = start / per, w1 = (start + L - 1) / per;
  if (w0 == w1) return;
  float mx = -INFINITY;
  for (long long s = w0; s <= w1; ++s) mx = fmaxf(mx, a.part_lse[(s + b) * kHeads + h]);
  float o[16];
#pragma unroll
  for (int d = 0; d < 16; ++d) o[d] = 0.f;
  float wsum = 0.f;
  for (long long s = w0; s <= w1; ++s) {
    const float wt = fast_exp2(a.part_lse[(s + b) * kHeads + h] - mx);
    wsum += wt;
    const float* prow = a.part_o + ((s + b) * kHeads + h) * kHeadDim + d0;
#pragma unroll
    for (int d = 0; d < 16; d += 4) {
      const f32x4 v = *(const f32x4*)(prow + d);
      o[d] = fmaf(wt, v[0], o[d]);
      o[d + 1] = fmaf(wt, v[1], o[d + 1]);
      o[d + 2] = fmaf(wt, v[2], o[d + 2]);
      o[d + 3] = fmaf(wt, v[3], o[d + 3]);
    }
  }
  const float inv = 1.f / wsum;
#pragma unroll
  for (int d = 0; d < 16; ++d) orow[d] = (OutT)(o[d] * inv);
  if (a.lse != nullptr && (threadIdx.x & 15) == 0)
    a.lse[(long long)b * kHeads + h] = (mx + fast_log2(wsum)) * kLn2;
}

// ---------------------------------------------------------------------------
hipError_t launch_decode_attn(const AttnLaunch& p, hipStream_t stream) {
  AttnArgs a;
  a.q = p.q;
  a.k = p.k;
  a.v = p.v;
  a.seq_off = p.seq_off;
  a.seq_len = p.seq_len;
  a.out = p.out;
  a.lse = p.lse;
  a.part_o = (float*)p.ws;
  a.part_lse = (float*)((char*)p.ws + attn_part_o_bytes(p.B, p.G));
  a.B = p.B;
  a.G = p.G;
  a.score_mul = p.softmax_scale * p.k_scale * kLog2e;
  a.v_mul = p.v_scale;
  const dim3 block(256);
  const dim3 comb(p.B, 4);
  hipError_t e = hipSuccess;
  switch (p.kind) {
    case AttnKind::F32:
      e = launch(attn_f32_kernel, dim3(p.G), block, stream, a);
      if (e == hipSuccess) e = launch(attn_combine_kernel<float>, comb, block, stream, a);
      break;
    case AttnKind::BF16:
      e = launch(attn_mfma_kernel<false>, dim3(p.G), block, stream, a);
      if (e == hipSuccess) e = launch(attn_combine_kernel<bf16>, comb, block, stream, a);
      break;
    case AttnKind::BF16_FP8KV:
      e = launch(attn_mfma_kernel<true>, dim3(p.G), block, stream, a);
      if (e == hipSuccess) e = launch(attn_combine_kernel<bf16>, comb, block, stream, a);
      break;
  }
  return e;
}

}  // namespace mfa
