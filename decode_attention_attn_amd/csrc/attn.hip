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
//    into G equal pieces (G = one workgroup per CU), each a multiple of 64
//    rows. A workgroup walks its piece, which may cover the tail of one
//    sequence and the head of the next, so ragged lengths never leave CUs
//    idle. A sequence cut into several pieces is merged afterwards by a
//    log-sum-exp combine; a sequence inside one piece is written directly.
//    A split piece stores its normalised partial in bf16 in the MFMA register
//    layout (eight 1 KB contiguous stores per wave), and the workgroup holding
//    a sequence's first piece records where its pieces are, so the combine
//    kernel goes straight to its loads.
//  * Data path. Tiles of 32 KB (32 bf16 rows or 64 fp8 rows of K, then of V)
//    go HBM -> LDS by direct-to-LDS DMA (global_load_lds_dwordx4: each lane
//    moves 16 B, a wave 1 KB) into a 4-stage ring, three tiles ahead of the
//    compute, one barrier per tile. Rows are XOR-swizzled in 16-byte chunks at
//    DMA time so that the MFMA operand reads below are bank-conflict free;
//    every row is still read as one full run.
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
//  * Softmax in base 2: scores are multiplied by scale*log2(e) once; the
//    running max and sum live in registers; the reference max moves only when
//    a score exceeds it by more than 8 (a factor 256), so the O accumulator is
//    rescaled on a piece's first tile and rarely after; row sums are combined
//    across the 4 lanes of a head with the gfx950 row swaps at piece end.
#include <atomic>

#include "attn_core.h"

namespace mfa {

// ---------------------------------------------------------------------------
// One new token per sequence, with producer waves. Waves 0..3 compute (heads
// 16w..16w+15); kProducers more waves only move data:
// they issue every DMA of the cache tiles (and of q, see kQLds) into the LDS
// ring and wait for their own, so a compute wave never stalls on a DMA issue (the
// memory system takes requests only as fast as it drains them) and never
// computes a DMA address. The per-tile barrier hands each landed tile from
// the producers to the compute waves and each consumed stage back. Both
// sides walk the same cursor, so they agree on every barrier.
// Two producers keep three tiles in flight within the 6-bit wait counter
// (measured: four producers, or a fifth ring stage, no faster).
constexpr int kProducers = 2;  // producer waves per workgroup

// DMA issue for the producer waves: the per-lane byte offsets of a full tile
// (row and swizzled chunk, as issue_tile computes them) are computed once, so
// a full tile costs one 64-bit uniform base and no per-lane address math;
// tiles with rows past the end take issue_tile (rows clamped).
template <bool FP8, bool PAGED, int kIssuers>
struct TileIssuer {
  using C = Cfg<FP8>;
  static constexpr int kBlocks = C::kHalfBytes / 1024 / kIssuers;
  int koff[kBlocks], voff[kBlocks];
  __device__ __forceinline__ TileIssuer(int w, int lane) {
    const int r_in = lane / C::kChunksPerRow;
    const int pc = lane % C::kChunksPerRow;
#pragma unroll
    for (int jj = 0; jj < kBlocks; ++jj) {
      const int r = (w * kBlocks + jj) * C::kRowsPerBlock + r_in;
      const int r32 = r & 31;
      koff[jj] = r * C::kRowBytes + ((pc ^ swz_k(r32)) << 4);
      voff[jj] = r * C::kRowBytes + ((pc ^ (FP8 ? swz_v8(r32) : swz_v16(r32))) << 4);
    }
  }
  __device__ __forceinline__ void issue(const AttnArgs& a, const Cursor<C::kRows, PAGED>& c, char* stage, int w,
                                        int lane) const {
    long long lo, hi;
    c.tile(lo, hi);
    if (c.valid_rows(lo, hi) < C::kRows) {
      issue_tile<FP8, PAGED, kIssuers>(a, c, stage, w, lane);
      return;
    }
    long long row0;
    if constexpr (PAGED) {
      const long long page = load_scalar(a.table, (long long)c.b * a.max_blocks + (lo >> a.page_shift));
      row0 = (page << a.page_shift) + (lo & ((1LL << a.page_shift) - 1));
    } else {
      row0 = c.off + lo;
    }
    const char* kb = (const char*)a.k + uniform(row0) * C::kRowBytes;
    const char* vb = (const char*)a.v + uniform(row0) * C::kRowBytes;
#pragma unroll
    for (int jj = 0; jj < kBlocks; ++jj) {
      const int blk = w * kBlocks + jj;
      __builtin_amdgcn_global_load_lds((const void*)(kb + koff[jj]), (MFA_LDS void*)(stage + blk * 1024), 16, 0,
                                       kCpolNT);
      __builtin_amdgcn_global_load_lds((const void*)(vb + voff[jj]), (MFA_LDS void*)(stage + C::kHalfBytes + blk * 1024),
                                       16, 0, kCpolNT);
    }
  }
};

// Where the compute waves get q from. kQLds: the producers DMA the first q
// of the piece into an LDS buffer beside the ring, as a tile (requested
// before the work split is known, for the sequence the piece starts in when
// all lengths are equal); once every compute wave has read a sequence's q into
// registers (by the barrier of its second tile), the compute waves DMA the
// next sequence's q into the same buffer, so a piece that runs into the next
// sequence finds its q there without stopping the tile stream. Otherwise the
// compute waves load q straight into registers (they issue no other loads, so
// waiting for q never waits for a tile) and split it for the fp8 product
// while the first tile is still in flight. Measured on MI355X, 4K context:
// bf16 33.1 us with q in LDS against 33.6 us in registers; fp8 cache 44.0 us
// against 42.8 us.
template <bool FP8>
constexpr bool kQLds = !FP8;

// The producer side: the same cursor walk, the same barriers, only DMAs.
// b_guess: the sequence whose q the producers already requested before the
// work split was known (kQLds only); another is requested now.
template <bool FP8, bool PAGED, int kNP>
__device__ __forceinline__ void pc_producer(const AttnArgs& a, Cursor<Cfg<FP8>::kRows, PAGED> prod, char* ring,
                                            char* qs, int pw, int lane, int b_guess) {
  using C = Cfg<FP8>;
  constexpr int kDpp = 2 * (C::kHalfBytes / 1024) / kNP;  // DMAs per producer per tile
  static_assert((C::kStages - 1) * kDpp < 64, "tiles in flight exceed the wait counter");
  const TileIssuer<FP8, PAGED, kNP> tiles(pw, lane);
  Cursor<C::kRows, PAGED> cons = prod;
  int issued = 0;
  if (kQLds<FP8> && cons.b != b_guess) issue_q<kNP>(a, cons.b, qs, pw, lane);  // lands after the guessed one
#pragma unroll
  for (int st = 0; st < C::kStages - 1; ++st) {
    if (prod.valid()) {
      tiles.issue(a, prod, ring + st * C::kTileBytes, pw, lane);
      prod.advance(a.seq_len, a.seq_off);
      ++issued;
    }
  }
  if constexpr (kQLds<FP8>) {
    // q and tile 0 have landed once at most the later prologue tiles are in flight
    wait_tiles<kDpp>(issued - 1);
    __builtin_amdgcn_s_barrier();
  }
  for (int t = 0; cons.valid(); ++t) {
    // tile t has landed once at most the later ones are in flight
    wait_tiles<kDpp>(issued - t - 1);
    __builtin_amdgcn_s_barrier();
    if (prod.valid()) {
      tiles.issue(a, prod, ring + ((t + C::kStages - 1) % C::kStages) * C::kTileBytes, pw, lane);
      prod.advance(a.seq_len, a.seq_off);
      ++issued;
    }
    cons.advance(a.seq_len, a.seq_off);
  }
}

template <bool FP8, bool PAGED, int kNP>
__global__ __launch_bounds__(64 * (4 + kNP), 1) void attn_pc_kernel(AttnArgs a) {
  using C = Cfg<FP8>;
  constexpr bool kQL = kQLds<FP8>;
  __shared__ __attribute__((aligned(1024))) char ring[kQL ? C::kLdsBytes : C::kStages * C::kTileBytes];
  char* const qs = ring + C::kStages * C::kTileBytes;
  const int lane = threadIdx.x & 63;
  const int wv = uniform((int)(threadIdx.x >> 6));
  const int wgi = piece_index(a.G);
  const int w = wv;  // compute waves: heads 16w..16w+15
  const int n = lane & 15;
  const int g = lane >> 4;
  // q is requested before the work split is known, for the sequence this
  // piece starts in when all lengths are equal, so that it travels during the
  // split's round trip (if the guess is wrong the right q is requested once
  // the split is known; q is only read after that).
  const int b_guess = uniform((int)(((long long)wgi * a.B) / a.G));
  bf16x8 qf[8];
  if constexpr (kQL) {
    if (wv >= 4) issue_q<kNP>(a, b_guess, qs, wv - 4, lane);
  } else {
    if (wv < 4) load_q<FP8>(a, b_guess, w, n, g, qf);
  }

  Cursor<C::kRows, PAGED> cons;
  if (!init_cursor(a, wgi, lane, cons)) {
    wait_vmcnt<0>();  // no piece: let the q request land before leaving
    return;
  }
  if (wv >= 4) {
    pc_producer<FP8, PAGED, kNP>(a, cons, ring, qs, wv - 4, lane, b_guess);
    return;
  }
  Q8 q8;
  if constexpr (kQL) {
    __builtin_amdgcn_s_barrier();  // q and tile 0 have landed
    read_q<FP8>(qs, w, n, g, qf);
  } else {
    if (cons.b != b_guess) {
      wait_vmcnt<0>();
      load_q<FP8>(a, cons.b, w, n, g, qf);
    }
    wait_vmcnt<0>();
  }
  if constexpr (FP8) split_q8(qf, q8);
  f32x4 acc[16];
#pragma unroll
  for (int db = 0; db < 16; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  const VReader<FP8> vr(n, g);
  float m_run = -INFINITY, l_run = 0.f;
  long long piece_lo = cons.gpos - cons.seq_start;
  bool fresh = false;
  int t_first = 0;  // the piece's first tile of the current sequence
  int q_next = -1;  // kQL: the sequence whose q the compute waves put into the q buffer

  for (int t = 0; cons.valid(); ++t) {
    if (!kQL && fresh) {
      // the piece's next sequence: its q
      load_q<FP8>(a, cons.b, w, n, g, qf);
      wait_vmcnt<0>();  // (also waits for the partial's stores just issued)
      if constexpr (FP8) split_q8(qf, q8);
    }
    __builtin_amdgcn_s_barrier();  // tile t has landed
    if constexpr (kQL) {
      if (fresh) {
        // every compute wave waited for its part of the q DMA before the barrier
        if (q_next == cons.b) {
          read_q<FP8>(qs, w, n, g, qf);
        } else {  // (a one-tile sequence before this one, or empty sequences between)
          load_q<FP8>(a, cons.b, w, n, g, qf);
          wait_vmcnt<0>();
        }
      } else if (t == t_first + 1 && cons.seq_end < cons.r1) {
        // every compute wave has this sequence's q in registers (the previous
        // tile's MFMAs consumed it): fetch the next sequence's q into the buffer
        issue_q<4>(a, cons.b + 1, qs, w, lane);
        q_next = cons.b + 1;
      }
    }
    if (fresh) {
      m_run = -INFINITY;  // the first block rescales acc and l by exp2(-inf) = 0
      piece_lo = cons.gpos - cons.seq_start;
      t_first = t;
      fresh = false;
    }
    long long lo, hi;
    cons.tile(lo, hi);
    char* stage = ring + (t % C::kStages) * C::kTileBytes;
    const int nvalid = cons.valid_rows(lo, hi);
    if constexpr (FP8)
      attend_tile_fp8<true>(stage, stage + C::kHalfBytes, nvalid, n, g, vr, q8, a.score_mul, m_run, l_run, acc);
    else
      attend_tile_bf16(stage, stage + C::kHalfBytes, nvalid, n, g, vr, qf, a.score_mul, m_run, l_run, acc);
    if (hi == cons.part_end() - cons.seq_start) {
      // the next q's DMA (issued tiles ago) has landed: waited for here, before
      // the partial's stores join the counter
      if (kQL && q_next == cons.b + 1) wait_vmcnt<0>();
      finish_segment(a, cons, wgi, piece_lo, hi, w, lane, sum_over_rows(l_run), m_run, 0.f, acc);
      fresh = true;
    }
    cons.advance(a.seq_len, a.seq_off);
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel (fp32 q and cache): plain VALU dot products, same work split and
// partial format. Lane (n, g) of wave w owns head 16w+n and channels 64g..64g+63.
constexpr int kF32Rows = 32;

__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int wgi = piece_index(a.G);
  Cursor<kF32Rows> cons;
  if (!init_cursor(a, wgi, lane, cons)) return;
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
        qr[d] = v[0];
        qr[d + 1] = v[1];
        qr[d + 2] = v[2];
        qr[d + 3] = v[3];
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
    float s[kF32Rows];
#pragma unroll
    for (int j = 0; j < kF32Rows; ++j) {
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
    for (int j = 1; j < kF32Rows; ++j) mx = fmaxf(mx, s[j]);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < 64; ++d) acc[d] *= alpha;
#pragma unroll
    for (int j = 0; j < kF32Rows; ++j) {
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
      if (piece_lo == 0 && threadIdx.x == 0) {
        const int np = hi == L ? 0 : (int)((cons.seq_start + L - 1) / cons.per - wgi + 1);
        *(i32x2*)(a.meta + 2 * cons.b) = i32x2{wgi + cons.b, np};
      }
      float* dst;
      if (piece_lo == 0 && hi == L) {
        dst = (float*)a.out + ((long long)cons.b * kHeads + h) * kHeadDim + 64 * g;
        if (a.lse != nullptr && g == 0) a.lse[(long long)cons.b * kHeads + h] = lse2 * kLn2;
      } else {
        const long long slot = (long long)wgi + cons.b;
        dst = (float*)a.part_o + (slot * kHeads + h) * kHeadDim + 64 * g;
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
// Log-sum-exp merge of the pieces of each split sequence (the combine rule of
// split-KV decoding: weights exp(lse_s - lse), lse = log sum exp lse_s).
// Sequences inside one piece were written by the attention kernel and are
// skipped; empty sequences get out = 0, lse = -inf. Partials are read 8 at a
// time and merged with a running max (one pass).

// fp32 partials in [slot][head][channel] layout. Grid (B, 16): block (b, hq)
// merges heads 4hq..4hq+3; thread t owns head 4hq + t/64, channels 4(t%64)..+3.
__global__ __launch_bounds__(256) void attn_combine_f32_kernel(AttnArgs a) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int h = 4 * blockIdx.y + (threadIdx.x >> 6);
  const int d0 = 4 * lane;
  // the length and the piece record are loaded together (one round trip);
  // the record is written by the attention kernel for every non-empty
  // sequence and is not looked at for an empty one
  const long long L = load_scalar(a.seq_len, b);
  const i32x2 rec = load_scalar((const i32x2*)a.meta, b);
  float* orow = (float*)a.out + ((long long)b * kHeads + h) * kHeadDim + d0;
  // (np >= 0 always: the test only keeps the record load ahead of the branch)
  if ((L == 0) | (rec[1] < 0)) {
    *(f32x4*)orow = f32x4{0.f, 0.f, 0.f, 0.f};
    if (a.lse != nullptr && lane == 0) a.lse[(long long)b * kHeads + h] = -INFINITY;
    return;
  }
  const int np = rec[1];
  if (np == 0) return;
  const long long slot0 = rec[0];
  const float* lrow = a.part_lse + slot0 * kHeads + h;
  const float* prow = (const float*)a.part_o + (slot0 * kHeads + h) * kHeadDim + d0;
  constexpr int kBatch = 8;
  float m = -INFINITY, wsum = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < np; s0 += kBatch) {
    f32x4 part[kBatch];
    float lw[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int s = s0 + k < np ? s0 + k : np - 1;
      part[k] = *(const f32x4*)(prow + (long long)s * kHeads * kHeadDim);
      lw[k] = s0 + k < np ? lrow[(long long)s * kHeads] : -INFINITY;
    }
    float mb = lw[0];
#pragma unroll
    for (int k = 1; k < kBatch; ++k) mb = fmaxf(mb, lw[k]);
    const float m_new = fmaxf(m, mb);
    const float sc = fast_exp2(m - m_new);  // 0 on the first batch
    wsum *= sc;
    o *= sc;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const float wt = fast_exp2(lw[k] - m_new);  // 0 for the padding entries
      wsum += wt;
      o += part[k] * wt;
    }
    m = m_new;
  }
  *(f32x4*)orow = o * (1.f / wsum);
  if (a.lse != nullptr && lane == 0) a.lse[(long long)b * kHeads + h] = (m + fast_log2(wsum)) * kLn2;
}

// bf16 partials in the MFMA kernel's register layout: 16-byte chunk
// c = (w*8 + dp)*64 + lane of a slot holds head 16w + (lane%16), channels
// 32dp + 4(lane/16) + {0..3} and the same + 16. Grid (B, 8): thread c of the
// sequence merges chunk c of every partial.
__global__ __launch_bounds__(256) void attn_combine_mfma_kernel(AttnArgs a) {
  // workgroup (bt, y): channel block y of output row bt = (sequence b, token tok).
  // The attention kernel gives each XCD a contiguous run of pieces, so with
  // equal lengths sequence b's pieces ran on XCD 8b / B; its merge is placed
  // there too (workgroup i runs on XCD i % 8), where the partials may still
  // be in L2. Placement only affects speed.
  const int nt = a.nt;  // new tokens per sequence (1 .. 4)
  const int wgs = a.B * nt * 8;
  const int i = blockIdx.x;
  const int j = (a.B & 7) == 0 ? (i & 7) * (wgs >> 3) + (i >> 3) : i;
  const int bt = j >> 3;
  const int b = bt / nt;
  const int tok = bt - b * nt;
  const int c = (j & 7) * 256 + threadIdx.x;
  const int lane = c & 63, dp = (c >> 6) & 7, w = c >> 9;
  const int n = lane & 15, g = lane >> 4;
  const int h = 16 * w + n;
  // length and piece record in one round trip (the record of an empty
  // sequence is never written and not looked at)
  const long long L = load_scalar(a.seq_len, b);
  const i32x2 rec = load_scalar((const i32x2*)a.meta, b);
  bf16* orow = (bf16*)a.out + ((long long)bt * kHeads + h) * kHeadDim + 32 * dp + 4 * g;
  const bool lse_owner = a.lse != nullptr && dp == 0 && g == 0;
  // (np >= 0 always: the test only keeps the record load ahead of the branch)
  if ((L == 0) | (rec[1] < 0)) {
    *(bf16x4*)orow = bf16x4{};
    *(bf16x4*)(orow + 16) = bf16x4{};
    if (lse_owner) a.lse[(long long)bt * kHeads + h] = -INFINITY;
    return;
  }
  const int np = rec[1];
  if (np == 0) return;
  // piece s of the sequence holds slot (slot0 + s) * nt + tok
  const long long slot0 = (long long)rec[0] * nt + tok;
  const long long lstride = (long long)nt * kHeads, pstride = (long long)nt * (kHeads * kHeadDim / 8);
  const float* lrow = a.part_lse + slot0 * kHeads + h;
  const bf16x8* prow = (const bf16x8*)a.part_o + slot0 * (kHeads * kHeadDim / 8) + c;
  constexpr int kBatch = 8;
  float m = -INFINITY, wsum = 0.f;
  f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < np; s0 += kBatch) {
    bf16x8 part[kBatch];
    float lw[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int s = s0 + k < np ? s0 + k : np - 1;
      part[k] = prow[s * pstride];
      lw[k] = s0 + k < np ? lrow[s * lstride] : -INFINITY;
    }
    float mb = lw[0];
#pragma unroll
    for (int k = 1; k < kBatch; ++k) mb = fmaxf(mb, lw[k]);
    const float m_new = fmaxf(m, mb);
    // (m_new = -inf only while every piece so far is empty for this token)
    const bool none = m_new == -INFINITY;
    const float sc = none ? 0.f : fast_exp2(m - m_new);  // 0 on the first batch
    wsum *= sc;
    o0 *= sc;
    o1 *= sc;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const float wt = none ? 0.f : fast_exp2(lw[k] - m_new);  // 0 for the padding entries
      wsum += wt;
      o0 += f32x4{(float)part[k][0], (float)part[k][1], (float)part[k][2], (float)part[k][3]} * wt;
      o1 += f32x4{(float)part[k][4], (float)part[k][5], (float)part[k][6], (float)part[k][7]} * wt;
    }
    m = m_new;
  }
  // wsum = 0: the token saw no row at all (multi-token decode on a short
  // sequence): output 0 and lse -inf, as for an empty sequence
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  o0 *= inv;
  o1 *= inv;
  *(bf16x4*)orow = bf16x4{(bf16)o0[0], (bf16)o0[1], (bf16)o0[2], (bf16)o0[3]};
  *(bf16x4*)(orow + 16) = bf16x4{(bf16)o1[0], (bf16)o1[1], (bf16)o1[2], (bf16)o1[3]};
  if (lse_owner) a.lse[(long long)bt * kHeads + h] = wsum > 0.f ? (m + fast_log2(wsum)) * kLn2 : -INFINITY;
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
  a.part_o = p.ws;
  a.part_lse = (float*)((char*)p.ws + attn_part_o_bytes(p.B, p.G, p.nt));
  a.meta = (int*)((char*)p.ws + attn_meta_offset(p.B, p.G, p.nt));
  a.table = p.table;
  a.max_blocks = p.max_blocks;
  a.page_shift = p.page_shift;
  a.nt = p.nt;
  a.t0 = 0;
  a.B = p.B;
  a.G = p.G;
  a.score_mul = p.softmax_scale * p.k_scale * kLog2e;
  a.v_mul = p.v_scale;
  const dim3 block(256);
  const dim3 comb_f32(p.B, 16);
  const dim3 comb_mfma(p.B * p.nt * 8);
  hipError_t e = hipSuccess;
  switch (p.kind) {
    case AttnKind::F32:
      e = launch(attn_f32_kernel, dim3(p.G), block, stream, a);
      if (e == hipSuccess) e = launch(attn_combine_f32_kernel, comb_f32, block, stream, a);
      break;
    case AttnKind::BF16:
      if (p.nt > 1)
        e = launch_attn_mt(a, false, p.table != nullptr, stream);
      else
        e = p.table ? launch(attn_pc_kernel<false, true, kProducers>, dim3(p.G), dim3(64 * (4 + kProducers)), stream, a)
                    : launch(attn_pc_kernel<false, false, kProducers>, dim3(p.G), dim3(64 * (4 + kProducers)), stream, a);
      if (e == hipSuccess) e = launch(attn_combine_mfma_kernel, comb_mfma, block, stream, a);
      break;
    case AttnKind::BF16_FP8KV:
      if (p.nt > 1)
        e = launch_attn_mt(a, true, p.table != nullptr, stream);
      else
        e = p.table ? launch(attn_pc_kernel<true, true, kProducers>, dim3(p.G), dim3(64 * (4 + kProducers)), stream, a)
                    : launch(attn_pc_kernel<true, false, kProducers>, dim3(p.G), dim3(64 * (4 + kProducers)), stream, a);
      if (e == hipSuccess) e = launch(attn_combine_mfma_kernel, comb_mfma, block, stream, a);
      break;
  }
  return e;
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free entry point: partial outputs, their lse and
// the merge records, laid out as in a caller's workspace. The runtime places
// one copy on every GPU that loads this code object. On the host `scratch`
// only stands for the symbol and is never passed to a kernel or a copy: host
// code uses the device address hipGetSymbolAddress returns for the current
// device, looked up on the first call on that device and kept.
static __device__ __align__(256) char scratch[kAttnScratchBytes];

hipError_t attn_scratch(void** ptr) {
  constexpr int kDevices = 64;
  static std::atomic<void*> addr[kDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kDevices) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace mfa
